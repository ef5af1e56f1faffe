"""The inputs of the n_eff precision test are discriminating.

The participation ratio n_eff = S1^2 / S2 [ATMA §2.1] must come out within 1e-2 of the
oracle for bf16 inputs.  If the prefill formed S1 and S2 from the bf16-rounded weights
that enter the P V product (relative rounding error up to u = 2^-8 each), a row whose
weight mass sits on many identical weak keys while its squared mass sits on one strong
key, the two rounded in opposite directions, would be off by up to about 4u = 1.6e-2.
These tests model that arithmetic on the rows of polar_inputs.rounding_adversary_qkv
(weights formed in fp32 as exp2 of c times the score, relative to the row's first-tile
maximum, which is the score 0 of key 0) and check that sums of bf16 weights exceed the
tolerance on them, while sums of the fp32 weights stay far inside it; the oracle gives
the exact value.  The GPU test over the same inputs then tells the two apart.
"""
import math

import numpy as np
import pytest
import torch

import polar_inputs as pin
from oracle import polar_attention
from tests.parity import to_np

T = 2048 + 64


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _modelled_neff(strong, weak, d, n_weak, bf16_weights):
    scale = np.float32(1.0 / math.sqrt(d))
    c = np.float32(np.float32(1.0 * scale) * np.float32(1.4426950408889634))
    w = np.exp2(np.array([np.float32(c * np.float32(strong)), np.float32(c * np.float32(weak))],
                         np.float64)).astype(np.float32)
    a, b = (_bf16(w) if bf16_weights else w.astype(np.float64))
    s1 = 1.0 + a + n_weak * b
    s2 = 1.0 + a * a + n_weak * b * b
    return s1 * s1 / s2


@pytest.mark.parametrize("d", [64, 128])
def test_rounding_rows_discriminate(d):
    q, k, v = pin.rounding_adversary_qkv(T, d, seed=3)
    rows = np.arange(65, T, 7)
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, null_bias=[0.0] * q.shape[1], rows=rows)
    worst_bf16, worst_f32 = 0.0, 0.0
    for h, (strong, weak) in enumerate(pin.ROUNDING_PAIRS[d]):
        exact = ref["n_eff"][0, h]
        n_weak = rows - 1  # keys 1..63 and 65..i
        for bf, name in ((True, "bf16"), (False, "f32")):
            err = np.abs(_modelled_neff(strong, weak, d, n_weak, bf) / exact - 1).max()
            if bf:
                worst_bf16 = max(worst_bf16, err)
            else:
                worst_f32 = max(worst_f32, err)
    # at T = 2112 the bf16-weight sums already leave the tolerance on some row; the test on
    # the GPU runs T = 8192, where the effect is larger still
    assert worst_bf16 > 1.0e-2, worst_bf16
    assert worst_f32 < 1.0e-5, worst_f32

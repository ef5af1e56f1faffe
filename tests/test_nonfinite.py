"""Non-finite inputs in the oracle: the policy the library states for them.

The operator is defined for finite inputs.  A NaN in an input propagates: every output
channel of each row whose computation it enters is NaN, and so are the sums S1 and S2
of its statistics (the maximum m is unspecified; the oracle's is NaN), and every other
row is exactly what it is without it.  A NaN in q_i enters row i; in k_j, every row
that sees key j; in v_j, the direction of every row that sees key j (n_eff, confidence,
count and the statistics do not depend on v), and it may also reach the direction of
earlier rows evaluated together with key j (a zero weight times NaN is NaN): the oracle
evaluates rows in blocks of 512, the kernels in query tiles.
"""
import numpy as np
import pytest
import torch

import polar_inputs as pin
from oracle import polar_attention
from tests.parity import to_np

CHANNELS = ("direction", "n_eff", "confidence", "count", "m", "s1", "s2")
MAGNITUDES = ("n_eff", "confidence", "count", "m", "s1", "s2")


def _inputs(T=1100, d=64, H=2, seed=41):
    q, k, v, _ = pin.random_qkv(1, H, H, T, T, d, torch.float32, seed)
    return to_np(q), to_np(k), to_np(v)


def _run(q, k, v, causal=True):
    return polar_attention(q, k, v, causal=causal, len_temp=[0.1, 0.0], null_bias=[0.0, 0.5])


def _all_nan(out, h, rows, keys=CHANNELS):
    return all(np.isnan(out[c][0, h, rows]).all() for c in keys)


def _same(a, b, h, rows, keys=CHANNELS):
    return all(np.array_equal(a[c][0, h, rows], b[c][0, h, rows]) for c in keys)


def test_nan_in_a_query_row():
    q, k, v = _inputs()
    clean = _run(q, k, v)
    q[0, 1, 123, 17] = np.nan
    out = _run(q, k, v)
    assert _all_nan(out, 1, [123])
    others = np.setdiff1d(np.arange(q.shape[2]), [123])
    assert _same(out, clean, 1, others) and _same(out, clean, 0, slice(None))


def test_nan_in_a_key():
    q, k, v = _inputs()
    clean = _run(q, k, v)
    j = 700
    k[0, 0, j, 5] = np.nan
    out = _run(q, k, v)
    assert _all_nan(out, 0, slice(j, None))                 # every row that sees key j
    assert _same(out, clean, 0, slice(0, j))                # the rows before it do not
    assert _same(out, clean, 1, slice(None))                # nor another head
    # without the mask every row sees it
    out_nc = _run(q, k, v, causal=False)
    assert _all_nan(out_nc, 0, slice(None))


def test_nan_in_a_value():
    q, k, v = _inputs()
    clean = _run(q, k, v)
    j = 1000
    v[0, 0, j, 7] = np.nan
    out = _run(q, k, v)
    assert _all_nan(out, 0, slice(j, None), ("direction",))
    assert _same(out, clean, 0, slice(None), MAGNITUDES)     # n_eff and the rest ignore v
    assert _same(out, clean, 0, slice(0, 512))               # rows evaluated apart from key j
    assert _same(out, clean, 1, slice(None))


def test_zero_values_still_give_zero_direction():
    """The NaN rule leaves reading A-10 as it was: acc = 0 gives u = 0, not NaN."""
    q, k, v = _inputs(T=70)
    v[:] = 0.0
    out = _run(q, k, v)
    assert np.all(out["direction"] == 0.0) and np.isfinite(out["n_eff"]).all()

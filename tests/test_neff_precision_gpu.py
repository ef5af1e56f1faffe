"""n_eff where bf16 weights would miss it: rows with one strong key and thousands of
identical weak keys whose weights round to bf16 in opposite directions
(polar_inputs.rounding_adversary_qkv; tests/test_rounding_inputs.py shows that sums of
bf16-rounded weights leave the 1e-2 tolerance on these rows).  The prefill forms S1 and
S2 from its fp32 weights, so n_eff = S1^2 / S2 [ATMA §2.1] must hold to fp32 accuracy:
every row is compared with the oracle within the bf16 tolerances, and n_eff and the
statistics within 1e-4 besides.  Checked on the call the benchmark times (no
statistics, outputs allocated by the caller), on the call with statistics, and on a
prefill split into two partial forwards and merged."""
import numpy as np
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import polar_attention
from tests.parity import assert_parity, errors, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
T = 8192
NEFF_TIGHT = 1.0e-4


@pytest.mark.parametrize("d", [64, 128])
def test_neff_rounding_rows(d):
    q, k, v = pin.rounding_adversary_qkv(T, d, seed=3 + d)
    H = q.shape[1]
    beta = [0.0] * H
    print(f"[neff] rounding rows T={T} d={d}", flush=True)
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, null_bias=beta)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    timed = pa.fwd(qd, kd, vd, out=pa.allocate_outputs(1, H, T, d, qd.device), causal=True, null_bias=beta)
    with_stats = pa.fwd(qd, kd, vd, causal=True, null_bias=beta, stats=True)
    # two partial forwards over keys [0, T/2) and [T/2, T) for the rows [T/2, T), merged
    c0 = T // 2
    qc = qd[:, :, c0:].contiguous()
    parts = pa.fwd_partial(qc, kd[:, :, :c0].contiguous(), vd[:, :, :c0].contiguous(), causal=False, context_k=T,
                           num_splits=2, split=0, null_bias=beta)
    parts = pa.fwd_partial(qc, kd[:, :, c0:].contiguous(), vd[:, :, c0:].contiguous(), causal=True, context_k=T,
                           partials=parts, num_splits=2, split=1, null_bias=beta)
    merged = pa.merge(parts, seq_k=T, causal=True, null_bias=beta, stats=True)
    torch.cuda.synchronize()
    e1 = assert_parity(timed, ref, "bf16", label=f"timed call d={d}")
    e2 = assert_parity(with_stats, ref, "bf16", label=f"statistics call d={d}")
    half = {key: val[:, :, c0:] for key, val in ref.items()}
    e3 = assert_parity(merged, half, "bf16", label=f"two partials merged d={d}")
    print(f"[neff] d={d}: timed {e1}; statistics {e2}; merged {e3}", flush=True)
    for e, name in ((e1, "timed"), (e2, "statistics"), (e3, "merged")):
        assert e["n_eff"] <= NEFF_TIGHT, f"{name} d={d}: n_eff {e['n_eff']:.3e}"
    for e in (e2, e3):
        assert e["s1"] <= NEFF_TIGHT and e["s2"] <= NEFF_TIGHT, e
    # the timed call and the statistics call agree bitwise on every channel
    for key in ("direction", "n_eff", "confidence", "count"):
        assert torch.equal(timed[key], with_stats[key]), key

"""GPU test of the no-allocation decode (polar_attn_decode_noalloc) through the C ABI.

The entry point runs the kernels of polar_attn_decode with the split partials in the
library's own per-GPU device array instead of a caller workspace, so its outputs must be
bitwise those of polar_attn_decode at the same split count.  Two calls in a row, the
second with a smaller problem, check that the array's leftover contents from the first
call never reach the second; a problem whose partials exceed the array is rejected.
"""
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import polar_attention
from tests.parity import assert_parity, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("direction", "n_eff", "confidence", "count")


def one_case(B, H, Hkv, Tk, d, seed, num_splits, kw):
    print(f"[noalloc] B={B} H={H} Hkv={Hkv} Tk={Tk} d={d} splits={num_splits}", flush=True)
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, Tk, d, torch.bfloat16, seed)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref = pa.decode(qd, kd, vd, num_splits=num_splits, **kw)
    out = pa.allocate_outputs(B, H, 1, d, DEV)
    got = pa.decode_noalloc(qd, kd, vd, out, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    assert got is out
    for key in KEYS:
        assert torch.equal(ref[key], got[key]), key
    assert_parity(got, polar_attention(to_np(q), to_np(k), to_np(v), causal=True, **kw), "bf16",
                  label=f"noalloc B={B} H={H} Tk={Tk}")
    return got


def test_noalloc_decode_matches_decode_twice():
    """A large call, then a smaller one (fewer rows, fewer splits, other head_dim): each
    bitwise equal to polar_attn_decode and within the tolerance of the oracle."""
    H = 8
    kw = dict(len_temp=[0.02 * h for h in range(H)], null_bias=[0.0] * H)
    one_case(4, H, H, 3001, 128, 401, 0, kw)
    kw2 = dict(len_temp=[0.1, 0.0, 0.05, 0.2], null_bias=[0.5, 0.0, -1.0, 0.0])
    one_case(2, 4, 4, 700, 64, 402, 3, kw2)


def test_noalloc_grouped_decode():
    """Query heads sharing KV heads: the grouped kernel writes the partials."""
    kw = dict(null_bias=[0.0] * 8)
    one_case(3, 8, 2, 1500, 128, 403, 0, kw)
    one_case(1, 8, 2, 200, 128, 404, 2, kw)


def test_noalloc_rejects_partials_beyond_the_array():
    """64 sequences x 8 heads x 64 splits x 131 floats = 17 MB > 8 MiB: rejected before any
    launch, and the outputs are left untouched."""
    B, H, Tk, d = 64, 8, 64, 128
    q = torch.zeros(B, H, 1, d, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, H, Tk, d, dtype=torch.bfloat16, device=DEV)
    out = pa.allocate_outputs(B, H, 1, d, DEV)
    out["n_eff"].fill_(-7.0)
    with pytest.raises(pa.PolarArgumentError) as err:
        pa.decode_noalloc(q, k, k.clone(), out, num_splits=64)
    assert err.value.name == "POLAR_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.all(out["n_eff"] == -7.0)
    # the largest split count that fits still runs
    fits = pa.NOALLOC_SCRATCH_BYTES // (B * H * (d + 3) * 4)
    pa.decode_noalloc(q, k, k.clone(), out, num_splits=int(min(fits, Tk)))
    torch.cuda.synchronize()
    assert torch.all(out["n_eff"] == Tk)

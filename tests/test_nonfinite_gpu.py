"""Non-finite inputs on the GPU: the policy of include/polar_attn.h, which the oracle
follows too (tests/test_nonfinite.py).  A NaN in q_i makes every channel of row i NaN; a
NaN in k_j every channel of the rows that see key j; a NaN in v_j the direction of the
rows that see key j (and possibly of earlier rows of the same query tile), with n_eff,
confidence and count unchanged.  In the statistics S1 and S2 follow the channels and the
maximum m is unspecified.  Every other row is bitwise what it is without the NaN."""
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHANNELS = ("direction", "n_eff", "confidence", "count")
MAGNITUDES = ("n_eff", "confidence", "count")
KW = dict(len_temp=[0.1, 0.0], null_bias=[0.0, 0.5])


def _fwd(q, k, v, stats, causal=True):
    out = pa.fwd(q, k, v, causal=causal, stats=stats, **KW)
    torch.cuda.synchronize()
    return out


def _keys(stats):
    return CHANNELS + (("stats",) if stats else ())


def _all_nan(out, h, rows, keys):
    # in the statistics the sums S1, S2 are NaN; the maximum m is left unspecified
    return all(torch.isnan(out[c][0, h, rows][..., 1:] if c == "stats" else out[c][0, h, rows]).all().item()
               for c in keys)


def _same(a, b, h, rows, keys):
    return all(torch.equal(a[c][0, h, rows], b[c][0, h, rows]) for c in keys)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("stats", [False, True])
def test_nan_inputs_prefill(dtype, d, stats):
    T = 1100
    q, k, v, _ = pin.random_qkv(1, 2, 2, T, T, d, dtype, 600 + d)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    keys = _keys(stats)
    clean = _fwd(q, k, v, stats)
    for name in CHANNELS:
        assert torch.isfinite(clean[name]).all()
    # a query row
    qn = q.clone()
    qn[0, 1, 123, 17] = float("nan")
    out = _fwd(qn, k, v, stats)
    assert _all_nan(out, 1, [123], keys)
    others = [i for i in range(T) if i != 123]
    assert _same(out, clean, 1, others, keys) and _same(out, clean, 0, slice(None), keys)
    # a key: the rows that see it, with and without the causal mask
    kn = k.clone()
    kn[0, 0, 700, 5] = float("nan")
    out = _fwd(q, kn, v, stats)
    assert _all_nan(out, 0, slice(700, None), keys)
    assert _same(out, clean, 0, slice(0, 700), keys) and _same(out, clean, 1, slice(None), keys)
    out = _fwd(q, kn, v, stats, causal=False)
    assert _all_nan(out, 0, slice(None), keys)
    # a value: the direction of the rows that see it; the magnitudes nowhere
    vn = v.clone()
    vn[0, 0, 1000, 7] = float("nan")
    out = _fwd(q, k, vn, stats)
    assert _all_nan(out, 0, slice(1000, None), ("direction",))
    assert _same(out, clean, 0, slice(None), MAGNITUDES + (("stats",) if stats else ()))
    assert _same(out, clean, 0, slice(0, 512), keys) and _same(out, clean, 1, slice(None), keys)


def test_nan_inputs_decode():
    """A NaN in one sequence's cache reaches the rows of that sequence and KV head only."""
    B, H, Hkv, Tk, d = 3, 4, 2, 1000, 128
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, Tk, d, torch.bfloat16, 640)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    kw = dict(num_splits=4, null_bias=[0.0] * H, stats=True)
    clean = pa.decode(q, k, v, **kw)
    for which in ("k", "v"):
        kn, vn = k.clone(), v.clone()
        (kn if which == "k" else vn)[1, 0, 500, 3] = float("nan")
        out = pa.decode(q, kn, vn, **kw)
        torch.cuda.synchronize()
        hit = CHANNELS + ("stats",) if which == "k" else ("direction",)
        for c in hit:  # query heads 0, 1 read KV head 0
            x = out[c][1, 0:2][..., 1:] if c == "stats" else out[c][1, 0:2]
            assert torch.isnan(x).all(), (which, c)
        for c in CHANNELS + ("stats",):
            assert torch.equal(out[c][1, 2:], clean[c][1, 2:]), (which, c)
            assert torch.equal(out[c][0], clean[c][0]) and torch.equal(out[c][2], clean[c][2]), (which, c)
            if c not in hit:
                assert torch.equal(out[c][1], clean[c][1]), (which, c)

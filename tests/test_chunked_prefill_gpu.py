"""Chunked prefill: a query chunk's statistics over a cached prefix (no mask) and over
the chunk itself (causal mask) are computed by separate partial forwards and merged;
the result must be the forward over the whole context, which the oracle computes.
The length temperature of every row uses its count in the whole context, which is what
makes the pieces agree with one pass."""
import numpy as np
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import polar_attention
from tests.parity import TOL, assert_parity, errors, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def chunked_case(B, H, Hkv, T, c0, cuts, d, dtype, seed, tau=None, beta=None, kappa=None):
    """Rows [c0, T) against keys [0, T): prefix pieces split at `cuts` (within [0, c0)),
    then the chunk [c0, T) with the causal mask."""
    q, k, v, _ = pin.random_qkv(B, H, Hkv, T, T, d, dtype, seed)
    kind = "f32" if dtype == torch.float32 else "bf16"
    rows = np.arange(c0, T)
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, len_temp=tau, null_bias=beta,
                          count_scale=kappa, rows=rows)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    qc = qd[:, :, c0:].contiguous()
    edges = [0] + list(cuts) + [c0]
    pieces = [(a, b, False) for a, b in zip(edges[:-1], edges[1:]) if b > a] + [(c0, T, True)]
    S = len(pieces) + 1  # one slot left empty on purpose (m = -inf)
    parts = None
    for s, (a, b, causal) in enumerate(pieces):
        parts = pa.fwd_partial(qc, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), causal=causal,
                               context_k=T, partials=parts, num_splits=S, split=s, len_temp=tau, null_bias=beta,
                               count_scale=kappa)
    out = pa.merge(parts, seq_k=T, causal=True, len_temp=tau, null_bias=beta, count_scale=kappa, stats=True)
    full = pa.fwd(qd, kd, vd, causal=True, len_temp=tau, null_bias=beta, count_scale=kappa)
    torch.cuda.synchronize()
    label = f"chunked T={T} c0={c0} cuts={cuts} d={d} {kind}"
    e = assert_parity(out, {key: val for key, val in ref.items()}, kind, label=label)
    # and the same as the one-pass forward on those rows, within the same tolerance
    channels = ("direction", "n_eff", "confidence", "count")
    assert_parity({key: out[key] for key in channels}, {key: to_np(full[key][:, :, c0:]) for key in channels}, kind,
                  label=label + " vs one pass")
    return e


@pytest.mark.parametrize("d", [64, 128])
def test_chunked_prefill_bf16(d):
    chunked_case(2, 4, 2, 1000, 600, [250], d, torch.bfloat16, 500 + d,
                 tau=[0.0, 0.1, 0.3, 0.05], beta=[0.0, 1.0, -1.0, 0.0], kappa=[1.0, 2.0, 1.0, 4.0])


def test_chunked_prefill_fp32_and_single_row_chunk():
    chunked_case(1, 2, 2, 300, 200, [64, 65], 64, torch.float32, 511, tau=[0.2, 0.0], beta=[0.0, 0.0])
    # a chunk of one row is a decode step over the cached prefix
    chunked_case(1, 2, 2, 257, 256, [100], 128, torch.bfloat16, 512, tau=[0.1, 0.0], beta=[0.0, 2.0])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,T,chunk", [(1, 4, 2500, 1024), (2, 2, 3000, 700)])
def test_chunked_over_cache_every_row(d, B, H, T, chunk):
    """Chunks as single forwards over the cache up to their last row (seq_q = chunk rows <
    seq_k, causal aligned to the end of the keys), two query heads per KV head: every row of
    every chunk against the oracle's forward over the whole context."""
    tau = [0.1 * (h + 1) for h in range(H)]
    q, k, v, _ = pin.random_qkv(B, H, H // 2, T, T, d, torch.bfloat16, 530 + d + chunk)  # GQA: 2 per KV head
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, len_temp=tau)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        out = pa.fwd(qd[:, :, c0:c1].contiguous(), kd[:, :, :c1].contiguous(), vd[:, :, :c1].contiguous(),
                     causal=True, len_temp=tau, stats=True)
        torch.cuda.synchronize()
        sub = {key: (val[:, :, c0:c1] if val is not None and val.ndim >= 3 else val) for key, val in ref.items()}
        assert_parity(out, sub, "bf16", label=f"over cache B={B} H={H} T={T} d={d} rows [{c0}, {c1})")


def test_partial_writes_only_its_slot():
    q, k, v, _ = pin.random_qkv(1, 2, 2, 70, 70, 64, torch.bfloat16, 513)
    parts = torch.full((1, 2, 70, 3, 67), 7.0, device=DEV)
    pa.fwd_partial(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, partials=parts, num_splits=3, split=1)
    torch.cuda.synchronize()
    assert torch.all(parts[:, :, :, 0] == 7.0) and torch.all(parts[:, :, :, 2] == 7.0)
    assert torch.isfinite(parts[:, :, :, 1]).all()


def test_workload_chunked_prefill_t65536():
    """The benchmark's chunked prefill of the T=65536 d=64 workload (8 chunks of 8192
    queries, each over its cached prefix and itself, merged) at full size: sampled rows of
    every chunk and head against the oracle within the bf16 tolerance, and every row
    against the one-pass forward, which is itself within that tolerance of the oracle on
    every row: two such results differ by at most twice the tolerance (their bf16 weights
    are rounded against different reference maxima)."""
    import bench
    w = pin.WORKLOADS["bf16_b1_h16_t65536_d64_lentemp"]
    print(f"[chunked] workload {w.name} in chunks of {bench.CHUNK}", flush=True)
    q, k, v, _ = pin.workload_inputs(w, "cpu")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    run, outs = bench.chunked_prefill_plan(pa, torch, qd, kd, vd, w, bench.CHUNK, keep_outputs=True)
    run()
    kw = dict(len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    full = pa.fwd(qd, kd, vd, causal=True, **kw)
    torch.cuda.synchronize()
    channels = ("direction", "n_eff", "confidence", "count")
    r = np.random.default_rng(90)
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    for c0, o in outs:
        c1 = c0 + o["n_eff"].shape[2]
        e = errors({key: o[key] for key in channels}, {key: to_np(full[key][:, :, c0:c1]) for key in channels})
        for key in channels:
            assert e[key] <= 2 * TOL["bf16"][key], f"chunk [{c0}, {c1}) vs one pass {key}: {e}"
        rows = np.unique(np.concatenate([[c0, c1 - 1], r.integers(c0, c1, 4)]))
        ref = polar_attention(qn, kn, vn, causal=True, rows=rows, **kw)
        sel = torch.as_tensor(rows - c0, device=DEV)
        sub = {key: o[key][:, :, sel] for key in channels}
        e2 = assert_parity(sub, {key: ref[key] for key in channels}, "bf16", label=f"chunk [{c0}, {c1}) vs oracle")
        print(f"[chunked] rows [{c0}, {c1}): vs one pass {e}; sampled rows vs oracle {e2}", flush=True)


def test_workload_chunked_prefill_over_cache_t65536():
    """The benchmark's second chunked plan of the T=65536 d=64 workload (8 chunks of 8192
    queries, each one forward over the cache up to its last row) at full size: sampled
    rows of every chunk and head against the oracle within the bf16 tolerance, and every
    row against the one-pass forward within twice that tolerance (both are within the
    tolerance of the oracle; their bf16 weights are rounded against different reference
    maxima)."""
    import bench
    w = pin.WORKLOADS["bf16_b1_h16_t65536_d64_lentemp"]
    print(f"[chunked over cache] workload {w.name} in chunks of {bench.CHUNK}", flush=True)
    q, k, v, _ = pin.workload_inputs(w, "cpu")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    run, outs = bench.chunked_over_cache_plan(pa, torch, qd, kd, vd, w, bench.CHUNK, keep_outputs=True)
    run()
    kw = dict(len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    full = pa.fwd(qd, kd, vd, causal=True, **kw)
    torch.cuda.synchronize()
    channels = ("direction", "n_eff", "confidence", "count")
    r = np.random.default_rng(91)
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    for c0, o in outs:
        c1 = c0 + o["n_eff"].shape[2]
        e = errors({key: o[key] for key in channels}, {key: to_np(full[key][:, :, c0:c1]) for key in channels})
        for key in channels:
            assert e[key] <= 2 * TOL["bf16"][key], f"chunk [{c0}, {c1}) vs one pass {key}: {e}"
        rows = np.unique(np.concatenate([[c0, c1 - 1], r.integers(c0, c1, 4)]))
        ref = polar_attention(qn, kn, vn, causal=True, rows=rows, **kw)
        sel = torch.as_tensor(rows - c0, device=DEV)
        sub = {key: o[key][:, :, sel] for key in channels}
        e2 = assert_parity(sub, {key: ref[key] for key in channels}, "bf16", label=f"chunk [{c0}, {c1}) vs oracle")
        print(f"[chunked over cache] rows [{c0}, {c1}): vs one pass {e}; sampled rows vs oracle {e2}", flush=True)

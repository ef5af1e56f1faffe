"""HIP graph capture of the library's calls, as a serving loop or a training step uses them.

Each call is captured once with torch.cuda.graph on static buffers, then the graph is
replayed several times with new inputs copied into those buffers between replays (eager
work and a synchronisation in between); every replay must give what the same call gives
eagerly on the same inputs, bitwise, since the same kernels run on the same data with no
atomics.  The library enqueues kernel launches only (no memset, copy or allocation), so
its calls are capturable as they are; the no-allocation decode looks its array up on its
first call, which the warm-up before capture makes.
"""
import pytest
import torch

import long_context_attention_polar_amd as pa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHANNELS = ("direction", "n_eff", "confidence", "count")
REPLAYS = 3


def _capture(fn):
    """Warm up on a side stream (as torch.cuda.graph asks), then capture one call of fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _refill(gen, *tensors):
    """New N(0,1) values (rounded to each tensor's dtype) copied into static buffers."""
    for t in tensors:
        t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))


def _static(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=DEV)


def _check_replays(graph, gen, inputs, captured_out, eager, label):
    for r in range(REPLAYS):
        _refill(gen, *inputs)
        graph.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        for key in CHANNELS:
            assert torch.equal(captured_out[key], ref[key]), f"{label}: replay {r}, {key}"


def test_graph_prefill():
    B, H, T, d = 1, 8, 1000, 64
    gen = torch.Generator().manual_seed(9101)
    q, k, v = _static((B, H, T, d)), _static((B, H, T, d)), _static((B, H, T, d))
    _refill(gen, q, k, v)
    kw = dict(causal=True, len_temp=[0.02 * h for h in range(H)], null_bias=[0.0] * H)
    out = pa.allocate_outputs(B, H, T, d, DEV)
    graph = _capture(lambda: pa.fwd(q, k, v, out=out, **kw))
    _check_replays(graph, gen, (q, k, v), out, lambda: pa.fwd(q, k, v, **kw), "prefill")


def test_graph_decode_with_workspace_and_merge():
    B, H, Hkv, Tk, d = 4, 8, 2, 3000, 128
    gen = torch.Generator().manual_seed(9102)
    q, k, v = _static((B, H, 1, d)), _static((B, Hkv, Tk, d)), _static((B, Hkv, Tk, d))
    _refill(gen, q, k, v)
    kw = dict(len_temp=[0.05] * H, null_bias=[0.0] * H)
    prob = pa.problem_for(q, k, causal=True, **kw)
    ws = torch.empty(max(16, pa.decode_workspace_bytes(prob, 0)), dtype=torch.uint8, device=DEV)
    out = pa.allocate_outputs(B, H, 1, d, DEV)
    assert pa.decode_num_splits(prob, 0) > 1  # the merge kernel is part of the graph
    graph = _capture(lambda: pa.decode(q, k, v, workspace=ws, out=out, **kw))
    _check_replays(graph, gen, (q, k, v), out, lambda: pa.decode(q, k, v, **kw), "decode")


@pytest.mark.parametrize("splits", [40, 100])
def test_graph_decode_parallel_merge(splits):
    """Explicit split counts past 16 and past 64: the merge runs over the splits in one
    wave's lanes, and in four waves, inside the graph."""
    B, H, Tk, d = 1, 8, 20000, 128
    gen = torch.Generator().manual_seed(9110 + splits)
    q, k, v = _static((B, H, 1, d)), _static((B, H, Tk, d)), _static((B, H, Tk, d))
    _refill(gen, q, k, v)
    kw = dict(len_temp=[0.05] * H, null_bias=[0.0] * H, num_splits=splits)
    prob = pa.problem_for(q, k, causal=True, len_temp=kw["len_temp"], null_bias=kw["null_bias"])
    assert pa.decode_num_splits(prob, splits) == splits
    ws = torch.empty(pa.decode_workspace_bytes(prob, splits), dtype=torch.uint8, device=DEV)
    out = pa.allocate_outputs(B, H, 1, d, DEV)
    graph = _capture(lambda: pa.decode(q, k, v, workspace=ws, out=out, **kw))
    _check_replays(graph, gen, (q, k, v), out, lambda: pa.decode(q, k, v, **kw), f"decode {splits} splits")


def test_graph_decode_noalloc():
    B, H, Hkv, Tk, d = 4, 8, 8, 2500, 64
    gen = torch.Generator().manual_seed(9103)
    q, k, v = _static((B, H, 1, d)), _static((B, Hkv, Tk, d)), _static((B, Hkv, Tk, d))
    _refill(gen, q, k, v)
    kw = dict(null_bias=[0.0] * H)
    out = pa.allocate_outputs(B, H, 1, d, DEV)
    graph = _capture(lambda: pa.decode_noalloc(q, k, v, out, **kw))
    _check_replays(graph, gen, (q, k, v), out, lambda: pa.decode(q, k, v, **kw), "decode_noalloc")


def test_graph_paged_grouped_decode():
    B, H, Hkv, d, bs, max_blocks = 3, 8, 2, 128, 64, 40
    gen = torch.Generator().manual_seed(9104)
    num_blocks = B * max_blocks
    q = _static((B, H, 1, d))
    k_pool, v_pool = _static((num_blocks, bs, Hkv, d)), _static((num_blocks, bs, Hkv, d))
    table = torch.randperm(num_blocks, generator=gen).to(torch.int32).reshape(B, max_blocks).to(DEV)
    lens = torch.tensor([2560, 1000, 77], dtype=torch.int32, device=DEV)
    _refill(gen, q, k_pool, v_pool)
    kw = dict(null_bias=[0.0] * H)
    kv = pa.paged_kv(k_pool, v_pool, table, lens)
    prob = pa.Problem(B, H, Hkv, 1, max_blocks * bs, d, False, pa.POLAR_BF16, 0.0, None, [0.0] * H, None, None)
    ws = torch.empty(max(16, pa.decode_paged_workspace_bytes(prob, kv, 0)), dtype=torch.uint8, device=DEV)
    out = pa.allocate_outputs(B, H, 1, d, DEV)
    graph = _capture(lambda: pa.decode_paged(q, k_pool, v_pool, table, lens, workspace=ws, out=out, **kw))
    _check_replays(graph, gen, (q, k_pool, v_pool), out,
                   lambda: pa.decode_paged(q, k_pool, v_pool, table, lens, **kw), "paged decode")


def test_graph_backward():
    B, H, Hkv, T, d = 1, 4, 2, 300, 128
    gen = torch.Generator().manual_seed(9105)
    q, k, v = _static((B, H, T, d)), _static((B, Hkv, T, d)), _static((B, Hkv, T, d))
    grads = {"direction": _static((B, H, T, d), torch.float32), "n_eff": _static((B, H, T), torch.float32)}
    _refill(gen, q, k, v, *grads.values())
    kw = dict(causal=True, null_bias=[0.0] * H)
    prob = pa.problem_for(q, k, **kw)
    ws = torch.empty(max(16, pa.bwd_workspace_bytes(prob)), dtype=torch.uint8, device=DEV)
    f32 = dict(device=DEV, dtype=torch.float32)
    out = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(k.shape, **f32), "dv": torch.empty(v.shape, **f32)}
    graph = _capture(lambda: pa.bwd(q, k, v, grads, workspace=ws, out=out, **kw))
    for r in range(REPLAYS):
        _refill(gen, q, k, v, *grads.values())
        graph.replay()
        torch.cuda.synchronize()
        ref = pa.bwd(q, k, v, grads, **kw)
        torch.cuda.synchronize()
        for key in ("dq", "dk", "dv"):
            assert torch.equal(out[key], ref[key]), f"backward: replay {r}, {key}"

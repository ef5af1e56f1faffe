#!/usr/bin/env python3
"""Benchmark of the Polar Attention hot path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic inputs that are
already resident in HBM:
  * fused prefill forward, bf16, B=1 H=16 T=16384 d=128, causal, planted match groups;
  * fused prefill forward, bf16, B=1 H=16 T=65536 d=64, causal, tau_h = 0.02 h
    (the longest context the ATMA summary evaluates, §3);
  * split-KV decode + merge, bf16, batch 64, H=8, d=128, one query against a
    65536-token KV cache;
  * grouped split-KV decode + merge over a paged cache, bf16, batch 64, 32 query heads
    over 8 KV heads, d=128, 65536 keys per sequence in shuffled 16-row blocks (reported
    beside the headline, not part of it);
  * backward (dq, dk, dv for upstream gradients of all four channels), bf16 inputs on the
    matrix cores, B=1, 16 query heads over 4 KV heads, T=16384, d=128, causal (reported
    beside the headline, not part of it, and timed in a loop of its own after the steps),
    once self-contained and once given the row statistics of the forward
    (polar_attn_bwd_saved), as a training step that keeps them runs it;
  * beside the headline, also in loops of their own: the B=4 H=8 T=4096 d=64 needle
    prefill, the T=65536 prefill as a chunked
    prefill (8 chunks of 8192 queries: partial forwards over the cached prefix and over
    the chunk, merged), and under two reading variants (a per-key soft floor; a sliding
    window of 4096 keys), and the decode latency at batch 1 (the first sequence of the
    decode cache alone).
`value` is the prefill throughput in TFLOP/s: the algorithmic flops of the two prefill
launches (4 d per computed causal (query, key) pair) over their HIP-event time.  The
decode bandwidth is reported beside it.  Per-launch durations come from HIP events
recorded on the stream the kernels run on (torch's current stream, which the library
launches on).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Polar-attn fwd TFLOP/s + % bf16 MFMA peak at T=16K/64K; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PREFILL = ["bf16_b1_h16_t16384_d128_groups", "bf16_b1_h16_t65536_d64_lentemp"]
DECODE = "bf16_decode_b64_h8_tk65536_d128"
PAGED = "bf16_paged_decode_b64_h32_kv8_tk65536_d128"
DECODE_B1 = "bf16_decode_b1_h8_tk65536_d128"
BWD = "bf16_bwd_b1_h16_kv4_t16384_d128"
BWD_SAVED = BWD + "_saved"
CHUNK = 8192
CHUNKED = f"bf16_chunked_prefill_b1_h16_t65536_d64_chunk{CHUNK}"
CHUNKED_CACHE = f"bf16_chunked_prefill_over_cache_b1_h16_t65536_d64_chunk{CHUNK}"
SOFT_FLOOR = "bf16_b1_h16_t65536_d64_soft_key_floor"
WIN = 4096
NEEDLE = "bf16_b4_h8_t4096_d64_needle"
FP32_SMALL = "fp32_b1_h2_t256_d64"
WINDOW = f"bf16_b1_h16_t65536_d64_window{WIN}"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


# Sources each profiled kernel is built from (besides the shared header, the ABI header
# and the launch-geometry constants of the host file), and the kernel's name, whose
# template arguments in the host file's dispatch lines are part of its build.
KERNEL_SOURCES = {
    "fwd_bf16_t65536_d64": (["fwd_bf16_pipe.h", "fwd_bf16.h"], "polar_fwd_bf16_pipe_kernel"),
    "fwd_bf16_t16384_d128": (["fwd_bf16_pipe.h", "fwd_bf16.h"], "polar_fwd_bf16_pipe_kernel"),
    "fwd_bf16_needle_b4_h8_t4096_d64": (["fwd_bf16_pipe.h", "fwd_bf16.h"], "polar_fwd_bf16_pipe_kernel"),
    "fwd_f32_b1_h2_t256_d64": (["fwd_f32.h"], "polar_fwd_f32_kernel"),
    "decode_b64_h8_tk65536_d128": (["decode.h"], "polar_decode_split_kernel"),
    "merge_b64_h8_d128": (["decode.h"], "polar_merge_few_kernel"),
    "decode_b1_h8_tk65536_d128": (["decode.h"], "polar_decode_split_kernel"),
    "merge_b1_h8_d128": (["decode.h"], "polar_merge_kernel"),
    "paged_gqa_decode_b64_h32_kv8_tk65536_d128": (["decode_group.h", "decode.h"], "polar_decode_group_kernel"),
    "bwd_dq_b1_h16_kv4_t16384_d128": (["bwd_mfma.h", "bwd.h", "fwd_bf16.h"], "polar_bwd_dq_mfma_kernel"),
    "bwd_dkdv_b1_h16_kv4_t16384_d128": (["bwd_mfma.h", "bwd.h", "fwd_bf16.h"], "polar_bwd_dkdv_mfma_kernel"),
    "bwd_split_sum_b1_h16_kv4_t16384_d128": (["bwd_mfma.h", "bwd.h", "fwd_bf16.h"], "polar_bwd_split_sum_kernel"),
}


def _code(text):
    """Source text without comments and blank space, so that edits of the documentation
    leave a digest unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel_key=None):
    """Digest of the code a kernel is built from: its headers, polar_common.h, the ABI
    header, the launch-geometry lines of polar_attn.hip and its lines that name the kernel
    (all of csrc/ when no kernel is named), comments excluded.  A profile stays valid
    while this digest is unchanged."""
    csrc = os.path.join(ROOT, "long_context_attention_polar_amd", "csrc")
    h = hashlib.sha256()
    if kernel_key is None:
        names = sorted(os.listdir(csrc))
    else:
        headers, kernel = KERNEL_SOURCES[kernel_key]
        names = sorted(set(headers) | {"polar_common.h"})
    for name in names:
        with open(os.path.join(csrc, name)) as f:
            h.update((name + _code(f.read())).encode())
    if kernel_key is not None:
        with open(os.path.join(ROOT, "include", "polar_attn.h")) as f:
            h.update(_code(f.read()).encode())
        with open(os.path.join(csrc, "polar_attn.hip")) as f:
            host = [ln for ln in _code_lines(f.read())
                    if ln.startswith(("constexpr int k", "#define POLAR_")) or kernel in ln]
        h.update("\n".join(host).encode())
    return h.hexdigest()[:16]


def _code_lines(text):
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return [" ".join(re.sub(r"//.*", "", ln).split()) for ln in text.split("\n")]


def prefill_flops(w):
    return 4 * w.d * w.pairs()


def window_pairs(T, W):
    """(query, key) pairs of a causal prefill whose rows see at most their last W keys."""
    W = min(W, T)
    return W * (W + 1) // 2 + (T - W) * W


def chunked_prefill_plan(pa, torch, q, k, v, w, chunk, keep_outputs=False):
    """A causal prefill in chunks of `chunk` queries, as a serving engine runs it: each
    chunk's rows take a partial forward over the cached keys before the chunk (no mask)
    and one over the chunk's own keys (causal), each with the length temperature of the
    row's count in the whole context, and polar_attn_merge combines the two.  The cached
    prefixes and the chunk slices are laid out once, outside the timed calls.  Returns the
    callable that runs every chunk, writing each chunk's channels into one buffer, or with
    keep_outputs also the list of (first row, outputs) of every chunk, each its own."""
    B, H, T, d = q.shape
    kw = dict(len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    out = pa.allocate_outputs(B, H, chunk, d, q.device)
    steps = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        S = 2 if c0 else 1
        parts = torch.empty(B, H, c1 - c0, S, d + 3, dtype=torch.float32, device=q.device)
        pre = (k[:, :, :c0].contiguous(), v[:, :, :c0].contiguous()) if c0 else None
        own = keep_outputs or c1 - c0 != chunk
        steps.append((c1, q[:, :, c0:c1].contiguous(), k[:, :, c0:c1].contiguous(), v[:, :, c0:c1].contiguous(),
                      pre, S, parts, pa.allocate_outputs(B, H, c1 - c0, d, q.device) if own else out))

    def run():
        for c1, qc, kc, vc, pre, S, parts, o in steps:
            if pre is not None:
                pa.fwd_partial(qc, pre[0], pre[1], causal=False, context_k=c1, partials=parts, num_splits=S,
                               split=0, **kw)
            pa.fwd_partial(qc, kc, vc, causal=True, context_k=c1, partials=parts, num_splits=S, split=S - 1, **kw)
            pa.merge(parts, seq_k=c1, causal=True, out=o, **kw)
    if keep_outputs:
        return run, [(c1 - len_q, o) for c1, qc, kc, vc, pre, S, parts, o in steps for len_q in [qc.shape[2]]]
    return run


def chunked_over_cache_plan(pa, torch, q, k, v, w, chunk, keep_outputs=False):
    """The same causal prefill in chunks of `chunk` queries, each chunk one polar_attn_fwd
    call whose keys are the whole cache up to the chunk's end (the prefix and the chunk's
    own keys, appended): seq_q = chunk rows < seq_k = the chunk's last row + 1, causal
    aligned to the end of the keys, so a row's visible count is its count in the whole
    context.  The per-chunk caches are laid out once, outside the timed calls.  Returns
    the callable that runs every chunk, or with keep_outputs also the list of (first row,
    outputs) of every chunk."""
    B, H, T, d = q.shape
    kw = dict(causal=True, len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    steps = []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        steps.append((c0, q[:, :, c0:c1].contiguous(), k[:, :, :c1].contiguous(), v[:, :, :c1].contiguous(),
                      pa.allocate_outputs(B, H, c1 - c0, d, q.device)))

    def run():
        for c0, qc, kc, vc, o in steps:
            pa.fwd(qc, kc, vc, out=o, **kw)
    if keep_outputs:
        return run, [(c0, o) for c0, qc, kc, vc, o in steps]
    return run


def backward_flops(w):
    """Algorithmic flops of the backward: 10 d per computed (query, key) pair -- the
    scores, <w, v_j>, and the three products into dq, dk and dv (2 d each)."""
    return 10 * w.d * w.pairs()


def decode_bytes(w):
    """Algorithmic bytes: K and V once per (sequence, KV head), q and the outputs."""
    kv = 2 * w.B * w.Hkv * w.Tk * w.d * 2
    q = w.B * w.H * w.d * 2
    outs = w.B * w.H * (w.d + 3) * 4   # direction, n_eff, confidence, count... (+ stats not requested)
    return kv + q + outs


def profiled(kernel_key, field):
    """A figure of the committed rocprofv3 counter digest (HBM bytes per launch, MFMA busy
    fraction, clock, ...), or None when the kernel's sources changed since the counters
    were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(kernel_key)
    if not entry or entry.get("source_digest") != source_digest(kernel_key):
        return None
    return entry.get(field)


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed PMC digest (None when out of date)."""
    return profiled(kernel_key, "hbm_bytes_per_launch")


def _oracle_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])


def cpu_baseline(seconds):
    """The fp64 oracle, as it is, on a bounded sample of the 16K prefill workload: whole
    heads, each in blocks of 512 query rows, until about `seconds` of wall time have
    passed (the rate is taken over the blocks done)."""
    import numpy as np
    import torch

    import polar_inputs as pin
    from oracle import polar_attention

    w = pin.WORKLOADS[PREFILL[0]]
    q, k, v, _ = pin.workload_inputs(w, "cpu")
    rows_done, heads_done, pairs, dt = 0, 0, 0, 0.0
    for h in range(w.H):
        qh = q[:, h:h + 1].float().numpy().astype(np.float64)
        kh = k[:, h:h + 1].float().numpy().astype(np.float64)
        vh = v[:, h:h + 1].float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        for end in range(w.Tq, 0, -512):
            rows = np.arange(max(0, end - 512), end)
            polar_attention(qh, kh, vh, causal=True, len_temp=w.len_temp()[h:h + 1],
                            null_bias=w.null_bias()[h:h + 1], count_scale=w.count_scale()[h:h + 1], rows=rows)
            pairs += int((rows + 1).sum())
            rows_done += len(rows)
        dt += time.perf_counter() - t0
        heads_done += 1
        if dt >= seconds:
            break
    threads = _oracle_threads()
    return {"value": 4 * w.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 NumPy oracle on {heads_done} of {w.H} heads ({rows_done} query rows, {pairs} causal "
                      f"(query,key) pairs) of the T=16384 d=128 prefill, {dt:.1f} s; host os.cpu_count()="
                      f"{os.cpu_count()}, BLAS threads={threads}, torch threads={torch.get_num_threads()}",
            "_pairs": pairs, "_seconds": dt}


def oracle_per_config(prefill16k_sample, gpu_ms, decode_inputs):
    """The fp64 oracle timed on every configuration: whole for the two small ones, on a
    bounded sample for the others, scaled to the whole configuration by its (query, key)
    pairs (the oracle's work is proportional to them: one row block costs its rows times
    its visible keys).  `prefill16k_sample` is the 16K prefill sample of cpu_baseline; the decode
    sample takes a few (sequence, head) slices copied from the device-resident cache."""
    import numpy as np

    import polar_inputs as pin
    from oracle import polar_attention

    def run(w, q, k, v, h0, h1, rows=None, b0=0, b1=None):
        b1 = w.B if b1 is None else b1
        q = q[b0:b1, h0:h1].float().numpy().astype(np.float64)
        kv = (h0 // (w.H // w.Hkv), (h1 - 1) // (w.H // w.Hkv) + 1)
        k = k[b0:b1, kv[0]:kv[1]].float().numpy().astype(np.float64)
        v = v[b0:b1, kv[0]:kv[1]].float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        polar_attention(q, k, v, causal=w.causal, len_temp=w.len_temp()[h0:h1],
                        null_bias=None if w.null_bias() is None else w.null_bias()[h0:h1],
                        count_scale=w.count_scale()[h0:h1], rows=rows)
        return time.perf_counter() - t0

    out = []

    def entry(name, sample, pairs_done, secs):
        w = pin.WORKLOADS[name]
        full = secs * w.pairs() / pairs_done
        e = {"workload": name, "sample": sample, "sample_s": round(secs, 3),
             "oracle_s_full": round(full, 3), "extrapolated": pairs_done != w.pairs()}
        if gpu_ms.get(name):
            e["gpu_ms"] = gpu_ms[name]
            e["oracle_over_gpu"] = round(full * 1e3 / gpu_ms[name], 1)
        out.append(e)

    for name in (FP32_SMALL, NEEDLE):
        w = pin.WORKLOADS[name]
        q, k, v, _ = pin.workload_inputs(w, "cpu")
        entry(name, "every row", w.pairs(), run(w, q, k, v, 0, w.H))
    entry(PREFILL[0], prefill16k_sample["sample"], prefill16k_sample["_pairs"], prefill16k_sample["_seconds"])
    # 64K prefill: blocks of 512 rows at four places along the sequence, in two heads
    w = pin.WORKLOADS[PREFILL[1]]
    q, k, v, _ = pin.workload_inputs(w, "cpu")
    secs, pairs = 0.0, 0
    for h in (0, w.H - 1):
        for end in (w.Tq // 4, w.Tq // 2, 3 * w.Tq // 4, w.Tq):
            rows = np.arange(end - 512, end)
            secs += run(w, q, k, v, h, h + 1, rows=rows)
            pairs += int((rows + 1).sum())
    entry(PREFILL[1], "rows [T/4-512, T/4), [T/2-512, T/2), [3T/4-512, 3T/4), [T-512, T) of heads 0 and 15",
          pairs, secs)
    # decode: four (sequence, head) slices of the 64K cache
    w = pin.WORKLOADS[DECODE]
    qd, kd, vd = decode_inputs
    secs, pairs = 0.0, 0
    for b, h in ((0, 0), (21, 3), (42, 5), (63, 7)):
        secs += run(w, qd[b:b + 1].cpu(), kd[b:b + 1].cpu(), vd[b:b + 1].cpu(), h, h + 1)
        pairs += w.Tk
    entry(DECODE, "4 of the 512 (sequence, head) rows: (0,0), (21,3), (42,5), (63,7)", pairs, secs)
    return out


def _percentile(sorted_ms, pct):
    """Linear-interpolated percentile of an ascending list."""
    x = (len(sorted_ms) - 1) * pct / 100.0
    i = int(x)
    j = min(i + 1, len(sorted_ms) - 1)
    return sorted_ms[i] + (sorted_ms[j] - sorted_ms[i]) * (x - i)


def rocm_version():
    """ROCm release of the installation, and the HIP version torch was built with."""
    ver = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                ver = f.read().strip()
            break
        except OSError:
            pass
    import torch
    return {"rocm": ver, "torch_hip": torch.version.hip, "torch": torch.__version__}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (prefill would shard by head, "
              "decode by KV range combined with the split merge). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_attention_polar_amd as pa
    import polar_inputs as pin

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()
    print(f"[bench] device {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    parts = []
    resident = {}
    for name in PREFILL:
        w = pin.WORKLOADS[name]
        q, k, v, _ = pin.workload_inputs(w, dev)
        resident[name] = (q, k, v)
        out = pa.allocate_outputs(w.B, w.H, w.Tq, w.d, dev)
        kw = dict(causal=w.causal, len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
        parts.append(dict(name=name, w=w, kind="prefill", flops=prefill_flops(w),
                          run=lambda q=q, k=k, v=v, out=out, kw=kw: pa.fwd(q, k, v, out=out, **kw)))
    # beside the headline, each timed in a loop of its own after the steps: the T=65536
    # prefill as a chunked prefill, and under two reading variants
    wl = pin.WORKLOADS[PREFILL[1]]
    ql, kl, vl = resident[PREFILL[1]]
    chunked = chunked_prefill_plan(pa, torch, ql, kl, vl, wl, CHUNK)
    parts.append(dict(name=CHUNKED, w=wl, kind="side", flops=prefill_flops(wl), headline=False, separate=True,
                      run=chunked))
    parts.append(dict(name=CHUNKED_CACHE, w=wl, kind="side", flops=prefill_flops(wl), headline=False,
                      separate=True, run=chunked_over_cache_plan(pa, torch, ql, kl, vl, wl, CHUNK)))
    outl = pa.allocate_outputs(wl.B, wl.H, wl.Tq, wl.d, dev)
    kwl = dict(causal=True, len_temp=wl.len_temp(), null_bias=wl.null_bias(), count_scale=wl.count_scale())
    parts.append(dict(name=SOFT_FLOOR, w=wl, kind="side", flops=prefill_flops(wl), headline=False, separate=True,
                      run=lambda: pa.fwd(ql, kl, vl, out=outl, variant={"key_floor": "soft"}, **kwl)))
    # the needle workload (B=4, H=8, T=4096, d=64): throughput reported, no peak target
    wn = pin.WORKLOADS[NEEDLE]
    qn, kn, vn, _ = pin.workload_inputs(wn, dev)
    outn = pa.allocate_outputs(wn.B, wn.H, wn.Tq, wn.d, dev)
    kwn = dict(causal=True, len_temp=wn.len_temp(), null_bias=wn.null_bias(), count_scale=wn.count_scale())
    parts.append(dict(name=NEEDLE, w=wn, kind="side", flops=prefill_flops(wn), headline=False, separate=True,
                      run=lambda: pa.fwd(qn, kn, vn, out=outn, **kwn)))
    # the fp32 workload (B=1, H=2, T=256, d=64): launch-bound, correctness path
    w1 = pin.WORKLOADS[FP32_SMALL]
    q1, k1, v1, _ = pin.workload_inputs(w1, dev)
    out1 = pa.allocate_outputs(w1.B, w1.H, w1.Tq, w1.d, dev)
    kw1 = dict(causal=True, len_temp=w1.len_temp(), null_bias=w1.null_bias(), count_scale=w1.count_scale())
    parts.append(dict(name=FP32_SMALL, w=w1, kind="side", flops=prefill_flops(w1), headline=False, separate=True,
                      run=lambda: pa.fwd(q1, k1, v1, out=out1, **kw1)))
    parts.append(dict(name=WINDOW, w=wl, kind="side", flops=4 * wl.d * wl.B * wl.H * window_pairs(wl.Tq, WIN),
                      headline=False, separate=True,
                      run=lambda: pa.fwd(ql, kl, vl, out=outl, variant={"window": WIN}, **kwl)))
    wd = pin.WORKLOADS[DECODE]
    qd, kd, vd, _ = pin.workload_inputs(wd, dev)
    prob = pa.problem_for(qd, kd, causal=True, len_temp=wd.len_temp(), null_bias=wd.null_bias(),
                          count_scale=wd.count_scale())
    splits = pa.decode_num_splits(prob, 0)
    ws = torch.empty(pa.decode_workspace_bytes(prob, 0), dtype=torch.uint8, device=dev)
    outd = pa.allocate_outputs(wd.B, wd.H, 1, wd.d, dev)
    kwd = dict(len_temp=wd.len_temp(), null_bias=wd.null_bias(), count_scale=wd.count_scale())
    parts.append(dict(name=DECODE, w=wd, kind="decode", bytes=decode_bytes(wd),
                      run=lambda: pa.decode(qd, kd, vd, workspace=ws, out=outd, **kwd)))
    # decode latency at batch 1: the first sequence of the same cache, automatic splits,
    # timed in a loop of its own
    w1b = dataclasses.replace(wd, B=1)
    q1b, k1b, v1b = qd[:1], kd[:1], vd[:1]
    prob1b = pa.problem_for(q1b, k1b, causal=True, len_temp=wd.len_temp(), null_bias=wd.null_bias(),
                            count_scale=wd.count_scale())
    splits1b = pa.decode_num_splits(prob1b, 0)
    ws1b = torch.empty(pa.decode_workspace_bytes(prob1b, 0), dtype=torch.uint8, device=dev)
    out1b = pa.allocate_outputs(1, wd.H, 1, wd.d, dev)
    parts.append(dict(name=DECODE_B1, w=w1b, kind="decode", bytes=decode_bytes(w1b), headline=False, separate=True,
                      run=lambda: pa.decode(q1b, k1b, v1b, workspace=ws1b, out=out1b, **kwd)))
    wp = pin.WORKLOADS[PAGED]
    qp, kpool, vpool, table, lens = pin.paged_decode_inputs(wp, dev)
    probp = pa.Problem(wp.B, wp.H, wp.Hkv, 1, wp.Tk, wp.d, False, pa.POLAR_BF16)
    need = pa.decode_paged_workspace_bytes(probp, pa.paged_kv(kpool, vpool, table, lens))
    wsp = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    outp = pa.allocate_outputs(wp.B, wp.H, 1, wp.d, dev)
    kwp = dict(seq_k=wp.Tk, len_temp=wp.len_temp(), null_bias=wp.null_bias(), count_scale=wp.count_scale())
    parts.append(dict(name=PAGED, w=wp, kind="decode", bytes=decode_bytes(wp), headline=False,
                      run=lambda: pa.decode_paged(qp, kpool, vpool, table, lens, workspace=wsp, out=outp, **kwp)))
    wb = pin.WORKLOADS[BWD]
    qb, kb, vb, _ = pin.workload_inputs(wb, dev)
    grb = {n: t.to(dev) for n, t in pin.random_grads(wb.B, wb.H, wb.Tq, wb.d, wb.extra["grad_seed"]).items()}
    probb = pa.problem_for(qb, kb, causal=True, len_temp=wb.len_temp(), null_bias=wb.null_bias(),
                           count_scale=wb.count_scale())
    wsb = torch.empty(pa.bwd_workspace_bytes(probb), dtype=torch.uint8, device=dev)
    f32 = dict(device=dev, dtype=torch.float32)
    outb = {"dq": torch.empty(qb.shape, **f32), "dk": torch.empty(kb.shape, **f32), "dv": torch.empty(vb.shape, **f32)}
    kwb = dict(causal=True, len_temp=wb.len_temp(), null_bias=wb.null_bias(), count_scale=wb.count_scale())
    parts.append(dict(name=BWD, w=wb, kind="backward", flops=backward_flops(wb), headline=False, separate=True,
                      run=lambda: pa.bwd(qb, kb, vb, grb, workspace=wsb, out=outb, **kwb)))
    # the same backward given the row statistics a training forward keeps (the one-split
    # partial forward); they are computed once, outside the timed calls
    savedb = pa.fwd_partial(qb, kb, vb, **kwb)
    wsbs = torch.empty(pa.bwd_saved_workspace_bytes(probb), dtype=torch.uint8, device=dev)
    parts.append(dict(name=BWD_SAVED, w=wb, kind="backward", flops=backward_flops(wb), headline=False,
                      separate=True,
                      run=lambda: pa.bwd(qb, kb, vb, grb, workspace=wsbs, out=outb, saved=savedb, **kwb)))
    torch.cuda.synchronize()
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        for p in parts:
            if not p.get("separate"):
                p["run"]()
    torch.cuda.synchronize()

    events = {p["name"]: [] for p in parts}

    def timed(p):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        p["run"]()
        e1.record()
        events[p["name"]].append((e0, e1))

    step_parts = [p for p in parts if not p.get("separate")]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for p in step_parts:
            timed(p)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # parts outside the step (the backward) are timed afterwards in their own loop, so
    # their long vector-ALU load does not change the clocks the step parts run at
    for p in parts:
        if p.get("separate"):
            for _ in range(args.warmup):
                p["run"]()
            for _ in range(args.steps):
                timed(p)
    torch.cuda.synchronize()

    res = {}
    for p in parts:
        ms = [a.elapsed_time(b) for a, b in events[p["name"]]]
        ms.sort()
        avg = sum(ms) / len(ms)
        entry = {"ms_avg": avg, "ms_median": ms[len(ms) // 2], "ms_p10": _percentile(ms, 10),
                 "ms_p90": _percentile(ms, 90), "ms_min": ms[0], "ms_max": ms[-1]}
        if p["kind"] == "prefill":
            entry["tflops"] = p["flops"] / (avg * 1e-3) / 1e12
            entry["frac_bf16_peak"] = entry["tflops"] / PEAK_BF16_TFLOPS
            entry["flops_per_launch"] = p["flops"]
        elif p["kind"] in ("backward", "side"):
            entry["tflops"] = p["flops"] / (avg * 1e-3) / 1e12
            entry["frac_bf16_peak"] = entry["tflops"] / PEAK_BF16_TFLOPS
            entry["flops_per_call"] = p["flops"]
        else:
            entry["gbs"] = p["bytes"] / (avg * 1e-3) / 1e9
            entry["frac_hbm_peak"] = entry["gbs"] / PEAK_HBM_GBS
            entry["bytes_per_launch"] = p["bytes"]
            entry["splits"] = {DECODE: splits, DECODE_B1: splits1b}.get(p["name"])
        res[p["name"]] = entry
    assert torch.isfinite(outd["direction"]).all()  # a sanity check; parity is in the tests

    pf_flops = sum(p["flops"] for p in parts if p["kind"] == "prefill")
    pf_ms = sum(res[p["name"]]["ms_avg"] for p in parts if p["kind"] == "prefill")
    value = pf_flops / (pf_ms * 1e-3) / 1e12
    digest = source_digest()
    big = res[PREFILL[1]]
    roofline = {"bound": "mfma", "achieved": big["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": big["tflops"] / PEAK_BF16_TFLOPS, "kernel": "polar_fwd_bf16_pipe_kernel<64,...> (T=65536 d=64)",
                "traffic": measured_traffic("fwd_bf16_t65536_d64"),
                # from the committed counter profile of this kernel: matrix-core busy cycles
                # over the dispatch's active cycles, and the clock it ran at
                "mfma_busy": profiled("fwd_bf16_t65536_d64", "mfma_busy"),
                "clock_ghz": profiled("fwd_bf16_t65536_d64", "clock_ghz"),
                # the vector ALU's share of the SIMD cycles: at d=64 it, not the matrix cores,
                # is the saturated unit (about 9.7 VALU instructions per MFMA, two of them exp)
                "valu_busy": profiled("fwd_bf16_t65536_d64", "valu_busy"),
                "mfma_valu_coexec": profiled("fwd_bf16_t65536_d64", "mfma_valu_coexec")}
    small = res[PREFILL[0]]
    small.update({"mfma_busy": profiled("fwd_bf16_t16384_d128", "mfma_busy"),
                  "clock_ghz": profiled("fwd_bf16_t16384_d128", "clock_ghz"),
                  "valu_busy": profiled("fwd_bf16_t16384_d128", "valu_busy"),
                  "traffic": measured_traffic("fwd_bf16_t16384_d128")})
    dec = res[DECODE]
    decode_roof = {"bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": dec["frac_hbm_peak"], "ms": dec["ms_avg"],
                   "traffic": measured_traffic("decode_b64_h8_tk65536_d128")}
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "polar attention hot path: prefill bf16 T=16384 d=128 H=16 + prefill bf16 "
                               "T=65536 d=64 H=16 (causal) + split-KV decode bf16 batch 64 H=8 d=128 KV=65536",
                   "prefill": PREFILL, "decode": DECODE, "value_is": "prefill TFLOP/s over both prefill launches",
                   "frac_bf16_peak": value / PEAK_BF16_TFLOPS},
        "roofline": roofline,
        "decode": decode_roof,
        "decode_batch1": {"bound": "hbm", "achieved": res[DECODE_B1]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": res[DECODE_B1]["frac_hbm_peak"], "us": res[DECODE_B1]["ms_avg"] * 1e3,
                          "splits": splits1b,
                          "note": "latency: one sequence, 8 heads, 64K keys (the first sequence of the decode "
                                  "cache), split kernel and merge"},
        "paged_gqa_decode": {"bound": "hbm", "achieved": res[PAGED]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": res[PAGED]["frac_hbm_peak"], "ms": res[PAGED]["ms_avg"],
                             "traffic": measured_traffic("paged_gqa_decode_b64_h32_kv8_tk65536_d128"),
                             "note": "32 query heads share 8 KV heads; K and V are read once per group"},
        "backward": {"bound": "mfma", "achieved": res[BWD]["tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": res[BWD]["frac_bf16_peak"], "ms": res[BWD]["ms_avg"],
                     "traffic_dkdv": measured_traffic("bwd_dkdv_b1_h16_kv4_t16384_d128"),
                     "note": "bf16 matrix-core path: forward statistics, row constants, dq, dk, dv; "
                             "10 d algorithmic flops per causal pair"},
        "chunked_prefill": {"bound": "mfma", "achieved": res[CHUNKED]["tflops"], "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": res[CHUNKED]["frac_bf16_peak"], "ms": res[CHUNKED]["ms_avg"],
                            "note": f"the T=65536 d=64 prefill in {65536 // CHUNK} chunks of {CHUNK} queries: per "
                                    "chunk a partial forward over the cached prefix and one over the chunk, then "
                                    "the merge; the one-pass prefill's algorithmic flops"},
        "chunked_prefill_over_cache": {
            "bound": "mfma", "achieved": res[CHUNKED_CACHE]["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": res[CHUNKED_CACHE]["frac_bf16_peak"], "ms": res[CHUNKED_CACHE]["ms_avg"],
            "note": f"the same {65536 // CHUNK} chunks, each one forward over the cache up to its last row "
                    "(fewer queries than keys, causal); the one-pass prefill's algorithmic flops"},
        "needle_prefill": {"bound": "mfma", "achieved": res[NEEDLE]["tflops"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": res[NEEDLE]["frac_bf16_peak"], "ms": res[NEEDLE]["ms_avg"],
                           "mfma_busy": profiled("fwd_bf16_needle_b4_h8_t4096_d64", "mfma_busy"),
                           "clock_ghz": profiled("fwd_bf16_needle_b4_h8_t4096_d64", "clock_ghz"),
                           "note": "bf16 B=4 H=8 T=4096 d=64 causal, one planted needle per head"},
        "fp32_prefill": {"bound": "alu", "achieved": res[FP32_SMALL]["tflops"], "ms": res[FP32_SMALL]["ms_avg"],
                         "note": "fp32 B=1 H=2 T=256 d=64 causal: a correctness path, launch-bound at this size"},
        "variants": {
            "soft_key_floor": {"bound": "mfma", "achieved": res[SOFT_FLOOR]["tflops"], "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": res[SOFT_FLOOR]["frac_bf16_peak"],
                               "ms": res[SOFT_FLOOR]["ms_avg"]},
            f"window_{WIN}": {"bound": "mfma", "achieved": res[WINDOW]["tflops"], "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": res[WINDOW]["frac_bf16_peak"], "ms": res[WINDOW]["ms_avg"],
                              "note": "flops of the (query, key) pairs inside the window"},
            "note": "the T=65536 d=64 prefill under reading variants: a per-key soft floor, and a sliding window"},
        "backward_saved": {"bound": "mfma", "achieved": res[BWD_SAVED]["tflops"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": res[BWD_SAVED]["frac_bf16_peak"],
                           "ms": res[BWD_SAVED]["ms_avg"],
                           "note": "the same backward given the forward's saved row statistics "
                                   "(polar_attn_bwd_saved): row constants, dq, dk, dv"},
        "parts": res,
        "source_digest": digest,
        "software": rocm_version(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        base = cpu_baseline(args.cpu_seconds)
        gpu_ms = {name: res[name]["ms_avg"] for name in (FP32_SMALL, NEEDLE, *PREFILL, DECODE)}
        print("[bench] timing the CPU oracle per configuration", file=sys.stderr, flush=True)
        base["per_config"] = oracle_per_config(base, gpu_ms, (qd, kd, vd))
        base.pop("_pairs")
        base.pop("_seconds")
        line["cpu_baseline"] = base
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

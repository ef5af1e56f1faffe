"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Inputs come from the seeded generators in polar_inputs; the oracle receives the very
tensors the GPU consumes (bf16 values upcast exactly).  Sizes the oracle finishes in
seconds are compared on every row.  The full-size workloads run in the launch
configuration the benchmark times and are compared on every row as well: the T=65536
prefill one head per test (about ten seconds of oracle time each), the decode one
(sequence, head) row at a time, its K and V slice copied back from the device.
"""
import math

import numpy as np
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import merge_reference, polar_attention, split_statistics
from tests.parity import assert_parity, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def kind_of(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


def run_case(B, H, Hkv, Tq, Tk, d, dtype, causal, seed, tau=None, beta=None, kappa=None, rows=None, stats=True,
             label=""):
    q, k, v, _ = pin.random_qkv(B, H, Hkv, Tq, Tk, d, dtype, seed)
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, len_temp=tau, null_bias=beta, count_scale=kappa,
                 stats=stats)
    torch.cuda.synchronize()
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=causal, len_temp=tau, null_bias=beta,
                          count_scale=kappa, rows=rows)
    return assert_parity(out, ref, kind_of(dtype), rows=rows, label=label)


# ---------------------------------------------------------------- reduced shapes, every row

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 300, 1000])
def test_fwd_shapes(dtype, d, causal, T):
    H = 2
    run_case(1, H, H, T, T, d, dtype, causal, seed=T * 7 + d, beta=[0.0] * H, label=f"T={T} d={d}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("tau,beta,kappa", [
    ([0.0, 0.1], [-2.0, 3.0], [1.0, 4.0]),
    ([0.1, 0.0], None, [4.0, 1.0]),
    ([0.3, 0.05], [0.0, 0.0], None),
])
def test_fwd_parameter_sweep(dtype, tau, beta, kappa):
    run_case(2, 2, 2, 333, 333, 64, dtype, True, seed=5, tau=tau, beta=beta, kappa=kappa)
    run_case(1, 2, 2, 200, 200, 128, dtype, False, seed=6, tau=tau, beta=beta, kappa=kappa)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fwd_gqa_and_bottom_right_causal(dtype):
    run_case(2, 4, 2, 150, 150, 128, dtype, True, seed=11, beta=[0.0] * 4, label="gqa")
    run_case(1, 4, 1, 70, 333, 64, dtype, True, seed=12, tau=[0.1] * 4, beta=[0.5] * 4, label="Tq<Tk causal")
    run_case(1, 2, 2, 70, 333, 64, dtype, False, seed=13, beta=[0.0] * 2, label="Tq<Tk")


@pytest.mark.parametrize("stats", [True, False])
@pytest.mark.parametrize("B,H,Tq,Tk", [(2, 16, 4100, 4100), (3, 16, 3000, 3300)])
def test_fwd_two_block_causal_path_ragged(B, H, Tq, Tk, stats):
    """Causal d=64 grids too large for one resident round keep two 32-row blocks per wave
    (smaller causal grids take one block per wave); these shapes reach that path with a
    ragged last query tile and a ragged last key tile, and (second case) bottom-right
    alignment with more keys than queries.  Every row against the oracle."""
    run_case(B, H, H, Tq, Tk, 64, torch.bfloat16, True, seed=Tq + Tk + B, beta=[0.0] * H, stats=stats,
             label=f"two-block causal B={B} H={H} Tq={Tq} Tk={Tk} stats={stats}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,T", [(1, 8, 8, 1000), (1, 8, 2, 700), (2, 8, 4, 520), (1, 16, 16, 300),
                                       (1, 8, 8, 4096)])
@pytest.mark.parametrize("causal", [True, False])
def test_fwd_one_round_grids(d, B, H, Hkv, T, causal):
    """Grids small enough to be resident at once, with heads in multiples of 8: the bf16
    prefill then pairs each XCD's heavy and light query tiles (an even tile count per XCD)
    or keeps the plain order (an odd one); every row of every tile against the oracle."""
    run_case(B, H, Hkv, T, T, d, torch.bfloat16, causal, seed=T + 3 * d + H, beta=[0.0] * H,
             label=f"one round B={B} H={H} T={T} d={d}")


@pytest.mark.parametrize("B,H,Hkv,T", [(2, 8, 8, 8192), (2, 8, 2, 8000)])
def test_fwd_half_height_tiles_beyond_one_round(B, H, Hkv, T):
    """d=64 causal grids that take half-height query tiles and have more of them than the
    chip holds at once (1024 and 1008 tiles for 768 resident workgroups, the needle
    workload's shape at half the heads and twice the length), the last with a ragged tile.
    Every row against the oracle with statistics on, and the statistics-off kernel, which
    the benchmark times, bitwise equal on every channel."""
    q, k, v, _ = pin.random_qkv(B, H, Hkv, T, T, 64, torch.bfloat16, T + 41)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    beta = [0.0] * H
    on = pa.fwd(qd, kd, vd, causal=True, null_bias=beta, stats=True)
    off = pa.fwd(qd, kd, vd, out=pa.allocate_outputs(B, H, T, 64, DEV), causal=True, null_bias=beta)
    torch.cuda.synchronize()
    for key in CHANNELS:
        assert torch.equal(on[key], off[key]), key
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, null_bias=beta)
    assert_parity(on, ref, "bf16", label=f"half-height tiles B={B} H={H} T={T}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Tq,Tk", [(300, 70), (70, 300), (1, 129), (257, 1)])
def test_fwd_noncausal_unequal_lengths(dtype, d, Tq, Tk):
    """Without the mask every query sees all Tk keys, whatever Tq is."""
    run_case(1, 4, 2, Tq, Tk, d, dtype, causal=False, seed=Tq * 7 + Tk + d, tau=[0.0, 0.1, 0.2, 0.05],
             beta=[0.0, 0.5, -1.0, 2.0], label=f"noncausal Tq={Tq} Tk={Tk} d={d}")


def test_fwd_scale_override_and_large_logits():
    q, k, v, _ = pin.random_qkv(1, 2, 2, 257, 257, 64, torch.bfloat16, 21)
    q = q * 4  # exact in bf16: large logits exercise the reference-maximum moves
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), softmax_scale=0.3, null_bias=[0.0, 1.0], stats=True)
    torch.cuda.synchronize()
    ref = polar_attention(to_np(q), to_np(k), to_np(v), softmax_scale=0.3, null_bias=[0.0, 1.0])
    assert_parity(out, ref, "bf16")


def test_fwd_uniform_logits_exact_neff():
    """q = 0: every visible key has p = 1, so n_eff equals the visible count exactly."""
    T, d = 700, 128
    g = torch.Generator(device=DEV).manual_seed(79)
    q = torch.zeros(1, 2, T, d, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(1, 2, T, d, device=DEV, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, T, d, device=DEV, generator=g).to(torch.bfloat16)
    out = pa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    n = torch.arange(1, T + 1, device=DEV, dtype=torch.float32)
    assert torch.equal(out["n_eff"][0, 0], n) and torch.equal(out["n_eff"][0, 1], n)


def test_fwd_maximum_key_count_closed_forms():
    """The longest key range the bf16 kernels address (one head's K and V at the top of the
    32-bit range of their buffer loads: 16,776,959 keys at d = 128), checked against closed
    forms of the definition, which the oracle cannot hold in memory at this size.
      row 0, q = 0: every score is 0, so S1 = S2 = n, n_eff = n, u = normalize(sum_j v_j),
        conf = n / (n + e^f) with f = sqrt(2 ln n).
      row 1, q = a e_0, and the only key with a component along e_0 is the last one,
        b e_0: its score is D = a b / sqrt(d), every other score is 0, so with m = D
        S1 = 1 + (n - 1) e^-D, S2 = 1 + (n - 1) e^-2D, n_eff = S1^2 / S2,
        u = normalize(v_last + e^-D sum_{j < last} v_j), conf = S1 / (S1 + e^(f - D)).
    Together they show that every key up to the last one is read and counted."""
    n, d, a, b = 16_776_959, 128, 16.0, 12.0
    print(f"[parity] maximum key count n={n}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(80)
    v = torch.randn(1, 1, n, d, device=DEV, generator=g).to(torch.bfloat16)
    k = torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=DEV)
    k[0, 0, n - 1, 0] = b
    q = torch.zeros(1, 1, 2, d, dtype=torch.bfloat16, device=DEV)
    q[0, 0, 1, 0] = a
    out = pa.fwd(q, k, v, causal=False, null_bias=[0.0], stats=True)
    torch.cuda.synchronize()
    # sum_j v_j in fp64 on the host, chunk by chunk
    total = torch.zeros(d, dtype=torch.float64)
    step = 1 << 20
    for s in range(0, n, step):
        total += v[0, 0, s:min(n, s + step)].cpu().double().sum(0)
    v_last = v[0, 0, n - 1].cpu().double()
    del k, v
    torch.cuda.empty_cache()
    D = a * b / math.sqrt(d)
    f = math.sqrt(2.0 * math.log(n))
    s1 = 1.0 + (n - 1) * math.exp(-D)
    s2 = 1.0 + (n - 1) * math.exp(-2.0 * D)
    acc1 = v_last + math.exp(-D) * (total - v_last)
    want = {
        "n_eff": [float(n), s1 * s1 / s2],
        "confidence": [n / (n + math.exp(f)), s1 / (s1 + math.exp(f - D))],
        "direction": [(total / total.norm()).numpy(), (acc1 / acc1.norm()).numpy()],
        "m": [0.0, D], "s1": [float(n), s1], "s2": [float(n), s2],
    }
    want["count"] = [c * math.tanh(math.log(x)) for c, x in zip(want["confidence"], want["n_eff"])]
    got = {key: to_np(t)[0, 0] for key, t in out.items() if torch.is_tensor(t)}
    for i in range(2):
        du = float(np.linalg.norm(got["direction"][i] - want["direction"][i]))
        dn = abs(got["n_eff"][i] - want["n_eff"][i]) / want["n_eff"][i]
        dc = abs(got["confidence"][i] - want["confidence"][i])
        dk = abs(got["count"][i] - want["count"][i])
        st = got["stats"][i]
        print(f"[parity] max keys row {i}: direction {du:.2e} n_eff {dn:.2e} (gpu {got['n_eff'][i]:.6g}) "
              f"confidence {dc:.2e} count {dk:.2e} stats {st}", flush=True)
        assert du <= 2e-2 and dn <= 1e-2 and dc <= 1e-2 and dk <= 1e-2, i
        assert abs(st[0] - want["m"][i]) <= 1e-3 * max(1.0, want["m"][i])
        assert abs(st[1] - want["s1"][i]) <= 1e-2 * want["s1"][i] and abs(st[2] - want["s2"][i]) <= 1e-2 * want["s2"][i]
    # q = 0: the weights are exactly 1 and their sums integers below 2^24
    assert got["stats"][0][1] == n and got["stats"][0][2] == n


def test_decode_long_cache_closed_forms():
    """Decode over a cache of 20,000,002 keys (past 2^24, where a count kept in fp32 by ones
    would stop growing), through the one-head split kernel with the merge and through the
    grouped kernel (two query heads over one KV head), against closed forms of the
    definition: head 0 has q = 0 (every score 0: n_eff = n, u = normalize(sum_j v_j)); head
    1 has q = a e_0 and only the last key has a component along e_0 (b e_0), so its score is
    D = a b / sqrt(d) and every other score 0 (n_eff = S1^2 / S2 with S1 = 1 + (n-1) e^-D,
    S2 = 1 + (n-1) e^-2D, u = normalize(v_last + e^-D sum_{j < last} v_j))."""
    n, d, a, b = 20_000_002, 128, 16.0, 12.0
    print(f"[parity] decode over n={n} keys", flush=True)
    g = torch.Generator(device=DEV).manual_seed(81)
    v = torch.randn(1, 1, n, d, device=DEV, generator=g, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=DEV)
    k[0, 0, n - 1, 0] = b
    q = torch.zeros(1, 2, 1, d, dtype=torch.bfloat16, device=DEV)
    q[0, 1, 0, 0] = a
    grouped = pa.decode(q, k, v, null_bias=[0.0, 0.0], stats=True)
    single = [pa.decode(q[:, h:h + 1].contiguous(), k, v, null_bias=[0.0], stats=True) for h in range(2)]
    torch.cuda.synchronize()
    total = torch.zeros(d, dtype=torch.float64)
    step = 1 << 20
    for s in range(0, n, step):
        total += v[0, 0, s:min(n, s + step)].cpu().double().sum(0)
    v_last = v[0, 0, n - 1].cpu().double()
    del k, v
    torch.cuda.empty_cache()
    D = a * b / math.sqrt(d)
    f = math.sqrt(2.0 * math.log(n))
    s1 = 1.0 + (n - 1) * math.exp(-D)
    s2 = 1.0 + (n - 1) * math.exp(-2.0 * D)
    acc1 = v_last + math.exp(-D) * (total - v_last)
    want_neff = [float(n), s1 * s1 / s2]
    want_conf = [n / (n + math.exp(f)), s1 / (s1 + math.exp(f - D))]
    want_dir = [(total / total.norm()).numpy(), (acc1 / acc1.norm()).numpy()]
    cases = [("grouped", grouped, h, h) for h in range(2)] + [("split", single[h], 0, h) for h in range(2)]
    for label, out, col, h in cases:
        assert out["splits"] > 1, label
        du = float(np.linalg.norm(to_np(out["direction"])[0, col, 0] - want_dir[h]))
        dn = abs(float(out["n_eff"][0, col, 0]) - want_neff[h]) / want_neff[h]
        dc = abs(float(out["confidence"][0, col, 0]) - want_conf[h])
        print(f"[parity] long cache {label} head {h}: direction {du:.2e} n_eff {dn:.2e} confidence {dc:.2e} "
              f"splits {out['splits']}", flush=True)
        assert du <= 2e-2 and dn <= 1e-2 and dc <= 1e-2, (label, h, du, dn, dc)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_zero_values_give_zero_direction(dtype, d):
    """acc = 0 (all values zero): the direction is the zero vector, exactly, on every path
    (the norm is never divided by zero), and the other channels still match the oracle."""
    print(f"[parity] zero values d={d} {dtype}", flush=True)
    q, k, v, _ = pin.random_qkv(1, 2, 2, 200, 200, d, dtype, seed=60 + d)
    v = torch.zeros_like(v)
    kw = dict(len_temp=[0.0, 0.1], null_bias=[0.0, 1.0])
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, **kw)
    assert not np.any(ref["direction"])
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, **kw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out["direction"]).item() == 0
    assert_parity(out, ref, kind_of(dtype), label=f"zero values fwd d={d}")
    if dtype == torch.bfloat16:
        qd = q[:, :, -1:].contiguous()
        ref_d = polar_attention(to_np(qd), to_np(k), to_np(v), causal=True, **kw)
        for splits in (1, 3):
            out_d = pa.decode(qd.to(DEV), k.to(DEV), v.to(DEV), num_splits=splits, **kw)
            torch.cuda.synchronize()
            assert torch.count_nonzero(out_d["direction"]).item() == 0
            assert_parity(out_d, ref_d, "bf16", label=f"zero values decode d={d} S={splits}")
        # paged: blocks of 8 keys, in order
        kp = k[0].permute(1, 0, 2).reshape(200 // 8, 8, 2, d).contiguous()
        vp = torch.zeros_like(kp)
        table = torch.arange(25, dtype=torch.int32).reshape(1, 25)
        lens = torch.tensor([200], dtype=torch.int32)
        out_p = pa.decode_paged(qd.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens.to(DEV), seq_k=200, **kw)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out_p["direction"]).item() == 0
        assert_parity(out_p, ref_d, "bf16", label=f"zero values paged decode d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,Tq,Tk,causal", [(1, 2, 2, 300, 300, True), (2, 4, 2, 1000, 1000, True),
                                                  (1, 4, 1, 70, 333, True), (1, 2, 2, 257, 129, False),
                                                  (1, 8, 8, 4097, 4097, True)])
def test_fwd_statistics_off_bitwise(d, B, H, Hkv, Tq, Tk, causal):
    """The instantiation without statistics (the one the benchmark times) and the one
    with them compute the same channels bitwise: tracking the true row maximum on the
    side changes no weight, sum or accumulator.  The statistics-on outputs are checked
    against the oracle here as well."""
    print(f"[parity] statistics off d={d} B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} causal={causal}", flush=True)
    q, k, v, _ = pin.random_qkv(B, H, Hkv, Tq, Tk, d, torch.bfloat16, seed=Tq + Tk + d + H)
    kw = dict(causal=causal, len_temp=[0.02 * h for h in range(H)], null_bias=[0.0] * H)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    on = pa.fwd(qd, kd, vd, stats=True, **kw)
    off = pa.fwd(qd, kd, vd, out=pa.allocate_outputs(B, H, Tq, d, DEV), **kw)
    torch.cuda.synchronize()
    assert_same_channels(on, off, "statistics off")
    assert_parity(on, polar_attention(to_np(q), to_np(k), to_np(v), **kw), "bf16", label=f"statistics on d={d}")


def test_fwd_optional_outputs_and_determinism():
    q, k, v, _ = pin.random_qkv(1, 2, 2, 300, 300, 64, torch.bfloat16, 31)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    a = pa.fwd(q, k, v, null_bias=[0.0, 0.0], stats=True)
    b = pa.fwd(q, k, v, null_bias=[0.0, 0.0], stats=True)
    out = pa.allocate_outputs(1, 2, 300, 64, DEV, confidence=False, count=False)
    c = pa.fwd(q, k, v, null_bias=[0.0, 0.0], out=out)
    off = pa.fwd(q, k, v, null_bias=None)
    hi = pa.fwd(q, k, v, null_bias=[3.0, -2.0])
    torch.cuda.synchronize()
    for key in ("direction", "n_eff", "confidence", "count", "stats"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["direction"], c["direction"]) and torch.equal(a["n_eff"], c["n_eff"])
    # the null floor moves only the confidence: direction and n_eff are bitwise unchanged
    for other in (off, hi):
        assert torch.equal(a["direction"], other["direction"]) and torch.equal(a["n_eff"], other["n_eff"])
    assert torch.equal(off["confidence"], torch.ones_like(off["confidence"]))


def test_fwd_empty_inputs():
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(1, 2, 5, 64, device=DEV, generator=torch.Generator(device=DEV).manual_seed(93)).to(torch.bfloat16)
    out = pa.fwd(q, k, k.clone(), causal=True)
    assert out["direction"].numel() == 0
    q0 = torch.empty(0, 2, 4, 64, dtype=torch.bfloat16, device=DEV)
    k0 = torch.empty(0, 2, 4, 64, dtype=torch.bfloat16, device=DEV)
    pa.fwd(q0, k0, k0.clone())
    torch.cuda.synchronize()


def test_fwd_rejects_bad_calls():
    q = torch.randn(1, 2, 8, 64, device=DEV, generator=torch.Generator(device=DEV).manual_seed(94)).to(torch.bfloat16)
    with pytest.raises(pa.PolarArgumentError):
        pa.fwd(q, q.clone(), q.clone(), len_temp=[0.0, -5.0])  # lam(8) <= 0
    with pytest.raises(pa.PolarArgumentError):
        pa.fwd(q[:, :, :, :32].contiguous(), q[:, :, :, :32].contiguous(), q[:, :, :, :32].contiguous())


# ---------------------------------------------------------------- decode and merge

def decode_case(B, H, Hkv, Tk, d, seed, splits_list, tau=None, beta=None, kappa=None):
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, Tk, d, torch.bfloat16, seed)
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, len_temp=tau, null_bias=beta,
                          count_scale=kappa)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    outs = []
    for s in splits_list:
        out = pa.decode(qd, kd, vd, num_splits=s, len_temp=tau, null_bias=beta, count_scale=kappa, stats=True)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", label=f"decode S={s}")
        # the partials, merged by the oracle, give the same outputs
        parts = to_np(out["partials"])
        merged = merge_reference(parts, Tk, len_temp=tau, null_bias=beta, count_scale=kappa)
        assert_parity(out, merged, "bf16", label=f"oracle merge of GPU partials S={s}")
        outs.append(out)
    return outs


@pytest.mark.parametrize("d", [64, 128])
def test_decode_split_invariance(d):
    # 17 and 64 splits take the one-wave parallel merge, 65 and 300 the four-wave one
    decode_case(2, 4, 4, 3001, d, seed=40 + d, splits_list=[1, 2, 3, 8, 17, 64, 65, 300, 0],
                tau=[0.0, 0.1, 0.2, 0.05], beta=[0.0, -1.0, 2.0, 0.0], kappa=[1.0, 2.0, 1.0, 4.0])


def test_decode_small_and_ragged():
    decode_case(1, 2, 2, 1, 128, seed=50, splits_list=[1, 0])
    decode_case(1, 2, 2, 17, 64, seed=51, splits_list=[1, 5, 17, 0], beta=[0.0, 0.0])
    decode_case(3, 8, 2, 1000, 128, seed=52, splits_list=[7, 0], beta=[0.0] * 8)  # GQA


def test_merge_entry_point_on_oracle_partials():
    """polar_attn_merge on partials written by the oracle (never by the GPU)."""
    rng = np.random.default_rng(60)
    B, H, Tq, Tk, d, S = 2, 3, 4, 500, 128, 6
    tau, beta, kappa = [0.0, 0.1, 0.3], [0.0, 1.0, -1.0], [1.0, 0.5, 2.0]
    q = rng.standard_normal((B, H, Tq, d))
    k, v = rng.standard_normal((2, B, H, Tk, d))
    bounds = np.linspace(0, Tk, S + 1).astype(int)
    part = np.zeros((B, H, Tq, S, d + 3))
    for b in range(B):
        for h in range(H):
            for i in range(Tq):
                n = i + 1 + Tk - Tq
                lam = 1 + tau[h] * math.log(n)
                for s in range(S):
                    lo, hi = bounds[s], min(bounds[s + 1], n)
                    if hi <= lo:
                        part[b, h, i, s, 0] = -np.inf
                        continue
                    m, s1, s2, acc = split_statistics(q[b, h, i], k[b, h], v[b, h], lam, 1 / math.sqrt(d), lo, hi)
                    part[b, h, i, s] = [m, s1, s2, *acc]
    ref = merge_reference(part, np.arange(Tk - Tq + 1, Tk + 1)[None, None, :], len_temp=tau, null_bias=beta,
                          count_scale=kappa)
    gp = torch.from_numpy(part).float().to(DEV)
    out = pa.merge(gp, seq_k=Tk, causal=True, len_temp=tau, null_bias=beta, count_scale=kappa, stats=True)
    torch.cuda.synchronize()
    assert_parity(out, ref, "f32", label="merge")


# ---------------------------------------------------------------- the named workloads

CHANNELS = ("direction", "n_eff", "confidence", "count")


def bench_call(q, k, v, w):
    """The prefill call the benchmark times: statistics off (the kernel instantiation
    that does not track the true row maximum), outputs from allocate_outputs."""
    out = pa.allocate_outputs(w.B, w.H, w.Tq, w.d, q.device)
    return pa.fwd(q, k, v, out=out, causal=w.causal, len_temp=w.len_temp(), null_bias=w.null_bias(),
                  count_scale=w.count_scale())


def assert_same_channels(a, b, label):
    """Bitwise equality of the four channels of two forward calls."""
    for key in CHANNELS:
        assert torch.equal(a[key], b[key]), f"{label}: {key} differs"


def workload_case(name):
    """A named workload: every row against the oracle (statistics on), and the
    benchmark's own call (statistics off) bitwise equal to it on every channel."""
    w = pin.WORKLOADS[name]
    print(f"[parity] {name}", flush=True)
    q, k, v, meta = pin.workload_inputs(w, "cpu")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = pa.fwd(qd, kd, vd, causal=w.causal, len_temp=w.len_temp(), null_bias=w.null_bias(),
                 count_scale=w.count_scale(), stats=True)
    timed = bench_call(qd, kd, vd, w)
    torch.cuda.synchronize()
    assert_same_channels(out, timed, f"{name} benchmark call")
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=w.causal, len_temp=w.len_temp(),
                          null_bias=w.null_bias(), count_scale=w.count_scale())
    e = assert_parity(out, ref, kind_of(w.dtype), label=name)
    print(f"[parity] {name} max errors over all rows {e}", flush=True)
    return out, meta


def test_workload_fp32_t256():
    workload_case("fp32_b1_h2_t256_d64")


def test_workload_needle_t4096():
    out, meta = workload_case("bf16_b4_h8_t4096_d64_needle")
    # the planted match dominates its row: n_eff close to 1
    for b, h, i, j in meta["needles"]:
        assert out["n_eff"][b, h, i].item() < 1.5


def test_workload_groups_t16384():
    out, meta = workload_case("bf16_b1_h16_t16384_d128_groups")
    for b, h, c, i, pos in meta["groups"]:
        assert abs(out["n_eff"][b, h, i].item() - c) < 0.1 * c + 0.5


_LENTEMP = {}


def lentemp_run():
    """The T=65536 workload: inputs on the host and the GPU outputs, computed once."""
    if not _LENTEMP:
        w = pin.WORKLOADS["bf16_b1_h16_t65536_d64_lentemp"]
        q, k, v, _ = pin.workload_inputs(w, "cpu")
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        out = pa.fwd(qd, kd, vd, causal=w.causal, len_temp=w.len_temp(),
                     null_bias=w.null_bias(), count_scale=w.count_scale(), stats=True)
        timed = bench_call(qd, kd, vd, w)
        torch.cuda.synchronize()
        same = {key: torch.equal(out[key], timed[key]) for key in CHANNELS}
        _LENTEMP.update(w=w, q=q, k=k, v=v, out={n: t.cpu() for n, t in out.items() if torch.is_tensor(t)},
                        bench_same=same)
        del out, timed, qd, kd, vd
        torch.cuda.empty_cache()
    return _LENTEMP


def test_workload_lentemp_bench_call_bitwise():
    """The T=65536 prefill as the benchmark times it (statistics off) gives bitwise the
    channels of the statistics-on call that the per-head tests check on every row."""
    r = lentemp_run()
    assert all(r["bench_same"].values()), r["bench_same"]


@pytest.mark.parametrize("h", range(16))
def test_workload_lentemp_t65536(h):
    r = lentemp_run()
    w, q, k, v = r["w"], r["q"], r["k"], r["v"]
    print(f"[parity] bf16_b1_h16_t65536_d64_lentemp head {h}", flush=True)
    one = lambda xs: None if xs is None else [xs[h]]
    ref = polar_attention(to_np(q[:, h:h + 1]), to_np(k[:, h:h + 1]), to_np(v[:, h:h + 1]), causal=w.causal,
                          len_temp=one(w.len_temp()), null_bias=one(w.null_bias()), count_scale=one(w.count_scale()))
    sub = {n: t[:, h:h + 1] for n, t in r["out"].items()}
    e = assert_parity(sub, ref, "bf16", label=f"t65536 head {h}")
    print(f"[parity] head {h} max errors over all rows {e}", flush=True)


def test_workload_decode_64k():
    w = pin.WORKLOADS["bf16_decode_b64_h8_tk65536_d128"]
    print("[parity] decode workload", flush=True)
    q, k, v, _ = pin.workload_inputs(w, DEV)
    out = pa.decode(q, k, v, len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale(),
                    stats=True)
    torch.cuda.synchronize()
    # every (sequence, head) row, its K and V slice copied back one at a time
    worst = {}
    for b in range(w.B):
        for h in range(w.H):
            ref = polar_attention(to_np(q[b:b + 1, h:h + 1]), to_np(k[b:b + 1, h:h + 1]),
                                  to_np(v[b:b + 1, h:h + 1]), causal=True, len_temp=[w.len_temp()[h]],
                                  null_bias=[w.null_bias()[h]], count_scale=[w.count_scale()[h]])
            sub = {key: (t[b:b + 1, h:h + 1] if torch.is_tensor(t) else t) for key, t in out.items()
                   if key not in ("partials", "splits")}
            e = assert_parity(sub, ref, "bf16", label=f"decode b={b} h={h}")
            worst = {n: max(worst.get(n, 0.0), x) for n, x in e.items()}
    print(f"[parity] decode max errors over all {w.B * w.H} rows {worst}", flush=True)
    del k, v
    torch.cuda.empty_cache()


def test_workload_decode_batch1_latency_call():
    """The batch-1 decode as the benchmark times it: the first sequence of the 64K decode
    cache alone (the per-sequence generator makes B=1 draw exactly that sequence), automatic
    split count, caller-given workspace and outputs, no statistics.  Its 128 splits take the
    four-wave merge; all 8 rows against the oracle."""
    import dataclasses
    w = dataclasses.replace(pin.WORKLOADS["bf16_decode_b64_h8_tk65536_d128"], B=1)
    print("[parity] batch-1 decode, first sequence of the decode workload", flush=True)
    q, k, v, _ = pin.workload_inputs(w, DEV)
    kw = dict(len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    prob = pa.problem_for(q, k, causal=True, **kw)
    splits = pa.decode_num_splits(prob, 0)
    assert splits > 64, splits  # the many-split merge
    ws = torch.empty(pa.decode_workspace_bytes(prob, 0), dtype=torch.uint8, device=DEV)
    out = pa.allocate_outputs(1, w.H, 1, w.d, DEV)
    res = pa.decode(q, k, v, workspace=ws, out=out, **kw)
    torch.cuda.synchronize()
    assert res["splits"] == splits
    ref = polar_attention(to_np(q), to_np(k), to_np(v), causal=True, **kw)
    sub = {key: t for key, t in res.items() if torch.is_tensor(t) and key != "partials"}
    e = assert_parity(sub, ref, "bf16", label="batch-1 decode")
    print(f"[parity] batch-1 decode ({splits} splits) max errors over its {w.H} rows {e}", flush=True)

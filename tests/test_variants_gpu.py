"""GPU parity of the reading variants against the variant oracle.

Every variant runs through the prefill kernels (bf16 and fp32), the split-KV decode, the
grouped/paged decode and the merge, and is compared with oracle.polar_attention_variant
(or its split/merge functions) at the usual tolerances.  A per-key floor decides, key by
key, whether a score is above the row's floor; a row with a score within a small margin
of its floor is undecidable in floating point (the GPU computes the score in fp32 from
the same inputs), so such rows are left out of the comparison and the test requires that
almost all rows are decidable.
"""
import math

import numpy as np
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import merge_variant, polar_attention_variant, split_statistics_variant, variant_of
from oracle.polar_variants import floor_level, temperature
from tests.parity import TOL, assert_parity, to_np
from tests.test_decode_paged_gpu import make_paged

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MARGIN = 1e-4      # tempered-logit distance to the floor below which a key's side is undecidable

H4 = dict(len_temp=[0.05, 0.2, 0.0, 0.1], null_bias=[-3.0, -2.0, -1.0, 0.5], count_scale=[1.0, 2.0, 1.0, 4.0])
VARIANTS = {
    "ssmax": dict(temperature="ssmax"),
    "train_ratio": dict(temperature="train_ratio", train_len=64),
    "gumbel2": dict(floor_level="gumbel2"),
    "qnorm": dict(floor_level="qnorm"),
    "log1p": dict(saturation="log1p"),
    "soft": dict(key_floor="soft"),
    "gate": dict(key_floor="gate"),
    "window": dict(window=37),
    "all": dict(temperature="ssmax", floor_level="gumbel2", key_floor="soft", saturation="log1p", window=50),
}


def decidable_rows(q, k, causal, kw, variant, rows=None):
    """[B, H, Tq] mask (or [B, H, len(rows)] for the given query rows): no visible score of
    the row within MARGIN of its floor (always true without a per-key floor)."""
    var = variant_of(variant)
    q, k = to_np(q), to_np(k)
    B, H, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    rows = range(Tq) if rows is None else [int(i) for i in rows]
    ok = np.ones((B, H, len(rows)), dtype=bool)
    if var["key_floor"] == "null":
        return ok
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(H):
            tau = kw["len_temp"][h] if kw.get("len_temp") else 0.0
            beta = kw["null_bias"][h]
            for r, i in enumerate(rows):
                hi = min(i + 1 + Tk - Tq, Tk) if causal else Tk
                lo = max(0, hi - var["window"]) if var["window"] else 0
                n = hi - lo
                lam = temperature(n, tau, var)
                qi = q[b, h, i]
                sigma = scale * float(np.sqrt(qi @ qi)) if var["floor_level"] == "qnorm" else 1.0
                f = lam * sigma * floor_level(n, var) + beta
                s = lam * scale * (k[b, h // (H // Hkv), lo:hi] @ qi)
                ok[b, h, r] = np.min(np.abs(s - f)) > MARGIN
    return ok


def soft_floor_condition(q, k, causal, kw, variant, v=None):
    """[B, H, Tq] condition numbers of S1 and S2 (and, given v, of the direction) under
    the soft per-key floor.

    A weight e^s - e^f near the floor is ill-conditioned in the score: a score error
    delta changes it by about e^s delta while the weight itself is e^s - e^f.  With score
    errors bounded by u (1 + |s|), the relative errors of S1 and S2 are bounded by
    u kappa1 and u kappa2, kappa1 = sum e^{s - m} (1 + |s|) / S1 and
    kappa2 = 2 max(w) sum e^{s - m} (1 + |s|) / S2, and the direction's error by u kappa_u,
    kappa_u = sum e^{s - m} (1 + |s|) ||v_j|| / ||acc||, the sums over the keys above the
    floor."""
    var = variant_of(variant)
    q, k = to_np(q), to_np(k)
    v = None if v is None else to_np(v)
    B, H, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    k1 = np.ones((B, H, Tq))
    k2 = np.ones((B, H, Tq))
    ku = np.ones((B, H, Tq))
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(H):
            tau = kw["len_temp"][h] if kw.get("len_temp") else 0.0
            for i in range(Tq):
                hi = min(i + 1 + Tk - Tq, Tk) if causal else Tk
                lo = max(0, hi - var["window"]) if var["window"] else 0
                n = hi - lo
                lam = temperature(n, tau, var)
                qi = q[b, h, i]
                sigma = scale * float(np.sqrt(qi @ qi)) if var["floor_level"] == "qnorm" else 1.0
                f = lam * sigma * floor_level(n, var) + kw["null_bias"][h]
                s = lam * scale * (k[b, h // (H // Hkv), lo:hi] @ qi)
                m = s.max()
                above = s > f
                if not above.any():
                    continue
                w = np.exp(s[above] - m) - np.exp(f - m)
                e = np.exp(s[above] - m) * (1.0 + np.abs(s[above]))
                gross = float(np.sum(e))
                k1[b, h, i] = max(1.0, gross / w.sum())
                k2[b, h, i] = max(1.0, 2.0 * w.max() * gross / np.sum(w * w))
                if v is not None:
                    vv = v[b, h // (H // Hkv), lo:hi][above]
                    acc = w @ vv
                    norm = float(np.sqrt(acc @ acc))
                    if norm > 0.0:
                        ku[b, h, i] = max(1.0, float(e @ np.sqrt(np.sum(vv * vv, axis=1))) / norm)
    return (k1, k2) if v is None else (k1, k2, ku)


def compare(out, ref, kind, ok, label, cond=None):
    """assert_parity on the decidable rows (rows with n_eff = 0 compared exactly).  With
    `cond` (the soft floor's condition numbers of S1 and S2, and of the direction) the
    statistics S1, S2 are checked against the tolerance times the row's condition number,
    and so are the channels, each by the condition of what it is formed from:
    n_eff = S1^2 / S2 by 2 kappa1 + kappa2, the confidence by kappa1, the count by
    3 kappa1 + kappa2, the direction by kappa_u (never below the plain tolerance)."""
    assert ok.mean() >= 0.9, f"{label}: only {ok.mean():.2f} of the rows are decidable"
    flat = lambda x: x.reshape(-1, *x.shape[3:])
    g = {key: to_np(t) for key, t in out.items() if torch.is_tensor(t) and key != "partials"}
    mask = ok.reshape(-1)
    zero = mask & (flat(ref["n_eff"]) == 0.0)
    live = mask & ~zero
    for key in ("n_eff", "confidence", "count"):
        assert np.all(flat(g[key])[zero] == 0.0), f"{label} {key} of rows with nothing above the floor"
    assert np.all(flat(g["direction"])[zero] == 0.0)
    keys = [key for key in g if not (cond is not None and key == "stats")]
    sub_g = {key: torch.from_numpy(flat(g[key])[live][None, None]) for key in keys}
    sub_r = {key: flat(v)[live][None, None] for key, v in ref.items()}
    if live.any() and cond is not None and len(cond) == 3:
        tol = TOL[kind]
        k1, k2, ku = (flat(c)[live] for c in cond)
        du = np.sqrt(((flat(g["direction"])[live] - flat(ref["direction"])[live]) ** 2).sum(-1))
        en = np.abs(flat(g["n_eff"])[live] - flat(ref["n_eff"])[live]) / flat(ref["n_eff"])[live]
        ec = np.abs(flat(g["confidence"])[live] - flat(ref["confidence"])[live])
        et = np.abs(flat(g["count"])[live] - flat(ref["count"])[live])
        for name, err, allow in (("direction", du, tol["direction"] * ku), ("n_eff", en, tol["n_eff"] * (2 * k1 + k2)),
                                 ("confidence", ec, tol["confidence"] * k1),
                                 ("count", et, tol["count"] * (3 * k1 + k2))):
            assert np.isfinite(err).all() and np.all(err <= allow), \
                f"{label} {name}: worst {err.max():.3e}, worst ratio to the conditioned tolerance {(err / allow).max():.3f}"
        for key in ("direction", "n_eff"):
            assert torch.isfinite(out[key]).all(), f"{label} non-finite {key}"
    elif live.any():
        assert_parity(sub_g, sub_r, kind, label=label)
    if live.any():
        if cond is not None and "stats" in g:
            tol = TOL[kind]
            st = flat(g["stats"])[live]
            m_ref, s1_ref, s2_ref = (flat(ref[x])[live] for x in ("m", "s1", "s2"))
            assert np.all(np.abs(st[:, 0] - m_ref) <= tol["m"] * np.maximum(1.0, np.abs(m_ref))), label
            e1 = np.abs(st[:, 1] - s1_ref) / s1_ref / flat(cond[0])[live]
            e2 = np.abs(st[:, 2] - s2_ref) / s2_ref / flat(cond[1])[live]
            assert e1.max() <= tol["s"] and e2.max() <= tol["s"], f"{label} S1, S2 per condition: {e1.max()} {e2.max()}"
    print(f"[variant] {label}: {int(live.sum())} rows compared, {int(zero.sum())} empty, "
          f"{int((~mask).sum())} undecidable", flush=True)


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_variant(name, d, dtype):
    variant = VARIANTS[name]
    B, H, Hkv, Tq, Tk = 1, 4, 2, 140, 200
    q, k, v, _ = pin.random_qkv(B, H, Hkv, Tq, Tk, d, dtype, seed=700 + d + len(name))
    ref = polar_attention_variant(to_np(q), to_np(k), to_np(v), causal=True, variant=variant, **H4)
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, stats=True, variant=variant, **H4)
    torch.cuda.synchronize()
    ok = decidable_rows(q, k, True, H4, variant)
    cond = soft_floor_condition(q, k, True, H4, variant, v) if variant.get("key_floor") == "soft" else None
    compare(out, ref, "bf16" if dtype == torch.bfloat16 else "f32", ok, f"prefill {name} d={d} {dtype}", cond)


@pytest.mark.parametrize("name", ["soft", "gate", "qnorm", "ssmax"])
def test_prefill_variant_non_causal(name):
    variant = VARIANTS[name]
    q, k, v, _ = pin.random_qkv(2, 4, 4, 70, 150, 128, torch.bfloat16, seed=720)
    ref = polar_attention_variant(to_np(q), to_np(k), to_np(v), causal=False, variant=variant, **H4)
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, variant=variant, **H4)
    torch.cuda.synchronize()
    compare(out, ref, "bf16", decidable_rows(q, k, False, H4, variant), f"prefill non-causal {name}")


@pytest.mark.parametrize("window", [1, 5, 64, 65, 129, 1000])
def test_prefill_window_sizes(window):
    """Windows shorter than, equal to and longer than a key tile, and longer than the
    sequence (same as no window)."""
    variant = dict(window=window)
    q, k, v, _ = pin.random_qkv(1, 2, 2, 300, 300, 64, torch.bfloat16, seed=730 + window)
    kw = dict(len_temp=[0.1, 0.0], null_bias=[0.0, 1.0])
    ref = polar_attention_variant(to_np(q), to_np(k), to_np(v), causal=True, variant=variant, **kw)
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, variant=variant, **kw)
    torch.cuda.synchronize()
    assert_parity(out, ref, "bf16", label=f"window {window}")


@pytest.mark.parametrize("variant", [dict(key_floor="soft"), dict(window=4096)], ids=["soft_floor", "window4096"])
def test_workload_variants_t65536(variant):
    """The T=65536 d=64 workload (16 heads, per-head length temperatures) under the soft
    per-key floor and under a 4096-key window, at full size and in the benchmark's launch
    configuration (no statistics): sampled rows of every head against the variant oracle."""
    w = pin.WORKLOADS["bf16_b1_h16_t65536_d64_lentemp"]
    print(f"[variant] workload {w.name} {variant}", flush=True)
    q, k, v, _ = pin.workload_inputs(w, "cpu")
    kw = dict(len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    out = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, variant=variant, **kw)
    torch.cuda.synchronize()
    r = np.random.default_rng(91)
    # short rows (few visible keys, where the soft floor leaves keys above it), both sides of
    # the window length, the last row and random ones
    rows = np.unique(np.concatenate([[0, 1, 2, 3, 10, 31, 32, 63, 64, 100, 255, 256, 4095, 4096, 4097, w.Tq - 1],
                                     r.integers(0, w.Tq, 8)]))
    ref = polar_attention_variant(to_np(q), to_np(k), to_np(v), causal=True, variant=variant, rows=rows, **kw)
    sel = torch.as_tensor(rows, device=DEV)
    sub = {key: out[key][:, :, sel] for key in ("direction", "n_eff", "confidence", "count")}
    compare(sub, ref, "bf16", decidable_rows(q, k, True, kw, variant, rows=rows), f"T=65536 {variant}")


H8 = {key: val + val[::-1] for key, val in H4.items()}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_decode_variant(name, d):
    """Split-KV decode (one query head per KV head) and the grouped kernel (4 and 8 query
    heads per KV head: the lanes of a key split the heads), several split counts; the
    oracle sees the query as the last row of a causal problem."""
    variant = VARIANTS[name]
    for H, Hkv, kw in ((4, 4, H4), (4, 1, H4), (8, 1, H8)):
        q, k, v, _ = pin.random_qkv(2, H, Hkv, 1, 700, d, torch.bfloat16, seed=740 + H + Hkv + d)
        ref = polar_attention_variant(to_np(q), to_np(k), to_np(v), causal=True, variant=variant, **kw)
        ok = decidable_rows(q, k, True, kw, variant)
        for splits in (1, 3, 0):
            out = pa.decode(q.to(DEV), k.to(DEV), v.to(DEV), num_splits=splits, stats=True, variant=variant, **kw)
            torch.cuda.synchronize()
            compare(out, ref, "bf16", ok, f"decode {name} d={d} H={H} Hkv={Hkv} S={splits}")


@pytest.mark.parametrize("name", ["window", "soft", "all", "qnorm"])
def test_paged_decode_variant(name):
    """Paged grouped decode with per-sequence lengths: the window keeps the last W keys of
    each sequence."""
    variant = VARIANTS[name]
    B, H, Hkv, d = 3, 8, 2, 128
    lens = [20, 333, 700]
    q, k, v, _ = pin.random_qkv(B, H, Hkv, 1, max(lens), d, torch.bfloat16, seed=760)
    kp, vp, table = make_paged(k, v, 16, 761)
    kw = dict(len_temp=[0.1] * H, null_bias=[-1.0, -2.0, 0.0, 0.5] * 2, count_scale=[1.0, 2.0] * 4)
    out = pa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), torch.tensor(lens, dtype=torch.int32,
                          device=DEV), seq_k=max(lens), num_splits=3, stats=True, variant=variant, **kw)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        qb, kb, vb = q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L]
        ref = polar_attention_variant(to_np(qb), to_np(kb), to_np(vb), causal=True, variant=variant, **kw)
        one = {key: t[b:b + 1] for key, t in out.items() if torch.is_tensor(t) and key != "partials"}
        compare(one, ref, "bf16", decidable_rows(qb, kb, True, kw, variant), f"paged {name} b={b} len={L}")


@pytest.mark.parametrize("name", ["soft", "gate", "log1p", "gumbel2"])
def test_merge_variant_of_oracle_partials(name):
    """The GPU merge of split statistics the oracle computed under the variant equals the
    oracle's merge (fp32 tolerance: no bf16 input here)."""
    variant = VARIANTS[name]
    d, n, H = 64, 90, 2
    r = np.random.default_rng(770)
    q, k, v = r.normal(size=(H, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    scale = 1.0 / math.sqrt(d)
    H = 3
    q = r.normal(size=(H, d))
    taus, betas, kappas = [0.1, 0.3, 0.0], [-2.0, -1.0, 3.0], [1.0, 2.0, 1.0]  # head 2: nothing above the floor
    cuts = [0, 20, 21, 60, 90]
    parts = np.zeros((1, H, 1, len(cuts) - 1, d + 3))
    refs = []
    for h in range(H):
        rows = [split_statistics_variant(q[h], k, v, a, b, n, taus[h], betas[h], scale, variant)
                for a, b in zip(cuts[:-1], cuts[1:])]
        for s, (m, s1, s2, acc) in enumerate(rows):
            parts[0, h, 0, s, :3] = (m, s1, s2)
            parts[0, h, 0, s, 3:] = acc
        refs.append(merge_variant(rows, q[h], n, taus[h], betas[h], kappas[h], scale, variant))
    out = pa.merge(torch.tensor(parts, dtype=torch.float32, device=DEV), seq_k=n, causal=False, len_temp=taus,
                   null_bias=betas, count_scale=kappas, stats=True, variant=variant)
    torch.cuda.synchronize()
    ref = {key: np.array([[[refs[h][key]] for h in range(H)]]) for key in ("n_eff", "confidence", "count", "m", "s1",
                                                                           "s2")}
    ref["direction"] = np.array([[[refs[h]["direction"]] for h in range(H)]])
    # the GPU takes no threshold decision here (the partials are given): every row counts
    compare(out, ref, "f32", np.ones((1, H, 1), dtype=bool), f"merge {name}")


def test_chunked_prefill_with_soft_floor():
    """Chunked prefill under the soft per-key floor: a cached prefix (no mask) and the new
    chunk (causal) merge into the one-pass result."""
    variant = dict(key_floor="soft")
    B, H, P, C, d = 1, 4, 150, 60, 128
    T = P + C
    q, k, v, _ = pin.random_qkv(B, H, H, C, T, d, torch.bfloat16, seed=780)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    parts = pa.fwd_partial(qd, kd[:, :, :P].contiguous(), vd[:, :, :P].contiguous(), causal=False, context_k=T,
                           num_splits=2, split=0, variant=variant, **H4)
    pa.fwd_partial(qd, kd[:, :, P:].contiguous(), vd[:, :, P:].contiguous(), causal=True, context_k=T,
                   partials=parts, num_splits=2, split=1, variant=variant, **H4)
    out = pa.merge(parts, seq_k=T, causal=True, variant=variant, **H4)
    torch.cuda.synchronize()
    ref = polar_attention_variant(to_np(q), to_np(k), to_np(v), causal=True, variant=variant, **H4)
    compare(out, ref, "bf16", decidable_rows(q, k, True, H4, variant), "chunked soft floor")


def test_default_variant_is_bitwise_reading_r():
    """An all-default variant struct selects exactly the default kernels."""
    q, k, v, _ = pin.random_qkv(1, 2, 2, 200, 200, 64, torch.bfloat16, seed=790)
    a = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), stats=True)
    b = pa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), stats=True, variant=dict(temperature="log", window=0))
    torch.cuda.synchronize()
    for key in ("direction", "n_eff", "confidence", "count", "stats"):
        assert torch.equal(a[key], b[key]), key

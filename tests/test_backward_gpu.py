"""GPU parity of the backward (polar_attn_bwd) against the fp64 gradient oracle.

Both sides see the same input values (bf16 inputs widened exactly); the oracle computes
in fp64.  Metric, per output tensor: max |gpu - oracle| over the tensor divided by
max |oracle|.
  fp32 inputs: the kernels compute in fp32; every output element is an fp32 sum over at
    most n visible terms (keys for dq, query rows times the group for dk and dv) of
    products whose size the largest output bounds, so its error stays within a small
    multiple of n * 2^-24: BWD_TOL = 1e-4 for the cases here (n <= 1200).
  bf16 inputs: the matrix-core path rounds P, dS and w to bf16 (relative 2^-9 each) and
    takes the row statistics from the bf16 forward (n_eff within 1e-2), so an output is
    off by a few times 2^-9 of the largest one: BWD_TOL_BF16 = 2e-2, the forward's bound
    for the direction.
A tensor whose exact gradient is zero (no upstream gradient reaches it) must come back
exactly zero.
"""
import numpy as np
import pytest
import torch

import long_context_attention_polar_amd as pa
import polar_inputs as pin
from oracle import polar_attention_backward
from tests.parity import to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BWD_TOL = 1e-4
BWD_TOL_BF16 = 2e-2
IDENTITY_TOL = 1e-4
ALL = ("direction", "n_eff", "confidence", "count")


def compare(out, ref, label, tol=BWD_TOL):
    errs = {}
    for key in ("dq", "dk", "dv"):
        g, r = to_np(out[key]), ref[key]
        assert g.shape == r.shape, (label, key)
        assert np.isfinite(g).all(), f"{label} {key} not finite"
        top = np.abs(r).max() if r.size else 0.0
        if top == 0.0:
            assert not np.any(g), f"{label} {key} should be exactly zero"
            errs[key] = 0.0
            continue
        errs[key] = float(np.abs(g - r).max() / top)
        assert errs[key] <= tol, f"{label} {key}: {errs[key]:.3e} > {tol:.0e} ({errs})"
    print(f"[bwd] {label} {errs}", flush=True)
    return errs


def bwd_case(B, H, Hkv, Tq, Tk, d, dtype, causal, seed, tau=None, beta=None, kappa=None, names=ALL, scale=None,
             variant=None):
    label = f"B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} {dtype} causal={causal} grads={names}"
    if variant:
        label += f" variant={variant}"
    print(f"[bwd] {label}", flush=True)
    q, k, v, _ = pin.random_qkv(B, H, Hkv, Tq, Tk, d, dtype, seed)
    gr = pin.random_grads(B, H, Tq, d, seed + 7, names)
    ref = polar_attention_backward(to_np(q), to_np(k), to_np(v), {n: t.double().numpy() for n, t in gr.items()},
                                   causal=causal, len_temp=tau, null_bias=beta, count_scale=kappa,
                                   softmax_scale=scale, variant=variant)
    out = pa.bwd(q.to(DEV), k.to(DEV), v.to(DEV), {n: t.to(DEV) for n, t in gr.items()}, causal=causal,
                 len_temp=tau, null_bias=beta, count_scale=kappa, softmax_scale=scale, variant=variant)
    torch.cuda.synchronize()
    return compare(out, ref, label, BWD_TOL if dtype == torch.float32 else BWD_TOL_BF16)


TAU4 = [0.05, 0.0, 0.2, 0.1]
BETA4 = [0.0, -1.0, 1.5, 0.5]
KAPPA4 = [1.0, 2.0, 0.5, 4.0]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_against_oracle(d, dtype, causal):
    """Several row blocks and LDS tiles with ragged tails, GQA groups of 2, per-head
    temperature, floor and saturation."""
    Tq, Tk = (150, 150) if causal else (70, 201)
    bwd_case(2, 4, 2, Tq, Tk, d, dtype, causal, seed=500 + d + causal, tau=TAU4, beta=BETA4, kappa=KAPPA4)


# the reading variants that change only per-row constants (temperature, count-only floor
# level, saturation); tau ln n needs positive tau to keep the logits
BWD_VARIANTS = {
    "ssmax": (dict(temperature="ssmax"), [0.3, 0.5, 0.2, 0.4]),
    "train_ratio": (dict(temperature="train_ratio", train_len=64), TAU4),
    "gumbel2": (dict(floor_level="gumbel2"), TAU4),
    "log1p": (dict(saturation="log1p"), TAU4),
    "combined": (dict(temperature="ssmax", floor_level="gumbel2", saturation="log1p"), [0.3, 0.5, 0.2, 0.4]),
}


@pytest.mark.parametrize("name", sorted(BWD_VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bwd_variant_against_oracle(name, d, dtype):
    """The backward under each reading variant it supports, against the gradient oracle
    under the same variant (causal, ragged tails, GQA groups of 2)."""
    variant, tau = BWD_VARIANTS[name]
    bwd_case(2, 4, 2, 150, 150, d, dtype, True, seed=700 + d, tau=tau, beta=BETA4, kappa=KAPPA4, variant=variant)


def test_bwd_variant_non_causal_and_floor_off():
    variant, tau = BWD_VARIANTS["combined"]
    bwd_case(1, 4, 4, 70, 201, 64, torch.bfloat16, False, seed=733, tau=tau, beta=BETA4, kappa=KAPPA4,
             variant=variant)
    bwd_case(1, 4, 4, 100, 100, 128, torch.bfloat16, True, seed=734, tau=tau, beta=None, kappa=KAPPA4,
             variant=variant)


def test_bwd_rejects_variants_that_change_the_gradient():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16, device=DEV)
    gr = {"n_eff": torch.zeros(1, 4, 8, device=DEV)}
    for variant in (dict(key_floor="soft"), dict(key_floor="gate"), dict(window=4), dict(floor_level="qnorm")):
        with pytest.raises(pa.PolarError):
            pa.bwd(q, q, q, gr, null_bias=BETA4, variant=variant)


@pytest.mark.parametrize("name", ALL)
def test_bwd_each_upstream_channel(name):
    """One upstream gradient at a time, so each term of the row constants dominates its
    own case."""
    bwd_case(1, 2, 1, 100, 100, 128, torch.bfloat16, True, seed=520, tau=[0.1, 0.0], beta=[0.5, -0.5],
             kappa=[1.0, 3.0], names=(name,))


def test_bwd_rows_at_end_of_keys_group_of_four():
    """Causal with fewer query rows than keys (rows aligned to the end), 4 query heads
    per KV head."""
    bwd_case(1, 8, 2, 37, 300, 64, torch.float32, True, seed=530, tau=[0.02 * h for h in range(8)],
             beta=[0.0] * 8)


@pytest.mark.parametrize("Tq,Tk,causal", [(1, 1, True), (1, 1, False), (33, 33, True), (1, 77, True), (5, 1, False)])
def test_bwd_tiny(Tq, Tk, causal):
    """One key (n_eff = 1, ln n = 0) and one-row problems; the first causal row sees one key."""
    bwd_case(1, 2, 2, Tq, Tk, 64, torch.float32, causal, seed=540 + Tq + Tk, beta=[0.0, 1.0], kappa=[1.0, 2.0])


def _split_free_workspace(B, H, Tq, d):
    rows = B * H * Tq
    up = lambda x: (x + 255) // 256 * 256
    return up(rows * (d + 3) * 4) + up(rows * d * 2) + up(rows * 16)


@pytest.mark.parametrize("B,H,Hkv,Tq,Tk,d,causal,runs", [
    (1, 16, 16, 24, 4096, 64, False, 1),   # 16 * 32 = 512 key tiles, full mask: one run each
    (4, 16, 16, 16, 4096, 128, True, 1),   # 4 * 16 * 32 = 2048 key tiles, causal: one run each
    (1, 16, 8, 24, 4096, 128, False, 2),   # 256 key tiles, full mask: two runs each
])
def test_bwd_key_tile_runs(B, H, Hkv, Tq, Tk, d, causal, runs):
    """dk and dv with the key side's work in one run per 128-key tile (written directly)
    and in two runs (partial sums added by a second kernel); the workspace size says
    which."""
    prob = pa.Problem(batch=B, heads=H, kv_heads=Hkv, seq_q=Tq, seq_k=Tk, head_dim=d, causal=causal,
                      dtype=pa.POLAR_BF16)
    extra = 0 if runs == 1 else 2 * runs * B * Hkv * Tk * d * 4
    assert pa.bwd_workspace_bytes(prob) == _split_free_workspace(B, H, Tq, d) + extra
    bwd_case(B, H, Hkv, Tq, Tk, d, torch.bfloat16, causal, seed=570 + d + runs, tau=[0.05] * H,
             beta=[0.5] * H)


def test_bwd_explicit_softmax_scale_and_floor_off():
    bwd_case(1, 2, 1, 64, 96, 128, torch.bfloat16, True, seed=550, tau=[0.1, 0.3], scale=0.3)


def test_bwd_constant_confidence_gives_zero():
    """With the floor off the confidence is the constant 1: its gradient alone gives
    exactly zero dq, dk, dv."""
    errs = bwd_case(1, 2, 2, 40, 40, 64, torch.bfloat16, True, seed=560, names=("confidence",))
    assert errs == {"dq": 0.0, "dk": 0.0, "dv": 0.0}


def test_bwd_no_query_rows():
    """seq_q == 0: dq is empty and dk, dv are written as zeros."""
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(1, 2, 50, 64, device=DEV, generator=torch.Generator(device=DEV).manual_seed(91)).to(torch.bfloat16)
    out = pa.bwd(q, k, k.clone(), {}, causal=False)
    torch.cuda.synchronize()
    assert out["dq"].numel() == 0
    assert torch.all(out["dk"] == 0) and torch.all(out["dv"] == 0)


def test_bwd_rejects_bad_gradients():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        pa.bwd(q, q, q, {"n_eff": torch.zeros(1, 2, 7, device=DEV)})
    with pytest.raises(ValueError):
        pa.bwd(q, q, q, {"direction": torch.zeros(1, 2, 8, 64, dtype=torch.float64, device=DEV)})
    with pytest.raises(ValueError):
        pa.bwd(q, q, q, {"logits": torch.zeros(1, 2, 8, device=DEV)})


@pytest.mark.parametrize("B,H,Hkv,Tq,Tk,d,causal", [
    (1, 4, 4, 300, 300, 64, True), (2, 4, 2, 130, 130, 128, True), (1, 2, 1, 77, 200, 64, False),
    (1, 4, 1, 1000, 1000, 128, True), (1, 2, 2, 1, 65, 128, True), (1, 2, 2, 64, 64, 64, False)])
def test_bwd_saved_statistics_bitwise(B, H, Hkv, Tq, Tk, d, causal):
    """polar_attn_bwd_saved fed the one-split partial forward gives exactly what
    polar_attn_bwd gives: the same kernels run, only the forward pass inside the call is
    replaced by the caller's statistics."""
    print(f"[bwd] saved statistics B={B} H={H} Hkv={Hkv} Tq={Tq} Tk={Tk} d={d} causal={causal}", flush=True)
    q, k, v, _ = pin.random_qkv(B, H, Hkv, Tq, Tk, d, torch.bfloat16, seed=Tq + d)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    gr = {n: t.to(DEV) for n, t in pin.random_grads(B, H, Tq, d, Tq + 3).items()}
    kw = dict(causal=causal, len_temp=[0.05 * (h % 3) for h in range(H)], null_bias=[0.5 * h - 1.0 for h in range(H)],
              count_scale=[1.0 + h for h in range(H)])
    ref = pa.bwd(q, k, v, gr, **kw)
    saved = pa.fwd_partial(q, k, v, **kw)
    got = pa.bwd(q, k, v, gr, saved=saved, **kw)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert torch.equal(ref[key], got[key]), key


def test_bwd_saved_statistics_bitwise_under_a_variant():
    """The saved-statistics backward under a variant: the caller's partial forward takes
    the same variant (its temperature sets the weights), and the results are bitwise those
    of the self-contained call."""
    variant, tau = BWD_VARIANTS["combined"]
    q, k, v, _ = pin.random_qkv(1, 4, 2, 300, 300, 128, torch.bfloat16, seed=741)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    gr = {n: t.to(DEV) for n, t in pin.random_grads(1, 4, 300, 128, 742).items()}
    kw = dict(causal=True, len_temp=tau, null_bias=BETA4, count_scale=KAPPA4, variant=variant)
    ref = pa.bwd(q, k, v, gr, **kw)
    saved = pa.fwd_partial(q, k, v, **kw)
    got = pa.bwd(q, k, v, gr, saved=saved, **kw)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert torch.equal(ref[key], got[key]), key


def test_bwd_saved_statistics_no_rows_and_fp32():
    k = torch.randn(1, 2, 50, 64, device=DEV, generator=torch.Generator(device=DEV).manual_seed(92)).to(torch.bfloat16)
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    saved = torch.empty(1, 2, 0, 67, device=DEV)
    out = pa.bwd(q, k, k.clone(), {}, causal=False, saved=saved)
    torch.cuda.synchronize()
    assert torch.all(out["dk"] == 0) and torch.all(out["dv"] == 0)
    q32 = torch.zeros(1, 2, 8, 64, device=DEV)
    with pytest.raises(pa.PolarError):
        pa.bwd(q32, q32, q32, {}, saved=torch.zeros(1, 2, 8, 67, device=DEV))
    with pytest.raises(ValueError):
        pa.bwd(q.new_zeros(1, 2, 8, 64), k, k, {}, causal=False, saved=torch.zeros(1, 2, 8, 66, device=DEV))


def test_workload_backward_saved_16k():
    """The benchmark's backward workload from saved statistics equals the self-contained
    backward bitwise at full size."""
    w = pin.WORKLOADS["bf16_bwd_b1_h16_kv4_t16384_d128"]
    print("[bwd] saved statistics, workload", w.name, flush=True)
    q, k, v, _ = pin.workload_inputs(w, DEV)
    gr = {n: t.to(DEV) for n, t in pin.random_grads(w.B, w.H, w.Tq, w.d, w.extra["grad_seed"]).items()}
    kw = dict(causal=True, len_temp=w.len_temp(), null_bias=w.null_bias(), count_scale=w.count_scale())
    ref = pa.bwd(q, k, v, gr, **kw)
    saved = pa.fwd_partial(q, k, v, **kw)
    got = pa.bwd(q, k, v, gr, saved=saved, **kw)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert torch.equal(ref[key], got[key]), key


def test_workload_backward_16k():
    """The benchmark's backward workload at full size: dq of sampled rows and dk, dv of
    two key tiles against the oracle (row i alone over its visible keys gives the same
    dq_i), and two identities of the gradient that hold at any size:
      sum_j <v_j, dv_j> = 0          (the outputs do not change when all values are scaled)
      sum_i <q_i, dq_i> = sum_j <k_j, dk_j>  per KV group  (scores are bilinear in q, k)."""
    w = pin.WORKLOADS["bf16_bwd_b1_h16_kv4_t16384_d128"]
    print("[bwd] workload", w.name, flush=True)
    q, k, v, _ = pin.workload_inputs(w, "cpu")
    gr = pin.random_grads(w.B, w.H, w.Tq, w.d, w.extra["grad_seed"])
    tau, beta, kappa = w.len_temp(), w.null_bias(), w.count_scale()
    out = pa.bwd(q.to(DEV), k.to(DEV), v.to(DEV), {n: t.to(DEV) for n, t in gr.items()}, causal=True,
                 len_temp=tau, null_bias=beta, count_scale=kappa)
    torch.cuda.synchronize()
    dq, dk, dv = out["dq"].double().cpu(), out["dk"].double().cpu(), out["dv"].double().cpu()
    for key, t in out.items():
        assert torch.isfinite(t).all(), key
    group = w.H // w.Hkv
    r = np.random.default_rng(81)
    for h, i in [(0, 0), (15, w.Tq - 1), (5, 1)] + [(int(a), int(b)) for a, b in
                                                    zip(r.integers(0, w.H, 6), r.integers(0, w.Tq, 6))]:
        n = i + 1
        hk = h // group
        row = {nm: t[:, h:h + 1, i:i + 1].double().numpy() for nm, t in gr.items()}
        ref = polar_attention_backward(to_np(q[:, h:h + 1, i:i + 1]), to_np(k[:, hk:hk + 1, :n]),
                                       to_np(v[:, hk:hk + 1, :n]), row, causal=False, len_temp=[tau[h]],
                                       null_bias=[beta[h]], count_scale=[kappa[h]])
        want = ref["dq"][0, 0, 0]
        got = dq[0, h, i].numpy()
        err = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
        print(f"[bwd] workload dq row h={h} i={i}: {err:.2e}", flush=True)
        assert err <= BWD_TOL_BF16, (h, i, err)
    # dk and dv of sampled key tiles, element by element: under the causal mask key j
    # receives gradient only from rows i >= j, so the oracle run on the rows from the
    # tile's first key on (a query chunk aligned to the end of the keys, whose rows keep
    # their visible counts) gives those keys' complete dk and dv
    hk = 1
    heads = slice(hk * group, (hk + 1) * group)
    for j0, nkeys in ((w.Tk - 256, 256), (w.Tk // 2, 128)):
        rows = {nm: t[:, heads, j0:].double().numpy() for nm, t in gr.items()}
        ref = polar_attention_backward(to_np(q[:, heads, j0:]), to_np(k[:, hk:hk + 1]), to_np(v[:, hk:hk + 1]),
                                       rows, causal=True, len_temp=tau[heads], null_bias=beta[heads],
                                       count_scale=kappa[heads])
        for name, got in (("dk", dk), ("dv", dv)):
            want = ref[name][0, 0, j0:j0 + nkeys]
            g = got[0, hk, j0:j0 + nkeys].numpy()
            err = np.abs(g - want).max() / np.abs(want).max()
            print(f"[bwd] workload {name} keys [{j0}, {j0 + nkeys}) hk={hk}: {err:.2e}", flush=True)
            assert err <= BWD_TOL_BF16, (name, j0, err)
    # identities of the gradient, which hold to fp32 rounding of the sums (measured
    # <= 1e-5 relative), at 1e-4
    qd, kd, vd = q.double(), k.double(), v.double()
    for hk in range(w.Hkv):
        heads = slice(hk * group, (hk + 1) * group)
        sv = float((vd[0, hk] * dv[0, hk]).sum())
        sv_abs = float((vd[0, hk] * dv[0, hk]).abs().sum())
        print(f"[bwd] workload identities hk={hk}: v.dv {abs(sv) / sv_abs:.2e}", flush=True)
        assert abs(sv) <= IDENTITY_TOL * sv_abs, (hk, sv, sv_abs)
        lhs = float((qd[0, heads] * dq[0, heads]).sum())
        rhs = float((kd[0, hk] * dk[0, hk]).sum())
        scale = float((qd[0, heads] * dq[0, heads]).abs().sum())
        print(f"[bwd] workload identities hk={hk}: q.dq - k.dk {abs(lhs - rhs) / scale:.2e}", flush=True)
        assert abs(lhs - rhs) <= IDENTITY_TOL * scale, (hk, lhs, rhs, scale)

"""Pins of the backward oracle (CPU).

The gradient oracle is pinned to things other than itself: central finite differences
of the forward oracle along random directions, torch autograd in float64 through a
forward written here independently with torch operations, and a closed form (n_eff is
stationary at uniform logits).  tests/test_backward_mutations.py checks that these pins
catch plausible mistakes.
"""
import importlib
import math

import numpy as np
import pytest
import torch

import oracle.polar_backward as pb_default
from oracle import polar_attention
from oracle.polar_variants import polar_attention_variant

CASES = [
    # B, H, Hkv, Tq, Tk, d, causal, tau, beta, kappa
    (1, 2, 1, 6, 6, 4, True, [0.0, 0.3], [0.0, -1.0], [1.0, 2.0]),
    (2, 2, 2, 5, 7, 3, True, [0.1, 0.0], None, None),
    (1, 3, 3, 4, 9, 5, False, [0.2, 0.0, 0.1], [1.5, 0.0, -0.5], [1.0, 4.0, 1.0]),
]


# the reading variants that change only per-row constants, each with a case whose length
# temperatures are all positive (tau ln n with tau = 0 would zero every logit)
VARIANT_CASES = [
    ({"temperature": "ssmax", "saturation": "log1p"},
     (1, 2, 1, 6, 6, 4, True, [0.5, 0.8], [0.0, -1.0], [1.0, 2.0])),
    ({"temperature": "train_ratio", "train_len": 16, "floor_level": "gumbel2"},
     (2, 2, 2, 5, 7, 3, True, [0.1, 0.0], [0.5, -0.5], [2.0, 1.0])),
    ({"floor_level": "gumbel2", "saturation": "log1p"},
     (1, 3, 3, 4, 9, 5, False, [0.2, 0.0, 0.1], [1.5, 0.0, -0.5], [1.0, 4.0, 1.0])),
    ({"saturation": "log1p"}, (1, 2, 1, 6, 6, 4, True, [0.0, 0.3], None, [1.0, 0.5])),
]


def loss(q, k, v, gr, causal, tau, beta, kappa, variant=None):
    if variant is None:
        out = polar_attention(q, k, v, causal=causal, len_temp=tau, null_bias=beta, count_scale=kappa)
    else:
        out = polar_attention_variant(q, k, v, causal=causal, len_temp=tau, null_bias=beta, count_scale=kappa,
                                      variant=variant)
    return float(np.sum(gr["direction"] * out["direction"]) + np.sum(gr["n_eff"] * out["n_eff"]) +
                 np.sum(gr["confidence"] * out["confidence"]) + np.sum(gr["count"] * out["count"]))


def case_inputs(B, H, Hkv, Tq, Tk, d, seed):
    r = np.random.default_rng(seed)
    q = r.normal(size=(B, H, Tq, d))
    k = r.normal(size=(B, Hkv, Tk, d))
    v = r.normal(size=(B, Hkv, Tk, d))
    gr = {"direction": r.normal(size=(B, H, Tq, d)), "n_eff": r.normal(size=(B, H, Tq)),
          "confidence": r.normal(size=(B, H, Tq)), "count": r.normal(size=(B, H, Tq))}
    return q, k, v, gr, r


def fd_check(mod, case, seed=0, eps=1e-5, tol=1e-6, variant=None):
    B, H, Hkv, Tq, Tk, d, causal, tau, beta, kappa = case
    q, k, v, gr, r = case_inputs(B, H, Hkv, Tq, Tk, d, seed)
    kw = {} if variant is None else {"variant": variant}
    g = mod.polar_attention_backward(q, k, v, gr, causal=causal, len_temp=tau, null_bias=beta, count_scale=kappa,
                                     **kw)
    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(3):
            delta = r.normal(size=x.shape)
            args = {"q": q, "k": k, "v": v}
            key = name[1]
            hi = dict(args)
            lo = dict(args)
            hi[key] = x + eps * delta
            lo[key] = x - eps * delta
            num = (loss(hi["q"], hi["k"], hi["v"], gr, causal, tau, beta, kappa, variant) -
                   loss(lo["q"], lo["k"], lo["v"], gr, causal, tau, beta, kappa, variant)) / (2 * eps)
            ana = float(np.sum(g[name] * delta))
            err = abs(num - ana) / max(1.0, abs(num))
            worst = max(worst, err)
            assert err <= tol, (name, num, ana)
    return worst


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    fd_check(pb_default, case)


@pytest.mark.parametrize("variant,case", VARIANT_CASES, ids=[str(v) for v, _ in VARIANT_CASES])
def test_backward_variant_matches_finite_differences(variant, case):
    """Under the row-constant reading variants the gradient oracle is the derivative of
    the variant forward oracle (an independent row-by-row definition)."""
    fd_check(pb_default, case, variant=variant)


def test_backward_default_variant_is_reading_r():
    """An explicit default variant gives the same gradients as none."""
    case = CASES[0]
    B, H, Hkv, Tq, Tk, d, causal, tau, beta, kappa = case
    q, k, v, gr, _ = case_inputs(B, H, Hkv, Tq, Tk, d, 3)
    kw = dict(causal=causal, len_temp=tau, null_bias=beta, count_scale=kappa)
    a = pb_default.polar_attention_backward(q, k, v, gr, **kw)
    b = pb_default.polar_attention_backward(q, k, v, gr, variant={"temperature": "log", "floor_level": "gauss",
                                                                  "saturation": "log"}, **kw)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("variant", [{"key_floor": "soft"}, {"window": 4}, {"floor_level": "qnorm"}])
def test_backward_rejects_variants_that_change_the_map(variant):
    B, H, Hkv, Tq, Tk, d, causal, tau, beta, kappa = CASES[0]
    q, k, v, gr, _ = case_inputs(B, H, Hkv, Tq, Tk, d, 0)
    with pytest.raises(ValueError):
        pb_default.polar_attention_backward(q, k, v, gr, causal=True, len_temp=tau, null_bias=beta,
                                            count_scale=kappa, variant=variant)


def torch_forward(q, k, v, causal, tau, beta, kappa):
    """The forward definition once more, in torch (float64), for autograd."""
    B, H, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    group = H // Hkv
    i = torch.arange(Tq, dtype=torch.float64)
    n = torch.clamp(i + 1 + (Tk - Tq), max=Tk) if causal else torch.full((Tq,), float(Tk), dtype=torch.float64)
    mask = torch.arange(Tk)[None, :] < n[:, None]
    terms = []
    for h in range(H):
        kh, vh = k[:, h // group], v[:, h // group]
        lam = 1.0 + (0.0 if tau is None else tau[h]) * torch.log(n)
        s = (lam / math.sqrt(d))[None, :, None] * torch.einsum("bid,bjd->bij", q[:, h], kh)
        s = s.masked_fill(~mask[None], float("-inf"))
        z = torch.logsumexp(s, dim=-1)                      # log Z1
        a = torch.softmax(s, dim=-1)                        # P_j / Z1
        n_eff = 1.0 / (a * a).sum(-1)
        acc = torch.einsum("bij,bjd->bid", a, vh)
        u = acc / acc.norm(dim=-1, keepdim=True)
        if beta is None:
            conf = torch.ones_like(z)
        else:
            f = lam * torch.sqrt(2.0 * torch.log(n)) + beta[h]
            conf = torch.sigmoid(z - f[None, :])
        kap = 1.0 if kappa is None else kappa[h]
        count = conf * torch.tanh(torch.log(n_eff) / kap)
        terms.append((u, n_eff, conf, count))
    return [torch.stack([t[j] for t in terms], dim=1) for j in range(4)]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_torch_autograd(case):
    B, H, Hkv, Tq, Tk, d, causal, tau, beta, kappa = case
    q, k, v, gr, _ = case_inputs(B, H, Hkv, Tq, Tk, d, 7)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    u, n_eff, conf, count = torch_forward(tq, tk, tv, causal, tau, beta, kappa)
    L = ((torch.tensor(gr["direction"]) * u).sum() + (torch.tensor(gr["n_eff"]) * n_eff).sum() +
         (torch.tensor(gr["confidence"]) * conf).sum() + (torch.tensor(gr["count"]) * count).sum())
    L.backward()
    g = pb_default.polar_attention_backward(q, k, v, gr, causal=causal, len_temp=tau, null_bias=beta,
                                            count_scale=kappa)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def test_n_eff_is_stationary_at_uniform_logits():
    """q = 0 makes every logit 0: n_eff = n is a maximum in the logits, so its gradient
    with respect to q, k and v vanishes."""
    r = np.random.default_rng(3)
    q = np.zeros((1, 2, 5, 4))
    k = r.normal(size=(1, 2, 5, 4))
    v = r.normal(size=(1, 2, 5, 4))
    gr = {"n_eff": np.ones((1, 2, 5))}
    g = pb_default.polar_attention_backward(q, k, v, gr, causal=True, len_temp=[0.2, 0.0])
    for name in ("dq", "dk", "dv"):
        assert np.abs(g[name]).max() < 1e-12, name


@pytest.mark.parametrize("case", CASES)
def test_backward_invariance_identities(case):
    """Identities from invariances of the forward, independent of how the gradient is
    written: scaling every value leaves all outputs unchanged (sum <v, dv> = 0); the
    scores are bilinear in q and k (sum <q, dq> = sum <k, dk> per KV head); with the
    floor off, shifting every key by one vector shifts each row's logits by a constant
    (sum_j dk_j = 0 per KV head)."""
    B, H, Hkv, Tq, Tk, d, causal, tau, beta, kappa = case
    q, k, v, gr, _ = case_inputs(B, H, Hkv, Tq, Tk, d, seed=3)
    g = pb_default.polar_attention_backward(q, k, v, gr, causal=causal, len_temp=tau, null_bias=beta,
                                            count_scale=kappa)
    group = H // Hkv
    for b in range(B):
        for hk in range(Hkv):
            heads = slice(hk * group, (hk + 1) * group)
            assert abs(np.sum(v[b, hk] * g["dv"][b, hk])) <= 1e-10 * np.sum(np.abs(v[b, hk] * g["dv"][b, hk]))
            lhs = np.sum(q[b, heads] * g["dq"][b, heads])
            rhs = np.sum(k[b, hk] * g["dk"][b, hk])
            assert abs(lhs - rhs) <= 1e-10 * np.sum(np.abs(q[b, heads] * g["dq"][b, heads]))
    g0 = pb_default.polar_attention_backward(q, k, v, gr, causal=causal, len_temp=tau, null_bias=None,
                                             count_scale=kappa)
    shift = g0["dk"].sum(axis=2)
    assert np.abs(shift).max() <= 1e-10 * np.abs(g0["dk"]).sum(axis=2).max()

"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms of the
definitions in the ATMA technical summary, section 2.1 (direction on the unit sphere,
participation ratio, bounded tanh-of-log count), textbook softmax attention from a
library routine, invariants of the definitions, hand-worked fixtures, and the algebra
of the streaming accumulators with squared correction factors (section 2.2).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (finish_rows, length_temperature, merge_reference, merge_statistics,
                    null_floor, polar_attention, split_statistics, visible_count)

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.default_rng(seed)


def normalize(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("tau", [0.0, 0.3])
def test_uniform_logits_neff_equals_visible_count(causal, tau):
    """q = 0 gives equal logits, so n_eff is exactly the number of visible keys and the
    direction is the normalised (prefix) sum of the visible values."""
    B, H, T, d = 1, 2, 37, 16
    r = rng(1)
    q = np.zeros((B, H, T, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, d))
    out = polar_attention(q, k, v, causal=causal, len_temp=[tau] * H)
    n = np.arange(1, T + 1) if causal else np.full(T, T)
    np.testing.assert_array_equal(out["n_eff"][0, 0], n.astype(np.float64))
    sums = np.cumsum(v, axis=2) if causal else np.repeat(v.sum(axis=2, keepdims=True), T, axis=2)
    np.testing.assert_allclose(out["direction"], normalize(sums), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(out["m"], 0.0)


def test_uniform_logits_bottom_right_alignment():
    """With fewer queries than keys, query row i is the (Tk - Tq + i)-th position, so it
    sees Tk - Tq + i + 1 keys."""
    Tq, Tk, d = 5, 23, 8
    r = rng(2)
    q = np.zeros((1, 1, Tq, d))
    k = r.standard_normal((1, 1, Tk, d))
    v = r.standard_normal((1, 1, Tk, d))
    out = polar_attention(q, k, v, causal=True)
    np.testing.assert_array_equal(out["n_eff"][0, 0], np.arange(Tk - Tq + 1, Tk + 1).astype(float))
    np.testing.assert_array_equal(visible_count(np.arange(Tq), Tq, Tk, True), np.arange(Tk - Tq + 1, Tk + 1))


def _planted(T, d, c, a, b, seed, positions=None):
    """All queries a*e0; keys orthogonal to e0 except c planted keys b*e0."""
    r = rng(seed)
    q = np.zeros((1, 1, T, d))
    q[..., 0] = a
    k = r.standard_normal((1, 1, T, d))
    k[..., 0] = 0.0
    pos = r.choice(T, size=c, replace=False) if positions is None else np.asarray(positions)
    k[0, 0, pos] = 0.0
    k[0, 0, pos, 0] = b
    v = r.standard_normal((1, 1, T, d))
    return q, k, v, np.sort(pos)


@pytest.mark.parametrize("c", [1, 4, 16])
@pytest.mark.parametrize("tau", [0.0, 0.25])
def test_dominant_keys_closed_form(c, tau):
    """c keys with logit Delta above n - c keys at logit 0:
    n_eff = (c + (n-c) e^-D)^2 / (c + (n-c) e^-2D), D = lam a b / sqrt(d);
    direction = normalize(sum_planted v + e^-D sum_rest v)."""
    T, d, a, b = 96, 16, 2.0, 3.0
    q, k, v, pos = _planted(T, d, c, a, b, seed=10 + c)
    out = polar_attention(q, k, v, causal=False, len_temp=[tau])
    n = T
    lam = 1.0 + tau * math.log(n)
    D = lam * a * b / math.sqrt(d)
    e1, e2 = math.exp(-D), math.exp(-2 * D)
    n_eff = (c + (n - c) * e1) ** 2 / (c + (n - c) * e2)
    mask = np.zeros(T, bool)
    mask[pos] = True
    acc = v[0, 0, mask].sum(0) + e1 * v[0, 0, ~mask].sum(0)
    np.testing.assert_allclose(out["n_eff"][0, 0], n_eff, rtol=1e-12)
    np.testing.assert_allclose(out["direction"][0, 0], np.broadcast_to(normalize(acc), (T, d)), atol=1e-12)
    np.testing.assert_allclose(out["m"][0, 0], D, rtol=1e-13)
    np.testing.assert_allclose(out["s1"][0, 0], c + (n - c) * e1, rtol=1e-12)
    np.testing.assert_allclose(out["s2"][0, 0], c + (n - c) * e2, rtol=1e-12)


def test_dominant_key_causal_rows_closed_form():
    """Causal, one planted key at position p: rows before p see equal logits (n_eff = i+1);
    rows from p on follow the one-dominant closed form with n = i + 1 and lam_i."""
    T, d, a, b, tau, p = 64, 8, 1.5, 2.0, 0.4, 20
    q, k, v, _ = _planted(T, d, 1, a, b, seed=7, positions=[p])
    out = polar_attention(q, k, v, causal=True, len_temp=[tau], null_bias=[0.5])
    for i in range(T):
        n = i + 1
        got = out["n_eff"][0, 0, i]
        if i < p:
            assert got == float(n)
            continue
        lam = 1.0 + tau * math.log(n)
        D = lam * a * b / math.sqrt(d)
        s1 = 1 + (n - 1) * math.exp(-D)
        s2 = 1 + (n - 1) * math.exp(-2 * D)
        assert got == pytest.approx(s1 * s1 / s2, rel=1e-12)
        f = lam * math.sqrt(2 * math.log(n)) + 0.5
        conf = s1 / (s1 + math.exp(f - D))
        assert out["confidence"][0, 0, i] == pytest.approx(conf, rel=1e-12)
        assert out["count"][0, 0, i] == pytest.approx(conf * math.tanh(math.log(s1 * s1 / s2)), rel=1e-11, abs=1e-15)


def test_neff_tends_to_match_count():
    """As the planted logit grows, n_eff -> c (the number of exact matches)."""
    for c in (1, 4, 16):
        q, k, v, _ = _planted(200, 16, c, 20.0, 20.0, seed=c)
        out = polar_attention(q, k, v, causal=False)
        np.testing.assert_allclose(out["n_eff"][0, 0], c, rtol=1e-9)


def test_floor_closed_form_uniform_logits():
    """q = 0: m = 0 and S1 = n, so conf = n / (n + exp(lam sqrt(2 ln n) + beta))."""
    T, d, tau, beta = 50, 8, 0.3, -1.25
    r = rng(3)
    q = np.zeros((1, 1, T, d))
    k, v = r.standard_normal((2, 1, 1, T, d))
    out = polar_attention(q, k, v, causal=True, len_temp=[tau], null_bias=[beta])
    for i in range(T):
        n = i + 1
        lam = 1 + tau * math.log(n)
        conf = n / (n + math.exp(lam * math.sqrt(2 * math.log(n)) + beta))
        assert out["confidence"][0, 0, i] == pytest.approx(conf, rel=1e-13)
        assert out["count"][0, 0, i] == pytest.approx(conf * (n * n - 1) / (n * n + 1), rel=1e-12, abs=1e-300)


def test_floor_off_and_beta_monotone():
    B, H, T, d = 1, 1, 40, 16
    r = rng(4)
    q, k, v = r.standard_normal((3, B, H, T, d))
    off = polar_attention(q, k, v, causal=True)
    np.testing.assert_array_equal(off["confidence"], 1.0)
    prev = None
    for beta in (-2.0, 0.0, 3.0):
        on = polar_attention(q, k, v, causal=True, null_bias=[beta])
        np.testing.assert_array_equal(on["direction"], off["direction"])
        np.testing.assert_array_equal(on["n_eff"], off["n_eff"])
        assert np.all((on["confidence"] > 0) & (on["confidence"] <= 1))
        if prev is not None:
            assert np.all(on["confidence"] < prev)
        prev = on["confidence"]


@pytest.mark.parametrize("kappa", [1.0, 4.0, 0.5])
def test_saturation_closed_form(kappa):
    """tanh(ln x / kappa) = (x^(2/kappa) - 1) / (x^(2/kappa) + 1): bounded in [0, 1) and
    monotone for n_eff >= 1."""
    B, H, T, d = 1, 1, 64, 8
    r = rng(5)
    q, k, v = r.standard_normal((3, B, H, T, d))
    out = polar_attention(q, k, v, causal=True, null_bias=[0.0], count_scale=[kappa])
    x = out["n_eff"] ** (2.0 / kappa)
    np.testing.assert_allclose(out["count"] / out["confidence"], (x - 1) / (x + 1), rtol=1e-12, atol=1e-15)
    assert np.all((out["count"] >= 0) & (out["count"] < 1))
    neff = np.linspace(1, 50, 1000)
    _, _, _, cnt = finish_rows(np.zeros(1000), neff, neff, np.ones((1000, 2)), np.full(1000, 10.0),
                               np.ones(1000), None, kappa)
    assert np.all(np.diff(cnt) > 0) and cnt[0] == 0.0 and cnt[-1] < 1


def test_first_causal_row():
    """Row 0 sees one key: lam = 1, n_eff = 1, direction = v0/|v0|, count = 0,
    floor = beta so conf = 1 / (1 + exp(beta - m)) with m = <q0, k0>/sqrt(d)."""
    B, H, T, d = 2, 3, 9, 32
    r = rng(6)
    q, k, v = r.standard_normal((3, B, H, T, d))
    beta = [0.0, 1.0, -2.0]
    out = polar_attention(q, k, v, causal=True, len_temp=[0.5, 1.0, 2.0], null_bias=beta)
    m0 = np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]) / math.sqrt(d)
    np.testing.assert_array_equal(out["n_eff"][:, :, 0], 1.0)
    np.testing.assert_allclose(out["direction"][:, :, 0], normalize(v[:, :, 0]), atol=1e-14)
    np.testing.assert_array_equal(out["count"][:, :, 0], 0.0)
    np.testing.assert_allclose(out["m"][:, :, 0], m0, rtol=1e-13)
    np.testing.assert_allclose(out["confidence"][:, :, 0], 1 / (1 + np.exp(np.array(beta)[None] - m0)), rtol=1e-13)


def test_temperature_helpers():
    assert length_temperature(1, 0.7) == 1.0
    assert length_temperature(np.e ** 2, 0.5) == pytest.approx(2.0)
    assert null_floor(1, 3.0, 0.25) == 0.25
    assert null_floor(np.e ** 8, 1.0, 0.0) == pytest.approx(4.0)


# --------------------------------------------------------------------------- library routines

@pytest.mark.parametrize("causal", [True, False])
def test_reduces_to_softmax_attention(causal):
    """tau = 0 and the floor off: the direction is the normalised output of textbook
    scaled-dot-product attention (torch, fp64, CPU), and n_eff is 1/sum of squared
    softmax probabilities (scipy)."""
    from scipy.special import softmax
    B, H, T, d = 2, 3, 45, 32
    r = rng(7)
    q, k, v = r.standard_normal((3, B, H, T, d))
    out = polar_attention(q, k, v, causal=causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal).numpy()
    np.testing.assert_allclose(out["direction"], normalize(ref), atol=1e-12)
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    P = softmax(s, axis=-1)
    np.testing.assert_allclose(out["n_eff"], 1.0 / (P ** 2).sum(-1), rtol=1e-12)


def test_length_temperature_equals_query_rescaling():
    """The length temperature multiplies row i's logits by lam_i = 1 + tau ln(i+1):
    the same as SDPA on queries scaled row-wise by lam_i."""
    B, H, T, d, tau = 1, 2, 33, 16, 0.35
    r = rng(8)
    q, k, v = r.standard_normal((3, B, H, T, d))
    out = polar_attention(q, k, v, causal=True, len_temp=[tau, tau])
    lam = 1 + tau * np.log(np.arange(1, T + 1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q * lam[:, None]), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    np.testing.assert_allclose(out["direction"], normalize(ref), atol=1e-12)


def test_explicit_softmax_scale():
    B, H, T, d = 1, 1, 20, 8
    r = rng(9)
    q, k, v = r.standard_normal((3, B, H, T, d))
    out = polar_attention(q, k, v, causal=True, softmax_scale=0.8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.8).numpy()
    np.testing.assert_allclose(out["direction"], normalize(ref), atol=1e-12)


# --------------------------------------------------------------------------- invariants

def test_key_permutation_invariance_noncausal():
    B, H, T, d = 1, 2, 31, 16
    r = rng(10)
    q, k, v = r.standard_normal((3, B, H, T, d))
    kw = dict(causal=False, len_temp=[0.1, 0.2], null_bias=[0.0, 1.0], count_scale=[1.0, 2.0])
    a = polar_attention(q, k, v, **kw)
    perm = r.permutation(T)
    b = polar_attention(q, k[:, :, perm], v[:, :, perm], **kw)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-12)


def test_duplication_invariance():
    """Count independence of the direction: duplicating every (k, v) pair leaves the
    direction unchanged and doubles n_eff (tau = 0, floor off, non-causal)."""
    B, H, T, d = 1, 2, 25, 16
    r = rng(11)
    q, k, v = r.standard_normal((3, B, H, T, d))
    a = polar_attention(q, k, v, causal=False)
    b = polar_attention(q, np.concatenate([k, k], 2), np.concatenate([v, v], 2), causal=False)
    np.testing.assert_allclose(b["direction"], a["direction"], atol=1e-13)
    np.testing.assert_allclose(b["n_eff"], 2 * a["n_eff"], rtol=1e-13)


def test_unit_norm_and_bounds():
    B, H, T, d = 2, 2, 70, 32
    r = rng(12)
    q, k, v = 2 * r.standard_normal((3, B, H, T, d))
    out = polar_attention(q, k, v, causal=True, len_temp=[0.1, 0.0], null_bias=[0.0, -1.0])
    np.testing.assert_allclose(np.linalg.norm(out["direction"], axis=-1), 1.0, atol=1e-13)
    n = np.arange(1, T + 1)
    assert np.all(out["n_eff"] >= 1 - 1e-12) and np.all(out["n_eff"] <= n + 1e-9)
    assert np.all((out["confidence"] > 0) & (out["confidence"] <= 1))
    assert np.all((out["count"] >= 0) & (out["count"] < 1))


def test_zero_values_give_zero_direction():
    r = rng(13)
    q, k = r.standard_normal((2, 1, 1, 6, 4))
    out = polar_attention(q, k, np.zeros((1, 1, 6, 4)), causal=True)
    np.testing.assert_array_equal(out["direction"], 0.0)


def test_gqa_equals_repeated_heads():
    """Query head h reads key/value head h // (H/Hkv): same as MHA on repeated k, v."""
    B, H, Hkv, T, d = 1, 4, 2, 19, 8
    r = rng(14)
    q = r.standard_normal((B, H, T, d))
    k, v = r.standard_normal((2, B, Hkv, T, d))
    a = polar_attention(q, k, v, causal=True, null_bias=[0.0] * H)
    b = polar_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), causal=True, null_bias=[0.0] * H)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_row_subset_and_blocking():
    B, H, T, d = 1, 2, 300, 16
    r = rng(15)
    q, k, v = r.standard_normal((3, B, H, T, d))
    kw = dict(causal=True, len_temp=[0.1, 0.3], null_bias=[0.0, 0.0])
    full = polar_attention(q, k, v, **kw)
    small = polar_attention(q, k, v, block=7, **kw)
    rows = np.array([0, 5, 64, 128, 299])
    sub = polar_attention(q, k, v, rows=rows, **kw)
    for key in full:
        np.testing.assert_allclose(small[key], full[key], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(sub[key], full[key][:, :, rows], rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------- merge algebra

def test_merge_reproduces_unsplit_statistics():
    """Any partition of a row's keys, merged with weights w and w^2, gives the unsplit
    (m, S1, S2, acc) of the definition."""
    r = rng(16)
    Tk, d = 257, 16
    q, k, v = 3 * r.standard_normal(d), r.standard_normal((Tk, d)), r.standard_normal((Tk, d))
    lam, scale = 1.3, 0.25
    whole = split_statistics(q, k, v, lam, scale, 0, Tk)
    for nsplit in (1, 2, 3, 8, 64, 257):
        cuts = np.sort(r.choice(np.arange(1, Tk), size=nsplit - 1, replace=False)) if nsplit > 1 else []
        bounds = [0, *cuts, Tk]
        parts = [split_statistics(q, k, v, lam, scale, lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:])]
        r.shuffle(parts)
        m, s1, s2, acc = merge_statistics(parts)
        assert m == whole[0]
        assert s1 == pytest.approx(whole[1], rel=1e-12)
        assert s2 == pytest.approx(whole[2], rel=1e-12)
        np.testing.assert_allclose(acc, whole[3], rtol=1e-11, atol=1e-12)


def test_merge_reference_equals_forward():
    """Split partials of a decode row, merged, give the forward's outputs when the
    global visible count is used for the length temperature and the floor."""
    r = rng(17)
    B, H, Tk, d, S = 2, 3, 100, 8, 5
    q = r.standard_normal((B, H, 1, d))
    k, v = r.standard_normal((2, B, H, Tk, d))
    tau, beta, kappa = [0.0, 0.2, 0.5], [0.0, -1.0, 2.0], [1.0, 2.0, 0.5]
    ref = polar_attention(q, k, v, causal=True, len_temp=tau, null_bias=beta, count_scale=kappa)
    bounds = np.linspace(0, Tk, S + 1).astype(int)
    part = np.zeros((B, H, 1, S, d + 3))
    for b in range(B):
        for h in range(H):
            lam = 1 + tau[h] * math.log(Tk)
            for s in range(S):
                m, s1, s2, acc = split_statistics(q[b, h, 0], k[b, h], v[b, h], lam, 1 / math.sqrt(d),
                                                  bounds[s], bounds[s + 1])
                part[b, h, 0, s] = [m, s1, s2, *acc]
    got = merge_reference(part, Tk, len_temp=tau, null_bias=beta, count_scale=kappa)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------- brute force and fixtures

def brute_force(q, k, v, causal, tau, beta, kappa):
    """Literal loops over (i, j) for tiny inputs, one output row at a time."""
    Tq, d = len(q), len(q[0])
    Tk = len(k)
    rows = []
    for i in range(Tq):
        vis = [j for j in range(Tk) if (not causal) or j <= i + Tk - Tq]
        n = len(vis)
        lam = 1 + tau * math.log(n)
        s = {j: lam * sum(q[i][t] * k[j][t] for t in range(d)) / math.sqrt(d) for j in vis}
        m = max(s.values())
        p = {j: math.exp(s[j] - m) for j in vis}
        s1 = sum(p.values())
        s2 = sum(x * x for x in p.values())
        acc = [sum(p[j] * v[j][t] for j in vis) for t in range(d)]
        nrm = math.sqrt(sum(a * a for a in acc))
        neff = s1 * s1 / s2
        conf = 1.0 if beta is None else s1 / (s1 + math.exp(lam * math.sqrt(2 * math.log(n)) + beta - m))
        rows.append(([a / nrm for a in acc], neff, conf, conf * math.tanh(math.log(neff) / kappa)))
    return rows


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    r = rng(100 + seed)
    Tk = int(r.integers(1, 13))
    Tq = int(r.integers(1, Tk + 1))
    d = int(r.choice([1, 2, 5, 8]))
    causal = bool(seed % 2)
    tau, beta, kappa = float(r.uniform(0, 0.5)), (None if seed % 3 == 0 else float(r.normal())), float(r.uniform(0.5, 3))
    q, k, v = r.standard_normal((1, 1, Tq, d)), r.standard_normal((1, 1, Tk, d)), r.standard_normal((1, 1, Tk, d))
    out = polar_attention(q, k, v, causal=causal, len_temp=[tau], null_bias=None if beta is None else [beta],
                          count_scale=[kappa])
    ref = brute_force(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, tau, beta, kappa)
    for i, (u, neff, conf, cnt) in enumerate(ref):
        np.testing.assert_allclose(out["direction"][0, 0, i], u, atol=1e-12)
        assert out["n_eff"][0, 0, i] == pytest.approx(neff, rel=1e-12)
        assert out["confidence"][0, 0, i] == pytest.approx(conf, rel=1e-12)
        assert out["count"][0, 0, i] == pytest.approx(cnt, rel=1e-11, abs=1e-14)


def _ev(expr):
    return float(eval(str(expr), {"__builtins__": {}},
                      {"log": math.log, "sqrt": math.sqrt, "exp": math.exp, "tanh": math.tanh}))


def test_hand_worked_fixtures():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q = np.array([[_ev(x) for x in row] for row in case["q"]])[None, None]
        k = np.array([[_ev(x) for x in row] for row in case["k"]])[None, None]
        v = np.array([[_ev(x) for x in row] for row in case["v"]])[None, None]
        out = polar_attention(q, k, v, causal=case["causal"], len_temp=[_ev(case["tau"])],
                              null_bias=[_ev(case["beta"])], count_scale=[_ev(case["kappa"])])
        for e in case["expected"]:
            i = e["row"]
            for key in ("n_eff", "confidence", "count", "m", "s1", "s2"):
                assert out[key][0, 0, i] == pytest.approx(_ev(e[key]), rel=1e-13, abs=1e-15), (case["name"], i, key)
            np.testing.assert_allclose(out["direction"][0, 0, i], [_ev(x) for x in e["direction"]], atol=1e-14)

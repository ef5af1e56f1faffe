"""Pins of the variant oracle (CPU).

Each variant is pinned to something other than its own formula: the reading-R oracle
(written separately, block-wise) at the default variant and on sliced keys for the
window, torch's scaled_dot_product_attention for the temperature forms, the exact
expected maximum of n standard normals (numerical quadrature) for the second-order
floor level, and closed forms for the per-key floors, the data-adaptive floor and the
log1p saturation.  tests/test_oracle_variant_mutations.py checks that these pins catch
plausible mistakes.
"""
import math

import numpy as np
import pytest
import torch
from scipy import integrate, stats

import oracle.polar_variants as pv_default
from oracle import polar_attention

MOD = pv_default


def rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


def run(mod, q, k, v, **kw):
    return mod.polar_attention_variant(q, k, v, **kw)


def close(a, b, tol=1e-10):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.allclose(a, b, rtol=tol, atol=tol)


def check_default_equals_reading_r(mod):
    q, k, v = rand((2, 4, 9, 8), 1), rand((2, 2, 13, 8), 2), rand((2, 2, 13, 8), 3)
    for causal in (True, False):
        kw = dict(causal=causal, len_temp=[0.0, 0.1, 0.3, 0.05], null_bias=[0.0, -1.0, 2.0, 0.5],
                  count_scale=[1.0, 2.0, 4.0, 1.0])
        a = run(mod, q, k, v, **kw)
        b = polar_attention(q, k, v, **kw)
        for key in ("direction", "n_eff", "confidence", "count", "m", "s1", "s2"):
            assert close(a[key], b[key]), key


def check_temperature_forms(mod):
    """Floor off: u_i = normalize(SDPA) with q_i scaled by lam_i (lam from the form's own
    closed value at n_i = i + 1)."""
    B, H, T, d = 1, 2, 12, 8
    q, k, v = rand((B, H, T, d), 4), rand((B, H, T, d), 5), rand((B, H, T, d), 6)
    n = np.arange(1, T + 1, dtype=np.float64)
    forms = {
        "ssmax": (dict(temperature="ssmax"), [0.7, 1.3], lambda tau: tau * np.log(n)),
        "train_ratio": (dict(temperature="train_ratio", train_len=6), [0.0, 0.0], lambda tau: np.log(n) / np.log(6)),
    }
    for name, (var, taus, lam_of) in forms.items():
        out = run(mod, q, k, v, causal=True, len_temp=taus, variant=var)
        for h in range(H):
            lam = lam_of(taus[h])
            qs = torch.tensor(q[:, h:h + 1] * lam[None, None, :, None])
            ref = torch.nn.functional.scaled_dot_product_attention(qs, torch.tensor(k[:, h:h + 1]),
                                                                   torch.tensor(v[:, h:h + 1]), is_causal=True)
            ref = ref.numpy()[0, 0]
            ref = ref / np.linalg.norm(ref, axis=-1, keepdims=True)
            assert close(out["direction"][0, h], ref, 1e-9), name


def expected_max_normal(n):
    """E[max of n i.i.d. N(0,1)] = integral of x n phi(x) Phi(x)^(n-1) dx, by quadrature."""
    f = lambda x: x * n * stats.norm.pdf(x) * stats.norm.cdf(x) ** (n - 1)
    val, _ = integrate.quad(f, -12.0, 12.0, limit=400, points=[0.0, math.sqrt(2 * math.log(n))])
    return val


def check_gumbel_level(mod):
    var2 = mod.variant_of({"floor_level": "gumbel2"})
    var1 = mod.variant_of({})
    assert mod.floor_level(1, var2) == 0.0 and mod.floor_level(1, var1) == 0.0
    for n in (100, 1000, 10000, 100000):
        e = expected_max_normal(n)
        assert abs(mod.floor_level(n, var2) - e) <= 0.06, (n, mod.floor_level(n, var2), e)
        assert mod.floor_level(n, var1) - e >= 0.4  # the leading order overshoots


def check_floor_levels_through_confidence(mod):
    """q = a e0, keys orthogonal to e0: every score is 0, S1 = n, m = 0, so
    conf = n / (n + e^f) with f = lam sigma l(n) + beta; qnorm gives sigma = scale * a."""
    d, n, a, beta = 8, 50, 3.0, 0.25
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = a
    k = rand((1, 1, n, d), 7)
    k[..., 0] = 0.0
    v = rand((1, 1, n, d), 8)
    scale = 1.0 / math.sqrt(d)
    for level, sigma, lvl in (("gauss", 1.0, math.sqrt(2 * math.log(n))),
                              ("qnorm", scale * a, math.sqrt(2 * math.log(n))),
                              ("gumbel2", 1.0, expected_max_normal(n))):
        out = run(mod, q, k, v, causal=False, len_temp=[0.2], null_bias=[beta], variant={"floor_level": level})
        lam = 1.0 + 0.2 * math.log(n)
        conf = out["confidence"][0, 0, 0]
        f = math.log(n * (1.0 - conf) / conf)   # solve n / (n + e^f) = conf for f
        tol = 0.06 * lam * sigma if level == "gumbel2" else 1e-9
        assert abs(f - (lam * sigma * lvl + beta)) <= tol, (level, f)
        assert out["n_eff"][0, 0, 0] == pytest.approx(n, rel=1e-12)


def check_soft_floor(mod):
    d, n = 8, 40
    v = rand((1, 1, n, d), 9)
    zero_q = np.zeros((1, 1, 1, d))
    k = rand((1, 1, n, d), 10)
    # all scores 0 below the floor (f = sqrt(2 ln n) > 0): nothing survives
    out = run(mod, zero_q, k, v, causal=False, null_bias=[0.0], variant={"key_floor": "soft"})
    assert out["n_eff"][0, 0, 0] == 0.0 and out["confidence"][0, 0, 0] == 0.0 and out["count"][0, 0, 0] == 0.0
    assert not np.any(out["direction"])
    # floor pushed below 0: every key keeps 1 - e^f; n_eff = n, u = normalised sum
    beta = -math.sqrt(2 * math.log(n)) - 1.5
    out = run(mod, zero_q, k, v, causal=False, null_bias=[beta], variant={"key_floor": "soft"})
    f = math.sqrt(2 * math.log(n)) + beta
    assert out["n_eff"][0, 0, 0] == pytest.approx(n, rel=1e-12)
    s = v[0, 0].sum(0)
    assert close(out["direction"][0, 0, 0], s / np.linalg.norm(s))
    w = 1.0 - math.exp(f)
    assert out["confidence"][0, 0, 0] == pytest.approx(n * w / (n * w + math.exp(f)), rel=1e-12)
    # one dominant key above the floor, the rest at 0 below it
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k2 = rand((1, 1, n, d), 11)
    k2[..., 0] = 0.0
    delta = 6.0
    k2[0, 0, 17, 0] = delta * math.sqrt(d)
    out = run(mod, q, k2, v, causal=False, null_bias=[0.0], variant={"key_floor": "soft"})
    f = math.sqrt(2 * math.log(n))
    assert out["n_eff"][0, 0, 0] == pytest.approx(1.0, rel=1e-12)
    assert close(out["direction"][0, 0, 0], v[0, 0, 17] / np.linalg.norm(v[0, 0, 17]))
    assert out["confidence"][0, 0, 0] == pytest.approx(1.0 - math.exp(f - delta), rel=1e-12)
    # two keys above: weights e^a - e^f and e^b - e^f (brute force)
    k2[0, 0, 3, 0] = 4.5 * math.sqrt(d)
    out = run(mod, q, k2, v, causal=False, null_bias=[0.0], variant={"key_floor": "soft"})
    w1, w2 = math.exp(delta) - math.exp(f), math.exp(4.5) - math.exp(f)
    assert out["n_eff"][0, 0, 0] == pytest.approx((w1 + w2) ** 2 / (w1 * w1 + w2 * w2), rel=1e-12)
    acc = w1 * v[0, 0, 17] + w2 * v[0, 0, 3]
    assert close(out["direction"][0, 0, 0], acc / np.linalg.norm(acc))


def check_gate_floor(mod):
    d, n = 8, 40
    v = rand((1, 1, n, d), 12)
    k = rand((1, 1, n, d), 13)
    zero_q = np.zeros((1, 1, 1, d))
    beta = -math.sqrt(2 * math.log(n)) - 0.5   # f = -0.5 < 0 = every score: all keys pass
    out = run(mod, zero_q, k, v, causal=False, null_bias=[beta], variant={"key_floor": "gate"})
    assert out["n_eff"][0, 0, 0] == pytest.approx(n, rel=1e-12)
    assert out["confidence"][0, 0, 0] == pytest.approx(n / (n + math.exp(-0.5)), rel=1e-12)
    out = run(mod, zero_q, k, v, causal=False, null_bias=[0.0], variant={"key_floor": "gate"})
    assert out["n_eff"][0, 0, 0] == 0.0 and out["count"][0, 0, 0] == 0.0
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k[..., 0] = 0.0
    k[0, 0, 5, 0] = 5.0 * math.sqrt(d)
    out = run(mod, q, k, v, causal=False, null_bias=[0.0], variant={"key_floor": "gate"})
    f = math.sqrt(2 * math.log(n))
    assert out["n_eff"][0, 0, 0] == pytest.approx(1.0, rel=1e-12)
    assert out["confidence"][0, 0, 0] == pytest.approx(math.exp(5.0) / (math.exp(5.0) + math.exp(f)), rel=1e-12)


def check_log1p_saturation(mod):
    q, k, v = rand((1, 2, 7, 8), 14), rand((1, 2, 7, 8), 15), rand((1, 2, 7, 8), 16)
    out = run(mod, q, k, v, causal=True, null_bias=[0.0, 1.0], count_scale=[1.0, 3.0],
              variant={"saturation": "log1p"})
    for h, kappa in ((0, 1.0), (1, 3.0)):
        x = (1.0 + out["n_eff"][0, h]) ** (2.0 / kappa)
        assert close(out["count"][0, h] / out["confidence"][0, h], (x - 1.0) / (x + 1.0))


def check_window(mod):
    B, H, Tq, Tk, d = 1, 2, 10, 16, 8
    q, k, v = rand((B, H, Tq, d), 17), rand((B, H, Tk, d), 18), rand((B, H, Tk, d), 19)
    kw = dict(len_temp=[0.1, 0.0], null_bias=[0.5, 0.0], count_scale=[1.0, 2.0])
    W = 5
    out = run(mod, q, k, v, causal=True, variant={"window": W}, **kw)
    off = Tk - Tq
    for i in range(Tq):
        hi = i + 1 + off
        lo = max(0, hi - W)
        ref = polar_attention(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi], causal=False, **kw)
        for key in ("direction", "n_eff", "confidence", "count", "m", "s1", "s2"):
            assert close(out[key][:, :, i], ref[key][:, :, 0]), (i, key)
    wide = run(mod, q, k, v, causal=True, variant={"window": Tk}, **kw)
    plain = polar_attention(q, k, v, causal=True, **kw)
    assert close(wide["n_eff"], plain["n_eff"]) and close(wide["direction"], plain["direction"])
    with pytest.raises(ValueError):
        run(mod, q, k, v, causal=False, variant={"window": 3})


def check_split_merge(mod):
    """Any partition of the keys into splits, each reduced by the variant's weights and
    merged with w and w^2, gives the unsplit outputs (the floored weights are linear
    in e^{s} - e^{f}, so the rescaling is exact)."""
    d, n = 8, 60
    q, k, v = rand((d,), 20), rand((n, d), 21), rand((n, d), 22)
    scale = 1.0 / math.sqrt(d)
    for var in ({"key_floor": "soft"}, {"key_floor": "gate"}, {"floor_level": "qnorm"},
                {"temperature": "ssmax", "saturation": "log1p"}):
        beta, tau, kappa = -1.0, 0.3, 2.0
        whole = run(mod, q[None, None, None], k[None, None], v[None, None], causal=False, len_temp=[tau],
                    null_bias=[beta], count_scale=[kappa], variant=var)
        for cuts in ([0, 60], [0, 7, 60], [0, 13, 14, 31, 60]):
            parts = [mod.split_statistics_variant(q, k, v, a, b, n, tau, beta, scale, var)
                     for a, b in zip(cuts[:-1], cuts[1:])]
            merged = mod.merge_variant(parts, q, n, tau, beta, kappa, scale, var)
            for key in ("n_eff", "confidence", "count", "m", "s1", "s2"):
                assert close(merged[key], whole[key][0, 0, 0], 1e-9), (var, cuts, key)
            assert close(merged["direction"], whole["direction"][0, 0, 0], 1e-9)


CHECKS = [check_default_equals_reading_r, check_temperature_forms, check_gumbel_level,
          check_floor_levels_through_confidence, check_soft_floor, check_gate_floor, check_log1p_saturation,
          check_window, check_split_merge]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_variant_oracle(check):
    check(MOD)

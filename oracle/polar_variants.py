"""Plain fp64 CPU oracle for the reading variants of the Polar Attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module.  The GPU library
never calls it and shares no code with it.

The ATMA summary names the parts of the operator without giving their formulas
[ATMA §2.1]: a length temperature that sharpens the logits as the context grows, an
extreme-value-corrected null floor that calibrates them against noise, a count gated by
the confidence of signal detection and mapped through a bounded tanh of a log; its
ablation also compares sliding-window attention [ATMA §3.1].  polar_oracle.py follows
one reading of each (reading R).  This module computes the same operator under the
alternative readings, one query row at a time, by the definition:

  temperature  "log"          lam = 1 + tau ln n                     (reading R)
               "ssmax"        lam = tau ln n                         (per-head scale times ln n)
               "train_ratio"  lam = ln n / ln L                      (L = training length)
  floor level  "gauss"        l(n) = sqrt(2 ln n)                    (reading R)
               "gumbel2"      l(n) = b_n + gamma a_n,  b_n = r - (ln ln n + ln 4 pi) / (2 r),
                              a_n = 1 / r,  r = sqrt(2 ln n)  (second-order expected maximum of
                              n standard normals; l(1) = 0, the mean of one normal)
               "qnorm"        l(n) = sqrt(2 ln n), noise scale sigma_i = scale ||q_i||_2 (the
                              standard deviation of scale <q_i, k> for unit-variance keys)
               f_i = lam_i sigma_i l(n_i) + beta_h   (sigma_i = 1 except for "qnorm")
  key floor    "null"         a null slot of logit f joins the normaliser: every visible key
                              keeps its weight e^{s_j}                (reading R)
               "soft"         w_j = max(e^{s_j} - e^{f}, 0)
               "gate"         w_j = e^{s_j} if s_j > f else 0
               with Z1 = sum w, Z2 = sum w^2, A = sum w v:
               n_eff = Z1^2 / Z2, u = A / ||A||, conf = Z1 / (Z1 + e^f);
               a row with Z1 = 0 gets n_eff = 0, u = 0, conf = 0, count = 0
  saturation   "log"          count = conf tanh(ln n_eff / kappa)      (reading R)
               "log1p"        count = conf tanh(ln(1 + n_eff) / kappa)
  window       W > 0          key j visible to row i iff i + off - W < j <= i + off
                              (off = Tk - Tq; causal only), so n_i = min(W, i + 1 + off)

The statistics m, S1, S2 are relative to the maximum m of the visible scores (below-floor
keys included), as in reading R.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["DEFAULT_VARIANT", "variant_of", "temperature", "floor_level", "key_weights",
           "polar_attention_variant", "split_statistics_variant", "merge_variant"]

EULER_GAMMA = 0.5772156649015329

DEFAULT_VARIANT = {"temperature": "log", "train_len": 2048, "floor_level": "gauss", "key_floor": "null",
                   "saturation": "log", "window": 0}


def variant_of(v=None) -> dict:
    """The full variant dict: the defaults (reading R) overridden by `v`."""
    out = dict(DEFAULT_VARIANT)
    if v:
        unknown = set(v) - set(out)
        if unknown:
            raise ValueError(f"unknown variant keys {sorted(unknown)}")
        out.update(v)
    return out


def temperature(n: int, tau: float, var: dict) -> float:
    ln_n = math.log(n)
    form = var["temperature"]
    if form == "log":
        return 1.0 + tau * ln_n
    if form == "ssmax":
        return tau * ln_n
    if form == "train_ratio":
        return ln_n / math.log(var["train_len"])
    raise ValueError(form)


def floor_level(n: int, var: dict) -> float:
    """l(n): the expected maximum of n standard normal logits, to the chosen order."""
    if n <= 1:
        return 0.0
    r = math.sqrt(2.0 * math.log(n))
    if var["floor_level"] in ("gauss", "qnorm"):
        return r
    if var["floor_level"] == "gumbel2":
        b = r - (math.log(math.log(n)) + math.log(4.0 * math.pi)) / (2.0 * r)
        return b + EULER_GAMMA / r
    raise ValueError(var["floor_level"])


def key_weights(s, m: float, f: float, var: dict):
    """Weights of the visible keys relative to e^m: e^{s-m}, floored by the key-floor kind."""
    p = np.exp(s - m)
    kind = var["key_floor"]
    if kind == "null":
        return p
    if kind == "soft":
        return np.maximum(p - math.exp(f - m), 0.0)
    if kind == "gate":
        return np.where(s > f, p, 0.0)
    raise ValueError(kind)


def _noise_scale(q_row, scale: float, var: dict) -> float:
    """sigma_i: 1, or for "qnorm" the standard deviation scale ||q_i|| of the raw logits."""
    return scale * float(np.sqrt(q_row @ q_row)) if var["floor_level"] == "qnorm" else 1.0


def _floor(n: int, lam: float, sigma: float, beta, var: dict) -> float:
    """The null floor f in tempered-logit units (0 when the floor is off)."""
    return lam * sigma * floor_level(n, var) + (0.0 if beta is None else beta)


def _channels(m: float, s1: float, s2: float, acc, f: float, floor_on: bool, kappa: float, var: dict) -> dict:
    """Output channels from the (floored) row statistics relative to e^m."""
    out = {"m": m, "s1": s1, "s2": s2, "direction": np.zeros(len(acc))}
    if s1 == 0.0:
        out.update(n_eff=0.0, confidence=0.0, count=0.0)
        return out
    norm = float(np.sqrt(acc @ acc))
    if norm != 0.0:  # u = 0 where acc = 0; a NaN in acc stays NaN
        out["direction"] = acc / norm
    n_eff = s1 * s1 / s2
    conf = 1.0 / (1.0 + math.exp(f - m - math.log(s1))) if floor_on else 1.0
    x = math.log1p(n_eff) if var["saturation"] == "log1p" else math.log(n_eff)
    out.update(n_eff=n_eff, confidence=conf, count=conf * math.tanh(x / kappa))
    return out


def _row(q_row, k, v, lo: int, hi: int, n: int, tau, beta, kappa, scale: float, var: dict):
    """All outputs of one query row whose visible keys are [lo, hi) and whose count is n."""
    if var["key_floor"] != "null" and beta is None:
        raise ValueError("a per-key floor needs the floor on")
    lam = temperature(n, tau, var)
    s = lam * scale * (k[lo:hi] @ q_row)
    m = float(s.max())
    f = _floor(n, lam, _noise_scale(q_row, scale, var), beta, var)
    w = key_weights(s, m, f, var)
    return _channels(m, float(w.sum()), float((w * w).sum()), w @ v[lo:hi], f, beta is not None, kappa, var)


def _visible(i: int, tq: int, tk: int, causal: bool, window: int):
    """[lo, hi) of the keys row i sees and their count."""
    if window and not causal:
        raise ValueError("a sliding window needs the causal alignment")
    hi = min(i + 1 + (tk - tq), tk) if causal else tk
    lo = max(0, hi - window) if window else 0
    return lo, hi, hi - lo


def polar_attention_variant(q, k, v, *, causal: bool = True, len_temp=None, null_bias=None, count_scale=None,
                            softmax_scale=None, variant=None, rows=None):
    """The forward under a reading variant, fp64, one row at a time.  Arguments and
    outputs as polar_oracle.polar_attention; `variant` is a dict of the keys of
    DEFAULT_VARIANT (missing keys keep reading R)."""
    var = variant_of(variant)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    group = H // Hkv
    scale = 1.0 / math.sqrt(d) if softmax_scale is None or softmax_scale <= 0 else float(softmax_scale)
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    out = {key: np.zeros((B, H, R)) for key in ("n_eff", "confidence", "count", "m", "s1", "s2")}
    out["direction"] = np.zeros((B, H, R, d))
    for b in range(B):
        for h in range(H):
            tau = 0.0 if len_temp is None else float(len_temp[h])
            beta = None if null_bias is None else float(null_bias[h])
            kappa = 1.0 if count_scale is None else float(count_scale[h])
            for r, i in enumerate(rows):
                lo, hi, n = _visible(int(i), Tq, Tk, causal, var["window"])
                one = _row(q[b, h, i], k[b, h // group], v[b, h // group], lo, hi, n, tau, beta, kappa, scale, var)
                for key in out:
                    out[key][b, h, r] = one[key]
    return out


def split_statistics_variant(q_row, k, v, lo: int, hi: int, n: int, tau: float, beta: float, scale: float,
                             variant=None):
    """(m, S1, S2, acc) of one query row over the keys [lo, hi), with the weights of the
    key-floor kind and the floor of the row's whole visible count n (one split of a
    split-KV decode [ATMA §2.2])."""
    var = variant_of(variant)
    q_row, k, v = (np.asarray(x, dtype=np.float64) for x in (q_row, k, v))
    lam = temperature(n, tau, var)
    s = lam * scale * (k[lo:hi] @ q_row)
    m = float(s.max())
    w = key_weights(s, m, _floor(n, lam, _noise_scale(q_row, scale, var), beta, var), var)
    return m, float(w.sum()), float((w * w).sum()), w @ v[lo:hi]


def merge_variant(parts, q_row, n: int, tau: float, beta, kappa: float, scale: float, variant=None):
    """Outputs of one row from split statistics: each part brought to the common maximum
    m* with w = e^{m_s - m*} (w on S1 and acc, w^2 on S2 [ATMA §2.2]), then the channels
    of the variant with the row's count n."""
    var = variant_of(variant)
    m_star = max(p[0] for p in parts)
    s1 = s2 = 0.0
    acc = np.zeros(len(parts[0][3]))
    for m, a, b2, c in parts:
        if m == -math.inf:
            continue
        wgt = math.exp(m - m_star)
        s1 += wgt * a
        s2 += wgt * wgt * b2
        acc = acc + wgt * np.asarray(c, dtype=np.float64)
    lam = temperature(n, tau, var)
    f = _floor(n, lam, _noise_scale(np.asarray(q_row, dtype=np.float64), scale, var), beta, var)
    return _channels(m_star, s1, s2, acc, f, beta is not None, kappa, var)

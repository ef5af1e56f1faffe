"""Plain fp64 CPU oracle for the gradients of the Polar Attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module.  The GPU library
never calls it and shares no code with it.

The ATMA summary trains models with the operator [ATMA §3] but describes no backward
pass.  The gradient here is the derivative of the forward map (the definition in
polar_oracle) written out with the chain rule.  Absolute weights are P_j = exp(s_j).
The row maximum cancels in every output, so the quantities below use p_j = P_j / e^m:

    Z1 = sum P = S1 e^m,  Z2 = sum P^2 = S2 e^{2m},  A = sum P v = acc e^m
    u = A / ||A||             du/dA = (I - u u^T) / ||A||
    n_eff = Z1^2 / Z2         d n_eff / dZ1 = 2 n_eff / Z1,  d n_eff / dZ2 = -n_eff / Z2
    conf = Z1 / (Z1 + e^f)    d conf / dZ1 = conf (1 - conf) / Z1       (floor on; 1 off)
    count = conf T,  T = tanh(ln(n_eff) / kappa)
                              d count / d conf = T,  d count / d n_eff = conf (1 - T^2) / (kappa n_eff)
    dP_j/ds_j = P_j,  ds/dq = lam scale k,  ds/dk = lam scale q   (lam depends on n only)

The same map holds under the reading variants that change only per-row constants
(polar_variants; [ATMA §2.1] names the parts without formulas): the temperature forms
change lam(n), the floor levels "gauss" and "gumbel2" change f(n) (both depend on the
count n alone, not on q or k), and the saturation "log1p" has T = tanh(ln(1 + n_eff) /
kappa), so d count / d n_eff = conf (1 - T^2) / (kappa (1 + n_eff)).  A per-key floor, a
window or the q-scaled floor level change the map itself and are not covered here.

Given upstream gradients g_u, g_n, g_c, g_k of one row:

    G_conf = g_c + g_k T,   G_neff = g_n + g_k conf (1 - T^2) / (kappa n_eff)
    c1 = (2 G_neff n_eff + G_conf conf (1 - conf)) / S1,   c2 = -G_neff n_eff / S2
    w  = (g_u - u (u . g_u)) / ||acc||
    ds_j = p_j (c1 + 2 c2 p_j + <w, v_j>)
    dq = lam scale sum_j ds_j k_j,   dk_j += lam scale ds_j q,   dv_j += p_j w

Parity pins (tests/test_backward_oracle.py): central finite differences of the forward
oracle along random directions, torch autograd (float64) through an independently
written forward, and closed forms (n_eff is stationary at uniform logits).
"""
from __future__ import annotations

import numpy as np

from .polar_oracle import length_temperature, null_floor, visible_count
from .polar_variants import floor_level, temperature, variant_of

__all__ = ["polar_attention_backward", "row_coefficients"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def row_coefficients(m, s1, s2, acc, n, lam, beta, kappa, g_u, g_n, g_c, g_k, f=None, saturation="log"):
    """c1, c2 [R] and w [R, d] of the rows from their statistics (relative to e^m) and the
    upstream gradients (see the module docstring).  f: the rows' null floor when it is not
    reading R's lam sqrt(2 ln n) + beta; saturation: "log" or "log1p"."""
    s1, s2, acc = _f64(s1), _f64(s2), _f64(acc)
    n_eff = s1 * s1 / s2
    norm = np.sqrt(np.sum(acc * acc, axis=-1))
    safe = np.where(norm > 0.0, norm, 1.0)
    u = acc / safe[:, None]
    if beta is None:
        conf = np.ones_like(s1)
        dconf_dz1 = np.zeros_like(s1)
    else:
        f = null_floor(n, lam, beta) if f is None else _f64(f)
        conf = 1.0 / (1.0 + np.exp(f - _f64(m) - np.log(s1)))
        dconf_dz1 = conf * (1.0 - conf)
    if saturation == "log1p":
        t = np.tanh(np.log1p(n_eff) / kappa)
        slope = (1.0 - t * t) / (kappa * (1.0 + n_eff))
    else:
        t = np.tanh(np.log(n_eff) / kappa)
        slope = (1.0 - t * t) / (kappa * n_eff)
    g_conf = g_c + g_k * t
    g_neff = g_n + g_k * conf * slope
    c1 = (2.0 * g_neff * n_eff + g_conf * dconf_dz1) / s1
    c2 = -g_neff * n_eff / s2
    w = np.where(norm[:, None] > 0.0, (g_u - u * np.sum(u * g_u, axis=-1, keepdims=True)) / safe[:, None], 0.0)
    return c1, c2, w


def polar_attention_backward(q, k, v, grads, *, causal: bool = True, len_temp=None, null_bias=None,
                             count_scale=None, softmax_scale=None, variant=None):
    """Gradients of sum(g_u . u) + sum(g_n n_eff) + sum(g_c conf) + sum(g_k count) with
    respect to q, k, v (fp64).

    q [B,H,Tq,d], k and v [B,Hkv,Tk,d]; grads: dict with any of "direction" [B,H,Tq,d],
    "n_eff", "confidence", "count" [B,H,Tq] (missing entries are zero).  variant: a dict
    of polar_variants keys; only the temperature, the floor levels "gauss" and "gumbel2"
    and the saturation may differ from reading R.
    Returns dict dq [B,H,Tq,d], dk, dv [B,Hkv,Tk,d].
    """
    var = variant_of(variant)
    if var["key_floor"] != "null" or var["window"] or var["floor_level"] == "qnorm":
        raise ValueError("gradients cover the variants that change only per-row constants")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    group = H // Hkv
    scale = 1.0 / np.sqrt(d) if softmax_scale is None or softmax_scale <= 0 else float(softmax_scale)

    def g(name, shape):
        x = grads.get(name)
        return np.zeros(shape) if x is None else _f64(x)

    g_u = g("direction", q.shape)
    g_n, g_c, g_k = (g(nm, (B, H, Tq)) for nm in ("n_eff", "confidence", "count"))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(Tq)
    n = visible_count(rows, Tq, Tk, causal)
    visible = np.arange(Tk)[None, :] < n[:, None]
    for b in range(B):
        for h in range(H):
            hk = h // group
            tau = 0.0 if len_temp is None else float(len_temp[h])
            beta = None if null_bias is None else float(null_bias[h])
            kappa = 1.0 if count_scale is None else float(count_scale[h])
            if var["temperature"] == "log":
                lam = length_temperature(n, tau)
            else:
                lam = np.array([temperature(int(ni), tau, var) for ni in n])
            f = None
            if beta is not None and var["floor_level"] != "gauss":
                f = lam * np.array([floor_level(int(ni), var) for ni in n]) + beta
            ls = lam * scale
            s = np.where(visible, ls[:, None] * (q[b, h] @ k[b, hk].T), -np.inf)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            s1 = p.sum(axis=1)
            s2 = (p * p).sum(axis=1)
            acc = p @ v[b, hk]
            c1, c2, w = row_coefficients(m, s1, s2, acc, n, lam, beta, kappa, g_u[b, h], g_n[b, h], g_c[b, h],
                                         g_k[b, h], f=f, saturation=var["saturation"])
            ds = p * (c1[:, None] + 2.0 * c2[:, None] * p + w @ v[b, hk].T)
            dq[b, h] = ls[:, None] * (ds @ k[b, hk])
            dk[b, hk] += (ls[:, None] * ds).T @ q[b, h]
            dv[b, hk] += p.T @ w
    return {"dq": dq, "dk": dk, "dv": dv}

"""Plain fp64 CPU oracle for the fused Polar Attention forward and its split-KV decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never calls it and
shares no code with it.

Source: the technical summary of "ATMA: Length-Invariant Language Modeling via Polar
Attention and Gated-Delta Compression Memory" (gist.science, paper 2606.25156; the
Spanish, Italian and French pages carry the same summary).  Citations below name a
section of that summary as [ATMA §x].

What is computed, per batch b, head h and query row i (reading R: where the pages
leave a point open, the plainest form consistent with the rest is taken, as written
here):

    V_i   = keys visible to query i: j <= i + (Tk - Tq) when causal, all Tk otherwise
    n_i   = |V_i|
    lam_i = 1 + tau_h * ln(n_i)                       length temperature [ATMA §2.1]
    s_ij  = lam_i * scale * <q_i, k_j>                 scale = 1/sqrt(d)
    m_i   = max_j s_ij,  p_ij = exp(s_ij - m_i)
    S1    = sum_j p_ij,  S2 = sum_j p_ij^2,  acc = sum_j p_ij v_j
    n_eff = S1^2 / S2                                  participation ratio [ATMA §2.1]
    u     = acc / ||acc||_2  (0 when acc == 0)         direction on the unit sphere [ATMA §2.1]
    floor f_i = lam_i * sqrt(2 ln n_i) + beta_h        extreme-value-corrected null floor [ATMA §2.1]
    conf  = S1 / (S1 + exp(f_i - m_i))   (floor on; 1 when off)
    count = conf * tanh(ln(n_eff) / kappa_h)           bounded tanh-of-log saturation [ATMA §2.1]

The forward is the plain definition written out: scores are materialised row block by
row block, with no online rescaling.  The merge of split statistics is the algebra of
the streaming accumulators with squared correction factors [ATMA §2.2, fused kernel]:
each part is brought to the common maximum with weight w = exp(m_s - m*), applied as
w to S1 and acc and as w^2 to S2.

Parity pins: closed forms, textbook softmax attention and invariants in
tests/test_oracle.py.  Nothing in the pages pins the chosen forms of the length
temperature, the null floor, the confidence gate or the saturation to what the
authors' model computes; those are pinned to reading R only.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible_count",
    "length_temperature",
    "null_floor",
    "finish_rows",
    "polar_attention",
    "split_statistics",
    "merge_statistics",
    "merge_reference",
    "PARTIAL_M",
    "PARTIAL_S1",
    "PARTIAL_S2",
    "PARTIAL_ACC",
]

# Column layout of one partial row: m, S1, S2, acc[0..d-1]  (m in natural-log units).
PARTIAL_M, PARTIAL_S1, PARTIAL_S2, PARTIAL_ACC = 0, 1, 2, 3


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible_count(i, tq: int, tk: int, causal: bool):
    """Number of keys query row i sees: a decoder attends to itself and the past
    [ATMA §2, decoder-only stack]; rows are aligned to the end of the key sequence."""
    i = np.asarray(i, dtype=np.int64)
    if causal:
        return np.minimum(i + 1 + (tk - tq), tk)
    return np.full_like(i, tk)


def length_temperature(n, tau: float):
    """lam(n) = 1 + tau ln n: sharpens the logits as the visible context grows [ATMA §2.1]."""
    return 1.0 + tau * np.log(_f64(n))


def null_floor(n, lam, beta: float):
    """Null logit level: the leading-order expected maximum of n unit-variance noise
    logits, sqrt(2 ln n), in tempered units, plus a per-head offset [ATMA §2.1]."""
    return _f64(lam) * np.sqrt(2.0 * np.log(_f64(n))) + beta


def finish_rows(m, s1, s2, acc, n, lam, beta, kappa: float):
    """Output channels from the row statistics [ATMA §2.1].

    m, s1, s2, n, lam: [R]; acc: [R, d]; beta: None (floor off) or float.
    Returns direction [R,d], n_eff [R], confidence [R], count [R].
    """
    m, s1, s2, acc = _f64(m), _f64(s1), _f64(s2), _f64(acc)
    n_eff = s1 * s1 / s2
    norm = np.sqrt(np.sum(acc * acc, axis=-1))
    # u = 0 exactly where acc = 0 (reading A-10); a NaN in acc stays NaN
    safe = np.where(norm == 0.0, 1.0, norm)
    direction = np.where(norm[:, None] == 0.0, 0.0, acc / safe[:, None])
    if beta is None:
        conf = np.ones_like(s1)
    else:
        f = null_floor(n, lam, beta)
        # null slot of zero value and logit f joins the normaliser: conf = S1 / (S1 + e^{f-m})
        z = f - m - np.log(s1)
        conf = 1.0 / (1.0 + np.exp(z))
    count = conf * np.tanh(np.log(n_eff) / kappa)
    return direction, n_eff, conf, count


def _per_head(arr, h: int, default):
    return default if arr is None else float(arr[h])


def polar_attention(q, k, v, *, causal: bool = True, len_temp=None, null_bias=None,
                    count_scale=None, softmax_scale=None, rows=None, block: int = 512):
    """Polar Attention forward by the plain definition, fp64.

    q: [B, H, Tq, d]; k, v: [B, Hkv, Tk, d] with H % Hkv == 0 (query head h reads
    key/value head h // (H // Hkv)).  len_temp / null_bias / count_scale: per-head
    sequences of length H or None (tau = 0; floor off; kappa = 1).
    rows: optional sorted 1-D array of query indices to evaluate (others are skipped).

    Returns a dict of numpy fp64 arrays: direction [B,H,R,d], n_eff, confidence,
    count, m, s1, s2 [B,H,R], where R = Tq or len(rows).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    assert k.shape == (B, Hkv, Tk, d) and v.shape == k.shape and H % Hkv == 0
    group = H // Hkv
    scale = 1.0 / np.sqrt(d) if softmax_scale is None or softmax_scale <= 0 else float(softmax_scale)
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = {
        "direction": np.zeros((B, H, R, d)),
        "n_eff": np.zeros((B, H, R)),
        "confidence": np.zeros((B, H, R)),
        "count": np.zeros((B, H, R)),
        "m": np.zeros((B, H, R)),
        "s1": np.zeros((B, H, R)),
        "s2": np.zeros((B, H, R)),
    }
    for b in range(B):
        for h in range(H):
            hk = h // group
            tau = _per_head(len_temp, h, 0.0)
            beta = None if null_bias is None else float(null_bias[h])
            kappa = _per_head(count_scale, h, 1.0)
            for r0 in range(0, R, block):
                ri = rows[r0:r0 + block]
                n = visible_count(ri, Tq, Tk, causal)
                last = int(n.max())                      # keys beyond this are invisible to the block
                lam = length_temperature(n, tau)
                raw = q[b, h, ri] @ k[b, hk, :last].T    # [r, last]
                s = (lam * scale)[:, None] * raw
                visible = np.arange(last)[None, :] < n[:, None]
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1)
                p = np.exp(s - m[:, None])               # exp(-inf) = 0 on masked keys
                s1 = p.sum(axis=1)
                s2 = (p * p).sum(axis=1)
                acc = p @ v[b, hk, :last]
                dirn, n_eff, conf, count = finish_rows(m, s1, s2, acc, n, lam, beta, kappa)
                sl = slice(r0, r0 + len(ri))
                out["direction"][b, h, sl] = dirn
                out["n_eff"][b, h, sl] = n_eff
                out["confidence"][b, h, sl] = conf
                out["count"][b, h, sl] = count
                out["m"][b, h, sl] = m
                out["s1"][b, h, sl] = s1
                out["s2"][b, h, sl] = s2
    return out


def split_statistics(q_row, k, v, lam: float, scale: float, lo: int, hi: int):
    """Statistics (m, S1, S2, acc) of one query row over the keys [lo, hi) by
    definition; the key range is one split of a split-KV decode [ATMA §2.2]."""
    q_row, k, v = _f64(q_row), _f64(k), _f64(v)
    s = lam * scale * (k[lo:hi] @ q_row)
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), (p * p).sum(), p @ v[lo:hi]


def merge_statistics(parts):
    """Combine per-split statistics into the statistics of the union of the splits.

    parts: iterable of (m, S1, S2, acc).  Each part is referred to the common maximum
    m* with w = exp(m_s - m*): S1 and acc scale by w, S2 by w^2 (the squared
    correction factor) [ATMA §2.2, fused kernel].  A part with m = -inf (no keys)
    contributes nothing.
    """
    parts = [(float(m), float(s1), float(s2), _f64(acc)) for m, s1, s2, acc in parts]
    m_star = max(m for m, _, _, _ in parts)
    s1 = s2 = 0.0
    acc = np.zeros_like(parts[0][3])
    for m, a, b2, c in parts:
        if m == -np.inf:
            continue
        w = np.exp(m - m_star)
        s1 += w * a
        s2 += w * w * b2
        acc = acc + w * c
    return m_star, s1, s2, acc


def merge_reference(partials, n, *, len_temp=None, null_bias=None, count_scale=None):
    """Outputs from split partials.

    partials: [B, H, Tq, S, d+3] with columns (m, S1, S2, acc...); n: number of keys
    visible to each row over all splits (the global count, never a per-split one),
    broadcastable to [B, H, Tq].  Returns the same dict keys as polar_attention.
    """
    P = _f64(partials)
    B, H, Tq, S, w = P.shape
    d = w - PARTIAL_ACC
    n = np.broadcast_to(np.asarray(n, dtype=np.float64), (B, H, Tq))
    out = {key: np.zeros((B, H, Tq)) for key in ("n_eff", "confidence", "count", "m", "s1", "s2")}
    out["direction"] = np.zeros((B, H, Tq, d))
    for b in range(B):
        for h in range(H):
            tau = _per_head(len_temp, h, 0.0)
            beta = None if null_bias is None else float(null_bias[h])
            kappa = _per_head(count_scale, h, 1.0)
            for i in range(Tq):
                parts = [(P[b, h, i, s, PARTIAL_M], P[b, h, i, s, PARTIAL_S1],
                          P[b, h, i, s, PARTIAL_S2], P[b, h, i, s, PARTIAL_ACC:]) for s in range(S)]
                m, s1, s2, acc = merge_statistics(parts)
                nn = np.array([n[b, h, i]])
                lam = length_temperature(nn, tau)
                dirn, n_eff, conf, count = finish_rows(np.array([m]), np.array([s1]), np.array([s2]),
                                                       acc[None, :], nn, lam, beta, kappa)
                out["direction"][b, h, i] = dirn[0]
                out["n_eff"][b, h, i] = n_eff[0]
                out["confidence"][b, h, i] = conf[0]
                out["count"][b, h, i] = count[0]
                out["m"][b, h, i], out["s1"][b, h, i], out["s2"][b, h, i] = m, s1, s2
    return out

"""Comparison of GPU outputs with the oracle, with the stated tolerances.

Norms: direction by the per-row L2 distance ||u_gpu - u_ref||_2 (a relative error, as
||u_ref|| = 1); n_eff by the per-row relative error; confidence and count (both in
[0, 1]) by the absolute error; stats m by the absolute error and S1, S2 relative.
Tolerances: 2e-2 (direction) and 1e-2 (n_eff, confidence, count) for bf16 inputs,
1e-5 for fp32 inputs.
"""
import numpy as np
import torch

TOL = {
    "bf16": dict(direction=2e-2, n_eff=1e-2, confidence=1e-2, count=1e-2, m=1e-3, s=1e-2),
    "f32": dict(direction=1e-5, n_eff=1e-5, confidence=1e-5, count=1e-5, m=1e-5, s=1e-5),
}


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(gpu, ref, rows=None):
    """Max errors of the GPU outputs (dict of tensors, all rows) against the oracle
    (dict of numpy arrays, possibly only `rows`)."""
    def sel(x):
        x = to_np(x)
        return x if rows is None else x[:, :, rows]
    e = {}
    du = sel(gpu["direction"]) - ref["direction"]
    e["direction"] = float(np.sqrt((du * du).sum(-1)).max())
    e["n_eff"] = float((np.abs(sel(gpu["n_eff"]) - ref["n_eff"]) / ref["n_eff"]).max())
    if gpu.get("confidence") is not None:
        e["confidence"] = float(np.abs(sel(gpu["confidence"]) - ref["confidence"]).max())
    if gpu.get("count") is not None:
        e["count"] = float(np.abs(sel(gpu["count"]) - ref["count"]).max())
    if gpu.get("stats") is not None:
        st = sel(gpu["stats"])
        e["m"] = float(np.abs(st[..., 0] - ref["m"]).max())
        e["s1"] = float((np.abs(st[..., 1] - ref["s1"]) / ref["s1"]).max())
        e["s2"] = float((np.abs(st[..., 2] - ref["s2"]) / ref["s2"]).max())
    return e


def assert_parity(gpu, ref, kind, rows=None, label=""):
    tol = TOL[kind]
    e = errors(gpu, ref, rows)
    for key in ("direction", "n_eff", "confidence", "count"):
        if key in e:
            assert np.isfinite(e[key]) and e[key] <= tol[key], f"{label} {key}: {e[key]:.3e} > {tol[key]:.1e} ({e})"
    if "m" in e:
        assert e["m"] <= tol["m"] * max(1.0, float(np.abs(ref["m"]).max())), f"{label} m: {e}"
        assert e["s1"] <= tol["s"] and e["s2"] <= tol["s"], f"{label} stats: {e}"
    # every row that exists must be finite, also the ones the oracle did not check
    for key in ("direction", "n_eff"):
        assert torch.isfinite(gpu[key]).all(), f"{label} non-finite {key}"
    return e

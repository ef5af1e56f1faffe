"""Polar Attention for AMD Instinct MI355X: a thin ctypes binding over libpolar_attn.so.

Every step of the operator runs in the HIP library; this module only marshals
arguments.  PyTorch provides device memory and the current stream.  The entry points
mirror the C ABI in include/polar_attn.h:

    fwd(q, k, v, ...)            -> polar_attn_fwd      (fused prefill forward)
    bwd(q, k, v, grads, ...)     -> polar_attn_bwd      (dq, dk, dv of the forward)
    decode(q, k_cache, v_cache)  -> polar_attn_decode   (split-KV decode + merge)
    decode_noalloc(...)          -> polar_attn_decode_noalloc (the same, no workspace)
    merge(partials, ...)         -> polar_attn_merge    (merge of split statistics)
    decode_num_splits / decode_workspace_bytes / status_string / abi_version

Operator source: the ATMA technical summary (gist.science, paper 2606.25156), §2.1
(direction and magnitude channels) and §2.2 (fused and decode kernels).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpolar_attn.so")

POLAR_BF16, POLAR_F32 = 0, 1
POLAR_MAX_PARAM_HEADS = 128
STATUS_NAMES = ["POLAR_OK", "POLAR_ERR_NULL_ARG", "POLAR_ERR_BAD_SHAPE", "POLAR_ERR_UNSUPPORTED",
                "POLAR_ERR_BAD_PARAM", "POLAR_ERR_MISALIGNED", "POLAR_ERR_WORKSPACE", "POLAR_ERR_ALIAS",
                "POLAR_ERR_HIP"]


class PolarVariant(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_int32), ("train_len", ctypes.c_int32), ("floor_level", ctypes.c_int32),
                ("key_floor", ctypes.c_int32), ("saturation", ctypes.c_int32), ("window", ctypes.c_int32)]


class PolarProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("seq_q", ctypes.c_int32), ("seq_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("len_temp", ctypes.POINTER(ctypes.c_float)), ("null_bias", ctypes.POINTER(ctypes.c_float)),
                ("count_scale", ctypes.POINTER(ctypes.c_float)), ("variant", ctypes.POINTER(PolarVariant))]


# Reading variants by name (polar_variant in include/polar_attn.h); a variant is a dict
# of any of these keys, the missing ones taking the first (default) value.
VARIANT_CODES = {
    "temperature": {"log": 0, "ssmax": 1, "train_ratio": 2},
    "floor_level": {"gauss": 0, "gumbel2": 1, "qnorm": 2},
    "key_floor": {"null": 0, "soft": 1, "gate": 2},
    "saturation": {"log": 0, "log1p": 1},
}


def _variant_c(variant):
    """polar_variant for a dict such as {"key_floor": "soft", "window": 256}, or None."""
    if not variant:
        return None
    unknown = set(variant) - set(VARIANT_CODES) - {"train_len", "window"}
    if unknown:
        raise ValueError(f"unknown variant keys {sorted(unknown)}")
    codes = {}
    for key, table in VARIANT_CODES.items():
        name = variant.get(key, next(iter(table)))
        if name not in table:
            raise ValueError(f"variant {key}={name!r}; choose from {sorted(table)}")
        codes[key] = table[name]
    return PolarVariant(codes["temperature"], int(variant.get("train_len", 2048)), codes["floor_level"],
                        codes["key_floor"], codes["saturation"], int(variant.get("window", 0)))


class PolarOutputs(ctypes.Structure):
    _fields_ = [("direction", ctypes.c_void_p), ("n_eff", ctypes.c_void_p), ("confidence", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("stats", ctypes.c_void_p)]


class PolarPagedKV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32)]


class PolarGrads(ctypes.Structure):
    _fields_ = [("d_direction", ctypes.c_void_p), ("d_n_eff", ctypes.c_void_p), ("d_confidence", ctypes.c_void_p),
                ("d_count", ctypes.c_void_p)]


class PolarError(RuntimeError):
    def __init__(self, status: int, lib_message: str):
        self.status = status
        self.name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{self.name}: {lib_message}")


class PolarArgumentError(PolarError, ValueError):
    """A status other than POLAR_ERR_HIP: the call was rejected before any launch."""


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_attention_polar_amd.build`")
    lib = ctypes.CDLL(path)
    P, O = ctypes.POINTER(PolarProblem), ctypes.POINTER(PolarOutputs)
    vp = ctypes.c_void_p
    lib.polar_attn_fwd.argtypes = [P, vp, vp, vp, O, vp]
    lib.polar_attn_fwd.restype = ctypes.c_int
    lib.polar_attn_decode.argtypes = [P, vp, vp, vp, ctypes.c_int32, vp, ctypes.c_size_t, O, vp]
    lib.polar_attn_decode.restype = ctypes.c_int
    lib.polar_attn_merge.argtypes = [P, vp, ctypes.c_int32, O, vp]
    lib.polar_attn_merge.restype = ctypes.c_int
    lib.polar_attn_decode_num_splits.argtypes = [P, ctypes.c_int32]
    lib.polar_attn_decode_num_splits.restype = ctypes.c_int32
    lib.polar_attn_decode_noalloc.argtypes = [P, vp, vp, vp, ctypes.c_int32, O, vp]
    lib.polar_attn_decode_noalloc.restype = ctypes.c_int
    lib.polar_attn_decode_workspace_bytes.argtypes = [P, ctypes.c_int32]
    lib.polar_attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.polar_attn_fwd_partial.argtypes = [P, vp, vp, vp, ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp]
    lib.polar_attn_fwd_partial.restype = ctypes.c_int
    K = ctypes.POINTER(PolarPagedKV)
    lib.polar_attn_decode_paged.argtypes = [P, vp, K, ctypes.c_int32, vp, ctypes.c_size_t, O, vp]
    lib.polar_attn_decode_paged.restype = ctypes.c_int
    lib.polar_attn_decode_paged_num_splits.argtypes = [P, K, ctypes.c_int32]
    lib.polar_attn_decode_paged_num_splits.restype = ctypes.c_int32
    lib.polar_attn_decode_paged_workspace_bytes.argtypes = [P, K, ctypes.c_int32]
    lib.polar_attn_decode_paged_workspace_bytes.restype = ctypes.c_size_t
    Gr = ctypes.POINTER(PolarGrads)
    lib.polar_attn_bwd.argtypes = [P, vp, vp, vp, Gr, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.polar_attn_bwd.restype = ctypes.c_int
    lib.polar_attn_bwd_workspace_bytes.argtypes = [P]
    lib.polar_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.polar_attn_bwd_saved.argtypes = [P, vp, vp, vp, vp, Gr, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.polar_attn_bwd_saved.restype = ctypes.c_int
    lib.polar_attn_bwd_saved_workspace_bytes.argtypes = [P]
    lib.polar_attn_bwd_saved_workspace_bytes.restype = ctypes.c_size_t
    lib.polar_status_string.argtypes = [ctypes.c_int]
    lib.polar_status_string.restype = ctypes.c_char_p
    lib.polar_abi_version.argtypes = []
    lib.polar_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().polar_abi_version())


def status_string(status: int) -> str:
    return load_library().polar_status_string(status).decode()


def _check(status: int):
    if status != 0:
        cls = PolarError if status == 8 else PolarArgumentError
        raise cls(status, status_string(status))


def _float_array(vals, heads):
    if vals is None:
        return None, None
    if len(vals) != heads:
        raise ValueError(f"per-head parameter needs {heads} values, got {len(vals)}")
    arr = (ctypes.c_float * heads)(*[float(x) for x in vals])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)), arr


@dataclass
class Problem:
    """Sizes and parameters of one call (see polar_problem in include/polar_attn.h)."""
    batch: int
    heads: int
    kv_heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    causal: bool = True
    dtype: int = POLAR_BF16
    softmax_scale: float = 0.0
    len_temp: list | None = None
    null_bias: list | None = None
    count_scale: list | None = None
    variant: dict | None = None

    def to_c(self):
        lt, k1 = _float_array(self.len_temp, self.heads)
        nb, k2 = _float_array(self.null_bias, self.heads)
        cs, k3 = _float_array(self.count_scale, self.heads)
        var = _variant_c(self.variant)
        vp = ctypes.pointer(var) if var is not None else None
        pr = PolarProblem(self.batch, self.heads, self.kv_heads, self.seq_q, self.seq_k, self.head_dim,
                          int(bool(self.causal)), self.dtype, self.softmax_scale, lt, nb, cs, vp)
        return pr, (k1, k2, k3, var)  # keep the arrays alive during the call


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return POLAR_BF16
    if t.dtype == torch.float32:
        return POLAR_F32
    raise ValueError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def allocate_outputs(B, H, Tq, d, device, confidence=True, count=True, stats=False):
    f = dict(device=device, dtype=torch.float32)
    return {
        "direction": torch.empty(B, H, Tq, d, **f),
        "n_eff": torch.empty(B, H, Tq, **f),
        "confidence": torch.empty(B, H, Tq, **f) if confidence else None,
        "count": torch.empty(B, H, Tq, **f) if count else None,
        "stats": torch.empty(B, H, Tq, 3, **f) if stats else None,
    }


def _outputs_c(out):
    return PolarOutputs(_ptr(out["direction"]), _ptr(out["n_eff"]), _ptr(out.get("confidence")),
                        _ptr(out.get("count")), _ptr(out.get("stats")))


def _check_tensor(name, t, device):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def problem_for(q, k, *, causal=True, len_temp=None, null_bias=None, count_scale=None, softmax_scale=None,
                variant=None):
    B, H, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    return Problem(B, H, Hkv, Tq, Tk, d, causal, _dtype_code(q), float(softmax_scale or 0.0),
                   None if len_temp is None else list(len_temp),
                   None if null_bias is None else list(null_bias),
                   None if count_scale is None else list(count_scale), variant)


def fwd(q, k, v, *, causal=True, len_temp=None, null_bias=None, count_scale=None, softmax_scale=None,
        out=None, stats=False, variant=None):
    """Fused Polar Attention forward (polar_attn_fwd).

    q [B,H,Tq,d], k and v [B,Hkv,Tk,d] (bf16 or fp32, contiguous, on one GPU).
    Returns a dict with direction [B,H,Tq,d], n_eff, confidence, count [B,H,Tq] (fp32)
    and stats [B,H,Tq,3] when stats=True.  `variant`: a reading variant (see
    VARIANT_CODES), None for the default reading.  Work is enqueued on the current stream.
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, dev)
    if k.shape != v.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must match each other and q's dtype")
    prob = problem_for(q, k, causal=causal, len_temp=len_temp, null_bias=null_bias, count_scale=count_scale,
                       softmax_scale=softmax_scale, variant=variant)
    if out is None:
        out = allocate_outputs(prob.batch, prob.heads, prob.seq_q, prob.head_dim, dev, stats=stats)
    pr, keep = prob.to_c()
    oc = _outputs_c(out)
    _check(load_library().polar_attn_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(oc),
                                         _stream(dev)))
    return out


def fwd_partial(q, k, v, *, causal=True, context_k=0, partials=None, num_splits=1, split=0, len_temp=None,
                null_bias=None, count_scale=None, softmax_scale=None, variant=None):
    """Partial forward (polar_attn_fwd_partial): writes the (m, S1, S2, acc) rows of this
    call's keys into slot `split` of partials [B,H,Tq,num_splits,d+3] fp32 (allocated, with
    m = -inf everywhere, when not given) and returns it.  context_k: keys of the whole
    causal context this call is a piece of (0: the call is the whole context)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, dev)
    if k.shape != v.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must match each other and q's dtype")
    prob = problem_for(q, k, causal=causal, len_temp=len_temp, null_bias=null_bias, count_scale=count_scale,
                       softmax_scale=softmax_scale, variant=variant)
    shape = (prob.batch, prob.heads, prob.seq_q, num_splits, prob.head_dim + 3)
    if partials is None:
        partials = torch.zeros(shape, dtype=torch.float32, device=dev)
        partials[..., 0] = float("-inf")
    elif tuple(partials.shape) != shape or partials.dtype != torch.float32:
        raise ValueError(f"partials must be float32 {shape}")
    _check_tensor("partials", partials, dev)
    pr, keep = prob.to_c()
    _check(load_library().polar_attn_fwd_partial(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), int(context_k),
                                                 _ptr(partials), num_splits, split, _stream(dev)))
    return partials


def decode_num_splits(prob: Problem, num_splits: int = 0) -> int:
    pr, keep = prob.to_c()
    return int(load_library().polar_attn_decode_num_splits(ctypes.byref(pr), num_splits))


def decode_workspace_bytes(prob: Problem, num_splits: int = 0) -> int:
    pr, keep = prob.to_c()
    return int(load_library().polar_attn_decode_workspace_bytes(ctypes.byref(pr), num_splits))


def decode(q, k_cache, v_cache, *, num_splits=0, len_temp=None, null_bias=None, count_scale=None,
           softmax_scale=None, workspace=None, out=None, stats=False, variant=None):
    """Split-KV decode (polar_attn_decode): q [B,H,1,d] against caches [B,Hkv,Tk,d], bf16.

    Returns the same dict as fwd(); `workspace` (a uint8 device tensor) is allocated
    when not given, and the partials it holds are returned under "partials"."""
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(name, t, dev)
    prob = problem_for(q, k_cache, causal=True, len_temp=len_temp, null_bias=null_bias,
                       count_scale=count_scale, softmax_scale=softmax_scale, variant=variant)
    lib = load_library()
    pr, keep = prob.to_c()
    splits = int(lib.polar_attn_decode_num_splits(ctypes.byref(pr), num_splits))
    need = int(lib.polar_attn_decode_workspace_bytes(ctypes.byref(pr), num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = allocate_outputs(prob.batch, prob.heads, prob.seq_q, prob.head_dim, dev, stats=stats)
    oc = _outputs_c(out)
    _check(lib.polar_attn_decode(ctypes.byref(pr), _ptr(q), _ptr(k_cache), _ptr(v_cache), num_splits,
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), ctypes.byref(oc),
                                 _stream(dev)))
    out["splits"] = splits
    if splits > 0:
        out["partials"] = _partials_view(workspace, prob, splits)
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # POLAR_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q, k_cache, v_cache, out, *, num_splits=0, len_temp=None, null_bias=None, count_scale=None,
                   softmax_scale=None, variant=None):
    """Split-KV decode that allocates nothing (polar_attn_decode_noalloc): as decode(),
    but the split partials live in the library's own per-GPU array, so the caller passes
    the outputs (see allocate_outputs) and no workspace.  Returns `out`."""
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(name, t, dev)
    prob = problem_for(q, k_cache, causal=True, len_temp=len_temp, null_bias=null_bias,
                       count_scale=count_scale, softmax_scale=softmax_scale, variant=variant)
    pr, keep = prob.to_c()
    oc = _outputs_c(out)
    _check(load_library().polar_attn_decode_noalloc(ctypes.byref(pr), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                    num_splits, ctypes.byref(oc), _stream(dev)))
    return out


def _partials_view(workspace, prob, splits):
    n = prob.batch * prob.heads * prob.seq_q * splits * (prob.head_dim + 3)
    return workspace[:n * 4].view(torch.float32).view(prob.batch, prob.heads, prob.seq_q, splits, prob.head_dim + 3)


def paged_kv(k_pool, v_pool, block_table, seq_lens):
    """Describe a paged cache: pools [num_blocks, block_size, Hkv, d] bf16, block_table
    [B, max_blocks] int32 and seq_lens [B] int32, all on one GPU."""
    dev = k_pool.device
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool), ("block_table", block_table), ("seq_lens", seq_lens)):
        _check_tensor(name, t, dev)
    if k_pool.shape != v_pool.shape or k_pool.dim() != 4:
        raise ValueError("k_pool and v_pool must both be [num_blocks, block_size, kv_heads, head_dim]")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or seq_lens.dim() != 1 or seq_lens.shape[0] != block_table.shape[0]:
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    nb, bs = k_pool.shape[0], k_pool.shape[1]
    return PolarPagedKV(_ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), nb, bs, block_table.shape[1])


def decode_paged_workspace_bytes(prob: Problem, kv: PolarPagedKV, num_splits: int = 0) -> int:
    pr, keep = prob.to_c()
    return int(load_library().polar_attn_decode_paged_workspace_bytes(ctypes.byref(pr), ctypes.byref(kv),
                                                                      num_splits))


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, *, seq_k=None, num_splits=0, len_temp=None,
                 null_bias=None, count_scale=None, softmax_scale=None, workspace=None, out=None, stats=False,
                 variant=None):
    """Grouped split-KV decode over a paged cache (polar_attn_decode_paged).

    q [B,H,1,d] bf16; pools [num_blocks, block_size, Hkv, d] bf16; block_table [B, max_blocks]
    and seq_lens [B] int32.  seq_k: the largest sequence length (default: the table's
    capacity, max_blocks * block_size).  Returns the same dict as decode()."""
    dev = q.device
    _check_tensor("q", q, dev)
    kv = paged_kv(k_pool, v_pool, block_table, seq_lens)
    B, H, Tq, d = q.shape
    Hkv = k_pool.shape[2]
    if k_pool.shape[3] != d or block_table.shape[0] != B:
        raise ValueError("q, the pools and the block table disagree")
    if seq_k is None:
        seq_k = kv.max_blocks * kv.block_size
    prob = Problem(B, H, Hkv, Tq, int(seq_k), d, False, _dtype_code(q), float(softmax_scale or 0.0),
                   None if len_temp is None else list(len_temp),
                   None if null_bias is None else list(null_bias),
                   None if count_scale is None else list(count_scale), variant)
    lib = load_library()
    pr, keep = prob.to_c()
    splits = int(lib.polar_attn_decode_paged_num_splits(ctypes.byref(pr), ctypes.byref(kv), num_splits))
    need = int(lib.polar_attn_decode_paged_workspace_bytes(ctypes.byref(pr), ctypes.byref(kv), num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = allocate_outputs(B, H, Tq, d, dev, stats=stats)
    oc = _outputs_c(out)
    _check(lib.polar_attn_decode_paged(ctypes.byref(pr), _ptr(q), ctypes.byref(kv), num_splits, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), ctypes.byref(oc),
                                       _stream(dev)))
    out["splits"] = splits
    if splits > 0:
        out["partials"] = _partials_view(workspace, prob, splits)
    return out


GRAD_NAMES = ("direction", "n_eff", "confidence", "count")


def bwd_workspace_bytes(prob: Problem) -> int:
    pr, keep = prob.to_c()
    return int(load_library().polar_attn_bwd_workspace_bytes(ctypes.byref(pr)))


def bwd_saved_workspace_bytes(prob: Problem) -> int:
    pr, keep = prob.to_c()
    return int(load_library().polar_attn_bwd_saved_workspace_bytes(ctypes.byref(pr)))


def bwd(q, k, v, grads, *, causal=True, len_temp=None, null_bias=None, count_scale=None, softmax_scale=None,
        workspace=None, out=None, variant=None, saved=None):
    """Backward of the forward (polar_attn_bwd): gradients of
    sum(grads["direction"] * direction) + sum(grads["n_eff"] * n_eff) + ... with respect to
    q, k, v.  grads maps any of "direction" [B,H,Tq,d], "n_eff", "confidence", "count"
    [B,H,Tq] to fp32 tensors on q's device (a missing entry is zero).  Returns a dict with
    dq [B,H,Tq,d] and dk, dv [B,Hkv,Tk,d], fp32.  Work is enqueued on the current stream.
    saved: the forward's row statistics [B,H,Tq,d+3] (or [B,H,Tq,1,d+3]) fp32 as
    fwd_partial writes them with one split; bf16 inputs only (polar_attn_bwd_saved)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, dev)
    if k.shape != v.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must match each other and q's dtype")
    unknown = set(grads) - set(GRAD_NAMES)
    if unknown:
        raise ValueError(f"unknown gradient names {sorted(unknown)}")
    prob = problem_for(q, k, causal=causal, len_temp=len_temp, null_bias=null_bias, count_scale=count_scale,
                       softmax_scale=softmax_scale, variant=variant)
    row_shape = (prob.batch, prob.heads, prob.seq_q)
    for name in GRAD_NAMES:
        t = grads.get(name)
        if t is None:
            continue
        shape = tuple(q.shape) if name == "direction" else row_shape
        if tuple(t.shape) != shape or t.dtype != torch.float32:
            raise ValueError(f"grads[{name!r}] must be float32 {shape}")
        _check_tensor(f"grads[{name!r}]", t, dev)
    g = PolarGrads(*[_ptr(grads.get(name)) for name in GRAD_NAMES])
    if saved is not None:
        d = q.shape[-1]
        if saved.dtype != torch.float32 or saved.numel() != prob.batch * prob.heads * prob.seq_q * (d + 3) or \
                not saved.is_contiguous():
            raise ValueError(f"saved must be contiguous float32 [B,H,Tq,{d + 3}]")
        _check_tensor("saved", saved, dev)
    need = bwd_saved_workspace_bytes(prob) if saved is not None else bwd_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_tensor("workspace", workspace, dev)
    if out is None:
        f = dict(device=dev, dtype=torch.float32)
        out = {"dq": torch.empty(q.shape, **f), "dk": torch.empty(k.shape, **f), "dv": torch.empty(v.shape, **f)}
    for name, like in (("dq", q), ("dk", k), ("dv", v)):
        t = out[name]
        if tuple(t.shape) != tuple(like.shape) or t.dtype != torch.float32:
            raise ValueError(f"out[{name!r}] must be float32 {tuple(like.shape)}")
        _check_tensor(f"out[{name!r}]", t, dev)
    pr, keep = prob.to_c()
    nbytes = workspace.numel() * workspace.element_size()
    if saved is not None:
        _check(load_library().polar_attn_bwd_saved(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(saved),
                                                   ctypes.byref(g), _ptr(out["dq"]), _ptr(out["dk"]),
                                                   _ptr(out["dv"]), _ptr(workspace), nbytes, _stream(dev)))
    else:
        _check(load_library().polar_attn_bwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(g),
                                             _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(workspace),
                                             nbytes, _stream(dev)))
    return out


def merge(partials, *, seq_k, causal=True, len_temp=None, null_bias=None, count_scale=None, out=None,
          stats=False, variant=None):
    """Merge split statistics (polar_attn_merge): partials [B,H,Tq,S,d+3] fp32 on the GPU."""
    dev = partials.device
    _check_tensor("partials", partials, dev)
    if partials.dtype != torch.float32:
        raise ValueError("partials must be float32")
    B, H, Tq, S, W = partials.shape
    d = W - 3
    prob = Problem(B, H, H, Tq, seq_k, d, causal, POLAR_BF16, 0.0,
                   None if len_temp is None else list(len_temp),
                   None if null_bias is None else list(null_bias),
                   None if count_scale is None else list(count_scale), variant)
    if out is None:
        out = allocate_outputs(B, H, Tq, d, dev, stats=stats)
    pr, keep = prob.to_c()
    oc = _outputs_c(out)
    _check(load_library().polar_attn_merge(ctypes.byref(pr), _ptr(partials), S, ctypes.byref(oc), _stream(dev)))
    return out


__all__ = ["PolarVariant", "VARIANT_CODES", "fwd", "bwd", "decode_noalloc", "NOALLOC_SCRATCH_BYTES", "bwd_workspace_bytes", "bwd_saved_workspace_bytes", "PolarGrads", "fwd_partial", "decode", "decode_paged", "paged_kv", "decode_paged_workspace_bytes", "merge", "decode_num_splits", "decode_workspace_bytes", "abi_version",
           "status_string", "load_library", "Problem", "PolarError", "PolarArgumentError", "allocate_outputs",
           "LIB_PATH"]

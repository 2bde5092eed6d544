"""Fused linear cross-entropy (forward + backward) on MI355X: Python binding.

Thin ctypes layer over ``libflce.so`` (built from ``csrc/`` by
``linear_cross_entropy_bwd_amd.build``).  The functions named like the C
entry points take the same arguments as the C ABI; tensor arguments may be
passed as torch tensors (their ``data_ptr()`` is used) or raw device
addresses.  Every step of the computation runs in the library's HIP kernels;
torch only provides device memory and the stream.  There is no fallback: if
the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflce.so")

FLCE_BF16, FLCE_F32 = 0, 1
FLCE_MEAN, FLCE_SUM = 0, 1
FLCE_OK, FLCE_ERR_INVALID_ARG, FLCE_ERR_ALIGNMENT, FLCE_ERR_OOM, FLCE_ERR_HIP = 0, -1, -2, -3, -4
FLCE_ERR_SCRATCH = -5
FLCE_NOALLOC_SCRATCH_BYTES = 64 << 20
ENGINE_MFMA, ENGINE_FMA = 0, 1

EXPORTED = (
    "flce_fwd_bwd",
    "flce_fwd_bwd_lowmem",
    "flce_fwd",
    "flce_fwd_noalloc",
    "flce_bwd",
    "flce_ce_logits",
    "flce_fwd_fp8",
    "flce_bwd_fp8",
    "flce_fwd_shard",
    "flce_merge_shards",
    "flce_bwd_shard",
    "flce_bwd_shard_accumulate",
    "flce_sum_parts",
    "flce_scale",
    "flce_workspace_bytes",
    "flce_workspace_bytes_lowmem",
    "flce_plan_info",
    "flce_lowmem_plan_info",
    "flce_strerror",
    "flce_profile_enable",
    "flce_profile_read",
    "flce_profile_kind_name",
    "flce_memory_high_water",
    "flce_memory_reserved",
    "flce_pool_trim",
)


class FlceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {strerror(status)}")


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("chunk_rows", ctypes.c_int64),
        ("num_chunks", ctypes.c_int64),
        ("vocab_pitch", ctypes.c_int64),
        ("group_cols", ctypes.c_int64),
        ("dh_splits", ctypes.c_int64),
        ("engine", ctypes.c_int32),
        ("dw_accumulator", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("prob_buffer_bytes", ctypes.c_size_t),
        ("dw_pairs", ctypes.c_int32),
        ("folded_factor", ctypes.c_int32),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class LowmemPlanInfo(ctypes.Structure):
    _fields_ = [
        ("slice_cols", ctypes.c_int64),
        ("num_slices", ctypes.c_int64),
        ("slice_chunk_rows", ctypes.c_int64),
        ("slice_chunks", ctypes.c_int64),
        ("fwd_chunk_rows", ctypes.c_int64),
        ("buffer_budget_bytes", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflce.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m linear_cross_entropy_bwd_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.flce_fwd_bwd.argtypes = [p, p, p, i64, i64, i64, i32, i64, i32, p, p, p, p, p]
    L.flce_fwd_bwd.restype = i32
    L.flce_fwd_bwd_lowmem.argtypes = [p, p, p, i64, i64, i64, i32, i64, i32, p, p, p, p, p]
    L.flce_fwd_bwd_lowmem.restype = i32
    L.flce_workspace_bytes_lowmem.argtypes = [i64, i64, i64, i32]
    L.flce_workspace_bytes_lowmem.restype = ctypes.c_size_t
    L.flce_lowmem_plan_info.argtypes = [i64, i64, i64, i32, ctypes.POINTER(LowmemPlanInfo)]
    L.flce_lowmem_plan_info.restype = i32
    L.flce_memory_reserved.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    L.flce_memory_reserved.restype = i32
    L.flce_pool_trim.argtypes = [ctypes.c_uint64]
    L.flce_pool_trim.restype = i32
    L.flce_fwd.argtypes = [p, p, p, i64, i64, i64, i32, i64, i32, p, p, p]
    L.flce_fwd.restype = i32
    L.flce_fwd_noalloc.argtypes = [p, p, p, i64, i64, i64, i32, i64, i32, p, p, p]
    L.flce_fwd_noalloc.restype = i32
    L.flce_bwd.argtypes = [p, p, p, p, p, i64, i64, i64, i32, i64, i32, p, p, p]
    L.flce_bwd.restype = i32
    L.flce_ce_logits.argtypes = [p, p, i64, i64, i32, i64, i32, p, p, p, p, p, p]
    L.flce_ce_logits.restype = i32
    L.flce_fwd_fp8.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, p, p, p]
    L.flce_fwd_fp8.restype = i32
    L.flce_bwd_fp8.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i32, p, p, p]
    L.flce_bwd_fp8.restype = i32
    L.flce_fwd_shard.argtypes = [p, p, p, i64, i64, i64, i64, i32, i64, p, p, p]
    L.flce_fwd_shard.restype = i32
    L.flce_merge_shards.argtypes = [p, p, i64, p, i64, i64, i32, p, p, p]
    L.flce_merge_shards.restype = i32
    L.flce_bwd_shard.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, i64, i32, p, p, p]
    L.flce_bwd_shard.restype = i32
    L.flce_bwd_shard_accumulate.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, i64, i32, p, p, p]
    L.flce_bwd_shard_accumulate.restype = i32
    L.flce_sum_parts.argtypes = [p, i64, i64, i32, p, p]
    L.flce_sum_parts.restype = i32
    L.flce_scale.argtypes = [p, i64, i32, p, p]
    L.flce_scale.restype = i32
    L.flce_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.flce_workspace_bytes.restype = ctypes.c_size_t
    L.flce_plan_info.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(PlanInfo)]
    L.flce_plan_info.restype = i32
    L.flce_strerror.argtypes = [i32]
    L.flce_strerror.restype = ctypes.c_char_p
    L.flce_profile_enable.argtypes = [i32]
    L.flce_profile_enable.restype = i32
    L.flce_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    L.flce_profile_read.restype = i32
    L.flce_profile_kind_name.argtypes = [i32]
    L.flce_profile_kind_name.restype = ctypes.c_char_p
    L.flce_memory_high_water.argtypes = [i32, ctypes.POINTER(ctypes.c_uint64)]
    L.flce_memory_high_water.restype = i32
    del f
    _lib = L
    return L


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def strerror(status: int) -> str:
    try:
        return lib().flce_strerror(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


# --- the C entry points ------------------------------------------------------------

def flce_fwd_bwd(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, dh_out, dw_out,
                 stream) -> int:
    return lib().flce_fwd_bwd(_ptr(h), _ptr(w), _ptr(labels), n, d, v, dtype, ignore_index, reduction,
                              _ptr(loss_out), _ptr(lse_out), _ptr(dh_out), _ptr(dw_out), _stream(stream))


def flce_fwd_bwd_lowmem(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, dh_out, dw_out,
                        stream) -> int:
    return lib().flce_fwd_bwd_lowmem(_ptr(h), _ptr(w), _ptr(labels), n, d, v, dtype, ignore_index, reduction,
                                     _ptr(loss_out), _ptr(lse_out), _ptr(dh_out), _ptr(dw_out), _stream(stream))


def flce_fwd(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, stream) -> int:
    return lib().flce_fwd(_ptr(h), _ptr(w), _ptr(labels), n, d, v, dtype, ignore_index, reduction,
                          _ptr(loss_out), _ptr(lse_out), _stream(stream))


def flce_fwd_noalloc(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, stream) -> int:
    return lib().flce_fwd_noalloc(_ptr(h), _ptr(w), _ptr(labels), n, d, v, dtype, ignore_index, reduction,
                                  _ptr(loss_out), _ptr(lse_out), _stream(stream))


def flce_bwd(h, w, labels, lse, grad_out, n, d, v, dtype, ignore_index, reduction, dh_out, dw_out, stream) -> int:
    return lib().flce_bwd(_ptr(h), _ptr(w), _ptr(labels), _ptr(lse), _ptr(grad_out), n, d, v, dtype, ignore_index,
                          reduction, _ptr(dh_out), _ptr(dw_out), _stream(stream))


def flce_ce_logits(logits, labels, n, v, dtype, ignore_index, reduction, lse_in, grad_scale, loss_out, lse_out,
                   grad_out, stream) -> int:
    return lib().flce_ce_logits(_ptr(logits), _ptr(labels), n, v, dtype, ignore_index, reduction, _ptr(lse_in),
                                _ptr(grad_scale), _ptr(loss_out), _ptr(lse_out), _ptr(grad_out), _stream(stream))


def flce_fwd_fp8(h_q, h_scale, w_q, w_scale, labels, n, d, v, ignore_index, reduction, loss_out, lse_out,
                 stream) -> int:
    return lib().flce_fwd_fp8(_ptr(h_q), _ptr(h_scale), _ptr(w_q), _ptr(w_scale), _ptr(labels), n, d, v,
                              ignore_index, reduction, _ptr(loss_out), _ptr(lse_out), _stream(stream))


def flce_bwd_fp8(h_q, h_scale, w_q, w_scale, labels, lse, grad_out, n, d, v, ignore_index, reduction, dh_out, dw_out,
                 stream) -> int:
    return lib().flce_bwd_fp8(_ptr(h_q), _ptr(h_scale), _ptr(w_q), _ptr(w_scale), _ptr(labels), _ptr(lse),
                              _ptr(grad_out), n, d, v, ignore_index, reduction, _ptr(dh_out), _ptr(dw_out),
                              _stream(stream))


def flce_fwd_shard(h, w_shard, labels, n, d, v_shard, v_first, dtype, ignore_index, lse_part_out, zy_part_out,
                   stream) -> int:
    return lib().flce_fwd_shard(_ptr(h), _ptr(w_shard), _ptr(labels), n, d, v_shard, v_first, dtype, ignore_index,
                                _ptr(lse_part_out), _ptr(zy_part_out), _stream(stream))


def flce_merge_shards(lse_parts, zy_parts, num_shards, labels, n, ignore_index, reduction, loss_out, lse_out,
                      stream) -> int:
    return lib().flce_merge_shards(_ptr(lse_parts), _ptr(zy_parts), num_shards, _ptr(labels), n, ignore_index,
                                   reduction, _ptr(loss_out), _ptr(lse_out), _stream(stream))


def flce_bwd_shard(h, w_shard, labels, lse, grad_out, n, d, v_shard, v_first, dtype, ignore_index, reduction,
                   dh_part_out, dw_shard_out, stream) -> int:
    return lib().flce_bwd_shard(_ptr(h), _ptr(w_shard), _ptr(labels), _ptr(lse), _ptr(grad_out), n, d, v_shard,
                                v_first, dtype, ignore_index, reduction, _ptr(dh_part_out), _ptr(dw_shard_out),
                                _stream(stream))


def flce_bwd_shard_accumulate(h, w_shard, labels, lse, grad_out, n, d, v_shard, v_first, dtype, ignore_index,
                              reduction, dh_acc, dw_shard_out, stream) -> int:
    return lib().flce_bwd_shard_accumulate(_ptr(h), _ptr(w_shard), _ptr(labels), _ptr(lse), _ptr(grad_out), n, d,
                                           v_shard, v_first, dtype, ignore_index, reduction, _ptr(dh_acc),
                                           _ptr(dw_shard_out), _stream(stream))


def flce_sum_parts(parts, num_parts, count, dtype, out, stream) -> int:
    return lib().flce_sum_parts(_ptr(parts), num_parts, count, dtype, _ptr(out), _stream(stream))


def flce_scale(x, count, dtype, scale, stream) -> int:
    return lib().flce_scale(_ptr(x), count, dtype, _ptr(scale), _stream(stream))


def flce_workspace_bytes(n, d, v, dtype, with_bwd) -> int:
    return int(lib().flce_workspace_bytes(n, d, v, dtype, int(with_bwd)))


def flce_plan_info(n, d, v, dtype, with_bwd) -> dict:
    info = PlanInfo()
    st = lib().flce_plan_info(n, d, v, dtype, int(with_bwd), ctypes.byref(info))
    if st != FLCE_OK:
        raise FlceError(st, "flce_plan_info")
    return info.as_dict()


def flce_workspace_bytes_lowmem(n, d, v, dtype) -> int:
    return int(lib().flce_workspace_bytes_lowmem(n, d, v, dtype))


def flce_lowmem_plan_info(n, d, v, dtype) -> dict:
    info = LowmemPlanInfo()
    st = lib().flce_lowmem_plan_info(n, d, v, dtype, ctypes.byref(info))
    if st != FLCE_OK:
        raise FlceError(st, "flce_lowmem_plan_info")
    return info.as_dict()


def flce_strerror(status: int) -> str:
    return strerror(status)


def flce_profile_enable(on: bool) -> int:
    return lib().flce_profile_enable(1 if on else 0)


def flce_profile_read() -> dict:
    """{kind name: (launches, total ms)} since the previous read."""
    n = 16
    launches = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    st = lib().flce_profile_read(n, launches, ms)
    if st != FLCE_OK:
        raise FlceError(st, "flce_profile_read")
    out = {}
    for k in range(n):
        name = lib().flce_profile_kind_name(k)
        if name is not None:
            out[name.decode()] = (int(launches[k]), float(ms[k]))
    return out


def flce_memory_high_water(reset: bool = False) -> int:
    v = ctypes.c_uint64(0)
    st = lib().flce_memory_high_water(1 if reset else 0, ctypes.byref(v))
    if st != FLCE_OK:
        raise FlceError(st, "flce_memory_high_water")
    return int(v.value)


def flce_memory_reserved() -> int:
    """Bytes the library's pool on the current device holds (in use or cached)."""
    v = ctypes.c_uint64(0)
    st = lib().flce_memory_reserved(ctypes.byref(v))
    if st != FLCE_OK:
        raise FlceError(st, "flce_memory_reserved")
    return int(v.value)


def flce_pool_trim(keep_bytes: int = 0) -> int:
    """Return the pool's cached memory beyond keep_bytes to the device."""
    st = lib().flce_pool_trim(int(keep_bytes))
    if st != FLCE_OK:
        raise FlceError(st, "flce_pool_trim")
    return st


# --- tensor-level convenience ---------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FLCE_BF16
    if t.dtype == torch.float32:
        return FLCE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _red_code(reduction: str) -> int:
    if reduction == "mean":
        return FLCE_MEAN
    if reduction == "sum":
        return FLCE_SUM
    raise ValueError(f"unknown reduction {reduction!r}")


def _check_inputs(h, w, labels):
    import torch
    if not (h.is_cuda and w.is_cuda and labels.is_cuda):
        raise ValueError("h, w and labels must be device tensors")
    if h.dim() != 2 or w.dim() != 2 or labels.dim() != 1:
        raise ValueError("expected h [n, d], w [v, d], labels [n]")
    if h.shape[1] != w.shape[1] or labels.shape[0] != h.shape[0]:
        raise ValueError("shape mismatch between h, w and labels")
    if h.dtype != w.dtype:
        raise TypeError("h and w must share a dtype")
    if labels.dtype != torch.int64:
        raise TypeError("labels must be int64")
    if not (h.is_contiguous() and w.is_contiguous() and labels.is_contiguous()):
        raise ValueError("h, w and labels must be contiguous")
    if not (h.device == w.device == labels.device):
        raise ValueError("h, w and labels must be on one device")


def _debug_labels(labels, v: int, ignore_index: int):
    """With FLCE_CHECK_LABELS=1 in the environment: raise ValueError on a label that is
    neither ignore_index nor in [0, v).  Off by default: it synchronises with the host,
    and the kernels give such a row the documented meaning (target logit 0, no one-hot
    term) without reading out of bounds."""
    if os.environ.get("FLCE_CHECK_LABELS", "") in ("", "0"):
        return
    bad = (labels != ignore_index) & ((labels < 0) | (labels >= v))
    if bool(bad.any()):
        i = int(bad.nonzero()[0, 0])
        raise ValueError(f"label {int(labels[i])} at row {i} is outside [0, {v}) and is not "
                         f"ignore_index ({ignore_index})")


def _check_vec(t, n: int, device, name: str):
    """A contiguous fp32 [n] tensor on `device` (a saved LSE or an LSE output)."""
    import torch
    if t.dtype != torch.float32 or tuple(t.shape) != (n,) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous fp32 [{n}] tensor on {device}")


def _check_scalar(t, device, name: str):
    """None, or a contiguous one-element fp32 tensor on `device` (an upstream gradient, a loss output)."""
    import torch
    if t is None:
        return
    if t.dtype != torch.float32 or t.numel() != 1 or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous one-element fp32 tensor on {device}")


def _check_out(t, like, name: str):
    """A caller-supplied output: same shape, dtype and device as `like`, contiguous."""
    if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {like.dtype} {tuple(like.shape)} tensor on {like.device}")


def linear_cross_entropy(h, w, labels, ignore_index: int = -100, reduction: str = "mean", out=None):
    """Loss, per-row LSE, dH and dW of softmax(h w^T) against labels (one library call).

    Returns (loss fp32 [1], lse fp32 [n], dh [n, d], dw [v, d]) on h's device,
    computed on the current torch stream.  ``out`` may supply preallocated
    (loss, lse, dh, dw) tensors.
    """
    import torch
    _check_inputs(h, w, labels)
    n, d = h.shape
    v = w.shape[0]
    _debug_labels(labels, v, ignore_index)
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=h.device)
        lse = torch.empty(n, dtype=torch.float32, device=h.device)
        dh = torch.empty_like(h)
        dw = torch.empty_like(w)
    else:
        loss, lse, dh, dw = out
        _check_scalar(loss, h.device, "out loss")
        _check_vec(lse, n, h.device, "out lse")
        _check_out(dh, h, "out dh")
        _check_out(dw, w, "out dw")
    st = flce_fwd_bwd(h, w, labels, n, d, v, _dtype_code(h), ignore_index, _red_code(reduction), loss, lse, dh, dw,
                      torch.cuda.current_stream(h.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_fwd_bwd")
    return loss, lse, dh, dw


def scale_(x, scale):
    """x *= scale in place (flce_scale): ``x`` a contiguous bf16 or fp32 device tensor,
    ``scale`` a one-element fp32 tensor on the same device; a scale of exactly 1
    leaves x untouched.  Returns x."""
    import torch
    if not x.is_contiguous() or x.numel() == 0:
        raise ValueError("x must be a non-empty contiguous tensor")
    _check_scalar(scale, x.device, "scale")
    st = flce_scale(x, x.numel(), _dtype_code(x), scale, torch.cuda.current_stream(x.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_scale")
    return x


def linear_cross_entropy_lowmem(h, w, labels, ignore_index: int = -100, reduction: str = "mean", out=None):
    """As linear_cross_entropy, through flce_fwd_bwd_lowmem: the backward recomputes the
    logits slice by slice of the vocabulary, so the workspace stays near 4 n d bytes plus
    a 256 MiB slice buffer (8 N D V flop instead of 6)."""
    import torch
    _check_inputs(h, w, labels)
    n, d = h.shape
    v = w.shape[0]
    _debug_labels(labels, v, ignore_index)
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=h.device)
        lse = torch.empty(n, dtype=torch.float32, device=h.device)
        dh = torch.empty_like(h)
        dw = torch.empty_like(w)
    else:
        loss, lse, dh, dw = out
        _check_scalar(loss, h.device, "out loss")
        _check_vec(lse, n, h.device, "out lse")
        _check_out(dh, h, "out dh")
        _check_out(dw, w, "out dw")
    st = flce_fwd_bwd_lowmem(h, w, labels, n, d, v, _dtype_code(h), ignore_index, _red_code(reduction), loss, lse,
                             dh, dw, torch.cuda.current_stream(h.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_fwd_bwd_lowmem")
    return loss, lse, dh, dw


def linear_cross_entropy_forward(h, w, labels, ignore_index: int = -100, reduction: str = "mean"):
    """Loss and per-row LSE only (flce_fwd)."""
    import torch
    _check_inputs(h, w, labels)
    n, d = h.shape
    v = w.shape[0]
    _debug_labels(labels, v, ignore_index)
    loss = torch.empty(1, dtype=torch.float32, device=h.device)
    lse = torch.empty(n, dtype=torch.float32, device=h.device)
    st = flce_fwd(h, w, labels, n, d, v, _dtype_code(h), ignore_index, _red_code(reduction), loss, lse,
                  torch.cuda.current_stream(h.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_fwd")
    return loss, lse


def linear_cross_entropy_backward(h, w, labels, lse, grad_out=None, ignore_index: int = -100, reduction: str = "mean",
                                  out=None):
    """dH and dW of ``grad_out * loss`` from the saved per-row LSE, recomputing the logits (flce_bwd).

    ``lse`` is the fp32 [n] tensor the forward returned; ``grad_out`` a one-element
    fp32 device tensor (the upstream gradient) or None for 1.  ``out`` may supply
    preallocated (dh, dw).
    """
    import torch
    _check_inputs(h, w, labels)
    n, d = h.shape
    v = w.shape[0]
    _debug_labels(labels, v, ignore_index)
    _check_vec(lse, n, h.device, "lse")
    _check_scalar(grad_out, h.device, "grad_out")
    dh, dw = (torch.empty_like(h), torch.empty_like(w)) if out is None else out
    if out is not None:
        _check_out(dh, h, "out dh")
        _check_out(dw, w, "out dw")
    st = flce_bwd(h, w, labels, lse, grad_out, n, d, v, _dtype_code(h), ignore_index, _red_code(reduction), dh, dw,
                  torch.cuda.current_stream(h.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_bwd")
    return dh, dw


def _check_logits(logits, labels):
    import torch
    if not (logits.is_cuda and labels.is_cuda):
        raise ValueError("logits and labels must be device tensors")
    if logits.dim() != 2 or labels.dim() != 1 or labels.shape[0] != logits.shape[0]:
        raise ValueError("expected logits [n, v] and labels [n]")
    if labels.dtype != torch.int64:
        raise TypeError("labels must be int64")
    if not (logits.is_contiguous() and labels.is_contiguous()):
        raise ValueError("logits and labels must be contiguous")
    if logits.device != labels.device:
        raise ValueError("logits and labels must be on one device")


def cross_entropy(logits, labels, ignore_index: int = -100, reduction: str = "mean", grad: Optional[str] = None):
    """Cross-entropy on given logits (flce_ce_logits): returns (loss fp32 [1], lse fp32 [n], gradient or None).

    ``grad``: None (no gradient), "separate" (a new [n, v] tensor) or "inplace"
    (the gradient overwrites ``logits``, which is returned as the gradient).
    """
    import torch
    _check_logits(logits, labels)
    n, v = logits.shape
    _debug_labels(labels, v, ignore_index)
    loss = torch.empty(1, dtype=torch.float32, device=logits.device)
    lse = torch.empty(n, dtype=torch.float32, device=logits.device)
    if grad is None:
        g = None
    elif grad == "separate":
        g = torch.empty_like(logits)
    elif grad == "inplace":
        g = logits
    else:
        raise ValueError(f"unknown grad mode {grad!r}")
    st = flce_ce_logits(logits, labels, n, v, _dtype_code(logits), ignore_index, _red_code(reduction), None, None,
                        loss, lse, g, torch.cuda.current_stream(logits.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_ce_logits")
    return loss, lse, g


def cross_entropy_backward(logits, labels, lse, grad_scale=None, ignore_index: int = -100, reduction: str = "mean",
                           out=None):
    """Gradient of ``grad_scale * loss`` w.r.t. the logits from the saved LSE (flce_ce_logits with lse_in)."""
    import torch
    _check_logits(logits, labels)
    n, v = logits.shape
    _debug_labels(labels, v, ignore_index)
    _check_vec(lse, n, logits.device, "lse")
    _check_scalar(grad_scale, logits.device, "grad_scale")
    g = torch.empty_like(logits) if out is None else out
    if out is not None:
        _check_out(g, logits, "out")   # may be `logits` itself: the gradient over the logits
    st = flce_ce_logits(logits, labels, n, v, _dtype_code(logits), ignore_index, _red_code(reduction), lse,
                        grad_scale, None, None, g, torch.cuda.current_stream(logits.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_ce_logits")
    return g


def vocab_shard_bounds(v: int, num_shards: int):
    """Contiguous shards [a, b) covering [0, v): sizes differ by at most 256 (whole 256-row blocks)."""
    if num_shards < 1 or num_shards > v:
        raise ValueError("need 1 <= num_shards <= v")
    blocks = (v + 255) // 256
    if num_shards > blocks:
        cuts = [v * q // num_shards for q in range(num_shards + 1)]
    else:
        cuts = [min(v, (blocks * q // num_shards) * 256) for q in range(num_shards + 1)]
    return list(zip(cuts[:-1], cuts[1:]))


def linear_cross_entropy_vocab_split(h, w, labels, num_shards: int = 2, ignore_index: int = -100,
                                     reduction: str = "mean", grad_out=None, shards=None):
    """Fused linear cross-entropy with W's vocabulary rows split into shards, on one GPU.

    Per shard the partial forward (flce_fwd_shard), then the exact merge
    (flce_merge_shards), then per shard the backward from the merged LSE, its
    dH term added into one fp32 [n, d] sum (flce_bwd_shard for the first,
    flce_bwd_shard_accumulate for the others), rounded to the input dtype by
    flce_sum_parts.  Returns (loss fp32 [1], lse fp32 [n], dh, dw) as
    flce_fwd_bwd does; the logits of each shard are recomputed in its backward.
    ``shards`` may give explicit [a, b) bounds instead of ``num_shards``.
    """
    import torch
    _check_inputs(h, w, labels)
    n, d = h.shape
    v = w.shape[0]
    _debug_labels(labels, v, ignore_index)
    bounds = list(shards) if shards is not None else vocab_shard_bounds(v, num_shards)
    if bounds[0][0] != 0 or bounds[-1][1] != v or any(a >= b for a, b in bounds) or any(
            bounds[q][1] != bounds[q + 1][0] for q in range(len(bounds) - 1)):
        raise ValueError("shards must be contiguous, non-empty and cover [0, v)")
    _check_scalar(grad_out, h.device, "grad_out")
    q_n = len(bounds)
    dev = h.device
    stream = torch.cuda.current_stream(dev)
    dt, red = _dtype_code(h), _red_code(reduction)
    lse_parts = torch.empty(q_n, n, dtype=torch.float32, device=dev)
    zy_parts = torch.empty(q_n, n, dtype=torch.float32, device=dev)
    for q, (a, b) in enumerate(bounds):
        st = flce_fwd_shard(h, w[a:b], labels, n, d, b - a, a, dt, ignore_index, lse_parts[q], zy_parts[q], stream)
        if st != FLCE_OK:
            raise FlceError(st, "flce_fwd_shard")
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    st = flce_merge_shards(lse_parts, zy_parts, q_n, labels, n, ignore_index, red, loss, lse, stream)
    if st != FLCE_OK:
        raise FlceError(st, "flce_merge_shards")
    dh_sum = torch.empty(n, d, dtype=torch.float32, device=dev)
    dw = torch.empty_like(w)
    for q, (a, b) in enumerate(bounds):
        call = flce_bwd_shard if q == 0 else flce_bwd_shard_accumulate
        st = call(h, w[a:b], labels, lse, grad_out, n, d, b - a, a, dt, ignore_index, red, dh_sum, dw[a:b], stream)
        if st != FLCE_OK:
            raise FlceError(st, call.__name__)
    dh = torch.empty_like(h)
    st = flce_sum_parts(dh_sum, 1, n * d, dt, dh, stream)
    if st != FLCE_OK:
        raise FlceError(st, "flce_sum_parts")
    return loss, lse, dh, dw


def _check_fp8_inputs(h_q, h_scale, w_q, w_scale, labels):
    """(n, d, v) of e4m3 operands with per-row fp32 scales and int64 labels, all
    contiguous tensors on one device; raises before anything reaches the library."""
    import torch
    for t, name in ((h_q, "h_q"), (w_q, "w_q")):
        if not t.is_cuda or t.dim() != 2 or t.element_size() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D one-byte device tensor")
    for t, name in ((h_scale, "h_scale"), (w_scale, "w_scale")):
        if not t.is_cuda or t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 1-D device tensor")
    if not labels.is_cuda or labels.dtype != torch.int64 or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int64 device tensor")
    if len({t.device for t in (h_q, h_scale, w_q, w_scale, labels)}) != 1:
        raise ValueError("all inputs must be on one device")
    n, d = h_q.shape
    v = w_q.shape[0]
    if w_q.shape[1] != d or h_scale.shape[0] != n or w_scale.shape[0] != v or labels.shape != (n,):
        raise ValueError("shape mismatch")
    return n, d, v


def linear_cross_entropy_forward_fp8(h_q, h_scale, w_q, w_scale, labels, ignore_index: int = -100,
                                     reduction: str = "mean"):
    """Loss and LSE (flce_fwd_fp8) from e4m3 H [n, d] and W [v, d] (uint8 or float8_e4m3fn
    device tensors) with fp32 per-row scales [n] and [v]."""
    import torch
    n, d, v = _check_fp8_inputs(h_q, h_scale, w_q, w_scale, labels)
    _debug_labels(labels, v, ignore_index)
    loss = torch.empty(1, dtype=torch.float32, device=h_q.device)
    lse = torch.empty(n, dtype=torch.float32, device=h_q.device)
    st = flce_fwd_fp8(h_q, h_scale, w_q, w_scale, labels, n, d, v, ignore_index, _red_code(reduction), loss, lse,
                      torch.cuda.current_stream(h_q.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_fwd_fp8")
    return loss, lse


def linear_cross_entropy_backward_fp8(h_q, h_scale, w_q, w_scale, labels, lse, grad_out=None,
                                      ignore_index: int = -100, reduction: str = "mean"):
    """dH and dW (bf16) of ``grad_out * loss`` with respect to the dequantised H and W,
    from the LSE flce_fwd_fp8 returned (flce_bwd_fp8)."""
    import torch
    n, d, v = _check_fp8_inputs(h_q, h_scale, w_q, w_scale, labels)
    _debug_labels(labels, v, ignore_index)
    _check_vec(lse, n, h_q.device, "lse")
    _check_scalar(grad_out, h_q.device, "grad_out")
    dh = torch.empty(n, d, dtype=torch.bfloat16, device=h_q.device)
    dw = torch.empty(v, d, dtype=torch.bfloat16, device=h_q.device)
    st = flce_bwd_fp8(h_q, h_scale, w_q, w_scale, labels, lse, grad_out, n, d, v, ignore_index, _red_code(reduction), dh,
                      dw, torch.cuda.current_stream(h_q.device))
    if st != FLCE_OK:
        raise FlceError(st, "flce_bwd_fp8")
    return dh, dw


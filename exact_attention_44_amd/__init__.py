"""Python binding of the attention forward C ABI (include/attn.h).

Argument marshalling only: every step of the computation runs in the HIP
library libattn.so, built in-tree by exact_attention_44_amd.build. torch is
used for device memory and the current stream, nothing else. There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

from .build import LIB_PATH

__all__ = [
    "ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_HEAD_DIM", "ATTN_ERR_ALIGN",
    "ATTN_ERR_ALIAS", "ATTN_ERR_SCALE", "ATTN_ERR_LAUNCH", "ATTN_ERR_WORKSPACE", "AttnError",
    "ATTN_SPLIT_SCRATCH_BYTES", "load_library", "attn_fwd", "attn_fwd_validate", "attn_fwd_split",
    "attn_fwd_split_noalloc", "attn_fwd_split_workspace_bytes", "attn_bwd",
    "attn_bwd_workspace_bytes", "attn_status_str", "attn_last_hip_error", "attn_fwd_fp8",
    "attn_fwd_fp8_validate", "attn_fwd_unfused", "attn_fwd_unfused_workspace_bytes", "fwd",
    "fwd_split", "fwd_split_noalloc", "bwd", "fwd_fp8", "fwd_unfused", "LIB_PATH",
]

ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_HEAD_DIM = 3
ATTN_ERR_ALIGN = 4
ATTN_ERR_ALIAS = 5
ATTN_ERR_SCALE = 6
ATTN_ERR_LAUNCH = 7
ATTN_ERR_WORKSPACE = 8
# size of the fixed device array attn_fwd_split_noalloc uses (include/attn.h)
ATTN_SPLIT_SCRATCH_BYTES = 64 << 20

_lib: Optional[ctypes.CDLL] = None


class AttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = attn_status_str(status)
        if status == ATTN_ERR_LAUNCH:
            msg += f" (hipError_t {attn_last_hip_error()})"
        super().__init__(msg)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with "
            "`python -m exact_attention_44_amd.build` (hipcc, gfx950)")
    # torch bundles its own HIP runtime; load it first so the process holds a
    # single runtime (the library's libamdhip64 dependency then resolves to it)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                             ctypes.c_float, ctypes.c_int, vp, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_validate.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                      ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd_validate.restype = ctypes.c_int
    lib.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                   ctypes.c_float, ctypes.c_int, vp, i64, vp, i64, vp]
    lib.attn_fwd_split.restype = ctypes.c_int
    lib.attn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                           ctypes.c_float, ctypes.c_int, vp, i64, vp]
    lib.attn_fwd_split_noalloc.restype = ctypes.c_int
    lib.attn_fwd_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.attn_fwd_split_workspace_bytes.restype = i64
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                             ctypes.c_float, ctypes.c_int, vp, vp, i64, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace_bytes.restype = i64
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                 ctypes.c_float, ctypes.c_int, vp, vp]
    lib.attn_fwd_fp8.restype = ctypes.c_int
    lib.attn_fwd_fp8_validate.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                          i64, ctypes.c_float, ctypes.c_int, vp]
    lib.attn_fwd_fp8_validate.restype = ctypes.c_int
    lib.attn_fwd_unfused.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     ctypes.c_float, ctypes.c_int, vp, vp, i64, vp]
    lib.attn_fwd_unfused.restype = ctypes.c_int
    lib.attn_fwd_unfused_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_fwd_unfused_workspace_bytes.restype = i64
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def attn_fwd(q, k, v, out, lse, B: int, H: int, s_q: int, s_k: int, d: int, scale: float,
             causal: bool, key_padding_mask, stream) -> int:
    """The C entry point with the same arguments. Tensors may be passed as
    torch tensors or raw device addresses; stream as a hipStream_t handle (int)
    or None. Returns the attn_status code."""
    return load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   B, H, s_q, s_k, d, float(scale), 1 if causal else 0,
                                   _ptr(key_padding_mask), stream)


def attn_fwd_validate(q, k, v, out, lse, B: int, H: int, s_q: int, s_k: int, d: int,
                      scale: float, causal: bool, key_padding_mask) -> int:
    return load_library().attn_fwd_validate(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                            B, H, s_q, s_k, d, float(scale),
                                            1 if causal else 0, _ptr(key_padding_mask))


def attn_fwd_split(q, k, v, out, lse, B: int, H: int, s_q: int, s_k: int, d: int, scale: float,
                   causal: bool, key_padding_mask, n_splits: int, workspace, workspace_bytes: int,
                   stream) -> int:
    """The C entry point attn_fwd_split with the same arguments."""
    return load_library().attn_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                         B, H, s_q, s_k, d, float(scale), 1 if causal else 0,
                                         _ptr(key_padding_mask), n_splits, _ptr(workspace),
                                         workspace_bytes, stream)


def attn_fwd_split_noalloc(q, k, v, out, lse, B: int, H: int, s_q: int, s_k: int, d: int,
                           scale: float, causal: bool, key_padding_mask, n_splits: int,
                           stream) -> int:
    """The C entry point attn_fwd_split_noalloc with the same arguments."""
    return load_library().attn_fwd_split_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                 B, H, s_q, s_k, d, float(scale),
                                                 1 if causal else 0, _ptr(key_padding_mask),
                                                 n_splits, stream)


def attn_fwd_split_workspace_bytes(B: int, H: int, s_q: int, d: int, n_splits: int) -> int:
    return load_library().attn_fwd_split_workspace_bytes(B, H, s_q, d, n_splits)


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B: int, H: int, s_q: int, s_k: int, d: int,
             scale: float, causal: bool, key_padding_mask, workspace, workspace_bytes: int,
             stream) -> int:
    """The C entry point attn_bwd with the same arguments."""
    return load_library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, s_q, s_k, d, float(scale),
                                   1 if causal else 0, _ptr(key_padding_mask), _ptr(workspace),
                                   workspace_bytes, stream)


def attn_bwd_workspace_bytes(B: int, H: int, s_q: int) -> int:
    return load_library().attn_bwd_workspace_bytes(B, H, s_q)


def attn_fwd_fp8(q, k, v, descale_q, descale_k, descale_v, out, lse, B: int, H: int, s_q: int,
                 s_k: int, d: int, scale: float, causal: bool, key_padding_mask, stream) -> int:
    """The C entry point attn_fwd_fp8 with the same arguments."""
    return load_library().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(descale_q),
                                       _ptr(descale_k), _ptr(descale_v), _ptr(out), _ptr(lse),
                                       B, H, s_q, s_k, d, float(scale), 1 if causal else 0,
                                       _ptr(key_padding_mask), stream)


def attn_fwd_fp8_validate(q, k, v, descale_q, descale_k, descale_v, out, lse, B: int, H: int,
                          s_q: int, s_k: int, d: int, scale: float, causal: bool,
                          key_padding_mask) -> int:
    return load_library().attn_fwd_fp8_validate(_ptr(q), _ptr(k), _ptr(v), _ptr(descale_q),
                                                _ptr(descale_k), _ptr(descale_v), _ptr(out),
                                                _ptr(lse), B, H, s_q, s_k, d, float(scale),
                                                1 if causal else 0, _ptr(key_padding_mask))


def attn_fwd_unfused(q, k, v, out, lse, B: int, H: int, s_q: int, s_k: int, d: int, scale: float,
                     causal: bool, key_padding_mask, scores, scores_bytes: int, stream) -> int:
    """The C entry point attn_fwd_unfused with the same arguments."""
    return load_library().attn_fwd_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                           B, H, s_q, s_k, d, float(scale), 1 if causal else 0,
                                           _ptr(key_padding_mask), _ptr(scores), scores_bytes,
                                           stream)


def attn_fwd_unfused_workspace_bytes(B: int, H: int, s_q: int, s_k: int) -> int:
    return load_library().attn_fwd_unfused_workspace_bytes(B, H, s_q, s_k)


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(status).decode()


def attn_last_hip_error() -> int:
    return load_library().attn_last_hip_error()


def _check_inputs(q, k, v, key_padding_mask, dtypes=None):
    import torch

    dtypes = dtypes or (torch.bfloat16,)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype not in dtypes or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-D torch tensor of dtype {' or '.join(map(str, dtypes))}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, H, s_q, d = q.shape
    s_k = k.shape[2]
    if tuple(k.shape) != (B, H, s_k, d) or tuple(v.shape) != (B, H, s_k, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    if key_padding_mask is not None:
        m = key_padding_mask
        if m.dtype not in (torch.uint8, torch.bool) or tuple(m.shape) != (B, s_k):
            raise ValueError("key_padding_mask must be uint8/bool [B, s_k]")
        if not m.is_cuda or not m.is_contiguous() or m.device != q.device:
            raise ValueError("key_padding_mask must be a contiguous tensor on q's device")
    return B, H, s_q, s_k, d


def _check_given(t, name, shape, dtype, device):
    """A caller-supplied output or workspace tensor: the kernels write exactly
    `shape` elements of `dtype` from its first byte, so anything else is
    refused before the call."""
    import torch

    if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)}")
    if t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    return t


def _out_lse(out, lse, B, H, s_q, d, device):
    import torch

    if out is None:
        out = torch.empty((B, H, s_q, d), dtype=torch.bfloat16, device=device)
    else:
        _check_given(out, "out", (B, H, s_q, d), torch.bfloat16, device)
    if lse is None:
        lse = torch.empty((B, H, s_q), dtype=torch.float32, device=device)
    else:
        _check_given(lse, "lse", (B, H, s_q), torch.float32, device)
    return out, lse


def fwd(q, k, v, *, causal: bool = False, key_padding_mask=None, scale: Optional[float] = None,
        out=None, lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Attention forward on torch device tensors: q [B,H,s_q,d], k/v [B,H,s_k,d]
    bf16 contiguous; key_padding_mask None or uint8/bool [B,s_k] (nonzero =
    padded). Returns (out bf16 [B,H,s_q,d], lse float32 [B,H,s_q]). Runs on
    torch's current stream of q's device."""
    import torch

    B, H, s_q, s_k, d = _check_inputs(q, k, v, key_padding_mask)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(q.device):
        out, lse = _out_lse(out, lse, B, H, s_q, d, q.device)
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal, key_padding_mask, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def fwd_split(q, k, v, *, n_splits: int, causal: bool = False, key_padding_mask=None,
              scale: Optional[float] = None, out=None, lse=None,
              workspace=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """As fwd, computed over n_splits key chunks merged through their
    log-sum-exps (attn_fwd_split). `workspace` is an optional device tensor of
    at least attn_fwd_split_workspace_bytes(...) bytes, 256-byte aligned; when
    None, one is allocated with torch for this call."""
    import torch

    B, H, s_q, s_k, d = _check_inputs(q, k, v, key_padding_mask)
    if scale is None:
        scale = d ** -0.5
    chunks = max(1, min(int(n_splits), (s_k + 63) // 64))
    need = attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks)
    if need < 0:
        raise AttnError(ATTN_ERR_SHAPE)
    with torch.cuda.device(q.device):
        out, lse = _out_lse(out, lse, B, H, s_q, d, q.device)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_split(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                            key_padding_mask, int(n_splits), workspace, ws_bytes, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def fwd_split_noalloc(q, k, v, *, n_splits: int, causal: bool = False, key_padding_mask=None,
                      scale: Optional[float] = None, out=None,
                      lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """As fwd_split, with the partial results in the library's fixed device
    array instead of a workspace (attn_fwd_split_noalloc). With `out` and
    `lse` given, nothing is allocated; calls that overlap on one device race
    on the array."""
    import torch

    B, H, s_q, s_k, d = _check_inputs(q, k, v, key_padding_mask)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(q.device):
        out, lse = _out_lse(out, lse, B, H, s_q, d, q.device)
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_split_noalloc(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                                    key_padding_mask, int(n_splits), stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def bwd(q, k, v, out, dout, lse, *, causal: bool = False, key_padding_mask=None,
        scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of fwd's output for the output gradient `dout`
    (attn_bwd); `out` and `lse` are what fwd returned for q, k, v. All bf16
    tensors contiguous on one device; a workspace of
    attn_bwd_workspace_bytes(B, H, s_q) bytes is allocated with torch when
    not given."""
    import torch

    B, H, s_q, s_k, d = _check_inputs(q, k, v, key_padding_mask)
    for name, t in (("out", out), ("dout", dout)):
        _check_given(t, name, (B, H, s_q, d), torch.bfloat16, q.device)
    _check_given(lse, "lse", (B, H, s_q), torch.float32, q.device)
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(q.device):
        dq = torch.empty_like(q) if dq is None else _check_given(dq, "dq", q.shape, q.dtype, q.device)
        dk = torch.empty_like(k) if dk is None else _check_given(dk, "dk", k.shape, k.dtype, q.device)
        dv = torch.empty_like(v) if dv is None else _check_given(dv, "dv", v.shape, v.dtype, q.device)
        need = attn_bwd_workspace_bytes(B, H, s_q)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
        ws_bytes = workspace.numel() * workspace.element_size()
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, H, s_q, s_k, d, scale, causal,
                      key_padding_mask, workspace, ws_bytes, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return dq, dk, dv


def fwd_fp8(q, k, v, *, descale_q=None, descale_k=None, descale_v=None, causal: bool = False,
            key_padding_mask=None, scale: Optional[float] = None, out=None,
            lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Attention forward over OCP E4M3 inputs (attn_fwd_fp8): q [B,H,s_q,d],
    k/v [B,H,s_k,d] contiguous device tensors of dtype torch.float8_e4m3fn or
    uint8 (the codes); descale_* None or float32 [B, H] device tensors (the
    real value of a code is descale times its E4M3 value). Returns (out bf16
    [B,H,s_q,d], lse float32 [B,H,s_q]) on torch's current stream."""
    import torch

    B, H, s_q, s_k, d = _check_inputs(q, k, v, key_padding_mask,
                                      (torch.float8_e4m3fn, torch.uint8))
    for name, t in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        if t is None:
            continue
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != B * H
                or t.device != q.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 device tensor of {B * H} elements")
    if scale is None:
        scale = d ** -0.5
    with torch.cuda.device(q.device):
        out, lse = _out_lse(out, lse, B, H, s_q, d, q.device)
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_fp8(q, k, v, descale_q, descale_k, descale_v, out, lse, B, H, s_q, s_k, d,
                          scale, causal, key_padding_mask, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse


def fwd_unfused(q, k, v, *, causal: bool = False, key_padding_mask=None,
                scale: Optional[float] = None, out=None, lse=None, scores=None):
    """The materialising forward (attn_fwd_unfused) on torch device tensors, as
    fwd. `scores` is an optional bf16 [B, H, s_q, s_k] device tensor for the
    score matrix (allocated with torch when None); on return it holds the
    softmax weights. Returns (out, lse, scores)."""
    import torch

    B, H, s_q, s_k, d = _check_inputs(q, k, v, key_padding_mask)
    if scale is None:
        scale = d ** -0.5
    need = attn_fwd_unfused_workspace_bytes(B, H, s_q, s_k)
    if need < 0:
        raise AttnError(ATTN_ERR_SHAPE)
    with torch.cuda.device(q.device):
        out, lse = _out_lse(out, lse, B, H, s_q, d, q.device)
        if scores is None:
            scores = torch.empty((B, H, s_q, s_k), dtype=torch.bfloat16, device=q.device)
        else:
            _check_given(scores, "scores", (B, H, s_q, s_k), torch.bfloat16, q.device)
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_unfused(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                              key_padding_mask, scores if need > 0 else None, need, stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse, scores

"""MI355X-native fused attention: thin Python binding over the C ABI.

Every step of the computation runs in the HIP library ``libattn_fwd.so``
(built from ``csrc/attn_fwd.hip``, ``csrc/attn_bwd.hip`` and ``csrc/gemm.hip`` for gfx950).  This module only checks and
marshals arguments: PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing, calls raise.

    o, lse = attn_fwd(q, k, v, causal=False, scale=None)

computes o = softmax(scale * q k^T) v and lse = ln sum exp(scale * q k^T) per
row, for bf16 tensors of shape [B, H, N, d] (the flash-attention forward of the
ThunderKittens write-up, 88811315.cn, "H100 FlashAttention-2 forward example"), and

    dq, dk, dv, delta = attn_bwd(q, k, v, o, lse, dout, causal=False, scale=None)

its derivative for a loss whose gradient with respect to o is ``dout``
(``delta`` = rowsum(dout * o), the backward's per-row intermediate), and

    c = gemm(a, b, layout="nn")

the bf16 matrix product c = a b (``"nt"``: c = a b^T) on the matrix cores.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = ["attn_fwd", "attn_fwd_raw", "attn_fwd_ex", "attn_fwd_ex_raw", "attn_fwd_splitkv",
           "attn_fwd_splitkv_raw", "attn_fwd_splitkv_noalloc", "attn_fwd_splitkv_noalloc_raw",
           "splitkv_splits", "attn_bwd",
           "attn_bwd_raw", "attn_bwd_ex", "attn_bwd_ex_raw", "gemm", "gemm_raw", "GEMM_NN", "GEMM_NT", "attn_fwd_strerror",
           "load_library", "LIBRARY", "Status", "AttnError", "attention"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libattn_fwd.so")

_lock = threading.Lock()
_lib = None


class Status:
    """Status codes of include/attn_fwd.h."""
    OK = 0
    ERR_NULL = 1
    ERR_SHAPE = 2
    ERR_HEAD_DIM = 3
    ERR_SEQ_MULTIPLE = 4
    ERR_ALIGN = 5
    ERR_SCALE = 6
    ERR_HIP = 7
    ERR_DEVICE = 8
    ERR_WORKSPACE = 9


class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"attn_fwd failed ({status}): {message}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (``libattn_fwd.so`` next to this file by default)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise RuntimeError(
                    f"{LIBRARY} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
                    " or `python attention_attn_fwd_08_amd/_build.py`")
            _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp = ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_int, ctypes.c_float, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_strerror.argtypes = [ctypes.c_int]
    lib.attn_fwd_strerror.restype = ctypes.c_char_p
    lib.attn_fwd_abi_version.argtypes = []
    lib.attn_fwd_abi_version.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = [vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, vp]
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_fwd_splitkv.argtypes = ([vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int]
                                     + [vp] * 3)
    lib.attn_fwd_splitkv.restype = ctypes.c_int
    lib.attn_fwd_splitkv_noalloc.argtypes = ([vp] * 5 + [ctypes.c_int] * 6
                                             + [ctypes.c_float, ctypes.c_int, vp])
    lib.attn_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [vp] * 10 + [ctypes.c_int] * 5 + [ctypes.c_float, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_ex.argtypes = [vp] * 10 + [ctypes.c_int] * 6 + [ctypes.c_float, vp]
    lib.attn_bwd_ex.restype = ctypes.c_int
    lib.attn_gemm_bf16.argtypes = [vp] * 3 + [ctypes.c_int] * 4 + [vp]
    lib.attn_gemm_bf16.restype = ctypes.c_int
    return lib


def attn_fwd_strerror(status: int) -> str:
    return load_library().attn_fwd_strerror(int(status)).decode()


def attn_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                 B: int, H: int, N: int, d: int, causal: bool, scale: float,
                 stream: int = 0) -> int:
    """Call the C entry point with raw integer addresses; returns the status."""
    lib = load_library()
    return lib.attn_fwd(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None,
                        lse_ptr or None, int(B), int(H), int(N), int(d), int(bool(causal)),
                        float(scale), stream or None)


def attn_bwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int,
                 dq_ptr: int, dk_ptr: int, dv_ptr: int, delta_ptr: int,
                 B: int, H: int, N: int, d: int, causal: bool, scale: float,
                 stream: int = 0) -> int:
    """Call the backward C entry point with raw integer addresses; returns the status."""
    lib = load_library()
    ptrs = [p or None for p in (q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                dv_ptr, delta_ptr)]
    return lib.attn_bwd(*ptrs, int(B), int(H), int(N), int(d), int(bool(causal)), float(scale),
                        stream or None)


def _check_bf16(name, t, shape, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU device of q")
    if t.dim() != 4 or not t.is_contiguous() or (shape is not None and t.shape != shape):
        raise ValueError(f"{name} must be a contiguous tensor [B, H, N, d] shaped like q")


def _check_f32(name, t, shape, device):
    import torch
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device
            or tuple(t.shape) != shape or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 tensor {list(shape)} on q's device")


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, delta=None):
    """Attention backward on torch device tensors.

    ``q, k, v, o, dout``: bf16 [B, H, N, d]; ``lse``: float32 [B, H, N] from
    :func:`attn_fwd` with the same ``causal`` and ``scale``.  Returns
    ``(dq, dk, dv, delta)`` (bf16 x3, float32 [B, H, N]); any of them may be
    given to write into existing tensors.  Runs asynchronously on the current
    stream of ``q``'s device.
    """
    import torch

    _check_bf16("q", q, None, None)
    shape, dev = q.shape, q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_bf16(name, t, shape, dev)
    B, H, N, d = shape
    _check_f32("lse", lse, (B, H, N), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bf16(name, t, shape, dev)
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check_f32("delta", delta, (B, H, N), dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        status = attn_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), delta.data_ptr(), B, H, N, d, causal, scale, stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return dq, dk, dv, delta


def attn_bwd_ex_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int,
                    dq_ptr: int, dk_ptr: int, dv_ptr: int, delta_ptr: int,
                    B: int, H: int, Nq: int, Nk: int, d: int, causal: bool, scale: float,
                    stream: int = 0) -> int:
    """Call ``attn_bwd_ex`` with raw integer addresses; returns the status."""
    lib = load_library()
    ptrs = [p or None for p in (q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                dv_ptr, delta_ptr)]
    return lib.attn_bwd_ex(*ptrs, int(B), int(H), int(Nq), int(Nk), int(d), int(bool(causal)),
                           float(scale), stream or None)


def attn_bwd_ex(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                dq=None, dk=None, dv=None, delta=None):
    """Backward of :func:`attn_fwd_ex`: q, o, dout [B, H, Nq, d], k, v
    [B, H, Nk, d], lse [B, H, Nq]; bottom-right causal.  Returns
    ``(dq, dk, dv, delta)``."""
    import torch

    _check_bf16("q", q, None, None)
    B, H, Nq, d = q.shape
    dev = q.device
    _check_bf16("k", k, None, dev)
    if k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError("k must be [B, H, Nk, d] with q's B, H and d")
    _check_bf16("v", v, k.shape, dev)
    for name, t in (("o", o), ("dout", dout)):
        _check_bf16(name, t, q.shape, dev)
    Nk = k.shape[2]
    _check_f32("lse", lse, (B, H, Nq), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check_bf16("dq", dq, q.shape, dev)
    _check_bf16("dk", dk, k.shape, dev)
    _check_bf16("dv", dv, k.shape, dev)
    if delta is None:
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _check_f32("delta", delta, (B, H, Nq), dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        status = attn_bwd_ex_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                 dv.data_ptr(), delta.data_ptr(), B, H, Nq, Nk, d, causal, scale,
                                 stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return dq, dk, dv, delta


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Fused attention forward on torch bf16 device tensors [B, H, N, d].

    Returns ``(o, lse)``: ``o`` bf16 [B, H, N, d] and ``lse`` float32 [B, H, N].
    ``out`` / ``lse`` may be given to write into existing tensors.  Runs
    asynchronously on the current stream of ``q``'s device.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D tensor [B, H, N, d]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != torch.bfloat16 or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 tensor shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device
          or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N] on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        status = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, N, d, causal, scale, stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return out, lse


def attn_fwd_ex_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                    B: int, H: int, Nq: int, Nk: int, d: int, causal: bool, scale: float,
                    stream: int = 0) -> int:
    """Call attn_fwd_ex with raw integer addresses; returns the status."""
    lib = load_library()
    return lib.attn_fwd_ex(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None,
                           lse_ptr or None, int(B), int(H), int(Nq), int(Nk), int(d),
                           int(bool(causal)), float(scale), stream or None)


def attn_fwd_ex(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Attention forward for q [B, H, Nq, d] against k, v [B, H, Nk, d].

    Causal masks are aligned bottom-right (key j visible to query i iff
    j <= i + Nk - Nq); rows that see no key come back as o = 0, lse = -inf.
    Returns ``(o, lse)`` like :func:`attn_fwd`.
    """
    import torch

    _check_bf16("q", q, None, None)
    B, H, Nq, d = q.shape
    _check_bf16("k", k, None, q.device)
    if k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError("k must be [B, H, Nk, d] with q's B, H and d")
    _check_bf16("v", v, k.shape, q.device)
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (B, H, Nq), q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        status = attn_fwd_ex_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, H, Nq, Nk, d, causal, scale, stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return out, lse


def attn_fwd_splitkv_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                         B: int, H: int, Nq: int, Nk: int, d: int, causal: bool, scale: float,
                         n_splits: int, o_part_ptr: int, lse_part_ptr: int, stream: int = 0) -> int:
    """Call attn_fwd_splitkv with raw integer addresses; returns the status."""
    lib = load_library()
    return lib.attn_fwd_splitkv(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None,
                                lse_ptr or None, int(B), int(H), int(Nq), int(Nk), int(d),
                                int(bool(causal)), float(scale), int(n_splits),
                                o_part_ptr or None, lse_part_ptr or None, stream or None)


def splitkv_splits(B: int, H: int, Nq: int, Nk: int, d: int, cus: int = 256) -> int:
    """A split count that fills the GPU once: as many workgroups as fit at a
    time (one per compute unit at d = 128 and 256, two otherwise; measured
    best on one-query decoding from 1 x 32 to 16 x 32 heads), with at least
    256 keys per split (the library rounds splits to 64-key tiles)."""
    per_wg_queries = 256 if d == 128 else 128
    resident = 1 if d in (128, 256) else 2
    wgs = B * H * ((Nq + per_wg_queries - 1) // per_wg_queries)
    want = max(1, (resident * cus + max(wgs, 1) - 1) // max(wgs, 1))
    return int(max(1, min(want, Nk // 256 if Nk >= 256 else 1)))


def attn_fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None,
                     n_splits: int | None = None, out=None, lse=None, o_part=None, lse_part=None):
    """:func:`attn_fwd_ex` computed over ``n_splits`` key ranges and merged.

    ``o_part`` (float32 [n_splits, B, H, Nq, d]) and ``lse_part`` (float32
    [n_splits, B, H, Nq]) are the workspace; they are allocated here when not
    given.  ``n_splits=None`` picks :func:`splitkv_splits`.
    """
    import torch

    _check_bf16("q", q, None, None)
    B, H, Nq, d = q.shape
    _check_bf16("k", k, None, q.device)
    if k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError("k must be [B, H, Nk, d] with q's B, H and d")
    _check_bf16("v", v, k.shape, q.device)
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = splitkv_splits(B, H, Nq, Nk, d)
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (B, H, Nq), q.device)
    if o_part is None:
        o_part = torch.empty((n_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
    _check_f32("o_part", o_part, (n_splits, B, H, Nq, d), q.device)
    if lse_part is None:
        lse_part = torch.empty((n_splits, B, H, Nq), dtype=torch.float32, device=q.device)
    _check_f32("lse_part", lse_part, (n_splits, B, H, Nq), q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        status = attn_fwd_splitkv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), B, H, Nq, Nk, d, causal, scale, n_splits,
                                      o_part.data_ptr(), lse_part.data_ptr(), stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return out, lse


def attn_fwd_splitkv_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                                 B: int, H: int, Nq: int, Nk: int, d: int, causal: bool,
                                 scale: float, n_splits: int, stream: int = 0) -> int:
    """Call attn_fwd_splitkv_noalloc with raw integer addresses; returns the status."""
    lib = load_library()
    return lib.attn_fwd_splitkv_noalloc(q_ptr or None, k_ptr or None, v_ptr or None,
                                        o_ptr or None, lse_ptr or None, int(B), int(H), int(Nq),
                                        int(Nk), int(d), int(bool(causal)), float(scale),
                                        int(n_splits), stream or None)


def attn_fwd_splitkv_noalloc(q, k, v, causal: bool = False, scale: float | None = None,
                             n_splits: int | None = None, out=None, lse=None):
    """:func:`attn_fwd_splitkv` with its partial results in the library's fixed
    device workspace instead of caller tensors (the library allocates nothing;
    calls that overlap in time on one GPU race).  With ``out`` and ``lse``
    given, this call allocates nothing either."""
    import torch

    _check_bf16("q", q, None, None)
    B, H, Nq, d = q.shape
    _check_bf16("k", k, None, q.device)
    if k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError("k must be [B, H, Nk, d] with q's B, H and d")
    _check_bf16("v", v, k.shape, q.device)
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if n_splits is None:
        n_splits = splitkv_splits(B, H, Nq, Nk, d)
    out = torch.empty_like(q) if out is None else out
    _check_bf16("out", out, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_f32("lse", lse, (B, H, Nq), q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        status = attn_fwd_splitkv_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                                              causal, scale, n_splits, stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return out, lse


# Layout codes of include/attn_gemm.h.
GEMM_NN = 0  # b is [K, N]: c = a b
GEMM_NT = 1  # b is [N, K]: c = a b^T


def gemm_raw(a_ptr: int, b_ptr: int, c_ptr: int, M: int, N: int, K: int, layout: int,
             stream: int = 0) -> int:
    """Call ``attn_gemm_bf16`` with raw integer addresses; returns the status."""
    lib = load_library()
    return lib.attn_gemm_bf16(a_ptr or None, b_ptr or None, c_ptr or None, int(M), int(N), int(K),
                              int(layout), stream or None)


def gemm(a, b, layout: str = "nn", out=None):
    """c = a b (``layout="nn"``, b [K, N]) or c = a b^T (``"nt"``, b [N, K])
    for contiguous bf16 GPU matrices a [M, K]; returns c, bf16 [M, N]."""
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 torch.Tensor")
        if t.device.type != "cuda" or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D GPU tensor")
    if b.device != a.device:
        raise ValueError("a and b must be on the same device")
    if layout not in ("nn", "nt"):
        raise ValueError("layout must be 'nn' or 'nt'")
    M, K = a.shape
    if layout == "nn":
        if b.shape[0] != K:
            raise ValueError("b must be [K, N]")
        N = b.shape[1]
    else:
        if b.shape[1] != K:
            raise ValueError("b must be [N, K]")
        N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    elif (not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or out.device != a.device
          or tuple(out.shape) != (M, N) or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bfloat16 [M, N] tensor on a's device")
    with torch.cuda.device(a.device):
        stream = torch.cuda.current_stream(a.device).cuda_stream
        status = gemm_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                          GEMM_NN if layout == "nn" else GEMM_NT, stream)
    if status != Status.OK:
        raise AttnError(status, attn_fwd_strerror(status))
    return out


def _attention_function():
    """The autograd Function behind :func:`attention`, built on first use so
    that importing the package does not import torch."""
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            o, lse = attn_fwd_ex(q, k, v, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale = causal, scale
            return o

        @staticmethod
        def backward(ctx, dout):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv, _ = attn_bwd_ex(q, k, v, o, lse, dout.contiguous(), causal=ctx.causal,
                                        scale=ctx.scale)
            return dq, dk, dv, None, None

    return _Attention


_ATTENTION = None


def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """``softmax(scale * q k^T) v`` with autograd: q [B, H, Nq, d] and k, v
    [B, H, Nk, d] bf16 on the GPU (bottom-right causal mask when Nq != Nk).
    The forward runs :func:`attn_fwd_ex` and keeps its O and log-sum-exp; the
    backward runs :func:`attn_bwd_ex` on them.  Returns o, bf16 [B, H, Nq, d]."""
    global _ATTENTION
    if _ATTENTION is None:
        _ATTENTION = _attention_function()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _ATTENTION.apply(q, k, v, bool(causal), float(scale))

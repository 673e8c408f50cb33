"""Oracle for the fused attention forward: plain fp64 CPU evaluation.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It shares no code with the HIP library and never imports it.

The arithmetic lives in ``attn_oracle.c`` (forward), ``attn_bwd_oracle.c``
and ``attn_bwd_ex_oracle.c`` (backward: the derivative of the same definition,
full matrices per head, square and general shapes) and ``gemm_oracle.c`` (the
plain matrix product), all single-threaded C, fp64, with libm exp/log.  This module only compiles that file with gcc, loads it with ctypes and
hands it buffers.  ``threads > 1`` splits the list of query rows between host
threads, each running the same single-threaded C routine on its own rows (the
rows are independent, so the result does not depend on the split).

What is computed, per head (b, h) and query row i (ThunderKittens write-up,
88811315.cn, "RTX 4090 flash-attention example" / "H100 FlashAttention-2
forward example": the fixed point of the running-max recurrence):

    s_j = scale * q_i . k_j   for visible j  (all j, or j <= i when causal)
    o_i = sum_j softmax(s)_j v_j,   lse_i = ln sum_j exp(s_j)

Inputs are bf16 bit patterns in numpy ``uint16`` arrays of shape [B, H, N, d].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
SOURCES = (SOURCE, os.path.join(_HERE, "attn_bwd_oracle.c"), os.path.join(_HERE, "gemm_oracle.c"),
           os.path.join(_HERE, "attn_bwd_ex_oracle.c"))
GEMM_SOURCE = SOURCES[2]
BWD_EX_SOURCE = SOURCES[3]
LIBRARY = os.path.join(_HERE, "libattn_oracle.so")

_lock = threading.Lock()
_lib = None


def build(sources=SOURCES, output: str = LIBRARY) -> str:
    """Compile the oracle sources with gcc -O2 (no fast-math) into one shared
    library.  ``sources`` may be one path or a sequence of paths."""
    if isinstance(sources, str):
        sources = (sources,)
    out_dir = os.path.dirname(os.path.abspath(output))
    fd, tmp = tempfile.mkstemp(suffix=".so.tmp", dir=out_dir)
    os.close(fd)
    try:
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-fPIC", "-shared",
             "-o", tmp, *sources, "-lm"])
        os.replace(tmp, output)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return output


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, u16p, f64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_double)
    if hasattr(lib, "attn_oracle_rows"):
        lib.attn_oracle_rows.argtypes = [
            u16p, u16p, u16p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double,
            ctypes.POINTER(ctypes.c_int64), i64, f64p, f64p]
        lib.attn_oracle_rows.restype = ctypes.c_int
    if hasattr(lib, "attn_oracle_rows_ex"):
        lib.attn_oracle_rows_ex.argtypes = [
            u16p, u16p, u16p, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double,
            ctypes.POINTER(ctypes.c_int64), i64, f64p, f64p]
        lib.attn_oracle_rows_ex.restype = ctypes.c_int
    if hasattr(lib, "attn_bwd_oracle_heads"):
        lib.attn_bwd_oracle_heads.argtypes = [
            u16p, u16p, u16p, u16p, i64, i64, i64, ctypes.c_int, ctypes.c_double, i64, i64,
            f64p, f64p, f64p, f64p]
        lib.attn_bwd_oracle_heads.restype = ctypes.c_int
        lib.attn_fwd_oracle_head_f64.argtypes = [
            f64p, f64p, f64p, i64, i64, ctypes.c_int, ctypes.c_double, f64p, f64p, f64p]
        lib.attn_fwd_oracle_head_f64.restype = ctypes.c_int
        lib.attn_bwd_oracle_head_f64.argtypes = [
            f64p, f64p, f64p, f64p, i64, i64, ctypes.c_int, ctypes.c_double,
            f64p, f64p, f64p, f64p, f64p, f64p, f64p]
        lib.attn_bwd_oracle_head_f64.restype = ctypes.c_int
    if hasattr(lib, "attn_bwd_oracle_heads_ex"):
        lib.attn_bwd_oracle_heads_ex.argtypes = [
            u16p, u16p, u16p, u16p, i64, i64, i64, i64, ctypes.c_int, ctypes.c_double, i64, i64,
            f64p, f64p, f64p, f64p]
        lib.attn_bwd_oracle_heads_ex.restype = ctypes.c_int
        lib.attn_fwd_oracle_head_ex_f64.argtypes = [
            f64p, f64p, f64p, i64, i64, i64, ctypes.c_int, ctypes.c_double, f64p, f64p, f64p]
        lib.attn_fwd_oracle_head_ex_f64.restype = ctypes.c_int
        lib.attn_bwd_oracle_head_ex_f64.argtypes = [
            f64p, f64p, f64p, f64p, i64, i64, i64, ctypes.c_int, ctypes.c_double,
            f64p, f64p, f64p, f64p, f64p, f64p, f64p]
        lib.attn_bwd_oracle_head_ex_f64.restype = ctypes.c_int
    if hasattr(lib, "gemm_oracle_rows"):
        lib.gemm_oracle_rows.argtypes = [u16p, u16p, i64, i64, i64, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int64), i64, f64p]
        lib.gemm_oracle_rows.restype = ctypes.c_int
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load a compiled oracle.  With no path: the in-tree library, built here
    first if it is missing or older than its source."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            stale = (not os.path.exists(LIBRARY)
                     or any(os.path.getmtime(LIBRARY) < os.path.getmtime(s) for s in SOURCES))
            if stale:
                build()
            _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check_inputs(q, k, v):
    for name, a in (("q", q), ("k", k), ("v", v)):
        if not isinstance(a, np.ndarray) or a.dtype != np.uint16 or a.ndim != 4:
            raise TypeError(f"{name} must be a 4-D numpy uint16 array of bf16 bits")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape [B, H, N, d]")
    return (np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v))


def attention_rows(q, k, v, causal: bool, scale: float, rows, threads: int = 1,
                   lib: ctypes.CDLL | None = None):
    """Oracle output for the listed query rows.

    ``rows`` holds flat row indices r = (b*H + h)*N + i.  Returns
    ``(o, lse)`` with ``o`` float64 [len(rows), d] and ``lse`` float64 [len(rows)].
    """
    q, k, v = _check_inputs(q, k, v)
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    if rows.size and (rows.min() < 0 or rows.max() >= B * H * N):
        raise ValueError("row index out of range")
    lib = lib or load()
    o = np.zeros((rows.size, d), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    threads = max(1, min(int(threads), rows.size or 1))
    bounds = np.linspace(0, rows.size, threads + 1).astype(np.int64)

    def run(part):
        lo, hi = int(bounds[part]), int(bounds[part + 1])
        if hi <= lo:
            return 0
        sub_rows = rows[lo:hi]
        sub_o = o[lo:hi]
        sub_lse = lse[lo:hi]
        return lib.attn_oracle_rows(
            _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
            B, H, N, d, int(bool(causal)), float(scale),
            _ptr(sub_rows, ctypes.c_int64), hi - lo,
            _ptr(sub_o, ctypes.c_double), _ptr(sub_lse, ctypes.c_double))

    if threads == 1:
        statuses = [run(0)]
    else:
        with ThreadPoolExecutor(max_workers=threads) as pool:
            statuses = list(pool.map(run, range(threads)))
    if any(s != 0 for s in statuses):
        raise RuntimeError(f"oracle failed with status {statuses}")
    return o, lse


def attention(q, k, v, causal: bool, scale: float, threads: int = 1,
              lib: ctypes.CDLL | None = None):
    """Oracle output for every row: ``o`` float64 [B,H,N,d], ``lse`` float64 [B,H,N]."""
    q, k, v = _check_inputs(q, k, v)
    B, H, N, d = q.shape
    o, lse = attention_rows(q, k, v, causal, scale, np.arange(B * H * N), threads, lib)
    return o.reshape(B, H, N, d), lse.reshape(B, H, N)


# ---------------------------------------------------------------------------
# Backward pass (the derivative of the forward definition; attn_bwd_oracle.c)
# ---------------------------------------------------------------------------

def attention_bwd(q, k, v, dout, causal: bool, scale: float, threads: int = 1,
                  lib: ctypes.CDLL | None = None):
    """Gradients of sum(O * dout) for bf16-bit inputs [B, H, N, d].

    Returns ``(dq, dk, dv, delta)``: float64 [B,H,N,d] x 3 and [B,H,N], where
    ``delta`` is the row sum of dout * O (O the exact forward output).
    ``threads > 1`` splits the heads between host threads.
    """
    q, k, v = _check_inputs(q, k, v)
    dout = np.ascontiguousarray(dout)
    if dout.dtype != np.uint16 or dout.shape != q.shape:
        raise TypeError("dout must be a uint16 array of bf16 bits shaped like q")
    B, H, N, d = q.shape
    BH = B * H
    lib = lib or load()
    dq = np.zeros((B, H, N, d)); dk = np.zeros_like(dq); dv = np.zeros_like(dq)
    delta = np.zeros((B, H, N))
    threads = max(1, min(int(threads), BH))
    bounds = np.linspace(0, BH, threads + 1).astype(np.int64)

    def run(part):
        lo, hi = int(bounds[part]), int(bounds[part + 1])
        if hi <= lo:
            return 0
        return lib.attn_bwd_oracle_heads(
            _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
            _ptr(dout, ctypes.c_uint16), BH, N, d, int(bool(causal)), float(scale), lo, hi,
            _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double),
            _ptr(delta, ctypes.c_double))

    if threads == 1:
        statuses = [run(0)]
    else:
        with ThreadPoolExecutor(max_workers=threads) as pool:
            statuses = list(pool.map(run, range(threads)))
    if any(s != 0 for s in statuses):
        raise RuntimeError(f"oracle failed with status {statuses}")
    return dq, dk, dv, delta


def forward_head_f64(q, k, v, causal: bool, scale: float, lib: ctypes.CDLL | None = None):
    """Forward of one head on float64 inputs [N, d]: returns (o, lse, p)."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    N, d = q.shape
    lib = lib or load()
    o = np.zeros((N, d)); lse = np.zeros(N); p = np.zeros((N, N))
    st = lib.attn_fwd_oracle_head_f64(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                      _ptr(v, ctypes.c_double), N, d, int(bool(causal)),
                                      float(scale), _ptr(o, ctypes.c_double),
                                      _ptr(lse, ctypes.c_double), _ptr(p, ctypes.c_double))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return o, lse, p


def backward_head_f64(q, k, v, dout, causal: bool, scale: float,
                      lib: ctypes.CDLL | None = None):
    """Backward of one head on float64 inputs [N, d]: (dq, dk, dv, delta, o, lse)."""
    q, k, v, dout = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, dout))
    N, d = q.shape
    lib = lib or load()
    dq = np.zeros((N, d)); dk = np.zeros((N, d)); dv = np.zeros((N, d))
    delta = np.zeros(N); o = np.zeros((N, d)); lse = np.zeros(N)
    scratch = np.zeros(2 * N * N)
    f = lambda a: _ptr(a, ctypes.c_double)  # noqa: E731
    st = lib.attn_bwd_oracle_head_f64(f(q), f(k), f(v), f(dout), N, d, int(bool(causal)),
                                      float(scale), f(dq), f(dk), f(dv), f(delta), f(o), f(lse),
                                      f(scratch))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return dq, dk, dv, delta, o, lse


# ---------------------------------------------------------------------------
# General shapes: Nq queries, Nk keys, bottom-right causal (attn_oracle.c)
# ---------------------------------------------------------------------------

def attention_ex(q, k, v, causal: bool, scale: float, threads: int = 1,
                 lib: ctypes.CDLL | None = None):
    """Oracle output for q [B,H,Nq,d] against k, v [B,H,Nk,d] (bf16 bits).

    Causal masks are bottom-right aligned: key j is visible to query i iff
    j <= i + Nk - Nq.  Rows that see no key give o = 0, lse = -inf.
    Returns ``o`` float64 [B,H,Nq,d] and ``lse`` float64 [B,H,Nq].
    """
    B, H, Nq, d = np.shape(q)
    o, lse = attention_ex_rows(q, k, v, causal, scale, np.arange(B * H * Nq, dtype=np.int64),
                               threads=threads, lib=lib)
    return o.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)


def attention_ex_rows(q, k, v, causal: bool, scale: float, rows, threads: int = 1,
                      lib: ctypes.CDLL | None = None):
    """:func:`attention_ex` for the listed query rows only.

    ``rows`` holds flat row indices r = (b*H + h)*Nq + i.  Returns ``(o, lse)``
    with ``o`` float64 [len(rows), d] and ``lse`` float64 [len(rows)].
    """
    for name, a in (("q", q), ("k", k), ("v", v)):
        if not isinstance(a, np.ndarray) or a.dtype != np.uint16 or a.ndim != 4:
            raise TypeError(f"{name} must be a 4-D numpy uint16 array of bf16 bits")
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    B, H, Nq, d = q.shape
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError("k and v must be [B, H, Nk, d] matching q's B, H and d")
    Nk = k.shape[2]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    if rows.size and (rows.min() < 0 or rows.max() >= B * H * Nq):
        raise ValueError("row index out of range")
    lib = lib or load()
    o = np.zeros((rows.size, d)); lse = np.zeros(rows.size)
    threads = max(1, min(int(threads), rows.size or 1))
    bounds = np.linspace(0, rows.size, threads + 1).astype(np.int64)

    def run(part):
        lo, hi = int(bounds[part]), int(bounds[part + 1])
        if hi <= lo:
            return 0
        sub = rows[lo:hi]
        return lib.attn_oracle_rows_ex(
            _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
            B, H, Nq, Nk, d, int(bool(causal)), float(scale), _ptr(sub, ctypes.c_int64), hi - lo,
            _ptr(o[lo:hi], ctypes.c_double), _ptr(lse[lo:hi], ctypes.c_double))

    if threads == 1:
        statuses = [run(0)]
    else:
        with ThreadPoolExecutor(max_workers=threads) as pool:
            statuses = list(pool.map(run, range(threads)))
    if any(s != 0 for s in statuses):
        raise RuntimeError(f"oracle failed with status {statuses}")
    return o, lse


def attention_bwd_ex(q, k, v, dout, causal: bool, scale: float, threads: int = 1,
                     lib: ctypes.CDLL | None = None):
    """Gradients of sum(O * dout) for q, dout [B,H,Nq,d] against k, v
    [B,H,Nk,d] (bf16 bits), bottom-right causal.  Returns (dq, dk, dv, delta)
    in fp64; rows that see no key have dq = 0 and delta = 0."""
    for name, a in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        if not isinstance(a, np.ndarray) or a.dtype != np.uint16 or a.ndim != 4:
            raise TypeError(f"{name} must be a 4-D numpy uint16 array of bf16 bits")
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    B, H, Nq, d = q.shape
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d or dout.shape != q.shape:
        raise ValueError("k, v must be [B, H, Nk, d] and dout shaped like q")
    Nk = k.shape[2]
    BH = B * H
    lib = lib or load()
    dq = np.zeros((B, H, Nq, d)); dk = np.zeros((B, H, Nk, d)); dv = np.zeros((B, H, Nk, d))
    delta = np.zeros((B, H, Nq))
    threads = max(1, min(int(threads), BH))
    bounds = np.linspace(0, BH, threads + 1).astype(np.int64)

    def run(part):
        lo, hi = int(bounds[part]), int(bounds[part + 1])
        if hi <= lo:
            return 0
        return lib.attn_bwd_oracle_heads_ex(
            _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
            _ptr(dout, ctypes.c_uint16), BH, Nq, Nk, d, int(bool(causal)), float(scale), lo, hi,
            _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double),
            _ptr(delta, ctypes.c_double))

    if threads == 1:
        statuses = [run(0)]
    else:
        with ThreadPoolExecutor(max_workers=threads) as pool:
            statuses = list(pool.map(run, range(threads)))
    if any(s != 0 for s in statuses):
        raise RuntimeError(f"oracle failed with status {statuses}")
    return dq, dk, dv, delta


def forward_head_ex_f64(q, k, v, causal: bool, scale: float, lib: ctypes.CDLL | None = None):
    """General-shape forward of one head on float64 q [Nq, d], k, v [Nk, d]."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v))
    Nq, d = q.shape
    Nk = k.shape[0]
    lib = lib or load()
    o = np.zeros((Nq, d)); lse = np.zeros(Nq); p = np.zeros((Nq, max(Nk, 1)))
    st = lib.attn_fwd_oracle_head_ex_f64(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                         _ptr(v, ctypes.c_double), Nq, Nk, d, int(bool(causal)),
                                         float(scale), _ptr(o, ctypes.c_double),
                                         _ptr(lse, ctypes.c_double), _ptr(p, ctypes.c_double))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return o, lse, p[:, :Nk]


def backward_head_ex_f64(q, k, v, dout, causal: bool, scale: float,
                         lib: ctypes.CDLL | None = None):
    """General-shape backward of one head on float64 inputs: (dq, dk, dv, delta, o, lse)."""
    q, k, v, dout = (np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, dout))
    Nq, d = q.shape
    Nk = k.shape[0]
    lib = lib or load()
    dq = np.zeros((Nq, d)); dk = np.zeros((Nk, d)); dv = np.zeros((Nk, d))
    delta = np.zeros(Nq); o = np.zeros((Nq, d)); lse = np.zeros(Nq)
    scratch = np.zeros(2 * Nq * Nk + 1)
    f = lambda a: _ptr(a, ctypes.c_double)  # noqa: E731
    st = lib.attn_bwd_oracle_head_ex_f64(f(q), f(k), f(v), f(dout), Nq, Nk, d, int(bool(causal)),
                                         float(scale), f(dq), f(dk), f(dv), f(delta), f(o), f(lse),
                                         f(scratch))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return dq, dk, dv, delta, o, lse


# ---------------------------------------------------------------------------
# Matrix product (gemm_oracle.c)
# ---------------------------------------------------------------------------

def gemm(a, b, b_layout: str = "nn", rows=None, threads: int = 1, lib: ctypes.CDLL | None = None):
    """C = A B (``b_layout="nn"``, b is [K, N]) or C = A B^T (``"nt"``, b is
    [N, K]) for bf16-bit a [M, K], in fp64.  ``rows``: the rows of C to
    compute (default all); returns float64 [len(rows), N].  ``threads > 1``
    splits the rows between host threads."""
    for name, x in (("a", a), ("b", b)):
        if not isinstance(x, np.ndarray) or x.dtype != np.uint16 or x.ndim != 2:
            raise TypeError(f"{name} must be a 2-D numpy uint16 array of bf16 bits")
    if b_layout not in ("nn", "nt"):
        raise ValueError("b_layout must be 'nn' or 'nt'")
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    M, K = a.shape
    if b_layout == "nn":
        if b.shape[0] != K:
            raise ValueError("b must be [K, N]")
        N = b.shape[1]
    else:
        if b.shape[1] != K:
            raise ValueError("b must be [N, K]")
        N = b.shape[0]
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    rows = np.ascontiguousarray(rows)
    lib = lib or load()
    c = np.zeros((rows.size, N))
    threads = max(1, min(int(threads), rows.size or 1))
    bounds = np.linspace(0, rows.size, threads + 1).astype(np.int64)
    lay = 0 if b_layout == "nn" else 1

    def run(part):
        lo, hi = int(bounds[part]), int(bounds[part + 1])
        if hi <= lo:
            return 0
        return lib.gemm_oracle_rows(_ptr(a, ctypes.c_uint16), _ptr(b, ctypes.c_uint16), M, N, K, lay,
                                    _ptr(rows[lo:hi], ctypes.c_int64), hi - lo,
                                    _ptr(c[lo:hi], ctypes.c_double))

    if threads == 1:
        statuses = [run(0)]
    else:
        with ThreadPoolExecutor(max_workers=threads) as pool:
            statuses = list(pool.map(run, range(threads)))
    if any(s != 0 for s in statuses):
        raise RuntimeError(f"oracle failed with status {statuses}")
    return c

"""Seeded synthetic inputs for the attention forward.

This module holds no attention arithmetic.  It draws Gaussian samples with
numpy's PCG64 generator, rounds them to bf16 on their bit patterns, and names
the workloads.  Both the HIP path (through its tests and benchmark) and the
oracle receive the very same bf16 bytes from here.

Recipe: ``rng = numpy.random.default_rng(seed)``; Q, then K, then V (then, for
the backward, dO) are drawn, each as
``rng.standard_normal(B*H*N*d, dtype=float32) * sigma`` and rounded to bf16
with round-to-nearest-even.  Layout [B, H, N, d], contiguous row-major.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest, ties to even).

    Works on the raw bits: add 0x7FFF plus the lowest kept bit, then drop the
    low 16 bits.  NaNs stay quiet NaNs; infinities stay infinities.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, mask, scale and input recipe."""
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    qk_sigma: float = 1.0
    v_sigma: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d, halved when causal (the usual attention-forward count)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O written once (bf16), LSE (fp32)."""
        return 4 * self.B * self.H * self.N * self.d * 2 + self.B * self.H * self.N * 4


# The five problems this library is measured and checked on.
WORKLOADS = {
    w.name: w for w in (
        Workload("B1-H1-N256-d64", 1, 1, 256, 64, False, seed=1),
        Workload("B16-H16-N1024-d64", 16, 16, 1024, 64, False, seed=2),
        Workload("B16-H16-N4096-d128", 16, 16, 4096, 128, False, seed=3),
        Workload("B4-H32-N8192-d128-causal", 4, 32, 8192, 128, True, seed=4),
        Workload("B2-H16-N16384-d64-causal-sharp", 2, 16, 16384, 64, True, seed=5,
                 qk_sigma=2.0),
    )
}

# The problem whose throughput is the headline number.
HEADLINE = "B16-H16-N4096-d128"


def make_qkv(B: int, H: int, N: int, d: int, seed: int,
             qk_sigma: float = 1.0, v_sigma: float = 1.0):
    """Seeded bf16 Q, K, V as uint16 bit arrays of shape [B, H, N, d]."""
    rng = np.random.default_rng(seed)
    n = B * H * N * d
    out = []
    for sigma in (qk_sigma, qk_sigma, v_sigma):
        x = rng.standard_normal(n, dtype=np.float32)
        if sigma != 1.0:
            x = x * np.float32(sigma)
        out.append(f32_to_bf16_bits(x).reshape(B, H, N, d))
    return tuple(out)


def make_qkv_dout(B: int, H: int, N: int, d: int, seed: int,
                  qk_sigma: float = 1.0, v_sigma: float = 1.0, dout_sigma: float = 1.0):
    """Seeded bf16 Q, K, V (the same arrays as ``make_qkv``) and then dO, the
    next draw of the same generator: four uint16 bit arrays [B, H, N, d]."""
    rng = np.random.default_rng(seed)
    n = B * H * N * d
    out = []
    for sigma in (qk_sigma, qk_sigma, v_sigma, dout_sigma):
        x = rng.standard_normal(n, dtype=np.float32)
        if sigma != 1.0:
            x = x * np.float32(sigma)
        out.append(f32_to_bf16_bits(x).reshape(B, H, N, d))
    return tuple(out)


def make_stepped_qkv(B: int, H: int, Nq: int, Nk: int, d: int, seed: int,
                     q_shift: float, k_step: float, span: int, levels: int):
    """Seeded bf16 Q [B,H,Nq,d], K and V [B,H,Nk,d] whose scores rise in steps
    along the keys: every element of Q is offset by ``q_shift``, and every
    element of key row j by ``k_step * min(j // span, levels - 1)`` (key
    "level"), on top of standard normal samples (Q, then K, then V from one
    PCG64 generator, rounded to bf16 like :func:`make_qkv`).  A query's score
    against a key then grows by about ``q_shift * k_step * d`` per level, so
    keys of a higher level dominate every key below it by a wide margin."""
    rng = np.random.default_rng(seed)
    zq = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    zk = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    zv = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    level = np.minimum(np.arange(Nk) // span, levels - 1).astype(np.float32)
    q = zq + np.float32(q_shift)
    k = zk + (np.float32(k_step) * level)[None, None, :, None]
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(zv)


def workload_inputs(w: Workload):
    """Seeded bf16 Q, K, V for a named workload."""
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.qk_sigma, w.v_sigma)


def sha256(a: np.ndarray) -> str:
    """SHA-256 of an array's bytes (pins the generated inputs)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def sample_rows(w: Workload, per_head: int = 16, block: int = 128, seed: int = 0):
    """Flat row indices (b*H + h)*N + i to check at full size.

    Every head contributes the fixed rows 0, 1, block-1, block, N/2, N-1, the
    last row before and the first row of each of two other query blocks, the
    same edges of 256-row blocks (255, 256, 511, 512), and seeded random rows
    up to ``per_head``.
    """
    rng = np.random.default_rng(1000 + seed)
    N = w.N
    fixed = {0, 1, block - 1, block, N // 2, N - 1, min(N - 1, 2 * block - 1),
             min(N - 1, 3 * block), 255, 256, 511, 512}
    fixed = sorted(r for r in fixed if 0 <= r < N)
    rows = []
    for bh in range(w.B * w.H):
        extra = rng.choice(N, size=max(0, per_head - len(fixed)), replace=False)
        for i in sorted(set(fixed) | set(int(e) for e in extra)):
            rows.append(bh * N + i)
    return np.asarray(rows, dtype=np.int64)

"""Pins for the oracle: facts fixed by mathematics, not by the oracle itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load()`` or a
deliberately broken build of it) and raises ``AssertionError`` when the
library disagrees with the fact it checks.  ``tests/test_oracle_pins.py`` runs
them against the real oracle; ``tests/test_oracle_mutants.py`` runs them
against mutated copies of the oracle source and demands that each mutation
trips at least one pin.

What pins what (the computation is softmax(scale * Q K^T) V with the row
log-sum-exp, per the ThunderKittens write-up's flash-attention examples):
  * brute force in 50-digit decimal arithmetic on tiny inputs, with no max
    subtraction and the whole score matrix formed;
  * a library routine: scipy.special.softmax / logsumexp over scores formed
    by a numpy fp64 matmul;
  * closed forms: V = 1, Q = 0, N = 1, causal row 0, two keys, one dominant key;
  * invariants: key/value row permutation, key shift, linearity in V, causal
    prefix, causal last row, power-of-two scale transfer, per-head independence.
"""
from __future__ import annotations

import decimal
import math

import numpy as np
import scipy.special

import oracle
from attention_attn_fwd_08_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def bf(x) -> np.ndarray:
    """float values -> bf16 bits (values chosen by the pins are bf16-exact)."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def fl(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def rand_bf16(rng, shape, sigma=1.0):
    return bf(rng.standard_normal(shape).astype(np.float32) * np.float32(sigma))


def small_ints(rng, shape, lo=-3, hi=4):
    return bf(rng.integers(lo, hi, size=shape).astype(np.float32))


def run(lib, q, k, v, causal, scale):
    return oracle.attention(q, k, v, causal, scale, threads=1, lib=lib)


def close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    ok = np.isfinite(a).all() and np.allclose(a, b, rtol=rtol, atol=atol)
    if not ok:
        diff = np.abs(a - b)
        err = float(np.max(np.where(np.isnan(diff), np.inf, diff))) if a.size else 0.0
        raise AssertionError(f"{what}: max |diff| = {err}")


# --------------------------------------------------------------------------
# Brute force in high-precision decimal arithmetic.
# --------------------------------------------------------------------------
def decimal_attention_head(qf, kf, vf, causal, scale, prec=50):
    """softmax(scale Q K^T) V and ln(sum exp) for one head, in `prec`-digit
    decimal arithmetic: every score formed, exponentiated without any max
    subtraction, summed and divided.  Inputs are exact binary floats."""
    ctx = decimal.Context(prec=prec)
    D = decimal.Decimal
    N, d = qf.shape
    sc = D(float(scale))
    o = np.zeros((N, d))
    lse = np.zeros(N)
    kd = [[D(float(x)) for x in row] for row in kf]
    vd = [[D(float(x)) for x in row] for row in vf]
    for i in range(N):
        qi = [D(float(x)) for x in qf[i]]
        vis = range(i + 1) if causal else range(N)
        e = []
        for j in vis:
            dot = sum((ctx.multiply(a, b) for a, b in zip(qi, kd[j])), D(0))
            e.append(ctx.exp(ctx.multiply(sc, dot)))
        z = sum(e, D(0))
        for t in range(d):
            num = sum((ctx.multiply(ej, vd[j][t]) for ej, j in zip(e, vis)), D(0))
            o[i, t] = float(ctx.divide(num, z))
        lse[i] = float(ctx.ln(z))
    return o, lse


def pin_bruteforce_decimal(lib):
    rng = np.random.default_rng(11)
    for N in (1, 2, 3, 5, 8):
        for d in (1, 2, 4, 8):
            for causal in (False, True):
                B, H = 1, 2
                q = rand_bf16(rng, (B, H, N, d))
                k = rand_bf16(rng, (B, H, N, d))
                v = rand_bf16(rng, (B, H, N, d))
                scale = 1.0 / math.sqrt(d) * 1.5
                o, lse = run(lib, q, k, v, causal, scale)
                for h in range(H):
                    eo, el = decimal_attention_head(fl(q[0, h]), fl(k[0, h]), fl(v[0, h]),
                                                    causal, scale)
                    close(o[0, h], eo, 1e-12, 1e-13, f"O N={N} d={d} causal={causal}")
                    close(lse[0, h], el, 1e-12, 1e-13, f"LSE N={N} d={d} causal={causal}")


# --------------------------------------------------------------------------
# A library routine: scipy's softmax and logsumexp over numpy fp64 scores.
# --------------------------------------------------------------------------
def pin_scipy_softmax(lib):
    rng = np.random.default_rng(12)
    B, H, N, d = 2, 3, 48, 16
    for causal in (False, True):
        q = rand_bf16(rng, (B, H, N, d))
        k = rand_bf16(rng, (B, H, N, d), sigma=2.0)
        v = rand_bf16(rng, (B, H, N, d))
        scale = 0.25
        o, lse = run(lib, q, k, v, causal, scale)
        s = scale * np.matmul(fl(q), np.swapaxes(fl(k), -1, -2))
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        eo = np.matmul(scipy.special.softmax(s, axis=-1), fl(v))
        el = scipy.special.logsumexp(s, axis=-1)
        close(o, eo, 1e-11, 1e-12, f"O vs scipy causal={causal}")
        close(lse, el, 1e-11, 1e-12, f"LSE vs scipy causal={causal}")


# --------------------------------------------------------------------------
# Closed forms.
# --------------------------------------------------------------------------
def pin_values_all_one(lib):
    """V = 1 everywhere: softmax rows sum to one, so O = 1 everywhere."""
    rng = np.random.default_rng(13)
    B, H, N, d = 2, 2, 40, 8
    q = rand_bf16(rng, (B, H, N, d))
    k = rand_bf16(rng, (B, H, N, d))
    v = bf(np.ones((B, H, N, d)))
    for causal in (False, True):
        o, _ = run(lib, q, k, v, causal, 0.35)
        close(o, np.ones_like(o), 0.0, 1e-14, f"V=1 causal={causal}")


def pin_query_zero(lib):
    """Q = 0: every score is 0, so O_i is the mean of the visible values and
    LSE_i = ln(number of visible keys)."""
    rng = np.random.default_rng(14)
    B, H, N, d = 1, 3, 33, 4
    q = bf(np.zeros((B, H, N, d)))
    k = rand_bf16(rng, (B, H, N, d))
    v = rand_bf16(rng, (B, H, N, d))
    vf = fl(v)
    o, lse = run(lib, q, k, v, False, 0.5)
    close(o, np.broadcast_to(vf.mean(axis=2, keepdims=True), o.shape), 1e-13, 1e-14,
          "Q=0 non-causal O")
    close(lse, np.full(lse.shape, math.log(N)), 1e-14, 1e-14, "Q=0 non-causal LSE")
    o, lse = run(lib, q, k, v, True, 0.5)
    counts = np.arange(1, N + 1, dtype=np.float64)
    prefix_mean = np.cumsum(vf, axis=2) / counts[None, None, :, None]
    close(o, prefix_mean, 1e-13, 1e-14, "Q=0 causal O")
    close(lse, np.broadcast_to(np.log(counts), lse.shape), 1e-14, 1e-14, "Q=0 causal LSE")


def pin_single_key(lib):
    """N = 1, and causal row 0: the only visible key gets weight 1, so O = v_0
    exactly and LSE = scale * q_0 . k_0."""
    rng = np.random.default_rng(15)
    q = rand_bf16(rng, (2, 2, 1, 8))
    k = rand_bf16(rng, (2, 2, 1, 8))
    v = rand_bf16(rng, (2, 2, 1, 8))
    o, lse = run(lib, q, k, v, False, 0.3)
    if not np.array_equal(o, fl(v)):
        raise AssertionError("N=1: O != v_0")
    close(lse, 0.3 * np.sum(fl(q) * fl(k), axis=-1), 1e-14, 1e-15, "N=1 LSE")
    q = rand_bf16(rng, (1, 2, 9, 8))
    k = rand_bf16(rng, (1, 2, 9, 8))
    v = rand_bf16(rng, (1, 2, 9, 8))
    o, lse = run(lib, q, k, v, True, 0.3)
    if not np.array_equal(o[:, :, 0], fl(v)[:, :, 0]):
        raise AssertionError("causal row 0: O != v_0")
    close(lse[:, :, 0], 0.3 * np.sum(fl(q)[:, :, 0] * fl(k)[:, :, 0], axis=-1), 1e-14, 1e-15,
          "causal row 0 LSE")


def pin_two_keys(lib):
    """N = 2: O = sigma(s0 - s1) v0 + sigma(s1 - s0) v1, LSE = s0 + ln(1 + e^(s1 - s0))."""
    rng = np.random.default_rng(16)
    for _ in range(5):
        q = rand_bf16(rng, (1, 1, 2, 4))
        k = rand_bf16(rng, (1, 1, 2, 4))
        v = rand_bf16(rng, (1, 1, 2, 4))
        o, lse = run(lib, q, k, v, False, 0.7)
        qf, kf, vf = fl(q)[0, 0], fl(k)[0, 0], fl(v)[0, 0]
        for i in range(2):
            s0 = 0.7 * float(qf[i] @ kf[0])
            s1 = 0.7 * float(qf[i] @ kf[1])
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            close(o[0, 0, i], w0 * vf[0] + w1 * vf[1], 1e-13, 1e-14, "two keys O")
            close(lse[0, 0, i], s0 + math.log1p(math.exp(s1 - s0)), 1e-13, 1e-14,
                  "two keys LSE")


def pin_dominant_key(lib):
    """One key whose scaled score beats every other by > 60: O equals its value
    row to fp64 precision (e^-60 < 1e-26), LSE equals its score."""
    rng = np.random.default_rng(17)
    B, H, N, d = 1, 1, 16, 8
    q = bf(np.ones((B, H, N, d)))
    kf = rng.integers(-1, 2, size=(B, H, N, d)).astype(np.float32)
    star = 11
    kf[0, 0, star] = 16.0   # score gap >= 8 * 17 * scale
    k = bf(kf)
    v = rand_bf16(rng, (B, H, N, d))
    scale = 1.0
    o, lse = run(lib, q, k, v, False, scale)
    close(o[0, 0], np.broadcast_to(fl(v)[0, 0, star], (N, d)), 1e-20, 1e-24, "dominant key O")
    close(lse[0, 0], np.full(N, 16.0 * d * scale), 1e-15, 1e-13, "dominant key LSE")


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------
def pin_permutation(lib):
    """Non-causal: permuting the rows of K and V together changes nothing."""
    rng = np.random.default_rng(18)
    B, H, N, d = 2, 2, 37, 8
    q = rand_bf16(rng, (B, H, N, d))
    k = rand_bf16(rng, (B, H, N, d))
    v = rand_bf16(rng, (B, H, N, d))
    perm = rng.permutation(N)
    o1, l1 = run(lib, q, k, v, False, 0.4)
    o2, l2 = run(lib, q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                 False, 0.4)
    close(o1, o2, 1e-13, 1e-14, "permutation O")
    close(l1, l2, 1e-14, 1e-14, "permutation LSE")


def pin_key_shift(lib):
    """k_j <- k_j + u for every j: O unchanged, LSE_i <- LSE_i + scale q_i . u."""
    rng = np.random.default_rng(19)
    B, H, N, d = 1, 2, 20, 8
    q = small_ints(rng, (B, H, N, d))
    k = small_ints(rng, (B, H, N, d))
    v = rand_bf16(rng, (B, H, N, d))
    u = rng.integers(-2, 3, size=d).astype(np.float32)
    k2 = bf(fl(k) + u)
    scale = 0.125
    for causal in (False, True):
        o1, l1 = run(lib, q, k, v, causal, scale)
        o2, l2 = run(lib, q, k2, v, causal, scale)
        close(o2, o1, 1e-12, 1e-13, f"key shift O causal={causal}")
        close(l2, l1 + scale * (fl(q) @ u.astype(np.float64)), 1e-12, 1e-12,
              f"key shift LSE causal={causal}")


def pin_linear_in_v(lib):
    """O(a V1 + b V2) = a O(V1) + b O(V2)."""
    rng = np.random.default_rng(20)
    B, H, N, d = 1, 2, 24, 8
    q = rand_bf16(rng, (B, H, N, d))
    k = rand_bf16(rng, (B, H, N, d))
    v1 = small_ints(rng, (B, H, N, d))
    v2 = small_ints(rng, (B, H, N, d))
    v = bf(2.0 * fl(v1) - 3.0 * fl(v2))
    for causal in (False, True):
        o1, _ = run(lib, q, k, v1, causal, 0.3)
        o2, _ = run(lib, q, k, v2, causal, 0.3)
        o, _ = run(lib, q, k, v, causal, 0.3)
        close(o, 2.0 * o1 - 3.0 * o2, 1e-12, 1e-12, f"linearity causal={causal}")


def pin_causal_prefix(lib):
    """Causal row i equals non-causal attention over keys/values 0..i; the
    causal last row equals the non-causal last row."""
    rng = np.random.default_rng(21)
    B, H, N, d = 1, 2, 19, 8
    q = rand_bf16(rng, (B, H, N, d))
    k = rand_bf16(rng, (B, H, N, d))
    v = rand_bf16(rng, (B, H, N, d))
    oc, lc = run(lib, q, k, v, True, 0.45)
    on, ln_ = run(lib, q, k, v, False, 0.45)
    close(oc[:, :, -1], on[:, :, -1], 1e-14, 1e-15, "causal last row O")
    close(lc[:, :, -1], ln_[:, :, -1], 1e-14, 1e-15, "causal last row LSE")
    for i in (0, 1, 7, 13):
        sub = slice(0, i + 1)
        op, lp = run(lib, np.ascontiguousarray(q[:, :, sub]), np.ascontiguousarray(k[:, :, sub]),
                     np.ascontiguousarray(v[:, :, sub]), False, 0.45)
        close(oc[:, :, i], op[:, :, i], 1e-14, 1e-15, f"causal prefix O row {i}")
        close(lc[:, :, i], lp[:, :, i], 1e-14, 1e-15, f"causal prefix LSE row {i}")


def pin_scale_transfer(lib):
    """attn(2^e Q, K, V, scale 2^-e) == attn(Q, K, V, scale), bit for bit."""
    rng = np.random.default_rng(22)
    B, H, N, d = 1, 2, 17, 8
    q = rand_bf16(rng, (B, H, N, d))
    k = rand_bf16(rng, (B, H, N, d))
    v = rand_bf16(rng, (B, H, N, d))
    q4 = bf(fl(q) * 4.0)
    for causal in (False, True):
        o1, l1 = run(lib, q, k, v, causal, 0.5)
        o2, l2 = run(lib, q4, k, v, causal, 0.125)
        if not (np.array_equal(o1, o2) and np.array_equal(l1, l2)):
            raise AssertionError(f"scale transfer not exact, causal={causal}")


def pin_heads_independent(lib):
    """Each (b, h) head is computed from its own slices only: a batched call
    equals one call per head (B != H catches swapped head indexing)."""
    rng = np.random.default_rng(23)
    B, H, N, d = 2, 3, 10, 4
    q = rand_bf16(rng, (B, H, N, d))
    k = rand_bf16(rng, (B, H, N, d))
    v = rand_bf16(rng, (B, H, N, d))
    for causal in (False, True):
        o, lse = run(lib, q, k, v, causal, 0.6)
        for b in range(B):
            for h in range(H):
                sl = (slice(b, b + 1), slice(h, h + 1))
                oh, lh = run(lib, np.ascontiguousarray(q[sl]), np.ascontiguousarray(k[sl]),
                             np.ascontiguousarray(v[sl]), causal, 0.6)
                if not (np.array_equal(o[b, h], oh[0, 0]) and np.array_equal(lse[b, h], lh[0, 0])):
                    raise AssertionError(f"head ({b},{h}) depends on other heads")


ALL_PINS = [
    pin_bruteforce_decimal,
    pin_scipy_softmax,
    pin_values_all_one,
    pin_query_zero,
    pin_single_key,
    pin_two_keys,
    pin_dominant_key,
    pin_permutation,
    pin_key_shift,
    pin_linear_in_v,
    pin_causal_prefix,
    pin_scale_transfer,
    pin_heads_independent,
]

"""The matrix-product oracle against facts fixed by mathematics, and planted
mistakes in it against those pins.

Pins: exact rational arithmetic (Python fractions over the exactly widened
bf16 values) on small matrices in both layouts; numpy's fp64 matmul (a
library routine) at a size with several hundred terms per sum; closed forms
(identity factor, all-ones factors, K = 0 gives zeros, a rank-one product);
and row selection returns the same rows as the full product.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def _bits(rng, *shape, sigma=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def _f(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def pin_exact_rational(lib):
    """Every element equals the exact rational sum (the terms are dyadic, so a
    correct fp64 evaluation of these small sums is within 1e-15 relative)."""
    rng = np.random.default_rng(31)
    for M, K, N in ((5, 7, 6), (3, 1, 4), (1, 9, 1)):
        a = _bits(rng, M, K, sigma=3.0)
        b_kn = _bits(rng, K, N, sigma=0.25)
        af = [[Fraction(float(x)) for x in row] for row in _f(a)]
        bf = [[Fraction(float(x)) for x in row] for row in _f(b_kn)]
        exact = np.array([[float(sum(af[m][k] * bf[k][n] for k in range(K))) for n in range(N)]
                          for m in range(M)])
        for layout, b in (("nn", b_kn), ("nt", np.ascontiguousarray(b_kn.T))):
            c = oracle.gemm(a, b, layout, lib=lib)
            assert np.allclose(c, exact, rtol=1e-15, atol=1e-15), f"exact {layout} {M}x{K}x{N}"


def pin_numpy_matmul(lib):
    rng = np.random.default_rng(32)
    M, K, N = 37, 300, 29
    a, b = _bits(rng, M, K), _bits(rng, K, N)
    ref = _f(a) @ _f(b)
    scale = np.abs(_f(a)) @ np.abs(_f(b))
    for layout, bb in (("nn", b), ("nt", np.ascontiguousarray(b.T))):
        c = oracle.gemm(a, bb, layout, lib=lib)
        assert np.all(np.abs(c - ref) <= 1e-13 * scale), f"numpy matmul {layout}"


def pin_closed_forms(lib):
    rng = np.random.default_rng(33)
    K, N = 12, 10
    eye = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    b = _bits(rng, K, N)
    assert np.array_equal(oracle.gemm(eye, b, "nn", lib=lib), _f(b)), "I B = B"
    bt = np.ascontiguousarray(b.T)
    assert np.array_equal(oracle.gemm(eye, bt, "nt", lib=lib), _f(b)), "I (B^T)^T = B"
    ones_a = f32_to_bf16_bits(np.ones((4, K), np.float32))
    ones_b = f32_to_bf16_bits(np.ones((K, 3), np.float32))
    assert np.all(oracle.gemm(ones_a, ones_b, "nn", lib=lib) == K), "ones: C = K"
    empty = oracle.gemm(np.zeros((3, 0), np.uint16), np.zeros((0, 5), np.uint16), "nn", lib=lib)
    assert empty.shape == (3, 5) and np.all(empty == 0.0), "K = 0: C = 0"
    # rank one: a = u 1^T, b = 1 w^T (small integers, exact): c = K u w^T
    u = np.arange(1, 6, dtype=np.float32)
    w = np.arange(-3, 4, dtype=np.float32)
    a1 = f32_to_bf16_bits(np.repeat(u[:, None], K, axis=1))
    b1 = f32_to_bf16_bits(np.repeat(w[None, :], K, axis=0))
    assert np.array_equal(oracle.gemm(a1, b1, "nn", lib=lib), K * np.outer(u, w)), "rank one"


def pin_row_selection(lib):
    rng = np.random.default_rng(34)
    a, b = _bits(rng, 20, 16), _bits(rng, 11, 16)
    full = oracle.gemm(a, b, "nt", lib=lib)
    rows = np.array([19, 0, 7, 7, 3])
    assert np.array_equal(oracle.gemm(a, b, "nt", rows=rows, lib=lib), full[rows]), "rows"
    assert np.array_equal(oracle.gemm(a, b, "nt", threads=3, lib=lib), full), "threads"


ALL_GEMM_PINS = [pin_exact_rational, pin_numpy_matmul, pin_closed_forms, pin_row_selection]


@pytest.mark.parametrize("pin", ALL_GEMM_PINS, ids=lambda p: p.__name__)
def test_gemm_pin_holds(pin):
    pin(oracle.load())


MUTANTS = {
    "nn stride uses K": ("b[k * N + n] : b[n * K + k]", "b[k * K + n] : b[n * K + k]"),
    "nt stride uses N": ("b[k * N + n] : b[n * K + k]", "b[k * N + n] : b[n * N + k]"),
    "layouts swapped": ("b_layout == 0 ? b[k * N + n]", "b_layout == 1 ? b[k * N + n]"),
    "last k dropped": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "a row stride uses N": ("const uint16_t *arow = a + m * K;", "const uint16_t *arow = a + m * N;"),
    "float accumulator": ("double sum = 0.0;", "float sum = 0.0f;"),
    "row taken from r": ("const uint16_t *arow = a + m * K;", "const uint16_t *arow = a + r * K;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gemm_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle.GEMM_SOURCE).read()
    assert src.count(before) == 1, f"anchor for '{name}' not found exactly once"
    mutated = tmp_path / "gemm_oracle_mutant.c"
    mutated.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libgemm_mutant.so")
    oracle.build(str(mutated), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_GEMM_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin detects the mutation '{name}'"

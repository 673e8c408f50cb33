"""The backward oracle against its pins, and mutations of it against the pins.

The mutations are textual edits of ``oracle/attn_bwd_oracle.c`` compiled (with
the unmodified forward oracle) into a temporary library on the CPU; the real
oracle is never modified.  Every edit keeps all memory accesses in bounds.
"""
import os

import pytest

import oracle
from oracle_bwd_pins import ALL_BWD_PINS

BWD_SOURCE = os.path.join(os.path.dirname(oracle.SOURCE), "attn_bwd_oracle.c")


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_pin_holds(pin):
    pin(oracle.load())


MUTANTS = {
    "delta not subtracted": ("ds[i * N + j] = pij * (dp - delta[i]);", "ds[i * N + j] = pij * dp;"),
    "dS sign flipped": ("ds[i * N + j] = pij * (dp - delta[i]);", "ds[i * N + j] = pij * (delta[i] - dp);"),
    "dK scale dropped": ("dk[j * d + t] = scale * ak;", "dk[j * d + t] = ak;"),
    "dQ scale dropped": ("dq[i * d + t] = scale * aq;", "dq[i * d + t] = aq;"),
    "dQ contracts with V": ("aq += ds[i * N + j] * k[j * d + t];", "aq += ds[i * N + j] * v[j * d + t];"),
    "dK contracts with dO": ("ak += ds[i * N + j] * q[i * d + t];", "ak += ds[i * N + j] * dout[i * d + t];"),
    "dV uses P untransposed": ("av += p[i * N + j] * dout[i * d + t];", "av += p[j * N + i] * dout[i * d + t];"),
    "causal dS mask off by one": ("if (causal && j > i) { ds[i * N + j] = 0.0; continue; }",
                                  "if (causal && j >= i) { ds[i * N + j] = 0.0; continue; }"),
    "delta from V": ("acc += dout[i * d + t] * o[i * d + t];", "acc += dout[i * d + t] * v[i * d + t];"),
    "head offset stuck": ("const int64_t off = hh * nd;", "const int64_t off = h_begin * nd;"),
    "forward scale dropped": ("pi[j] = scale * dot;", "pi[j] = dot;"),
    "softmax not normalised": ("for (int64_t j = 0; j < nvis; ++j) pi[j] /= l;",
                               "for (int64_t j = 0; j < nvis; ++j) pi[j] /= 1.0;"),
    "dP uses Q": ("dp += dout[i * d + t] * v[j * d + t];", "dp += dout[i * d + t] * q[j * d + t];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(BWD_SOURCE).read()
    assert src.count(before) == 1, f"anchor for '{name}' not found exactly once"
    mutated = tmp_path / "attn_bwd_mutant.c"
    mutated.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build((oracle.SOURCE, str(mutated)), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin detects the mutation '{name}'"

"""Each plausible mistake planted in a copy of the oracle trips some pin.

The mutations are textual edits of ``oracle/attn_oracle.c`` compiled into a
temporary library on the CPU; the real oracle is never modified.  Every edit
keeps all memory accesses in bounds.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "scale dropped": ("scores[j] = scale * dot;", "scores[j] = dot;"),
    "causal bound off by one": ("causal ? i + 1 : N", "causal ? i : N"),
    "key feature index reversed": ("widen_bf16(kh[j * d + t])", "widen_bf16(kh[j * d + (d - 1 - t)])"),
    "exp sign flipped": ("exp(scores[j] - m)", "exp(m - scores[j])"),
    "max not subtracted": ("exp(scores[j] - m)", "exp(scores[j])"),
    "lse sign flipped": ("*lse_out = m + log(l);", "*lse_out = m - log(l);"),
    "normalisation dropped": ("o_row[t] /= l;", "o_row[t] /= 1.0;"),
    "head index transposed": ("(b * H + h) * N * d", "(h * B + b) * N * d"),
    "value row is the query row": ("widen_bf16(vh[j * d + t])", "widen_bf16(vh[i * d + t])"),
    "query row fixed at zero": ("q + head + i * d", "q + head"),
    "max taken over raw dot": ("if (scores[j] > m) m = scores[j];", "if (dot > m) m = dot;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(before) >= 1, f"anchor for '{name}' not found in the oracle source"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(str(mutated), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin detects the mutation '{name}'"

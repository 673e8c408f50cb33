"""The general-shape backward oracle (Nq queries, Nk keys, bottom-right causal
mask) against facts fixed by mathematics, and planted mistakes in it against
those pins.

Pins:
  * central finite differences of sum(O * dO) through the oracle's own
    general-shape fp64 forward, for Nq < Nk, Nq > Nk (rows with no visible
    key) and Nq = Nk; that forward is itself checked against the pinned
    general-shape forward oracle;
  * a library routine: torch's CPU fp64 autograd through
    scaled_dot_product_attention with an explicit bottom-right boolean mask
    (shapes where every row sees a key);
  * closed forms: rows that see no key get dq = 0 and delta = 0 and leave dK
    and dV unchanged when they are removed; with Nq = Nk the result equals
    the square backward oracle;
  * the bf16 entry point equals the fp64 one on the widened inputs.
"""
import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _loss(lib, q, k, v, g, causal, scale):
    o, _, _ = oracle.forward_head_ex_f64(q, k, v, causal, scale, lib=lib)
    return float(np.sum(o * g))


def pin_ex_bwd_finite_difference(lib):
    rng = np.random.default_rng(41)
    for Nq, Nk, causal in ((3, 6, True), (6, 3, True), (4, 4, True), (3, 5, False)):
        d, scale = 3, 0.7
        q, g = rng.standard_normal((Nq, d)), rng.standard_normal((Nq, d))
        k, v = rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
        dq, dk, dv, _, _, _ = oracle.backward_head_ex_f64(q, k, v, g, causal, scale, lib=lib)
        h = 1e-6
        for name, grad in (("q", dq), ("k", dk), ("v", dv)):
            num = np.zeros_like(grad)
            for idx in np.ndindex(*grad.shape):
                args_p = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args_m = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args_p[name][idx] += h
                args_m[name][idx] -= h
                num[idx] = (_loss(lib, args_p["q"], args_p["k"], args_p["v"], g, causal, scale)
                            - _loss(lib, args_m["q"], args_m["k"], args_m["v"], g, causal, scale)) / (2 * h)
            _close(grad, num, 1e-7, f"d{name} vs finite differences (Nq={Nq} Nk={Nk} causal={causal})")


def pin_ex_forward_matches_forward_oracle(lib):
    rng = np.random.default_rng(42)
    Nq, Nk, d = 5, 9, 4
    qb = f32_to_bf16_bits(rng.standard_normal((1, 1, Nq, d)).astype(np.float32))
    kb = f32_to_bf16_bits(rng.standard_normal((1, 1, Nk, d)).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((1, 1, Nk, d)).astype(np.float32))
    w = lambda b: bf16_bits_to_f32(b[0, 0]).astype(np.float64)  # noqa: E731
    for causal in (False, True):
        o, lse, _ = oracle.forward_head_ex_f64(w(qb), w(kb), w(vb), causal, 0.6, lib=lib)
        o_ref, lse_ref = oracle.attention_ex(qb, kb, vb, causal, 0.6)
        _close(o, o_ref[0, 0], 1e-13, f"forward o (causal={causal})")
        _close(lse, lse_ref[0, 0], 1e-13, f"forward lse (causal={causal})")


def pin_ex_bwd_torch_autograd(lib):
    import torch
    rng = np.random.default_rng(43)
    for Nq, Nk, causal in ((4, 10, True), (7, 7, True), (5, 8, False)):
        d, scale = 6, 0.5
        q, g = rng.standard_normal((Nq, d)), rng.standard_normal((Nq, d))
        k, v = rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
        dq, dk, dv, _, o, _ = oracle.backward_head_ex_f64(q, k, v, g, causal, scale, lib=lib)
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = (j <= i + (Nk - Nq)) if causal else torch.ones(Nq, Nk, dtype=torch.bool)
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            to = torch.nn.functional.scaled_dot_product_attention(
                tq[None, None], tk[None, None], tv[None, None], attn_mask=mask, scale=scale)[0, 0]
        (to * torch.tensor(g)).sum().backward()
        _close(o, to.detach().numpy(), 1e-12, f"o vs torch (Nq={Nq} Nk={Nk})")
        for name, mine, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
            _close(mine, ref.numpy(), 1e-11, f"d{name} vs torch autograd (Nq={Nq} Nk={Nk} causal={causal})")


def pin_ex_bwd_empty_rows(lib):
    rng = np.random.default_rng(44)
    Nq, Nk, d, scale = 7, 3, 4, 0.9
    q, g = rng.standard_normal((Nq, d)), rng.standard_normal((Nq, d))
    k, v = rng.standard_normal((Nk, d)), rng.standard_normal((Nk, d))
    dq, dk, dv, delta, o, lse = oracle.backward_head_ex_f64(q, k, v, g, True, scale, lib=lib)
    n_empty = Nq - Nk
    assert np.all(dq[:n_empty] == 0.0) and np.all(delta[:n_empty] == 0.0), "empty rows: dq = delta = 0"
    assert np.all(o[:n_empty] == 0.0) and np.all(np.isneginf(lse[:n_empty])), "empty rows: o = 0, lse = -inf"
    # the rows that see keys alone give the same dK and dV (square, Nq' = Nk)
    dq2, dk2, dv2, _, _, _ = oracle.backward_head_ex_f64(q[n_empty:], k, v, g[n_empty:], True, scale, lib=lib)
    _close(dk, dk2, 1e-14, "dk without the empty rows")
    _close(dv, dv2, 1e-14, "dv without the empty rows")
    _close(dq[n_empty:], dq2, 1e-14, "dq of the remaining rows")


def pin_ex_bwd_square_and_bf16(lib):
    rng = np.random.default_rng(45)
    B, H, N, d = 1, 2, 9, 4
    bits = [f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)) for _ in range(4)]
    for causal in (False, True):
        got = oracle.attention_bwd_ex(*bits, causal, 0.5, lib=lib)
        ref = oracle.attention_bwd(*bits, causal, 0.5)
        for name, a, b in zip(("dq", "dk", "dv", "delta"), got, ref):
            _close(a, b, 1e-13, f"square case {name} (causal={causal})")
    # bf16 entry point = fp64 entry point on the widened inputs, per head
    qb = f32_to_bf16_bits(rng.standard_normal((1, 2, 4, 3)).astype(np.float32))
    gb = f32_to_bf16_bits(rng.standard_normal((1, 2, 4, 3)).astype(np.float32))
    kb = f32_to_bf16_bits(rng.standard_normal((1, 2, 6, 3)).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((1, 2, 6, 3)).astype(np.float32))
    dq, dk, dv, delta = oracle.attention_bwd_ex(qb, kb, vb, gb, True, 0.8, lib=lib)
    w = lambda b, h: bf16_bits_to_f32(b[0, h]).astype(np.float64)  # noqa: E731
    for h in range(2):
        r = oracle.backward_head_ex_f64(w(qb, h), w(kb, h), w(vb, h), w(gb, h), True, 0.8, lib=lib)
        for name, a, b in zip(("dq", "dk", "dv", "delta"), (dq[0, h], dk[0, h], dv[0, h], delta[0, h]), r[:4]):
            _close(a, b, 0.0, f"bf16 entry point head {h} {name}")


ALL_EX_BWD_PINS = [pin_ex_bwd_finite_difference, pin_ex_forward_matches_forward_oracle,
                   pin_ex_bwd_torch_autograd, pin_ex_bwd_empty_rows, pin_ex_bwd_square_and_bf16]


@pytest.mark.parametrize("pin", ALL_EX_BWD_PINS, ids=lambda p: p.__name__)
def test_ex_bwd_pin_holds(pin):
    pin(oracle.load())


MUTANTS = {
    "top-left mask": ("const int64_t last = i + (Nk - Nq);", "const int64_t last = i;"),
    "mask bound off by one": ("return last < 0 ? 0 : (last + 1 < Nk ? last + 1 : Nk);",
                              "return last < 0 ? 0 : (last < Nk ? last : Nk);"),
    "softmax over masked keys": ("""        for (int64_t j = 0; j < nvis; ++j) {
            pi[j] = exp(pi[j] - m);""", """        for (int64_t j = 0; j < Nk; ++j) {
            pi[j] = exp(pi[j] - m);"""),
    "delta from q": ("acc += dout[i * d + t] * o[i * d + t];", "acc += dout[i * d + t] * q[i * d + t];"),
    "dK from dout": ("ak += ds[i * Nk + j] * q[i * d + t];", "ak += ds[i * Nk + j] * dout[i * d + t];"),
    "dQ scale dropped": ("dq[i * d + t] = scale * aq;", "dq[i * d + t] = aq;"),
    "key rows strided by Nq": ("kf[x] = ex_widen_bf16(k[hh * nkd + x]);", "kf[x] = ex_widen_bf16(k[hh * nqd + x]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_ex_bwd_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle.BWD_EX_SOURCE).read()
    assert src.count(before) == 1, f"anchor for '{name}' not found exactly once"
    mutated = tmp_path / "attn_bwd_ex_mutant.c"
    mutated.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build((oracle.SOURCES[0], oracle.SOURCES[1], str(mutated)), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_EX_BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin detects the mutation '{name}'"

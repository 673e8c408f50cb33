"""Pins for the backward oracle: facts fixed by mathematics, not by the oracle.

Each ``pin_bwd_*`` function takes a loaded oracle library (``oracle.load()`` or
a deliberately broken build of it) and raises ``AssertionError`` when the
library disagrees with the fact it checks.  ``tests/test_oracle_bwd.py`` runs
them against the real oracle and against mutated copies of
``oracle/attn_bwd_oracle.c``; each mutation must trip at least one pin.

The backward pass is the derivative of the forward definition (softmax of the
scaled scores, times V).  What pins it:
  * central finite differences of sum(O * dO) through the oracle's own fp64
    forward, which is in turn pinned to the forward oracle (itself pinned by
    brute force, closed forms and a library softmax);
  * a library routine: torch's CPU fp64 autograd through its reference
    attention (scaled_dot_product_attention with the math backend);
  * closed forms: constant values (dQ = dK = 0), one key (dV = dO, dQ = dK = 0),
    zero dO (everything 0), delta = rowsum(dO * O);
  * invariants: linearity in dO; the bf16 entry point equals the fp64 one on
    the widened inputs, head by head.
"""
from __future__ import annotations

import numpy as np

import oracle
from attention_attn_fwd_08_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(lib, q, k, v, g, causal, scale):
    o, _, _ = oracle.forward_head_f64(q, k, v, causal, scale, lib=lib)
    return float(np.sum(o * g))


def pin_bwd_finite_difference(lib):
    rng = np.random.default_rng(11)
    for causal in (False, True):
        N, d, scale = 5, 3, 0.8
        q, k, v, g = (_rand(rng, N, d) for _ in range(4))
        dq, dk, dv, _, _, _ = oracle.backward_head_f64(q, k, v, g, causal, scale, lib=lib)
        h = 1e-6
        for name, grad in (("q", dq), ("k", dk), ("v", dv)):
            num = np.zeros((N, d))
            for idx in np.ndindex(N, d):
                args_p = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args_m = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args_p[name][idx] += h
                args_m[name][idx] -= h
                num[idx] = (_loss(lib, args_p["q"], args_p["k"], args_p["v"], g, causal, scale)
                            - _loss(lib, args_m["q"], args_m["k"], args_m["v"], g, causal, scale)) / (2 * h)
            _close(grad, num, 1e-7, f"d{name} vs finite differences (causal={causal})")


def pin_bwd_forward_is_the_forward_oracle(lib):
    """The fp64 forward inside the backward oracle equals the pinned forward
    oracle on bf16-representable inputs."""
    rng = np.random.default_rng(12)
    for causal in (False, True):
        N, d, scale = 9, 8, 0.35
        bits = [f32_to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32)) for _ in range(3)]
        o_ref, lse_ref = oracle.attention(*bits, causal, scale, lib=lib)
        qf, kf, vf = (bf16_bits_to_f32(b).astype(np.float64)[0, 0] for b in bits)
        o, lse, _ = oracle.forward_head_f64(qf, kf, vf, causal, scale, lib=lib)
        _close(o, o_ref[0, 0], 1e-12, f"fp64 forward O (causal={causal})")
        _close(lse, lse_ref[0, 0], 1e-12, f"fp64 forward lse (causal={causal})")


def pin_bwd_torch_autograd(lib):
    import torch
    rng = np.random.default_rng(13)
    B, H, N, d, scale = 1, 2, 7, 8, 0.3
    bits = [f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)) for _ in range(4)]
    q, k, v, g = (torch.from_numpy(bf16_bits_to_f32(b).astype(np.float64)) for b in bits)
    for causal in (False, True):
        qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
        with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
            out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=causal,
                                                                   scale=scale)
        out.backward(g)
        dq, dk, dv, _ = oracle.attention_bwd(*bits, causal, scale, lib=lib)
        _close(dq, qq.grad.numpy(), 1e-10, f"dq vs torch autograd (causal={causal})")
        _close(dk, kk.grad.numpy(), 1e-10, f"dk vs torch autograd (causal={causal})")
        _close(dv, vv.grad.numpy(), 1e-10, f"dv vs torch autograd (causal={causal})")


def pin_bwd_constant_values(lib):
    """Every value row the same: O no longer depends on Q or K."""
    rng = np.random.default_rng(14)
    for causal in (False, True):
        N, d = 6, 4
        q, k, g = (_rand(rng, N, d) for _ in range(3))
        v = np.tile(_rand(rng, 1, d), (N, 1))
        dq, dk, dv, delta, o, _ = oracle.backward_head_f64(q, k, v, g, causal, 0.6, lib=lib)
        _close(dq, 0.0, 1e-12, f"dq with constant V (causal={causal})")
        _close(dk, 0.0, 1e-12, f"dk with constant V (causal={causal})")
        _close(o, v, 1e-12, "O with constant V")


def pin_bwd_single_key(lib):
    rng = np.random.default_rng(15)
    q, k, v, g = (_rand(rng, 1, 5) for _ in range(4))
    dq, dk, dv, delta, _, _ = oracle.backward_head_f64(q, k, v, g, False, 0.9, lib=lib)
    _close(dv, g, 1e-14, "dv with one key")
    _close(dq, 0.0, 1e-14, "dq with one key")
    _close(dk, 0.0, 1e-14, "dk with one key")
    _close(delta, [float(g[0] @ v[0])], 1e-14, "delta with one key")


def pin_bwd_zero_dout(lib):
    rng = np.random.default_rng(16)
    q, k, v = (_rand(rng, 4, 3) for _ in range(3))
    out = oracle.backward_head_f64(q, k, v, np.zeros((4, 3)), True, 0.5, lib=lib)
    for name, a in zip(("dq", "dk", "dv", "delta"), out[:4]):
        _close(a, 0.0, 0.0, f"{name} with dO = 0")


def pin_bwd_delta(lib):
    rng = np.random.default_rng(17)
    q, k, v, g = (_rand(rng, 6, 4) for _ in range(4))
    _, _, _, delta, _, _ = oracle.backward_head_f64(q, k, v, g, True, 0.7, lib=lib)
    o, _, _ = oracle.forward_head_f64(q, k, v, True, 0.7, lib=lib)
    _close(delta, np.sum(g * o, axis=1), 1e-13, "delta = rowsum(dO * O)")


def pin_bwd_linear_in_dout(lib):
    rng = np.random.default_rng(18)
    q, k, v, g1, g2 = (_rand(rng, 5, 4) for _ in range(5))
    a = oracle.backward_head_f64(q, k, v, 2.0 * g1 + g2, False, 0.4, lib=lib)
    b1 = oracle.backward_head_f64(q, k, v, g1, False, 0.4, lib=lib)
    b2 = oracle.backward_head_f64(q, k, v, g2, False, 0.4, lib=lib)
    for i, name in enumerate(("dq", "dk", "dv", "delta")):
        _close(a[i], 2.0 * b1[i] + b2[i], 1e-12, f"{name} linear in dO")


def pin_bwd_bf16_entry_per_head(lib):
    rng = np.random.default_rng(19)
    B, H, N, d, scale = 2, 3, 5, 4, 0.5
    bits = [f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)) for _ in range(4)]
    for causal in (False, True):
        dq, dk, dv, delta = oracle.attention_bwd(*bits, causal, scale, threads=2, lib=lib)
        for b in range(B):
            for h in range(H):
                f = [bf16_bits_to_f32(x[b, h]).astype(np.float64) for x in bits]
                ref = oracle.backward_head_f64(*f, causal, scale, lib=lib)
                for got, want, name in zip((dq, dk, dv, delta), ref[:4], ("dq", "dk", "dv", "delta")):
                    _close(got[b, h], want, 0.0, f"{name} head ({b},{h}) bf16 entry (causal={causal})")


ALL_BWD_PINS = [
    pin_bwd_finite_difference,
    pin_bwd_forward_is_the_forward_oracle,
    pin_bwd_torch_autograd,
    pin_bwd_constant_values,
    pin_bwd_single_key,
    pin_bwd_zero_dout,
    pin_bwd_delta,
    pin_bwd_linear_in_dout,
    pin_bwd_bf16_entry_per_head,
]

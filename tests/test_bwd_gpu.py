"""GPU parity of the attention backward (attn_bwd) against the fp64 oracle.

Tolerances come from the arithmetic: the kernels round P and dS to bf16 as
MFMA operands (relative error up to 2^-9 each), take delta from the forward's
bf16 O, and round dQ/dK/dV to bf16 (2^-9); products accumulate in fp32.  The
resulting error is a few units of 2^-9 relative to the magnitude of the
gradient, so each gradient must satisfy
    max |err| <= 1e-2 * max |ref|   and   mean |err| <= 1e-2 * mean |ref|,
and, block by block (every head, every 32 rows of dQ, dK or dV: the rows
one wave computes), so that an error confined to small-magnitude rows cannot
hide under the gradient's overall maximum,
    max |err| <= 2e-2 * max |ref of the block| + 2e-3 * max |ref of the head|
(the head-level floor covers blocks whose dS = P (dP - delta) cancels, where
the rounding of P and of delta stays at the size of the uncancelled terms;
both bars carry the same 1e-6 absolute slack for gradients that are exactly
0, e.g. dQ of a row that sees a single key).
delta, an fp32 sum of d bf16 products, must match rowsum(dO * O) of the
forward's own O to 1e-5 relative.
"""
import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import make_qkv_dout
from gpu_util import ORACLE_THREADS, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 1e-2
GRAD_MEAN_REL = 1e-2
BLOCK_REL = 2e-2      # per 32-row block, relative to the block's own maximum
BLOCK_HEAD_FLOOR = 2e-3  # plus this fraction of the head's maximum
BLOCK_ROWS = 32
DELTA_REL = 1e-5


def run_fwd_bwd(bits, causal, scale):
    import torch
    import attention_attn_fwd_08_amd as af
    q, k, v, g = (to_device(x) for x in bits)
    o, lse = af.attn_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv, delta = af.attn_bwd(q, k, v, o, lse, g, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, (dq, dk, dv, delta), g


def check_grads(got, ref, what):
    for name, a, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        a = to_host_f64(a) if not isinstance(a, np.ndarray) else a
        assert np.isfinite(a).all(), f"{what} {name}: non-finite"
        e = np.abs(a - r)
        log(f"  {what} {name}: max {e.max():.3e} (ref max {np.abs(r).max():.3e}) "
            f"mean {e.mean():.3e} (ref mean {np.abs(r).mean():.3e})")
        assert e.max() <= GRAD_MAX_REL * np.abs(r).max() + 1e-6, f"{what} {name} max err"
        assert e.mean() <= GRAD_MEAN_REL * np.abs(r).mean() + 1e-7, f"{what} {name} mean err"
        check_blocks(e, r, f"{what} {name}")


def check_blocks(err, ref, what):
    """Per head and per 32-row block: max |err| <= BLOCK_REL * block max |ref|
    + BLOCK_HEAD_FLOOR * head max |ref| (arrays [..., rows, d])."""
    rows, d = err.shape[-2], err.shape[-1]
    e = err.reshape(-1, rows, d)
    r = np.abs(ref).reshape(-1, rows, d)
    worst = 0.0
    for h in range(e.shape[0]):
        head_max = r[h].max()
        for r0 in range(0, rows, BLOCK_ROWS):
            be = e[h, r0:r0 + BLOCK_ROWS].max()
            bound = BLOCK_REL * r[h, r0:r0 + BLOCK_ROWS].max() + BLOCK_HEAD_FLOOR * head_max + 1e-6
            worst = max(worst, be / bound)
            assert be <= bound, f"{what}: head {h} rows {r0}..{r0 + BLOCK_ROWS - 1} err {be:.3e} > {bound:.3e}"
    log(f"  {what}: worst block err / bound {worst:.3f}")


def check_delta(delta, o, g, what):
    d_gpu = delta.cpu().numpy().astype(np.float64)
    prod = to_host_f64(g) * to_host_f64(o)
    ref = prod.sum(axis=-1)
    bound = DELTA_REL * np.maximum(1.0, np.abs(prod).sum(axis=-1))
    err = np.abs(d_gpu - ref)
    log(f"  {what} delta: max {err.max():.3e}")
    assert (err <= bound).all(), f"{what} delta"


SHAPES = [
    # (B, H, N, d, causal): several tiles, ragged tails, every head dim
    (1, 2, 256, 64, False), (1, 2, 256, 64, True),
    (1, 2, 256, 128, False), (1, 2, 256, 128, True),
    (2, 1, 640, 128, True), (1, 3, 1024, 64, True),
    (1, 2, 1024, 128, False),
    (1, 2, 1, 128, True), (1, 2, 1, 64, False),
    (1, 1, 31, 64, True), (1, 1, 33, 128, True),
    (2, 1, 200, 128, True), (1, 2, 333, 64, False), (1, 1, 1000, 128, True),
    (1, 2, 256, 32, False), (2, 1, 333, 32, True), (1, 2, 256, 96, True), (1, 1, 700, 96, False),
    (1, 2, 256, 256, False), (1, 2, 256, 256, True), (2, 1, 333, 256, True), (1, 1, 700, 256, False),
    # d=128 problems with at least one key block per CU: the 8-wave dK/dV
    # workgroups (dV and dK waves sharing the Q and dO tiles)
    (1, 64, 512, 128, False), (2, 40, 700, 128, True), (1, 256, 160, 128, True),
]


@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
def test_bwd_parity(B, H, N, d, causal):
    log(f"bwd parity B{B} H{H} N{N} d{d} causal={causal}")
    bits = make_qkv_dout(B, H, N, d, seed=31 + N + d)
    scale = 1.0 / np.sqrt(d)
    o, got, g = run_fwd_bwd(bits, causal, scale)
    ref = oracle.attention_bwd(*bits, causal, scale, threads=ORACLE_THREADS)
    check_grads(got, ref, f"B{B}H{H}N{N}d{d}c{int(causal)}")
    check_delta(got[3], o, g, f"B{B}H{H}N{N}d{d}c{int(causal)}")


def test_bwd_full_size_sampled_heads():
    """The 16x16x4096x128 configuration, launched as a whole; two heads
    (first and last) checked against the oracle in full."""
    B, H, N, d = 16, 16, 4096, 128
    log("bwd full size B16 H16 N4096 d128 (heads 0 and 255 checked)")
    bits = make_qkv_dout(B, H, N, d, seed=3)
    scale = 1.0 / np.sqrt(d)
    o, got, g = run_fwd_bwd(bits, False, scale)
    heads = [(0, 0), (B - 1, H - 1)]
    sub = [np.ascontiguousarray(np.stack([x[b, h] for b, h in heads])[None]) for x in bits]
    ref = oracle.attention_bwd(*sub, False, scale, threads=2)
    got_sub = [np.stack([to_host_f64(t[b, h]) for b, h in heads])[None] for t in got[:3]]
    check_grads(got_sub, ref, "full-size heads")


def test_bwd_zero_dout_gives_zero():
    import torch
    import attention_attn_fwd_08_amd as af
    B, H, N, d = 1, 2, 300, 128
    q, k, v, _ = (to_device(x) for x in make_qkv_dout(B, H, N, d, seed=5))
    o, lse = af.attn_fwd(q, k, v, causal=True)
    g = torch.zeros_like(q)
    dq, dk, dv, delta = af.attn_bwd(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, delta):
        assert torch.count_nonzero(t).item() == 0


def test_bwd_deterministic():
    import torch
    import attention_attn_fwd_08_amd as af
    B, H, N, d = 1, 2, 500, 64
    q, k, v, g = (to_device(x) for x in make_qkv_dout(B, H, N, d, seed=6))
    o, lse = af.attn_fwd(q, k, v, causal=True)
    a = af.attn_bwd(q, k, v, o, lse, g, causal=True)
    a = [t.clone() for t in a]
    b = af.attn_bwd(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)

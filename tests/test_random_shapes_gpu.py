"""Seeded random shapes through every attention entry point, against the fp64
oracles at the usual tolerances: a sweep over sizes that are not multiples
of any tile (query and key counts from 1 to a few hundred, all head dims,
causal or not), so that edge cases the hand-picked shapes miss still get
checked.  The shapes are drawn from a fixed seed, so every run checks the
same cases."""
import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import f32_to_bf16_bits
from gpu_util import LSE_MAX_TOL, O_MAX_TOL, O_MEAN_TOL, ORACLE_THREADS, log, to_device, to_host_f64
from test_bwd_gpu import check_delta, check_grads

pytestmark = pytest.mark.gpu


def _cases(n, seed, dims):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        Nq, Nk = int(rng.integers(1, 400)), int(rng.integers(1, 400))
        out.append((B, H, Nq, Nk, int(rng.choice(dims)), bool(rng.integers(0, 2)), int(rng.integers(0, 1 << 30))))
    return out


def _inputs(B, H, Nq, Nk, d, seed, dout=False):
    rng = np.random.default_rng(seed)
    mk = lambda n: f32_to_bf16_bits(rng.standard_normal((B, H, n, d)).astype(np.float32))  # noqa: E731
    q, k, v = mk(Nq), mk(Nk), mk(Nk)
    return (q, k, v, mk(Nq)) if dout else (q, k, v)


def _check_fwd(o, lse, o_ref, lse_ref):
    o_g, l_g = to_host_f64(o), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty)
    assert np.all(o_g[empty] == 0.0)
    full = ~empty
    if full.any():
        eo = np.abs(o_g[full] - o_ref[full])
        el = np.abs(l_g[full] - lse_ref[full])
        assert eo.max() <= O_MAX_TOL and eo.mean() <= O_MEAN_TOL and el.max() <= LSE_MAX_TOL


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,seed", _cases(24, 71, [32, 64, 96, 128, 256]))
def test_random_forward(B, H, Nq, Nk, d, causal, seed):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"random fwd B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    qb, kb, vb = _inputs(B, H, Nq, Nk, d, seed)
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    o_ref, lse_ref = oracle.attention_ex(qb, kb, vb, causal, scale, threads=ORACLE_THREADS)
    o, lse = af.attn_fwd_ex(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check_fwd(o, lse, o_ref, lse_ref)
    splits = 1 + seed % 5
    o2, lse2 = af.attn_fwd_splitkv(q, k, v, causal=causal, scale=scale, n_splits=splits)
    torch.cuda.synchronize()
    _check_fwd(o2, lse2, o_ref, lse_ref)


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,seed",
                         _cases(20, 72, [32, 64, 96, 128]) + _cases(6, 73, [256]))
def test_random_backward(B, H, Nq, Nk, d, causal, seed):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"random bwd B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    bits = _inputs(B, H, Nq, Nk, d, seed, dout=True)
    scale = 1.0 / np.sqrt(d)
    q, k, v, g = (to_device(x) for x in bits)
    o, lse = af.attn_fwd_ex(q, k, v, causal=causal, scale=scale)
    got = af.attn_bwd_ex(q, k, v, o, lse, g, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_ex(*bits, causal, scale, threads=ORACLE_THREADS)
    what = f"B{B}H{H}Nq{Nq}Nk{Nk}d{d}c{int(causal)}"
    check_grads(got, ref, what)
    check_delta(got[3], o, g, what)


def _window_cases(n, seed):
    """Causal shapes at d=32/64/96 with hundreds to thousands of 128-query
    tiles, so that the persistent windows (few rounds of workgroups) and
    their edges are crossed: square, or a query block at the end of a longer
    key range."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 96]))
        H = int(rng.integers(40, 201))
        Nq = int(rng.integers(600, 3001))
        Nk = Nq if rng.integers(0, 2) else Nq + int(rng.integers(1, 2001))
        out.append((1, H, Nq, Nk, d, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("B,H,Nq,Nk,d,seed", _window_cases(12, 76))
def test_random_persistent_windows(B, H, Nq, Nk, d, seed):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"random window B{B} H{H} Nq{Nq} Nk{Nk} d{d} ({B * H * ((Nq + 127) // 128)} query tiles)")
    qb, kb, vb = _inputs(B, H, Nq, Nk, d, seed)
    scale = 1.0 / np.sqrt(d)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    o, lse = af.attn_fwd_ex(q, k, v, causal=True, scale=scale)
    # Every row written, and the same bits again into NaN-filled outputs.
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    af.attn_fwd_ex(q, k, v, causal=True, scale=scale, out=o2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse)
    # Rows at query-tile edges and random rows of every head.
    rng = np.random.default_rng(seed ^ 0x5A5A)
    rows = []
    for bh in range(B * H):
        picks = {0, 127, 128, Nq - 1} | set(int(x) for x in rng.integers(0, Nq, 3))
        rows += [bh * Nq + i for i in sorted(picks) if 0 <= i < Nq]
    rows = np.asarray(rows, dtype=np.int64)
    o_ref, lse_ref = oracle.attention_ex_rows(qb, kb, vb, True, scale, rows, threads=ORACLE_THREADS)
    idx = torch.from_numpy(rows).to(o.device)
    _check_fwd(o.reshape(-1, d)[idx], lse.reshape(-1)[idx], o_ref, lse_ref)

"""GPU parity of attn_bwd_ex (Nq queries against Nk keys, bottom-right causal)
against the general-shape fp64 backward oracle, at the backward's
tolerances (see test_bwd_gpu.py).  Rows that see no key must give dq = 0 and
delta = 0 exactly."""
import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import f32_to_bf16_bits
from gpu_util import ORACLE_THREADS, log, to_device, to_host_f64
from test_bwd_gpu import check_delta, check_grads

pytestmark = pytest.mark.gpu


def _bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


SHAPES = [
    # (B, H, Nq, Nk, d, causal)
    (1, 2, 100, 300, 128, True), (1, 2, 100, 300, 64, False),
    (1, 2, 300, 100, 128, True), (1, 2, 300, 100, 64, True),
    (2, 1, 64, 1000, 128, True), (1, 3, 1, 777, 128, False),
    (1, 1, 513, 257, 64, False), (1, 2, 200, 450, 64, True),
    (1, 1, 77, 33, 128, True), (1, 2, 100, 300, 32, True), (1, 2, 300, 130, 96, True),
    (1, 1, 64, 500, 96, False), (1, 2, 100, 300, 256, True), (1, 1, 300, 130, 256, True),
    # at least one key block per CU at d=128: the 8-wave dK/dV workgroups
    (1, 80, 300, 700, 128, True), (1, 128, 700, 256, 128, True), (2, 64, 200, 500, 128, False),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", SHAPES)
def test_bwd_ex_parity(B, H, Nq, Nk, d, causal):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"bwd_ex parity B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    rng = np.random.default_rng(6000 + Nq + 3 * Nk + d)
    qb, gb = _bits(rng, (B, H, Nq, d)), _bits(rng, (B, H, Nq, d))
    kb, vb = _bits(rng, (B, H, Nk, d)), _bits(rng, (B, H, Nk, d))
    scale = 1.0 / np.sqrt(d)
    q, k, v, g = (to_device(x) for x in (qb, kb, vb, gb))
    o, lse = af.attn_fwd_ex(q, k, v, causal=causal, scale=scale)
    got = af.attn_bwd_ex(q, k, v, o, lse, g, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_ex(qb, kb, vb, gb, causal, scale, threads=ORACLE_THREADS)
    what = f"B{B}H{H}Nq{Nq}Nk{Nk}d{d}c{int(causal)}"
    check_grads(got, ref, what)
    check_delta(got[3], o, g, what)
    empty = np.isneginf(lse.cpu().numpy())
    if empty.any():
        assert np.all(to_host_f64(got[0])[empty] == 0.0), "rows without keys: dq = 0"
        assert np.all(got[3].cpu().numpy()[empty] == 0.0), "rows without keys: delta = 0"


def test_bwd_ex_square_is_attn_bwd():
    import torch
    import attention_attn_fwd_08_amd as af
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q, k, v, do = (torch.randn(1, 2, 300, 128, device="cuda", generator=g).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = af.attn_fwd(q, k, v, causal=True)
    a = af.attn_bwd(q, k, v, o, lse, do, causal=True)
    b = af.attn_bwd_ex(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_ex_without_queries_or_keys():
    import torch
    import attention_attn_fwd_08_amd as af
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    k, v = (torch.randn(1, 2, 200, 64, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    q0 = torch.zeros(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    lse0 = torch.zeros(1, 2, 0, device="cuda")
    dk = torch.full_like(k, 3.0)
    dv = torch.full_like(v, 3.0)
    af.attn_bwd_ex(q0, k, v, q0, lse0, q0, causal=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0, "no queries: dK = dV = 0"
    q, do = (torch.randn(1, 2, 50, 64, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    k0 = torch.zeros(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = af.attn_fwd_ex(q, k0, k0)
    dq, _, _, delta = af.attn_bwd_ex(q, k0, k0, o, lse, do)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq).item() == 0 and torch.count_nonzero(delta).item() == 0, "no keys: dQ = 0"

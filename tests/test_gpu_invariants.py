"""Closed forms and invariants checked on the HIP path's own outputs."""
import math

import numpy as np
import pytest

from attention_attn_fwd_08_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_qkv
from gpu_util import log, run_gpu, to_host_f64

pytestmark = pytest.mark.gpu


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True),
                                      (32, True), (96, False), (256, True)])
def test_values_all_one(d, causal):
    """V = 1: every output is 1 (up to bf16 P rounding against an fp32 sum)."""
    log(f"[V=1] d={d} causal={causal}")
    q, k, _ = make_qkv(2, 2, 512, d, seed=7)
    v = bits(np.ones(q.shape))
    o, _ = run_gpu(q, k, v, causal, 1 / math.sqrt(d))
    assert np.abs(to_host_f64(o) - 1.0).max() <= 8e-3


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True),
                                      (32, True), (96, False), (256, True)])
def test_query_zero(d, causal):
    """Q = 0: O is the (prefix) mean of V and LSE = ln(#visible keys)."""
    log(f"[Q=0] d={d} causal={causal}")
    _, k, v = make_qkv(1, 2, 384, d, seed=8)
    q = bits(np.zeros(k.shape))
    o, lse = run_gpu(q, k, v, causal, 1 / math.sqrt(d))
    vf = bf16_bits_to_f32(v).astype(np.float64)
    N = k.shape[2]
    if causal:
        cnt = np.arange(1, N + 1, dtype=np.float64)
        ref = np.cumsum(vf, axis=2) / cnt[None, None, :, None]
        lref = np.broadcast_to(np.log(cnt), (1, 2, N))
    else:
        ref = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
        lref = np.full((1, 2, N), math.log(N))
    assert np.abs(to_host_f64(o) - ref).max() <= 1e-2
    assert np.abs(to_host_f64(lse) - lref).max() <= 1e-4


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_causal_row_zero_is_exact(d):
    """Causal row 0 sees only key 0: O[0] equals V[0] bit for bit."""
    log(f"[causal row 0] d={d}")
    q, k, v = make_qkv(2, 2, 256, d, seed=9, qk_sigma=2.0)
    o, lse = run_gpu(q, k, v, True, 1 / math.sqrt(d))
    o0 = o[:, :, 0].contiguous().view(dtype=__import__("torch").int16).cpu().numpy()
    assert np.array_equal(o0.view(np.uint16), v[:, :, 0])
    qf = bf16_bits_to_f32(q[:, :, 0]).astype(np.float64)
    kf = bf16_bits_to_f32(k[:, :, 0]).astype(np.float64)
    assert np.abs(to_host_f64(lse[:, :, 0]) - (qf * kf).sum(-1) / math.sqrt(d)).max() <= 1e-4


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_permutation_non_causal(d):
    """Permuting the rows of K and V together leaves non-causal O and LSE unchanged."""
    log(f"[permutation] d={d}")
    q, k, v = make_qkv(1, 2, 512, d, seed=10)
    perm = np.random.default_rng(3).permutation(512)
    o1, l1 = run_gpu(q, k, v, False, 1 / math.sqrt(d))
    o2, l2 = run_gpu(q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                     False, 1 / math.sqrt(d))
    assert np.abs(to_host_f64(o1) - to_host_f64(o2)).max() <= 1e-2
    assert np.abs(to_host_f64(l1) - to_host_f64(l2)).max() <= 1e-4


@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_deterministic(d, causal):
    """Three runs give bit-identical O and LSE (no atomics, static schedule)."""
    import torch
    log(f"[determinism] d={d} causal={causal}")
    q, k, v = make_qkv(2, 4, 1024, d, seed=11)
    outs = [run_gpu(q, k, v, causal, 1 / math.sqrt(d)) for _ in range(3)]
    for o, lse in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), outs[0][1].view(torch.int32))


def test_empty_problem():
    import torch
    import attention_attn_fwd_08_amd as af
    x = torch.zeros(0, 2, 128, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = af.attn_fwd(x, x, x)
    assert o.shape == x.shape and lse.shape == (0, 2, 128)


def test_bad_head_dim_raises_on_gpu():
    import torch
    import attention_attn_fwd_08_amd as af
    x = torch.zeros(1, 1, 128, 80, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(af.AttnError):
        af.attn_fwd(x, x, x)

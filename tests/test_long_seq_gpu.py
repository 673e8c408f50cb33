"""Long sequences: the forward at N = 131 072 and split-KV decoding over
262 181 keys, checked against the oracle on sampled rows.

These sizes take the index arithmetic (per-head byte offsets, buffer
ranges, key-tile counts, persistent tile ids, split chunks) far past the
workloads' and end on ragged tails.  Each oracle row is O(N d), so the
checks stay cheap.
"""
import math

import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import Workload, make_qkv, sample_rows
from gpu_util import ORACLE_THREADS, assert_parity, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
def test_forward_n131072(causal):
    import attention_attn_fwd_08_amd as af
    import torch
    B, H, N, d = 1, 2, 131072, 128
    log(f"[long] forward B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B, H, N, d, seed=600 + int(causal))
    scale = 1.0 / math.sqrt(d)
    o, lse = af.attn_fwd(*(to_device(x) for x in (q, k, v)), causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = sample_rows(Workload("long", B, H, N, d, causal, seed=0), per_head=12, block=256)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, causal, scale, rows, threads=ORACLE_THREADS)
    o_g = to_host_f64(o.reshape(-1, d)[torch.from_numpy(rows).to(o.device)])
    l_g = to_host_f64(lse.reshape(-1)[torch.from_numpy(rows).to(o.device)])
    assert_parity(o_g, l_g, o_ref, lse_ref, f"N={N} ({rows.size} rows)")


def test_splitkv_decode_262181_keys():
    import attention_attn_fwd_08_amd as af
    import torch
    B, H, Nq, Nk, d = 1, 4, 1, 262181, 128
    log(f"[long] split-KV B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    q = make_qkv(B, H, Nq, d, seed=610)[0]
    _, k, v = make_qkv(B, H, Nk, d, seed=611)
    scale = 1.0 / math.sqrt(d)
    splits = af.splitkv_splits(B, H, Nq, Nk, d)
    o, lse = af.attn_fwd_splitkv(*(to_device(x) for x in (q, k, v)), causal=True, scale=scale,
                                 n_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ex(q, k, v, True, scale, threads=ORACLE_THREADS)
    log(f"  {splits} splits")
    assert_parity(to_host_f64(o).reshape(-1, d), to_host_f64(lse).reshape(-1),
                  np.asarray(o_ref).reshape(-1, d), np.asarray(lse_ref).reshape(-1), "decode")

"""The entry points called concurrently on several streams.

The library keeps no per-call state and the caller owns every buffer, so
calls on different streams may overlap in time on one GPU.  Each case runs the
forward (persistent and one-workgroup-per-tile grids), the split-KV forward
(with its own workspace), the backward and the GEMM once serially, then again
with each entry point on a stream of its own, all in flight together (three
rounds per stream, outputs refilled with NaN first so a call that writes
nothing is seen), and requires every result to equal the serial one bit for
bit: the kernels are deterministic, so overlap may change timing only.
The split-KV entry point that keeps its partial results in a fixed device
array is left out: calls that overlap on one GPU share that array.
"""
import math

import pytest

from attention_attn_fwd_08_amd.inputs import make_qkv, make_qkv_dout
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu

ROUNDS = 3


def _jobs():
    """(name, inputs, fn(outputs) -> None, make_outputs() -> list of tensors)."""
    import torch
    import attention_attn_fwd_08_amd as af
    jobs = []

    # Forward at d=128 with more query tiles than CUs (persistent grid).
    q, k, v = (to_device(x) for x in make_qkv(2, 80, 1800, 128, seed=901))
    s128 = 1.0 / math.sqrt(128)
    jobs.append(("fwd persistent d=128 causal",
                 lambda outs, q=q, k=k, v=v: af.attn_fwd(q, k, v, causal=True, scale=s128,
                                                         out=outs[0], lse=outs[1]),
                 lambda q=q: [torch.empty_like(q),
                              torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)]))

    # Forward at d=64, one workgroup per tile.
    q2, k2, v2 = (to_device(x) for x in make_qkv(1, 12, 1000, 64, seed=902))
    jobs.append(("fwd d=64",
                 lambda outs, q=q2, k=k2, v=v2: af.attn_fwd(q, k, v, causal=False, scale=0.125,
                                                            out=outs[0], lse=outs[1]),
                 lambda q=q2: [torch.empty_like(q),
                               torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)]))

    # Split-KV decode-like call with its own workspace.
    qd = to_device(make_qkv(1, 8, 3, 128, seed=903)[0])
    _, kd, vd = (to_device(x) for x in make_qkv(1, 8, 4000, 128, seed=904))
    splits = 5
    jobs.append(("split-KV",
                 lambda outs, q=qd, k=kd, v=vd: af.attn_fwd_splitkv(
                     q, k, v, causal=True, scale=s128, n_splits=splits, out=outs[0], lse=outs[1],
                     o_part=outs[2], lse_part=outs[3]),
                 lambda q=qd: [torch.empty_like(q),
                               torch.empty(q.shape[:3], dtype=torch.float32, device=q.device),
                               torch.empty((splits,) + tuple(q.shape), dtype=torch.float32,
                                           device=q.device),
                               torch.empty((splits,) + tuple(q.shape[:3]), dtype=torch.float32,
                                           device=q.device)]))

    # Backward at d=128 (paired dK/dV workgroups).
    qb, kb, vb, gb = (to_device(x) for x in make_qkv_dout(1, 64, 512, 128, seed=905))
    ob, lseb = af.attn_fwd(qb, kb, vb, causal=False, scale=s128)
    jobs.append(("bwd d=128",
                 lambda outs, q=qb, k=kb, v=vb, o=ob, l=lseb, g=gb: af.attn_bwd(
                     q, k, v, o, l, g, causal=False, scale=s128,
                     dq=outs[0], dk=outs[1], dv=outs[2], delta=outs[3]),
                 lambda q=qb: [torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                               torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)]))

    # GEMM, C = A B^T.
    g = torch.Generator(device="cuda").manual_seed(906)
    a = torch.randn(1000, 512, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(776, 512, device="cuda", generator=g).to(torch.bfloat16)
    jobs.append(("gemm nt",
                 lambda outs, a=a, b=b: af.gemm(a, b, "nt", out=outs[0]),
                 lambda: [torch.empty(1000, 776, dtype=torch.bfloat16, device="cuda")]))
    return jobs


def test_concurrent_streams_match_serial():
    import torch
    jobs = _jobs()
    torch.cuda.synchronize()
    serial = []
    for name, fn, make in jobs:
        outs = make()
        fn(outs)
        serial.append(outs)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in jobs]  # default priority
    results = [[make() for _ in range(ROUNDS)] for _, _, make in jobs]
    for per_job in results:
        for outs in per_job:
            for t in outs:
                t.fill_(float("nan"))
    torch.cuda.synchronize()
    log(f"[streams] {len(jobs)} entry points x {ROUNDS} rounds on {len(streams)} streams")
    for r in range(ROUNDS):
        for (name, fn, _), st, per_job in zip(jobs, streams, results):
            with torch.cuda.stream(st):
                fn(per_job[r])
    torch.cuda.synchronize()
    for (name, _, _), ref, per_job in zip(jobs, serial, results):
        for r, outs in enumerate(per_job):
            for i, (got, want) in enumerate(zip(outs, ref)):
                assert torch.equal(got, want), f"{name}: output {i} differs in round {r}"

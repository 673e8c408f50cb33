"""The entry points under HIP graph capture.

A caller that launches from a captured graph (decoding loops, serving) must
get the eager results on every replay.  Each case captures one call into a
torch CUDA graph with preallocated outputs, then replays it several times,
with eager work on the same stream between replays (the outputs are refilled
with NaN, so a replay that writes nothing is seen), and compares every replay
bit for bit with an eager call.  The kernels are deterministic (no atomics,
static schedules), so equality is exact.
"""
import math

import pytest

from attention_attn_fwd_08_amd.inputs import make_qkv
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_and_check(capture_fn, outputs, expected, what):
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        capture_fn()  # one eager call on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        capture_fn()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref, name in zip(outputs, expected, [f"out{i}" for i in range(len(outputs))]):
            assert torch.equal(got, ref), f"{what}: replay {r}: {name} differs from the eager result"
    log(f"  {what}: {REPLAYS} replays equal the eager call")


# (B, H, N, d, causal): d=128 with more tiles than CUs takes the persistent
# path; the d=64 case one workgroup per tile.
FWD = [(1, 40, 1800, 128, True), (2, 3, 700, 64, False)]


@pytest.mark.parametrize("B,H,N,d,causal", FWD)
def test_forward_graph(B, H, N, d, causal):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"[graph fwd] B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = (to_device(x) for x in make_qkv(B, H, N, d, seed=400 + N + d))
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = af.attn_fwd(q, k, v, causal=causal, scale=scale)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    _replay_and_check(lambda: af.attn_fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse),
                      [o, lse], [o_ref, lse_ref], "attn_fwd")


def test_splitkv_graph():
    import torch
    import attention_attn_fwd_08_amd as af
    B, H, Nq, Nk, d = 1, 8, 1, 5000, 128
    log(f"[graph split-KV] B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    q = to_device(make_qkv(B, H, Nq, d, seed=401)[0])
    _, k, v = (to_device(x) for x in make_qkv(B, H, Nk, d, seed=402))
    scale = 1.0 / math.sqrt(d)
    n_splits = 6
    o_ref, lse_ref = af.attn_fwd_splitkv(q, k, v, causal=True, scale=scale, n_splits=n_splits)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    o_part = torch.empty(n_splits, B, H, Nq, d, device=q.device, dtype=torch.float32)
    lse_part = torch.empty(n_splits, B, H, Nq, device=q.device, dtype=torch.float32)
    _replay_and_check(lambda: af.attn_fwd_splitkv(q, k, v, causal=True, scale=scale, n_splits=n_splits,
                                                  out=o, lse=lse, o_part=o_part, lse_part=lse_part),
                      [o, lse], [o_ref, lse_ref], "attn_fwd_splitkv")


def test_backward_graph():
    import torch
    import attention_attn_fwd_08_amd as af
    B, H, N, d, causal = 2, 3, 700, 128, True
    log(f"[graph bwd] B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = (to_device(x) for x in make_qkv(B, H, N, d, seed=403))
    dout = to_device(make_qkv(B, H, N, d, seed=404)[0])
    scale = 1.0 / math.sqrt(d)
    o, lse = af.attn_fwd(q, k, v, causal=causal, scale=scale)
    refs = af.attn_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale)
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    delta = torch.empty_like(lse)
    _replay_and_check(lambda: af.attn_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale,
                                          dq=dq, dk=dk, dv=dv, delta=delta),
                      [dq, dk, dv, delta], list(refs), "attn_bwd")

"""Stale-LDS detection: the forward built with every LDS byte first set to a
NaN pattern must give the library's results bit for bit.

An operand read of an LDS location that no copy of the current tile has
written (a missing wait, a wrong stage, a tail row the copies skip) would
read NaN there and turn its outputs into NaN, or at least change them.
Both libraries run the same kernels otherwise, so the comparison is exact.
The debug library is built beside the main one by the package's build step.
"""
import ctypes
import math
import os

import pytest

from attention_attn_fwd_08_amd import _build
from attention_attn_fwd_08_amd.inputs import make_qkv
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu

vp = ctypes.c_void_p


def _poison_lib():
    if not os.path.exists(_build.POISON_LIBRARY):
        pytest.fail(f"{_build.POISON_LIBRARY} is missing: run the build step first")
    lib = ctypes.CDLL(_build.POISON_LIBRARY)
    lib.attn_fwd.argtypes = [vp] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, vp]
    lib.attn_fwd_ex.argtypes = [vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, vp]
    lib.attn_fwd_splitkv.argtypes = ([vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int]
                                     + [vp] * 3)
    for f in (lib.attn_fwd, lib.attn_fwd_ex, lib.attn_fwd_splitkv):
        f.restype = ctypes.c_int
    return lib


# (B, H, Nq, Nk, d, causal, splits): square shapes (persistent at d=128/256
# with more tiles than CUs, and at d=32, 64 and 96 causal with few rounds of
# workgroups; ragged tails), general shapes and split-KV.
CASES = [
    (1, 40, 1800, 1800, 128, True, 0),
    (2, 40, 3000, 3000, 64, True, 0),
    (3, 32, 2000, 2000, 32, True, 0),
    (2, 40, 1500, 1500, 96, True, 0),
    (1, 80, 1500, 2000, 96, True, 0),
    (2, 3, 700, 700, 128, False, 0),
    (1, 20, 1700, 1700, 256, True, 0),
    (2, 3, 333, 333, 64, True, 0),
    (1, 2, 257, 257, 32, False, 0),
    (1, 2, 300, 300, 96, True, 0),
    (1, 3, 100, 900, 128, True, 0),
    (1, 2, 900, 100, 64, True, 0),
    (1, 4, 1, 5000, 128, True, 6),
    (1, 2, 3, 2000, 64, False, 4),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,splits", CASES)
def test_poisoned_lds_gives_identical_results(B, H, Nq, Nk, d, causal, splits):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"[lds poison] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={splits}")
    lib = _poison_lib()
    q = to_device(make_qkv(B, H, Nq, d, seed=500 + Nq + d)[0])
    _, k, v = (to_device(x) for x in make_qkv(B, H, Nk, d, seed=501 + Nk + d))
    scale = 1.0 / math.sqrt(d)
    if splits:
        o_ref, lse_ref = af.attn_fwd_splitkv(q, k, v, causal=causal, scale=scale, n_splits=splits)
    else:
        o_ref, lse_ref = af.attn_fwd_ex(q, k, v, causal=causal, scale=scale)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    stream = vp(torch.cuda.current_stream().cuda_stream)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    if splits:
        o_part = torch.empty(splits, B, H, Nq, d, device=q.device, dtype=torch.float32)
        lse_part = torch.empty(splits, B, H, Nq, device=q.device, dtype=torch.float32)
        st = lib.attn_fwd_splitkv(*ptrs, B, H, Nq, Nk, d, int(causal), scale, splits,
                                  o_part.data_ptr(), lse_part.data_ptr(), stream)
    elif Nq == Nk:
        st = lib.attn_fwd(*ptrs, B, H, Nq, d, int(causal), scale, stream)
    else:
        st = lib.attn_fwd_ex(*ptrs, B, H, Nq, Nk, d, int(causal), scale, stream)
    assert st == 0, af.attn_fwd_strerror(st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "O differs with poisoned LDS"
    assert torch.equal(lse, lse_ref), "LSE differs with poisoned LDS"

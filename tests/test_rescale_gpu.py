"""The online-softmax rescale under test on the GPU.

The running-max recurrence rescales the accumulated output and normaliser
whenever a new key block raises the row maximum (ThunderKittens write-up,
88811315.cn, "RTX 4090 flash-attention example": the max/norm update and the
rescale of o; the same update in its "H100 FlashAttention-2 forward
example").  The kernel keeps the first key tile's maximum as its reference
and takes the rescale branch only when a lane's probabilities over one tile,
formed against that reference, sum past 2^64; Gaussian scores never get
there after the first tile.  Two kinds of test make the branch run:

* planted scores (production library): queries and keys are shifted so that
  the scores rise by 70-190 log2 units at fixed key tiles (``make_stepped_qkv``);
  a host-side replay of the kernel's rule on the exact fp64 scores predicts,
  per query row, how many tiles must take the branch (a single probability
  past 2^64 puts its lane's sum past the cap), the test checks that the
  prediction is unambiguous and non-zero, and compares O and LSE with the
  oracle at the forward's tolerances.  Without the rescale these inputs
  overflow fp32 (probabilities up to 2^190), and a rescale that left O or l
  unscaled would weight old keys by 2^70 or more;
* forced rescale (debug build ``libattn_fwd_force_rescale.so``, compiled with
  ATTN_DEBUG_FORCE_RESCALE): every tile takes the branch, at every head dim
  and entry point, including waves in which rows that see no key (N_q > N_k,
  bottom-right causal) sit beside rows that do: their factor must stay 1, so
  their O = 0 and LSE = -inf come out exact instead of NaN.
"""
import ctypes
import math
import os

import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd import _build
from attention_attn_fwd_08_amd.inputs import bf16_bits_to_f32, make_qkv, make_stepped_qkv
from gpu_util import LSE_MAX_TOL, O_MAX_TOL, O_MEAN_TOL, ORACLE_THREADS, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu

KEY_TILE = 64          # keys per tile of the kernel
WAVE_ROWS = 32         # queries per wave (the branch is taken wave by wave)
CAP_LOG2 = 64.0        # the kernel's cap on a lane's tile sum, 2^64
LANE_KEYS = 32         # keys one lane holds per tile (its sum has at most 32 terms)
MARGIN = 0.5           # log2 units kept clear of the cap on both sides


def chunk_of(Nk: int, n_splits: int) -> int:
    """Keys per split range as the library forms them: ceil(Nk / n_splits)
    rounded up to whole 64-key tiles (include/attn_fwd.h, attn_fwd_splitkv)."""
    c = -(-Nk // n_splits)
    return -(-c // KEY_TILE) * KEY_TILE


def predicted_rescales(qf, kf, causal, scale, kb, ke):
    """Replay of the lazy reference rule on fp64 scores for one head and one
    key range [kb, ke): returns (fires, ambiguous), per query row, the number
    of tiles whose lane sums must exceed the cap, and whether any tile came
    within the margin of it (then the replay is not a prediction).

    The reference m of a row is the maximum of its visible scores in the
    range's first tile.  A later tile must take the branch if one of the
    row's visible keys scores more than CAP_LOG2 + MARGIN above m (in units
    of scale*log2 e); it cannot if every one is below CAP_LOG2 - log2(32) -
    MARGIN.  When a row's tile takes the branch, every row of its wave
    (32 consecutive queries) moves its reference to max(m, tile maximum)."""
    Nq, Nk = qf.shape[0], kf.shape[0]
    c = float(np.float32(scale) * np.float32(1.0 / math.log(2.0)))
    j = np.arange(kb, ke)
    s = qf @ kf[kb:ke].T
    if causal:
        vis = j[None, :] <= (np.arange(Nq)[:, None] + (Nk - Nq))
        s = np.where(vis, s, -np.inf)
    n_tiles = -(-(ke - kb) // KEY_TILE)
    tmax = np.stack([s[:, t * KEY_TILE:(t + 1) * KEY_TILE].max(axis=1) for t in range(n_tiles)], 1)
    m = tmax[:, 0].copy()
    fires = np.zeros(Nq, dtype=np.int64)
    ambiguous = np.zeros(Nq, dtype=bool)
    pad = -(-Nq // WAVE_ROWS) * WAVE_ROWS - Nq
    for t in range(1, n_tiles):
        tm = tmax[:, t]
        has = np.isfinite(tm)
        with np.errstate(invalid="ignore"):
            x = (tm - m) * c
        ambiguous |= has & ~np.isfinite(m)  # a first visible key after the first tile
        ok = has & np.isfinite(m)
        fire = ok & (x > CAP_LOG2 + MARGIN)
        ambiguous |= ok & ~fire & (x > CAP_LOG2 - math.log2(LANE_KEYS) - MARGIN)
        fires += fire
        wave = np.repeat(np.concatenate([fire, np.zeros(pad, bool)]).reshape(-1, WAVE_ROWS).any(1),
                         WAVE_ROWS)[:Nq]
        m = np.where(wave & has, np.maximum(m, tm), m)
    return fires, ambiguous


def predict(q, k, causal, scale, n_splits=1):
    """Per row of every head: tiles that must take the branch, over every
    split range; and whether any replay was ambiguous."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    qf = bf16_bits_to_f32(q).astype(np.float64).reshape(B * H, Nq, d)
    kf = bf16_bits_to_f32(k).astype(np.float64).reshape(B * H, Nk, d)
    chunk = chunk_of(Nk, n_splits) if n_splits > 1 else Nk
    fires = np.zeros((B * H, Nq), dtype=np.int64)
    amb = False
    for bh in range(B * H):
        for kb in range(0, Nk, chunk):
            f, a = predicted_rescales(qf[bh], kf[bh], causal, scale, kb, min(Nk, kb + chunk))
            fires[bh] += f
            amb |= bool(a.any())
    return fires, amb


def check(o, lse, o_ref, lse_ref, what):
    o_g, l_g = to_host_f64(o), lse.detach().cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty), f"{what}: rows without keys must have lse = -inf"
    assert np.all(o_g[empty] == 0.0), f"{what}: rows without keys must have o = 0"
    full = ~empty
    assert np.isfinite(o_g[full]).all() and np.isfinite(l_g[full]).all(), f"{what}: non-finite output"
    eo = np.abs(o_g[full] - o_ref[full])
    el = np.abs(l_g[full] - lse_ref[full])
    log(f"  {what}: O max {eo.max():.3e} mean {eo.mean():.3e}  LSE max {el.max():.3e}")
    assert eo.max() <= O_MAX_TOL, f"{what}: O max err {eo.max()}"
    assert eo.mean() <= O_MEAN_TOL, f"{what}: O mean err {eo.mean()}"
    assert el.max() <= LSE_MAX_TOL, f"{what}: LSE max err {el.max()}"


# B, H, Nq, Nk, d, causal, n_splits, q_shift, k_step, span (keys per level), levels.
# Rows of d=128 problems with more than 256 query tiles (B*H*ceil(N/256) > CUs)
# run in the persistent kernel.
PLANTED = [
    (1, 2, 1024, 1024, 128, False, 1, 1.0, 8.0, 256, 4),
    (1, 2, 1024, 1024, 128, True, 1, 1.0, 8.0, 256, 4),
    (1, 2, 1024, 1024, 64, False, 1, 2.0, 6.0, 256, 4),
    (1, 2, 1024, 1024, 64, True, 1, 2.0, 6.0, 256, 4),
    (1, 40, 1800, 1800, 128, False, 1, 1.0, 8.0, 512, 4),   # persistent
    (1, 40, 1800, 1800, 128, True, 1, 1.0, 8.0, 512, 4),    # persistent, causal
    (1, 2, 300, 1000, 128, True, 1, 1.0, 8.0, 256, 4),      # N_q < N_k
    (1, 2, 1000, 700, 64, True, 1, 2.0, 6.0, 192, 4),       # N_q > N_k: rows with no key
    (1, 4, 5, 3000, 128, True, 4, 1.0, 8.0, 320, 4),        # split-KV
    (1, 4, 40, 2500, 64, False, 3, 2.0, 6.0, 256, 4),       # split-KV
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,n_splits,q_shift,k_step,span,levels", PLANTED)
def test_planted_score_steps_take_the_rescale_branch(B, H, Nq, Nk, d, causal, n_splits, q_shift,
                                                     k_step, span, levels):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"[planted rescale] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={n_splits}")
    q, k, v = make_stepped_qkv(B, H, Nq, Nk, d, seed=700 + Nq + Nk + d, q_shift=q_shift,
                               k_step=k_step, span=span, levels=levels)
    scale = 1.0 / math.sqrt(d)
    fires, amb = predict(q, k, causal, scale, n_splits)
    rows = int((fires > 0).sum())
    log(f"  predicted: {int(fires.sum())} rescale events in {rows} of {fires.size} rows "
        f"(max {int(fires.max())} per row)")
    assert not amb, "a tile comes within the margin of the cap: the prediction is not exact"
    assert rows >= fires.size // 4 and fires.max() >= 2, "the inputs do not reach the cap"
    qd, kd, vd = (to_device(x) for x in (q, k, v))
    if n_splits > 1:
        o, lse = af.attn_fwd_splitkv(qd, kd, vd, causal=causal, scale=scale, n_splits=n_splits)
    elif Nq == Nk:
        o, lse = af.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    else:
        o, lse = af.attn_fwd_ex(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ex(q, k, v, causal, scale, threads=ORACLE_THREADS)
    check(o, lse, o_ref, lse_ref, "planted")


vp = ctypes.c_void_p


def _rescale_lib():
    if not os.path.exists(_build.RESCALE_LIBRARY):
        pytest.fail(f"{_build.RESCALE_LIBRARY} is missing: run the build step first")
    lib = ctypes.CDLL(_build.RESCALE_LIBRARY)
    lib.attn_fwd.argtypes = [vp] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, vp]
    lib.attn_fwd_ex.argtypes = [vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, vp]
    lib.attn_fwd_splitkv.argtypes = ([vp] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int]
                                     + [vp] * 3)
    for f in (lib.attn_fwd, lib.attn_fwd_ex, lib.attn_fwd_splitkv):
        f.restype = ctypes.c_int
    return lib


# (B, H, Nq, Nk, d, causal, splits, qk_sigma): square (persistent at d=128/256
# with more query tiles than CUs), ragged, N_q > N_k with rows that see no key
# in the same waves as rows that do, N_q < N_k, and split-KV.
FORCED = [
    (1, 40, 1800, 1800, 128, True, 0, 1.0),
    (2, 3, 700, 700, 128, False, 0, 2.0),
    (1, 20, 1700, 1700, 256, True, 0, 1.0),
    (2, 3, 333, 333, 64, True, 0, 2.0),
    (1, 128, 1600, 1600, 64, True, 0, 2.0),  # persistent at d=64 (1664 causal query tiles)
    (3, 32, 2000, 2000, 32, True, 0, 1.0),   # persistent at d=32 (1536)
    (2, 40, 1500, 1500, 96, True, 0, 1.0),   # persistent at d=96 (960)
    (1, 80, 1500, 2000, 96, True, 0, 1.0),   # persistent, general shape (960)
    (1, 2, 257, 257, 32, False, 0, 1.0),
    (1, 2, 300, 300, 96, True, 0, 1.0),
    (1, 3, 100, 900, 128, True, 0, 1.0),
    (1, 2, 900, 100, 64, True, 0, 1.0),
    (1, 2, 900, 116, 128, True, 0, 2.0),
    (1, 2, 500, 70, 256, True, 0, 1.0),
    (1, 2, 400, 90, 32, True, 0, 1.0),
    (1, 2, 400, 90, 96, True, 0, 1.0),
    (1, 4, 1, 5000, 128, True, 6, 1.0),
    (1, 2, 3, 2000, 64, False, 4, 2.0),
    (1, 2, 300, 200, 256, True, 2, 1.0),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,splits,sigma", FORCED)
def test_forced_rescale_matches_the_oracle(B, H, Nq, Nk, d, causal, splits, sigma):
    import torch
    log(f"[forced rescale] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={splits} "
        f"sigma={sigma}")
    lib = _rescale_lib()
    q = make_qkv(B, H, Nq, d, seed=800 + Nq + d, qk_sigma=sigma)[0]
    _, k, v = make_qkv(B, H, Nk, d, seed=801 + Nk + d, qk_sigma=sigma)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = (to_device(x) for x in (q, k, v))
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device=qd.device)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=qd.device)
    stream = vp(torch.cuda.current_stream().cuda_stream)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())
    if splits:
        o_part = torch.empty(splits, B, H, Nq, d, device=qd.device, dtype=torch.float32)
        lse_part = torch.empty(splits, B, H, Nq, device=qd.device, dtype=torch.float32)
        st = lib.attn_fwd_splitkv(*ptrs, B, H, Nq, Nk, d, int(causal), scale, splits,
                                  o_part.data_ptr(), lse_part.data_ptr(), stream)
    elif Nq == Nk:
        st = lib.attn_fwd(*ptrs, B, H, Nq, d, int(causal), scale, stream)
    else:
        st = lib.attn_fwd_ex(*ptrs, B, H, Nq, Nk, d, int(causal), scale, stream)
    assert st == 0, f"status {st}"
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ex(q, k, v, causal, scale, threads=ORACLE_THREADS)
    check(o, lse, o_ref, lse_ref, "forced")

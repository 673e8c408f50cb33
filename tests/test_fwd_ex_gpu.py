"""GPU parity of attn_fwd_ex (Nq queries against Nk keys, bottom-right causal)
against the general-shape fp64 oracle, at the forward's tolerances.  Rows that
see no key must come back as exactly o = 0 and lse = -inf."""
import numpy as np
import pytest

import oracle
from attention_attn_fwd_08_amd.inputs import f32_to_bf16_bits
from gpu_util import LSE_MAX_TOL, O_MAX_TOL, O_MEAN_TOL, ORACLE_THREADS, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu


def _bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


SHAPES = [
    # (B, H, Nq, Nk, d, causal)
    (1, 2, 1, 1000, 128, True), (1, 2, 1, 1000, 64, False),
    (1, 2, 100, 300, 128, True), (1, 2, 100, 300, 64, False),
    (1, 2, 300, 100, 128, True), (1, 2, 300, 100, 64, False),
    (2, 1, 256, 4096, 128, True), (1, 1, 513, 257, 64, True),
    (1, 1, 77, 1, 64, True), (1, 3, 40, 2000, 128, False),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", SHAPES)
def test_fwd_ex_parity(B, H, Nq, Nk, d, causal):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"fwd_ex parity B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    rng = np.random.default_rng(1000 + Nq + 7 * Nk + d)
    qb, kb, vb = _bits(rng, (B, H, Nq, d)), _bits(rng, (B, H, Nk, d)), _bits(rng, (B, H, Nk, d))
    scale = 1.0 / np.sqrt(d)
    o, lse = af.attn_fwd_ex(to_device(qb), to_device(kb), to_device(vb), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ex(qb, kb, vb, causal, scale, threads=ORACLE_THREADS)
    o_g, l_g = to_host_f64(o), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty), "rows without keys must have lse = -inf"
    assert np.all(o_g[empty] == 0.0), "rows without keys must have o = 0"
    full = ~empty
    if full.any():
        eo = np.abs(o_g[full] - o_ref[full])
        el = np.abs(l_g[full] - lse_ref[full])
        log(f"  O max {eo.max():.3e} mean {eo.mean():.3e}  LSE max {el.max():.3e}  empty rows {empty.sum()}")
        assert eo.max() <= O_MAX_TOL and eo.mean() <= O_MEAN_TOL and el.max() <= LSE_MAX_TOL


def test_fwd_ex_no_keys():
    import torch
    import attention_attn_fwd_08_amd as af
    q = torch.randn(1, 2, 70, 128, device="cuda").to(torch.bfloat16)
    k = torch.zeros(1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    o, lse = af.attn_fwd_ex(q, k, k)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    assert torch.isneginf(lse).all().item()


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_ex_square_is_attn_fwd(causal):
    import torch
    import attention_attn_fwd_08_amd as af
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    q, k, v = (torch.randn(2, 2, 300, 128, device="cuda", generator=g).to(torch.bfloat16)
               for _ in range(3))
    o1, l1 = af.attn_fwd(q, k, v, causal=causal)
    o2, l2 = af.attn_fwd_ex(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# At d=128 and d=256, problems with more query tiles than the GPU has compute
# units run one persistent workgroup per CU.  These general shapes include
# query tiles that see no key at all (Nq > Nk, causal) and partial last tiles
# whose waves past Nq compute nothing; both continue to the next tile.  At
# d=32, 64 and 96 causal problems with Nq <= Nk and few rounds of workgroups
# run persistent too: the last three cases have 1536, 2048 and 960 query
# tiles of 128, inside those windows at any plausible number of workgroups
# per CU.
PERSISTENT = [
    # (B, H, Nq, Nk, d, causal)
    (1, 40, 1800, 2600, 128, True),
    (1, 40, 2600, 1800, 128, True),
    (1, 50, 700, 3000, 128, False),
    (1, 20, 1700, 2100, 256, True),
    (1, 24, 2100, 1500, 256, True),
    (1, 192, 1024, 2048, 32, True),
    (1, 128, 2000, 2600, 64, True),
    (1, 80, 1500, 2000, 96, True),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", PERSISTENT)
def test_fwd_ex_persistent_sampled(B, H, Nq, Nk, d, causal):
    import torch
    import attention_attn_fwd_08_amd as af
    log(f"fwd_ex persistent B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    rng = np.random.default_rng(2000 + Nq + 7 * Nk + d)
    qb, kb, vb = _bits(rng, (B, H, Nq, d)), _bits(rng, (B, H, Nk, d)), _bits(rng, (B, H, Nk, d))
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = to_device(qb), to_device(kb), to_device(vb)
    o, lse = af.attn_fwd_ex(qd, kd, vd, causal=causal, scale=scale)
    # Every row written, and the same bits on a second call into NaN-filled outputs.
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    af.attn_fwd_ex(qd, kd, vd, causal=causal, scale=scale, out=o2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse), "rows unwritten or results not repeatable"
    # Per head: rows at both ends, around the first row that sees a key, at
    # query-tile edges, and seeded random rows.
    first_seen = max(0, Nq - Nk) if causal else 0
    fixed = {0, 1, first_seen - 1, first_seen, first_seen + 1, Nq // 2, Nq - 1, 255, 256, 511, 512}
    rows = []
    for bh in range(B * H):
        extra = rng.choice(Nq, size=6, replace=False)
        rows += [bh * Nq + i for i in sorted((fixed | set(int(e) for e in extra))) if 0 <= i < Nq]
    rows = np.asarray(rows, dtype=np.int64)
    o_ref, lse_ref = oracle.attention_ex_rows(qb, kb, vb, causal, scale, rows, threads=ORACLE_THREADS)
    o_g = to_host_f64(o.reshape(-1, d)[torch.from_numpy(rows).to(o.device)])
    l_g = lse.reshape(-1)[torch.from_numpy(rows).to(o.device)].cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty), "rows with no visible key must have lse = -inf"
    assert (o_g[empty] == 0).all(), "rows with no visible key must have o = 0"
    eo = np.abs(o_g[~empty] - o_ref[~empty])
    el = np.abs(l_g[~empty] - lse_ref[~empty])
    log(f"  {rows.size} rows ({int(empty.sum())} empty): O max {eo.max():.3e} mean {eo.mean():.3e}  LSE max {el.max():.3e}")
    assert eo.max() <= O_MAX_TOL and eo.mean() <= O_MEAN_TOL and el.max() <= LSE_MAX_TOL

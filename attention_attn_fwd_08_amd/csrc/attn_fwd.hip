// attn_fwd.hip -- fused attention forward for gfx950 (MI355X, CDNA4).
//
// O = softmax(scale * Q K^T) V and the per-row log-sum-exp, bf16 in, fp32
// accumulate, following the flash-attention recurrence of the ThunderKittens
// write-up (88811315.cn, "RTX 4090 flash-attention example" and "H100
// FlashAttention-2 forward example"): Q is tiled per workgroup, K and V are
// streamed through LDS tile by tile, and each query keeps a running maximum m
// and normaliser l so the N x N matrix never exists.
//
// Mapping to CDNA4 (not to the examples' warp/warpgroup design):
//   * each wave of 64 lanes owns 32 queries; at d=128 a workgroup is 8 waves
//     (256 queries, one workgroup per CU), at the other head dims 4 waves
//     (128 queries, two or more per CU; one at d=256).  Two waves share each
//     SIMD, so the MFMA pipe of one overlaps the softmax VALU work of the
//     other (d=256: one wave per SIMD, with the O accumulator in AGPRs);
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q^T (held in
//     registers for the whole workgroup) the B operand.  In the 32x32
//     accumulator lane L holds query L%32 and 16 of the 32 keys; lane L^32
//     holds the other 16.  Row max / row sum are in-lane plus one
//     v_permlane32_swap, and the per-query rescale factor is a per-lane scalar;
//   * the probabilities P^T stay in registers: the accumulator of S^T,
//     rounded to bf16, is directly the B operand of O^T += V^T P^T.  The key
//     order inside each 16-key step is permuted the same way in V^T (read with
//     ds_read_b64_tr_b16), which the contraction does not see;
//   * softmax uses exp2 with log2(e) folded into the scale: p = 2^(s*c - m*c)
//     with c = scale*log2(e), and lse = (m*c + log2 l) * ln 2.  The
//     reference maximum m is the first tile's; later tiles are not reduced
//     to their maxima.  O is rescaled only when a tile's probabilities against
//     the stale m grow past 2^64 (seen in the lane's tile sum), which ordinary
//     scores never reach after the first tile;
//   * the 64-key tile loop is software pipelined: while the scores of tile t
//     become probabilities (VALU) the MFMA pipe computes the scores of tile
//     t+1, and O^T += V_t^T P_t^T follows on the MFMA pipe; K therefore runs
//     one tile ahead of V;
//   * K and V tiles stream global -> LDS with buffer loads that write LDS
//     directly (no register staging), double-buffered, with XOR swizzles
//     that make every operand read bank-conflict free;
//   * causal: key tiles past the workgroup's last query are never loaded,
//     and only the tiles on the workgroup's diagonal are masked;
//   * any N: a partial last query tile reads clamped Q rows and stores only
//     rows < N; keys >= N read as zeros and are masked in the last key tile;
//   * general shapes (Nq queries against Nk keys, bottom-right causal mask)
//     and split-KV (key ranges in separate workgroups, fp32 partial results
//     merged by log-sum-exp in attn_merge_kernel) are instances of the same
//     kernel; waves whose queries all lie past Nq only copy and wait;
//   * workgroup ids are remapped so that tiles of one head run on one XCD
//     (workgroups are dispatched round-robin over the 8 XCDs), keeping that
//     head's K/V in the XCD's L2; causal tiles of a head run longest first;
//   * at d=128 and d=256, where one workgroup fills a CU, problems with
//     more query tiles than CUs run one persistent workgroup per CU:
//     it walks its XCD's tiles and issues the next tile's K/V/Q loads before
//     storing the current tile's output, so the CU does not idle between
//     tiles; causal rounds alternate long and short tiles per workgroup.
//     Causal problems at d=32, 64 and 96 with few rounds of workgroups
//     (square, or Nq <= Nk) run persistent too, which evens out a ragged
//     last round.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "attn_fwd.h"
#include "fwd_tile_layout.h"

namespace {

// Waves per workgroup: d=128 runs one 8-wave workgroup per CU (two waves per
// SIMD; each K/V tile is fetched into LDS once per 256 queries); d=32, 64 and
// 96 run 4-wave workgroups, two or more per CU; d=256 runs one 4-wave
// workgroup per CU, one wave per SIMD with the whole register file (its O
// accumulator alone is 128 registers per lane).
template <int D>
struct Launch {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "unsupported head dim");
  static constexpr int kWaves = D == 128 ? 8 : 4;
  static constexpr int kThreads = kWave * kWaves;
  static constexpr int kBlockM = kWaves * kQueriesPerWave;  // queries per workgroup
  static constexpr int kMinBlocks = (D == 128 || D == 256) ? 1 : 2;  // launch-bounds occupancy hint
};
constexpr int kXcds = 8;
// Probabilities are formed against a stale reference maximum for as long as
// a lane's sum over one tile stays at or below this (2^64): each is then at
// most 2^64, which bf16 and the fp32 accumulators hold with their usual
// relative precision (and far from overflow).  Beyond it (or NaN / inf), the
// tile's exact maximum becomes the reference, O and l are rescaled, and the
// tile's probabilities are formed again.
[[maybe_unused]] constexpr float kProbSumCap = 18446744073709551616.0f;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// max / sum of a value held by lanes L and L^32 (the two halves of one query).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Mask of a tile whose keys start at key0 for the queries q0 + L%32: a key is
// visible iff key < N and, when causal, key <= query.
template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int key0, int q0, int N, int l32,
                                          int half) {
  const int last = CAUSAL ? min(q0 + l32, N - 1) : N - 1;  // last visible key
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    int lim = last - key0 - sb * 32 - 4 * half;  // visible iff in-block offset <= lim
    // Opaque to the optimiser: the 16 lane masks below are then formed where
    // they are used, not hoisted out of the tile loops, where they would hold
    // 32 scalar register pairs across the whole loop.
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) > lim) s[sb][r] = -INFINITY;
  }
}

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float m0 = fmaxf(s[0][0], s[0][1]);
  float m1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) {
    m0 = fmaxf(m0, s[0][r]);
    m1 = fmaxf(m1, s[1][r]);
  }
  return pair_max(fmaxf(m0, m1));
}

// N is the number of queries.  GENERAL: the keys number Nk (not N) and a
// causal mask is offset by `off` (key j visible to query i iff j <= i + off);
// rows that see no key get o = 0 and lse = -inf.  Otherwise Nk = N, off = 0
// and every row sees key 0.  SPLIT (implies GENERAL): workgroup row
// blockIdx.y takes only keys [y*kv_chunk, (y+1)*kv_chunk) and writes its
// normalised partial O (fp32) and partial lse to o_part / lse_part, laid out
// [split, head, query, d] and [split, head, query]; a merge kernel combines
// the splits.  PERSIST (not with SPLIT): the grid is one workgroup per
// resident slot and each workgroup walks n_work query tiles' worth of
// logical ids; the next tile's K/V/Q loads are issued before the current
// tile's output is stored, so a tile's start-up overlaps the previous
// tile's epilogue instead of leaving the CU idle between workgroups.
template <int D, bool CAUSAL, bool GENERAL, bool SPLIT = false, bool PERSIST = false>
__global__ __launch_bounds__(Launch<D>::kThreads, Launch<D>::kMinBlocks)  // <= 256 registers
void attn_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, __bf16* __restrict__ o,
                     float* __restrict__ lse, int N, float c, int nk_arg, int off_arg,
                     int kv_chunk, float* __restrict__ o_part, float* __restrict__ lse_part,
                     int n_work) {
  static_assert(!SPLIT || GENERAL, "a split is a general-shape problem");
  static_assert(!PERSIST || !SPLIT, "split workgroups are not persistent");
  const int Nk_all = GENERAL ? nk_arg : N;
  const int kv_begin = SPLIT ? (int)blockIdx.y * kv_chunk : 0;  // first key of this split
  const int Nk = SPLIT ? min(kv_chunk, Nk_all - kv_begin) : Nk_all;
  const int off = GENERAL ? off_arg - kv_begin : 0;
  using T = Tile<D>;
  constexpr int kRowBytes = T::kRowBytes;
  constexpr int kSteps = T::kSteps;
  constexpr int kDBlocks = T::kDBlocks;
  constexpr int kStageBytes = T::kStageBytes;
  constexpr int kWaves = Launch<D>::kWaves;
  constexpr int kBlockM = Launch<D>::kBlockM;
  constexpr int kLoadBytes = kWave * 16;                              // one wave load
  constexpr int kLoadsPerWave = kStageBytes / (kLoadBytes * kWaves);  // per tensor per stage
  static_assert(kStageBytes % (kLoadBytes * kWaves) == 0, "stage must split evenly over the waves");

  // K stages 0,1 then V stages 0,1.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * kStageBytes];
  unsigned char* const k_base = smem;
  unsigned char* const v_base = smem + 2 * kStageBytes;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Workgroup -> logical ids -> (head, query tile).  Workgroups are
  // dispatched round-robin over the XCDs; the remap gives each XCD a
  // contiguous range of logical ids, and consecutive logical ids walk the
  // query tiles of one head, so the workgroups resident on an XCD share one
  // head's K/V in that XCD's L2.  Causal tiles of a head run longest first,
  // so each XCD ends on short ones.  A persistent workgroup (slot j of the
  // S = grid/8 on its XCD) takes, in round r, position j of the r-th run of
  // S ids in its XCD's range; causal rounds alternate with position S-1-j, so
  // a slot's long diagonal tiles pair with short ones.
  const int n_qt = (N + kBlockM - 1) / kBlockM;
  const int grid = gridDim.x;
  int lid = blockIdx.x;
  int lid_begin = 0, lid_end = n_work, slots = grid, slot = lid, round = 0;
  auto lid_at = [&](int r) __attribute__((always_inline)) {
    return lid_begin + r * slots + ((CAUSAL && (r & 1)) ? slots - 1 - slot : slot);
  };
  if constexpr (PERSIST) {
    if (grid % kXcds == 0) {
      const int per_xcd = (n_work + kXcds - 1) / kXcds;
      lid_begin = (lid % kXcds) * per_xcd;
      lid_end = min(n_work, lid_begin + per_xcd);
      slots = grid / kXcds;
      slot = lid / kXcds;
    }
    lid = lid_at(0);
    if (lid >= lid_end) return;  // no tile for this workgroup (uniform)
  } else {
    if (grid % kXcds == 0) lid = (lid % kXcds) * (grid / kXcds) + lid / kXcds;
  }

  // Global -> LDS copy of one K or V tile: lane i of wave load w fills LDS
  // chunk g = 64w + i of the stage from the tile offset k_copy_offset /
  // v_copy_offset (the swizzled layout).  The buffer starts at the tile, so
  // rows past the keys fall outside its size.
  int k_ld_off[kLoadsPerWave], v_ld_off[kLoadsPerWave];
#pragma unroll
  for (int it = 0; it < kLoadsPerWave; ++it) {
    const unsigned g = (wave * kLoadsPerWave + it) * kWave + lane;
    k_ld_off[it] = k_copy_offset<D>(g);
    v_ld_off[it] = v_copy_offset<D>(g);
  }
  const unsigned lds_wave = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)smem +
                            wave * kLoadsPerWave * kLoadBytes;
  auto load_tile = [&](const __bf16* base, const int (&ld_off)[kLoadsPerWave], auto region_tag,
                       int tile, int stage) __attribute__((always_inline)) {
    constexpr unsigned kRegion = decltype(region_tag)::value * 2u * kStageBytes;
    const i32x4 rsrc = make_rsrc(base + (size_t)tile * kBlockN * D, (Nk - tile * kBlockN) * kRowBytes);
    const unsigned dst = lds_wave + stage * kStageBytes;
    static_for<0, kLoadsPerWave>([&](auto it_tag) __attribute__((always_inline)) {
      constexpr int it = decltype(it_tag)::value;
      load16_to_lds<kRegion + it * kLoadBytes>(rsrc, ld_off[it], dst);
    });
  };
  using kRegionK = std::integral_constant<int, 0>;
  using kRegionV = std::integral_constant<int, 1>;

  // Per-lane LDS byte offsets (stage-relative) of the operand reads: K at
  // row L%32, features 16*st + 8*(L/32) ..; V transposed, so that lane L
  // holds the keys of P^T's slots (fwd_tile_layout.h).
  int k_off[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) k_off[st] = k_operand_offset<D>(l32, half, st);
  int v_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) v_off[h] = v_operand_offset<D>(lane, h);

  // Number of key tiles a query tile visits (causal: up to its last query).
  auto tiles_of = [&](int qt) __attribute__((always_inline)) {
    const int kv_end = CAUSAL ? min((qt + 1) * kBlockM + off, Nk) : Nk;
    return (kv_end + kBlockN - 1) / kBlockN;
  };
  // Q^T as MFMA B operand (q_operand): lane L holds query q0+L%32.  Loaded
  // once per query tile.
  bf16x8 qf[kSteps];
  // Start of a query tile: its first K, V and second K tiles go to LDS and
  // its Q to registers.
  auto begin_tile = [&](int lid_t) __attribute__((always_inline)) {
    const int head_t = lid_t / n_qt;
    const int qt_t = CAUSAL ? n_qt - 1 - lid_t % n_qt : lid_t % n_qt;
    const size_t kv_off_t = ((size_t)head_t * Nk_all + kv_begin) * D;
    const int nt = tiles_of(qt_t);
    if (GENERAL && nt <= 0) return;
    load_tile(k + kv_off_t, k_ld_off, kRegionK{}, 0, 0);
    load_tile(v + kv_off_t, v_ld_off, kRegionV{}, 0, 0);
    if (nt > 1) load_tile(k + kv_off_t, k_ld_off, kRegionK{}, 1, 1);
    const int row = min(qt_t * kBlockM + wave * kQueriesPerWave + l32, N - 1);  // rows past N: any valid row
    q_operand<D>(q + (size_t)head_t * N * D + (size_t)row * D, half, qf);
  };
#ifdef ATTN_DEBUG_POISON_LDS
  // Debug build: every LDS byte starts as a NaN pattern, so an operand read
  // of a location no copy has written turns the output into NaN.
  for (int i = tid; i < (int)(sizeof(smem) / 4); i += Launch<D>::kThreads)
    reinterpret_cast<unsigned*>(smem)[i] = 0x7fc07fc0u;
  __syncthreads();
#endif
  begin_tile(lid);

  for (;;) {
    const int head = lid / n_qt;
    const int qt = CAUSAL ? n_qt - 1 - lid % n_qt : lid % n_qt;

    const size_t head_off = (size_t)head * N * D;
    const size_t kv_head_off = ((size_t)head * Nk_all + kv_begin) * D;
    // SPLIT: this row's slot in the partial results.
    const size_t part_row0 = SPLIT ? ((size_t)blockIdx.y * (grid / n_qt) + head) * N : 0;
    const __bf16* const kh = k + kv_head_off;
    const __bf16* const vh = v + kv_head_off;
    const int q0 = qt * kBlockM + wave * kQueriesPerWave;  // this wave's first query

    // Tiles this workgroup visits; tiles from first_mask on are masked:
    // causal, the tiles on the diagonal of at least one of its waves; else
    // only a last tile that runs past N.
    const int n_tiles = tiles_of(qt);
    int first_mask;
    if constexpr (!GENERAL) {
      first_mask = CAUSAL ? qt * (kBlockM / kBlockN) : (N % kBlockN ? n_tiles - 1 : n_tiles);
    } else if constexpr (CAUSAL) {
      // Tiles wholly at or below the workgroup's first query (+ off) need no mask.
      const int first_last_key = qt * kBlockM + off;  // last key its first query sees
      first_mask = first_last_key < 0 ? 0 : min((first_last_key + 1) / kBlockN, n_tiles);
      const int kv_end = min((qt + 1) * kBlockM + off, Nk);
      if (kv_end == Nk && Nk % kBlockN) first_mask = min(first_mask, n_tiles - 1);
    } else {
      first_mask = Nk % kBlockN ? n_tiles - 1 : n_tiles;
    }
    if constexpr (GENERAL) {
      if (n_tiles <= 0) {  // no query of the workgroup sees a key
        const int qrow = q0 + l32;
        if (qrow < N) {
          if constexpr (SPLIT) {
            float* const prow = o_part + (part_row0 + qrow) * D;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(prow + 32 * b + 8 * j + 4 * half) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (half == 0) lse_part[part_row0 + qrow] = -INFINITY;
          } else {
            __bf16* const orow = o + head_off + (size_t)qrow * D;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * j + 4 * half) = bf16x4{0, 0, 0, 0};
            if (half == 0) lse[(size_t)head * N + qrow] = -INFINITY;
          }
        }
        if constexpr (PERSIST) goto next_tile;
        else return;
      }
    }

    {  // the tile's computation (persistent general-shape exits jump past it)
    auto load_k = [&](int tile, int stage) __attribute__((always_inline)) {
      load_tile(kh, k_ld_off, kRegionK{}, tile, stage);
    };
    auto load_v = [&](int tile, int stage) __attribute__((always_inline)) {
      load_tile(vh, v_ld_off, kRegionV{}, tile, stage);
    };

    f32x16 acc[kDBlocks];
#pragma unroll
    for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

    wait_lds_dma<0>();
    __syncthreads();  // K0, V0, K1 have landed

    if constexpr (GENERAL) {
      // A wave whose 32 queries all lie past the last query (a short query
      // block, e.g. decoding) computes nothing; it still issues its share of
      // the copies and meets every barrier the tile loop below does.
      if (q0 >= N) {
        for (int t = 0; t < n_tiles; ++t) {
          wait_lds_dma<0>();
          __syncthreads();
          if (t + 2 < n_tiles) load_k(t + 2, t & 1);
          if (t + 1 < n_tiles) load_v(t + 1, (t + 1) & 1);
        }
        if constexpr (PERSIST) goto next_tile;
        else return;
      }
    }

    // Prologue: scores of tile 0 and the reference maximum, tile 0's (finite
    // for every query in the square case, where tile 0 holds key 0).
    f32x16 s_a[2], s_b[2];
    scores<D>(k_base, k_off, qf, s_a);
    if (first_mask == 0) mask_tile<CAUSAL>(s_a, 0, q0 + off, Nk, l32, half);
    float m_ref = tile_max(s_a);  // reference maximum (raw score units), query q0+L%32
    float l_run = 0.f;            // this lane's half of the normaliser

    // One tile: s_cur holds tile t's (masked) scores, s_next receives tile
    // t+1's.  HAS_NEXT and MASK_NEXT are compile-time so the body is straight
    // line code the scheduler can interleave (MFMA of one phase against VALU).
    // A 32-key block is live for this wave iff its first key is visible to at
    // least one of the wave's queries; dead blocks (above the diagonal, or past
    // N) skip their MFMAs and exponentials.  Only the steps that can meet one
    // (masked successor, or the last tile) test this.
    const int wave_last_key = CAUSAL ? min(q0 + kQueriesPerWave - 1 + off, Nk - 1) : Nk - 1;
    auto live = [&](int tile, int sb) __attribute__((always_inline)) {
      return tile * kBlockN + sb * 32 <= wave_last_key;
    };
    auto step = [&](auto has_next_tag, auto mask_next_tag, int t, f32x16(&s_cur)[2],
                    f32x16(&s_next)[2]) __attribute__((always_inline)) {
      constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
      constexpr bool MASK_NEXT = decltype(mask_next_tag)::value;
      constexpr bool CHECK = MASK_NEXT || !HAS_NEXT;  // may meet dead blocks
      wait_lds_dma<0>();
      __syncthreads();  // K_{t+1} and V_t have landed; K_t and V_{t-1} are free
      if (t + 2 < n_tiles) load_k(t + 2, t & 1);
      if (HAS_NEXT) load_v(t + 1, (t + 1) & 1);

      // Phase A: probabilities of tile t (VALU) while S_{t+1} runs on MFMA.
      // The wave runs this phase at raised issue priority: where the two waves
      // of a SIMD contend, the one interleaving score MFMAs with the softmax
      // goes first (measured 2-3 % faster than equal priorities).
      __builtin_amdgcn_s_setprio(1);
      if constexpr (HAS_NEXT) {
        const unsigned char* const k_lds = k_base + ((t + 1) & 1) * kStageBytes;
        if constexpr (CHECK) {
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            if (live(t + 1, sb)) {
              scores_block<D>(k_lds, sb, k_off, qf, s_next[sb]);
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) s_next[sb][r] = -INFINITY;
            }
          }
        } else {
          scores<D>(k_lds, k_off, qf, s_next);
        }
      }
      // A row that has seen no key yet has m_ref = -inf and only -inf scores.
      float mc = (GENERAL && m_ref == -INFINITY) ? 0.f : m_ref * c;
      bf16x8 pb[2][2];
      float l_tile = 0.f;
      auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          if (CHECK && !live(t, sb)) continue;  // its probabilities are all 0
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              p[j] = __builtin_amdgcn_exp2f(fmaf(s_cur[sb][8 * cc + j], c, -mc));
              pb[sb][cc][j] = (__bf16)p[j];
            }
            l_tile += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          }
        }
      };
      probs();
      // The bf16 probabilities are formed here, before the rescale test, so
      // their conversions interleave with the exponentials instead of
      // waiting for the branch (measured 1 % faster at d=128, 1.6 % at d=64;
      // the common path's results are unchanged).
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) asm volatile("" : "+v"(pb[sb][cc]));
      // Lazy rescale, checked on the probabilities themselves (the lane's tile
      // sum; NaN and inf fail the test too).  Rare: the tile's exact maximum
      // becomes the reference (lanes L and L^32 agree on it), O and l are
      // rescaled and the probabilities formed again.  A row that has seen no
      // key until now (m = -inf, general shapes) takes its first finite m here.
#ifdef ATTN_DEBUG_FORCE_RESCALE
      const bool redo = true;  // debug build: every tile takes the rescale branch
#else
      bool redo = !(l_tile <= kProbSumCap);
      if constexpr (GENERAL) redo = redo || (m_ref == -INFINITY && l_tile > 0.f);
#endif
      if (__builtin_amdgcn_ballot_w64(redo)) {
        const float m_new = fmaxf(m_ref, tile_max(s_cur));
        // A lane whose row has seen no key keeps m = -inf (its O and l are 0
        // and stay 0): its factor is 1, not exp2(-inf - -inf) = NaN.
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
        m_ref = m_new;
        mc = (GENERAL && m_ref == -INFINITY) ? 0.f : m_ref * c;
        l_tile = 0.f;
        probs();
      }
      l_run += l_tile;

      __builtin_amdgcn_s_setprio(0);

      // Phase B: O^T += V_t^T P_t^T on MFMA (and the mask of tile t+1 when it needs one).
      const unsigned char* const v_lds = v_base + (t & 1) * kStageBytes;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (CHECK && !live(t, sb)) continue;
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const bf16x8 vf = v_operand<D>(v_lds + (sb * 32 + cc * 16) * kRowBytes, v_off, b);
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[sb][cc], acc[b], 0, 0, 0);
          }
      }
      if constexpr (HAS_NEXT) {
        if constexpr (MASK_NEXT) mask_tile<CAUSAL>(s_next, (t + 1) * kBlockN, q0 + off, Nk, l32, half);
      }
    };
    using yes = std::true_type;
    using no = std::false_type;
    auto copy_scores = [](f32x16(&dst)[2], const f32x16(&src)[2]) __attribute__((always_inline)) {
      dst[0] = src[0];
      dst[1] = src[1];
    };

    // Steps whose successor tile needs no mask run in pairs, so the two score
    // buffers alternate without copies; the steps from first_mask-1 on mask
    // their successor.
    const int n_plain = first_mask - 1 > 0 ? first_mask - 1 : 0;
    int t = 0;
    for (; t + 1 < n_plain; t += 2) {
      step(yes{}, no{}, t, s_a, s_b);
      step(yes{}, no{}, t + 1, s_b, s_a);
    }
    if (t < n_plain) {
      step(yes{}, no{}, t, s_a, s_b);
      copy_scores(s_a, s_b);
      ++t;
    }
    for (; t + 1 < n_tiles; ++t) {
      step(yes{}, yes{}, t, s_a, s_b);
      copy_scores(s_a, s_b);
    }
    step(no{}, no{}, t, s_a, s_b);  // the last tile has no successor

    // Epilogue: O = acc / l, rounded to bf16; lse = (m*c + log2 l) * ln 2.
    const float l_tot = pair_sum(l_run);
    const float inv = (GENERAL && l_tot == 0.f) ? 0.f : 1.0f / l_tot;
    const float row_lse = (GENERAL && l_tot == 0.f) ? -INFINITY : (m_ref * c + log2f(l_tot)) * kLn2;
    const int next = PERSIST ? lid_at(round + 1) : lid_end;  // ids only grow with the round
    if constexpr (PERSIST) {
      if (next < lid_end) {
        __syncthreads();  // every wave is done reading this tile's LDS stages
        begin_tile(next);
      }
    }
    if (q0 + l32 < N) {  // a partial last query tile stores only rows < N
      if constexpr (SPLIT) {
        float* const prow = o_part + (part_row0 + q0 + l32) * D;
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4*>(prow + 32 * b + 8 * j + 4 * half) =
                f32x4{acc[b][4 * j] * inv, acc[b][4 * j + 1] * inv, acc[b][4 * j + 2] * inv,
                      acc[b][4 * j + 3] * inv};
        if (half == 0) lse_part[part_row0 + q0 + l32] = row_lse;
      } else {
        __bf16* const orow = o + head_off + (size_t)(q0 + l32) * D;
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x4 ov;
#pragma unroll
            for (int r = 0; r < 4; ++r) ov[r] = (__bf16)(acc[b][4 * j + r] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * j + 4 * half) = ov;
          }
        }
        if (half == 0) lse[(size_t)head * N + q0 + l32] = row_lse;
      }
    }
    if (!PERSIST || next >= lid_end) return;
    lid = next;
    ++round;
    continue;
    }
  next_tile: __attribute__((unused));
    // A persistent workgroup that computed nothing for this tile (general
    // shapes: no query sees a key, or waves past the last query) goes on to
    // the next tile with the same barrier as the others.
    if constexpr (PERSIST) {
      const int nxt = lid_at(round + 1);
      if (nxt >= lid_end) return;
      __syncthreads();  // every wave is done reading this tile's LDS stages
      begin_tile(nxt);
      lid = nxt;
      ++round;
    }
  }
}

// Merge of the splits of one row: lse = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s (rows no split sees: O = 0, lse = -inf).
// D/4 threads per row, four features each.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         __bf16* __restrict__ o,
                                                         float* __restrict__ lse, long long rows,
                                                         int n_splits) {
  constexpr int kPerRow = D / 4;
  constexpr int kRowsPerBlock = 256 / kPerRow;
  if (threadIdx.x >= kRowsPerBlock * kPerRow) return;  // d=96: 240 of the 256 threads
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kPerRow;
  const int f = (threadIdx.x % kPerRow) * 4;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < n_splits; ++s) m = fmaxf(m, lse_part[(size_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float w = __expf(lse_part[(size_t)s * rows + row] - m);
      const f32x4 x = *reinterpret_cast<const f32x4*>(o_part + ((size_t)s * rows + row) * D + f);
      acc += w * x;
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  bf16x4 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) out[r] = (__bf16)(acc[r] * inv);
  *reinterpret_cast<bf16x4*>(o + row * D + f) = out;
  if (f == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool gfx950 = false;
  int n_cu = 0;  // compute units
};

std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

const DeviceInfo* device_info(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      g_info[dev].gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      g_info[dev].n_cu = prop.multiProcessorCount;
    }
  });
  return &g_info[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups of the persistent kernel that fit on the GPU at
// once (resident per CU, from the occupancy query, times the CU count);
// cached per device.  0 if unknown.
template <int D, bool CAUSAL, bool GENERAL>
int persistent_grid(int dev, int n_cu) {
  static std::once_flag once[kMaxDevices];
  static int per_cu[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices || n_cu <= 0) return 0;
  std::call_once(once[dev], [dev] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &b, attn_fwd_kernel<D, CAUSAL, GENERAL, false, true>, Launch<D>::kThreads, 0) != hipSuccess)
      b = 0;
    per_cu[dev] = b;
  });
  return per_cu[dev] * n_cu;
}

template <int D, bool CAUSAL, bool GENERAL>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Nq, int Nk,
           int off, float c, int dev, int n_cu, hipStream_t stream) {
  const int n_qt = (Nq + Launch<D>::kBlockM - 1) / Launch<D>::kBlockM;
  const int n_work = n_qt * BH;
  // Problems with more query tiles than fit on the GPU at once, at the
  // head dims that run one workgroup per CU: one persistent workgroup per CU,
  // so a CU is not idle while one workgroup drains and the next starts.
  // Where several workgroups share a CU (d = 32, 64, 96) they already cover
  // each other's start-up, and the persistent form measured no better on
  // problems without a mask.  Causal problems with few rounds of workgroups
  // (query tiles over resident slots) are the exception: their tiles of
  // unequal length leave a ragged last round, which the persistent schedule
  // (long and short tiles paired per slot) evens out.  Measured (same box,
  // always persistent against never), square: d=32 +9 to +29 % at 1.5-3
  // rounds, +1 % at 4, -2 % at 8; d=64 +1 to +12 % at 2.7-4 rounds, -1.5 % at
  // 1.3 and 5.3; d=96 +4 to +29 % at 1.5-8 rounds, +0.2 % at 16.  General
  // shapes with Nq <= Nk (queries at the end of a longer key range): +3 to
  // +11 % at 2-2.7 rounds, +1 % at 4; with Nq > Nk -6 %, so not there.
  if constexpr (D == 128 || D == 256 || CAUSAL) {
    const int grid = persistent_grid<D, CAUSAL, GENERAL>(dev, n_cu);
    bool persist = grid > 0 && n_work > grid;
    if constexpr (GENERAL && D != 128 && D != 256) persist = persist && Nq <= Nk;
    if constexpr (D == 32) persist = persist && n_work <= 4 * grid;
    if constexpr (D == 64) persist = persist && n_work > 2 * grid && n_work <= 4 * grid;
    if constexpr (D == 96) persist = persist && n_work <= 8 * grid;
    if (persist) {
      hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, GENERAL, false, true>), dim3(grid),
                         dim3(Launch<D>::kThreads), 0, stream, static_cast<const __bf16*>(q),
                         static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                         static_cast<__bf16*>(o), lse, Nq, c, Nk, off, 0, nullptr, nullptr, n_work);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, GENERAL>), dim3(n_work), dim3(Launch<D>::kThreads), 0,
                     stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, Nq, c, Nk, off, 0,
                     nullptr, nullptr, n_work);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <int D, bool CAUSAL>
int launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Nq,
                 int Nk, int off, float c, int n_splits, int chunk, float* o_part, float* lse_part,
                 hipStream_t stream) {
  const int n_qt = (Nq + Launch<D>::kBlockM - 1) / Launch<D>::kBlockM;
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, true, true>), dim3(n_qt * BH, n_splits),
                     dim3(Launch<D>::kThreads), 0, stream, static_cast<const __bf16*>(q),
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                     static_cast<__bf16*>(o), lse, Nq, c, Nk, off, chunk, o_part, lse_part, n_qt * BH);
  const long long rows = (long long)BH * Nq;
  constexpr int kRowsPerBlock = 256 / (D / 4);
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, stream, o_part, lse_part, static_cast<__bf16*>(o), lse, rows,
                     n_splits);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <bool GENERAL>
int dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Nq,
             int Nk, int d, int causal, float scale, hipStream_t s) {
  const float c = scale * kLog2e;
  const int off = causal ? Nk - Nq : 0;
  int dev = 0;
  const DeviceInfo* info = hipGetDevice(&dev) == hipSuccess ? device_info(dev) : nullptr;
  const int n_cu = info ? info->n_cu : 0;
  auto go = [&](auto d_tag) {
    constexpr int D = decltype(d_tag)::value;
    return causal ? launch<D, true, GENERAL>(q, k, v, o, lse, BH, Nq, Nk, off, c, dev, n_cu, s)
                  : launch<D, false, GENERAL>(q, k, v, o, lse, BH, Nq, Nk, off, c, dev, n_cu, s);
  };
  switch (d) {
    case 32: return go(std::integral_constant<int, 32>{});
    case 64: return go(std::integral_constant<int, 64>{});
    case 96: return go(std::integral_constant<int, 96>{});
    case 128: return go(std::integral_constant<int, 128>{});
    default: return go(std::integral_constant<int, 256>{});
  }
}

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }

// Argument checks shared by the entry points (before any HIP call).
int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, bool* nothing) {
  *nothing = false;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (!head_dim_ok(d)) return ATTN_ERR_HEAD_DIM;
  if (!(scale > 0.0f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT32_MAX) return ATTN_ERR_SHAPE;
  if (bh * (((int64_t)Nq + 127) / 128) > INT32_MAX) return ATTN_ERR_SHAPE;  // grid (any d)
  if ((int64_t)Nq * d * 2 > INT32_MAX || (int64_t)Nk * d * 2 > INT32_MAX)
    return ATTN_ERR_SHAPE;  // one head's bytes fit an int
  if (bh == 0 || Nq == 0) {
    *nothing = true;
    return ATTN_OK;
  }
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return ATTN_ERR_NULL;  // k, v unread if Nk = 0
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  const DeviceInfo* info = device_info(dev);
  if (!info || !info->gfx950) return ATTN_ERR_DEVICE;
  return ATTN_OK;
}

// The split-KV forward with its partial results in o_part / lse_part
// (caller workspace, or the fixed device workspace below); `used` ranges of
// `chunk` keys, computed by the caller from the request.
int splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
            int Nk, int d, int causal, float scale, int used, int chunk, float* o_part,
            float* lse_part, hipStream_t s) {
  if (used <= 1)  // nothing to split (or no key at all)
    return dispatch<true>(q, k, v, o, lse, B * H, Nq, Nk, d, causal, scale, s);
  const float c = scale * kLog2e;
  const int off = causal ? Nk - Nq : 0;
  const int BH = B * H;
  auto go = [&](auto d_tag) {
    constexpr int D = decltype(d_tag)::value;
    return causal
               ? launch_split<D, true>(q, k, v, o, lse, BH, Nq, Nk, off, c, used, chunk, o_part, lse_part, s)
               : launch_split<D, false>(q, k, v, o, lse, BH, Nq, Nk, off, c, used, chunk, o_part, lse_part, s);
  };
  switch (d) {
    case 32: return go(std::integral_constant<int, 32>{});
    case 64: return go(std::integral_constant<int, 64>{});
    case 96: return go(std::integral_constant<int, 96>{});
    case 128: return go(std::integral_constant<int, 128>{});
    default: return go(std::integral_constant<int, 256>{});
  }
}

// Split-KV argument checks shared by both split entry points (before any HIP
// call): ranges of whole 64-key tiles, `used` of them.
int check_split(int B, int H, int Nq, int Nk, int d, int n_splits, int* chunk, int* used) {
  if (n_splits < 1) return ATTN_ERR_SHAPE;
  const int64_t chunk64 = ((int64_t)Nk + n_splits - 1) / n_splits;
  *chunk = (int)(((chunk64 + 63) / 64) * 64);
  *used = Nk > 0 ? (int)(((int64_t)Nk + *chunk - 1) / *chunk) : 0;
  if (*used > 65535) return ATTN_ERR_SHAPE;
  if ((int64_t)*used * B * H * Nq * d > ((int64_t)1 << 40)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

constexpr size_t kScratchBytes = size_t(32) << 20;

}  // namespace

// Fixed device workspace of attn_fwd_splitkv_noalloc: the fp32 partial O of
// every split, then (from a 256-byte boundary) the partial LSE.  One copy per
// GPU, for the life of the process.  Host code never passes this symbol to a
// kernel (on the host it names a stand-in, not device memory): it uses the
// device address looked up once per device by scratch_on().
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (the current device), or null
// if the runtime cannot give it.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) ptr = nullptr;
    g_scratch_ptr[dev] = ptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, int causal, float scale, void* stream) {
  bool nothing = false;
  int st = check_args(q, k, v, o, lse, B, H, N, N, d, scale, &nothing);
  if (st != ATTN_OK || nothing) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  return dispatch<false>(q, k, v, o, lse, B * H, N, N, d, causal, scale,
                         static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int Nq, int Nk, int d, int causal, float scale, void* stream) {
  bool nothing = false;
  int st = check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, &nothing);
  if (st != ATTN_OK || nothing) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Nq == Nk) return dispatch<false>(q, k, v, o, lse, B * H, Nq, Nk, d, causal, scale, s);
  return dispatch<true>(q, k, v, o, lse, B * H, Nq, Nk, d, causal, scale, s);
}

extern "C" int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Nq, int Nk, int d, int causal, float scale,
                                int n_splits, float* o_part, float* lse_part, void* stream) {
  bool nothing = false;
  int st = check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, &nothing);
  if (st != ATTN_OK) return st;
  int chunk = 0, used = 0;
  if ((st = check_split(B, H, Nq, Nk, d, n_splits, &chunk, &used)) != ATTN_OK) return st;
  if (nothing) return ATTN_OK;
  if (used > 1 && (!o_part || !lse_part)) return ATTN_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(lse_part)) return ATTN_ERR_ALIGN;
  if ((st = check_device()) != ATTN_OK) return st;
  return splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, used, chunk, o_part, lse_part,
                 static_cast<hipStream_t>(stream));
}

extern "C" int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int B, int H, int Nq, int Nk, int d,
                                        int causal, float scale, int n_splits, void* stream) {
  bool nothing = false;
  int st = check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, &nothing);
  if (st != ATTN_OK) return st;
  int chunk = 0, used = 0;
  if ((st = check_split(B, H, Nq, Nk, d, n_splits, &chunk, &used)) != ATTN_OK) return st;
  if (nothing) return ATTN_OK;
  // Partial O, then the partial LSE from a 256-byte boundary, in the fixed workspace.
  const size_t rows = (size_t)used * B * H * Nq;
  const size_t o_bytes = (rows * d * sizeof(float) + 255) & ~(size_t)255;
  if (used > 1 && o_bytes + rows * sizeof(float) > kScratchBytes) return ATTN_ERR_WORKSPACE;
  if ((st = check_device()) != ATTN_OK) return st;
  float* o_part = nullptr;
  float* lse_part = nullptr;
  if (used > 1) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
    unsigned char* base = static_cast<unsigned char*>(scratch_on(dev));
    if (!base) return ATTN_ERR_HIP;
    o_part = reinterpret_cast<float*>(base);
    lse_part = reinterpret_cast<float*>(base + o_bytes);
  }
  return splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, used, chunk, o_part, lse_part,
                 static_cast<hipStream_t>(stream));
}

extern "C" const char* attn_fwd_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or N is negative, or the problem size overflows";
    case ATTN_ERR_HEAD_DIM: return "head dimension d must be 32, 64, 96, 128 or 256";
    case ATTN_ERR_SEQ_MULTIPLE: return "reserved (any sequence length is accepted)";
    case ATTN_ERR_ALIGN: return "q, k, v, o and lse must be 16-byte aligned";
    case ATTN_ERR_SCALE: return "scale must be finite and greater than 0";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error";
    case ATTN_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
    case ATTN_ERR_WORKSPACE: return "the partial results exceed the library's fixed 32 MiB workspace";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_abi_version(void) { return 4; }

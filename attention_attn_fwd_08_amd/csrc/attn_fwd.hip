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
//   * one workgroup = 4 waves of 64 lanes; each wave owns 32 queries;
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q^T (held in
//     registers for the whole tile) the B operand.  In the 32x32 accumulator
//     lane L holds query L%32 and 16 of the 32 keys; lane L^32 holds the other
//     16.  Row max / row sum are therefore in-lane plus one exchange with
//     lane L^32, and the per-query rescale factor is a per-lane scalar;
//   * the probabilities P^T stay in registers: the accumulator of S^T,
//     rounded to bf16, is directly the B operand of O^T += V^T P^T.  The key
//     order inside each 16-key step is permuted the same way in V^T, which the
//     contraction does not see;
//   * softmax uses exp2 with log2(e) folded into the scale: p = 2^(s*c - m*c)
//     with c = scale*log2(e), and lse = (m*c + log2 l) * ln 2;
//   * K and V tiles move global -> LDS as 16-byte loads with an XOR-swizzled
//     row layout so the 32 rows an MFMA operand read touches fall in distinct
//     banks;
//   * causal: key tiles past the workgroup's last query are never loaded,
//     score blocks past a wave's last query are skipped, and only blocks on the
//     diagonal are masked;
//   * workgroup ids are remapped so that tiles of one head run on one XCD
//     (workgroups are dispatched round-robin over the 8 XCDs), keeping that
//     head's K/V in the XCD's L2; causal tiles of a head run longest first.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "attn_fwd.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kQueriesPerWave = 32;
constexpr int kBlockM = kWaves * kQueriesPerWave;  // queries per workgroup
constexpr int kBlockN = 64;                        // keys per LDS stage
constexpr int kSeqMultiple = kBlockM;
constexpr int kXcds = 8;
// O is rescaled only when a query's block maximum exceeds the reference
// maximum by more than this many powers of two; until then probabilities are
// formed against the stale reference (they stay <= 2^8, exact to rescale).
constexpr float kRescaleLog2 = 8.0f;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// LDS layouts.  A K or V stage is kBlockN rows of D bf16 (D*2 bytes), the
// 16-byte chunks of each row permuted by an XOR with a function of the row.
//
// K is read as the MFMA A operand: 32 lanes read the same chunk of 32
// consecutive rows (16 bytes each).  XOR with row%16 (d=128) spreads any 16
// consecutive rows over all 16 chunk positions of a 256-byte bank sweep.  For
// d=64 a row is 128 bytes; the extra (row>>3)&1 term separates rows r and r+8.
//
// V is read with ds_read_b64_tr_b16: each 16-lane group reads 4 consecutive
// rows x 32 contiguous bytes (a chunk pair).  The V function moves the chunk
// pair of those 4 rows to 4 different places, and is still a permutation of
// the chunks of any 16 consecutive rows.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row & 7) ^ ((row >> 3) & 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  if constexpr (D == 128) return 2 * (row & 3) + 8 * ((row >> 2) & 1) + ((row >> 3) & 1);
  else return 2 * (row & 3) + ((row >> 2) & 1);
}

// 16 bytes global -> LDS without passing through registers: lane i of the
// wave writes bytes [16i, 16i+16) after the wave-uniform LDS address `dst`.
// (Only the device pass sees the builtin; the host pass, which compiles just
// the launch stub, drops a kernel template that names it.)
__device__ __forceinline__ void load16_to_lds(const void* src, unsigned char* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
#endif
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2)  // two waves per SIMD: <= 256 registers each
void attn_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, __bf16* __restrict__ o,
                     float* __restrict__ lse, int N, float c) {
  constexpr int kRowBytes = D * 2;
  constexpr int kChunksPerRow = D / 8;
  constexpr int kSteps = D / 16;                 // MFMA k-steps of one score block
  constexpr int kDBlocks = D / 32;               // 32-row blocks of O^T
  constexpr int kStageBytes = kBlockN * kRowBytes;
  constexpr int kRowsPerLoad = kWave * 16 / kRowBytes;            // rows one wave load fills
  constexpr int kLoadsPerWave = kBlockN / (kRowsPerLoad * kWaves);  // per tensor per stage

  // [stage][K | V][kBlockN rows]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Workgroup -> (head, query tile).  Workgroups are dispatched round-robin
  // over the XCDs; the remap gives each XCD a contiguous range of logical ids,
  // and consecutive logical ids walk the query tiles of one head, so the
  // workgroups resident on an XCD share one head's K/V in that XCD's L2.
  // Causal tiles of a head run longest first, so each XCD ends on short ones.
  const int n_qt = N / kBlockM;
  const int grid = gridDim.x;
  int lid = blockIdx.x;
  if (grid % kXcds == 0) lid = (lid % kXcds) * (grid / kXcds) + lid / kXcds;
  const int head = lid / n_qt;
  const int qt = CAUSAL ? n_qt - 1 - lid % n_qt : lid % n_qt;

  const size_t head_off = (size_t)head * N * D;
  const __bf16* const qh = q + head_off;
  const __bf16* const kh = k + head_off;
  const __bf16* const vh = v + head_off;
  const int q0 = qt * kBlockM + wave * kQueriesPerWave;  // this wave's first query

  // Global -> LDS copy of one K and one V stage.  Lane i of a wave load fills
  // bytes [16i, 16i+16) after the wave's base: row base+i/kChunksPerRow,
  // physical chunk i%kChunksPerRow, which holds logical chunk (that ^ swz).
  const int ld_row = lane / kChunksPerRow;
  const int ld_chunk = lane % kChunksPerRow;
  auto load_stage = [&](int kt0, int stage) {
#pragma unroll
    for (int it = 0; it < kLoadsPerWave; ++it) {
      const int row0 = (wave * kLoadsPerWave + it) * kRowsPerLoad;
      const int row = row0 + ld_row;
      const size_t g = (size_t)(kt0 + row) * D;
      unsigned char* kdst = smem + (2 * stage) * kStageBytes + row0 * kRowBytes;
      unsigned char* vdst = smem + (2 * stage + 1) * kStageBytes + row0 * kRowBytes;
      load16_to_lds(kh + g + (ld_chunk ^ k_swz<D>(row)) * 8, kdst);
      load16_to_lds(vh + g + (ld_chunk ^ v_swz<D>(row)) * 8, vdst);
    }
  };

  const int n_tiles = (CAUSAL ? (qt + 1) * kBlockM : N) / kBlockN;
  load_stage(0, 0);

  // Q^T as MFMA B operand: lane L holds query q0+L%32, features 8*(L/32)..+7
  // of each 16-feature step.  Loaded once per tile.
  bf16x8 qf[kSteps];
  {
    const __bf16* qrow = qh + (size_t)(q0 + l32) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
  }

  // Per-lane LDS byte offsets (stage-relative) of the MFMA operand reads.
  // K: row sb*32 + L%32, logical chunk 2*st + L/32.
  // V (transposed reads): 16-lane group G = L/16 and s = L%16 read row
  // 16*cc + 4*(G/2) + s/4 (+8 for the second read) and features
  // 32*b + 16*(G%2) + 4*(s%4) .. +3; lane L then holds feature 32*b + L%32 of
  // keys 16cc + 4*(L/32) + 0..3 (first read) and 16cc + 8 + 4*(L/32) + 0..3
  // (second read): the order the P^T registers use.
  const int g16 = lane >> 4;
  const int s16 = lane & 15;
  const int v_row = 4 * (g16 >> 1) + (s16 >> 2);  // < 8; the second read adds 8
  const int v_col = 16 * (g16 & 1) + 4 * (s16 & 3);

  f32x16 acc[kDBlocks];
#pragma unroll
  for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum (raw score units) for query q0+L%32
  float l_run = 0.f;        // this lane's half of the normaliser

  for (int t = 0; t < n_tiles; ++t) {
    const int stage = t & 1;
    const int kt0 = t * kBlockN;
    __syncthreads();  // stage `stage` has landed; stage^1 is free again
    if (t + 1 < n_tiles) load_stage(kt0 + kBlockN, stage ^ 1);
    const unsigned char* const k_lds = smem + (2 * stage) * kStageBytes;
    const unsigned char* const v_lds = smem + (2 * stage + 1) * kStageBytes;

#pragma unroll
    for (int sb = 0; sb < kBlockN / 32; ++sb) {
      const int key0 = kt0 + sb * 32;
      if (CAUSAL && key0 > q0 + kQueriesPerWave - 1) continue;  // wave-uniform

      // S^T block: 32 keys x 32 queries.
      f32x16 s = {};
      {
        const int row = sb * 32 + l32;
        const unsigned char* krow = k_lds + row * kRowBytes;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              krow + (((2 * st + half) ^ k_swz<D>(row)) << 4));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s, 0, 0, 0);
        }
      }

      // Accumulator layout: register r of lane L is key 8*(r/4) + 4*(L/32) + r%4
      // of the block, query L%32.
      if (CAUSAL && key0 == q0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = 8 * (r >> 2) + 4 * half + (r & 3);
          if (kj > l32) s[r] = -INFINITY;
        }
      }

      float mx = fmaxf(s[0], s[1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // Lanes L and L^32 hold the same query and agree on every value below.
      // The first block a wave sees holds key 0, so mx is finite there and
      // m_ref becomes finite at once.
      const bool grow = (mx - m_ref) * c > kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform, rare after the first block
        const float m_new = grow ? mx : m_ref;
        const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
        m_ref = m_new;
      }
      const float mc = m_ref * c;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -mc));
        l_run += p[r];
      }

      // P^T as B operand: 16-key step cc uses registers 8cc..8cc+7, i.e. keys
      // 16cc + 8*(j/4) + 4*(L/32) + j%4 for slot j.
      bf16x8 pb[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[cc][j] = (__bf16)p[8 * cc + j];

      // V^T as A operand with the same key order, via transposed LDS reads.
#pragma unroll
      for (int b = 0; b < kDBlocks; ++b) {
        const int col = 32 * b + v_col;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int r1 = sb * 32 + 16 * cc + v_row;
          const int r2 = r1 + 8;
          const unsigned char* a1 =
              v_lds + r1 * kRowBytes + (((col >> 3) ^ v_swz<D>(r1)) << 4) + (col & 7) * 2;
          const unsigned char* a2 =
              v_lds + r2 * kRowBytes + (((col >> 3) ^ v_swz<D>(r2)) << 4) + (col & 7) * 2;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a1);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a2);
          const bf16x4 lob = __builtin_bit_cast(bf16x4, lo);
          const bf16x4 hib = __builtin_bit_cast(bf16x4, hi);
          const bf16x8 vf = {lob[0], lob[1], lob[2], lob[3], hib[0], hib[1], hib[2], hib[3]};
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[cc], acc[b], 0, 0, 0);
        }
      }
    }
  }

  // Epilogue: O = acc / l, rounded to bf16; lse = (m*c + log2 l) * ln 2.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
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
  if (half == 0) lse[(size_t)head * N + q0 + l32] = (m_ref * c + log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool gfx950 = false;
};

std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

const DeviceInfo* device_info(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
      g_info[dev].gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  return &g_info[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int D, bool CAUSAL>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
           float c, hipStream_t stream) {
  const int n_qt = N / kBlockM;
  const int grid = n_qt * BH;
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, N, c);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, int causal, float scale, void* stream) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!(scale > 0.0f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  if (N % kSeqMultiple != 0) return ATTN_ERR_SEQ_MULTIPLE;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT32_MAX) return ATTN_ERR_SHAPE;
  if (bh * (N / kBlockM) > INT32_MAX) return ATTN_ERR_SHAPE;  // grid size
  if ((int64_t)N * d > INT32_MAX) return ATTN_ERR_SHAPE;
  if (bh == 0 || N == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  const DeviceInfo* info = device_info(dev);
  if (!info || !info->gfx950) return ATTN_ERR_DEVICE;

  const float c = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = static_cast<int>(bh);
  if (d == 64) {
    return causal ? launch<64, true>(q, k, v, o, lse, BH, N, c, s)
                  : launch<64, false>(q, k, v, o, lse, BH, N, c, s);
  }
  return causal ? launch<128, true>(q, k, v, o, lse, BH, N, c, s)
                : launch<128, false>(q, k, v, o, lse, BH, N, c, s);
}

extern "C" const char* attn_fwd_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or N is negative, or the problem size overflows";
    case ATTN_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case ATTN_ERR_SEQ_MULTIPLE: return "sequence length N must be a multiple of 128";
    case ATTN_ERR_ALIGN: return "q, k, v, o and lse must be 16-byte aligned";
    case ATTN_ERR_SCALE: return "scale must be finite and greater than 0";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error";
    case ATTN_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
    default: return "unknown status";
  }
}

extern "C" int attn_fwd_abi_version(void) { return 1; }

// attn_bwd.hip -- attention backward for gfx950 (MI355X, CDNA4).
//
// The derivative of O = softmax(scale * Q K^T) V (ThunderKittens write-ups,
// flash-attention forward examples; the backward is named there, not
// listed), computed the flash-attention way: the N x N matrices are never
// stored; P is recomputed tile by tile from Q, K and the forward's LSE.
// Three kernels on one stream:
//   1. delta_i = rowsum(dO_i * O_i)                     (memory bound)
//   2. per 128-key block: dV^T += dO^T P and dK^T += Q^T dS while Q and dO
//      stream through LDS (S = Q K^T, dP = dO V^T, dS = P o (dP - delta));
//      at d=128 and d=256 dV and dK are computed by separate waves (d=128:
//      the two groups of one 8-wave workgroup sharing the streamed tiles on
//      problems that fill the GPU; d=256: two workgroups per key block, one
//      per CU, one wave per SIMD)
//   3. per 128-query block: dQ^T += K^T dS^T while K and V stream through
//      LDS (S^T = K Q^T, dP^T = V dO^T)
// Mapping to CDNA4, as in the forward kernel: v_mfma_f32_32x32x16_bf16 with
// the operand held for the whole workgroup (K and V in kernel 2, Q and dO in
// kernel 3) in registers as the B operand, the streamed tile read from LDS as
// the A operand, and the accumulator of one product reused in registers as
// the B operand of the next (its 32-element column order is permuted the
// same way in the transposed LDS reads, which the contraction does not see).
// Tiles read both row-wise (ds_read_b128) and transposed
// (ds_read_b64_tr_b16) use one XOR swizzle that is conflict-free for both.

#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "attn_bwd.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr int kRows = 32;    // keys (kernel 2) or queries (kernel 3) per wave
constexpr int kWaves = 4;    // waves per workgroup, one per SIMD
constexpr int kBlock = kWaves * kRows;  // keys or queries per workgroup
constexpr int kTile = 64;    // rows of a streamed LDS tile
// Workgroups per CU the kernels are compiled for: two (two waves per SIMD,
// 256 registers each) up to d=128; one at d=256, where a wave's operands and
// accumulators need the SIMD's whole register file (512 per lane).
template <int D>
constexpr int kMinBlocks = D == 256 ? 1 : 2;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct Geo {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "unsupported head dim");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kSteps = D / 16;    // MFMA k-steps over the head dimension
  static constexpr int kDBlocks = D / 32;  // 32-row blocks of a transposed accumulator
  static constexpr int kTileBytes = kTile * kRowBytes;
};

// Chunk swizzle for a tile read both ways.  A row read (16 lanes read one
// 16-byte chunk of 16 consecutive rows) needs the 16 rows in 16 distinct
// bank groups; a transposed read (32 lanes read 4 rows x 4 adjacent chunks)
// needs those 16 (row, chunk) pairs distinct.  d=128 (256-byte rows):
// 4*(row%4) + 2*(row/4 %2) + (row/8 %2); d=256 (512-byte rows, so chunks c
// and c+16 of a row share a bank group) uses the same XOR on the low four
// chunk bits.  d=64 (128-byte rows, two per bank
// sweep): 4*(row/2 %2) + (row/4 %4).  d=32 and d=96 (rows of 4 and 12
// chunks: rows r, r+4, r+8, r+12 share a bank group, the residues of r mod 4
// use disjoint ones, and the 4 rows of a transposed read already fall in 4
// distinct bank quarters): (row/4 %4), which keeps a chunk in its group of 4.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128 || D == 256) return 4 * (row & 3) + 2 * ((row >> 2) & 1) + ((row >> 3) & 1);
  else if constexpr (D == 64) return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  else return (row >> 2) & 3;
}

__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  // Word 3 = 0x00020000: raw (untyped) 32-bit data for gfx9-family buffers.
  return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, 0x00020000};
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes global -> LDS (lane i writes LDS bytes [16i, 16i+16) after the
// wave-uniform address in M0); offsets past the buffer size read as zeros.
__device__ __forceinline__ void load16_to_lds(i32x4 rsrc, int voff, unsigned lds_addr) {
  // The descriptor and the LDS address are wave-uniform: keep them in SGPRs.
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_lds_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same wait through the compiler builtin, which the compiler's own
// wait-count bookkeeping sees (vmcnt 0; expcnt and lgkmcnt left at their
// maxima, 7 and 15).  Issued once before a tile loop whose MFMAs read
// registers loaded from global memory before it: without it the compiler
// cannot tell inside the loop that those loads have landed, and counts the
// vector-memory counter down before each such MFMA on every tile -- a
// counter that by then also covers the next tile's copies, whose latency
// those waits would expose.
__device__ __forceinline__ void wait_vmem_known() { __builtin_amdgcn_s_waitcnt(0x0f70); }

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

// Copy rows [row0, row0 + ROWS) of a [N, D] bf16 matrix into a swizzled LDS
// tile (rows past N read as zeros).  Every wave copies its share of slices.
// The tile is a row-major array of 16-byte chunks: lane i of wave copy w fills
// chunk g = 64w + i (row g / chunks-per-row, physical chunk g % chunks-per-row,
// holding the logical chunk physical ^ swz(row)).
template <int D, int ROWS = kTile, int NW = kWaves>
__device__ __forceinline__ void copy_tile(const __bf16* mat, int N, int row0, unsigned tile_lds,
                                          int wave, int lane) {
  using G = Geo<D>;
  constexpr int kChunks = D / 8;
  constexpr int kLoads = ROWS * kChunks / (kWave * NW);
  static_assert(ROWS * kChunks % (kWave * NW) == 0, "tile must split evenly over the waves");
  const i32x4 rsrc = make_rsrc(mat + (size_t)row0 * D, (N - row0) * G::kRowBytes);
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const unsigned g = (wave * kLoads + it) * kWave + lane;
    const int r = (int)(g / kChunks);
    const int voff = r * G::kRowBytes + ((((int)(g % kChunks)) ^ swz<D>(r)) << 4);
    load16_to_lds(rsrc, voff, tile_lds + (wave * kLoads + it) * kWave * 16);
  }
}

// Copy ROWS floats [row0, row0 + ROWS) of a length-N vector into LDS (lanes
// 0..ROWS/4-1 of one wave; entries past N read as zeros).
template <int ROWS = kTile>
__device__ __forceinline__ void copy_vec(const float* vec, int N, int row0, unsigned dst, int lane) {
  if (lane < ROWS / 4) {
    const i32x4 rsrc = make_rsrc(vec + row0, (N - row0) * 4);
    load16_to_lds(rsrc, lane * 16, dst);
  }
}

// Per-lane LDS byte offsets (tile-relative, for tile rows 0..31 of a 32-row
// block) of the two operand reads.  Row read (A operand of X Y^T with X the
// tile): row L%32, logical chunk 2*st + L/32.
template <int D>
__device__ __forceinline__ int row_off(int l32, int half, int st) {
  return l32 * Geo<D>::kRowBytes + (((2 * st + half) ^ swz<D>(l32)) << 4);
}
// Transposed read (A operand of X^T Y): 16-lane group G = L/16 and s = L%16
// read row 16*cc + 4*(G/2) + s/4 (+8 for the second read) and columns
// 32*b + 16*(G%2) + 4*(s%4)..+3; lane L then holds column 32*b + L%32 of rows
// 16cc + 4*(L/32) + 0..3 and 16cc + 8 + 4*(L/32) + 0..3 -- the row order of a
// 32x32 accumulator's registers 8cc..8cc+7.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int h, int b, int cc) {
  const int g16 = lane >> 4, s16 = lane & 15;
  const int r = 16 * cc + 4 * (g16 >> 1) + (s16 >> 2) + 8 * h;
  const int col = 32 * b + 16 * (g16 & 1) + 4 * (s16 & 3);
  return r * Geo<D>::kRowBytes + (((col >> 3) ^ swz<D>(r)) << 4) + (col & 7) * 2;
}
// Transposed-read offsets are held per workgroup as tro[cc][b][h] =
// tr_off(lane, h, b, cc).  At d=256 only block 0's are filled and read
// (kTroBlocks): with 512-byte rows the row, the 16-byte chunk and the place in
// the chunk occupy disjoint bits of an offset, and block b's chunk is block
// 0's XOR 4b (the swizzle changes the low four chunk bits only), so block b's
// offset is block 0's XOR (b << 6) (tro_xor).  That keeps 28 registers free
// in kernels that hold the whole register file.
template <int D>
constexpr int kTroBlocks = D == 256 ? 1 : Geo<D>::kDBlocks;
template <int D>
constexpr int tro_block(int b) { return D == 256 ? 0 : b; }
template <int D>
constexpr int tro_xor(int b) { return D == 256 ? b << 6 : 0; }

__device__ __forceinline__ bf16x8 read_tr(const unsigned char* base, int off_lo, int off_hi) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_lo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Wave issue priority around a block's score products and softmax (raised)
// and its gradient products (normal): where the two waves of a SIMD contend,
// the one in the score phase goes first.  Measured 3-4 % faster at d=128 and
// no better at d=64 and d=96, where it is left off.
template <int D>
__device__ __forceinline__ void set_prio(int level) {
  if constexpr (D == 128) {
    if (level) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
}

// Logical workgroup id: workgroups are dispatched round-robin over the XCDs;
// the remap gives each XCD a contiguous range, so the blocks of one head run
// on one XCD and share its L2.
__device__ __forceinline__ int logical_block() {
  const int grid = gridDim.x;
  int lid = blockIdx.x;
  if (grid % kXcds == 0) lid = (lid % kXcds) * (grid / kXcds) + lid / kXcds;
  return lid;
}

// ---------------------------------------------------------------------------
// Kernel 1: delta_i = sum_t dO[i,t] * O[i,t].  Eight lanes per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const __bf16* __restrict__ o,
                                                        const __bf16* __restrict__ dout,
                                                        float* __restrict__ delta, long long rows) {
  constexpr int kPer = D / 8;  // elements per lane (4, 8, 12 or 16)
  const long long row = (long long)blockIdx.x * 32 + threadIdx.x / 8;
  const int sub = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const bf16x4* po = reinterpret_cast<const bf16x4*>(o + row * D + sub * kPer);
    const bf16x4* pg = reinterpret_cast<const bf16x4*>(dout + row * D + sub * kPer);
#pragma unroll
    for (int c = 0; c < kPer / 4; ++c) {
      const bf16x4 a = po[c], g = pg[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf((float)a[j], (float)g[j], acc);
    }
  }
  acc += __shfl_xor(acc, 1, 8);
  acc += __shfl_xor(acc, 2, 8);
  acc += __shfl_xor(acc, 4, 8);
  if (sub == 0 && row < rows) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// Kernel 2: dK, dV for one 128-key block of one head (32 keys per wave).
// ---------------------------------------------------------------------------
constexpr int kQT = 64;  // queries per streamed Q / dO tile
template <int D>
constexpr int dkdv_smem_bytes() { return 2 * (2 * kQT * D * 2 + 2 * kQT * 4); }  // 2 stages
// The paired workgroup's P exchange (PART 3 / 4 below): per dV wave, per
// 32-query block of the tile, the bf16 P of its 32 keys (16 values per lane,
// two 16-byte chunks), behind the two stages.
constexpr int kPShareBytes = kWaves * (kQT / kRows) * 2 * kWave * 16;
template <int D>
constexpr int dkdv_pair_smem_bytes() { return dkdv_smem_bytes<D>() + kPShareBytes; }

// The work of one group of four waves on key block `lid` (head * blocks +
// block).  PART 0: dK and dV together (d=64: several waves per SIMD fit).
// PART 1: dV only (S, then dV^T += dO^T P); PART 2: dK only (S and dP, then
// dK^T += Q^T dS).  At d=128 the two accumulators together do not fit beside
// K, V and the scores in the registers of two waves per SIMD, so the parts
// run in separate waves: S is formed twice, but every wave runs at two waves
// per SIMD (measured: about 18 % less time than one combined wave per SIMD).
// At d=256 the dK part alone (K, V, the dK accumulator and the scores) needs
// ~350 registers, so the parts run at one wave per SIMD.
//
// PART 3 and PART 4 are the two halves of one 8-wave workgroup (NW = 8: the
// dV waves 0-3 and the dK waves 4-7 share every Q and dO tile, copied once),
// used at d=128 when the problem has enough key blocks to fill the GPU.
// There S is formed once: each tile runs in two phases split by a barrier.
// In the first, a PART 3 wave forms S and the bf16 P of its 32 keys and
// leaves P in LDS while its PART 4 partner (same keys) forms dP; in the
// second, the PART 3 wave accumulates dV^T += dO^T P and the PART 4 wave
// reads P, forms dS = P (dP - delta) and accumulates dK^T += Q^T dS.  Each
// wave then runs two products per query block (the dK part three before),
// and the pair's exponentials are taken once.
//
// GENERAL: Nq queries against Nk keys, causal mask offset by `off` (key j
// visible to query i iff j <= i + off); otherwise Nk = Nq and off = 0.
template <int D, bool CAUSAL, int PART, bool GENERAL, int NW = kWaves>
__device__ __forceinline__ void dkdv_body(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                          const __bf16* __restrict__ v, const float* __restrict__ lse,
                                          const __bf16* __restrict__ dout,
                                          const float* __restrict__ delta, __bf16* __restrict__ dk,
                                          __bf16* __restrict__ dv, int Nq, int nk_arg, int off_arg,
                                          float scale, float c, unsigned char* smem, int lid) {
  using G = Geo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kDBlocks = G::kDBlocks;
  static_assert(PART >= 0 && PART <= 4, "PART");
  static_assert(PART < 3 || NW == 2 * kWaves, "P is exchanged within an 8-wave workgroup");
  constexpr bool kDoV = PART == 0 || PART == 1 || PART == 3;
  constexpr bool kDoK = PART == 0 || PART == 2 || PART == 4;
  constexpr bool kShare = PART >= 3;  // S formed once per pair, P exchanged through LDS
  constexpr int kQBlocks = kQT / kRows;       // 32-query blocks per tile
  constexpr int kTileBytes = kQT * G::kRowBytes;
  constexpr int kStageBytes = 2 * kTileBytes + 2 * kQT * 4;  // Q, dO, lse, delta
  static_assert(2 * kStageBytes == dkdv_smem_bytes<D>(), "LDS layout");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave_g: the wave in the workgroup (its share of the copies, the lse
  // duty); wave: which 32 keys of the block it owns (the dV and the dK waves
  // of an 8-wave workgroup cover the same 128 keys).
  const int wave_g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wave = wave_g % kWaves;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int Nk = GENERAL ? nk_arg : Nq;
  const int off = GENERAL ? off_arg : 0;
  const int n_kb = (Nk + kBlock - 1) / kBlock;
  const int head = lid / n_kb;
  const int kb = lid % n_kb;
  const size_t q_off = (size_t)head * Nq * D;   // q, dO: [head, Nq, D]
  const size_t kv_off = (size_t)head * Nk * D;  // k, v, dK, dV: [head, Nk, D]
  const __bf16* const qh = q + q_off;
  const __bf16* const doh = dout + q_off;
  const float* const lseh = lse + (size_t)head * Nq;
  const float* const dlth = delta + (size_t)head * Nq;
  const int key0 = kb * kBlock + wave * kRows;  // this wave's first key

  // K^T and V^T as B operands: lane L holds key key0 + L%32 (rows past Nk:
  // any valid row; their outputs are not stored), features 16*st + 8*(L/32)..+7.
  bf16x8 kf[kSteps], vf[kSteps];
  {
    const int row = min(key0 + l32, Nk - 1);
    const __bf16* kr = k + kv_off + (size_t)row * D + 8 * half;
    const __bf16* vr = v + kv_off + (size_t)row * D + 8 * half;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      kf[st] = *reinterpret_cast<const bf16x8*>(kr + 16 * st);
      vf[st] = *reinterpret_cast<const bf16x8*>(vr + 16 * st);
    }
  }
  f32x16 dkt[kDBlocks], dvt[kDBlocks];  // dK^T, dV^T: [d, keys]; lane = key
#pragma unroll
  for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkt[b][r] = dvt[b][r] = 0.f;

  int ro[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) ro[st] = row_off<D>(l32, half, st);
  int tro[2][kDBlocks][2];  // [cc][b][h]
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int b = 0; b < kTroBlocks<D>; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) tro[cc][b][h] = tr_off<D>(lane, h, b, cc);

  // Query tiles that see at least one key of the block (query i sees the
  // block's first key iff i >= kb*kBlock - off).
  const int qt_first = CAUSAL ? max(kb * kBlock - off, 0) / kQT : 0;
  const int n_qt = (Nq + kQT - 1) / kQT;
  auto stage_ptr = [&](int s) __attribute__((always_inline)) { return smem + s * kStageBytes; };
  // The stage's lse slot holds lse * log2(e) (0 past Nq): wave 0 reads the 64
  // values with ordinary loads when it issues the tile and writes the
  // products before the barrier that publishes the tile, so the exponent of
  // P below is one fma.
  static_assert(kQT == kWave, "one lse value per lane of wave 0");
  float lse_next = 0.f;
  auto issue = [&](int qt, int s) __attribute__((always_inline)) {
    unsigned char* st_base = stage_ptr(s);
    const int row0 = qt * kQT;
    copy_tile<D, kQT, NW>(qh, Nq, row0, lds_addr(st_base), wave_g, lane);
    copy_tile<D, kQT, NW>(doh, Nq, row0, lds_addr(st_base + kTileBytes), wave_g, lane);
    if (wave_g == 0) {
      copy_vec<kQT>(dlth, Nq, row0, lds_addr(st_base + 2 * kTileBytes + kQT * 4), lane);
      lse_next = row0 + lane < Nq ? lseh[row0 + lane] : 0.f;
    }
  };
  auto publish_lse = [&](int s) __attribute__((always_inline)) {
    if (wave_g == 0) reinterpret_cast<float*>(stage_ptr(s) + 2 * kTileBytes)[lane] = lse_next * kLog2e;
  };
  if (qt_first < n_qt) {
    issue(qt_first, 0);
    publish_lse(0);
  }

  // One Q/dO tile; the stage is a compile-time constant, so every LDS read
  // is a lane offset plus an immediate.
  auto tile = [&](auto stage_tag, int qt) __attribute__((always_inline)) {
    constexpr int s = decltype(stage_tag)::value;
    wait_lds_dma_all();
    __syncthreads();  // tile qt has landed; the other stage is free
    if (qt + 1 < n_qt) issue(qt + 1, s ^ 1);
    const unsigned char* const qt_lds = stage_ptr(s);
    const unsigned char* const dot_lds = qt_lds + kTileBytes;
    const float* const lse_lds = reinterpret_cast<const float*>(qt_lds + 2 * kTileBytes);
    const float* const dlt_lds = lse_lds + kQT;

    // S = Q K^T and dP = dO V^T of query block qb: [queries, keys]; lane =
    // key, register r = query 8*(r/4) + 4*(L/32) + r%4 of the block.
    auto sdp = [&](int qb, f32x16& sacc, f32x16& pacc) __attribute__((always_inline)) {
      const unsigned char* const qa = qt_lds + qb * kRows * G::kRowBytes;
      const unsigned char* const da = dot_lds + qb * kRows * G::kRowBytes;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        sacc = mfma(*reinterpret_cast<const bf16x8*>(qa + ro[st]), kf[st], sacc);
        if (kDoK) pacc = mfma(*reinterpret_cast<const bf16x8*>(da + ro[st]), vf[st], pacc);
      }
    };
    // P = 2^(s*c - lse*log2 e) and dS = P (dP - delta), as bf16 B operands;
    // with MASK, entries a query does not see are 0.
    auto soft = [&](auto mask_tag, int qb, const f32x16& sacc, const f32x16& pacc, bf16x8(&pb)[2],
                    bf16x8(&sb)[2]) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = qb * kRows + 8 * g + 4 * half;  // tile row of registers 4g..4g+3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_lds + qi);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlt_lds + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -l4[j]));
          if constexpr (MASK) {  // (a row that sees no key has lse = -inf: p is selected away)
            const int query = qt * kQT + qi + j;
            const bool vis = CAUSAL ? (key0 + l32 <= query + off && query < Nq) : (query < Nq);
            p = vis ? p : 0.f;
          }
          if (kDoV) pb[r >> 3][r & 7] = (__bf16)p;
          if (kDoK) sb[r >> 3][r & 7] = (__bf16)(p * (pacc[r] - d4[j]));
        }
      }
    };
    // PART 3: S = Q K^T of the live query blocks, then P as bf16 B operands
    // (0 where MASK hides an entry).  PART 4: dP = dO V^T of the live query
    // blocks.  With both blocks live their two accumulator chains are
    // interleaved, so neither MFMA waits on its predecessor's result.
    auto prod2 = [&](const unsigned char* tile_lds, const bf16x8(&bop)[kSteps], bool live0, bool live1,
                     f32x16(&acc)[kQBlocks]) __attribute__((always_inline)) {
      static_assert(kQBlocks == 2, "two query blocks per tile");
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][r] = 0.f;
      if (live0 && live1) {
        // All operand reads first: the products have no VALU work to hide
        // LDS latency behind, so the reads run ahead of the MFMAs.
        bf16x8 a0[kSteps], a1[kSteps];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          a0[st] = *reinterpret_cast<const bf16x8*>(tile_lds + ro[st]);
          a1[st] = *reinterpret_cast<const bf16x8*>(tile_lds + kRows * G::kRowBytes + ro[st]);
        }
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          acc[0] = mfma(a0[st], bop[st], acc[0]);
          acc[1] = mfma(a1[st], bop[st], acc[1]);
        }
        // Keep the reads ahead: six first, then two per pair of MFMAs (the
        // scheduler otherwise places each read right before its product).
        if constexpr (kSteps >= 4) {
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // DS reads
#pragma unroll
          for (int i = 0; i < kSteps - 3; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        }
      } else if (live0 || live1) {
        const int qb = live0 ? 0 : 1;
        const unsigned char* const a = tile_lds + qb * kRows * G::kRowBytes;
        f32x16 one = acc[0];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) one = mfma(*reinterpret_cast<const bf16x8*>(a + ro[st]), bop[st], one);
        acc[qb] = one;
      }
    };
    auto probs = [&](auto mask_tag, int qb, const f32x16& sacc, bf16x8(&pb)[2]) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = qb * kRows + 8 * g + 4 * half;  // tile row of registers 4g..4g+3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_lds + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -l4[j]));
          if constexpr (MASK) {
            const int query = qt * kQT + qi + j;
            const bool vis = CAUSAL ? (key0 + l32 <= query + off && query < Nq) : (query < Nq);
            p = vis ? p : 0.f;
          }
          pb[r >> 3][r & 7] = (__bf16)p;
        }
      }
    };
    // PART 4: dS = P (dP - delta) from the exchanged bf16 P.
    auto ds_from_p = [&](int qb, const bf16x8(&pb)[2], const f32x16& pacc, bf16x8(&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = qb * kRows + 8 * g + 4 * half;
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlt_lds + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          sb[r >> 3][r & 7] = (__bf16)((float)pb[r >> 3][r & 7] * (pacc[r] - d4[j]));
        }
      }
    };
    // This lane's slot for chunk cc of query block qb of dV wave `wave`.
    auto pslot = [&](int qb, int cc) __attribute__((always_inline)) {
      return smem + 2 * kStageBytes + ((wave * kQBlocks + qb) * 2 + cc) * (kWave * 16) + lane * 16;
    };

    // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-query steps.
    auto pv = [&](int qb, const bf16x8(&pb)[2], const bf16x8(&sb)[2]) __attribute__((always_inline)) {
      const unsigned char* const qa = qt_lds + qb * kRows * G::kRowBytes;
      const unsigned char* const da = dot_lds + qb * kRows * G::kRowBytes;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b) {
          if (kDoV) dvt[b] = mfma(read_tr(da, tro[cc][tro_block<D>(b)][0] ^ tro_xor<D>(b), tro[cc][tro_block<D>(b)][1] ^ tro_xor<D>(b)), pb[cc], dvt[b]);
          if (kDoK) dkt[b] = mfma(read_tr(qa, tro[cc][tro_block<D>(b)][0] ^ tro_xor<D>(b), tro[cc][tro_block<D>(b)][1] ^ tro_xor<D>(b)), sb[cc], dkt[b]);
        }
    };

    const int qrow_first = qt * kQT;
    const bool interior = (!CAUSAL || qrow_first + off >= key0 + kRows - 1) && qrow_first + kQT <= Nq;
    // Query block qb is skipped when no query of it sees a key of the wave
    // (the same for both waves of a pair, which own the same keys).
    auto skip = [&](int qb) __attribute__((always_inline)) {
      const int qrow0 = qrow_first + qb * kRows;
      return (CAUSAL && qrow0 + kRows - 1 + off < key0) || qrow0 >= Nq;
    };
    if constexpr (kShare) {
      // Phase 1: S and P (PART 3, P left in LDS) / dP (PART 4).
      const bool live0 = !skip(0), live1 = !skip(1);
      bf16x8 pb[kQBlocks][2];
      f32x16 acc2[kQBlocks];  // S (PART 3) or dP (PART 4)
      if constexpr (PART == 3) {
        set_prio<D>(1);
        prod2(qt_lds, kf, live0, live1, acc2);
#pragma unroll
        for (int qb = 0; qb < kQBlocks; ++qb) {
          if (!(qb ? live1 : live0)) continue;
          if (interior) probs(std::false_type{}, qb, acc2[qb], pb[qb]);
          else probs(std::true_type{}, qb, acc2[qb], pb[qb]);
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) *reinterpret_cast<bf16x8*>(pslot(qb, cc)) = pb[qb][cc];
        }
      } else {
        prod2(dot_lds, vf, live0, live1, acc2);
      }
      if constexpr (PART == 3) set_prio<D>(0);
      __syncthreads();  // every P of the tile is in LDS
      // Phase 2: dV (PART 3) / dS and dK (PART 4).
      if constexpr (PART == 4) set_prio<D>(1);
#pragma unroll
      for (int qb = 0; qb < kQBlocks; ++qb) {
        if (!(qb ? live1 : live0)) continue;
        if constexpr (PART == 3) {
          pv(qb, pb[qb], pb[qb]);
        } else {
          bf16x8 pr[2], sb[2];
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) pr[cc] = *reinterpret_cast<const bf16x8*>(pslot(qb, cc));
          ds_from_p(qb, pr, acc2[qb], sb);
          pv(qb, sb, sb);
        }
      }
      if constexpr (PART == 4) set_prio<D>(0);
      if (qt + 1 < n_qt) publish_lse(s ^ 1);
      return;
    }
#pragma unroll
    for (int qb = 0; qb < kQBlocks; ++qb) {
      const int qrow0 = qrow_first + qb * kRows;
      if (CAUSAL && qrow0 + kRows - 1 + off < key0) continue;  // no query sees a key of the wave
      if (qrow0 >= Nq) continue;
      set_prio<D>(1);
      f32x16 sacc, pacc;
      sdp(qb, sacc, pacc);
      bf16x8 pb[2], sb[2];
      if (interior) soft(std::false_type{}, qb, sacc, pacc, pb, sb);
      else soft(std::true_type{}, qb, sacc, pacc, pb, sb);
      set_prio<D>(0);
      pv(qb, pb, sb);
    }
    if (qt + 1 < n_qt) publish_lse(s ^ 1);
  };
  wait_vmem_known();  // K^T, V^T (and the first tile's copies) have landed
  for (int qt = qt_first; qt < n_qt; qt += 2) {
    tile(std::integral_constant<int, 0>{}, qt);
    if (qt + 1 < n_qt) tile(std::integral_constant<int, 1>{}, qt + 1);
  }

  // Epilogue: lane = key; registers 4j..4j+3 of block b are features
  // 32b + 8j + 4*(L/32) + 0..3.
  const int key = key0 + l32;
  if (key < Nk) {
    __bf16* const kr = dk + kv_off + (size_t)key * D;
    __bf16* const vr = dv + kv_off + (size_t)key * D;
#pragma unroll
    for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 kv4, vv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          kv4[r] = (__bf16)(dkt[b][4 * j + r] * scale);
          vv4[r] = (__bf16)dvt[b][4 * j + r];
        }
        if (kDoK) *reinterpret_cast<bf16x4*>(kr + 32 * b + 8 * j + 4 * half) = kv4;
        if (kDoV) *reinterpret_cast<bf16x4*>(vr + 32 * b + 8 * j + 4 * half) = vv4;
      }
  }
}

// d=32, 64 and 96: dK and dV in one workgroup per key block.
template <int D, bool CAUSAL, bool GENERAL>
__global__ __launch_bounds__(kWaves * kWave, 2)
void bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, const float* __restrict__ lse,
                     const __bf16* __restrict__ dout, const float* __restrict__ delta,
                     __bf16* __restrict__ dk, __bf16* __restrict__ dv, int Nq, int Nk, int off,
                     float scale, float c) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[dkdv_smem_bytes<D>()];
  dkdv_body<D, CAUSAL, 0, GENERAL>(q, k, v, lse, dout, delta, dk, dv, Nq, Nk, off, scale, c, smem,
                                   logical_block());
}

// d=128 and d=256: two workgroups per key block, one for dV and one for dK.  Logical
// ids 2b and 2b+1 are the two parts of key block b, so they run side by side
// on one XCD and share the Q and dO tiles in its L2.
template <int D, bool CAUSAL, bool GENERAL>
__global__ __launch_bounds__(kWaves * kWave, kMinBlocks<D>)
void bwd_dkdv_split_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                           const __bf16* __restrict__ v, const float* __restrict__ lse,
                           const __bf16* __restrict__ dout, const float* __restrict__ delta,
                           __bf16* __restrict__ dk, __bf16* __restrict__ dv, int Nq, int Nk, int off,
                           float scale, float c) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[dkdv_smem_bytes<D>()];
  const int lid = logical_block();
  if (lid & 1)
    dkdv_body<D, CAUSAL, 2, GENERAL>(q, k, v, lse, dout, delta, dk, dv, Nq, Nk, off, scale, c, smem,
                                     lid >> 1);
  else
    dkdv_body<D, CAUSAL, 1, GENERAL>(q, k, v, lse, dout, delta, dk, dv, Nq, Nk, off, scale, c, smem,
                                     lid >> 1);
}

// d=128 with at least one key block per CU: one 8-wave workgroup per key
// block, waves 0-3 computing dV and waves 4-7 dK over the same Q and dO tiles
// in LDS (copied once for both parts; 81 KB of LDS per CU with the P
// exchange, instead of two workgroups' 133 KB), S formed once per pair.
// Sharing the tiles measured 4 % faster than the two-workgroup form on
// B16-H16-N4096 and B4-H32-N8192 causal, and forming S once a further 0-6 %
// (most with causal masks); with fewer key blocks than CUs the two-workgroup
// form wins (twice as many workgroups to spread).
template <int D, bool CAUSAL, bool GENERAL>
__global__ __launch_bounds__(2 * kWaves * kWave, 1)
void bwd_dkdv_pair_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                          const __bf16* __restrict__ v, const float* __restrict__ lse,
                          const __bf16* __restrict__ dout, const float* __restrict__ delta,
                          __bf16* __restrict__ dk, __bf16* __restrict__ dv, int Nq, int Nk, int off,
                          float scale, float c) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[dkdv_pair_smem_bytes<D>()];
  const int lid = logical_block();
  if (__builtin_amdgcn_readfirstlane(threadIdx.x / kWave) >= kWaves)
    dkdv_body<D, CAUSAL, 4, GENERAL, 2 * kWaves>(q, k, v, lse, dout, delta, dk, dv, Nq, Nk, off, scale,
                                                 c, smem, lid);
  else
    dkdv_body<D, CAUSAL, 3, GENERAL, 2 * kWaves>(q, k, v, lse, dout, delta, dk, dv, Nq, Nk, off, scale,
                                                 c, smem, lid);
}

// ---------------------------------------------------------------------------
// Kernel 3: dQ for one 128-query block of one head (32 queries per wave).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool GENERAL>
__global__ __launch_bounds__(kWaves * kWave, kMinBlocks<D>)
void bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                   const __bf16* __restrict__ v, const float* __restrict__ lse,
                   const __bf16* __restrict__ dout, const float* __restrict__ delta,
                   __bf16* __restrict__ dq, int Nq, int nk_arg, int off_arg, float scale, float c) {
  using G = Geo<D>;
  constexpr int kSteps = G::kSteps;
  constexpr int kDBlocks = G::kDBlocks;
  constexpr int kTileBytes = G::kTileBytes;
  constexpr int kStageBytes = 2 * kTileBytes;  // K, V
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int Nk = GENERAL ? nk_arg : Nq;
  const int off = GENERAL ? off_arg : 0;
  const int n_qb = (Nq + kBlock - 1) / kBlock;
  const int lid = logical_block();
  const int head = lid / n_qb;
  const int qb = CAUSAL ? n_qb - 1 - lid % n_qb : lid % n_qb;  // causal: longest first
  const size_t q_off = (size_t)head * Nq * D;
  const size_t kv_off = (size_t)head * Nk * D;
  const __bf16* const kh = k + kv_off;
  const __bf16* const vh = v + kv_off;
  const int q0 = qb * kBlock + wave * kRows;  // this wave's first query

  // Q^T and dO^T as B operands: lane L holds query q0 + L%32 (rows past Nq:
  // any valid row, not stored), features 16*st + 8*(L/32)..+7.
  bf16x8 qf[kSteps], gf[kSteps];
  const int row = min(q0 + l32, Nq - 1);
  {
    const __bf16* qr = q + q_off + (size_t)row * D + 8 * half;
    const __bf16* gr = dout + q_off + (size_t)row * D + 8 * half;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      qf[st] = *reinterpret_cast<const bf16x8*>(qr + 16 * st);
      gf[st] = *reinterpret_cast<const bf16x8*>(gr + 16 * st);
    }
  }
  // (a row that sees no key has lse = -inf; every key is masked for it)
  const float lse2 = lse[(size_t)head * Nq + row] * kLog2e;
  const float dlt = delta[(size_t)head * Nq + row];
  const int query = q0 + l32;

  f32x16 dqt[kDBlocks];  // dQ^T: [d, queries]; lane = query
#pragma unroll
  for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[b][r] = 0.f;

  int ro[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) ro[st] = row_off<D>(l32, half, st);
  int tro[2][kDBlocks][2];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int b = 0; b < kTroBlocks<D>; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) tro[cc][b][h] = tr_off<D>(lane, h, b, cc);

  const int kv_end = CAUSAL ? min((qb + 1) * kBlock + off, Nk) : Nk;
  const int n_kt = kv_end > 0 ? (kv_end + kTile - 1) / kTile : 0;
  const int wave_last_key = CAUSAL ? min(q0 + kRows - 1 + off, Nk - 1) : Nk - 1;
  auto issue = [&](int kt, int s) __attribute__((always_inline)) {
    unsigned char* st_base = smem + s * kStageBytes;
    copy_tile<D>(kh, Nk, kt * kTile, lds_addr(st_base), wave, lane);
    copy_tile<D>(vh, Nk, kt * kTile, lds_addr(st_base + kTileBytes), wave, lane);
  };
  if (n_kt > 0) issue(0, 0);

  // One K/V tile; the stage is a compile-time constant, so every LDS read is
  // a lane offset plus an immediate.
  auto tile = [&](auto stage_tag, int kt) __attribute__((always_inline)) {
    constexpr int s = decltype(stage_tag)::value;
    wait_lds_dma_all();
    __syncthreads();  // tile kt has landed; the other stage is free
    if (kt + 1 < n_kt) issue(kt + 1, s ^ 1);
    const unsigned char* const k_lds = smem + s * kStageBytes;
    const unsigned char* const v_lds = k_lds + kTileBytes;
    // One 32-key block; with MASK, keys past Nk or above the diagonal get P = 0.
    auto block = [&](auto mask_tag, int sb) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int key0 = kt * kTile + sb * kRows;
      const unsigned char* const ka = k_lds + sb * kRows * G::kRowBytes;
      const unsigned char* const va = v_lds + sb * kRows * G::kRowBytes;
      set_prio<D>(1);
      // S^T = K Q^T and dP^T = V dO^T: [keys, queries]; lane = query,
      // register r = key 8*(r/4) + 4*(L/32) + r%4 of the block.
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        sacc = mfma(*reinterpret_cast<const bf16x8*>(ka + ro[st]), qf[st], sacc);
        pacc = mfma(*reinterpret_cast<const bf16x8*>(va + ro[st]), gf[st], pacc);
      }
      bf16x8 sbf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], c, -lse2));
        if constexpr (MASK) {
          const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key < Nk && (!CAUSAL || key <= query + off);
          p = vis ? p : 0.f;
        }
        sbf[r >> 3][r & 7] = (__bf16)(p * (pacc[r] - dlt));
      }
      set_prio<D>(0);
      // dQ^T += K^T dS^T over the block's two 16-key steps.
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int b = 0; b < kDBlocks; ++b)
          dqt[b] = mfma(read_tr(ka, tro[cc][tro_block<D>(b)][0] ^ tro_xor<D>(b), tro[cc][tro_block<D>(b)][1] ^ tro_xor<D>(b)), sbf[cc], dqt[b]);
    };
    const bool partial =
        kt * kTile + kTile - 1 > wave_last_key || (CAUSAL && kt * kTile + kTile - 1 > q0 + off);
    if (partial) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)  // a block past the wave's last visible key is skipped
        if (kt * kTile + sb * kRows <= wave_last_key) block(std::true_type{}, sb);
    } else {
      block(std::false_type{}, 0);
      block(std::false_type{}, 1);
    }
  };
  wait_vmem_known();  // Q^T, dO^T (and the first tile's copies) have landed
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < n_kt) tile(std::integral_constant<int, 1>{}, kt + 1);
  }

  if (query < Nq) {
    __bf16* const qr = dq + q_off + (size_t)query * D;
#pragma unroll
    for (int b = 0; b < kDBlocks; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = (__bf16)(dqt[b][4 * j + r] * scale);
        *reinterpret_cast<bf16x4*>(qr + 32 * b + 8 * j + 4 * half) = x;
      }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
bool g_gfx950[kMaxDevices];
int g_cus[kMaxDevices];

bool device_is_gfx950(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t prop;
    const bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess;
    g_gfx950[dev] = ok && strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_cus[dev] = ok ? prop.multiProcessorCount : 0;
  });
  return g_gfx950[dev];
}

// Compute units of the current device (0 if unknown; the device was checked).
int current_cus() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices ? g_cus[dev] : 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Nq, Nk >= 0 (square: Nq = Nk); a launch with an empty grid is skipped.
template <int D, bool CAUSAL, bool GENERAL>
int launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int Nq, int Nk,
           float scale, hipStream_t stream) {
  const long long rows = (long long)BH * Nq;
  const float c = scale * kLog2e;
  const int off = Nk - Nq;
  if (rows > 0)
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, stream,
                       static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), delta, rows);
  const int n_kblk = (Nk + kBlock - 1) / kBlock;
  const int n_qblk = (Nq + kBlock - 1) / kBlock;
  bool paired = false;  // d=128 with at least one key block per CU: 8-wave workgroups
  if constexpr (D == 128) {
    const int cus = current_cus();
    paired = n_kblk > 0 && cus > 0 && (long long)n_kblk * BH >= cus;
    if (paired)
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL, GENERAL>), dim3(n_kblk * BH),
                         dim3(2 * kWaves * kWave), 0, stream, static_cast<const __bf16*>(q),
                         static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), lse,
                         static_cast<const __bf16*>(dout), delta, static_cast<__bf16*>(dk),
                         static_cast<__bf16*>(dv), Nq, Nk, off, scale, c);
  }
  if (n_kblk > 0 && !paired) {
    if constexpr (D == 128 || D == 256)
      hipLaunchKernelGGL((bwd_dkdv_split_kernel<D, CAUSAL, GENERAL>), dim3(2 * n_kblk * BH),
                         dim3(kWaves * kWave), 0, stream, static_cast<const __bf16*>(q),
                         static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), lse,
                         static_cast<const __bf16*>(dout), delta, static_cast<__bf16*>(dk),
                         static_cast<__bf16*>(dv), Nq, Nk, off, scale, c);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, GENERAL>), dim3(n_kblk * BH), dim3(kWaves * kWave),
                         0, stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                         static_cast<const __bf16*>(v), lse, static_cast<const __bf16*>(dout), delta,
                         static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), Nq, Nk, off, scale, c);
  }
  if (n_qblk > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, GENERAL>), dim3(n_qblk * BH), dim3(kWaves * kWave), 0,
                       stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(v), lse, static_cast<const __bf16*>(dout), delta,
                       static_cast<__bf16*>(dq), Nq, Nk, off, scale, c);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

namespace {

// Argument checks shared by both entry points (before any HIP call).
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, const void* dq, const void* dk, const void* dv, const float* delta,
              int B, int H, int Nq, int Nk, int d, float scale, bool* nothing) {
  *nothing = false;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return ATTN_ERR_HEAD_DIM;
  if (!(scale > 0.0f) || !isfinite(scale)) return ATTN_ERR_SCALE;
  const int64_t bh = (int64_t)B * H;
  if (bh > INT32_MAX) return ATTN_ERR_SHAPE;
  if (2 * bh * (((int64_t)Nk + kBlock - 1) / kBlock) > INT32_MAX) return ATTN_ERR_SHAPE;  // grids
  if (bh * (((int64_t)Nq + kBlock - 1) / kBlock) > INT32_MAX) return ATTN_ERR_SHAPE;
  if ((int64_t)Nq * d * 2 > INT32_MAX || (int64_t)Nk * d * 2 > INT32_MAX)
    return ATTN_ERR_SHAPE;  // one head's bytes fit an int
  if (bh * Nq > (int64_t)INT32_MAX * 32) return ATTN_ERR_SHAPE;  // delta grid
  if (bh == 0 || (Nq == 0 && Nk == 0)) {
    *nothing = true;
    return ATTN_OK;
  }
  // Query-side buffers are unread when Nq = 0, key-side ones when Nk = 0.
  if (Nq > 0 && (!q || !o || !lse || !dout || !dq || !delta)) return ATTN_ERR_NULL;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, delta};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (!device_is_gfx950(dev)) return ATTN_ERR_DEVICE;
  return ATTN_OK;
}

template <bool GENERAL>
int dispatch(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* delta, int BH, int Nq, int Nk,
             int d, int causal, float scale, hipStream_t s) {
  auto go = [&](auto d_tag) {
    constexpr int D = decltype(d_tag)::value;
    return causal ? launch<D, true, GENERAL>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, Nq, Nk, scale, s)
                  : launch<D, false, GENERAL>(q, k, v, o, lse, dout, dq, dk, dv, delta, BH, Nq, Nk, scale, s);
  };
  switch (d) {
    case 32: return go(std::integral_constant<int, 32>{});
    case 64: return go(std::integral_constant<int, 64>{});
    case 96: return go(std::integral_constant<int, 96>{});
    case 128: return go(std::integral_constant<int, 128>{});
    default: return go(std::integral_constant<int, 256>{});
  }
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* delta, int B, int H, int N, int d, int causal, float scale,
                        void* stream) {
  bool nothing = false;
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, N, d, scale, &nothing);
  if (st != ATTN_OK || nothing) return st;
  return dispatch<false>(q, k, v, o, lse, dout, dq, dk, dv, delta, B * H, N, N, d, causal, scale,
                         static_cast<hipStream_t>(stream));
}

extern "C" int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* delta, int B, int H, int Nq, int Nk, int d, int causal,
                           float scale, void* stream) {
  bool nothing = false;
  const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Nq, Nk, d, scale, &nothing);
  if (st != ATTN_OK || nothing) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Nq == Nk)
    return dispatch<false>(q, k, v, o, lse, dout, dq, dk, dv, delta, B * H, Nq, Nk, d, causal, scale, s);
  return dispatch<true>(q, k, v, o, lse, dout, dq, dk, dv, delta, B * H, Nq, Nk, d, causal, scale, s);
}

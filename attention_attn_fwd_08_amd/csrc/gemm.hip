// gemm.hip -- bf16 matrix product on gfx950 matrix cores (MI355X, CDNA4).
//
// C = A B or C = A B^T, bf16 in, fp32 accumulate, bf16 out: the plain matrix
// product that the ThunderKittens paper summary (abstract, key points) lists
// as GEMM beside its attention kernels.
//
// Design:
//   * a workgroup of 8 waves computes a 256 x 256 tile of C; wave w owns rows
//     64*(w%4) .. +63 and columns 128*(w/4) .. +127 of it, as 2 x 4 blocks of
//     32 x 32 fp32 accumulators (v_mfma_f32_32x32x16_bf16), two waves per SIMD;
//   * each block is formed transposed, C^T = B-tile x A-tile^T: the B tile is
//     the MFMA A operand and the A tile the B operand, so a lane holds one row
//     of C and 16 of its columns in four runs of four, stored as 8-byte
//     bf16x4 writes;
//   * K advances 64 at a time; both operand tiles of a step go global -> LDS
//     through buffer loads that write LDS directly (no register staging),
//     double-buffered: the loads of step t+1 are issued during step t (all
//     at once after the barrier for C = A B^T; one pair before each of the
//     four MFMA k-steps for C = A B, which measured faster there) and land
//     while step t computes;
//   * LDS tiles are XOR-swizzled on 16-byte chunks so that every operand read
//     is bank-conflict free; an NN B tile ([64 k][256 n], n contiguous) is
//     read with ds_read_b64_tr_b16, which hands each lane 8 consecutive k of
//     one column, the order the A operand has;
//   * tails: rows past M, N or K read as zeros through the buffer range check
//     (rows past the end of the matrix) or an out-of-range offset (16-byte
//     chunks past K, or past N in an NN B tile); stores are guarded;
//   * workgroup ids are remapped so that each XCD (workgroups are dispatched
//     round-robin over the 8 XCDs) walks a compact group of tiles whose A rows
//     and B columns are shared in its L2.

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>

#include "attn_gemm.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr int kBM = 256, kBN = 256, kBK = 64;  // workgroup tile and K step
constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;
constexpr int kWavesM = 4;                // waves along M (2 along N)
constexpr int kWaveM = kBM / kWavesM, kWaveN = kBN / (kWaves / kWavesM);  // one wave's part
constexpr int kMBlocks = kWaveM / 32;
constexpr int kNBlocks = kWaveN / 32;
constexpr int kSteps = kBK / 16;           // MFMA k-steps per K step
constexpr int kTileBytes = 256 * kBK * 2;  // one operand tile of one K step
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kLoadBytes = kWave * 16;     // one wave-wide 16-byte-per-lane load
constexpr int kLoadsPerWave = kTileBytes / (kLoadBytes * kWaves);
constexpr int kKcRowBytes = kBK * 2;       // row of a k-contiguous tile (128 B)
constexpr int kNcRowBytes = kBN * 2;       // row of an n-contiguous tile (512 B)
constexpr int kXcds = 8;
constexpr int kGroupM = 8;                 // tile rows per group of the tile order

// Buffer resource {base, byte size}; word 3 = raw 32-bit data (gfx9 family).
// Every component is made wave-uniform (it must live in scalar registers).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(unsigned)p),
               __builtin_amdgcn_readfirstlane((int)((unsigned)(p >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes at byte offset voff of the buffer -> LDS bytes [lds + 16*lane, +16)
// (offsets at or past the buffer size read as zeros).
__device__ __forceinline__ void load16_to_lds(i32x4 rsrc, int voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_lds_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Chunk swizzles (16-byte chunks, XOR with a function of the row).
// k-contiguous tile (A; B for NT), 8 chunks per row: an operand read has 16
// lanes read one logical chunk of 16 consecutive rows, two rows per 256-byte
// bank window; the 8 even and the 8 odd rows each land in distinct chunks.
__device__ __forceinline__ int kc_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// n-contiguous tile (B for NN), 32 chunks per row (rows alias modulo 256
// bytes): a transposed read has 32 lanes read 4 consecutive rows x 4 chunks;
// the XOR moves row r's chunks by 4*(r%4) (+2 every 4 rows), 16 distinct
// chunk positions.
__device__ __forceinline__ int nc_swz(int row) { return 4 * (row & 3) + 2 * ((row >> 2) & 1); }

template <bool NT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(const __bf16* __restrict__ a,
                                                                const __bf16* __restrict__ b,
                                                                __bf16* __restrict__ c, int M, int N,
                                                                int K) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int wm = wave % kWavesM;  // 64-row quarter of the tile
  const int wn = wave / kWavesM;  // 128-column half of the tile

  // Workgroup -> tile.  Logical ids are contiguous per XCD; they run down
  // groups of kGroupM tile rows, column by column.
  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles_n = (N + kBN - 1) / kBN;
  const int grid = gridDim.x;
  int lid = blockIdx.x;
  if (grid % kXcds == 0) lid = (lid % kXcds) * (grid / kXcds) + lid / kXcds;
  const int per_group = kGroupM * tiles_n;
  const int group = lid / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = lid - group * per_group;
  const int m0 = (first_m + in_group % gsize) * kBM;
  const int n0 = (in_group / gsize) * kBN;
  const int n_kt = (K + kBK - 1) / kBK;

  // Global -> LDS copy of one K step.  Lane i of wave load w fills chunk
  // g = 64w + i of the tile: (row, physical chunk) of the tile's layout, which
  // holds the logical chunk (physical ^ swizzle).  *_first: the first k (or n,
  // NN B) of that chunk relative to the step, for the tail test.
  int a_ld[kLoadsPerWave], b_ld[kLoadsPerWave], a_first[kLoadsPerWave], b_first[kLoadsPerWave];
#pragma unroll
  for (int it = 0; it < kLoadsPerWave; ++it) {
    const unsigned g = (wave * kLoadsPerWave + it) * kWave + lane;
    const int row = (int)(g >> 3);
    const int lg = (int)(g & 7) ^ kc_swz(row);
    a_ld[it] = row * (K * 2) + lg * 16;
    a_first[it] = lg * 8;
    if constexpr (NT) {
      b_ld[it] = a_ld[it];
      b_first[it] = a_first[it];
    } else {
      const int brow = (int)(g >> 5);
      const int blg = (int)(g & 31) ^ nc_swz(brow);
      b_ld[it] = brow * (N * 2) + blg * 16;
      b_first[it] = blg * 8;
    }
  }
  const unsigned smem_base = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const unsigned lds_wave = smem_base + wave * kLoadsPerWave * kLoadBytes;

  // Copies of step kt into `stage`: all of them (part < 0) or only the
  // part-th A and B load of this wave.
  auto load_step = [&](int kt, int stage, int part) __attribute__((always_inline)) {
    const int k0 = kt * kBK;
    const unsigned dst = __builtin_amdgcn_readfirstlane(lds_wave + stage * kStageBytes);
    {
      const long long rem = ((long long)(M - m0) * K - k0) * 2;  // bytes to the end of A
      const unsigned bytes = (unsigned)(rem < 0x7fffffffLL ? rem : 0x7fffffffLL);
      const i32x4 rsrc = make_rsrc(a + (size_t)m0 * K + k0, bytes);
#pragma unroll
      for (int it = 0; it < kLoadsPerWave; ++it)
        if (part < 0 || part == it)
          load16_to_lds(rsrc, k0 + a_first[it] < K ? a_ld[it] : (int)bytes, dst + it * kLoadBytes);
    }
    {
      const long long rem = NT ? ((long long)(N - n0) * K - k0) * 2 : ((long long)(K - k0) * N - n0) * 2;
      const unsigned bytes = (unsigned)(rem < 0x7fffffffLL ? rem : 0x7fffffffLL);
      const __bf16* base = NT ? b + (size_t)n0 * K + k0 : b + (size_t)k0 * N + n0;
      const i32x4 rsrc = make_rsrc(base, bytes);
#pragma unroll
      for (int it = 0; it < kLoadsPerWave; ++it) {
        if (part >= 0 && part != it) continue;
        const bool in = NT ? k0 + b_first[it] < K : n0 + b_first[it] < N;
        load16_to_lds(rsrc, in ? b_ld[it] : (int)bytes, dst + kTileBytes + it * kLoadBytes);
      }
    }
  };

  // Operand reads.  k-contiguous tiles: lane L reads row (block + L%32),
  // logical chunk 2*st + L/32 (k = 16 st + 8 (L/32) .. +7); the swizzle
  // depends on row%16 = L%16 only, so one offset per step serves every block.
  int kc_rd[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) kc_rd[st] = l32 * kKcRowBytes + (((2 * st + half) ^ kc_swz(l32)) << 4);
  // NN B tile, transposed reads: 16-lane group G = L/16, s = L%16; read h
  // (0, 1) takes row k = 8 (G/2) + s/4 + 4h (+16 st) and columns
  // n = 16 (G%2) + 4 (s%4) .. +3 of the 32-column block.  Lane L then holds
  // column L%32 at k = 16 st + 8 (L/32) + 4h + 0..3: the two reads together
  // are the 8 consecutive k of the A operand's lane.
  int nc_rd[kNBlocks][2];
  {
    const int g16 = lane >> 4;
    const int s16 = lane & 15;
#pragma unroll
    for (int j = 0; j < kNBlocks; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = 8 * (g16 >> 1) + (s16 >> 2) + 4 * h;
        const int n = wn * kWaveN + 32 * j + 16 * (g16 & 1) + 4 * (s16 & 3);
        nc_rd[j][h] = kr * kNcRowBytes + (((n >> 3) ^ nc_swz(kr)) << 4) + (n & 7) * 2;
      }
  }

  f32x16 acc[kMBlocks][kNBlocks];
#pragma unroll
  for (int i = 0; i < kMBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kNBlocks; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  constexpr bool kSpread = !NT;  // copies spread over the k-steps
  static_assert(kLoadsPerWave == kSteps, "one A and one B copy per k-step");
  if (n_kt > 0) load_step(0, 0, -1);
  for (int kt = 0; kt < n_kt; ++kt) {
    wait_lds_dma();
    __syncthreads();  // step kt has landed; everyone is done with step kt-1's stage
    const bool has_next = kt + 1 < n_kt;
    if (!kSpread && has_next) load_step(kt + 1, (kt + 1) & 1, -1);
    const unsigned char* const sa = smem + (kt & 1) * kStageBytes;
    const unsigned char* const sb = sa + kTileBytes;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (kSpread && has_next) load_step(kt + 1, (kt + 1) & 1, st);
      bf16x8 af[kMBlocks], bf[kNBlocks];
#pragma unroll
      for (int i = 0; i < kMBlocks; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sa + (wm * kWaveM + 32 * i) * kKcRowBytes + kc_rd[st]);
#pragma unroll
      for (int j = 0; j < kNBlocks; ++j) {
        if constexpr (NT) {
          bf[j] = *reinterpret_cast<const bf16x8*>(sb + (wn * kWaveN + 32 * j) * kKcRowBytes + kc_rd[st]);
        } else {
          const unsigned char* p = sb + st * 16 * kNcRowBytes;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + nc_rd[j][0]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + nc_rd[j][1]));
          bf[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int i = 0; i < kMBlocks; ++i)
#pragma unroll
        for (int j = 0; j < kNBlocks; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  Block (i, j), lane L: row m0 + 64 wm + 32 i + L%32; register
  // 4q + r: column n0 + 128 wn + 32 j + 8 q + 4 (L/32) + r.
#pragma unroll
  for (int i = 0; i < kMBlocks; ++i) {
    const int m = m0 + wm * kWaveM + 32 * i + l32;
    if (m >= M) continue;
    __bf16* const crow = c + (size_t)m * N;
#pragma unroll
    for (int j = 0; j < kNBlocks; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * kWaveN + 32 * j + 8 * q + 4 * half;
        if (n < N) {
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (__bf16)acc[i][j][4 * q + r];
          *reinterpret_cast<bf16x4*>(crow + n) = v;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
bool g_gfx950[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_gfx950[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                    strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  return g_gfx950[dev] ? ATTN_OK : ATTN_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int attn_gemm_bf16(const void* a, const void* b, void* c, int M, int N, int K, int layout,
                              void* stream) {
  if (M < 0 || N < 0 || K < 0) return ATTN_ERR_SHAPE;
  if (layout != ATTN_GEMM_NN && layout != ATTN_GEMM_NT) return ATTN_ERR_SHAPE;
  if (N % 8 != 0 || K % 8 != 0) return ATTN_ERR_SHAPE;
  if (N >= (1 << 22) || K >= (1 << 22)) return ATTN_ERR_SHAPE;
  const int64_t tiles = (((int64_t)M + kBM - 1) / kBM) * (((int64_t)N + kBN - 1) / kBN);
  if (tiles > INT32_MAX) return ATTN_ERR_SHAPE;
  if (M == 0 || N == 0) return ATTN_OK;
  if (!c || (K > 0 && (!a || !b))) return ATTN_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return ATTN_ERR_ALIGN;
  int st = check_device();
  if (st != ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const __bf16* pa = static_cast<const __bf16*>(a);
  const __bf16* pb = static_cast<const __bf16*>(b);
  __bf16* pc = static_cast<__bf16*>(c);
  if (layout == ATTN_GEMM_NT)
    hipLaunchKernelGGL((gemm_bf16_kernel<true>), dim3((unsigned)tiles), dim3(kThreads), 0, s, pa, pb, pc,
                       M, N, K);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<false>), dim3((unsigned)tiles), dim3(kThreads), 0, s, pa, pb, pc,
                       M, N, K);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

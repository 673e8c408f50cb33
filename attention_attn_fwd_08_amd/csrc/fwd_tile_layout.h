// fwd_tile_layout.h -- register-fragment and LDS layouts of the attention
// forward on gfx950: the MFMA operand and accumulator layouts of
// v_mfma_f32_32x32x16_bf16 as the forward uses them, the swizzled LDS
// layout of a K or V stage, the global -> LDS copy that fills it, and the
// operand reads of the two products S^T = K Q^T and O^T += V^T P^T.
//
// The forward kernel (attn_fwd.hip) and the layout probes (layout_probe.hip,
// a test library that runs these same functions on one tile and returns
// every fragment) both include this file, so the probes pin the layouts the
// kernel actually uses.  The tile scheme follows the flash-attention
// examples of the ThunderKittens write-up (88811315.cn, "RTX 4090
// flash-attention example": K and V tiles staged in shared memory, V read in
// the column layout its product needs); the layouts are gfx950's own.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr int kQueriesPerWave = 32;
constexpr int kBlockN = 64;  // keys per LDS stage

// MFMA layouts (v_mfma_f32_32x32x16_bf16, D = A B + C with A 32x16, B 16x32):
//   A operand: lane L holds A[L%32][8*(L/32) + i], i = 0..7;
//   B operand: lane L holds B[8*(L/32) + i][L%32], i = 0..7;
//   accumulator: register r of lane L holds D[8*(r/4) + 4*(L/32) + r%4][L%32].
// In S^T = K Q^T the rows are keys and the columns queries; in
// O^T += V^T P^T the rows are features and the columns queries.

// LDS layouts.  A K or V stage is kBlockN rows of D bf16 (D*2 bytes); the
// 16-byte chunks of each row are permuted by an XOR with a function of the
// row, chosen against the way gfx950 services each read (measured with the
// LDS bank-conflict counter: 16-byte reads are serviced 16 lanes at a time,
// the 8-byte transposed reads 32 lanes at a time, 256 bytes per pass).
//
// K is read as the MFMA A operand: 16 lanes read the same chunk of 16
// consecutive rows.  d=128 and d=256 (rows a multiple of 256 bytes): XOR with
// row%16 puts them in 16 distinct chunk positions.  d=64 (128-byte rows, two
// rows per 256-byte pass): the 8 even and the 8 odd rows of the 16 each land
// in distinct chunks.  d=32 and d=96 (row stride 4 or 12 chunks, so rows
// r, r+4, r+8, r+12 share a bank group and the four residues of r mod 4 use
// disjoint ones): XOR with (row/4)%4 separates the four rows of a residue
// inside their group of four chunks (and keeps a chunk below D/8).
//
// V is read with ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x 2
// adjacent 32-byte chunk pairs; the XOR moves the pair index by 2*(row%4) (+1
// every 4 rows), so the 8 (row, pair) reads cover 8 distinct pair positions.
// d=64: the two even (and two odd) rows of the 4 get pair offsets 0 and 2.
// d=32 (the 4 rows are 256 contiguous bytes) and d=96 (row offsets 0, 192,
// 384, 576 fall in 4 distinct 64-byte bank quarters) need no swizzle.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  if constexpr (D == 128 || D == 256) return row & 15;
  else if constexpr (D == 64) return (row & 7) ^ ((row >> 3) & 1);
  else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  if constexpr (D == 128 || D == 256) return 4 * (row & 3) + 2 * ((row >> 2) & 1);
  else if constexpr (D == 64) return 4 * ((row >> 1) & 1);
  else return 0;
}
// Byte offset of 32-feature block b of a V row read at `off` (block 0): with
// rows a multiple of 128 bytes the block index is chunk bits 2.. of the
// swizzled offset (XOR, which composes with the swizzle); d=96 rows are not,
// and are unswizzled, so the block is a plain displacement.
template <int D>
__device__ __forceinline__ int v_block(int off, int b) {
  if constexpr (D == 96) return off + 64 * b;
  else return off ^ (b << 6);
}

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kSteps = D / 16;    // MFMA k-steps of one 32x32 score block
  static constexpr int kDBlocks = D / 32;  // 32-row blocks of O^T
  static constexpr int kStageBytes = kBlockN * kRowBytes;
  static constexpr int kChunksPerRow = D / 8;
};

// Copy of a stage: the stage is a row-major array of 16-byte chunks, filled
// in order (LDS chunk g, bytes [16g, 16g+16), is written by the g-th lane of
// the copy), and LDS chunk g -- row g / (D/8), physical chunk p = g % (D/8)
// -- receives logical chunk p ^ swizzle(row) of that row of the tile.  The
// XOR is its own inverse, so logical chunk c of a row sits at physical chunk
// c ^ swizzle(row).  These return the byte offset, within the tile in
// global memory (rows of D bf16), that LDS chunk g is read from, for K and
// for V.
template <int D>
__device__ __forceinline__ int k_copy_offset(unsigned g) {
  const int row = (int)(g / Tile<D>::kChunksPerRow);
  const int chunk = (int)(g % Tile<D>::kChunksPerRow);
  return row * Tile<D>::kRowBytes + ((chunk ^ k_swz<D>(row)) << 4);
}
template <int D>
__device__ __forceinline__ int v_copy_offset(unsigned g) {
  const int row = (int)(g / Tile<D>::kChunksPerRow);
  const int chunk = (int)(g % Tile<D>::kChunksPerRow);
  return row * Tile<D>::kRowBytes + ((chunk ^ v_swz<D>(row)) << 4);
}

// 16 bytes global -> LDS without passing through registers, through a buffer
// resource {base, byte size}: lane i of the wave reads bytes [voff, voff+16)
// of the buffer (offsets past the size, which the hardware range-checks,
// return zeros) and writes them to LDS bytes [16i, 16i+16) after the
// wave-uniform LDS byte address `lds_addr + OFF` (set through M0; OFF is a
// compile-time byte offset added inside the asm, so only the base occupies a
// scalar register).  Issued as inline assembly so the compiler does not wait
// for these loads before unrelated LDS reads; the caller waits for them
// itself (wait_lds_dma) before the barrier that publishes them.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  // Word 3 = 0x00020000: raw (untyped) 32-bit data for gfx9-family buffers.
  return i32x4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xffffu), bytes, 0x00020000};
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <unsigned OFF>
__device__ __forceinline__ void load16_to_lds(i32x4 rsrc, int voff, unsigned lds_addr) {
  asm volatile("s_add_u32 m0, %2, %3\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_addr), "n"(OFF)
               : "memory", "m0", "scc");
}
#pragma clang diagnostic pop
// f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Wait until at most N of this wave's LDS-bound loads are still in flight.
template <int N>
__device__ __forceinline__ void wait_lds_dma() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Stage-relative LDS byte offset of the K operand read of MFMA step st
// (A operand of S^T = K Q^T): row L%32 (+32 per 32-key block), logical
// chunk 2*st + L/32, i.e. features 16*st + 8*(L/32) .. +7.
template <int D>
__device__ __forceinline__ int k_operand_offset(int l32, int half, int st) {
  return l32 * Tile<D>::kRowBytes + (((2 * st + half) ^ k_swz<D>(l32)) << 4);
}

// Stage-relative LDS byte offsets of the two transposed V reads (A operand
// of O^T += V^T P^T), for read h = 0, 1: 16-lane group G = L/16 and
// s = L%16 read row 16*cc + 4*(G/2) + s/4 (+8 for h = 1) and features
// 32*b + 16*(G%2) + 4*(s%4) .. +3; lane L then holds feature 32*b + L%32 of
// keys 16cc + 4*(L/32) + 0..3 (h = 0) and 16cc + 8 + 4*(L/32) + 0..3
// (h = 1), the key order of P^T's slots in the score accumulator.  The
// swizzle depends on row%16 only, identical for every (sb, cc), and the
// d-block b only flips bits 6-7 of the offset (chunk bits 2-3).
template <int D>
__device__ __forceinline__ int v_operand_offset(int lane, int h) {
  const int g16 = lane >> 4;
  const int s16 = lane & 15;
  const int r = 4 * (g16 >> 1) + (s16 >> 2) + 8 * h;
  const int col = 16 * (g16 & 1) + 4 * (s16 & 3);
  return r * Tile<D>::kRowBytes + (((col >> 3) ^ v_swz<D>(r)) << 4) + (col & 7) * 2;
}

// The V^T operand of one 16-key MFMA step: `a` is the stage's row 16*cc
// (+32 per 32-key block), b the 32-feature block of O^T.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const unsigned char* a, const int (&v_off)[2], int b) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + v_block<D>(v_off[0], b)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + v_block<D>(v_off[1], b)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Q^T as the B operand of S^T = K Q^T: lane L holds the query whose row
// `qrow` points at (query L%32 of the wave), features 16*st + 8*(L/32) .. +7
// in qf[st].
template <int D>
__device__ __forceinline__ void q_operand(const __bf16* qrow, int half, bf16x8 (&qf)[Tile<D>::kSteps]) {
#pragma unroll
  for (int st = 0; st < Tile<D>::kSteps; ++st)
    qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 8 * half + 16 * st);
}

// Scores S^T of one 32-key block (sb) of a K stage against this wave's 32
// queries (Q^T held as the B operand: lane L holds query L%32, features
// 16*st + 8*(L/32) .. +7 in qf[st]).
template <int D>
__device__ __forceinline__ void scores_block(const unsigned char* k_lds, int sb,
                                             const int (&k_off)[Tile<D>::kSteps],
                                             const bf16x8 (&qf)[Tile<D>::kSteps], f32x16& s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int st = 0; st < Tile<D>::kSteps; ++st) {
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_lds + sb * 32 * Tile<D>::kRowBytes + k_off[st]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s, 0, 0, 0);
  }
}

// Scores S^T of the two 32-key blocks of a K stage against this wave's 32
// queries.  Accumulator register r of lane L: key 8*(r/4) + 4*(L/32) + r%4 of
// the block, query L%32.
template <int D>
__device__ __forceinline__ void scores(const unsigned char* k_lds, const int (&k_off)[Tile<D>::kSteps],
                                       const bf16x8 (&qf)[Tile<D>::kSteps], f32x16 (&s)[2]) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
#pragma unroll
    for (int st = 0; st < Tile<D>::kSteps; ++st) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_lds + sb * 32 * Tile<D>::kRowBytes + k_off[st]);
      s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[sb], 0, 0, 0);
    }
  }
}

}  // namespace

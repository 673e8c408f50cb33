// layout_probe.hip -- test library: runs the forward's layout functions
// (fwd_tile_layout.h) on one 64-key tile with one wave and returns every
// fragment they produce, so a test can check each against the matrices on
// the host:
//   * the K and V copies global -> LDS through the swizzled layout, with the
//     buffer's size check zero-filling rows past the valid keys;
//   * the K operand (A of S^T = K Q^T) and the Q^T operand (B) of every
//     MFMA step, and the S^T accumulators;
//   * the V^T operand of every step of O^T += V^T P^T (transposed LDS reads)
//     and the O^T accumulators, with P^T taken, as the forward takes it,
//     from the S^T accumulator registers rounded to bf16.
// A second entry point runs one bare v_mfma_f32_32x32x16_bf16 on fragments
// the caller lays out, to pin the operand and accumulator layouts the
// forward's comments state.  The tile scheme is the flash-attention
// example's of the ThunderKittens write-up (88811315.cn, "RTX 4090
// flash-attention example": tiles of K and V in shared memory, V read in the
// column layout of its product).
//
// Not part of the attention library: nothing in it is called by it.

#include <hip/hip_runtime.h>

#include "fwd_tile_layout.h"

namespace {

// One wave.  Outputs (element counts; T = Tile<D>):
//   kfrag [2 blocks][T::kSteps][64 lanes][8] bf16  -- K operand of (block, step)
//   qfrag [T::kSteps][64][8] bf16                  -- Q^T operand of step
//   s     [2 blocks][64][16] f32                   -- S^T accumulators
//   vfrag [2 blocks][2 steps][T::kDBlocks][64][8] bf16 -- V^T operand
//   o     [T::kDBlocks][64][16] f32                -- O^T accumulators
template <int D>
__global__ __launch_bounds__(kWave, 1) void probe_tile_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, const __bf16* __restrict__ q,
    int nk_valid, __bf16* __restrict__ kfrag, __bf16* __restrict__ qfrag, float* __restrict__ s_out,
    __bf16* __restrict__ vfrag, float* __restrict__ o_out) {
  using T = Tile<D>;
  constexpr int kLoads = T::kStageBytes / (kWave * 16);  // 16-byte loads per lane per tensor
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * T::kStageBytes];
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Copies: lane i of load `it` fills LDS chunk 64*it + i of each stage.
  const unsigned lds = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const i32x4 rk = make_rsrc(k, nk_valid * T::kRowBytes);
  const i32x4 rv = make_rsrc(v, nk_valid * T::kRowBytes);
  static_for<0, kLoads>([&](auto it_tag) __attribute__((always_inline)) {
    constexpr int it = decltype(it_tag)::value;
    load16_to_lds<it * kWave * 16>(rk, k_copy_offset<D>(it * kWave + lane), lds);
    load16_to_lds<T::kStageBytes + it * kWave * 16>(rv, v_copy_offset<D>(it * kWave + lane), lds);
  });
  wait_lds_dma<0>();
  __syncthreads();
  const unsigned char* const k_lds = smem;
  const unsigned char* const v_lds = smem + T::kStageBytes;

  int k_off[T::kSteps];
#pragma unroll
  for (int st = 0; st < T::kSteps; ++st) k_off[st] = k_operand_offset<D>(l32, half, st);
  int v_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) v_off[h] = v_operand_offset<D>(lane, h);

  bf16x8 qf[T::kSteps];
  q_operand<D>(q + (size_t)l32 * D, half, qf);
  for (int st = 0; st < T::kSteps; ++st)
    *reinterpret_cast<bf16x8*>(qfrag + ((size_t)st * kWave + lane) * 8) = qf[st];
  for (int sb = 0; sb < 2; ++sb)
    for (int st = 0; st < T::kSteps; ++st)
      *reinterpret_cast<bf16x8*>(kfrag + ((size_t)(sb * T::kSteps + st) * kWave + lane) * 8) =
          *reinterpret_cast<const bf16x8*>(k_lds + sb * 32 * T::kRowBytes + k_off[st]);

  f32x16 s[2];
  scores<D>(k_lds, k_off, qf, s);
  for (int sb = 0; sb < 2; ++sb)
    for (int r = 0; r < 16; ++r) s_out[((size_t)sb * kWave + lane) * 16 + r] = s[sb][r];

  // P^T from the score registers, as the forward forms it: registers
  // 8*cc .. 8*cc+7 of block sb, rounded to bf16, are the B operand of step
  // (sb, cc).
  f32x16 acc[T::kDBlocks];
  for (int b = 0; b < T::kDBlocks; ++b)
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  for (int sb = 0; sb < 2; ++sb)
    for (int cc = 0; cc < 2; ++cc) {
      bf16x8 pb;
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)s[sb][8 * cc + j];
      for (int b = 0; b < T::kDBlocks; ++b) {
        const bf16x8 vf = v_operand<D>(v_lds + (sb * 32 + cc * 16) * T::kRowBytes, v_off, b);
        *reinterpret_cast<bf16x8*>(vfrag + ((size_t)((sb * 2 + cc) * T::kDBlocks + b) * kWave + lane) * 8) = vf;
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, acc[b], 0, 0, 0);
      }
    }
  for (int b = 0; b < T::kDBlocks; ++b)
    for (int r = 0; r < 16; ++r) o_out[((size_t)b * kWave + lane) * 16 + r] = acc[b][r];
}

// One bare MFMA: lane L passes a[L] (8 bf16), b[L] (8 bf16) and c[L]
// (16 f32) and receives d[L] (16 f32).
__global__ __launch_bounds__(kWave, 1) void probe_mfma_kernel(const __bf16* __restrict__ a,
                                                              const __bf16* __restrict__ b,
                                                              const float* __restrict__ c,
                                                              float* __restrict__ d) {
  const int lane = threadIdx.x;
  const bf16x8 af = *reinterpret_cast<const bf16x8*>(a + lane * 8);
  const bf16x8 bf = *reinterpret_cast<const bf16x8*>(b + lane * 8);
  f32x16 acc;
  for (int r = 0; r < 16; ++r) acc[r] = c[lane * 16 + r];
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
  for (int r = 0; r < 16; ++r) d[lane * 16 + r] = acc[r];
}

template <int D>
int launch_tile(const void* k, const void* v, const void* q, int nk_valid, void* kfrag, void* qfrag,
                void* s, void* vfrag, void* o, hipStream_t stream) {
  hipLaunchKernelGGL(probe_tile_kernel<D>, dim3(1), dim3(kWave), 0, stream,
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                     static_cast<const __bf16*>(q), nk_valid, static_cast<__bf16*>(kfrag),
                     static_cast<__bf16*>(qfrag), static_cast<float*>(s), static_cast<__bf16*>(vfrag),
                     static_cast<float*>(o));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

// Device pointers (16-byte aligned, HIP device memory): k, v 64 x d bf16
// row-major (rows >= nk_valid are never read); q 32 x d bf16; outputs sized
// as probe_tile_kernel states.  d in {32, 64, 96, 128, 256}, 0 <= nk_valid
// <= 64.  Returns 0 on success, 1 for an invalid argument (nothing is
// launched), 2 when the launch fails.  Asynchronous on `stream`.
extern "C" int layout_probe_tile(int d, const void* k, const void* v, const void* q, int nk_valid,
                                 void* kfrag, void* qfrag, void* s, void* vfrag, void* o,
                                 hipStream_t stream) {
  if (!k || !v || !q || !kfrag || !qfrag || !s || !vfrag || !o) return 1;
  if (nk_valid < 0 || nk_valid > kBlockN) return 1;
  switch (d) {
    case 32: return launch_tile<32>(k, v, q, nk_valid, kfrag, qfrag, s, vfrag, o, stream);
    case 64: return launch_tile<64>(k, v, q, nk_valid, kfrag, qfrag, s, vfrag, o, stream);
    case 96: return launch_tile<96>(k, v, q, nk_valid, kfrag, qfrag, s, vfrag, o, stream);
    case 128: return launch_tile<128>(k, v, q, nk_valid, kfrag, qfrag, s, vfrag, o, stream);
    case 256: return launch_tile<256>(k, v, q, nk_valid, kfrag, qfrag, s, vfrag, o, stream);
    default: return 1;
  }
}

// Device pointers: a, b 64 x 8 bf16; c, d 64 x 16 f32.  Returns 0, 1
// (null pointer) or 2 (launch failed).
extern "C" int layout_probe_mfma(const void* a, const void* b, const void* c, void* d,
                                 hipStream_t stream) {
  if (!a || !b || !c || !d) return 1;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(1), dim3(kWave), 0, stream, static_cast<const __bf16*>(a),
                     static_cast<const __bf16*>(b), static_cast<const float*>(c), static_cast<float*>(d));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

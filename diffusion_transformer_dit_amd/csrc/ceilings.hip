// Ceiling probes of the chip, for placing the block's kernels against what
// the hardware delivers and not only against the published peaks:
//   copy16_kernel    a plain streaming copy (16-byte loads and stores, four
//                    chunks in flight per thread): the practical HBM rate at
//                    a given size, the ceiling of the memory-bound chain;
//   mfma_peak_kernel back-to-back bf16 MFMAs on register operands, either
//                    the same operands every time or ones that change with
//                    every instruction (as in a GEMM, whose matrix cores then
//                    draw more power): the practical bf16 matrix-core rate.
// Neither is part of the block's path.
#include "dit_common.hpp"
#include "launch.hpp"

namespace dit {

constexpr int kCopyThreads = 256;
constexpr int kCopyChunks = 4;  // 16-byte chunks per thread

__global__ void __launch_bounds__(kCopyThreads)
copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t base = size_t(blockIdx.x) * (kCopyThreads * kCopyChunks) + threadIdx.x;
  u32x4 v[kCopyChunks];
#pragma unroll
  for (int j = 0; j < kCopyChunks; ++j) {
    const size_t i = base + size_t(j) * kCopyThreads;
    if (i < n16) v[j] = src[i];
  }
#pragma unroll
  for (int j = 0; j < kCopyChunks; ++j) {
    const size_t i = base + size_t(j) * kCopyThreads;
    if (i < n16) dst[i] = v[j];
  }
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t per_block = size_t(kCopyThreads) * kCopyChunks;
  const size_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  copy16_kernel<<<unsigned(blocks), kCopyThreads, 0, st>>>(static_cast<const u32x4*>(src),
                                                           static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

// Pseudo-random bf16 operand bits with a full mantissa (values in [-2, 2)),
// distinct per lane, register and element.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ bf16x8 operand(uint32_t seed) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t r = mix32(seed * 4u + e);
    // sign and mantissa random, exponent of 1 (values in [1, 2) and (-2, -1])
    const uint32_t lo = 0x3F80u | (r & 0x807Fu);
    const uint32_t hi = 0x3F80u | ((r >> 16) & 0x807Fu);
    w[e] = lo | (hi << 16);
  }
  return __builtin_bit_cast(bf16x8, w);
}

// 4 waves per workgroup; every wave issues `iters` rounds of 4 independent
// v_mfma_f32_32x32x16_bf16 (32768 flop each; the same flop rate per cycle as
// the GEMMs' 16x16x32 instruction, and the attention's instruction), so no
// instruction waits on the previous one.  VARY: the operands change from one
// instruction to the next (two A and two B fragments in rotation) instead of
// staying the same.
template <bool VARY>
__global__ void __launch_bounds__(256)
mfma_peak_kernel(float* __restrict__ out, int iters) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  const bf16x8 a0 = operand(gid * 4u), a1 = operand(gid * 4u + 1);
  const bf16x8 b0 = operand(gid * 4u + 2), b1 = operand(gid * 4u + 3);
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VARY ? a1 : a0, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, VARY ? b1 : b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VARY ? a1 : a0, VARY ? b1 : b0, c3, 0, 0, 0);
  }
  const f32x16 sv = (c0 + c1) + (c2 + c3);
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += sv[i];
  out[gid] = t;
}

hipError_t launch_probe_mfma(float* out, int n_workgroups, int iters, int vary, hipStream_t st) {
  if (n_workgroups <= 0) return hipSuccess;
  if (vary)
    mfma_peak_kernel<true><<<n_workgroups, 256, 0, st>>>(out, iters);
  else
    mfma_peak_kernel<false><<<n_workgroups, 256, 0, st>>>(out, iters);
  return hipGetLastError();
}

}  // namespace dit

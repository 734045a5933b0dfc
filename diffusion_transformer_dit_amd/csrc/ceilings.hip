// Ceiling probes of the chip, for placing the block's kernels against what
// the hardware delivers and not only against the published peaks:
//   copy16_kernel    a plain streaming copy (16-byte loads and stores, four
//                    chunks in flight per thread): the practical HBM rate at
//                    a given size, the ceiling of the memory-bound chain;
//   mfma_peak_kernel back-to-back v_mfma_f32_16x16x32_bf16 on register
//                    operands, either the same operands every time or ones
//                    that change with every instruction (as in a GEMM, whose
//                    matrix cores then draw more power): the practical rate
//                    of the GEMMs' instruction.
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

// 4 waves per workgroup; every wave issues `iters` rounds of 16 independent
// MFMAs (16 accumulators, so no instruction waits on the previous one).
__global__ void __launch_bounds__(256)
mfma_peak_kernel(float* __restrict__ out, int iters, int vary) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a[r] = operand(gid * 8u + r);
    b[r] = operand(gid * 8u + 4 + r);
  }
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (vary) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i >> 2], b[i & 3], acc[i], 0, 0, 0);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[0], acc[i], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
  out[gid] = s;
}

hipError_t launch_probe_mfma(float* out, int n_workgroups, int iters, int vary, hipStream_t st) {
  if (n_workgroups <= 0) return hipSuccess;
  mfma_peak_kernel<<<n_workgroups, 256, 0, st>>>(out, iters, vary);
  return hipGetLastError();
}

}  // namespace dit

// Modulation GEMV rows, shared by the modulation kernels and the attention
// launch that also computes the next block's modulation in its last round.
//   mod[r] = sum_c W[r, c] * SiLU(temb[c]) + b[r]
// for the matrices of a table (one block, the two streams of a block, or a
// whole block stack): matrix m (rows_per_mat rows) gives
// mods[m * rows_per_mat + r].  The Flux page (ChituDiffusion, section 2)
// names this adaLN modulation as one of the block's small launches.
#pragma once

#include "dit_common.hpp"

namespace dit {

// Where the matrices come from: a device array of pointers (a stack's
// blocks) or up to two pointers passed by value (the two streams of a block).
struct ModTabDev {
  const bf16_t* const* ws;
  const bf16_t* const* bs;
  __device__ __forceinline__ const bf16_t* w(int m) const { return ws[m]; }
  __device__ __forceinline__ const bf16_t* b(int m) const { return bs[m]; }
};
struct ModTab2 {
  const bf16_t* ws[2];
  const bf16_t* bs[2];
  __device__ __forceinline__ const bf16_t* w(int m) const { return m ? ws[1] : ws[0]; }
  __device__ __forceinline__ const bf16_t* b(int m) const { return m ? bs[1] : bs[0]; }
};

// The rows of global wave `wave` of the launch (rows_per_wave consecutive
// rows), with s_act an LDS buffer of NCH * 512 floats.  Every thread of the
// workgroup calls it (it holds a workgroup barrier).
template <int NCH, class Tab>
__device__ __forceinline__ void mod_gemv_rows(const bf16_t* __restrict__ temb, const Tab& tab, float* __restrict__ mods,
                                              int rows_per_mat, int rows, int cols, int rows_per_wave, int wave,
                                              float* s_act) {
  const int nchunk = cols >> 3;
  const int lane = threadIdx.x & 63;
  const int r0 = wave * rows_per_wave;
  const int r1 = min(rows, r0 + rows_per_wave);
  auto load_row = [&](int r, u32x4 (&v)[NCH]) {
    const int m = r / rows_per_mat;
    const bf16_t* w = tab.w(m) + size_t(r - m * rows_per_mat) * cols;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) v[j] = reinterpret_cast<const u32x4*>(w)[c];
    }
  };
  // the first row's loads are in flight while the workgroup computes SiLU
  u32x4 cur[NCH], nxt[NCH];
  if (r0 < rows) load_row(r0, cur);
  for (int i = threadIdx.x; i < cols; i += blockDim.x) s_act[i] = silu(bf2f(temb[i]));
  __syncthreads();
  if (r0 >= rows) return;
  for (int r = r0; r < r1; ++r) {
    if (r + 1 < r1) load_row(r + 1, nxt);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) {
        float f[8];
        unpack8(cur[j], f);
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(&s_act[8 * c]);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(&s_act[8 * c + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += f[e] * a0[e];
          acc += f[4 + e] * a1[e];
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      const int m = r / rows_per_mat;
      const bf16_t* b = tab.b(m);
      mods[r] = acc + (b ? bf2f(b[r - m * rows_per_mat]) : 0.f);
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) cur[j] = nxt[j];
  }
}

}  // namespace dit

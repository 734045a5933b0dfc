// Memory-bound kernels of the single-stream block, for gfx950:
//   modulation GEMV (SiLU(temb) -> shift | scale | gate),
//   fused LayerNorm + adaLN modulate, gated residual,
//   per-head QK RMSNorm + RoPE, RoPE cos/sin tables, and the output
//   prediction of a skipped denoising step.
// These are the "cast / modulate / norm" HBM round trips between the GEMMs
// that the Flux page (ChituDiffusion, section 2) finds in the eager trace and
// that its section 1.1 fuses; here each is one pass over HBM with 16-byte
// loads and stores and wavefront-reduced row statistics in fp32.
#include <cmath>

#include "dit_common.hpp"
#include "launch.hpp"
#include "mod_gemv.hpp"

namespace dit {

// ------------------------------------------------------------------------
// Row kernels: one wavefront per row, each lane owning NCH 16-byte chunks
// (8 bf16) at chunk index lane + 64*j.
// ------------------------------------------------------------------------
// 8 consecutive input values of a row: one 16-byte load of bf16, or two of fp32
template <class TI>
struct Chunk8;
template <>
struct Chunk8<bf16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const bf16_t* row, int c) { v = reinterpret_cast<const u32x4*>(row)[c]; }
  __device__ __forceinline__ void get(float* f) const { unpack8(v, f); }
};
template <>
struct Chunk8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* row, int c) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row) + 2 * c;
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void get(float* f) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
};

// LayerNorm + modulate: one wavefront per row and two per workgroup, so all
// of a row's loads are in flight at once and 18 rows per CU at the Flux shape
// (4608 rows); (1 + scale) and shift are read at the store from L1/L2.
// Measured at 4608 x 3072 from HBM: 15.4 us, against 17.2 us when each wave
// walked 3 rows with the next row's loads in flight and the per-column
// vectors held in registers.
// Rows [0, split) use (shift, scale), rows [split, rows) (shift1, scale1):
// the two streams of a two-stream block in one launch.
template <int NCH, class TI>
__global__ void __launch_bounds__(128)
ln_modulate_kernel(const TI* x, const float* __restrict__ shift, const float* __restrict__ scale,
                   bf16_t* out, int rows, int cols, float eps, int split, const float* __restrict__ shift1,
                   const float* __restrict__ scale1) {  // out may alias x
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 2 + (threadIdx.x >> 6);
  if (r >= rows) return;
  if (r >= split) {
    shift = shift1;
    scale = scale1;
  }
  const int nchunk = cols >> 3;
  Chunk8<TI> in[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) in[j].load(x + size_t(r) * cols, c);
  }
  const float inv_n = 1.0f / float(cols);
  float v[NCH][8];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      in[j].get(v[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[j][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    }
  }
  const float mean = wave_sum(s) * inv_n;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dlt = v[j][e] - mean;
        q += dlt * dlt;
      }
    }
  }
  const float var = wave_sum(q) * inv_n;
  const float rstd = __frsqrt_rn(var + eps);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      const f32x4* ps = reinterpret_cast<const f32x4*>(scale + 8 * c);
      const f32x4* pt = reinterpret_cast<const f32x4*>(shift + 8 * c);
      const f32x4 s0 = ps[0], s1 = ps[1], t0 = pt[0], t1 = pt[1];
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (v[j][e] - mean) * rstd * (1.0f + s0[e]) + t0[e];
        o[4 + e] = (v[j][4 + e] - mean) * rstd * (1.0f + s1[e]) + t1[e];
      }
      reinterpret_cast<u32x4*>(out + size_t(r) * cols)[c] = pack8(o);
    }
  }
}

// Gated residual y = x + gate * h: one wavefront per row, two per workgroup;
// the gate is read at the store from L1/L2 (19.2 us at 4608 x 3072 from HBM,
// against 20.9 us with 3 rows per wave and the gate held in registers).
template <int NCH>
__global__ void __launch_bounds__(128)
gated_residual_kernel(const bf16_t* x, const bf16_t* h, const float* __restrict__ gate, bf16_t* y,
                      int rows, int cols) {  // y may alias x or h
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 2 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nchunk = cols >> 3;
  u32x4 xv[NCH], hv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      xv[j] = reinterpret_cast<const u32x4*>(x + size_t(r) * cols)[c];
      hv[j] = reinterpret_cast<const u32x4*>(h + size_t(r) * cols)[c];
    }
  }
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      const f32x4* pg = reinterpret_cast<const f32x4*>(gate + 8 * c);
      const f32x4 g0 = pg[0], g1 = pg[1];
      float a[8], b[8], o[8];
      unpack8(xv[j], a);
      unpack8(hv[j], b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = a[e] + g0[e] * b[e];
        o[4 + e] = a[4 + e] + g1[e] * b[4 + e];
      }
      reinterpret_cast<u32x4*>(y + size_t(r) * cols)[c] = pack8(o);
    }
  }
}

// ------------------------------------------------------------------------
// Per-head QK RMSNorm + RoPE, in place.  One thread owns 8 consecutive dims
// (4 rotation pairs) of one (token, q|k, head) row; the DH/8 threads of a row
// reduce the sum of squares with lane shuffles.
// ------------------------------------------------------------------------
template <int DH>
__global__ void __launch_bounds__(256)
qk_rmsnorm_rope_kernel(bf16_t* __restrict__ qkv, const float* __restrict__ qw,
                       const float* __restrict__ kw, const float* __restrict__ rcos,
                       const float* __restrict__ rsin, int S, int H, float eps) {
  constexpr int TPR = DH / 8;  // threads per head row
  const int d = H * DH;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)S * 2 * H * TPR;
  // Rows never straddle a wave (TPR divides 64), so inactive lanes are whole rows.
  const bool active = gid < nthreads;
  const long long g = active ? gid : 0;
  const int part = int(g % TPR);  // chunk inside the head row
  const long long row = g / TPR;  // (token, q|k, head)
  const int head = int(row % H);
  const int qk = int((row / H) % 2);
  const int t = int(row / (2 * H));
  bf16_t* p = qkv + (size_t)t * 3 * d + qk * d + head * DH + part * 8;
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  float f[8];
  unpack8(v, f);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  ss = group_sum<TPR>(ss);
  const float rs = __frsqrt_rn(ss * (1.0f / DH) + eps);
  const float* w = (qk == 0 ? qw : kw) + part * 8;
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(w);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + 4);
  const f32x4 c4 = *reinterpret_cast<const f32x4*>(rcos + (size_t)t * (DH / 2) + part * 4);
  const f32x4 s4 = *reinterpret_cast<const f32x4*>(rsin + (size_t)t * (DH / 2) + part * 4);
  float n[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    n[e] = f[e] * rs * w0[e];
    n[4 + e] = f[4 + e] * rs * w1[e];
  }
  float o[8];
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const float a = n[2 * pr], b = n[2 * pr + 1];
    o[2 * pr] = a * c4[pr] - b * s4[pr];
    o[2 * pr + 1] = a * s4[pr] + b * c4[pr];
  }
  if (active) *reinterpret_cast<u32x4*>(p) = pack8(o);
}

// ------------------------------------------------------------------------
// RoPE tables: angle = pos[t, a] * base^(-2 j' / D_a) for pair j (axis a,
// index j' inside the axis chunk of D_a dims).
// ------------------------------------------------------------------------
struct RopeAxes {
  int n_axes;
  int dims[8];
};

__global__ void rope_table_kernel(const int32_t* __restrict__ pos, RopeAxes ax, int S, int half,
                                  float log2_base, float* __restrict__ rcos,
                                  float* __restrict__ rsin) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)S * half) return;
  const int t = int(i / half);
  const int j = int(i % half);
  int a = 0, start = 0;
  while (a < ax.n_axes - 1 && j >= start + ax.dims[a] / 2) {
    start += ax.dims[a] / 2;
    ++a;
  }
  const int jp = j - start;
  const float freq = exp2f(-(2.0f * float(jp) / float(ax.dims[a])) * log2_base);
  const float ang = float(pos[(size_t)t * ax.n_axes + a]) * freq;
  float s, c;
  sincosf(ang, &s, &c);
  rcos[i] = c;
  rsin[i] = s;
}

// ------------------------------------------------------------------------
// Modulation GEMVs: mod[r] = sum_c W[r, c] * SiLU(temb[c]) + b[r] for the
// matrices of a table (one block, the two streams of a block, or a whole
// block stack in one launch): matrix m (rows_per_mat rows) gives
// mods[m * rows_per_mat + r].  SiLU(temb) is computed once per workgroup into
// LDS; a wave walks `rows_per_wave` consecutive rows with 16-byte loads,
// loads the next row's chunks before it reduces the current one, and reduces
// across the wave.  Every row's arithmetic is the same whatever the table,
// so a stack's batched launch gives bitwise the results of per-block ones.
// ------------------------------------------------------------------------
template <int NCH, class Tab>
__global__ void __launch_bounds__(256)
mod_gemv_multi_kernel(const bf16_t* __restrict__ temb, Tab tab, float* __restrict__ mods, int rows_per_mat,
                      int rows, int cols, int rows_per_wave) {
  __shared__ __attribute__((aligned(16))) float s_act[NCH * 512];
  mod_gemv_rows<NCH>(temb, tab, mods, rows_per_mat, rows, cols, rows_per_wave,
                     blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), s_act);
}

// ------------------------------------------------------------------------
// Step prediction for a skipped denoising step: y = a + w (a - b) over n
// bf16 values (a, b the outputs of the last two computed steps), or y = a
// when b is NULL; written to y1 and, when non-NULL, also to y2.  Flat
// streaming: each workgroup owns a contiguous run of 4 x 256 16-byte chunks.
// ------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
extrapolate_kernel(const bf16_t* __restrict__ a, const bf16_t* __restrict__ b, float w, bf16_t* __restrict__ y1,
                   bf16_t* __restrict__ y2, long long n8) {
  const long long base = (long long)blockIdx.x * 1024;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const long long i = base + k * 256 + threadIdx.x;
    if (i >= n8) return;
    float fa[8], o[8];
    unpack8(reinterpret_cast<const u32x4*>(a)[i], fa);
    if (b) {
      float fb[8];
      unpack8(reinterpret_cast<const u32x4*>(b)[i], fb);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(w, fa[e] - fb[e], fa[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fa[e];
    }
    const u32x4 v = pack8(o);
    reinterpret_cast<u32x4*>(y1)[i] = v;
    if (y2) reinterpret_cast<u32x4*>(y2)[i] = v;
  }
}

// ------------------------------------------------------------------------ launchers
static int rows_per_wave_for(int rows, int target_waves) {
  int rpw = (rows + target_waves - 1) / target_waves;
  return rpw < 1 ? 1 : rpw;
}

template <class TI>
static hipError_t launch_ln_modulate(const TI* x, const float* shift, const float* scale, bf16_t* out, int rows,
                                     int cols, float eps, hipStream_t st, int split, const float* shift1,
                                     const float* scale1) {
  if (rows == 0) return hipSuccess;
  const int nch = (cols / 8 + 63) / 64;
  dim3 grid((rows + 1) / 2), block(128);
  switch (nch) {
#define CASE(N) \
  case N:                                                                                             \
    ln_modulate_kernel<N, TI><<<grid, block, 0, st>>>(x, shift, scale, out, rows, cols, eps, split, shift1, \
                                                      scale1);                                            \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10) CASE(11) CASE(12)
    CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_modulate_norm(const bf16_t* x, const float* shift, const float* scale,
                                bf16_t* out, int rows, int cols, float eps, hipStream_t st) {
  return launch_ln_modulate(x, shift, scale, out, rows, cols, eps, st, rows, shift, scale);
}

hipError_t launch_modulate_norm(const float* x, const float* shift, const float* scale,
                                bf16_t* out, int rows, int cols, float eps, hipStream_t st) {
  return launch_ln_modulate(x, shift, scale, out, rows, cols, eps, st, rows, shift, scale);
}

hipError_t launch_modulate_norm_pair(const bf16_t* x, const float* shift0, const float* scale0, const float* shift1,
                                     const float* scale1, int split, bf16_t* out, int rows, int cols, float eps,
                                     hipStream_t st) {
  return launch_ln_modulate(x, shift0, scale0, out, rows, cols, eps, st, split, shift1, scale1);
}

hipError_t launch_modulate_norm_pair(const float* x, const float* shift0, const float* scale0, const float* shift1,
                                     const float* scale1, int split, bf16_t* out, int rows, int cols, float eps,
                                     hipStream_t st) {
  return launch_ln_modulate(x, shift0, scale0, out, rows, cols, eps, st, split, shift1, scale1);
}

hipError_t launch_gated_residual(const bf16_t* x, const bf16_t* h, const float* gate, bf16_t* y,
                                 int rows, int cols, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int nch = (cols / 8 + 63) / 64;
  dim3 grid((rows + 1) / 2), block(128);
  switch (nch) {
#define CASE(N) \
  case N: gated_residual_kernel<N><<<grid, block, 0, st>>>(x, h, gate, y, rows, cols); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10) CASE(11) CASE(12)
    CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class Tab>
static hipError_t launch_mod_multi(const bf16_t* temb, const Tab& tab, float* mods, int n_mats, int rows_per_mat,
                                   int cols, int target_waves, hipStream_t st) {
  const int rows = n_mats * rows_per_mat;
  if (rows == 0) return hipSuccess;
  const int nch = (cols / 8 + 63) / 64;
  const int rpw = rows_per_wave_for(rows, target_waves);
  const int waves = (rows + rpw - 1) / rpw;
  dim3 grid((waves + 3) / 4), block(256);
  switch (nch) {
#define CASE(N) \
  case N: mod_gemv_multi_kernel<N, Tab><<<grid, block, 0, st>>>(temb, tab, mods, rows_per_mat, rows, cols, rpw); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10) CASE(11) CASE(12)
    CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_modulation_multi(const bf16_t* temb, const bf16_t* const* ws, const bf16_t* const* bs,
                                   float* mods, int n_mats, int rows_per_mat, int cols, hipStream_t st) {
  return launch_mod_multi(temb, ModTabDev{ws, bs}, mods, n_mats, rows_per_mat, cols, 8192, st);
}

hipError_t launch_modulation_pair(const bf16_t* temb, const bf16_t* w0, const bf16_t* b0, const bf16_t* w1,
                                  const bf16_t* b1, int n_mats, float* mods, int rows_per_mat, int cols,
                                  hipStream_t st) {
  if (n_mats < 0 || n_mats > 2) return hipErrorInvalidValue;
  ModTab2 tab;
  tab.ws[0] = w0;
  tab.ws[1] = w1;
  tab.bs[0] = b0;
  tab.bs[1] = b1;
  return launch_mod_multi(temb, tab, mods, n_mats, rows_per_mat, cols, 4096, st);
}

hipError_t launch_modulation(const bf16_t* temb, const bf16_t* w, const bf16_t* b, float* mod, int rows, int cols,
                             hipStream_t st) {
  return launch_modulation_pair(temb, w, b, nullptr, nullptr, 1, mod, rows, cols, st);
}

hipError_t launch_qk_rmsnorm_rope(bf16_t* qkv, const float* qw, const float* kw, const float* rcos,
                                  const float* rsin, int S, int H, int DH, float eps,
                                  hipStream_t st) {
  if (S == 0) return hipSuccess;
  const long long threads = (long long)S * 2 * H * (DH / 8);
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (DH == 128)
    qk_rmsnorm_rope_kernel<128><<<grid, block, 0, st>>>(qkv, qw, kw, rcos, rsin, S, H, eps);
  else if (DH == 64)
    qk_rmsnorm_rope_kernel<64><<<grid, block, 0, st>>>(qkv, qw, kw, rcos, rsin, S, H, eps);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rope_table(const int32_t* pos, int S, int n_axes, const int32_t* axes_dims,
                             int DH, float base, float* rcos, float* rsin, hipStream_t st) {
  if (S == 0) return hipSuccess;
  RopeAxes ax;
  ax.n_axes = n_axes;
  for (int i = 0; i < 8; ++i) ax.dims[i] = i < n_axes ? axes_dims[i] : 0;
  const int half = DH / 2;
  const long long n = (long long)S * half;
  const double l2b = std::log2((double)base);
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(pos, ax, S, half, (float)l2b,
                                                                 rcos, rsin);
  return hipGetLastError();
}

// Timing probe: one thread reads the constant-rate wall clock.  finish == 0
// stores the stamp in ch[0]; finish != 0 adds (now - ch[0]) to ch[1].  Nodes of
// a captured stream run in order, so the read-modify-write needs no atomics.
__global__ void probe_stamp_kernel(unsigned long long* ch, int finish) {
  if (threadIdx.x != 0) return;
  const unsigned long long t = wall_clock64();
  if (finish)
    ch[1] += t - ch[0];
  else
    ch[0] = t;
}

hipError_t launch_probe_stamp(unsigned long long* ch, int finish, hipStream_t st) {
  probe_stamp_kernel<<<1, 64, 0, st>>>(ch, finish);
  return hipGetLastError();
}

hipError_t launch_extrapolate(const bf16_t* a, const bf16_t* b, float w, bf16_t* y1, bf16_t* y2, size_t n,
                              hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (n % 8 != 0) return hipErrorInvalidValue;
  const long long n8 = (long long)(n / 8);
  extrapolate_kernel<<<dim3((unsigned)((n8 + 1023) / 1024)), dim3(256), 0, st>>>(a, b, w, y1, y2, n8);
  return hipGetLastError();
}

}  // namespace dit

// Internal launch functions of libdit_block (one per kernel family).  Each
// only enqueues on `st` and returns the launch status; callers validate the
// arguments first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;

// Cache device properties used for launch shapes (call before a stream capture).
void prepare_device();
// compute units of the current device (cached on first use)
int num_cus();

hipError_t launch_modulation(const bf16_t* temb, const bf16_t* w, const bf16_t* b, float* mod,
                             int rows, int cols, hipStream_t st);
// n_mats modulation GEMVs in one launch: mods[m * rows_per_mat + r] from
// ws[m] [rows_per_mat, cols] and bs[m] (DEVICE arrays of pointers; bs[m] may be NULL)
hipError_t launch_modulation_multi(const bf16_t* temb, const bf16_t* const* ws, const bf16_t* const* bs,
                                   float* mods, int n_mats, int rows_per_mat, int cols, hipStream_t st);
// the same for n_mats <= 2 matrices passed by value (the streams of one block)
hipError_t launch_modulation_pair(const bf16_t* temb, const bf16_t* w0, const bf16_t* b0, const bf16_t* w1,
                                  const bf16_t* b1, int n_mats, float* mods, int rows_per_mat, int cols,
                                  hipStream_t st);
hipError_t launch_modulate_norm(const bf16_t* x, const float* shift, const float* scale,
                                bf16_t* out, int rows, int cols, float eps, hipStream_t st);
// the same with an fp32 input x [rows, cols]
hipError_t launch_modulate_norm(const float* x, const float* shift, const float* scale,
                                bf16_t* out, int rows, int cols, float eps, hipStream_t st);
// the two streams of a two-stream block in one launch: rows [0, split) with
// (shift0, scale0), rows [split, rows) with (shift1, scale1)
hipError_t launch_modulate_norm_pair(const bf16_t* x, const float* shift0, const float* scale0, const float* shift1,
                                     const float* scale1, int split, bf16_t* out, int rows, int cols, float eps,
                                     hipStream_t st);
hipError_t launch_modulate_norm_pair(const float* x, const float* shift0, const float* scale0, const float* shift1,
                                     const float* scale1, int split, bf16_t* out, int rows, int cols, float eps,
                                     hipStream_t st);
hipError_t launch_gated_residual(const bf16_t* x, const bf16_t* h, const float* gate, bf16_t* y,
                                 int rows, int cols, hipStream_t st);
hipError_t launch_qk_rmsnorm_rope(bf16_t* qkv, const float* qw, const float* kw, const float* rcos,
                                  const float* rsin, int S, int H, int DH, float eps,
                                  hipStream_t st);
hipError_t launch_rope_table(const int32_t* pos, int S, int n_axes, const int32_t* axes_dims,
                             int DH, float base, float* rcos, float* rsin, hipStream_t st);

// linear1: z = u W1^T + b1; cols < 3d -> qkv[S,3d]; cols >= 3d -> gelu -> cat[:, d + ...]
hipError_t launch_linear1(const bf16_t* u, const bf16_t* w1, const bf16_t* b1, bf16_t* qkv,
                          bf16_t* cat, int S, int d, int mlp, hipStream_t st);
// linear1 with the q/k RMSNorm + RoPE fused into its epilogue (q and k are
// rounded to bf16 once, after both); for the shapes where linear1_fuses_qk()
// holds (head_dim 64 or 128, dim % 64 == 0)
bool linear1_fuses_qk(int S, int d, int mlp, int DH);
hipError_t launch_linear1_qk(const bf16_t* u, const bf16_t* w1, const bf16_t* b1, bf16_t* qkv, bf16_t* cat,
                             int S, int d, int mlp, int DH, const float* qw, const float* kw, const float* rcos,
                             const float* rsin, float eps, hipStream_t st);
// linear2: y = x + gate * (cat W2^T + b2)
hipError_t launch_linear2(const bf16_t* cat, const bf16_t* w2, const bf16_t* b2, const bf16_t* x,
                          const float* gate, bf16_t* y, int S, int d, int mlp, hipStream_t st);
// Grouped linears: one launch for 1 or 2 independent problems (the text and
// image streams of a two-stream block), tiles of both spread over the chip.
// z = A W^T + b with A [M, K], W [N, K]; columns [0, n_plain) -> plain (row
// stride ld_plain), columns [n_plain, N) -> GELU-tanh -> gelu[:, gelu_col0 + ...]
// (row stride ld_gelu).  qk_dim: width of q and of k for the fused head norm.
struct BiasActArgs {
  const bf16_t* A;
  const bf16_t* W;
  const bf16_t* b;
  int M, N, K, n_plain;
  bf16_t* plain;
  int ld_plain;
  bf16_t* gelu;
  int ld_gelu, gelu_col0, qk_dim;
};
// per-head RMSNorm + RoPE of the q and k columns (tables [M, head_dim/2] for these rows)
struct QKNormArgs {
  const float* qw;
  const float* kw;
  const float* rcos;
  const float* rsin;
  float eps;
};
// y = x + gate * (A W^T + b), x and y [M, N] (may alias), gate [N] fp32
struct GatedArgs {
  const bf16_t* A;
  const bf16_t* W;
  const bf16_t* b;
  const bf16_t* x;
  const float* gate;
  bf16_t* y;
  int M, N, K;
};
hipError_t launch_bias_act_group(const BiasActArgs* a, int np, hipStream_t st);
bool bias_act_fuses_qk(const BiasActArgs* a, int np, int DH);
hipError_t launch_bias_act_qk_group(const BiasActArgs* a, const QKNormArgs* q, int np, int DH, hipStream_t st);
hipError_t launch_gated_group(const GatedArgs* a, int np, hipStream_t st);
// the same with an fp32 output y32[i] [M, N] (a[i].y unused) ...
hipError_t launch_gated_f32out_group(const GatedArgs* a, float* const* y32, int np, hipStream_t st);
// ... or with an fp32 residual x32[i] [M, N] (a[i].x unused)
hipError_t launch_gated_f32in_group(const GatedArgs* a, const float* const* x32, int np, hipStream_t st);

// attention over qkv [S, 3*H*DH] -> out [S, ld_out] columns [0, H*DH)
hipError_t launch_attention(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out,
                            hipStream_t st);
// whether launch_attention_mod takes this shape: an attention on 8-wave
// workgroups whose last round leaves CUs idle, and a supported GEMV width
bool attention_hosts_modulation(int S, int H, int DH, int mod_cols);
// the same attention plus, in workgroups dispatched after it, the
// modulation GEMVs of n_mats (1 or 2) matrices of rows_per_mat rows and
// mod_cols columns: mods[m * rows_per_mat + r] = W_m[r] . SiLU(temb) + b_m[r],
// bitwise those of launch_modulation / launch_modulation_pair
hipError_t launch_attention_mod(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out,
                                const bf16_t* temb, const bf16_t* w0, const bf16_t* b0, const bf16_t* w1,
                                const bf16_t* b1, int n_mats, float* mods, int rows_per_mat, int mod_cols,
                                hipStream_t st);
// attention over keys [kv_begin, kv_end): o_part [S, H*DH] fp32, lse [H, S] fp32
hipError_t launch_attention_partial(const bf16_t* qkv, int S, int H, int DH, int kv_begin, int kv_end,
                                    float* o_part, float* lse, hipStream_t st);
// number of non-empty key chunks when S keys are cut into n_chunks equal chunks
int attention_chunks(int S, int n_chunks);
// attention over all S keys as attention_chunks(S, n_chunks) partials in one
// launch (scratch o_parts [n, S, H*DH], lses [n, H, S]) plus the merge
hipError_t launch_attention_split(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out, int n_chunks,
                                  float* o_parts, float* lses, hipStream_t st);
// out[t, :H*DH] (row stride ld_out) = lse-weighted sum of n_chunks partials
hipError_t launch_attention_merge(const float* o_parts, const float* lses, int n_chunks, int S, int H, int DH,
                                  bf16_t* out, int ld_out, hipStream_t st);

// y1 (and y2 if non-NULL) = a + w (a - b), or a when b is NULL; n bf16 values, n % 8 == 0
hipError_t launch_extrapolate(const bf16_t* a, const bf16_t* b, float w, bf16_t* y1, bf16_t* y2, size_t n,
                              hipStream_t st);

// timing probe channel ch[2]: finish == 0 stamps ch[0], else ch[1] += now - ch[0]
hipError_t launch_probe_stamp(unsigned long long* ch, int finish, hipStream_t st);

// ceiling probes: a streaming copy of `bytes` (a multiple of 16) and
// n_workgroups x 4 waves x iters x 4 bf16 32x32x16 MFMAs (out: n_workgroups*256 floats)
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
hipError_t launch_probe_mfma(float* out, int n_workgroups, int iters, int vary, hipStream_t st);

}  // namespace dit

// C ABI of libdit_block: argument checks, the block schedules (single-stream,
// two-stream and sequential blocks) and the captured block stack.  Host code
// only; the kernels live in elementwise.hip, gemm.hip and attention.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "dit_block.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  if (std::getenv("DIT_LOG")) std::fprintf(stderr, "[libdit_block] error %d: %s\n", code, buf);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define DIT_CHECK_HIP(expr, what)          \
  do {                                     \
    hipError_t _e = (expr);                \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxRowCols = 8192;  // row kernels keep a row in one wavefront's registers
constexpr int64_t kMaxInt = 0x7fffffff;

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int check_rows_cols(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return fail(DIT_ERR_INVALID_ARG, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
  if (cols % 8 != 0 || cols > kMaxRowCols)
    return fail(DIT_ERR_UNSUPPORTED, "cols=%lld must be a multiple of 8 and <= %lld", (long long)cols, (long long)kMaxRowCols);
  if (rows > kMaxInt || rows * cols > (int64_t(1) << 40)) return fail(DIT_ERR_UNSUPPORTED, "rows=%lld too large", (long long)rows);
  return DIT_OK;
}

// dims shared by the whole-block paths
struct Dims {
  int S, d, H, Dh, mlp, tdim;
};

int check_dims(int64_t S, int64_t d, int64_t H, int64_t Dh, int64_t mlp, int64_t tdim) {
  if (S < 0 || d <= 0 || H <= 0 || Dh <= 0 || mlp <= 0 || tdim <= 0)
    return fail(DIT_ERR_INVALID_ARG, "bad dims S=%lld d=%lld H=%lld Dh=%lld mlp=%lld temb=%lld",
                (long long)S, (long long)d, (long long)H, (long long)Dh, (long long)mlp, (long long)tdim);
  if (Dh != 64 && Dh != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim=%lld not in {64,128}", (long long)Dh);
  if (H * Dh != d) return fail(DIT_ERR_INVALID_ARG, "num_heads*head_dim=%lld != dim=%lld", (long long)(H * Dh), (long long)d);
  if (d % 64 != 0 || d > kMaxRowCols) return fail(DIT_ERR_UNSUPPORTED, "dim=%lld must be a multiple of 64 and <= 8192", (long long)d);
  if (mlp % 64 != 0 || mlp > (int64_t(1) << 20)) return fail(DIT_ERR_UNSUPPORTED, "mlp_hidden=%lld must be a multiple of 64", (long long)mlp);
  if (tdim % 8 != 0 || tdim > kMaxRowCols) return fail(DIT_ERR_UNSUPPORTED, "temb_dim=%lld must be a multiple of 8 and <= 8192", (long long)tdim);
  if (S > (1 << 24)) return fail(DIT_ERR_UNSUPPORTED, "seq_len=%lld too large", (long long)S);
  return DIT_OK;
}

int dims_of(const dit_block_config* cfg, Dims* out) {
  if (!cfg) return fail(DIT_ERR_INVALID_ARG, "cfg is NULL");
  const int tdim = cfg->temb_dim ? cfg->temb_dim : cfg->dim;
  int rc = check_dims(cfg->seq_len, cfg->dim, cfg->num_heads, cfg->head_dim, cfg->mlp_hidden, tdim);
  if (rc) return rc;
  if (!(cfg->ln_eps >= 0.f) || !(cfg->qk_eps >= 0.f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
  *out = Dims{cfg->seq_len, cfg->dim, cfg->num_heads, cfg->head_dim, cfg->mlp_hidden, tdim};
  return DIT_OK;
}

// Tensor pointers must be 16-byte aligned (the kernels use 16-byte vector and
// direct-to-LDS accesses); NULL entries are skipped (optional tensors).
int check_aligned(std::initializer_list<const void*> ps) {
  int i = 0;
  for (const void* p : ps) {
    if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return fail(DIT_ERR_INVALID_ARG, "tensor pointer %d (%p) is not 16-byte aligned", i, p);
    ++i;
  }
  return DIT_OK;
}

int check_weights(const dit_block_weights* w) {
  if (!w) return fail(DIT_ERR_INVALID_ARG, "weights is NULL");
  if (!w->w_mod || !w->w1 || !w->w2 || !w->q_norm_w || !w->k_norm_w)
    return fail(DIT_ERR_INVALID_ARG, "a required weight pointer is NULL");
  return check_aligned({w->w_mod, w->b_mod, w->w1, w->b1, w->w2, w->b2, w->q_norm_w, w->k_norm_w});
}

// Workspace of one single-stream block forward.
struct WsLayout {
  size_t mod, u, qkv, cat, block_end;
};

WsLayout layout(const Dims& D) {
  WsLayout L;
  size_t o = 0;
  L.mod = o; o = align256(o + size_t(3) * D.d * sizeof(float));
  L.u = o;   o = align256(o + size_t(D.S) * D.d * 2);
  L.qkv = o; o = align256(o + size_t(D.S) * 3 * D.d * 2);
  L.cat = o; o = align256(o + size_t(D.S) * (D.d + D.mlp) * 2);
  L.block_end = o;
  return L;
}

// Optional timing probes.  Each probed kernel is bracketed by two one-thread
// stamp kernels that read the device wall clock; the second adds the interval
// to an accumulator.  Channel 6 brackets nothing: its interval is the probe's
// own overhead, subtracted on the host.
constexpr int kProbeChannels = 7;
struct Probe {
  uint32_t mask = 0;                   // bit i: kernel i of the block (0..5)
  unsigned long long* ch = nullptr;    // [kProbeChannels][2] for this block
};

// The next block's modulation, computed by a block's attention launch in
// the CUs its last round leaves idle: n_mats (1 or 2: a two-stream block's
// present streams, text first) matrices W_mod of rows_per_mat rows, their
// biases, and the output vectors [n_mats][rows_per_mat].
struct NextMod {
  const dit_bf16* w[2];
  const dit_bf16* b[2];
  int n_mats, rows_per_mat;
  float* out;
};

// The attention of a block, with the next block's modulation when `next`.
hipError_t enqueue_attention(const Dims& D, const dit_bf16* qkv, dit_bf16* out, int ld_out, const dit_bf16* temb,
                             const NextMod* next, hipStream_t st) {
  if (!next) return dit::launch_attention(qkv, out, D.S, D.H, D.Dh, ld_out, st);
  return dit::launch_attention_mod(qkv, out, D.S, D.H, D.Dh, ld_out, temb, next->w[0], next->b[0], next->w[1],
                                   next->b[1], next->n_mats, next->out, next->rows_per_mat, D.tdim, st);
}

// The launches of one block on `st`.  x and y may alias.  With mod_pre the
// modulation vectors were computed beforehand (by a stack's step-level
// launch or by the previous block's attention launch) and the block's GEMV
// is skipped.  With next (only where attention_hosts_modulation holds), the
// attention launch also computes the next block's modulation vectors.
int enqueue_block(const Dims& D, const dit_block_config* cfg, const dit_block_weights* w,
                  const dit_bf16* x, const dit_bf16* temb, const float* rcos, const float* rsin,
                  dit_bf16* y, unsigned char* ws, hipStream_t st, const Probe& pr = Probe(),
                  const float* mod_pre = nullptr, const NextMod* next = nullptr) {
  const WsLayout L = layout(D);
  const float* mod = mod_pre ? mod_pre : reinterpret_cast<float*>(ws + L.mod);
  dit_bf16* u = reinterpret_cast<dit_bf16*>(ws + L.u);
  dit_bf16* qkv = reinterpret_cast<dit_bf16*>(ws + L.qkv);
  dit_bf16* cat = reinterpret_cast<dit_bf16*>(ws + L.cat);
  auto pre = [&](int k) -> hipError_t {
    return (pr.mask >> k & 1u) ? dit::launch_probe_stamp(pr.ch + 2 * k, 0, st) : hipSuccess;
  };
  auto post = [&](int k) -> hipError_t {
    return (pr.mask >> k & 1u) ? dit::launch_probe_stamp(pr.ch + 2 * k, 1, st) : hipSuccess;
  };
  if (pr.mask) {
    DIT_CHECK_HIP(dit::launch_probe_stamp(pr.ch + 12, 0, st), "probe");
    DIT_CHECK_HIP(dit::launch_probe_stamp(pr.ch + 12, 1, st), "probe");
  }
  // with mod_pre the bracket of kernel 0 is empty (its probe then reads ~0)
  DIT_CHECK_HIP(pre(0), "probe");
  if (!mod_pre)
    DIT_CHECK_HIP(dit::launch_modulation(temb, w->w_mod, w->b_mod, reinterpret_cast<float*>(ws + L.mod), 3 * D.d,
                                         D.tdim, st), "modulation");
  DIT_CHECK_HIP(post(0), "probe");
  if (D.S == 0) return DIT_OK;
  DIT_CHECK_HIP(pre(1), "probe");
  DIT_CHECK_HIP(dit::launch_modulate_norm(x, mod, mod + D.d, u, D.S, D.d, cfg->ln_eps, st), "modulate_norm");
  DIT_CHECK_HIP(post(1), "probe");
  if (dit::linear1_fuses_qk(D.S, D.d, D.mlp, D.Dh)) {
    // the q/k RMSNorm + RoPE runs in linear1's epilogue (kernel 3 is empty)
    DIT_CHECK_HIP(pre(2), "probe");
    DIT_CHECK_HIP(dit::launch_linear1_qk(u, w->w1, w->b1, qkv, cat, D.S, D.d, D.mlp, D.Dh, w->q_norm_w,
                                         w->k_norm_w, rcos, rsin, cfg->qk_eps, st), "linear1_qk");
    DIT_CHECK_HIP(post(2), "probe");
    DIT_CHECK_HIP(pre(3), "probe");
    DIT_CHECK_HIP(post(3), "probe");
  } else {
    DIT_CHECK_HIP(pre(2), "probe");
    DIT_CHECK_HIP(dit::launch_linear1(u, w->w1, w->b1, qkv, cat, D.S, D.d, D.mlp, st), "linear1");
    DIT_CHECK_HIP(post(2), "probe");
    DIT_CHECK_HIP(pre(3), "probe");
    DIT_CHECK_HIP(dit::launch_qk_rmsnorm_rope(qkv, w->q_norm_w, w->k_norm_w, rcos, rsin, D.S, D.H, D.Dh,
                                              cfg->qk_eps, st), "qk_rmsnorm_rope");
    DIT_CHECK_HIP(post(3), "probe");
  }
  DIT_CHECK_HIP(pre(4), "probe");
  DIT_CHECK_HIP(enqueue_attention(D, qkv, cat, D.d + D.mlp, temb, next, st), "attention");
  DIT_CHECK_HIP(post(4), "probe");
  DIT_CHECK_HIP(pre(5), "probe");
  DIT_CHECK_HIP(dit::launch_linear2(cat, w->w2, w->b2, x, mod + 2 * D.d, y, D.S, D.d, D.mlp, st), "linear2");
  DIT_CHECK_HIP(post(5), "probe");
  return DIT_OK;
}

// ---------------------------------------------- two-stream / sequential blocks
int check_stream_weights(const dit_stream_weights* w, const char* which) {
  if (!w) return fail(DIT_ERR_INVALID_ARG, "%s weights are NULL", which);
  if (!w->w_mod || !w->w_qkv || !w->q_norm_w || !w->k_norm_w || !w->w_o || !w->w_fc1 || !w->w_fc2)
    return fail(DIT_ERR_INVALID_ARG, "a required %s weight pointer is NULL", which);
  return check_aligned({w->w_mod, w->b_mod, w->w_qkv, w->b_qkv, w->q_norm_w, w->k_norm_w, w->w_o, w->b_o,
                        w->w_fc1, w->b_fc1, w->w_fc2, w->b_fc2});
}

struct MmLayout {
  size_t mod, u, qkv, o, x1, h, end;
};

MmLayout mm_layout(const Dims& D) {
  MmLayout L;
  size_t o = 0;
  L.mod = o; o = align256(o + size_t(2) * 6 * D.d * sizeof(float));
  L.u = o;   o = align256(o + size_t(D.S) * D.d * 2);
  L.qkv = o; o = align256(o + size_t(D.S) * 3 * D.d * 2);
  L.o = o;   o = align256(o + size_t(D.S) * D.d * 2);
  L.x1 = o;  o = align256(o + size_t(D.S) * D.d * 4);
  L.h = o;   o = align256(o + size_t(D.S) * D.mlp * 2);
  L.end = o;
  return L;
}

// The launches of one two-stream block on `st`: stream 0 = text rows
// [0, T), stream 1 = image rows [T, S); empty streams are skipped.  Each
// linear is one grouped launch over both streams.  The residual between the
// attention and MLP halves (x') stays fp32.  x and y may alias.
int enqueue_mmdit(const Dims& D, int T, const dit_block_config* cfg, const dit_stream_weights* wt,
                  const dit_stream_weights* wi, const dit_bf16* x, const dit_bf16* temb, const float* rcos,
                  const float* rsin, dit_bf16* y, unsigned char* ws, hipStream_t st, const float* mod_pre = nullptr,
                  const NextMod* next = nullptr) {
  const MmLayout L = mm_layout(D);
  const int d = D.d, mlp = D.mlp, half = D.Dh / 2;
  // mod_pre: the present streams' six vectors, text first, computed beforehand
  float* mod0 = mod_pre ? const_cast<float*>(mod_pre) : reinterpret_cast<float*>(ws + L.mod);
  dit_bf16* u = reinterpret_cast<dit_bf16*>(ws + L.u);
  dit_bf16* qkv = reinterpret_cast<dit_bf16*>(ws + L.qkv);
  dit_bf16* o = reinterpret_cast<dit_bf16*>(ws + L.o);
  float* x1 = reinterpret_cast<float*>(ws + L.x1);
  dit_bf16* h = reinterpret_cast<dit_bf16*>(ws + L.h);
  struct Stream {
    const dit_stream_weights* w;
    int r0, rows;
    float* mod;
  } ss[2];
  int n = 0;
  if (T > 0) ss[n++] = Stream{wt, 0, T, mod0};
  if (D.S - T > 0) ss[n++] = Stream{wi, T, D.S - T, mod0 + n * 6 * d};
  if (n == 0) return DIT_OK;
  const size_t rd = size_t(d);
  if (!mod_pre)  // both streams' GEMVs in one launch
    DIT_CHECK_HIP(dit::launch_modulation_pair(temb, ss[0].w->w_mod, ss[0].w->b_mod, ss[n - 1].w->w_mod,
                                              ss[n - 1].w->b_mod, n, mod0, 6 * d, D.tdim, st),
                  "modulation");
  // one launch over both streams' rows: rows below T take the text vectors
  DIT_CHECK_HIP(dit::launch_modulate_norm_pair(x, ss[0].mod, ss[0].mod + d, ss[n - 1].mod, ss[n - 1].mod + d, T, u,
                                               D.S, d, cfg->ln_eps, st), "modulate_norm");
  // q | k | v of both streams into one [S, 3d] buffer (text rows first)
  dit::BiasActArgs qa[2];
  dit::QKNormArgs qn[2];
  for (int i = 0; i < n; ++i) {
    const Stream& s = ss[i];
    qa[i] = dit::BiasActArgs{u + s.r0 * rd, s.w->w_qkv, s.w->b_qkv, s.rows, 3 * d, d, 3 * d,
                             qkv + s.r0 * 3 * rd, 3 * d, nullptr, 0, 0, d};
    qn[i] = dit::QKNormArgs{s.w->q_norm_w, s.w->k_norm_w, rcos + size_t(s.r0) * half, rsin + size_t(s.r0) * half,
                            cfg->qk_eps};
  }
  if (dit::bias_act_fuses_qk(qa, n, D.Dh)) {
    DIT_CHECK_HIP(dit::launch_bias_act_qk_group(qa, qn, n, D.Dh, st), "qkv_qk");
  } else {
    DIT_CHECK_HIP(dit::launch_bias_act_group(qa, n, st), "qkv");
    for (int i = 0; i < n; ++i)
      DIT_CHECK_HIP(dit::launch_qk_rmsnorm_rope(qkv + ss[i].r0 * 3 * rd, qn[i].qw, qn[i].kw, qn[i].rcos, qn[i].rsin,
                                                ss[i].rows, D.H, D.Dh, cfg->qk_eps, st), "qk_rmsnorm_rope");
  }
  DIT_CHECK_HIP(enqueue_attention(D, qkv, o, d, temb, next, st), "attention");
  dit::GatedArgs ga[2];
  float* x1s[2];
  for (int i = 0; i < n; ++i) {
    const Stream& s = ss[i];
    ga[i] = dit::GatedArgs{o + s.r0 * rd, s.w->w_o, s.w->b_o, x + s.r0 * rd, s.mod + 2 * d, nullptr, s.rows, d, d};
    x1s[i] = x1 + s.r0 * rd;
  }
  DIT_CHECK_HIP(dit::launch_gated_f32out_group(ga, x1s, n, st), "proj");
  DIT_CHECK_HIP(dit::launch_modulate_norm_pair(static_cast<const float*>(x1), ss[0].mod + 3 * d, ss[0].mod + 4 * d,
                                               ss[n - 1].mod + 3 * d, ss[n - 1].mod + 4 * d, T, u, D.S, d,
                                               cfg->ln_eps, st), "modulate_norm2");
  dit::BiasActArgs fa[2];
  for (int i = 0; i < n; ++i) {
    const Stream& s = ss[i];
    fa[i] = dit::BiasActArgs{u + s.r0 * rd, s.w->w_fc1, s.w->b_fc1, s.rows, mlp, d, 0, nullptr, 0,
                             h + s.r0 * size_t(mlp), mlp, 0, 0};
  }
  DIT_CHECK_HIP(dit::launch_bias_act_group(fa, n, st), "fc1");
  const float* x1c[2];
  for (int i = 0; i < n; ++i) {
    const Stream& s = ss[i];
    ga[i] = dit::GatedArgs{h + s.r0 * size_t(mlp), s.w->w_fc2, s.w->b_fc2, nullptr, s.mod + 5 * d, y + s.r0 * rd,
                           s.rows, d, mlp};
    x1c[i] = x1s[i];
  }
  DIT_CHECK_HIP(dit::launch_gated_f32in_group(ga, x1c, n, st), "fc2");
  return DIT_OK;
}

int check_linear(int64_t S, int64_t d, int64_t mlp) {
  if (S < 0 || d <= 0 || mlp <= 0)
    return fail(DIT_ERR_INVALID_ARG, "seq_len=%lld dim=%lld mlp_hidden=%lld", (long long)S, (long long)d, (long long)mlp);
  if (d % 64 != 0 || mlp % 64 != 0 || d > kMaxRowCols || mlp > (int64_t(1) << 20) || S > (1 << 24))
    return fail(DIT_ERR_UNSUPPORTED, "dim=%lld and mlp_hidden=%lld must be multiples of 64 (dim <= 8192)",
                (long long)d, (long long)mlp);
  return DIT_OK;
}

int check_not_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone) return fail(DIT_ERR_CAPTURE, "stream is capturing");
  return DIT_OK;
}

}  // namespace

// ============================================================== single steps
extern "C" int dit_modulation(const dit_bf16* temb, const dit_bf16* w_mod, const dit_bf16* b_mod,
                              float* mod, int64_t dim, int64_t temb_dim, void* stream) {
  if (!temb || !w_mod || !mod) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if (dim <= 0 || temb_dim <= 0) return fail(DIT_ERR_INVALID_ARG, "dim=%lld temb_dim=%lld", (long long)dim, (long long)temb_dim);
  if (temb_dim % 8 != 0 || temb_dim > kMaxRowCols) return fail(DIT_ERR_UNSUPPORTED, "temb_dim=%lld", (long long)temb_dim);
  int rc = check_aligned({temb, w_mod, b_mod, mod});
  if (rc) return rc;
  if (3 * dim > kMaxInt) return fail(DIT_ERR_UNSUPPORTED, "dim too large");
  DIT_CHECK_HIP(dit::launch_modulation(temb, w_mod, b_mod, mod, int(3 * dim), int(temb_dim), as_stream(stream)), "modulation");
  return DIT_OK;
}

extern "C" int dit_modulate_norm(const dit_bf16* x, const float* shift, const float* scale, dit_bf16* out,
                                 int64_t rows, int64_t cols, float eps, void* stream) {
  int rc = check_rows_cols(rows, cols);
  if (rc) return rc;
  if (rows == 0) return DIT_OK;  // empty input: nothing to read or write
  if (!x || !shift || !scale || !out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({x, shift, scale, out}))) return rc;
  if (!(eps >= 0.f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
  DIT_CHECK_HIP(dit::launch_modulate_norm(x, shift, scale, out, int(rows), int(cols), eps, as_stream(stream)), "modulate_norm");
  return DIT_OK;
}

extern "C" int dit_gated_residual(const dit_bf16* x, const dit_bf16* h, const float* gate, dit_bf16* y,
                                  int64_t rows, int64_t cols, void* stream) {
  int rc = check_rows_cols(rows, cols);
  if (rc) return rc;
  if (rows == 0) return DIT_OK;
  if (!x || !h || !gate || !y) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({x, h, gate, y}))) return rc;
  DIT_CHECK_HIP(dit::launch_gated_residual(x, h, gate, y, int(rows), int(cols), as_stream(stream)), "gated_residual");
  return DIT_OK;
}

extern "C" int dit_linear1_gelu(const dit_bf16* u, const dit_bf16* w1, const dit_bf16* b1, dit_bf16* qkv,
                                dit_bf16* cat, int64_t seq_len, int64_t dim, int64_t mlp_hidden, void* stream) {
  int rc = check_linear(seq_len, dim, mlp_hidden);
  if (rc) return rc;
  if (seq_len == 0) return DIT_OK;
  if (!u || !w1 || !qkv || !cat) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({u, w1, b1, qkv, cat}))) return rc;
  DIT_CHECK_HIP(dit::launch_linear1(u, w1, b1, qkv, cat, int(seq_len), int(dim), int(mlp_hidden), as_stream(stream)), "linear1");
  return DIT_OK;
}

extern "C" int dit_qk_rmsnorm_rope(dit_bf16* qkv, const float* q_norm_w, const float* k_norm_w,
                                   const float* rope_cos, const float* rope_sin, int64_t seq_len,
                                   int64_t num_heads, int64_t head_dim, float eps, void* stream) {
  int rc = check_dims(seq_len, num_heads * head_dim, num_heads, head_dim, 64, 8);
  if (rc) return rc;
  if (seq_len == 0) return DIT_OK;
  if (!qkv || !q_norm_w || !k_norm_w || !rope_cos || !rope_sin) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({qkv, q_norm_w, k_norm_w, rope_cos, rope_sin}))) return rc;
  if (!(eps >= 0.f)) return fail(DIT_ERR_INVALID_ARG, "eps must be >= 0");
  DIT_CHECK_HIP(dit::launch_qk_rmsnorm_rope(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, int(seq_len),
                                            int(num_heads), int(head_dim), eps, as_stream(stream)), "qk_rmsnorm_rope");
  return DIT_OK;
}

extern "C" int dit_attention(const dit_bf16* qkv, dit_bf16* out, int64_t seq_len, int64_t num_heads,
                             int64_t head_dim, int64_t ld_out, void* stream) {
  int rc = check_dims(seq_len, num_heads * head_dim, num_heads, head_dim, 64, 8);
  if (rc) return rc;
  if (seq_len == 0) return DIT_OK;
  if (!qkv || !out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({qkv, out}))) return rc;
  if (ld_out < num_heads * head_dim || ld_out % 4 != 0 || ld_out > kMaxInt)
    return fail(DIT_ERR_INVALID_ARG, "ld_out=%lld must be >= H*Dh and a multiple of 4", (long long)ld_out);
  DIT_CHECK_HIP(dit::launch_attention(qkv, out, int(seq_len), int(num_heads), int(head_dim), int(ld_out),
                                      as_stream(stream)), "attention");
  return DIT_OK;
}

extern "C" int dit_attention_partial(const dit_bf16* qkv, int64_t seq_len, int64_t num_heads, int64_t head_dim,
                                     int64_t kv_begin, int64_t kv_end, float* o_part, float* lse, void* stream) {
  int rc = check_dims(seq_len, num_heads * head_dim, num_heads, head_dim, 64, 8);
  if (rc) return rc;
  if (seq_len == 0) return DIT_OK;
  if (!qkv || !o_part || !lse) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({qkv, o_part}))) return rc;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(DIT_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (kv_begin < 0 || kv_end <= kv_begin || kv_end > seq_len)
    return fail(DIT_ERR_INVALID_ARG, "key range [%lld, %lld) must be non-empty and inside [0, %lld)",
                (long long)kv_begin, (long long)kv_end, (long long)seq_len);
  DIT_CHECK_HIP(dit::launch_attention_partial(qkv, int(seq_len), int(num_heads), int(head_dim), int(kv_begin),
                                              int(kv_end), o_part, lse, as_stream(stream)), "attention_partial");
  return DIT_OK;
}

extern "C" int dit_attention_split(const dit_bf16* qkv, dit_bf16* out, int64_t seq_len, int64_t num_heads,
                                   int64_t head_dim, int64_t ld_out, int64_t n_chunks, float* o_parts, float* lses,
                                   void* stream) {
  int rc = check_dims(seq_len, num_heads * head_dim, num_heads, head_dim, 64, 8);
  if (rc) return rc;
  if (n_chunks < 1 || n_chunks > 64) return fail(DIT_ERR_INVALID_ARG, "n_chunks=%lld must be in [1, 64]", (long long)n_chunks);
  if (seq_len == 0) return DIT_OK;
  if (!qkv || !out || !o_parts || !lses) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({qkv, out, o_parts}))) return rc;
  if (reinterpret_cast<uintptr_t>(lses) % 4 != 0) return fail(DIT_ERR_INVALID_ARG, "lses must be 4-byte aligned");
  if (ld_out < num_heads * head_dim || ld_out % 4 != 0 || ld_out > kMaxInt)
    return fail(DIT_ERR_INVALID_ARG, "ld_out=%lld must be >= H*Dh and a multiple of 4", (long long)ld_out);
  DIT_CHECK_HIP(dit::launch_attention_split(qkv, out, int(seq_len), int(num_heads), int(head_dim), int(ld_out),
                                            int(n_chunks), o_parts, lses, as_stream(stream)), "attention_split");
  return DIT_OK;
}

extern "C" int dit_attention_merge(const float* o_parts, const float* lses, int64_t n_chunks, int64_t seq_len,
                                   int64_t num_heads, int64_t head_dim, dit_bf16* out, int64_t ld_out,
                                   void* stream) {
  int rc = check_dims(seq_len, num_heads * head_dim, num_heads, head_dim, 64, 8);
  if (rc) return rc;
  if (n_chunks < 1 || n_chunks > 64) return fail(DIT_ERR_INVALID_ARG, "n_chunks=%lld not in [1, 64]", (long long)n_chunks);
  if (seq_len == 0) return DIT_OK;
  if (!o_parts || !lses || !out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({o_parts, out}))) return rc;
  if (reinterpret_cast<uintptr_t>(lses) % 4 != 0) return fail(DIT_ERR_INVALID_ARG, "lses must be 4-byte aligned");
  if (ld_out < num_heads * head_dim || ld_out % 4 != 0 || ld_out > kMaxInt)
    return fail(DIT_ERR_INVALID_ARG, "ld_out=%lld must be >= H*Dh and a multiple of 4", (long long)ld_out);
  DIT_CHECK_HIP(dit::launch_attention_merge(o_parts, lses, int(n_chunks), int(seq_len), int(num_heads),
                                            int(head_dim), out, int(ld_out), as_stream(stream)), "attention_merge");
  return DIT_OK;
}

extern "C" int dit_linear2_gated_residual(const dit_bf16* cat, const dit_bf16* w2, const dit_bf16* b2,
                                          const dit_bf16* x, const float* gate, dit_bf16* y, int64_t seq_len,
                                          int64_t dim, int64_t mlp_hidden, void* stream) {
  int rc = check_linear(seq_len, dim, mlp_hidden);
  if (rc) return rc;
  if (seq_len == 0) return DIT_OK;
  if (!cat || !w2 || !x || !gate || !y) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({cat, w2, b2, x, gate, y}))) return rc;
  DIT_CHECK_HIP(dit::launch_linear2(cat, w2, b2, x, gate, y, int(seq_len), int(dim), int(mlp_hidden),
                                    as_stream(stream)), "linear2");
  return DIT_OK;
}

extern "C" int dit_rope_table(const int32_t* positions, int64_t seq_len, int32_t n_axes, const int32_t* axes_dims,
                              int64_t head_dim, float base, float* rope_cos, float* rope_sin, void* stream) {
  if (!positions || !axes_dims || !rope_cos || !rope_sin) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if (seq_len < 0 || seq_len > (1 << 24)) return fail(DIT_ERR_INVALID_ARG, "seq_len=%lld", (long long)seq_len);
  if (n_axes < 1 || n_axes > 8) return fail(DIT_ERR_INVALID_ARG, "n_axes=%d not in [1,8]", n_axes);
  if (head_dim <= 0 || head_dim % 8 != 0 || head_dim > 1024) return fail(DIT_ERR_INVALID_ARG, "head_dim=%lld", (long long)head_dim);
  if (!(base > 1.0f)) return fail(DIT_ERR_INVALID_ARG, "base must be > 1");
  int64_t sum = 0;
  for (int a = 0; a < n_axes; ++a) {
    if (axes_dims[a] <= 0 || axes_dims[a] % 2 != 0) return fail(DIT_ERR_INVALID_ARG, "axes_dims[%d]=%d must be even and > 0", a, axes_dims[a]);
    sum += axes_dims[a];
  }
  if (sum != head_dim) return fail(DIT_ERR_INVALID_ARG, "axes_dims sum to %lld, head_dim is %lld", (long long)sum, (long long)head_dim);
  if (int rc = check_aligned({rope_cos, rope_sin})) return rc;
  DIT_CHECK_HIP(dit::launch_rope_table(positions, int(seq_len), n_axes, axes_dims, int(head_dim), base, rope_cos,
                                       rope_sin, as_stream(stream)), "rope_table");
  return DIT_OK;
}

// ============================================================== whole block
extern "C" size_t dit_block_workspace_bytes(const dit_block_config* cfg) {
  Dims D;
  if (dims_of(cfg, &D)) return 0;
  return layout(D).block_end;
}

extern "C" int dit_block_forward(const dit_block_config* cfg, const dit_block_weights* w, const dit_bf16* x,
                                 const dit_bf16* temb, const float* rope_cos, const float* rope_sin, dit_bf16* y,
                                 void* workspace, size_t ws_bytes, void* stream) {
  Dims D;
  int rc = dims_of(cfg, &D);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (!x || !temb || !rope_cos || !rope_sin || !y) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({x, temb, rope_cos, rope_sin, y}))) return rc;
  const WsLayout L = layout(D);
  if (!workspace || ws_bytes < L.block_end)
    return fail(DIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.block_end);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(DIT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return enqueue_block(D, cfg, w, x, temb, rope_cos, rope_sin, y, static_cast<unsigned char*>(workspace),
                       as_stream(stream));
}

// ======================================== whole block without any allocation
// For callers that cannot allocate device memory at all: the block's scratch
// (modulation vectors, u, q|k|v, concat buffer) lives in one file-scope device
// array, one copy per GPU, held until the process ends.  Host code never uses
// the array's name as an address: the first call on each device looks up that
// device's copy with hipGetSymbolAddress and keeps the pointer.
constexpr size_t kNoAllocScratchBytes = size_t(256) << 20;  // one Flux-shape block needs 243 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch`, looked up once per device.
int scratch_for_current_device(unsigned char** out) {
  int dev = 0;
  DIT_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DIT_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DIT_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0)
      return fail(DIT_ERR_HIP, "scratch array of device %d is missing or misaligned", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return DIT_OK;
}
}  // namespace

extern "C" size_t dit_block_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int dit_block_forward_noalloc(const dit_block_config* cfg, const dit_block_weights* w, const dit_bf16* x,
                                         const dit_bf16* temb, const float* rope_cos, const float* rope_sin,
                                         dit_bf16* y, void* stream) {
  Dims D;
  int rc = dims_of(cfg, &D);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (!x || !temb || !rope_cos || !rope_sin || !y) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({x, temb, rope_cos, rope_sin, y}))) return rc;
  const WsLayout L = layout(D);
  if (L.block_end > kNoAllocScratchBytes)
    return fail(DIT_ERR_WORKSPACE, "this config needs %zu bytes of scratch; the built-in array holds %zu",
                L.block_end, kNoAllocScratchBytes);
  unsigned char* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return enqueue_block(D, cfg, w, x, temb, rope_cos, rope_sin, y, ws, as_stream(stream));
}

// ================================================= two-stream / sequential blocks
extern "C" size_t dit_mmdit_block_workspace_bytes(const dit_block_config* cfg) {
  Dims D;
  if (dims_of(cfg, &D)) return 0;
  return mm_layout(D).end;
}

extern "C" int dit_mmdit_block_forward(const dit_block_config* cfg, int64_t txt_len, const dit_stream_weights* txt,
                                       const dit_stream_weights* img, const dit_bf16* x, const dit_bf16* temb,
                                       const float* rope_cos, const float* rope_sin, dit_bf16* y, void* workspace,
                                       size_t ws_bytes, void* stream) {
  Dims D;
  int rc = dims_of(cfg, &D);
  if (rc) return rc;
  if (txt_len < 0 || txt_len > D.S)
    return fail(DIT_ERR_INVALID_ARG, "txt_len=%lld outside [0, seq_len=%d]", (long long)txt_len, D.S);
  const int T = int(txt_len);
  if (T > 0 && (rc = check_stream_weights(txt, "text"))) return rc;
  if (D.S - T > 0 && (rc = check_stream_weights(img, "image"))) return rc;
  if (D.S == 0) return DIT_OK;
  if (!x || !temb || !rope_cos || !rope_sin || !y) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({x, temb, rope_cos, rope_sin, y}))) return rc;
  const MmLayout L = mm_layout(D);
  if (!workspace || ws_bytes < L.end) return fail(DIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, L.end);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(DIT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return enqueue_mmdit(D, T, cfg, txt, img, x, temb, rope_cos, rope_sin, y, static_cast<unsigned char*>(workspace),
                       as_stream(stream));
}

extern "C" int dit_sequential_block_forward(const dit_block_config* cfg, const dit_stream_weights* w,
                                            const dit_bf16* x, const dit_bf16* temb, const float* rope_cos,
                                            const float* rope_sin, dit_bf16* y, void* workspace, size_t ws_bytes,
                                            void* stream) {
  return dit_mmdit_block_forward(cfg, 0, nullptr, w, x, temb, rope_cos, rope_sin, y, workspace, ws_bytes, stream);
}

// ============================================================== block stack
struct dit_stack {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipStream_t cap = nullptr;
  std::vector<uintptr_t> key;
  uint32_t probe_mask = 0;
  int probe_blocks = 0;
  long long probe_replays = 0;         // probed graph launches since the last read
  int wall_khz = 0;                    // device wall-clock rate
  unsigned long long* probe_buf = nullptr;  // in the caller's workspace: [n_blocks][kProbeChannels][2]
  // host copy of the table of the blocks' W_mod / b_mod pointers (two-stream
  // blocks first), staged into the caller's workspace before every replay
  std::vector<const dit_bf16*> mod_tab;
};

namespace {
// The blocks a stack replays: n_double two-stream blocks (text rows [0, T)),
// then n_single single-stream blocks, all on one [S, d] activation.
struct StackPlan {
  int64_t T = 0;
  const dit_stream_weights* txt = nullptr;
  const dit_stream_weights* img = nullptr;
  int n_double = 0;
  const dit_block_weights* singles = nullptr;
  int n_single = 0;
};

// Workspace of a stack: the per-block scratch (the larger of the two block
// kinds when the plan has two-stream blocks), then the activation carried
// from block to block, the staged temb, every block's modulation vectors
// (two-stream blocks' present streams first, 6d floats each, then 3d per
// single-stream block), the table of their W_mod / b_mod pointers and the
// timing-probe counters of the single-stream blocks.
struct StackWs {
  size_t xbuf, tbuf, mods, tab, probe, end;
  int n_streams, n_dm, n_mats;
};

StackWs stack_ws(const Dims& D, int64_t T, int n_double, int n_single) {
  const bool mixed = n_double > 0;
  size_t o = layout(D).block_end;
  if (mixed) o = std::max(o, mm_layout(D).end);
  StackWs W;
  W.n_streams = mixed ? int(T > 0) + int(T < D.S) : 0;
  W.n_dm = n_double * W.n_streams;
  W.n_mats = W.n_dm + n_single;
  W.xbuf = o;  o = align256(o + size_t(D.S) * D.d * 2);
  W.tbuf = o;  o = align256(o + size_t(D.tdim) * 2);
  W.mods = o;  o = align256(o + (size_t(W.n_dm) * 6 * D.d + size_t(n_single) * 3 * D.d) * sizeof(float));
  W.tab = o;   o = align256(o + size_t(2) * W.n_mats * sizeof(void*));
  W.probe = o; o = align256(o + size_t(n_single) * kProbeChannels * 2 * sizeof(unsigned long long));
  W.end = o;
  return W;
}
StackWs stack_ws(const Dims& D, const StackPlan& P) { return stack_ws(D, P.T, P.n_double, P.n_single); }

std::vector<uintptr_t> make_key(const dit_block_config* cfg, const StackPlan& P, const dit_bf16* x_in,
                                const float* rcos, const float* rsin, void* ws, size_t ws_bytes, uint32_t probe_mask) {
  std::vector<uintptr_t> k;
  k.push_back(uintptr_t(cfg->seq_len));
  k.push_back(uintptr_t(cfg->dim));
  k.push_back(uintptr_t(cfg->num_heads));
  k.push_back(uintptr_t(cfg->head_dim));
  k.push_back(uintptr_t(cfg->mlp_hidden));
  k.push_back(uintptr_t(cfg->temb_dim));
  uint32_t e1, e2;
  std::memcpy(&e1, &cfg->ln_eps, 4);
  std::memcpy(&e2, &cfg->qk_eps, 4);
  k.push_back(e1);
  k.push_back(e2);
  k.push_back(cfg->flags);
  k.push_back(uintptr_t(P.n_double));
  k.push_back(uintptr_t(P.T));
  k.push_back(uintptr_t(P.n_single));
  k.push_back(uintptr_t(x_in));
  k.push_back(uintptr_t(rcos));
  k.push_back(uintptr_t(rsin));
  k.push_back(uintptr_t(ws));
  k.push_back(uintptr_t(ws_bytes));
  k.push_back(uintptr_t(probe_mask));
  for (int b = 0; b < P.n_double; ++b)
    for (const dit_stream_weights* sw : {P.txt ? &P.txt[b] : nullptr, P.img ? &P.img[b] : nullptr}) {
      if (!sw) {
        k.push_back(0);
        continue;
      }
      for (const void* q : {(const void*)sw->w_mod, (const void*)sw->b_mod, (const void*)sw->w_qkv,
                            (const void*)sw->b_qkv, (const void*)sw->q_norm_w, (const void*)sw->k_norm_w,
                            (const void*)sw->w_o, (const void*)sw->b_o, (const void*)sw->w_fc1, (const void*)sw->b_fc1,
                            (const void*)sw->w_fc2, (const void*)sw->b_fc2})
        k.push_back(uintptr_t(q));
    }
  for (int b = 0; b < P.n_single; ++b) {
    const dit_block_weights& w = P.singles[b];
    for (const void* q : {(const void*)w.w_mod, (const void*)w.b_mod, (const void*)w.w1, (const void*)w.b1,
                          (const void*)w.w2, (const void*)w.b2, (const void*)w.q_norm_w, (const void*)w.k_norm_w})
      k.push_back(uintptr_t(q));
  }
  return k;
}
}  // namespace

extern "C" int dit_stack_create(dit_stack** out) {
  if (!out) return fail(DIT_ERR_INVALID_ARG, "out is NULL");
  *out = new (std::nothrow) dit_stack();
  if (!*out) return fail(DIT_ERR_INVALID_ARG, "out of host memory");
  return DIT_OK;
}

extern "C" int dit_stack_destroy(dit_stack* st) {
  if (!st) return DIT_OK;
  if (st->exec) (void)hipGraphExecDestroy(st->exec);
  if (st->graph) (void)hipGraphDestroy(st->graph);
  if (st->cap) (void)hipStreamDestroy(st->cap);
  delete st;
  return DIT_OK;
}

extern "C" size_t dit_stack_workspace_bytes(const dit_block_config* cfg, int n_blocks) {
  Dims D;
  if (dims_of(cfg, &D) || n_blocks <= 0) return 0;
  return stack_ws(D, 0, 0, n_blocks).end;
}

extern "C" size_t dit_stack_mixed_workspace_bytes(const dit_block_config* cfg, int64_t txt_len, int n_double,
                                                  int n_single) {
  Dims D;
  if (dims_of(cfg, &D) || n_double < 0 || n_single < 0 || n_double + n_single <= 0) return 0;
  if (n_double > 0 && (txt_len < 0 || txt_len > D.S)) return 0;
  return stack_ws(D, n_double > 0 ? txt_len : 0, n_double, n_single).end;
}

namespace {
// Argument checks shared by the replay entry points, then the capture of the
// block sequence on first use.
int stack_setup(dit_stack* st, const dit_block_config* cfg, const StackPlan& P, const dit_bf16* x_in,
                const dit_bf16* temb_steps, int n_steps, const float* rope_cos, const float* rope_sin, dit_bf16* out,
                void* workspace, size_t ws_bytes, hipStream_t s, Dims* Dout) {
  if (!st) return fail(DIT_ERR_INVALID_ARG, "stack is NULL");
  Dims D;
  int rc = dims_of(cfg, &D);
  if (rc) return rc;
  if (P.n_double < 0 || P.n_single < 0 || P.n_double + P.n_single <= 0)
    return fail(DIT_ERR_INVALID_ARG, "n_double=%d n_single=%d", P.n_double, P.n_single);
  if (n_steps < 0) return fail(DIT_ERR_INVALID_ARG, "n_steps=%d", n_steps);
  if (P.n_single > 0 && !P.singles) return fail(DIT_ERR_INVALID_ARG, "single-stream blocks are NULL");
  for (int b = 0; b < P.n_single; ++b)
    if ((rc = check_weights(&P.singles[b]))) return rc;
  if (P.n_double > 0) {
    if (P.T < 0 || P.T > D.S) return fail(DIT_ERR_INVALID_ARG, "txt_len=%lld outside [0, %d]", (long long)P.T, D.S);
    if (P.T > 0 && !P.txt) return fail(DIT_ERR_INVALID_ARG, "text stream weights are NULL");
    if (P.T < D.S && !P.img) return fail(DIT_ERR_INVALID_ARG, "image stream weights are NULL");
    for (int b = 0; b < P.n_double; ++b) {
      if (P.T > 0 && (rc = check_stream_weights(&P.txt[b], "text"))) return rc;
      if (P.T < D.S && (rc = check_stream_weights(&P.img[b], "image"))) return rc;
    }
  }
  if (!x_in || !temb_steps || !rope_cos || !rope_sin || !out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if ((rc = check_aligned({x_in, temb_steps, rope_cos, rope_sin, out}))) return rc;
  const StackWs W = stack_ws(D, P);
  if (!workspace || ws_bytes < W.end) return fail(DIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, W.end);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(DIT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (st->probe_mask && P.n_double > 0)
    return fail(DIT_ERR_INVALID_ARG, "timing probes cover stacks of single-stream blocks only");
  if ((rc = check_not_capturing(s))) return rc;
  *Dout = D;

  const bool chain = (cfg->flags & DIT_STACK_CHAIN) != 0;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  dit_bf16* xbuf = reinterpret_cast<dit_bf16*>(ws + W.xbuf);
  dit_bf16* tbuf = reinterpret_cast<dit_bf16*>(ws + W.tbuf);

  std::vector<uintptr_t> key = make_key(cfg, P, x_in, rope_cos, rope_sin, workspace, ws_bytes, st->probe_mask);
  if (st->exec && key != st->key)
    return fail(DIT_ERR_GRAPH_KEY, "stack was captured for another config / pointer set; destroy and re-create it");
  if (st->exec) return DIT_OK;
  dit::prepare_device();  // device queries happen before capture
  if (!st->cap) DIT_CHECK_HIP(hipStreamCreateWithFlags(&st->cap, hipStreamNonBlocking), "hipStreamCreate");
  if (st->probe_mask) {
    int dev = 0;
    DIT_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
    DIT_CHECK_HIP(hipDeviceGetAttribute(&st->wall_khz, hipDeviceAttributeWallClockRate, dev),
                  "hipDeviceGetAttribute");
    if (st->wall_khz <= 0) return fail(DIT_ERR_HIP, "device reports no wall-clock rate");
    st->probe_buf = reinterpret_cast<unsigned long long*>(ws + W.probe);
    DIT_CHECK_HIP(hipMemsetAsync(st->probe_buf, 0,
                                 size_t(P.n_single) * kProbeChannels * 2 * sizeof(unsigned long long), s),
                  "hipMemsetAsync");
    st->probe_blocks = P.n_single;
    st->probe_replays = 0;
  }
  // Every block's modulation depends on temb only: one launch per block kind
  // computes them all at the start of the step.  Where the attention's last
  // round of workgroups leaves CUs idle (chain), the step's launch covers the
  // first block only and every later block's vectors come from the previous
  // block's attention launch.  Table: W_mod pointers of
  // the two-stream blocks' present streams (text first), then of the
  // single-stream blocks; the b_mod pointers after them in the same order.
  // Its host copy stays with the stack; run_steps stages it into the
  // workspace on the caller's stream before the steps of every replay.
  const int n_dm = W.n_dm, n_mats = W.n_mats;
  std::vector<const dit_bf16*> tab(2 * size_t(n_mats));
  for (int b = 0, m = 0; b < P.n_double; ++b) {
    if (P.T > 0) tab[m] = P.txt[b].w_mod, tab[n_mats + m] = P.txt[b].b_mod, ++m;
    if (P.T < D.S) tab[m] = P.img[b].w_mod, tab[n_mats + m] = P.img[b].b_mod, ++m;
  }
  for (int b = 0; b < P.n_single; ++b)
    tab[n_dm + b] = P.singles[b].w_mod, tab[n_mats + n_dm + b] = P.singles[b].b_mod;
  const dit_bf16** mod_ptrs = reinterpret_cast<const dit_bf16**>(ws + W.tab);
  float* mods_d = reinterpret_cast<float*>(ws + W.mods);     // [n_dm][6d]
  float* mods_s = mods_d + size_t(n_dm) * 6 * D.d;           // [n_single][3d]
  const int n_streams = W.n_streams;
  const bool chain_mod = P.n_double + P.n_single > 1 && dit::attention_hosts_modulation(D.S, D.H, D.Dh, D.tdim);
  // the vectors of two-stream block b / single-stream block b, produced by the previous block's attention
  auto double_next = [&](int b) {
    NextMod nm{{nullptr, nullptr}, {nullptr, nullptr}, 0, 6 * D.d, mods_d + size_t(b) * n_streams * 6 * D.d};
    if (P.T > 0) nm.w[nm.n_mats] = P.txt[b].w_mod, nm.b[nm.n_mats] = P.txt[b].b_mod, ++nm.n_mats;
    if (P.T < D.S) nm.w[nm.n_mats] = P.img[b].w_mod, nm.b[nm.n_mats] = P.img[b].b_mod, ++nm.n_mats;
    return nm;
  };
  auto single_next = [&](int b) {
    return NextMod{{P.singles[b].w_mod, nullptr}, {P.singles[b].b_mod, nullptr}, 1, 3 * D.d,
                   mods_s + size_t(b) * 3 * D.d};
  };

  DIT_CHECK_HIP(hipStreamBeginCapture(st->cap, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
  int brc = DIT_OK;
  hipError_t me = hipSuccess;
  if (n_dm > 0)  // with chain, the first two-stream block's streams only
    me = dit::launch_modulation_multi(tbuf, mod_ptrs, mod_ptrs + n_mats, mods_d, chain_mod ? n_streams : n_dm,
                                      6 * D.d, D.tdim, st->cap);
  if (me == hipSuccess && P.n_single > 0 && !(chain_mod && P.n_double > 0)) {
    // probes: kernel 0 of block 0 brackets this launch
    const bool pb = (st->probe_mask & 1u) != 0;
    if (pb) me = dit::launch_probe_stamp(st->probe_buf, 0, st->cap);
    if (me == hipSuccess)
      me = dit::launch_modulation_multi(tbuf, mod_ptrs + n_dm, mod_ptrs + n_mats + n_dm, mods_s,
                                        chain_mod ? 1 : P.n_single, 3 * D.d, D.tdim, st->cap);
    if (me == hipSuccess && pb) me = dit::launch_probe_stamp(st->probe_buf, 1, st->cap);
  }
  if (me != hipSuccess) brc = hip_fail(me, "modulation");
  int idx = 0;  // position in the whole sequence: only block 0 reads x_in
  for (int b = 0; b < P.n_double && brc == DIT_OK; ++b, ++idx) {
    const dit_bf16* xin = (idx == 0 && !chain) ? x_in : xbuf;
    NextMod nm{};
    const bool has_next = chain_mod && (b + 1 < P.n_double || P.n_single > 0);
    if (has_next) nm = b + 1 < P.n_double ? double_next(b + 1) : single_next(0);
    brc = enqueue_mmdit(D, int(P.T), cfg, P.txt ? &P.txt[b] : nullptr, P.img ? &P.img[b] : nullptr, xin, tbuf,
                        rope_cos, rope_sin, xbuf, ws, st->cap, mods_d + size_t(b) * n_streams * 6 * D.d,
                        has_next ? &nm : nullptr);
  }
  for (int b = 0; b < P.n_single && brc == DIT_OK; ++b, ++idx) {
    const dit_bf16* xin = (idx == 0 && !chain) ? x_in : xbuf;
    Probe pr;
    if (st->probe_mask) {
      pr.mask = st->probe_mask;
      pr.ch = st->probe_buf + size_t(b) * kProbeChannels * 2;
    }
    NextMod nm{};
    const bool has_next = chain_mod && b + 1 < P.n_single;
    if (has_next) nm = single_next(b + 1);
    brc = enqueue_block(D, cfg, &P.singles[b], xin, tbuf, rope_cos, rope_sin, xbuf, ws, st->cap, pr,
                        mods_s + size_t(b) * 3 * D.d, has_next ? &nm : nullptr);
  }
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(st->cap, &g);
  if (brc != DIT_OK) {
    if (g) (void)hipGraphDestroy(g);
    return brc;
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  st->graph = g;
  st->exec = ex;
  st->key = key;
  st->mod_tab = std::move(tab);
  return DIT_OK;
}

// Checks of the host arrays of a replay with skipped steps.
int check_schedule(int n_steps, const uint8_t* fresh, const float* t_steps) {
  if (n_steps > 0 && !fresh[0]) return fail(DIT_ERR_INVALID_ARG, "step 0 must be computed (no history before it)");
  if (t_steps) {
    for (int i = 0; i < n_steps; ++i)
      if (!std::isfinite(t_steps[i])) return fail(DIT_ERR_INVALID_ARG, "t_steps[%d] is not finite", i);
    for (int i = 1; i < n_steps; ++i) {
      const bool up = t_steps[1] > t_steps[0];
      if (up ? !(t_steps[i] > t_steps[i - 1]) : !(t_steps[i] < t_steps[i - 1]))
        return fail(DIT_ERR_INVALID_ARG, "t_steps must be strictly monotonic (step %d)", i);
    }
  }
  return DIT_OK;
}

// The denoising steps of a captured stack.  A computed step stages temb_s,
// launches the graph and copies the result to out[s]; a skipped step
// (fresh != NULL and fresh[s] == 0) predicts out[s] from the last two
// computed outputs by a first-order finite difference in t (a copy of the
// last one while only one exists).  With chain, the step's result is also
// the next step's input.
int run_steps(dit_stack* st, const Dims& D, bool chain, const StackPlan& P, const dit_bf16* x_in,
              const dit_bf16* temb_steps, int n_steps, dit_bf16* out, unsigned char* ws, const uint8_t* fresh,
              const float* t_steps, hipStream_t s) {
  const StackWs W = stack_ws(D, P);
  dit_bf16* xbuf = reinterpret_cast<dit_bf16*>(ws + W.xbuf);
  dit_bf16* tbuf = reinterpret_cast<dit_bf16*>(ws + W.tbuf);
  const size_t act = size_t(D.S) * D.d;
  // the modulation weight table the graph reads (a few bytes per block): the
  // host copy lives as long as the stack, so the copy may run asynchronously
  if (n_steps > 0 && !st->mod_tab.empty())
    DIT_CHECK_HIP(hipMemcpyAsync(ws + W.tab, st->mod_tab.data(), st->mod_tab.size() * sizeof(void*),
                                 hipMemcpyHostToDevice, s), "stage modulation table");
  int fa = -1, fb = -1;  // the last two computed steps
  auto tt = [&](int i) { return t_steps ? double(t_steps[i]) : double(i); };
  for (int step = 0; step < n_steps; ++step) {
    if (!fresh || fresh[step]) {
      if (chain && step == 0)
        DIT_CHECK_HIP(hipMemcpyAsync(xbuf, x_in, act * 2, hipMemcpyDeviceToDevice, s), "copy x_in");
      DIT_CHECK_HIP(hipMemcpyAsync(tbuf, temb_steps + size_t(step) * D.tdim, size_t(D.tdim) * 2,
                                   hipMemcpyDeviceToDevice, s), "copy temb");
      DIT_CHECK_HIP(hipGraphLaunch(st->exec, s), "hipGraphLaunch");
      if (st->probe_mask) ++st->probe_replays;
      DIT_CHECK_HIP(hipMemcpyAsync(out + size_t(step) * act, xbuf, act * 2, hipMemcpyDeviceToDevice, s), "copy out");
      fb = fa;
      fa = step;
      continue;
    }
    const float w = fb < 0 ? 0.f : float((tt(step) - tt(fa)) / (tt(fa) - tt(fb)));
    DIT_CHECK_HIP(dit::launch_extrapolate(out + size_t(fa) * act, fb < 0 ? nullptr : out + size_t(fb) * act, w,
                                          out + size_t(step) * act, chain ? xbuf : nullptr, act, s),
                  "extrapolate");
  }
  return DIT_OK;
}

int replay_plan(dit_stack* st, const dit_block_config* cfg, const StackPlan& P, const dit_bf16* x_in,
                const dit_bf16* temb_steps, int n_steps, const float* rope_cos, const float* rope_sin, dit_bf16* out,
                void* workspace, size_t ws_bytes, const uint8_t* fresh, const float* t_steps, void* stream) {
  int rc;
  if (fresh && (rc = check_schedule(n_steps, fresh, t_steps))) return rc;
  hipStream_t s = as_stream(stream);
  Dims D;
  if ((rc = stack_setup(st, cfg, P, x_in, temb_steps, n_steps, rope_cos, rope_sin, out, workspace, ws_bytes, s, &D)))
    return rc;
  return run_steps(st, D, (cfg->flags & DIT_STACK_CHAIN) != 0, P, x_in, temb_steps, n_steps, out,
                   static_cast<unsigned char*>(workspace), fresh, t_steps, s);
}
}  // namespace

extern "C" int dit_stack_replay(dit_stack* st, const dit_block_config* cfg, const dit_block_weights* blocks,
                                int n_blocks, const dit_bf16* x_in, const dit_bf16* temb_steps, int n_steps,
                                const float* rope_cos, const float* rope_sin, dit_bf16* out, void* workspace,
                                size_t ws_bytes, void* stream) {
  if (!blocks || n_blocks <= 0) return fail(DIT_ERR_INVALID_ARG, "n_blocks=%d", n_blocks);
  StackPlan P;
  P.singles = blocks;
  P.n_single = n_blocks;
  return replay_plan(st, cfg, P, x_in, temb_steps, n_steps, rope_cos, rope_sin, out, workspace, ws_bytes, nullptr,
                     nullptr, stream);
}

extern "C" int dit_stack_replay_cached(dit_stack* st, const dit_block_config* cfg, const dit_block_weights* blocks,
                                       int n_blocks, const dit_bf16* x_in, const dit_bf16* temb_steps, int n_steps,
                                       const float* rope_cos, const float* rope_sin, dit_bf16* out,
                                       void* workspace, size_t ws_bytes, const uint8_t* fresh, const float* t_steps,
                                       void* stream) {
  if (n_steps > 0 && !fresh) return fail(DIT_ERR_INVALID_ARG, "fresh is NULL");
  if (!blocks || n_blocks <= 0) return fail(DIT_ERR_INVALID_ARG, "n_blocks=%d", n_blocks);
  StackPlan P;
  P.singles = blocks;
  P.n_single = n_blocks;
  return replay_plan(st, cfg, P, x_in, temb_steps, n_steps, rope_cos, rope_sin, out, workspace, ws_bytes,
                     n_steps > 0 ? fresh : nullptr, t_steps, stream);
}

extern "C" int dit_stack_replay_mixed(dit_stack* st, const dit_block_config* cfg, int64_t txt_len,
                                      const dit_stream_weights* txt, const dit_stream_weights* img, int n_double,
                                      const dit_block_weights* singles, int n_single, const dit_bf16* x_in,
                                      const dit_bf16* temb_steps, int n_steps, const float* rope_cos,
                                      const float* rope_sin, dit_bf16* out, void* workspace, size_t ws_bytes,
                                      const uint8_t* fresh, const float* t_steps, void* stream) {
  StackPlan P;
  P.T = txt_len;
  P.txt = txt;
  P.img = img;
  P.n_double = n_double;
  P.singles = singles;
  P.n_single = n_single;
  return replay_plan(st, cfg, P, x_in, temb_steps, n_steps, rope_cos, rope_sin, out, workspace, ws_bytes, fresh,
                     t_steps, stream);
}

extern "C" int dit_stack_set_probe(dit_stack* st, uint32_t kernel_mask) {
  if (!st) return fail(DIT_ERR_INVALID_ARG, "stack is NULL");
  if (kernel_mask >> 6) return fail(DIT_ERR_INVALID_ARG, "kernel_mask=0x%x has bits above 5", kernel_mask);
  if (st->exec) return fail(DIT_ERR_GRAPH_KEY, "probes must be set before the first replay");
  st->probe_mask = kernel_mask;
  return DIT_OK;
}

extern "C" int dit_stack_probe_ms(dit_stack* st, float* ms, int n_blocks) {
  if (!st || !ms) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if (!st->exec || !st->probe_mask || st->probe_replays == 0)
    return fail(DIT_ERR_INVALID_ARG, "no probed replay has run since the last read");
  if (n_blocks != st->probe_blocks) return fail(DIT_ERR_INVALID_ARG, "n_blocks=%d, stack has %d", n_blocks, st->probe_blocks);
  const size_t n = size_t(n_blocks) * kProbeChannels * 2;
  std::vector<unsigned long long> h(n);
  DIT_CHECK_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  DIT_CHECK_HIP(hipMemcpy(h.data(), st->probe_buf, n * sizeof(unsigned long long), hipMemcpyDeviceToHost),
                "hipMemcpy");
  DIT_CHECK_HIP(hipMemset(st->probe_buf, 0, n * sizeof(unsigned long long)), "hipMemset");
  const double per_tick_ms = 1.0 / double(st->wall_khz) / double(st->probe_replays);
  st->probe_replays = 0;
  for (int b = 0; b < n_blocks; ++b) {
    const unsigned long long* c = h.data() + size_t(b) * kProbeChannels * 2;
    const double overhead = double(c[2 * 6 + 1]);
    for (int k = 0; k < 6; ++k)
      ms[size_t(b) * 6 + k] =
          (st->probe_mask >> k & 1u) ? float((double(c[2 * k + 1]) - overhead) * per_tick_ms) : -1.f;
  }
  return DIT_OK;
}

extern "C" int dit_stack_graph_info(dit_stack* st, int* n_kernel_nodes, int* n_nodes) {
  if (!st || !n_kernel_nodes || !n_nodes) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if (!st->graph) return fail(DIT_ERR_INVALID_ARG, "the stack has not been captured yet");
  size_t n = 0;
  DIT_CHECK_HIP(hipGraphGetNodes(st->graph, nullptr, &n), "hipGraphGetNodes");
  std::vector<hipGraphNode_t> nodes(n);
  if (n) DIT_CHECK_HIP(hipGraphGetNodes(st->graph, nodes.data(), &n), "hipGraphGetNodes");
  int k = 0;
  for (size_t i = 0; i < n; ++i) {
    hipGraphNodeType t;
    DIT_CHECK_HIP(hipGraphNodeGetType(nodes[i], &t), "hipGraphNodeGetType");
    if (t == hipGraphNodeTypeKernel) ++k;
  }
  *n_kernel_nodes = k;
  *n_nodes = int(n);
  return DIT_OK;
}

// ============================================================== ceiling probes
extern "C" int dit_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return DIT_OK;
  if (!src || !dst) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if (bytes % 16 != 0) return fail(DIT_ERR_INVALID_ARG, "bytes=%zu must be a multiple of 16", bytes);
  if (int rc = check_aligned({src, dst})) return rc;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return fail(DIT_ERR_INVALID_ARG, "src and dst overlap");
  DIT_CHECK_HIP(dit::launch_probe_copy(src, dst, bytes, as_stream(stream)), "probe_copy");
  return DIT_OK;
}

extern "C" int dit_probe_mfma(float* out, int64_t n_workgroups, int64_t iters, int32_t vary_operands, void* stream) {
  if (!out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
  if (n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
    return fail(DIT_ERR_INVALID_ARG, "n_workgroups=%lld iters=%lld", (long long)n_workgroups, (long long)iters);
  if (int rc = check_aligned({out})) return rc;
  DIT_CHECK_HIP(dit::launch_probe_mfma(out, int(n_workgroups), int(iters), vary_operands ? 1 : 0, as_stream(stream)),
                "probe_mfma");
  return DIT_OK;
}

// ============================================================== diagnostics
extern "C" const char* dit_last_error(void) { return g_err.c_str(); }
extern "C" const char* dit_version(void) { return "libdit_block 0.1.0 (gfx950)"; }

/*
 * libdit_block -- forward pass of a Flux-style single-stream DiT block on
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The block is the one profiled on the page "ChituDiffusion: torch.compile
 * and CUDA Graph on Flux.1-dev" (chenyy20.com), section 2: one Flux
 * single-stream block, S = 4608 tokens, dim 3072, 24 heads x 128, bf16.
 * Its memory-bound ops (LayerNorm, the adaLN modulation (1+scale)*x+shift,
 * GELU, the gated residual) are the ones section 1.1 of that page fuses;
 * the stack replay is the capture-once / replay-many scheme of sections
 * 1.2-1.3 and 7 (fixed shapes, fixed addresses, static buffers).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers unless marked HOST.  Matrices are
 *     row-major.  Activations are token-major [S, features] with heads in
 *     contiguous column blocks; weights use the [out, in] layout.
 *   - dit_bf16 holds raw bfloat16 bits.  Vectors marked float are fp32.
 *   - Device tensor pointers must be 16-byte aligned (every allocation from
 *     the HIP or PyTorch allocators is); others give DIT_ERR_INVALID_ARG.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream` and returns; none
 *     synchronises the host or allocates device memory.  The caller owns
 *     every buffer, the workspace and the stream.  The one exception is a
 *     block stack: it owns its captured graph (whose instantiation the HIP
 *     runtime backs with memory of its own) and the stream it captures on;
 *     everything the graph reads or writes lives in the caller's workspace.
 *     dit_stack_probe_ms (a diagnostic) synchronises the device.
 *   - The single-call entry points (everything except the stack replays)
 *     may be captured by the caller into its own graph: they enqueue only
 *     kernel launches on `stream` (the capture rules of the Flux page,
 *     section 1.2: no allocation and no host synchronisation inside a
 *     captured region).  A stack replay launches a graph of its own and
 *     returns DIT_ERR_CAPTURE on a capturing stream.
 *   - Every call returns DIT_OK (0) or an error code.  Arguments are checked
 *     before any HIP call; on error nothing is enqueued and dit_last_error()
 *     returns a message (thread-local).  HIP launch failures give DIT_ERR_HIP.
 *   - Empty inputs (rows or seq_len 0) are valid no-ops; their tensor
 *     pointers may then be NULL.
 *   - Supported shapes: any seq_len >= 0 (ragged tails are handled);
 *     dim % 64 == 0; head_dim in {64, 128} with num_heads*head_dim == dim;
 *     dim <= 8192; mlp_hidden % 64 == 0; temb_dim % 8 == 0;
 *     seq_len <= 2^24.  Others give DIT_ERR_UNSUPPORTED.
 */
#ifndef DIT_BLOCK_H
#define DIT_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dit_bf16;

enum {
  DIT_OK = 0,
  DIT_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad config field */
  DIT_ERR_UNSUPPORTED = 2,  /* shape outside the supported set */
  DIT_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  DIT_ERR_HIP = 4,          /* a HIP runtime call failed */
  DIT_ERR_CAPTURE = 5,      /* stream is capturing when the call may not be captured */
  DIT_ERR_GRAPH_KEY = 6     /* stack replay with a different (config, pointers) key */
};

/* flags of dit_block_config */
#define DIT_STACK_CHAIN 1u  /* step s+1 of a stack replay starts from step s's output */

typedef struct {
  int32_t seq_len;     /* S, tokens */
  int32_t dim;         /* d, model width */
  int32_t num_heads;   /* H */
  int32_t head_dim;    /* Dh, H*Dh == d */
  int32_t mlp_hidden;  /* width of the MLP branch */
  int32_t temb_dim;    /* length of the conditioning vector (0 means d) */
  float ln_eps;        /* LayerNorm epsilon, e.g. 1e-6 */
  float qk_eps;        /* QK RMSNorm epsilon, e.g. 1e-6 */
  uint32_t flags;      /* DIT_STACK_CHAIN */
} dit_block_config;

typedef struct {
  const dit_bf16* w_mod;  /* [3d, temb_dim]  modulation linear (shift|scale|gate rows) */
  const dit_bf16* b_mod;  /* [3d] or NULL */
  const dit_bf16* w1;     /* [3d+mlp, d]     linear1, output columns q | k | v | mlp */
  const dit_bf16* b1;     /* [3d+mlp] or NULL */
  const dit_bf16* w2;     /* [d, d+mlp]      linear2, input columns attn_out | gelu(mlp) */
  const dit_bf16* b2;     /* [d] or NULL */
  const float* q_norm_w;  /* [head_dim]      RMSNorm weight of q, shared by heads */
  const float* k_norm_w;  /* [head_dim]      RMSNorm weight of k */
} dit_block_weights;

/* ---- single steps of the block (each is one kernel launch) -------------- */

/* Modulation GEMV (adaLN): mod = W_mod . SiLU(temb) + b_mod, fp32 [3*dim],
 * laid out shift[dim] | scale[dim] | gate[dim].  SiLU(z) = z/(1+e^-z).
 * temb [temb_dim] bf16; w_mod [3*dim, temb_dim] bf16; b_mod [3*dim] or NULL. */
int dit_modulation(const dit_bf16* temb, const dit_bf16* w_mod, const dit_bf16* b_mod,
                   float* mod, int64_t dim, int64_t temb_dim, void* stream);

/* Fused LayerNorm + adaLN modulate (Flux page, section 1.1), one pass:
 * out[r,:] = (x[r,:] - mean_r) / sqrt(var_r + eps) * (1 + scale) + shift.
 * Row statistics in fp32, biased variance, no affine; one bf16 rounding at
 * the store.  x, out [rows, cols] bf16 (out may equal x); shift, scale
 * [cols] fp32.  cols % 8 == 0 and cols <= 8192. */
int dit_modulate_norm(const dit_bf16* x, const float* shift, const float* scale,
                      dit_bf16* out, int64_t rows, int64_t cols, float eps, void* stream);

/* Gated residual, the last step of the block's adaLN tail (the Flux page,
 * section 1.1, counts it among the elementwise ops between the GEMMs that
 * compilation fuses): y[r,c] = x[r,c] + gate[c] * h[r,c]; x, h, y [rows,
 * cols] bf16 (y may equal x or h); gate [cols] fp32, the third modulation
 * vector.  fp32 arithmetic, one bf16 rounding at the store.  cols % 8 == 0,
 * cols <= 8192. */
int dit_gated_residual(const dit_bf16* x, const dit_bf16* h, const float* gate,
                       dit_bf16* y, int64_t rows, int64_t cols, void* stream);

/* linear1 with fused epilogue: z = u . W1^T + b1 over [S, 3d+mlp];
 * columns [0,3d) -> qkv [S, 3d] (q | k | v); columns [3d, 3d+mlp) ->
 * GELU_tanh -> cat[:, d : d+mlp] of cat [S, d+mlp].
 * u [S, d] bf16; w1 [3d+mlp, d]; b1 [3d+mlp] or NULL. */
int dit_linear1_gelu(const dit_bf16* u, const dit_bf16* w1, const dit_bf16* b1,
                     dit_bf16* qkv, dit_bf16* cat, int64_t seq_len, int64_t dim,
                     int64_t mlp_hidden, void* stream);

/* Per-head QK RMSNorm then RoPE, in place on the q and k blocks of qkv
 * [S, 3*H*Dh]: t <- t / sqrt(mean(t^2) + eps) * w, then each pair
 * (t[2j], t[2j+1]) is turned by the angle whose cos/sin are rope_cos/sin
 * [S, Dh/2] fp32 (RoPE as complex rotation, Flux page section 3.1).
 * q_norm_w, k_norm_w [Dh] fp32.  v is untouched. */
int dit_qk_rmsnorm_rope(dit_bf16* qkv, const float* q_norm_w, const float* k_norm_w,
                        const float* rope_cos, const float* rope_sin, int64_t seq_len,
                        int64_t num_heads, int64_t head_dim, float eps, void* stream);

/* Exact softmax attention per head, no mask (the flash / sdpa backends of the
 * Flux page, sections 2 and 4), softmax statistics and accumulation in fp32:
 * out[t, h*Dh:(h+1)*Dh] = softmax_u(q_t . k_u / sqrt(Dh)) v_u, with q, k, v
 * read from qkv [S, 3*H*Dh]; out has leading dimension ld_out (>= H*Dh),
 * only columns [0, H*Dh) are written. */
int dit_attention(const dit_bf16* qkv, dit_bf16* out, int64_t seq_len, int64_t num_heads,
                  int64_t head_dim, int64_t ld_out, void* stream);

/* Chunked attention, the one-device math of ring attention (page
 * "ChituDiffusion: torch.compile and CUDA Graph on Flux.1-dev", sections 5
 * and 6.1: every hop attends to one K/V shard, yields a partial output and
 * its log-sum-exp, and the hops are merged by log-sum-exp).
 *
 * dit_attention_partial: queries of all seq_len tokens of qkv (layout as in
 * dit_attention) against the keys and values of tokens [kv_begin, kv_end)
 * only.  o_part [seq_len, H*Dh] fp32 receives the softmax average over the
 * chunk; lse [H, seq_len] fp32 receives ln sum_u exp(q.k_u / sqrt(Dh)) over
 * the chunk.  0 <= kv_begin < kv_end <= seq_len, else DIT_ERR_INVALID_ARG.
 * lse is written as scalars and needs only 4-byte alignment. */
int dit_attention_partial(const dit_bf16* qkv, int64_t seq_len, int64_t num_heads, int64_t head_dim,
                          int64_t kv_begin, int64_t kv_end, float* o_part, float* lse, void* stream);

/* dit_attention_merge: o_parts holds n_chunks consecutive [seq_len, H*Dh]
 * fp32 partials of disjoint key chunks and lses their n_chunks consecutive
 * [H, seq_len] log-sum-exps; writes out[t, h*Dh + i] (bf16, row stride
 * ld_out) = sum_c exp(lse_c - lse) o_c with lse = ln sum_c exp(lse_c), i.e.
 * attention over the union of the chunks.  1 <= n_chunks <= 64; lses needs
 * only 4-byte alignment. */
int dit_attention_merge(const float* o_parts, const float* lses, int64_t n_chunks, int64_t seq_len,
                        int64_t num_heads, int64_t head_dim, dit_bf16* out, int64_t ld_out, void* stream);

/* Attention over all seq_len keys with the keys split into up to n_chunks
 * equal chunks (n_chunks in [1, 64]; chunks are ceil(S / n_chunks) tokens,
 * so fewer may result, never an empty one): the partials of all chunks in
 * one launch, then dit_attention_merge's weighting into out (bf16, row stride
 * ld_out).  For head counts too small to fill the chip with workgroups of
 * 128 or 256 queries of one head (e.g. one GPU's heads after an all-to-all from
 * sequence to head sharding, the Flux page, section 5): the chunks give
 * n_chunks times as many workgroups.  o_parts [n_chunks, S, H*Dh] fp32 and
 * lses [n_chunks, H, S] fp32 are caller-owned scratch. */
int dit_attention_split(const dit_bf16* qkv, dit_bf16* out, int64_t seq_len, int64_t num_heads,
                        int64_t head_dim, int64_t ld_out, int64_t n_chunks, float* o_parts, float* lses,
                        void* stream);

/* linear2 with fused gated residual: y = x + gate * (cat . W2^T + b2).
 * cat [S, d+mlp]; w2 [d, d+mlp]; b2 [d] or NULL; x, y [S, d] (y may equal x);
 * gate [d] fp32. */
int dit_linear2_gated_residual(const dit_bf16* cat, const dit_bf16* w2, const dit_bf16* b2,
                               const dit_bf16* x, const float* gate, dit_bf16* y,
                               int64_t seq_len, int64_t dim, int64_t mlp_hidden, void* stream);

/* RoPE angle tables: for token t and pair j of the head, cos/sin of
 * positions[t, a] * base^(-2 j' / D_a), where the head dim is cut into
 * n_axes chunks of axes_dims[a] dims (HOST array, each even, summing to
 * head_dim), j' is the pair's index inside its chunk and a its axis.
 * positions [S, n_axes] int32; rope_cos, rope_sin [S, head_dim/2] fp32. */
int dit_rope_table(const int32_t* positions, int64_t seq_len, int32_t n_axes,
                   const int32_t* axes_dims, int64_t head_dim, float base,
                   float* rope_cos, float* rope_sin, void* stream);

/* ---- whole block --------------------------------------------------------- */

/* Bytes of workspace dit_block_forward needs (0 on an invalid config):
 * fp32 modulation vectors [3d], then bf16 u [S, d], q|k|v [S, 3d] and the
 * concat buffer [S, d + mlp] (attention output | GELU output), each section
 * 256-byte aligned; 255 MB at the Flux shape of the page "ChituDiffusion:
 * torch.compile and CUDA Graph on Flux.1-dev", section 2 (S = 4608,
 * d = 3072, MLP 12288). */
size_t dit_block_workspace_bytes(const dit_block_config* cfg);

/* One Flux single-stream block forward (the block profiled in section 2 of
 * the Flux page above; its adaLN modulation, LayerNorm and GELU are the ops
 * of section 1.1, RoPE the complex rotation of section 3.1, attention the
 * exact flash / sdpa attention of sections 2 and 4):
 *   shift|scale|gate = W_mod SiLU(temb) + b_mod
 *   u = LN(x)(1 + scale) + shift
 *   q|k|v|g = u W1^T + b1;  q, k <- per-head RMSNorm, then RoPE
 *   o = softmax(q k^T / sqrt(Dh)) v per head
 *   y = x + gate * ([o | GELU_tanh(g)] W2^T + b2)
 * Five launches on `stream`: modulation, LayerNorm+modulate, linear1 (whose
 * epilogue also does the q/k RMSNorm + RoPE, so q and k are rounded to bf16
 * once), attention, linear2 with the gated residual.
 * x, y [S, d] bf16 (y may equal x: the block then runs in place);
 * temb [temb_dim] bf16; rope_cos/sin [S, head_dim/2] fp32; workspace is a
 * device buffer of at least dit_block_workspace_bytes(cfg) bytes, 256-byte
 * aligned, owned by the caller and overwritten (it must not overlap x or y).
 * Errors: DIT_ERR_INVALID_ARG (NULL or misaligned pointer, bad config),
 * DIT_ERR_UNSUPPORTED (shape), DIT_ERR_WORKSPACE (missing, small or
 * misaligned workspace), DIT_ERR_HIP (launch failure). */
int dit_block_forward(const dit_block_config* cfg, const dit_block_weights* w,
                      const dit_bf16* x, const dit_bf16* temb, const float* rope_cos,
                      const float* rope_sin, dit_bf16* y, void* workspace, size_t ws_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): dit_block_forward
 * with the workspace taken from a scratch array built into the library, one
 * copy per GPU of dit_block_noalloc_max_bytes() = 256 MiB, held from the
 * first call on that GPU until the process ends (one Flux-shape block needs
 * 243 MiB).  Same kernels and results as dit_block_forward.  Configs whose
 * workspace exceeds the array give DIT_ERR_WORKSPACE.  The first call on
 * each device looks up that device's copy of the array (hipGetSymbolAddress;
 * make that first call outside a capture); no call allocates.  Every call on
 * one GPU uses the same array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be ordered by
 * the caller.  The array keeps the last call's contents; nothing in it needs
 * to start at zero. */
size_t dit_block_noalloc_max_bytes(void);
int dit_block_forward_noalloc(const dit_block_config* cfg, const dit_block_weights* w, const dit_bf16* x,
                              const dit_bf16* temb, const float* rope_cos, const float* rope_sin, dit_bf16* y,
                              void* stream);

/* ---- two-stream (MMDiT) and sequential blocks ------------------------------ */

/* Weights of one stream.  The Flux page (section 3.1) names the block lists
 * of the models it compiles: Flux's transformer_blocks (two-stream) and
 * single_transformer_blocks, and Wan's blocks.  A stream of a two-stream
 * block has its own adaLN modulation with six vectors, attention
 * projections and MLP: */
typedef struct {
  const dit_bf16* w_mod;   /* [6d, temb_dim]  rows shift1|scale1|gate1|shift2|scale2|gate2 */
  const dit_bf16* b_mod;   /* [6d] or NULL */
  const dit_bf16* w_qkv;   /* [3d, d]         output columns q | k | v */
  const dit_bf16* b_qkv;   /* [3d] or NULL */
  const float* q_norm_w;   /* [head_dim]      RMSNorm weight of q, shared by heads */
  const float* k_norm_w;   /* [head_dim] */
  const dit_bf16* w_o;     /* [d, d]          attention output projection */
  const dit_bf16* b_o;     /* [d] or NULL */
  const dit_bf16* w_fc1;   /* [mlp, d]        MLP in (GELU-tanh follows) */
  const dit_bf16* b_fc1;   /* [mlp] or NULL */
  const dit_bf16* w_fc2;   /* [d, mlp]        MLP out */
  const dit_bf16* b_fc2;   /* [d] or NULL */
} dit_stream_weights;

/* Bytes of workspace dit_mmdit_block_forward and dit_sequential_block_forward
 * need (0 on an invalid config). */
size_t dit_mmdit_block_workspace_bytes(const dit_block_config* cfg);

/* One two-stream block forward.  x, y [S, d] hold the text tokens (rows
 * [0, txt_len)) followed by the image tokens (rows [txt_len, S)); y may
 * equal x.  For each stream s with its own weights and rows x_s:
 *   shift1, scale1, gate1, shift2, scale2, gate2 = W_mod.SiLU(temb) + b_mod
 *   u = LN(x_s)(1 + scale1) + shift1;  q|k|v = u W_qkv^T + b_qkv;
 *   q, k <- per-head RMSNorm (the stream's weights), then RoPE (table rows
 *   of the stream's tokens);
 * then one attention over the concatenated q, k, v of all S tokens (text and
 * image attend to each other), and per stream, with o_s its output rows:
 *   x' = x_s + gate1 * (o_s W_o^T + b_o)
 *   y_s = x' + gate2 * (GELU_tanh((LN(x')(1 + scale2) + shift2) W_fc1^T + b_fc1) W_fc2^T + b_fc2)
 * Same LayerNorm, RMSNorm, RoPE, attention and GELU as the single-stream
 * block; x' is kept in fp32 (workspace), other intermediates in bf16.  txt_len in [0, S]; txt may be NULL when txt_len == 0 (then the
 * block is one stream: see dit_sequential_block_forward).  Each linear is
 * one launch for both streams (their tiles share the chip).  workspace:
 * dit_mmdit_block_workspace_bytes(cfg) bytes, 256-byte aligned. */
int dit_mmdit_block_forward(const dit_block_config* cfg, int64_t txt_len, const dit_stream_weights* txt,
                            const dit_stream_weights* img, const dit_bf16* x, const dit_bf16* temb,
                            const float* rope_cos, const float* rope_sin, dit_bf16* y, void* workspace,
                            size_t ws_bytes, void* stream);

/* One sequential block (the block of the Wan video page: attention, gated
 * residual, then the MLP with its own LayerNorm+modulate and gated
 * residual), i.e. one stream of the two-stream block over all S tokens.
 * Cross-attention to a text context is not part of it. */
int dit_sequential_block_forward(const dit_block_config* cfg, const dit_stream_weights* w, const dit_bf16* x,
                                 const dit_bf16* temb, const float* rope_cos, const float* rope_sin,
                                 dit_bf16* y, void* workspace, size_t ws_bytes, void* stream);

/* ---- block stack replayed over denoising steps --------------------------- */

/* opaque: owns the captured graph, its capture stream and a host copy of
 * the table of the blocks' W_mod / b_mod pointers.  Everything the graph
 * reads or writes is in the caller's workspace: the per-block scratch, the
 * activation carried from block to block, the staged temb, every block's
 * modulation vectors (they depend on temb alone: one launch per block kind
 * at the start of every step computes them, or, where the attention's last
 * round of workgroups leaves CUs idle, that launch computes the first
 * block's and every block's attention launch computes the next block's),
 * the pointer table (staged with an asynchronous copy on the caller's
 * stream at every replay call) and the timing-probe counters. */
typedef struct dit_stack dit_stack;

int dit_stack_create(dit_stack** out);
int dit_stack_destroy(dit_stack* st);

/* Bytes of workspace dit_stack_replay and dit_stack_replay_cached need for
 * a stack of n_blocks single-stream blocks (0 on an invalid config). */
size_t dit_stack_workspace_bytes(const dit_block_config* cfg, int n_blocks);

/* Runs n_steps denoising steps of the n_blocks-block stack: step s feeds
 * x_in (or, with DIT_STACK_CHAIN, step s-1's output) through blocks
 * 0..n_blocks-1 in order with temb_steps[s], and writes out[s].  The block
 * sequence is captured once as a hipGraph on the first call and replayed
 * once per step (capture-once / replay-many, Flux page sections 1.2-1.3).
 * blocks: HOST array [n_blocks] of device weight pointers; temb_steps
 * [n_steps, temb_dim]; out [n_steps, S, d]; workspace of at least
 * dit_stack_workspace_bytes(cfg, n_blocks) bytes, 256-byte aligned, which
 * the replay overwrites.  The graph is keyed by the config, every pointer
 * (the workspace's included) and n_blocks; a later call with another key
 * returns DIT_ERR_GRAPH_KEY and enqueues nothing (destroy and re-create the
 * stack to re-capture: the Wan2.1 video page, section 5.2, warns that a
 * shape change needs a new capture).  On a capturing stream: DIT_ERR_CAPTURE.
 * The first call captures on the stack's own stream (graph instantiation
 * allocates the runtime's own memory for the graph). */
int dit_stack_replay(dit_stack* st, const dit_block_config* cfg, const dit_block_weights* blocks,
                     int n_blocks, const dit_bf16* x_in, const dit_bf16* temb_steps,
                     int n_steps, const float* rope_cos, const float* rope_sin, dit_bf16* out,
                     void* workspace, size_t ws_bytes, void* stream);

/* Step-level replay/skip (the control of a model-level feature cache such as
 * MeanCache, Flux page section 7: the captured forward stays whole and the
 * cache only decides, per denoising step, whether to replay it or to
 * predict the step's output from history).  As dit_stack_replay, except
 * that only the steps with fresh[s] != 0 replay the graph.  A skipped step
 * s gets the first-order finite difference through the outputs of the last
 * two computed steps a > b:
 *   out[s] = out[a] + (t_s - t_a) / (t_a - t_b) * (out[a] - out[b])
 * (out[a] itself while only one step has been computed), in fp32 from the
 * stored bf16 outputs, rounded once to bf16.  With DIT_STACK_CHAIN the
 * prediction is also the next step's input.  fresh: HOST array [n_steps],
 * fresh[0] must be nonzero.  t_steps: HOST array [n_steps] of strictly
 * monotonic step times (e.g. the sampler's timesteps) or NULL for t_s = s.
 * Shares the stack's captured graph and key with dit_stack_replay. */
int dit_stack_replay_cached(dit_stack* st, const dit_block_config* cfg, const dit_block_weights* blocks,
                            int n_blocks, const dit_bf16* x_in, const dit_bf16* temb_steps, int n_steps,
                            const float* rope_cos, const float* rope_sin, dit_bf16* out, void* workspace,
                            size_t ws_bytes, const uint8_t* fresh, const float* t_steps, void* stream);

/* Bytes of workspace dit_stack_replay_mixed needs for n_double two-stream
 * blocks with txt_len text tokens and n_single single-stream blocks (0 on
 * an invalid config). */
size_t dit_stack_mixed_workspace_bytes(const dit_block_config* cfg, int64_t txt_len, int n_double, int n_single);

/* A Flux-style stack: n_double two-stream blocks (text rows [0, txt_len),
 * weights txt[b] and img[b], HOST arrays of n_double) followed by n_single
 * single-stream blocks (singles, HOST array), replayed per denoising step
 * as one captured graph (the Flux page, section 3.1: the model's
 * transformer_blocks then single_transformer_blocks; section 7: one graph
 * of the whole model per step).  Steps, chaining and step times as in
 * dit_stack_replay_cached; fresh may be NULL (every step computed).
 * txt may be NULL when txt_len == 0 and img when txt_len == S.  Timing
 * probes are not available for stacks with two-stream blocks.  workspace:
 * dit_stack_mixed_workspace_bytes(cfg) bytes.  One stack object holds one
 * captured graph: the key covers both block lists. */
int dit_stack_replay_mixed(dit_stack* st, const dit_block_config* cfg, int64_t txt_len,
                           const dit_stream_weights* txt, const dit_stream_weights* img, int n_double,
                           const dit_block_weights* singles, int n_single, const dit_bf16* x_in,
                           const dit_bf16* temb_steps, int n_steps, const float* rope_cos, const float* rope_sin,
                           dit_bf16* out, void* workspace, size_t ws_bytes, const uint8_t* fresh,
                           const float* t_steps, void* stream);

/* Timing probes (diagnostics for benchmarks; must be set before the first
 * replay, i.e. before the graph is captured; DIT_ERR_GRAPH_KEY after).  For
 * every block and every kernel i (0 modulation, 1 LayerNorm+modulate,
 * 2 linear1, 3 QK RMSNorm+RoPE, 4 attention, 5 linear2) with bit i of
 * kernel_mask set, the captured graph brackets that launch with two
 * one-thread kernels that read the device wall clock (hipDeviceAttribute-
 * WallClockRate) and accumulate the interval in a small device buffer owned
 * by the stack; a bracket around nothing, once per block, measures the
 * probe's own overhead.  The kernels being timed and their results are
 * unchanged; the graph gains 2 + 2*popcount(mask) tiny nodes per block.
 * A stack's step-level modulation launch is reported as kernel 0 of block
 * 0 (all blocks' GEMVs, or block 0's alone where the later blocks' run in
 * the attention launches, which kernel 4 then includes); kernel 0 of the
 * other blocks reads ~0.
 * kernel_mask bits above 5 -> DIT_ERR_INVALID_ARG. */
int dit_stack_set_probe(dit_stack* st, uint32_t kernel_mask);

/* Synchronises the device, then writes ms[b*6 + i] = mean duration in
 * milliseconds of kernel i of block b over the probed replay steps since
 * the previous call (or since capture), with the probe overhead subtracted
 * (so one dispatch gap remains in each figure); -1 for kernels not probed.
 * Restarts the accumulation.  ms is a HOST array of n_blocks*6 floats;
 * n_blocks must match the captured stack.  No probed step since the last
 * read, or a mismatched n_blocks -> DIT_ERR_INVALID_ARG. */
int dit_stack_probe_ms(dit_stack* st, float* ms, int n_blocks);

/* Structure of the captured graph: the number of kernel nodes and of all
 * nodes (the Flux page, sections 2 and 3.2, counts the kernels of one block
 * forward: 52 eager, 12 compiled).  Before the first replay:
 * DIT_ERR_INVALID_ARG. */
int dit_stack_graph_info(dit_stack* st, int* n_kernel_nodes, int* n_nodes);

/* ---- ceiling probes (not part of the block's path) ---------------------------
 * What the chip delivers, to place the kernels against it as well as against
 * the published peaks.
 * dit_probe_copy: a streaming copy of `bytes` bytes (a multiple of 16; src
 * and dst 16-byte aligned and disjoint), 16-byte loads and stores.
 * dit_probe_mfma: n_workgroups workgroups of 4 wavefronts; every wavefront
 * issues iters x 4 independent v_mfma_f32_32x32x16_bf16 (32768 flop each)
 * on register operands: the same operands every time (vary_operands 0) or
 * operands that change from one instruction to the next (1, as in a GEMM).
 * out [n_workgroups * 256] fp32 receives per-lane sums (keeps the work
 * live).  n_workgroups in [1, 2^20], iters in [1, 2^24]. */
int dit_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int dit_probe_mfma(float* out, int64_t n_workgroups, int64_t iters, int32_t vary_operands, void* stream);

/* ---- diagnostics ------------------------------------------------------------ */

const char* dit_last_error(void);  /* message for the last non-OK return on this thread */
const char* dit_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_BLOCK_H */

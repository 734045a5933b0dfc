"""CPU oracle of the Flux-style DiT block forwards (single-stream, two-stream
and sequential).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
``cpu_baseline`` leg may import this module.  The GPU library never calls it,
and it shares no code with the GPU library: the only common dependency is the
seeded input module ``dit_inputs``, which holds no block arithmetic.

Everything here is the plain definition of the block, computed in float64
with numpy (a matrix product is the only library primitive used as a step).
No blocking, fusion or reordering beyond what the definitions state.  The
block is the one named on the page "ChituDiffusion: torch.compile and CUDA
Graph on Flux.1-dev" (chenyy20.com, 2026-06-21), section 2 (one Flux
single-stream block, S=4608, dim 3072, 24 heads x 128, bf16); its ops are the
ones that page lists in section 1.1 (LayerNorm, GELU, the adaLN modulation
(1+scale)*x+shift), RoPE as complex rotation (section 3.1) and exact
attention (the flash / sdpa backends of sections 2 and 4).

Readings of what the pages leave open (all are documented with the tests):
  * block layout: parallel attention and MLP branches sharing one
    LayerNorm+modulate; linear1 emits [q | k | v | mlp], linear2 consumes
    [attn_out | gelu(mlp)]; one gated residual;
  * modulation chunks in the order shift, scale, gate; SiLU before the linear;
  * LayerNorm: biased variance, eps inside the square root, no affine;
  * QK RMSNorm per head (eps 1e-6, weight of length head_dim shared by heads),
    then RoPE on adjacent pairs (2j, 2j+1) with base 10000; the head dim is
    split in equal chunks, one per position axis, in axis order;
  * attention: no mask, scale 1/sqrt(head_dim), softmax over all tokens;
  * GELU in its tanh form;
  * two-stream block (Flux's transformer_blocks; internals not on the
    pages): per stream its own six-vector modulation (shift1, scale1,
    gate1, shift2, scale2, gate2), q|k|v linear, q/k RMSNorm weights,
    output projection and MLP; one attention over text then image tokens;
    attention and MLP branches in sequence, each with its own
    LayerNorm+modulate and gated residual; the sequential video block is
    the same with a single stream (no cross-attention);
  * step-level skip (the MeanCache-style control of the Flux page, section
    7): a skipped step's output is the first-order finite difference in the
    step time through the stored outputs of the last two computed steps;
  * chunked attention (the one-GPU math of ring attention): a chunk's
    partial output is the softmax average over the chunk's keys alone, its
    lse the natural log of the chunk's sum of exp(score); partials of
    disjoint chunks are merged with weights exp(lse_c - lse).

Parity status: every function below is pinned by the CPU tests in
tests/test_oracle_pins.py against library routines, closed forms, invariants
or brute force; the RoPE axis-split / pairing conventions are pinned by those
invariants but not by any value printed on the pages (the pages print no
numeric example of the block).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ------------------------------------------------------------ bf16 storage
def round_bf16(a):
    """Round to the nearest bfloat16 value (ties to even), returned as float64.
    The block takes and returns bf16 tensors (the Flux page, section 2, runs
    the block in bf16), so a stack of blocks hands bf16 values from one
    block to the next."""
    f = np.ascontiguousarray(np.asarray(a, F64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(F64)


# -------------------------------------------------------------- activations
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}); feeds the modulation linear."""
    z = np.asarray(z, F64)
    return z / (1.0 + np.exp(-z))


def gelu_tanh(g):
    """GELU, tanh form: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
    GELU is one of the fused elementwise ops of section 1.1 of the Flux page;
    the tanh form is the one fixed for this block."""
    g = np.asarray(g, F64)
    return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))


# ----------------------------------------------------------------- linears
def linear(a, w, b=None):
    """nn.Linear convention: a [rows, in] times w [out, in] transposed, plus b."""
    out = np.asarray(a, F64) @ np.asarray(w, F64).T
    if b is not None:
        out = out + np.asarray(b, F64)
    return out


# ----------------------------------------------------- adaLN modulation GEMV
def modulation(temb, w_mod, b_mod):
    """m = W_mod . SiLU(temb) + b_mod, split into (shift, scale, gate), each [d].
    adaLN modulation of section 1.1 of the Flux page."""
    m = linear(silu(temb)[None, :], w_mod, b_mod)[0]
    d = m.shape[0] // 3
    return m[:d], m[d:2 * d], m[2 * d:]


# ----------------------------------------------------- LayerNorm + modulate
def layer_norm(x, eps):
    """Row LayerNorm with no affine: (x - mean) / sqrt(var + eps), biased var."""
    x = np.asarray(x, F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(xn, shift, scale):
    """adaLN modulation (1 + scale) * x + shift (section 1.1 of the Flux page)."""
    return xn * (1.0 + np.asarray(scale, F64)) + np.asarray(shift, F64)


def layer_norm_modulate(x, shift, scale, eps=1e-6):
    return modulate(layer_norm(x, eps), shift, scale)


# ---------------------------------------------------------- gated residual
def gated_residual(x, gate, h):
    """y = x + gate * h, gate broadcast over rows (one per channel)."""
    return np.asarray(x, F64) + np.asarray(gate, F64) * np.asarray(h, F64)


# --------------------------------------------------------- QK RMSNorm heads
def rms_norm_heads(t, num_heads, head_dim, weight, eps=1e-6):
    """Per-token, per-head RMSNorm of t [S, H*Dh]: t_h / sqrt(mean(t_h^2) + eps) * w."""
    t = np.asarray(t, F64).reshape(t.shape[0], num_heads, head_dim)
    r = np.sqrt((t ** 2).mean(axis=-1, keepdims=True) + eps)
    return (t / r * np.asarray(weight, F64)).reshape(t.shape[0], num_heads * head_dim)


# -------------------------------------------------------------------- RoPE
def rope_angles(pos, axes_dims, head_dim, base=10000.0):
    """Rotation angle of every (token, pair) [S, head_dim/2].

    Pairs are consecutive dims (2j, 2j+1).  The head dim is cut into chunks of
    ``axes_dims`` dims, one per position axis; pair j' of a chunk of D dims on
    axis a turns by  pos[t, a] * base^(-2 j' / D).
    """
    pos = np.asarray(pos, F64)
    assert sum(axes_dims) == head_dim
    cols = []
    for a, D in enumerate(axes_dims):
        jp = np.arange(D // 2, dtype=F64)
        freq = base ** (-2.0 * jp / D)
        cols.append(pos[:, a:a + 1] * freq[None, :])
    return np.concatenate(cols, axis=1)


def rope_apply(t, theta, num_heads, head_dim):
    """Rotate each pair (a, b) = (t[2j], t[2j+1]) of every head by theta[t, j]:
    (a cos - b sin, a sin + b cos) -- the pair read as a complex number times
    e^{i theta} (RoPE as complex arithmetic, section 3.1 of the Flux page)."""
    S = t.shape[0]
    t = np.asarray(t, F64).reshape(S, num_heads, head_dim // 2, 2)
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    a, b = t[..., 0], t[..., 1]
    out = np.stack([a * c - b * s, a * s + b * c], axis=-1)
    return out.reshape(S, num_heads * head_dim)


# --------------------------------------------------------------- attention
def softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def attention(q, k, v, num_heads, head_dim, q_rows=None):
    """Exact softmax attention per head, no mask: o = softmax(q k^T / sqrt(Dh)) v.
    q, k, v are [S, H*Dh] (heads in column blocks); returns o [len(q_rows), H*Dh].
    ``q_rows`` restricts the queries (each output row is computed in full);
    query rows are processed in chunks only to bound memory."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    rows = np.arange(q.shape[0]) if q_rows is None else np.asarray(q_rows)
    out = np.empty((rows.shape[0], num_heads * head_dim), F64)
    scale = 1.0 / np.sqrt(head_dim)
    for h in range(num_heads):
        cs = slice(h * head_dim, (h + 1) * head_dim)
        kh, vh = k[:, cs], v[:, cs]
        for r0 in range(0, rows.shape[0], 1024):
            rr = rows[r0:r0 + 1024]
            p = softmax_rows((q[rr, cs] @ kh.T) * scale)
            out[r0:r0 + len(rr), cs] = p @ vh
    return out


# ------------------------------------------- chunked attention (one GPU)
def attention_partial(q, k, v, num_heads, head_dim, kv_begin, kv_end, q_rows=None):
    """Attention of the queries against the keys and values of tokens
    [kv_begin, kv_end) only, with the chunk's log-sum-exp: the step one hop
    of ring attention performs on its K/V shard (ChituDiffusion page,
    sections 5 and 6.1: every hop yields a partial output and its lse, and
    the hops are merged by lse).  Returns (o, lse): o [R, H*Dh] is the softmax
    average over the chunk alone; lse [H, R] is ln sum_u exp(s_tu) over the
    chunk with s = q.k / sqrt(Dh)."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)[kv_begin:kv_end]
    v = np.asarray(v, F64)[kv_begin:kv_end]
    rows = np.arange(q.shape[0]) if q_rows is None else np.asarray(q_rows)
    out = np.empty((rows.shape[0], num_heads * head_dim), F64)
    lse = np.empty((num_heads, rows.shape[0]), F64)
    scale = 1.0 / np.sqrt(head_dim)
    for h in range(num_heads):
        cs = slice(h * head_dim, (h + 1) * head_dim)
        s = (q[rows, cs] @ k[:, cs].T) * scale
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        z = e.sum(axis=1, keepdims=True)
        out[:, cs] = (e / z) @ v[:, cs]
        lse[h] = (mx + np.log(z))[:, 0]
    return out, lse


def attention_merge(parts, num_heads, head_dim):
    """Combine partial results (o_c, lse_c) of disjoint chunks: with
    lse = ln sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c, which is the
    softmax average over the union of the chunks."""
    lses = np.stack([np.asarray(l, F64) for _, l in parts])            # [C, H, R]
    mx = lses.max(axis=0)
    lse = mx + np.log(np.exp(lses - mx).sum(axis=0))                   # [H, R]
    out = np.zeros_like(np.asarray(parts[0][0], F64))
    for o_c, l_c in parts:
        wgt = np.exp(np.asarray(l_c, F64) - lse)                       # [H, R]
        for h in range(num_heads):
            cs = slice(h * head_dim, (h + 1) * head_dim)
            out[:, cs] += wgt[h][:, None] * np.asarray(o_c, F64)[:, cs]
    return out, lse


# ------------------------------------------------------------- whole block
def block_forward(shape, w, x, temb, pos, rows=None, return_intermediates=False):
    """One single-stream block forward.

    Steps (the order used throughout this project):
      1. shift, scale, gate = W_mod . SiLU(temb) + b_mod
      2. u = LN(x) * (1 + scale) + shift
      3. z = u W1^T + b1  ->  q, k, v, g
      4. q, k <- per-head RMSNorm (w_q, w_k); 5. RoPE on q and k
      6. o = softmax(q k^T / sqrt(Dh)) v per head
      7. a = GELU_tanh(g)
      8. h = [o | a] W2^T + b2
      9. y = x + gate * h
    ``rows`` restricts the output to those tokens (keys and values still cover
    every token, so each returned row is exact).
    """
    d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
    x = np.asarray(x, F64)
    shift, scale, gate = modulation(temb, w.w_mod, w.b_mod)
    u = layer_norm_modulate(x, shift, scale, shape.ln_eps)
    rr = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    theta = rope_angles(pos, shape.rope_axes_dims, Dh, shape.rope_base)
    # keys / values for every token
    w1 = np.asarray(w.w1, F64)
    b1 = np.asarray(w.b1, F64)
    kk = linear(u, w1[d:2 * d], b1[d:2 * d])
    vv = linear(u, w1[2 * d:3 * d], b1[2 * d:3 * d])
    kk = rope_apply(rms_norm_heads(kk, H, Dh, w.k_norm_w, shape.qk_eps), theta, H, Dh)
    # queries and mlp only for the requested rows
    ur = u[rr]
    qq = linear(ur, w1[0:d], b1[0:d])
    qq = rope_apply(rms_norm_heads(qq, H, Dh, w.q_norm_w, shape.qk_eps), theta[rr], H, Dh)
    g = linear(ur, w1[3 * d:], b1[3 * d:])
    # attention for the requested rows: queries are the rows' own q
    o = _attention_rows(qq, kk, vv, H, Dh)
    a = gelu_tanh(g)
    hb = linear(np.concatenate([o, a], axis=1), w.w2, w.b2)
    y = gated_residual(x[rr], gate, hb)
    if return_intermediates:
        return y, dict(shift=shift, scale=scale, gate=gate, u=u[rr], q=qq, k=kk[rr],
                       v=vv[rr], k_all=kk, v_all=vv, o=o, g=g, a=a, h=hb)
    return y


def _attention_rows(q_rows, k, v, num_heads, head_dim):
    """attention() with a query matrix that already holds only the wanted rows."""
    qfull = np.asarray(q_rows, F64)
    return attention(qfull, k, v, num_heads, head_dim, q_rows=np.arange(qfull.shape[0]))


# ------------------------------------------- two-stream / sequential blocks
def stream_modulation(temb, w_mod, b_mod):
    """Six adaLN vectors of one stream of a two-stream block:
    W_mod . SiLU(temb) + b_mod split into shift1, scale1, gate1 (attention
    branch) and shift2, scale2, gate2 (MLP branch), each [d]."""
    m = linear(silu(temb)[None, :], w_mod, b_mod)[0]
    d = m.shape[0] // 6
    return tuple(m[i * d:(i + 1) * d] for i in range(6))


def double_block_forward(shape, w_txt, w_img, x, temb, pos, n_txt=None, rows=None):
    """One two-stream (MMDiT) block forward: Flux's transformer_blocks, named
    beside single_transformer_blocks in section 3.1 of the Flux page.

    Tokens [0, n_txt) are the text stream (weights w_txt), tokens [n_txt, S)
    the image stream (w_img); n_txt defaults to shape.text_tokens.  Per
    stream, with its own weights:
      1. shift1, scale1, gate1, shift2, scale2, gate2 = W_mod . SiLU(temb) + b_mod
      2. u = LN(x) * (1 + scale1) + shift1
      3. q, k, v = u W_qkv^T + b_qkv; q, k <- per-head RMSNorm, then RoPE
    4. one attention over the q, k, v of all S tokens (both streams)
    then per stream, o being its rows of the attention output:
      5. x' = x + gate1 * (o W_o^T + b_o)
      6. y = x' + gate2 * (GELU_tanh((LN(x') (1 + scale2) + shift2) W_fc1^T + b_fc1) W_fc2^T + b_fc2)
    With n_txt = 0 this is the sequential block (one stream over all tokens).
    ``rows`` restricts the output to those tokens (keys and values still
    cover every token, so each returned row is exact).
    """
    d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
    eps, qeps = shape.ln_eps, shape.qk_eps
    x = np.asarray(x, F64)
    S = x.shape[0]
    n_txt = shape.text_tokens if n_txt is None else n_txt
    theta = rope_angles(pos, shape.rope_axes_dims, Dh, shape.rope_base)
    streams = [(w_txt, 0, n_txt), (w_img, n_txt, S)]
    # keys and values of every token, each stream with its own weights
    k = np.zeros((S, d), F64)
    v = np.zeros((S, d), F64)
    for w, a, b in streams:
        if b <= a:
            continue
        shift1, scale1 = stream_modulation(temb, w.w_mod, w.b_mod)[:2]
        u = layer_norm_modulate(x[a:b], shift1, scale1, eps)
        wq, bq = np.asarray(w.w_qkv, F64), np.asarray(w.b_qkv, F64)
        kk = linear(u, wq[d:2 * d], bq[d:2 * d])
        k[a:b] = rope_apply(rms_norm_heads(kk, H, Dh, w.k_norm_w, qeps), theta[a:b], H, Dh)
        v[a:b] = linear(u, wq[2 * d:], bq[2 * d:])
    rr = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty((rr.shape[0], d), F64)
    for w, a, b in streams:
        sel = (rr >= a) & (rr < b)
        if not sel.any():
            continue
        rs = rr[sel]
        shift1, scale1, gate1, shift2, scale2, gate2 = stream_modulation(temb, w.w_mod, w.b_mod)
        u = layer_norm_modulate(x[rs], shift1, scale1, eps)
        wq, bq = np.asarray(w.w_qkv, F64), np.asarray(w.b_qkv, F64)
        q = rope_apply(rms_norm_heads(linear(u, wq[:d], bq[:d]), H, Dh, w.q_norm_w, qeps), theta[rs], H, Dh)
        o = _attention_rows(q, k, v, H, Dh)
        x1 = gated_residual(x[rs], gate1, linear(o, w.w_o, w.b_o))
        u2 = layer_norm_modulate(x1, shift2, scale2, eps)
        mlp = linear(gelu_tanh(linear(u2, w.w_fc1, w.b_fc1)), w.w_fc2, w.b_fc2)
        out[sel] = gated_residual(x1, gate2, mlp)
    return out


def sequential_block_forward(shape, w, x, temb, pos, rows=None):
    """The sequential (Wan-style) block: attention, gated residual, then the
    MLP with its own LayerNorm+modulate and gated residual, over all tokens
    with one set of weights; the two-stream block with no text stream.
    Cross-attention to a text context is not part of it."""
    return double_block_forward(shape, None, w, x, temb, pos, n_txt=0, rows=rows)


def stack_forward(shape, weights_list, x_in, temb_steps, pos, chain=False, bf16_io=True):
    """Denoising-loop replay of a block stack: for each step s, run every block
    in order on the step input with temb_s; the step input is x_in, or the
    previous step's output when ``chain`` is set.  With ``bf16_io`` each
    block's output is handed to the next block (and to the next step) as a
    bf16 tensor; the last block's output is returned unrounded.
    Returns [n_steps, S, d]."""
    outs = []
    xs = np.asarray(x_in, F64)
    nb = len(weights_list)
    for s in range(len(temb_steps)):
        cur = xs if (chain and s > 0) else np.asarray(x_in, F64)
        for b, w in enumerate(weights_list):
            cur = block_forward(shape, w, cur, temb_steps[s], pos)
            if bf16_io and b + 1 < nb:
                cur = round_bf16(cur)
        outs.append(cur)
        xs = round_bf16(cur) if bf16_io else cur
    return np.stack(outs)


def flux_stack_forward(shape, doubles, singles, x_in, temb_steps, pos, n_txt=None, chain=False, bf16_io=True):
    """stack_forward for a Flux-style stack: the two-stream blocks ``doubles``
    (a list of (w_txt, w_img)) then the single-stream blocks ``singles``, in
    order, on one [S, d] activation with the text tokens first (the Flux
    page, section 3.1, names the two block lists, transformer_blocks then
    single_transformer_blocks).  Rounding and chaining as in stack_forward.
    Returns [n_steps, S, d]."""
    outs = []
    xs = np.asarray(x_in, F64)
    kinds = [("d", w) for w in doubles] + [("s", w) for w in singles]
    for s in range(len(temb_steps)):
        cur = xs if (chain and s > 0) else np.asarray(x_in, F64)
        for b, (kind, w) in enumerate(kinds):
            if kind == "d":
                cur = double_block_forward(shape, w[0], w[1], cur, temb_steps[s], pos, n_txt=n_txt)
            else:
                cur = block_forward(shape, w, cur, temb_steps[s], pos)
            if bf16_io and b + 1 < len(kinds):
                cur = round_bf16(cur)
        outs.append(cur)
        xs = round_bf16(cur) if bf16_io else cur
    return np.stack(outs)


# ------------------------------------------------ step-level replay / skip
def extrapolate_step(out_a, out_b, t_s, t_a, t_b):
    """Prediction of a skipped step's output from history: the first-order
    finite difference in the step time through the outputs of the last two
    computed steps a (most recent, time t_a) and b (time t_b),
        out_a + (t_s - t_a) / (t_a - t_b) * (out_a - out_b),
    or out_a itself when no second step exists (out_b is None).  The Flux
    page (section 7) describes MeanCache's skipped steps as a finite-
    difference prediction from history that never enters the model."""
    a = np.asarray(out_a, F64)
    if out_b is None:
        return a.copy()
    return a + (t_s - t_a) / (t_a - t_b) * (a - np.asarray(out_b, F64))


def stack_forward_cached(shape, weights_list, x_in, temb_steps, pos, fresh, t=None, chain=False):
    """stack_forward in which only the steps with fresh[s] run the block
    stack; a skipped step's output is extrapolate_step() from the stored
    (bf16) outputs of the last two computed steps, t[s] the step times
    (the step index when t is None).  With ``chain`` the next step starts
    from this step's stored output, computed or predicted.  Returns
    [n_steps, S, d]: computed steps unrounded, predicted steps from the
    rounded history."""
    n = len(temb_steps)
    tt = list(range(n)) if t is None else [float(v) for v in t]
    assert n == 0 or fresh[0], "step 0 has no history"
    outs, stored = [], []
    hist = []   # step indices of computed steps, most recent last
    cur_in = np.asarray(x_in, F64)
    for s in range(n):
        if fresh[s]:
            cur = cur_in if chain else np.asarray(x_in, F64)
            for b, w in enumerate(weights_list):
                cur = block_forward(shape, w, cur, temb_steps[s], pos)
                if b + 1 < len(weights_list):
                    cur = round_bf16(cur)
            hist.append(s)
            y = cur
        else:
            a = hist[-1]
            bb = hist[-2] if len(hist) > 1 else None
            y = extrapolate_step(stored[a], None if bb is None else stored[bb], tt[s], tt[a],
                                 None if bb is None else tt[bb])
        outs.append(y)
        stored.append(round_bf16(y))
        cur_in = stored[-1]
    return np.stack(outs) if outs else np.zeros((0,) + np.asarray(x_in).shape)


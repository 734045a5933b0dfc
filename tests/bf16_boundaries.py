"""Attribution model for the GPU parity misses at the Flux shape.

The oracle (oracle/dit_oracle.py) keeps every intermediate of a block in
float64.  The GPU path stores its intermediates in bf16 at the kernel
boundaries the design fixes (reading R16: u, q|k|v after RMSNorm+RoPE, the
attention output, the GELU output; the two-stream block also u2 and the
fc1+GELU output, its mid-block residual x' stays fp32), and its attention
weights the values by the probabilities rounded to bf16 (the matrix cores
take bf16 operands) with the sum of those rounded probabilities as the
denominator.

This module recomputes the oracle's blocks with bf16 rounding inserted at
exactly those boundaries, composed from the oracle's own steps.  It is test
infrastructure: it never touches the GPU library and no GPU value enters it.
Its role is to attribute an error of the GPU output against the float64
oracle: if the bf16-boundary model shows the same excess over the float64
oracle as the GPU does, and the GPU matches the model closely, the excess
is the cost of bf16 storage between the kernels, not a kernel defect.
"""
from __future__ import annotations

import numpy as np

from oracle import dit_oracle as O

F64 = np.float64


def _r(a, on=True):
    return O.round_bf16(a) if on else np.asarray(a, F64)


def attention_bf16p(q, k, v, num_heads, head_dim, round_p=True):
    """Softmax attention in which the probabilities (against the row max) are
    rounded to bf16 before they weight v and the denominator sums the rounded
    values, the arithmetic the GPU's PV product applies."""
    q, k, v = (np.asarray(t, F64) for t in (q, k, v))
    out = np.empty((q.shape[0], num_heads * head_dim), F64)
    scale = 1.0 / np.sqrt(head_dim)
    for h in range(num_heads):
        cs = slice(h * head_dim, (h + 1) * head_dim)
        kh, vh = k[:, cs], v[:, cs]
        for r0 in range(0, q.shape[0], 1024):
            s = (q[r0:r0 + 1024, cs] @ kh.T) * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p = _r(p, round_p)
            out[r0:r0 + 1024, cs] = (p @ vh) / p.sum(axis=1, keepdims=True)
    return out


def block_forward_bf16(shape, w, x, temb, pos, rows=None, round_u=True, round_qkv=True, round_p=True,
                       round_cat=True, return_intermediates=False):
    """oracle.block_forward with bf16 storage of u, q/k/v, the attention
    probabilities and the concat buffer [o | GELU(g)], as the GPU path
    stores them.  ``rows`` restricts the output rows (keys and values still
    cover every token).  With ``return_intermediates`` also returns each
    stored stage before its own rounding (u, q, k, v, o, a) and the branch
    h, each computed from the rounded stages before it."""
    d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
    x = np.asarray(x, F64)
    shift, scale, gate = O.modulation(temb, w.w_mod, w.b_mod)
    u_pre = O.layer_norm_modulate(x, shift, scale, shape.ln_eps)
    u = _r(u_pre, round_u)
    rr = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    theta = O.rope_angles(pos, shape.rope_axes_dims, Dh, shape.rope_base)
    w1, b1 = np.asarray(w.w1, F64), np.asarray(w.b1, F64)
    k_pre = O.rope_apply(O.rms_norm_heads(O.linear(u, w1[d:2 * d], b1[d:2 * d]), H, Dh, w.k_norm_w, shape.qk_eps),
                         theta, H, Dh)
    v_pre = O.linear(u, w1[2 * d:3 * d], b1[2 * d:3 * d])
    kk, vv = _r(k_pre, round_qkv), _r(v_pre, round_qkv)
    ur = u[rr]
    q_pre = O.rope_apply(O.rms_norm_heads(O.linear(ur, w1[0:d], b1[0:d]), H, Dh, w.q_norm_w, shape.qk_eps),
                         theta[rr], H, Dh)
    qq = _r(q_pre, round_qkv)
    o_pre = attention_bf16p(qq, kk, vv, H, Dh, round_p)
    a_pre = O.gelu_tanh(O.linear(ur, w1[3 * d:], b1[3 * d:]))
    o, a = _r(o_pre, round_cat), _r(a_pre, round_cat)
    hb = O.linear(np.concatenate([o, a], axis=1), w.w2, w.b2)
    y = O.gated_residual(x[rr], gate, hb)
    if return_intermediates:
        return y, dict(u=u_pre[rr], q=q_pre, k=k_pre[rr], v=v_pre[rr], o=o_pre, a=a_pre, h=hb)
    return y


def double_block_forward_bf16(shape, w_txt, w_img, x, temb, pos, n_txt=None, rows=None, round_u=True,
                              round_qkv=True, round_p=True, round_o=True, round_h=True, return_intermediates=False):
    """oracle.double_block_forward with bf16 storage of u, q/k/v, the
    attention probabilities, the attention output, u2 = LN(x')-modulated and
    the GELU output of fc1; x' stays unrounded (fp32 on the GPU).  With
    ``return_intermediates`` also returns, for the output rows, each stored
    stage before its own rounding (q, k, v, o, u2, h) and x'."""
    d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
    eps, qeps = shape.ln_eps, shape.qk_eps
    x = np.asarray(x, F64)
    S = x.shape[0]
    n_txt = shape.text_tokens if n_txt is None else n_txt
    theta = O.rope_angles(pos, shape.rope_axes_dims, Dh, shape.rope_base)
    streams = [(w_txt, 0, n_txt), (w_img, n_txt, S)]
    k = np.zeros((S, d), F64)
    v = np.zeros((S, d), F64)
    for w, a, b in streams:
        if b <= a:
            continue
        shift1, scale1 = O.stream_modulation(temb, w.w_mod, w.b_mod)[:2]
        u = _r(O.layer_norm_modulate(x[a:b], shift1, scale1, eps), round_u)
        wq, bq = np.asarray(w.w_qkv, F64), np.asarray(w.b_qkv, F64)
        kk = O.linear(u, wq[d:2 * d], bq[d:2 * d])
        k[a:b] = _r(O.rope_apply(O.rms_norm_heads(kk, H, Dh, w.k_norm_w, qeps), theta[a:b], H, Dh), round_qkv)
        v[a:b] = _r(O.linear(u, wq[2 * d:], bq[2 * d:]), round_qkv)
    rr = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty((rr.shape[0], d), F64)
    it = {n: np.empty((rr.shape[0], shape.mlp_hidden if n == "h" else d), F64)
          for n in ("q", "k", "v", "o", "x1", "u2", "h")} if return_intermediates else None
    for w, a, b in streams:
        sel = (rr >= a) & (rr < b)
        if not sel.any():
            continue
        rs = rr[sel]
        shift1, scale1, gate1, shift2, scale2, gate2 = O.stream_modulation(temb, w.w_mod, w.b_mod)
        u = _r(O.layer_norm_modulate(x[rs], shift1, scale1, eps), round_u)
        wq, bq = np.asarray(w.w_qkv, F64), np.asarray(w.b_qkv, F64)
        q_pre = O.rope_apply(O.rms_norm_heads(O.linear(u, wq[:d], bq[:d]), H, Dh, w.q_norm_w, qeps), theta[rs],
                             H, Dh)
        q = _r(q_pre, round_qkv)
        o_pre = attention_bf16p(q, k, v, H, Dh, round_p)
        o = _r(o_pre, round_o)
        x1 = O.gated_residual(x[rs], gate1, O.linear(o, w.w_o, w.b_o))
        u2_pre = O.layer_norm_modulate(x1, shift2, scale2, eps)
        u2 = _r(u2_pre, round_u)
        h_pre = O.gelu_tanh(O.linear(u2, w.w_fc1, w.b_fc1))
        hh = _r(h_pre, round_h)
        out[sel] = O.gated_residual(x1, gate2, O.linear(hh, w.w_fc2, w.b_fc2))
        if return_intermediates:
            # k and v of these rows before their rounding
            kk = O.linear(u, wq[d:2 * d], bq[d:2 * d])
            it["k"][sel] = O.rope_apply(O.rms_norm_heads(kk, H, Dh, w.k_norm_w, qeps), theta[rs], H, Dh)
            it["v"][sel] = O.linear(u, wq[2 * d:], bq[2 * d:])
            for n, val in (("q", q_pre), ("o", o_pre), ("x1", x1), ("u2", u2_pre), ("h", h_pre)):
                it[n][sel] = val
    if return_intermediates:
        return out, it
    return out

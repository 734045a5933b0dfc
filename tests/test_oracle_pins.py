"""Pins of the CPU oracle against things other than itself.

The pages print no numeric worked example of the block, so each oracle
function is pinned by library routines (PyTorch CPU float64), closed forms,
invariants, special cases and brute force on tiny inputs.  Each ``pin_*``
takes the oracle module so that the planted-mistake tests at the bottom can
show that a plausible error in the oracle fails at least one pin.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dit_inputs as DI
from oracle import dit_oracle as O

RNG = np.random.default_rng(1234)


def t64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


# ------------------------------------------------------------ pins
def pin_layer_norm(o):
    x = RNG.standard_normal((7, 96)) * RNG.uniform(0.1, 5.0, (7, 1)) + RNG.uniform(-3, 3, (7, 1))
    for eps in (1e-6, 0.5):
        y = o.layer_norm(x, eps)
        sig2 = x.var(axis=-1)            # biased variance (numpy default)
        assert np.allclose(y.mean(axis=-1), 0.0, atol=1e-12)
        # variance of the output is sigma^2 / (sigma^2 + eps) exactly
        assert np.allclose(y.var(axis=-1), sig2 / (sig2 + eps), rtol=1e-12)
        ref = F.layer_norm(t64(x), (96,), eps=eps).numpy()
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def pin_modulate(o):
    x = RNG.standard_normal((5, 64))
    shift = RNG.standard_normal(64)
    ln = F.layer_norm(t64(x), (64,), eps=1e-6).numpy()
    # scale = -1 removes the normalised row: the output is the shift
    assert np.allclose(o.layer_norm_modulate(x, shift, -np.ones(64), 1e-6), shift[None, :], atol=1e-12)
    # scale = shift = 0 is plain LayerNorm
    assert np.allclose(o.layer_norm_modulate(x, np.zeros(64), np.zeros(64), 1e-6), ln, atol=1e-12)
    # scale = 1 doubles it, shift adds
    assert np.allclose(o.layer_norm_modulate(x, shift, np.ones(64), 1e-6), 2 * ln + shift, atol=1e-12)


def pin_gated_residual(o):
    x = RNG.standard_normal((4, 32))
    h = RNG.standard_normal((4, 32))
    assert np.array_equal(o.gated_residual(x, np.zeros(32), h), x)          # gate = 0 -> identity
    assert np.array_equal(o.gated_residual(x, np.ones(32), -x), np.zeros_like(x))
    g = np.zeros(32)
    g[3] = 2.0
    y = o.gated_residual(x, g, np.ones((4, 32)))
    assert np.allclose(y[:, 3], x[:, 3] + 2.0) and np.array_equal(np.delete(y, 3, 1), np.delete(x, 3, 1))


def pin_silu(o):
    z = np.linspace(-30, 30, 601)
    assert np.allclose(o.silu(z), F.silu(t64(z)).numpy(), rtol=1e-13, atol=1e-300)
    assert o.silu(0.0) == 0.0
    assert np.allclose(o.silu(z) - o.silu(-z), z, atol=1e-12)


def pin_gelu(o):
    g = np.linspace(-12, 12, 481)
    assert np.allclose(o.gelu_tanh(g), F.gelu(t64(g), approximate="tanh").numpy(), rtol=1e-13, atol=1e-15)
    assert o.gelu_tanh(0.0) == 0.0
    assert np.allclose(o.gelu_tanh(g) - o.gelu_tanh(-g), g, atol=1e-12)  # odd part is x/2
    assert abs(o.gelu_tanh(40.0) - 40.0) < 1e-12 and abs(o.gelu_tanh(-40.0)) < 1e-12


def pin_linear(o):
    a = RNG.standard_normal((3, 5))
    w = RNG.standard_normal((4, 5))
    b = RNG.standard_normal(4)
    ref = np.zeros((3, 4))
    for i in range(3):
        for j in range(4):
            s = b[j]
            for kk in range(5):
                s += a[i, kk] * w[j, kk]
            ref[i, j] = s
    assert np.allclose(o.linear(a, w, b), ref, rtol=1e-13)
    sq = RNG.standard_normal((4, 4))
    wsq = RNG.standard_normal((4, 4))
    ref2 = np.array([[sum(sq[i, kk] * wsq[j, kk] for kk in range(4)) for j in range(4)] for i in range(4)])
    assert np.allclose(o.linear(sq, wsq), ref2, rtol=1e-13)


def pin_modulation(o):
    d, t = 6, 5
    # chunk order shift | scale | gate from the bias alone
    b = np.concatenate([np.full(d, 1.0), np.full(d, 2.0), np.full(d, 3.0)])
    sh, sc, ga = o.modulation(np.ones(t), np.zeros((3 * d, t)), b)
    assert np.all(sh == 1.0) and np.all(sc == 2.0) and np.all(ga == 3.0)
    # SiLU is applied to temb before the linear: W picks one temb entry per row
    temb = RNG.standard_normal(t) * 3
    w = np.zeros((3 * d, t))
    for r in range(3 * d):
        w[r, r % t] = 1.0
    sh, sc, ga = o.modulation(temb, w, np.zeros(3 * d))
    m = np.concatenate([sh, sc, ga])
    ref = F.silu(t64(temb)).numpy()[np.arange(3 * d) % t]
    assert np.allclose(m, ref, rtol=1e-13)


def pin_rms_norm(o):
    H, Dh = 3, 16
    q = RNG.standard_normal((5, H * Dh)) * RNG.uniform(0.1, 10, (5, 1))
    y = o.rms_norm_heads(q, H, Dh, np.ones(Dh), 1e-6).reshape(5, H, Dh)
    assert np.allclose(np.sqrt((y ** 2).mean(-1)), 1.0, atol=1e-6)
    # scale invariance per head (up to eps)
    y2 = o.rms_norm_heads(q * 7.0, H, Dh, np.ones(Dh), 0.0)
    y1 = o.rms_norm_heads(q, H, Dh, np.ones(Dh), 0.0)
    assert np.allclose(y1, y2, rtol=1e-12)
    w = 1 + 0.1 * RNG.standard_normal(Dh)
    ref = F.rms_norm(t64(q).reshape(5, H, Dh), (Dh,), weight=t64(w), eps=1e-6).reshape(5, H * Dh).numpy()
    assert np.allclose(o.rms_norm_heads(q, H, Dh, w, 1e-6), ref, rtol=1e-12)


def pin_rope(o):
    H, Dh = 2, 16
    axes = (8, 8)
    pos = np.array([[0, 0], [1, 0], [0, 1], [3, 5], [7, 2]], np.int32)
    th = o.rope_angles(pos, axes, Dh)
    q = RNG.standard_normal((5, H * Dh))
    r = o.rope_apply(q, th, H, Dh)
    # position 0 on every axis: identity, bitwise
    assert np.array_equal(r[0], q[0])
    # norm of every pair is preserved
    pn = lambda a: np.hypot(a.reshape(5, H, Dh // 2, 2)[..., 0], a.reshape(5, H, Dh // 2, 2)[..., 1])
    assert np.allclose(pn(r), pn(q), rtol=1e-13)
    # closed form: pair 0 at row position 1 turns by base^0 = 1 radian
    e = np.zeros((1, Dh))
    e[0, 0] = 1.0
    r1 = o.rope_apply(e, o.rope_angles(np.array([[1, 0]]), axes, Dh), 1, Dh)
    assert np.allclose(r1[0, :2], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    # pair j'=2 of a chunk of 8 dims turns by 10000^(-1/2) = 0.01 per unit position
    e = np.zeros((1, Dh))
    e[0, 4] = 1.0
    r2 = o.rope_apply(e, o.rope_angles(np.array([[3, 0]]), axes, Dh), 1, Dh)
    assert np.allclose(r2[0, 4:6], [math.cos(0.03), math.sin(0.03)], atol=1e-15)
    # the first half of each head follows the row axis, the second the column axis
    th_r = o.rope_angles(np.array([[4, 0]]), axes, Dh)
    th_c = o.rope_angles(np.array([[0, 4]]), axes, Dh)
    assert np.all(th_r[0, :4] != 0) and np.all(th_r[0, 4:] == 0)
    assert np.all(th_c[0, :4] == 0) and np.all(th_c[0, 4:] != 0)
    # complex-number form: (t[2j] + i t[2j+1]) * e^{i theta}
    z = (q[:, 0::2] + 1j * q[:, 1::2]).reshape(5, H, Dh // 2) * np.exp(1j * th)[:, None, :]
    assert np.allclose(r[:, 0::2], z.real.reshape(5, -1), atol=1e-13)
    assert np.allclose(r[:, 1::2], z.imag.reshape(5, -1), atol=1e-13)
    # relative position: <R_m a, R_n b> = <R_{m-n} a, b> along one axis
    a = RNG.standard_normal((1, Dh))
    b = RNG.standard_normal((1, Dh))
    R = lambda v, p: o.rope_apply(v, o.rope_angles(np.array([p]), axes, Dh), 1, Dh)
    assert np.isclose((R(a, [9, 2]) * R(b, [4, 2])).sum(), (R(a, [5, 0]) * b).sum(), rtol=1e-12)


def pin_attention(o):
    # brute force with Python loops on a tiny case
    S, H, Dh = 5, 2, 4
    q, k, v = (RNG.standard_normal((S, H * Dh)) for _ in range(3))
    out = o.attention(q, k, v, H, Dh)
    for h in range(H):
        for i in range(S):
            sc = [sum(q[i, h * Dh + c] * k[j, h * Dh + c] for c in range(Dh)) / math.sqrt(Dh) for j in range(S)]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            for c in range(Dh):
                ref = sum(e[j] / z * v[j, h * Dh + c] for j in range(S))
                assert abs(out[i, h * Dh + c] - ref) < 1e-12
    # PyTorch SDPA (CPU, float64)
    S, H, Dh = 37, 3, 16
    q, k, v = (RNG.standard_normal((S, H * Dh)) * 2 for _ in range(3))
    ref = F.scaled_dot_product_attention(*(t64(a).reshape(S, H, Dh).transpose(0, 1) for a in (q, k, v)))
    assert np.allclose(o.attention(q, k, v, H, Dh), ref.transpose(0, 1).reshape(S, H * Dh).numpy(), rtol=1e-11, atol=1e-12)
    # special cases: one key -> v; equal keys -> mean(v); q = 0 -> mean(v)
    assert np.allclose(o.attention(q[:1], k[:1], v[:1], H, Dh), v[:1], atol=1e-14)
    keq = np.repeat(k[:1], S, axis=0)
    assert np.allclose(o.attention(q, keq, v, H, Dh), np.repeat(v.mean(0, keepdims=True), S, 0), atol=1e-12)
    assert np.allclose(o.attention(np.zeros_like(q), k, v, H, Dh), np.repeat(v.mean(0, keepdims=True), S, 0), atol=1e-12)
    # restricting the query rows returns exactly those rows
    rows = np.array([3, 0, 36])
    assert np.allclose(o.attention(q, k, v, H, Dh, q_rows=rows), o.attention(q, k, v, H, Dh)[rows], rtol=1e-13)


def pin_attention_chunks(o):
    # merging the chunks of any partition of the keys gives full attention
    S, H, Dh = 29, 2, 8
    q, k, v = (RNG.standard_normal((S, H * Dh)) * 1.5 for _ in range(3))
    full = o.attention(q, k, v, H, Dh)
    for bounds in ([0, 13, 29], [0, 1, 2, 10, 11, 29], [0, 4, 8, 12, 16, 20, 24, 28, 29]):
        parts = [o.attention_partial(q, k, v, H, Dh, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
        merged, lse = o.attention_merge(parts, H, Dh)
        assert np.allclose(merged, full, rtol=1e-12, atol=1e-12)
        # the merged lse is the lse of the whole key range
        assert np.allclose(lse, o.attention_partial(q, k, v, H, Dh, 0, S)[1], rtol=1e-13, atol=1e-13)
    # lse against scipy on scores computed with plain loops
    from scipy.special import logsumexp
    _, lse = o.attention_partial(q, k, v, H, Dh, 5, 17)
    for h in range(H):
        for i in range(S):
            sc = [sum(q[i, h * Dh + c] * k[j, h * Dh + c] for c in range(Dh)) / math.sqrt(Dh) for j in range(5, 17)]
            assert abs(lse[h, i] - logsumexp(sc)) < 1e-12
    # a one-key chunk returns that key's value row and its score
    oc, lc = o.attention_partial(q, k, v, H, Dh, 6, 7)
    assert np.allclose(oc, np.repeat(v[6:7], S, 0), atol=1e-14)
    for h in range(H):
        cs = slice(h * Dh, (h + 1) * Dh)
        assert np.allclose(lc[h], q[:, cs] @ k[6, cs] / math.sqrt(Dh), rtol=1e-13)
    # query rows restrict the output rows only
    rows = np.array([28, 3])
    oa, la = o.attention_partial(q, k, v, H, Dh, 2, 20)
    ob, lb = o.attention_partial(q, k, v, H, Dh, 2, 20, q_rows=rows)
    assert np.allclose(ob, oa[rows], rtol=1e-13) and np.allclose(lb, la[:, rows], rtol=1e-13)


def torch_block(shape, w, x, temb, pos):
    """The block composed from PyTorch float64 library routines, RoPE done
    with complex numbers; an independent second writing of the same block."""
    d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
    S = x.shape[0]
    X = t64(x)
    m = F.linear(F.silu(t64(temb)), t64(w.w_mod), t64(w.b_mod))
    shift, scale, gate = m.chunk(3)
    u = F.layer_norm(X, (d,), eps=shape.ln_eps) * (1 + scale) + shift
    z = F.linear(u, t64(w.w1), t64(w.b1))
    q, k, v, g = torch.split(z, [d, d, d, shape.mlp_hidden], dim=1)
    q = F.rms_norm(q.reshape(S, H, Dh), (Dh,), weight=t64(w.q_norm_w), eps=shape.qk_eps)
    k = F.rms_norm(k.reshape(S, H, Dh), (Dh,), weight=t64(w.k_norm_w), eps=shape.qk_eps)
    ang = []
    for a, D in enumerate(shape.rope_axes_dims):
        freq = shape.rope_base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
        ang.append(torch.outer(t64(pos[:, a]), freq))
    rot = torch.polar(torch.ones(S, Dh // 2, dtype=torch.float64), torch.cat(ang, 1))[:, None, :]
    q = torch.view_as_real(torch.view_as_complex(q.reshape(S, H, Dh // 2, 2).contiguous()) * rot).reshape(S, H, Dh)
    k = torch.view_as_real(torch.view_as_complex(k.reshape(S, H, Dh // 2, 2).contiguous()) * rot).reshape(S, H, Dh)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.reshape(S, H, Dh).transpose(0, 1))
    o = o.transpose(0, 1).reshape(S, d)
    hb = F.linear(torch.cat([o, F.gelu(g, approximate="tanh")], 1), t64(w.w2), t64(w.b2))
    return (X + gate * hb).numpy()


def _small_block():
    sh = DI.small_shape(seq_len=40, dim=64, num_heads=2, head_dim=32, mlp_hidden=96,
                        grid=(4, 6), text_tokens=8, axes=(16, 16))
    w = DI.block_weights(sh, norm_weights="random", sigma=0.1)
    x, temb = DI.block_activations(sh)
    return sh, w, x, temb, DI.positions(sh)


def pin_block(o):
    sh, w, x, temb, pos = _small_block()
    y = o.block_forward(sh, w, x, temb, pos)
    ref = torch_block(sh, w, x, temb, pos)
    assert np.allclose(y, ref, rtol=1e-10, atol=1e-10)
    rows = np.array([0, 7, 8, 39])
    assert np.allclose(o.block_forward(sh, w, x, temb, pos, rows=rows), y[rows], rtol=1e-12, atol=1e-12)


def pin_round_bf16(o):
    a = RNG.standard_normal(4096) * np.exp(RNG.uniform(-20, 20, 4096))
    a = np.concatenate([a, [0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5]])
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(o.round_bf16(a), ref)


def pin_stack(o):
    sh, w, x, temb, pos = _small_block()
    w2 = DI.block_weights(sh, block=1, sigma=0.1)
    tembs = [temb, temb * 0.5]
    out = o.stack_forward(sh, [w, w2], x, tembs, pos)
    rb = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    for s in range(2):
        ref = o.block_forward(sh, w2, rb(o.block_forward(sh, w, x, tembs[s], pos)), tembs[s], pos)
        assert np.allclose(out[s], ref, rtol=1e-12, atol=1e-12)
    ch = o.stack_forward(sh, [w, w2], x, tembs, pos, chain=True)
    ref1 = o.block_forward(sh, w2, rb(o.block_forward(sh, w, rb(out[0]), tembs[1], pos)), tembs[1], pos)
    assert np.allclose(ch[1], ref1, rtol=1e-12, atol=1e-12)
    raw = o.stack_forward(sh, [w, w2], x, tembs, pos, bf16_io=False)
    ref2 = o.block_forward(sh, w2, o.block_forward(sh, w, x, tembs[0], pos), tembs[0], pos)
    assert np.allclose(raw[0], ref2, rtol=1e-12, atol=1e-12)
    # every gate zero (gate rows of W_mod and b_mod) -> the stack returns its input
    zw = []
    for wb in (w, w2):
        wm = wb.w_mod.copy()
        bm = wb.b_mod.copy()
        wm[2 * sh.dim:] = 0
        bm[2 * sh.dim:] = 0
        zw.append(DI.BlockWeights(wm, bm, wb.w1, wb.b1, wb.w2, wb.b2, wb.q_norm_w, wb.k_norm_w))
    assert np.array_equal(o.stack_forward(sh, zw, x, tembs, pos)[1], x.astype(np.float64))


# ------------------------------------------------- two-stream / sequential blocks
def _torch_rope(t, pos, shape):
    S, Dh = t.shape[0], shape.head_dim
    ang = []
    for a, D in enumerate(shape.rope_axes_dims):
        freq = shape.rope_base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
        ang.append(torch.outer(t64(pos[:, a]), freq))
    rot = torch.polar(torch.ones(S, Dh // 2, dtype=torch.float64), torch.cat(ang, 1))[:, None, :]
    return torch.view_as_real(torch.view_as_complex(t.reshape(S, -1, Dh // 2, 2).contiguous()) * rot).reshape(S, -1, Dh)


def torch_double_block(shape, wt, wi, x, temb, pos, n_txt):
    """The two-stream block from PyTorch float64 library routines: both
    streams' q, k, v concatenated for one scaled_dot_product_attention call,
    RoPE with complex numbers; an independent second writing."""
    d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
    X = t64(x)
    S = X.shape[0]
    parts = [(wt, slice(0, n_txt)), (wi, slice(n_txt, S))]
    qs, ks, vs, mods = [], [], [], []
    for w, sl in parts:
        m = F.linear(F.silu(t64(temb)), t64(w.w_mod), t64(w.b_mod)).chunk(6) if w is not None else None
        mods.append(m)
        if w is None or sl.stop <= sl.start:
            continue
        u = F.layer_norm(X[sl], (d,), eps=shape.ln_eps) * (1 + m[1]) + m[0]
        q, k, v = F.linear(u, t64(w.w_qkv), t64(w.b_qkv)).chunk(3, dim=1)
        n = sl.stop - sl.start
        q = F.rms_norm(q.reshape(n, H, Dh), (Dh,), weight=t64(w.q_norm_w), eps=shape.qk_eps)
        k = F.rms_norm(k.reshape(n, H, Dh), (Dh,), weight=t64(w.k_norm_w), eps=shape.qk_eps)
        qs.append(_torch_rope(q, pos[sl], shape))
        ks.append(_torch_rope(k, pos[sl], shape))
        vs.append(v.reshape(n, H, Dh))
    q, k, v = (torch.cat(t, 0).transpose(0, 1) for t in (qs, ks, vs))
    o = F.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(S, d)
    out = []
    for (w, sl), m in zip(parts, mods):
        if w is None or sl.stop <= sl.start:
            continue
        x1 = X[sl] + m[2] * F.linear(o[sl], t64(w.w_o), t64(w.b_o))
        u2 = F.layer_norm(x1, (d,), eps=shape.ln_eps) * (1 + m[4]) + m[3]
        hh = F.linear(F.gelu(F.linear(u2, t64(w.w_fc1), t64(w.b_fc1)), approximate="tanh"), t64(w.w_fc2), t64(w.b_fc2))
        out.append(x1 + m[5] * hh)
    return torch.cat(out, 0).numpy()


def _small_double(same_weights=False):
    sh = DI.small_shape(seq_len=40, dim=64, num_heads=2, head_dim=32, mlp_hidden=96,
                        grid=(4, 6), text_tokens=8, axes=(16, 16))
    wt = DI.stream_weights(sh, 0, norm_weights="random", sigma=0.1)
    wi = wt if same_weights else DI.stream_weights(sh, 1, norm_weights="random", sigma=0.1)
    x, temb = DI.block_activations(sh)
    return sh, wt, wi, x, temb, DI.positions(sh)


def _sw(w, **kw):
    f = dict(w.__dict__)
    f.update(kw)
    return DI.StreamWeights(**f)


def pin_double_block(o):
    sh, wt, wi, x, temb, pos = _small_double()
    for n_txt in (8, 1, 39, 40):
        y = o.double_block_forward(sh, wt, wi, x, temb, pos, n_txt=n_txt)
        ref = torch_double_block(sh, wt, wi, x, temb, pos, n_txt)
        assert np.allclose(y, ref, rtol=1e-10, atol=1e-10), n_txt
    y0 = o.sequential_block_forward(sh, wi, x, temb, pos)
    assert np.allclose(y0, torch_double_block(sh, None, wi, x, temb, pos, 0), rtol=1e-10, atol=1e-10)
    rows = np.array([0, 7, 8, 21, 39])
    y = o.double_block_forward(sh, wt, wi, x, temb, pos)
    assert np.allclose(o.double_block_forward(sh, wt, wi, x, temb, pos, rows=rows), y[rows], rtol=1e-12, atol=1e-12)


def pin_double_block_reductions(o):
    """Special cases that reduce the two-stream block to the (separately
    pinned) single-stream block, to its own halves, or to the identity."""
    sh, wt, wi, x, temb, pos = _small_double()
    d, T, S = sh.dim, sh.text_tokens, sh.seq_len
    y = o.double_block_forward(sh, wt, wi, x, temb, pos)
    # all six gates of both streams zero -> the input, bitwise
    zg = lambda w: _sw(w, w_mod=np.concatenate([w.w_mod[:2 * d], 0 * w.w_mod[2 * d:3 * d], w.w_mod[3 * d:5 * d],
                                                0 * w.w_mod[5 * d:]]),
                       b_mod=np.concatenate([w.b_mod[:2 * d], 0 * w.b_mod[2 * d:3 * d], w.b_mod[3 * d:5 * d],
                                             0 * w.b_mod[5 * d:]]))
    assert np.array_equal(o.double_block_forward(sh, zg(wt), zg(wi), x, temb, pos), x.astype(np.float64))
    # no attention branch (W_o = 0, b_o = 0): each stream is the single-stream
    # block whose linear2 ignores the attention columns, modulated by the
    # second triple (shift2, scale2, gate2)
    no_att = lambda w: _sw(w, w_o=0 * w.w_o, b_o=0 * w.b_o)
    ya = o.double_block_forward(sh, no_att(wt), no_att(wi), x, temb, pos)
    for w, sl in ((wt, slice(0, T)), (wi, slice(T, S))):
        bw = DI.BlockWeights(w_mod=w.w_mod[3 * d:], b_mod=w.b_mod[3 * d:],
                             w1=np.concatenate([w.w_qkv, w.w_fc1]), b1=np.concatenate([w.b_qkv, w.b_fc1]),
                             w2=np.concatenate([0 * w.w_o, w.w_fc2], axis=1), b2=w.b_fc2,
                             q_norm_w=w.q_norm_w, k_norm_w=w.k_norm_w)
        ref = o.block_forward(sh, bw, x[sl], temb, pos[sl])
        assert np.allclose(ya[sl], ref, rtol=1e-12, atol=1e-12)
    # no MLP branch (W_fc2 = 0, b_fc2 = 0) and one set of weights for both
    # streams: the single-stream block over all tokens whose linear2 ignores
    # the MLP columns, modulated by the first triple -- joint attention
    sh1, ws, _, x1, temb1, pos1 = _small_double(same_weights=True)
    no_mlp = _sw(ws, w_fc2=0 * ws.w_fc2, b_fc2=0 * ws.b_fc2)
    yb = o.double_block_forward(sh1, no_mlp, no_mlp, x1, temb1, pos1)
    bw = DI.BlockWeights(w_mod=ws.w_mod[:3 * d], b_mod=ws.b_mod[:3 * d],
                         w1=np.concatenate([ws.w_qkv, ws.w_fc1]), b1=np.concatenate([ws.b_qkv, ws.b_fc1]),
                         w2=np.concatenate([ws.w_o, 0 * ws.w_fc2], axis=1), b2=ws.b_o,
                         q_norm_w=ws.q_norm_w, k_norm_w=ws.k_norm_w)
    assert np.allclose(yb, o.block_forward(sh1, bw, x1, temb1, pos1), rtol=1e-12, atol=1e-12)
    # the block is its attention half followed by its MLP half
    half_a = lambda w: _sw(w, w_fc2=0 * w.w_fc2, b_fc2=0 * w.b_fc2)
    mid = o.double_block_forward(sh, half_a(wt), half_a(wi), x, temb, pos)
    yc = o.double_block_forward(sh, no_att(wt), no_att(wi), mid, temb, pos)
    assert np.allclose(yc, y, rtol=1e-12, atol=1e-12)
    # one set of weights: where the text/image boundary lies does not matter
    ys = [o.double_block_forward(sh1, ws, ws, x1, temb1, pos1, n_txt=t) for t in (0, 8, 40)]
    assert np.allclose(ys[0], ys[1], rtol=1e-12, atol=1e-12) and np.allclose(ys[0], ys[2], rtol=1e-12, atol=1e-12)
    # permuting image tokens together with their positions permutes the output
    perm = np.concatenate([np.arange(T), T + RNG.permutation(S - T)])
    yp = o.double_block_forward(sh, wt, wi, x[perm], temb, pos[perm])
    assert np.allclose(yp, y[perm], rtol=1e-12, atol=1e-12)


def pin_extrapolate_step(o):
    # exact on histories that are affine in the step time, for any times
    A = RNG.standard_normal((5, 7))
    Bv = RNG.standard_normal((5, 7))
    f = lambda t: A + Bv * t
    for ta, tb, ts in ((3.0, 2.0, 4.0), (0.7, 0.9, 0.1), (10.0, 2.0, 13.5), (1.0, 0.0, 1.0)):
        assert np.allclose(o.extrapolate_step(f(ta), f(tb), ts, ta, tb), f(ts), rtol=1e-12, atol=1e-12)
    # zero-order without a second point; the prediction at t_a is out_a
    assert np.array_equal(o.extrapolate_step(A, None, 5.0, 1.0, None), A)
    assert np.array_equal(o.extrapolate_step(A, Bv, 2.0, 2.0, 1.0), A)
    # uniform steps: out_s = 2 out_a - out_b
    assert np.allclose(o.extrapolate_step(A, Bv, 6, 5, 4), 2 * A - Bv, rtol=1e-14, atol=1e-14)


def pin_stack_cached(o):
    sh, w, x, temb, pos = _small_block()
    w2 = DI.block_weights(sh, block=1, sigma=0.1)
    tembs = [temb, temb * 0.5, temb * 0.25, temb * -0.5, temb * 0.75]
    full = o.stack_forward(sh, [w, w2], x, tembs, pos)
    # every step computed -> the plain stack, bitwise
    assert np.array_equal(o.stack_forward_cached(sh, [w, w2], x, tembs, pos, [1] * 5), full)
    # steps 2 and 4 skipped: computed steps unchanged, skipped ones predicted
    # from the bf16-stored history (times t)
    rb = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    t = [1.0, 0.8, 0.55, 0.3, 0.1]
    got = o.stack_forward_cached(sh, [w, w2], x, tembs, pos, [1, 1, 0, 1, 0], t=t)
    for s_ in (0, 1, 3):
        assert np.array_equal(got[s_], full[s_])
    p2 = rb(full[1]) + (t[2] - t[1]) / (t[1] - t[0]) * (rb(full[1]) - rb(full[0]))
    p4 = rb(full[3]) + (t[4] - t[3]) / (t[3] - t[1]) * (rb(full[3]) - rb(full[1]))
    assert np.allclose(got[2], p2, rtol=1e-12, atol=1e-12)
    assert np.allclose(got[4], p4, rtol=1e-12, atol=1e-12)
    # only step 0 computed: every later step holds its output
    hold = o.stack_forward_cached(sh, [w, w2], x, tembs, pos, [1, 0, 0, 0, 0])
    for s_ in range(1, 5):
        assert np.array_equal(hold[s_], rb(full[0]))
    # chained: the step after a skipped one starts from the stored prediction
    ch = o.stack_forward_cached(sh, [w, w2], x, tembs[:4], pos, [1, 1, 0, 1], chain=True)
    c0 = o.stack_forward(sh, [w, w2], x, tembs[:2], pos, chain=True)
    assert np.array_equal(ch[:2], c0)
    pred = rb(c0[1]) + (rb(c0[1]) - rb(c0[0]))
    assert np.allclose(ch[2], pred, rtol=1e-12, atol=1e-12)
    nxt = o.block_forward(sh, w2, rb(o.block_forward(sh, w, rb(ch[2]), tembs[3], pos)), tembs[3], pos)
    assert np.allclose(ch[3], nxt, rtol=1e-12, atol=1e-12)


def pin_flux_stack(o):
    sh, wt, wi, x, temb, pos = _small_double()
    wt2, wi2 = DI.stream_weights(sh, 0, block=1, sigma=0.1), DI.stream_weights(sh, 1, block=1, sigma=0.1)
    ws_ = DI.block_weights(sh, block=2, sigma=0.1)
    tembs = [temb, temb * 0.5]
    rb = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    out = o.flux_stack_forward(sh, [(wt, wi), (wt2, wi2)], [ws_], x, tembs, pos)
    for s_ in range(2):
        h1 = rb(o.double_block_forward(sh, wt, wi, x, tembs[s_], pos))
        h2 = rb(o.double_block_forward(sh, wt2, wi2, h1, tembs[s_], pos))
        assert np.allclose(out[s_], o.block_forward(sh, ws_, h2, tembs[s_], pos), rtol=1e-12, atol=1e-12)
    # no two-stream blocks: the single-stream stack
    assert np.array_equal(o.flux_stack_forward(sh, [], [ws_], x, tembs, pos), o.stack_forward(sh, [ws_], x, tembs, pos))
    # every gate zero -> the input, bitwise
    d = sh.dim
    zg = lambda w: _sw(w, w_mod=np.concatenate([w.w_mod[:2 * d], 0 * w.w_mod[2 * d:3 * d], w.w_mod[3 * d:5 * d],
                                                0 * w.w_mod[5 * d:]]),
                       b_mod=np.concatenate([w.b_mod[:2 * d], 0 * w.b_mod[2 * d:3 * d], w.b_mod[3 * d:5 * d],
                                             0 * w.b_mod[5 * d:]]))
    wz = DI.BlockWeights(np.concatenate([ws_.w_mod[:2 * d], 0 * ws_.w_mod[2 * d:]]),
                         np.concatenate([ws_.b_mod[:2 * d], 0 * ws_.b_mod[2 * d:]]), ws_.w1, ws_.b1, ws_.w2, ws_.b2,
                         ws_.q_norm_w, ws_.k_norm_w)
    z = o.flux_stack_forward(sh, [(zg(wt), zg(wi))], [wz], x, tembs, pos, chain=True)
    assert np.array_equal(z[1], x.astype(np.float64))


PINS = [pin_layer_norm, pin_modulate, pin_gated_residual, pin_silu, pin_gelu, pin_linear,
        pin_modulation, pin_rms_norm, pin_rope, pin_attention, pin_attention_chunks, pin_block, pin_round_bf16,
        pin_stack, pin_double_block, pin_double_block_reductions, pin_extrapolate_step, pin_stack_cached, pin_flux_stack]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(O)


# ------------------------------------------------------------ input module
def test_bf16_rounding_is_rne():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], np.float32)
    r = DI.round_bf16(a)
    # halfway 1 + 2^-8 ties to even (1.0); 1 + 3*2^-8 ties to even (1 + 2^-6)
    assert list(r) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]
    x = DI.draw(5, (1000,))
    assert np.array_equal(DI.round_bf16(x), x)            # already bf16 values
    assert torch.equal(torch.from_numpy(x).to(torch.bfloat16).float(), torch.from_numpy(x))


def test_positions_layout():
    pos = DI.positions(DI.FLUX)
    assert pos.shape == (4608, 2)
    assert np.all(pos[:512] == 0)
    assert tuple(pos[512]) == (0, 0) and tuple(pos[513]) == (0, 1) and tuple(pos[512 + 64]) == (1, 0)
    assert tuple(pos[-1]) == (63, 63)
    pv = DI.positions(DI.VIDEO)
    assert pv.shape == (16384, 3) and tuple(pv[-1]) == (15, 31, 31) and tuple(pv[1024]) == (1, 0, 0)
    assert sum(DI.VIDEO.rope_axes_dims) == 128 and sum(DI.FLUX.rope_axes_dims) == 128


# ------------------------------------------------- planted mistakes in the oracle
def _mut_gelu_no_cubic(g):
    g = np.asarray(g, np.float64)
    return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * g))


def _mut_ln_unbiased(x, eps):
    x = np.asarray(x, np.float64)
    mu = x.mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps)


def _mut_ln_eps_outside(x, eps):
    x = np.asarray(x, np.float64)
    mu = x.mean(-1, keepdims=True)
    return (x - mu) / (np.sqrt(x.var(-1, keepdims=True)) + eps)


def _mut_rope_sign(t, theta, H, Dh):
    S = t.shape[0]
    t = np.asarray(t, np.float64).reshape(S, H, Dh // 2, 2)
    c, s = np.cos(theta)[:, None, :], np.sin(theta)[:, None, :]
    a, b = t[..., 0], t[..., 1]
    return np.stack([a * c + b * s, -a * s + b * c], -1).reshape(S, H * Dh)


def _mut_rope_half_split(pos, axes_dims, head_dim, base=10000.0):
    # both axes share one frequency ladder over the whole head (wrong exponent)
    pos = np.asarray(pos, np.float64)
    cols = []
    off = 0
    for a, D in enumerate(axes_dims):
        jp = np.arange(off, off + D // 2, dtype=np.float64)
        cols.append(pos[:, a:a + 1] * (base ** (-2.0 * jp / head_dim))[None, :])
        off += D // 2
    return np.concatenate(cols, 1)


_ORIG_ATTENTION = O.attention


def _mut_attention_noscale(q, k, v, H, Dh, q_rows=None):
    return _ORIG_ATTENTION(q * math.sqrt(Dh), k, v, H, Dh, q_rows)


_ORIG_MODULATION = O.modulation


def _mut_modulation_order(temb, w_mod, b_mod):
    sh, sc, ga = _ORIG_MODULATION(temb, w_mod, b_mod)
    return sc, sh, ga


def _mut_rms_whole_row(t, H, Dh, w, eps=1e-6):
    t = np.asarray(t, np.float64)
    r = np.sqrt((t ** 2).mean(-1, keepdims=True) + eps)
    return ((t / r).reshape(t.shape[0], H, Dh) * np.asarray(w, np.float64)).reshape(t.shape[0], H * Dh)


def _mut_gated_on_x(x, gate, h):
    return np.asarray(gate, np.float64) * np.asarray(x, np.float64) + np.asarray(h, np.float64)


def _mut_silu_sigmoid(z):
    z = np.asarray(z, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _mut_round_truncate(a):
    f = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def _mut_merge_plain_mean(parts, num_heads, head_dim):
    out = sum(np.asarray(o_c, np.float64) for o_c, _ in parts) / len(parts)
    lses = np.stack([np.asarray(l, np.float64) for _, l in parts])
    return out, np.log(np.exp(lses).sum(0))


def _mut_partial_lse_log2(q, k, v, num_heads, head_dim, kv_begin, kv_end, q_rows=None):
    out, lse = _REAL_PARTIAL(q, k, v, num_heads, head_dim, kv_begin, kv_end, q_rows)
    return out, lse / np.log(2.0)


_REAL_PARTIAL = O.attention_partial

MUTANTS = [
    ("round_bf16", _mut_round_truncate, pin_round_bf16),
    ("round_bf16", _mut_round_truncate, pin_stack),
    ("gelu_tanh", _mut_gelu_no_cubic, pin_gelu),
    ("layer_norm", _mut_ln_unbiased, pin_layer_norm),
    ("layer_norm", _mut_ln_eps_outside, pin_layer_norm),
    ("rope_apply", _mut_rope_sign, pin_rope),
    ("rope_angles", _mut_rope_half_split, pin_rope),
    ("attention", _mut_attention_noscale, pin_attention),
    ("modulation", _mut_modulation_order, pin_modulation),
    ("rms_norm_heads", _mut_rms_whole_row, pin_rms_norm),
    ("gated_residual", _mut_gated_on_x, pin_gated_residual),
    ("silu", _mut_silu_sigmoid, pin_silu),
    ("attention_merge", _mut_merge_plain_mean, pin_attention_chunks),
    ("attention_partial", _mut_partial_lse_log2, pin_attention_chunks),
    # the same mistakes must also break the whole-block pin
    ("gelu_tanh", _mut_gelu_no_cubic, pin_block),
    ("rope_apply", _mut_rope_sign, pin_block),
    ("rms_norm_heads", _mut_rms_whole_row, pin_block),
    ("modulation", _mut_modulation_order, pin_block),
]


@pytest.mark.parametrize("name,mutant,pin", MUTANTS,
                         ids=[f"{m[0]}-{m[1].__name__}-{m[2].__name__}" for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pin):
    monkeypatch.setattr(O, name, mutant)
    with pytest.raises(AssertionError):
        pin(O)


def _double_with_bug(bug):
    """A two-stream block with one planted mistake, for the pins to catch."""
    def f(shape, w_txt, w_img, x, temb, pos, n_txt=None, rows=None):
        d, H, Dh = shape.dim, shape.num_heads, shape.head_dim
        x = np.asarray(x, np.float64)
        S = x.shape[0]
        n_txt = shape.text_tokens if n_txt is None else n_txt
        theta = O.rope_angles(pos, shape.rope_axes_dims, Dh, shape.rope_base)
        streams = [(w_txt, 0, n_txt), (w_img, n_txt, S)]
        if bug == "text_uses_image_weights":
            streams = [(w_img, 0, n_txt), (w_img, n_txt, S)]
        q, k, v = (np.zeros((S, d)) for _ in range(3))
        mods = []
        for w, a, b in streams:
            m = O.stream_modulation(temb, w.w_mod, w.b_mod) if w is not None else None
            if bug == "gates_swapped" and m is not None:
                m = (m[0], m[1], m[5], m[3], m[4], m[2])
            mods.append(m)
            if b <= a:
                continue
            u = O.layer_norm_modulate(x[a:b], m[0], m[1], shape.ln_eps)
            z = O.linear(u, w.w_qkv, w.b_qkv)
            th = theta[0:b - a] if bug == "rope_not_offset" else theta[a:b]
            q[a:b] = O.rope_apply(O.rms_norm_heads(z[:, :d], H, Dh, w.q_norm_w, shape.qk_eps), th, H, Dh)
            k[a:b] = O.rope_apply(O.rms_norm_heads(z[:, d:2 * d], H, Dh, w.k_norm_w, shape.qk_eps), th, H, Dh)
            v[a:b] = z[:, 2 * d:]
        out = np.zeros((S, d))
        for (w, a, b), m in zip(streams, mods):
            if b <= a:
                continue
            if bug == "stream_local_attention":
                o = O.attention(q[a:b], k[a:b], v[a:b], H, Dh)
            else:
                o = O.attention(q, k, v, H, Dh, q_rows=np.arange(a, b))
            x1 = O.gated_residual(x[a:b], m[2], O.linear(o, w.w_o, w.b_o))
            u2 = O.layer_norm_modulate(x[a:b] if bug == "ln2_on_x" else x1, m[3], m[4], shape.ln_eps)
            mlp = O.linear(O.gelu_tanh(O.linear(u2, w.w_fc1, w.b_fc1)), w.w_fc2, w.b_fc2)
            out[a:b] = O.gated_residual(x1, m[5], mlp)
        return out if rows is None else out[np.asarray(rows)]
    return f


def _mut_stream_modulation_branch_order(temb, w_mod, b_mod):
    m = _REAL_STREAM_MOD(temb, w_mod, b_mod)
    return m[3:] + m[:3]


_REAL_STREAM_MOD = O.stream_modulation


def test_double_block_bug_free_variant_passes():
    # the variant machinery itself, with no bug, satisfies every pin
    import types
    shim = types.SimpleNamespace(**{k: getattr(O, k) for k in dir(O) if not k.startswith("__")})
    shim.double_block_forward = _double_with_bug(None)
    shim.sequential_block_forward = lambda sh, w, x, temb, pos, rows=None: shim.double_block_forward(
        sh, None, w, x, temb, pos, n_txt=0, rows=rows)
    pin_double_block(shim)
    pin_double_block_reductions(shim)


@pytest.mark.parametrize("bug", ["text_uses_image_weights", "gates_swapped", "rope_not_offset",
                                 "stream_local_attention", "ln2_on_x"])
def test_planted_double_block_mistake_is_caught(monkeypatch, bug):
    monkeypatch.setattr(O, "double_block_forward", _double_with_bug(bug))
    with pytest.raises(AssertionError):
        pin_double_block(O)
    with pytest.raises(AssertionError):
        pin_double_block_reductions(O)


def test_planted_stream_modulation_order_is_caught(monkeypatch):
    monkeypatch.setattr(O, "stream_modulation", _mut_stream_modulation_branch_order)
    with pytest.raises(AssertionError):
        pin_double_block(O)


def _mut_extrapolate_sign(out_a, out_b, t_s, t_a, t_b):
    if out_b is None:
        return np.asarray(out_a, np.float64).copy()
    return np.asarray(out_a, np.float64) - (t_s - t_a) / (t_a - t_b) * (np.asarray(out_a) - np.asarray(out_b))


def _mut_extrapolate_step_index(out_a, out_b, t_s, t_a, t_b):
    # ignores the step times: always one step ahead
    if out_b is None:
        return np.asarray(out_a, np.float64).copy()
    return 2 * np.asarray(out_a, np.float64) - np.asarray(out_b)


@pytest.mark.parametrize("mutant", [_mut_extrapolate_sign, _mut_extrapolate_step_index])
def test_planted_extrapolation_mistake_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(O, "extrapolate_step", mutant)
    with pytest.raises(AssertionError):
        pin_extrapolate_step(O)
    with pytest.raises(AssertionError):
        pin_stack_cached(O)


def test_planted_linear_transpose_is_caught(monkeypatch):
    monkeypatch.setattr(O, "linear", lambda a, w, b=None: (np.asarray(a, float) @ np.asarray(w, float)) + (0 if b is None else b))
    with pytest.raises((AssertionError, ValueError)):
        pin_linear(O)


def test_planted_linear2_order_is_caught(monkeypatch):
    real = O.linear

    def swapped(a, w, b=None):
        a = np.asarray(a, float)
        if a.shape[1] == 64 + 96 and w.shape == (64, 160):     # linear2 of the small block
            a = np.concatenate([a[:, 64:], a[:, :64]], 1)
        return real(a, w, b)
    monkeypatch.setattr(O, "linear", swapped)
    with pytest.raises(AssertionError):
        pin_block(O)

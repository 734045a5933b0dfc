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


PINS = [pin_layer_norm, pin_modulate, pin_gated_residual, pin_silu, pin_gelu, pin_linear,
        pin_modulation, pin_rms_norm, pin_rope, pin_attention, pin_attention_chunks, pin_block, pin_round_bf16,
        pin_stack]


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

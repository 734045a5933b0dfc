"""GPU parity of each kernel of the block against the CPU oracle, through the
C ABI, on seeded inputs from dit_inputs.  Sizes span several tiles plus a
ragged tail; the Flux-size cases compare sampled rows the oracle computes
one by one."""
import numpy as np
import pytest

import dit_inputs as DI
from oracle import dit_oracle as O
from tests.parity import assert_parity, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def _rng(seed):
    return np.random.default_rng(seed)


def _vec(seed, n, sigma):
    return (_rng(seed).standard_normal(n, dtype=np.float32) * np.float32(sigma))


# ------------------------------------------------------------ modulation GEMV
@pytest.mark.parametrize("d,tdim", [(256, 256), (3072, 3072), (1536, 1536), (64, 40), (8192, 8192)])
def test_modulation(gpu_lib, d, tdim):
    temb = DI.draw(11, (tdim,), 1.0)
    w = DI.draw(12, (3 * d, tdim), 0.02)
    b = DI.draw(13, (3 * d,), 0.02)
    mod = gpu_lib.modulation(dev_bf16(temb), dev_bf16(w), dev_bf16(b))
    ref = np.concatenate(O.modulation(temb, w, b))
    assert_parity(host(mod), ref, f"modulation d={d}", quantum=None)
    # without a bias
    mod0 = gpu_lib.modulation(dev_bf16(temb), dev_bf16(w), None)
    assert_parity(host(mod0), np.concatenate(O.modulation(temb, w, np.zeros(3 * d))), "modulation nobias",
                  quantum=None)


# ------------------------------------------------------------ LN + modulate
@pytest.mark.parametrize("rows,cols", [(4608, 3072), (37, 264), (256, 256), (1, 8), (129, 8192), (300, 1536)])
def test_modulate_norm(gpu_lib, rows, cols):
    ch = DI.chain_inputs(rows, cols)
    x = ch["x"] * 1.5 + 0.25      # non-zero mean and non-unit spread per row
    x = DI.round_bf16(x.astype(np.float32))
    out = gpu_lib.modulate_norm(dev_bf16(x), dev_f32(ch["shift"]), dev_f32(ch["scale"]), 1e-6)
    ref = O.layer_norm_modulate(x, ch["shift"], ch["scale"], 1e-6)
    assert_parity(host(out), ref, f"modulate_norm {rows}x{cols}")


def test_modulate_norm_empty_and_inplace(gpu_lib):
    import torch
    x = dev_bf16(DI.draw(3, (0, 256)))
    z = dev_f32(np.zeros(256, np.float32))
    assert gpu_lib.modulate_norm(x, z, z).shape == (0, 256)
    xv = DI.draw(4, (64, 512))
    xt = dev_bf16(xv)
    z512 = dev_f32(np.zeros(512, np.float32))
    gpu_lib.modulate_norm(xt, z512, z512, 1e-6, out=xt)
    torch.cuda.synchronize()
    assert_parity(host(xt), O.layer_norm(xv, 1e-6), "modulate_norm in place")


def test_modulate_norm_scale_minus_one_gives_shift(gpu_lib):
    x = DI.draw(5, (64, 1024))
    shift = _vec(6, 1024, 1.0)
    out = gpu_lib.modulate_norm(dev_bf16(x), dev_f32(shift), dev_f32(-np.ones(1024, np.float32)))
    assert np.array_equal(host(out), np.repeat(DI.round_bf16(shift)[None, :], 64, 0).astype(np.float64))


# ------------------------------------------------------------ gated residual
@pytest.mark.parametrize("rows,cols", [(4608, 3072), (37, 264), (1, 8), (513, 8192)])
def test_gated_residual(gpu_lib, rows, cols):
    ch = DI.chain_inputs(rows, cols)
    y = gpu_lib.gated_residual(dev_bf16(ch["x"]), dev_bf16(ch["h"]), dev_f32(ch["gate"]))
    ref = O.gated_residual(ch["x"], ch["gate"], ch["h"])
    assert_parity(host(y), ref, f"gated_residual {rows}x{cols}")


@pytest.mark.parametrize("into", ["x", "h"])
def test_gated_residual_in_place(gpu_lib, into):
    """y may be x or h (the header allows both)."""
    import torch
    ch = DI.chain_inputs(513, 3072)
    xt, ht = dev_bf16(ch["x"]), dev_bf16(ch["h"])
    gpu_lib.gated_residual(xt, ht, dev_f32(ch["gate"]), out=xt if into == "x" else ht)
    torch.cuda.synchronize()
    ref = O.gated_residual(ch["x"], ch["gate"], ch["h"])
    assert_parity(host(xt if into == "x" else ht), ref, f"gated_residual in place into {into}")


def test_gated_residual_gate_zero_is_identity(gpu_lib):
    ch = DI.chain_inputs(300, 3072)
    y = gpu_lib.gated_residual(dev_bf16(ch["x"]), dev_bf16(ch["h"]), dev_f32(np.zeros(3072, np.float32)))
    assert np.array_equal(host(y), ch["x"].astype(np.float64))


# ------------------------------------------------------------ RoPE tables
@pytest.mark.parametrize("shape", [DI.TINY, DI.FLUX, DI.VIDEO])
def test_rope_table(gpu_lib, shape):
    import torch
    pos = DI.positions(shape)
    c, s = gpu_lib.rope_table(torch.from_numpy(pos).cuda(), list(shape.rope_axes_dims), shape.head_dim,
                              shape.rope_base)
    th = O.rope_angles(pos, shape.rope_axes_dims, shape.head_dim, shape.rope_base)
    assert np.max(np.abs(host(c) - np.cos(th))) < 2e-5
    assert np.max(np.abs(host(s) - np.sin(th))) < 2e-5
    # position 0 is exactly the identity rotation
    zero = np.all(pos == 0, axis=1)
    assert np.all(host(c)[zero] == 1.0) and np.all(host(s)[zero] == 0.0)


# ------------------------------------------------------------ QK RMSNorm + RoPE
@pytest.mark.parametrize("S,H,Dh", [(4608, 24, 128), (77, 3, 64), (130, 2, 128)])
def test_qk_rmsnorm_rope(gpu_lib, S, H, Dh):
    import torch
    d = H * Dh
    qkv = DI.draw(21, (S, 3 * d), 1.0)
    qw = (1 + 0.1 * _rng(22).standard_normal(Dh)).astype(np.float32)
    kw = (1 + 0.1 * _rng(23).standard_normal(Dh)).astype(np.float32)
    pos = _rng(24).integers(0, 64, size=(S, 2)).astype(np.int32)
    pos[:5] = 0
    th = O.rope_angles(pos, (Dh // 2, Dh // 2), Dh)
    cos_t, sin_t = gpu_lib.rope_table(torch.from_numpy(pos).cuda(), [Dh // 2, Dh // 2], Dh)
    t = dev_bf16(qkv)
    gpu_lib.qk_rmsnorm_rope(t, dev_f32(qw), dev_f32(kw), cos_t, sin_t, H, Dh, 1e-6)
    g = host(t)
    q_ref = O.rope_apply(O.rms_norm_heads(qkv[:, :d], H, Dh, qw, 1e-6), th, H, Dh)
    k_ref = O.rope_apply(O.rms_norm_heads(qkv[:, d:2 * d], H, Dh, kw, 1e-6), th, H, Dh)
    assert_parity(g[:, :d], q_ref, f"q rmsnorm+rope S={S}")
    assert_parity(g[:, d:2 * d], k_ref, f"k rmsnorm+rope S={S}")
    assert np.array_equal(g[:, 2 * d:], qkv[:, 2 * d:].astype(np.float64))  # v untouched


# ------------------------------------------------------------ attention
def _qkv_for_attention(S, H, Dh, seed):
    """q and k with unit RMS per head (as after the QK RMSNorm), v ~ N(0,1)."""
    d = H * Dh
    qkv = DI.draw(seed, (S, 3 * d), 1.0)
    return qkv


# The last two cases give grids of >= 256 eight-wave workgroups, which selects
# the 8-wave (256-query) kernel; the others run the 4-wave kernel.
@pytest.mark.parametrize("S,H,Dh", [(200, 2, 128), (256, 4, 64), (64, 1, 128), (1, 2, 64), (333, 3, 128),
                                    (129, 2, 64), (300, 128, 64), (800, 64, 128)])
def test_attention_small(gpu_lib, S, H, Dh):
    import torch
    d = H * Dh
    qkv = _qkv_for_attention(S, H, Dh, 31)
    out = torch.zeros(S, d + 64, dtype=torch.bfloat16, device="cuda")
    gpu_lib.attention(dev_bf16(qkv), out, H, Dh)
    ref = O.attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], H, Dh)
    g = host(out)
    assert_parity(g[:, :d], ref, f"attention S={S} H={H} Dh={Dh}")
    assert np.all(g[:, d:] == 0)  # columns past H*Dh untouched


@pytest.mark.parametrize("S,H", [(300, 2), (800, 64)])  # 4-wave and 8-wave kernels
def test_attention_sharp_scores(gpu_lib, S, H):
    """Scores far from 0 (large |q|, |k|) exercise the running max."""
    import torch
    Dh = 128
    d = H * Dh
    qkv = _qkv_for_attention(S, H, Dh, 32)
    qkv[:, :2 * d] = DI.round_bf16((qkv[:, :2 * d] * 3.0).astype(np.float32))
    out = torch.empty(S, d, dtype=torch.bfloat16, device="cuda")
    gpu_lib.attention(dev_bf16(qkv), out, H, Dh)
    ref = O.attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], H, Dh)
    assert_parity(host(out), ref, f"attention sharp S={S} H={H}")


@pytest.mark.parametrize("S,H", [(4608, 24), (16384, 12)])
def test_attention_full_size(gpu_lib, S, H):
    """The Flux shape on every query row; the video shape on sampled rows
    (every key is always used)."""
    import torch
    Dh = 128
    d = H * Dh
    qkv = _qkv_for_attention(S, H, Dh, 33)
    out = torch.empty(S, d, dtype=torch.bfloat16, device="cuda")
    gpu_lib.attention(dev_bf16(qkv), out, H, Dh)
    rows = np.arange(S) if S <= 8192 else \
        np.unique(np.concatenate([np.arange(0, S, S // 29), [S - 1, 127, 128, 511, 512]]))
    ref = O.attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], H, Dh, q_rows=rows)
    assert_parity(host(out)[rows], ref, f"attention S={S} ({len(rows)} rows)")


def test_attention_qkv_beyond_4gib(gpu_lib):
    """q|k|v larger than 4 GiB (S = 87500 tokens at width 8192): every key
    tile must be read whole wherever it sits.  Head h is the seeded one-head
    q, k, v rolled by h tokens; query rows 0 and S-1 point at key 120 (a
    needle that takes almost all of their softmax weight), so a key tile
    read as zeros would change their outputs completely."""
    import torch
    S, H, Dh, needle = 87500, 64, 128, 120
    d = H * Dh
    assert S * 3 * d * 2 > 1 << 32
    base = _qkv_for_attention(S, 1, Dh, 35)            # [S, 3*Dh]: q | k | v of one head
    rows = np.array([0, 1, 40000, S - 1])
    qb = base[:, :Dh].copy()
    kb, vb = base[:, Dh:2 * Dh], base[:, 2 * Dh:]

    def head(a, h):
        return np.roll(a, h, axis=0)

    # needle rows, per head: q = 2 k_needle (the rolled head's key at that token)
    qrows = {}
    for h in range(H):
        kh = kb[(needle - h) % S]
        for r in (0, S - 1):
            qrows[(h, r)] = DI.round_bf16((2.0 * kh).astype(np.float32))
    qkv = torch.empty(S, 3 * d, dtype=torch.bfloat16, device="cuda")
    parts = [dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)]
    for h in range(H):
        for part in range(3):
            qkv[:, part * d + h * Dh: part * d + (h + 1) * Dh] = torch.roll(parts[part], h, 0)
        for r in (0, S - 1):
            qkv[r, h * Dh:(h + 1) * Dh] = dev_bf16(qrows[(h, r)])
    del parts
    out = torch.empty(S, d, dtype=torch.bfloat16, device="cuda")
    gpu_lib.attention(qkv, out, H, Dh)
    torch.cuda.synchronize()
    g = host(out[torch.from_numpy(rows).cuda()])
    del qkv, out
    for h in (0, 1, 31, 63):
        qh = head(qb, h)
        for r in (0, S - 1):
            qh[r] = qrows[(h, r)]
        ref = O.attention(qh, head(kb, h), head(vb, h), 1, Dh, q_rows=rows)
        assert_parity(g[:, h * Dh:(h + 1) * Dh], ref, f"attention beyond 4 GiB, head {h}")


# ------------------------------------------ chunked attention + LSE merge
@pytest.mark.parametrize("S,H,Dh,bounds", [
    (333, 3, 128, [0, 100, 333]),                 # ragged chunks
    (333, 3, 128, [0, 1, 17, 18, 200, 333]),      # one-token chunks
    (256, 4, 64, [0, 64, 128, 192, 256]),         # tile-aligned, Dh = 64
    (129, 2, 64, [0, 65, 129]),
    (300, 128, 64, [0, 100, 300]),                # 8-wave partials (grid of 256 workgroups)
])
def test_attention_partial_and_merge(gpu_lib, S, H, Dh, bounds):
    import torch
    B = gpu_lib
    d = H * Dh
    qkv = _qkv_for_attention(S, H, Dh, 34)
    qd = dev_bf16(qkv)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    C = len(bounds) - 1
    o_parts = torch.empty(C, S, d, dtype=torch.float32, device="cuda")
    lses = torch.empty(C, H, S, dtype=torch.float32, device="cuda")
    for c, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        B.attention_partial(qd, H, Dh, a, b, o_part=o_parts[c], lse=lses[c])
    torch.cuda.synchronize()
    for c, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        ro, rl = O.attention_partial(q, k, v, H, Dh, a, b)
        assert_parity(host(o_parts[c]), ro, f"partial o [{a},{b})", quantum=None)
        gl = host(lses[c])
        assert np.max(np.abs(gl - rl)) <= 1e-3 * max(1.0, float(np.max(np.abs(rl)))), (a, b)
    out = torch.zeros(S, d + 64, dtype=torch.bfloat16, device="cuda")
    B.attention_merge(o_parts, lses, out, H, Dh)
    ref = O.attention(q, k, v, H, Dh)
    g = host(out)
    assert_parity(g[:, :d], ref, f"merged attention S={S} chunks={C}")
    assert np.all(g[:, d:] == 0)  # columns past H*Dh untouched


def test_attention_merge_row_stride_multiple_of_four(gpu_lib):
    """ld_out = H*Dh + 4: the merge's stores need only 8-byte alignment."""
    import torch
    B = gpu_lib
    S, H, Dh, bounds = 77, 2, 64, [0, 30, 77]
    d = H * Dh
    qkv = _qkv_for_attention(S, H, Dh, 36)
    qd = dev_bf16(qkv)
    C = len(bounds) - 1
    o_parts = torch.empty(C, S, d, dtype=torch.float32, device="cuda")
    lses = torch.empty(C, H, S, dtype=torch.float32, device="cuda")
    for c, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        B.attention_partial(qd, H, Dh, a, b, o_part=o_parts[c], lse=lses[c])
    out = torch.zeros(S, d + 4, dtype=torch.bfloat16, device="cuda")
    B.attention_merge(o_parts, lses, out, H, Dh)
    g = host(out)
    assert_parity(g[:, :d], O.attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], H, Dh), "merge ld_out = d + 4")
    assert np.all(g[:, d:] == 0)


def test_attention_chunked_flux_eight_chunks(gpu_lib):
    """The pages' 8-way split of the Flux sequence (8 x 576 keys), merged on one GPU."""
    import torch
    B = gpu_lib
    S, H, Dh, C = 4608, 24, 128, 8
    d = H * Dh
    qkv = _qkv_for_attention(S, H, Dh, 35)
    qd = dev_bf16(qkv)
    o_parts = torch.empty(C, S, d, dtype=torch.float32, device="cuda")
    lses = torch.empty(C, H, S, dtype=torch.float32, device="cuda")
    for c in range(C):
        B.attention_partial(qd, H, Dh, c * 576, (c + 1) * 576, o_part=o_parts[c], lse=lses[c])
    out = torch.empty(S, d, dtype=torch.bfloat16, device="cuda")
    B.attention_merge(o_parts, lses, out, H, Dh)
    full = torch.empty(S, d, dtype=torch.bfloat16, device="cuda")
    B.attention(qd, full, H, Dh)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, S, S // 23), [S - 1, 575, 576]]))
    ref = O.attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], H, Dh, q_rows=rows)
    assert_parity(host(out)[rows], ref, "merged attention flux 8x576")
    # and against the single-pass kernel on every row: two bf16 results, each
    # within the bar of the exact one, differ by at most twice the bar
    st = assert_parity(host(out), host(full), "merged vs single-pass attention", check_max_abs=False)
    assert st["excess"] <= 2 * 2e-2 * st["rms"], st


SPLIT_CASES = [(300, 2, 128, 3), (129, 2, 64, 2), (5, 1, 128, 8), (4608, 3, 128, 4), (256, 4, 64, 1),
               (300, 64, 128, 2)]  # the last: 8-wave partials


@pytest.mark.parametrize("S,H,Dh,n", SPLIT_CASES, ids=[f"S{c[0]}-H{c[1]}-D{c[2]}-n{c[3]}" for c in SPLIT_CASES])
def test_attention_split(gpu_lib, S, H, Dh, n):
    """Split-key attention (one launch of chunk partials + the merge) against
    the oracle; the 3-head Flux-length case is one GPU's share of the heads
    under an 8-way head split."""
    import torch
    B = gpu_lib
    d = H * Dh
    print(f"attention split S={S} H={H} Dh={Dh} n={n}", flush=True)
    qkv = _qkv_for_attention(S, H, Dh, 36)
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    out = torch.zeros(S, d + 64, dtype=torch.bfloat16, device="cuda")
    B.attention_split(dev_bf16(qkv), out, H, Dh, n)
    torch.cuda.synchronize()
    rows = np.arange(S) if S <= 512 else np.unique(np.concatenate([np.arange(0, S, 97), [S - 1]]))
    ref = O.attention(q, k, v, H, Dh, q_rows=rows)
    g = host(out)
    assert_parity(g[rows, :d], ref, f"split attention S={S} H={H} n={n}")
    assert np.all(g[:, d:] == 0)


def test_attention_split_rejects_bad_chunk_counts(gpu_lib):
    import torch
    B = gpu_lib
    qkv = torch.zeros(64, 3 * 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")
    for n in (0, 65):
        with pytest.raises(B.DitError):
            B.attention_split(qkv, out, 1, 128, n, o_parts=torch.empty(max(n, 1), 64, 128, device="cuda"),
                              lses=torch.empty(max(n, 1), 1, 64, device="cuda"))


def test_attention_partial_rejects_bad_ranges(gpu_lib):
    import torch
    B = gpu_lib
    qd = dev_bf16(_qkv_for_attention(64, 1, 64, 36))
    for a, b in ((0, 0), (10, 5), (-1, 10), (0, 65)):
        with pytest.raises(B.DitError):
            B.attention_partial(qd, 1, 64, a, b)


# ------------------------------------------------------------ linear1 + GELU
# (300, 8192, 8192): the largest dim the row kernels accept.  (3000, 64, 4288),
# (3000, 128, 4096) and (3000, 256, 3776) run on the four-wave 256x256 kernel
# with a partial last tile row and column and 1, 2 and 4 K slices of 64.
@pytest.mark.parametrize("S,d,mlp", [(300, 256, 1024), (4608, 3072, 12288), (97, 128, 192), (300, 8192, 8192),
                                   (3000, 64, 4288), (3000, 128, 4096), (3000, 256, 3776)])
def test_linear1_gelu(gpu_lib, S, d, mlp):
    import torch
    u = DI.draw(41, (S, d), 1.0)
    w1 = DI.draw(42, (3 * d + mlp, d), 0.02)
    b1 = DI.draw(43, (3 * d + mlp,), 0.02)
    qkv = torch.empty(S, 3 * d, dtype=torch.bfloat16, device="cuda")
    cat = torch.zeros(S, d + mlp, dtype=torch.bfloat16, device="cuda")
    gpu_lib.linear1_gelu(dev_bf16(u), dev_bf16(w1), dev_bf16(b1), qkv, cat, mlp)
    rows = np.arange(S) if S <= 8192 else np.unique(np.concatenate([np.arange(0, S, 61), [S - 1]]))
    z = O.linear(u[rows], w1, b1)
    assert_parity(host(qkv)[rows], z[:, :3 * d], f"linear1 qkv S={S}")
    c = host(cat)[rows]
    assert_parity(c[:, d:], O.gelu_tanh(z[:, 3 * d:]), f"linear1 gelu S={S}")
    assert np.all(c[:, :d] == 0)  # attention columns untouched


# ------------------------------------------------------------ linear2 + gated residual
# (16384, 1536, 8960) and (16000, 1536, 8960) run on 256x192 tiles, the
# second with a half-filled last tile row
@pytest.mark.parametrize("S,d,mlp", [(300, 256, 1024), (4608, 3072, 12288), (97, 128, 192), (16384, 1536, 8960),
                                   (16000, 1536, 8960), (300, 8192, 8192)])
def test_linear2_gated_residual(gpu_lib, S, d, mlp):
    cat = DI.draw(51, (S, d + mlp), 1.0)
    w2 = DI.draw(52, (d, d + mlp), 0.02)
    b2 = DI.draw(53, (d,), 0.02)
    x = DI.draw(54, (S, d), 1.0)
    gate = _vec(55, d, 0.5)
    xt = dev_bf16(x)
    y = gpu_lib.linear2_gated_residual(dev_bf16(cat), dev_bf16(w2), dev_bf16(b2), xt, dev_f32(gate),
                                       dev_bf16(np.zeros((S, d), np.float32)))
    rows = np.arange(S) if S <= 8192 else np.unique(np.concatenate([np.arange(0, S, 97), [S - 1]]))
    h = O.linear(cat[rows], w2, b2)
    yg = host(y)[rows]
    assert_parity(yg, O.gated_residual(x[rows], gate, h), f"linear2 y S={S}")
    # the branch alone (the residual hides branch errors in y): gate = 1, x = 0
    hb = gpu_lib.linear2_gated_residual(dev_bf16(cat), dev_bf16(w2), dev_bf16(b2),
                                        dev_bf16(np.zeros((S, d), np.float32)), dev_f32(np.ones(d, np.float32)),
                                        dev_bf16(np.zeros((S, d), np.float32)))
    assert_parity(host(hb)[rows], h, f"linear2 branch S={S}")


def test_linear1_gelu_without_bias(gpu_lib):
    """The epilogue path without a bias (no column loads), four-wave kernel, partial edge tiles."""
    import torch
    S, d, mlp = 3000, 256, 3776
    u = DI.draw(44, (S, d), 1.0)
    w1 = DI.draw(45, (3 * d + mlp, d), 0.02)
    qkv = torch.empty(S, 3 * d, dtype=torch.bfloat16, device="cuda")
    cat = torch.zeros(S, d + mlp, dtype=torch.bfloat16, device="cuda")
    gpu_lib.linear1_gelu(dev_bf16(u), dev_bf16(w1), None, qkv, cat, mlp)
    z = O.linear(u, w1)
    assert_parity(host(qkv), z[:, :3 * d], "linear1 qkv, no bias")
    assert_parity(host(cat)[:, d:], O.gelu_tanh(z[:, 3 * d:]), "linear1 gelu, no bias")


def test_linear2_in_place(gpu_lib):
    import torch
    S, d, mlp = 200, 256, 512
    cat = DI.draw(61, (S, d + mlp), 1.0)
    w2 = DI.draw(62, (d, d + mlp), 0.02)
    x = DI.draw(63, (S, d), 1.0)
    gate = _vec(64, d, 0.5)
    xt = dev_bf16(x)
    gpu_lib.linear2_gated_residual(dev_bf16(cat), dev_bf16(w2), None, xt, dev_f32(gate), xt)
    torch.cuda.synchronize()
    assert_parity(host(xt), O.gated_residual(x, gate, O.linear(cat, w2)), "linear2 in place")


def test_kernels_are_deterministic(gpu_lib):
    import torch
    S, d, mlp = 4608, 3072, 12288
    u = dev_bf16(DI.draw(71, (S, d)))
    w1 = dev_bf16(DI.draw(72, (3 * d + mlp, d), 0.02))
    outs = []
    for _ in range(2):
        qkv = torch.empty(S, 3 * d, dtype=torch.bfloat16, device="cuda")
        cat = torch.empty(S, d + mlp, dtype=torch.bfloat16, device="cuda")
        gpu_lib.linear1_gelu(u, w1, None, qkv, cat, mlp)
        o = torch.empty(S, d + mlp, dtype=torch.bfloat16, device="cuda")
        gpu_lib.attention(qkv, o, 24, 128)
        outs.append((qkv, cat[:, d:], o[:, :d]))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)

"""GPU parity of the whole block forward and of the captured block stack
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import dit_inputs as DI
from oracle import dit_oracle as O
from tests import bf16_boundaries as BB
from tests.parity import assert_attributed, assert_parity, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


class DevBlock:
    """Seeded weights of one block on the GPU plus the host copy for the oracle."""

    def __init__(self, B, shape, block=0, norm_weights="ones", w=None):
        self.w = w if w is not None else DI.block_weights(shape, block, norm_weights)
        w = self.w
        self.dev = B.BlockWeights(dev_bf16(w.w_mod), dev_bf16(w.b_mod), dev_bf16(w.w1), dev_bf16(w.b1),
                                  dev_bf16(w.w2), dev_bf16(w.b2), dev_f32(w.q_norm_w), dev_f32(w.k_norm_w))


def rope_dev(B, shape):
    import torch
    pos = DI.positions(shape)
    return (pos,) + B.rope_table(torch.from_numpy(pos).cuda(), list(shape.rope_axes_dims), shape.head_dim,
                                 shape.rope_base)


def cfg_of(B, shape, flags=0):
    return B.make_config(shape.seq_len, shape.dim, shape.num_heads, shape.head_dim, shape.mlp_hidden,
                         shape.tdim, shape.ln_eps, shape.qk_eps, flags)


# sequences up to this length are compared on every row (the oracle takes a
# few seconds per Flux-shape block); longer ones on sampled rows
FULL_ROWS_MAX_S = 8192


def sample_rows(S, extra=()):
    if S <= FULL_ROWS_MAX_S:
        return np.arange(S)
    return np.unique(np.concatenate([np.arange(0, S, max(1, S // 40)), [S - 1], list(extra)])).astype(np.int64)


BLOCK_SHAPES = [
    DI.TINY,
    DI.small_shape(seq_len=300, dim=256, num_heads=2, head_dim=128, mlp_hidden=512, grid=(10, 12),
                   text_tokens=60, axes=(64, 64), name="ragged300"),
    DI.small_shape(seq_len=77, dim=128, num_heads=2, head_dim=64, mlp_hidden=192, grid=(7, 11),
                   text_tokens=0, axes=(32, 32), name="ragged77"),
    DI.small_shape(seq_len=1, dim=256, num_heads=4, head_dim=64, mlp_hidden=256, grid=(1, 1),
                   text_tokens=0, axes=(32, 32), name="single_token"),
    DI.FLUX,
    DI.VIDEO,
    # Flux widths with a ragged sequence: linear1 runs on 256x256 tiles here,
    # so the q/k RMSNorm + RoPE happens in its epilogue (the small shapes
    # above take the separate kernel); the last tile has 160 rows
    DI.small_shape(seq_len=4000, dim=3072, num_heads=24, head_dim=128, mlp_hidden=12288, grid=(60, 60),
                   text_tokens=400, axes=(64, 64), name="flux_ragged4000"),
    # the last tile has 60 rows: its second row of waves lies wholly past the
    # sequence, so the head epilogue's row count is zero there
    DI.small_shape(seq_len=3900, dim=3072, num_heads=24, head_dim=128, mlp_hidden=12288, grid=(60, 58),
                   text_tokens=420, axes=(64, 64), name="flux_ragged3900"),
]


@pytest.mark.parametrize("shape", BLOCK_SHAPES, ids=[s.name for s in BLOCK_SHAPES])
def test_block_forward(gpu_lib, shape):
    """Block output y, and every stage of the branch, read back from the
    workspace (u, q/k after RMSNorm+RoPE, v, attention output, GELU output,
    and h = linear2 of the GPU's own concat buffer with gate 1, x 0)."""
    import torch
    B = gpu_lib
    blk = DevBlock(B, shape, norm_weights="random")
    x, temb = DI.block_activations(shape)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.block_workspace_bytes(cfg))
    y = B.block_forward(cfg, blk.dev, dev_bf16(x), dev_bf16(temb), rc, rs, workspace=ws)
    torch.cuda.synchronize()
    rows = sample_rows(shape.seq_len, extra=(shape.text_tokens - 1, shape.text_tokens))
    rows = rows[(rows >= 0) & (rows < shape.seq_len)]
    print(f"block {shape.name}: S={shape.seq_len}, comparing {len(rows)} rows", flush=True)
    ref, it = O.block_forward(shape, blk.w, x, temb, pos, rows=rows, return_intermediates=True)
    mref, mit = BB.block_forward_bf16(shape, blk.w, x, temb, pos, rows=rows, return_intermediates=True)
    assert_attributed(host(y)[rows], ref, mref, f"block y {shape.name}")

    S, d, mlp = shape.seq_len, shape.dim, shape.mlp_hidden
    a = lambda n: (n + 255) // 256 * 256
    off_u = a(3 * d * 4)
    off_qkv = off_u + a(S * d * 2)
    off_cat = off_qkv + a(S * 3 * d * 2)
    mod = ws[:3 * d * 4].view(torch.float32)
    u = ws[off_u:off_u + S * d * 2].view(torch.bfloat16).view(S, d)
    qkv = ws[off_qkv:off_qkv + S * 3 * d * 2].view(torch.bfloat16).view(S, 3 * d)
    cat = ws[off_cat:off_cat + S * (d + mlp) * 2].view(torch.bfloat16).view(S, d + mlp)
    assert_parity(host(mod), np.concatenate([it["shift"], it["scale"], it["gate"]]), "mod", quantum=None)
    assert_parity(host(u)[rows], it["u"], f"u {shape.name}")
    qg = host(qkv)[rows]
    assert_attributed(qg[:, :d], it["q"], mit["q"], f"q {shape.name}")
    assert_attributed(qg[:, d:2 * d], it["k"], mit["k"], f"k {shape.name}")
    assert_attributed(qg[:, 2 * d:], it["v"], mit["v"], f"v {shape.name}")
    cg = host(cat)[rows]
    assert_attributed(cg[:, :d], it["o"], mit["o"], f"attention out {shape.name}")
    assert_attributed(cg[:, d:], it["a"], mit["a"], f"gelu out {shape.name}")
    w = blk.dev.tensors
    hb = B.linear2_gated_residual(cat, w[4], w[5], torch.zeros(S, d, dtype=torch.bfloat16, device="cuda"),
                                  torch.ones(d, dtype=torch.float32, device="cuda"),
                                  torch.empty(S, d, dtype=torch.bfloat16, device="cuda"))
    assert_attributed(host(hb)[rows], it["h"], mit["h"], f"branch h {shape.name}")


def test_block_forward_in_place_and_deterministic(gpu_lib):
    import torch
    B = gpu_lib
    shape = DI.TINY
    blk = DevBlock(B, shape)
    x, temb = DI.block_activations(shape)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.block_workspace_bytes(cfg))
    y1 = B.block_forward(cfg, blk.dev, dev_bf16(x), dev_bf16(temb), rc, rs, workspace=ws)
    y2 = B.block_forward(cfg, blk.dev, dev_bf16(x), dev_bf16(temb), rc, rs, workspace=ws)
    xt = dev_bf16(x)
    B.block_forward(cfg, blk.dev, xt, dev_bf16(temb), rc, rs, y=xt, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, xt)


def test_block_gate_zero_is_identity(gpu_lib):
    import torch
    B = gpu_lib
    shape = DI.TINY
    w = DI.block_weights(shape)
    w.w_mod[2 * shape.dim:] = 0
    w.b_mod[2 * shape.dim:] = 0
    blk = DevBlock(B, shape, w=w)
    x, temb = DI.block_activations(shape)
    _, rc, rs = rope_dev(B, shape)
    y = B.block_forward(cfg_of(B, shape), blk.dev, dev_bf16(x), dev_bf16(temb), rc, rs)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), x.astype(np.float64))


# ------------------------------------------------------------------ stack
STACK_TINY = DI.BlockShape("stack_tiny", 3, 256, 256, 4, 64, 1024, (32, 32), (16, 16), 0)


def _stack_inputs(B, shape, n_blocks, n_steps):
    blocks = [DevBlock(B, shape, block=b) for b in range(n_blocks)]
    x, _ = DI.block_activations(shape)
    tembs = np.stack([DI.step_temb(shape, s) for s in range(n_steps)])
    return blocks, x, tembs


def _replay(B, shape, blocks, x, tembs, rc, rs, chain=False):
    import torch
    cfg = cfg_of(B, shape, B.DIT_STACK_CHAIN if chain else 0)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    n = tembs.shape[0]
    out = torch.empty(n, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    st.replay(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws)
    torch.cuda.synchronize()
    st.close()
    return host(out)


@pytest.mark.parametrize("chain", [False, True])
def test_stack_replay_per_block_parity(gpu_lib, chain):
    """Inside the replayed graph every block matches the oracle on the same
    bf16 input: the output of the k-block stack is compared with the oracle's
    block k applied to the GPU's (k-1)-block output, for every k."""
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 6, 2
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    pos, rc, rs = rope_dev(B, shape)
    prev = None
    for k in range(1, n_blocks + 1):
        out = _replay(B, shape, blocks[:k], x, tembs, rc, rs, chain)
        for s in range(n_steps):
            if k == 1:
                xin = x if (s == 0 or not chain) else out[s - 1]
            else:
                xin = prev[s]
            ref = O.block_forward(shape, blocks[k - 1].w, xin, tembs[s], pos)
            if chain and s > 0 and k > 1:
                continue  # its input (step s-1 of the full stack) is not this stack's output
            assert_parity(out[s], ref, f"stack block {k} step {s} chain={chain}")
        prev = out
    # free-running comparison with the oracle stack (bf16 between blocks): drift report
    ref = O.stack_forward(shape, [b.w for b in blocks], x, tembs, pos, chain=chain)
    for s in range(n_steps):
        assert_parity(out[s], ref[s], f"stack free-running step {s} chain={chain} (drift report)",
                      check_max_abs=False)


def test_stack_57_blocks(gpu_lib):
    """57 blocks at the tiny shape, 2 steps: the last block inside the 57-deep
    graph against the oracle on the same input (56-block output), plus the
    free-running drift against the oracle stack (cosine asserted, max-abs
    reported)."""
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 57, 2
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    pos, rc, rs = rope_dev(B, shape)
    out56 = _replay(B, shape, blocks[:56], x, tembs, rc, rs)
    out57 = _replay(B, shape, blocks, x, tembs, rc, rs)
    for s in range(n_steps):
        ref = O.block_forward(shape, blocks[56].w, out56[s], tembs[s], pos)
        assert_parity(out57[s], ref, f"57-block stack, block 57 step {s}")
    ref = O.stack_forward(shape, [b.w for b in blocks], x, tembs, pos)
    for s in range(n_steps):
        assert_parity(out57[s], ref[s], f"57-block stack free-running step {s} (drift report)",
                      check_max_abs=False)


def test_stack_replay_equals_eager_bitwise(gpu_lib):
    import torch
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 5, 3
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    out = torch.empty(n_steps, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    xd, td = dev_bf16(x), dev_bf16(tembs)
    # replay twice with eager work in between: every replay must match eager
    for rep in range(2):
        st.replay(cfg, [b.dev for b in blocks], xd, td, rc, rs, out, ws)
        wse = B.alloc_workspace(B.block_workspace_bytes(cfg))
        for s in range(n_steps):
            cur = xd.clone()
            for b in blocks:
                B.block_forward(cfg, b.dev, cur, td[s].contiguous(), rc, rs, y=cur, workspace=wse)
            torch.cuda.synchronize()
            assert torch.equal(cur, out[s]), f"replay {rep} step {s}"
    st.close()


def test_stack_replay_equals_eager_bitwise_flux_shape(gpu_lib):
    """At the Flux shape the stack takes the paths the small shapes do not
    (batched 6-chunk modulation, q/k RMSNorm + RoPE in linear1's epilogue,
    8-wave attention): 3 blocks x 2 steps replayed twice, each step bitwise
    the eager block forwards.  Inputs are seeded device draws; no oracle."""
    import torch
    B = gpu_lib
    shape = DI.FLUX
    S, d, mlp, Dh = shape.seq_len, shape.dim, shape.mlp_hidden, shape.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rn = lambda *sz, s=0.02: (torch.randn(*sz, generator=g, device="cuda") * s).to(torch.bfloat16)
    blocks = [B.BlockWeights(rn(3 * d, d), rn(3 * d), rn(3 * d + mlp, d), rn(3 * d + mlp), rn(d, d + mlp), rn(d),
                             torch.rand(Dh, generator=g, device="cuda") + 0.5,
                             torch.rand(Dh, generator=g, device="cuda") + 0.5) for _ in range(3)]
    x = rn(S, d, s=1.0)
    tembs = rn(2, d, s=1.0)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    out = torch.empty(2, S, d, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    wse = B.alloc_workspace(B.block_workspace_bytes(cfg))
    for rep in range(2):
        st.replay(cfg, blocks, x, tembs, rc, rs, out, ws)
        for s in range(2):
            cur = x.clone()
            for b in blocks:
                B.block_forward(cfg, b, cur, tembs[s].contiguous(), rc, rs, y=cur, workspace=wse)
            torch.cuda.synchronize()
            assert torch.isfinite(out[s].float()).all()
            assert torch.equal(cur, out[s]), f"replay {rep} step {s}"
    st.close()


def test_stack_all_gates_zero_returns_input(gpu_lib):
    import torch
    B = gpu_lib
    shape = STACK_TINY
    blocks = []
    for b in range(6):
        w = DI.block_weights(shape, b)
        w.w_mod[2 * shape.dim:] = 0
        w.b_mod[2 * shape.dim:] = 0
        blocks.append(DevBlock(B, shape, w=w))
    x, _ = DI.block_activations(shape)
    tembs = np.stack([DI.step_temb(shape, s) for s in range(2)])
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    out = torch.empty(2, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    st.replay(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws)
    torch.cuda.synchronize()
    for s in range(2):
        assert np.array_equal(host(out[s]), x.astype(np.float64))
    st.close()


def test_stack_graph_key_mismatch(gpu_lib):
    import torch
    B = gpu_lib
    shape = STACK_TINY
    blocks, x, tembs = _stack_inputs(B, shape, 2, 1)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    out = torch.empty(1, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    xd = dev_bf16(x)
    st.replay(cfg, [b.dev for b in blocks], xd, dev_bf16(tembs), rc, rs, out, ws)
    with pytest.raises(B.DitError) as e:
        st.replay(cfg, [b.dev for b in blocks[:1]], xd, dev_bf16(tembs), rc, rs, out, ws)
    assert e.value.code == B.DIT_ERR_GRAPH_KEY
    torch.cuda.synchronize()
    st.close()


def test_stack_probes_time_kernels_without_changing_results(gpu_lib):
    import torch
    B = gpu_lib
    shape = STACK_TINY
    blocks, x, tembs = _stack_inputs(B, shape, 3, 2)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    outs = []
    for probe in (False, True):
        ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
        out = torch.empty(2, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
        st = B.Stack()
        if probe:
            st.set_probe(B.Stack.KERNELS)
        st.replay(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws)
        torch.cuda.synchronize()
        if probe:
            pm = st.probe_ms(3)
            assert set(pm) == set(B.Stack.KERNELS)
            for k, v in pm.items():
                assert len(v) == 3, (k, v)
                if k == "modulation":
                    # one launch computes every block's modulation at the start
                    # of the step: block 0's bracket holds it, the others are empty
                    assert v[0] > 0 and all(abs(t) < 0.01 for t in v[1:]), (k, v)
                elif k == "qk_rmsnorm_rope":
                    # done in linear1's epilogue: the bracket is empty
                    assert all(abs(t) < 0.01 for t in v), (k, v)
                else:
                    assert all(t > 0 for t in v), (k, v)
            with pytest.raises(B.DitError):
                st.probe_ms(3)  # nothing replayed since the last read
            with pytest.raises(B.DitError):
                st.set_probe(["attention"])  # after capture
        st.close()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])


def test_stack_graph_kernel_count(gpu_lib):
    """Launches per block inside the captured stack, read from the graph
    itself: one batched modulation launch per step, then per block
    LayerNorm+modulate, linear1 (whose epilogue also does the q/k RMSNorm +
    RoPE, at head_dim 128 and 64), attention and linear2.  The Flux page
    (sections 2 and 3.2) counts 52 kernels per eager block forward and 12
    compiled."""
    import torch
    B = gpu_lib
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    for shape, n_blocks, per_block in ((DI.FLUX, 2, 4), (STACK_TINY, 3, 4)):
        S, d, mlp, Dh = shape.seq_len, shape.dim, shape.mlp_hidden, shape.head_dim
        rn = lambda *sz, s=0.02: (torch.randn(*sz, generator=g, device="cuda") * s).to(torch.bfloat16)
        blocks = [B.BlockWeights(rn(3 * d, d), rn(3 * d), rn(3 * d + mlp, d), rn(3 * d + mlp), rn(d, d + mlp),
                                 rn(d), torch.ones(Dh, device="cuda"), torch.ones(Dh, device="cuda"))
                  for _ in range(n_blocks)]
        _, rc, rs = rope_dev(B, shape)
        cfg = cfg_of(B, shape)
        ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
        out = torch.empty(1, S, d, dtype=torch.bfloat16, device="cuda")
        st = B.Stack()
        with pytest.raises(B.DitError):
            st.graph_info()  # nothing captured yet
        st.replay(cfg, blocks, rn(S, d, s=1.0), rn(1, d, s=1.0), rc, rs, out, ws)
        torch.cuda.synchronize()
        k, n = st.graph_info()
        print(f"[graph] {shape.name}: {n_blocks} blocks -> {k} kernel nodes of {n} nodes", flush=True)
        assert k == n == 1 + per_block * n_blocks
        st.close()

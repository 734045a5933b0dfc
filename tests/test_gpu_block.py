"""GPU parity of the whole block forward and of the captured block stack
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import dit_inputs as DI
from oracle import dit_oracle as O
from tests.parity import assert_parity, dev_bf16, dev_f32, host

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


def sample_rows(S, extra=()):
    if S <= 512:
        return np.arange(S)
    return np.unique(np.concatenate([np.arange(0, S, max(1, S // 40)), [S - 1], list(extra)]))


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
]


@pytest.mark.parametrize("shape", BLOCK_SHAPES, ids=[s.name for s in BLOCK_SHAPES])
def test_block_forward(gpu_lib, shape):
    B = gpu_lib
    blk = DevBlock(B, shape, norm_weights="random" if shape.seq_len < 1000 else "ones")
    x, temb = DI.block_activations(shape)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    y = B.block_forward(cfg, blk.dev, dev_bf16(x), dev_bf16(temb), rc, rs)
    rows = sample_rows(shape.seq_len, extra=(shape.text_tokens - 1, shape.text_tokens))
    rows = rows[(rows >= 0) & (rows < shape.seq_len)]
    ref, inter = O.block_forward(shape, blk.w, x, temb, pos, rows=rows, return_intermediates=True)
    yg = host(y)[rows]
    assert_parity(yg, ref, f"block y {shape.name}")
    # the branch before the residual: h = (y - x) / gate
    gate = inter["gate"]
    ok = np.abs(gate) > 0.05
    hg = (yg - x[rows])[:, ok] / gate[ok][None, :]
    print(f"[info] {shape.name}: branch compared on {ok.sum()} of {gate.size} channels")
    assert_parity(hg, inter["h"][:, ok], f"block branch h {shape.name}")


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


@pytest.mark.parametrize("chain", [False, True])
def test_stack_replay_matches_oracle(gpu_lib, chain):
    import torch
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 8, 3
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape, B.DIT_STACK_CHAIN if chain else 0)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg))
    out = torch.empty(n_steps, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    st.replay(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws)
    ref = O.stack_forward(shape, [b.w for b in blocks], x, tembs, pos, chain=chain)
    for s in range(n_steps):
        assert_parity(host(out[s]), ref[s], f"stack step {s} chain={chain}")
    st.close()


def test_stack_57_blocks_reduced_depth(gpu_lib):
    """57 blocks at the tiny shape, 2 steps, against the oracle (drift report)."""
    import torch
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 57, 2
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg))
    out = torch.empty(n_steps, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    st.replay(cfg, [b.dev for b in blocks], dev_bf16(x), dev_bf16(tembs), rc, rs, out, ws)
    ref = O.stack_forward(shape, [b.w for b in blocks], x, tembs, pos)
    for s in range(n_steps):
        assert_parity(host(out[s]), ref[s], f"57-block stack step {s}")
    st.close()


def test_stack_replay_equals_eager_bitwise(gpu_lib):
    import torch
    B = gpu_lib
    shape = STACK_TINY
    n_blocks, n_steps = 5, 3
    blocks, x, tembs = _stack_inputs(B, shape, n_blocks, n_steps)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg))
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
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg))
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
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg))
    out = torch.empty(1, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    xd = dev_bf16(x)
    st.replay(cfg, [b.dev for b in blocks], xd, dev_bf16(tembs), rc, rs, out, ws)
    with pytest.raises(B.DitError) as e:
        st.replay(cfg, [b.dev for b in blocks[:1]], xd, dev_bf16(tembs), rc, rs, out, ws)
    assert e.value.code == B.DIT_ERR_GRAPH_KEY
    torch.cuda.synchronize()
    st.close()

"""GPU tests of the Flux-style stack (two-stream blocks, then single-stream
blocks, in one captured graph) through dit_stack_replay_mixed."""
import numpy as np
import pytest

import dit_inputs as DI
from oracle import dit_oracle as O
from tests.parity import assert_parity, dev_bf16, host
from tests.test_gpu_block import DevBlock, cfg_of, rope_dev
from tests.test_gpu_mmdit import DevStream

pytestmark = pytest.mark.gpu

MIX = DI.small_shape(seq_len=256, dim=256, num_heads=4, head_dim=64, mlp_hidden=1024, grid=(16, 16),
                     text_tokens=64, axes=(32, 32), name="mix256")
T = MIX.text_tokens


def _weights(B, n_double, n_single):
    doubles = [(DevStream(B, MIX, 0, w=DI.stream_weights(MIX, 0, block=b)),
                DevStream(B, MIX, 1, w=DI.stream_weights(MIX, 1, block=b))) for b in range(n_double)]
    singles = [DevBlock(B, MIX, block=10 + b) for b in range(n_single)]
    return doubles, singles


def _run(B, doubles, singles, x, tembs, rc, rs, fresh=None, chain=False):
    import torch
    cfg = cfg_of(B, MIX, B.DIT_STACK_CHAIN if chain else 0)
    ws = B.alloc_workspace(B.stack_mixed_workspace_bytes(cfg, T, len(doubles), len(singles)))
    out = torch.empty(tembs.shape[0], MIX.seq_len, MIX.dim, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    st.replay_mixed(cfg, T, [(t.dev, i.dev) for t, i in doubles], [s.dev for s in singles], dev_bf16(x),
                    dev_bf16(tembs), rc, rs, out, ws, fresh)
    torch.cuda.synchronize()
    st.close()
    return host(out)


def test_mixed_stack_per_block_parity(gpu_lib):
    """Every block inside the captured graph against the oracle on the same
    bf16 input (the GPU's output of the stack one block shorter)."""
    B = gpu_lib
    doubles, singles = _weights(B, 2, 3)
    x, _ = DI.block_activations(MIX)
    tembs = np.stack([DI.step_temb(MIX, s) for s in range(2)])
    pos, rc, rs = rope_dev(B, MIX)
    prev = np.stack([x.astype(np.float64)] * 2)
    plan = [(1, 0), (2, 0), (2, 1), (2, 2), (2, 3)]
    for nd, ns in plan:
        print(f"mixed stack {nd} two-stream + {ns} single", flush=True)
        out = _run(B, doubles[:nd], singles[:ns], x, tembs, rc, rs)
        for s in range(2):
            if ns == 0:
                t, i = doubles[nd - 1]
                ref = O.double_block_forward(MIX, t.w, i.w, prev[s], tembs[s], pos, n_txt=T)
            else:
                ref = O.block_forward(MIX, singles[ns - 1].w, prev[s], tembs[s], pos)
            assert_parity(out[s], ref, f"mixed stack ({nd}, {ns}) step {s}")
        prev = out
    full = O.flux_stack_forward(MIX, [(t.w, i.w) for t, i in doubles], [s.w for s in singles], x, tembs, pos,
                                n_txt=T)
    for s in range(2):
        assert_parity(out[s], full[s], f"mixed stack free-running step {s} (drift report)", check_max_abs=False)


def test_mixed_stack_replay_equals_eager_bitwise(gpu_lib):
    import torch
    B = gpu_lib
    doubles, singles = _weights(B, 2, 2)
    x, _ = DI.block_activations(MIX)
    tembs = np.stack([DI.step_temb(MIX, s) for s in range(3)])
    _, rc, rs = rope_dev(B, MIX)
    out = _run(B, doubles, singles, x, tembs, rc, rs)
    cfg = cfg_of(B, MIX)
    wsm = B.alloc_workspace(B.mmdit_block_workspace_bytes(cfg))
    wsb = B.alloc_workspace(B.block_workspace_bytes(cfg))
    td = dev_bf16(tembs)
    for s in range(3):
        cur = dev_bf16(x)
        for t, i in doubles:
            B.mmdit_block_forward(cfg, T, t.dev, i.dev, cur, td[s].contiguous(), rc, rs, y=cur, workspace=wsm)
        for b in singles:
            B.block_forward(cfg, b.dev, cur, td[s].contiguous(), rc, rs, y=cur, workspace=wsb)
        torch.cuda.synchronize()
        assert np.array_equal(host(cur), out[s]), s


def test_mixed_stack_replay_equals_eager_bitwise_flux_shape(gpu_lib):
    """The Flux composition at the Flux shape (512 text + 4096 image tokens):
    2 two-stream + 2 single-stream blocks x 2 steps, replayed twice, each
    step bitwise the eager block forwards (at this shape every block after
    the first gets its modulation vectors from the previous block's
    attention launch: two-stream -> two-stream, two-stream -> single-stream
    and single-stream -> single-stream).  Seeded device draws; no oracle."""
    import torch
    B = gpu_lib
    shape = DI.FLUX
    S, d, mlp, Dh, txt = shape.seq_len, shape.dim, shape.mlp_hidden, shape.head_dim, shape.text_tokens
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    rn = lambda *sz, s=0.02: (torch.randn(*sz, generator=g, device="cuda") * s).to(torch.bfloat16)
    nw = lambda: torch.rand(Dh, generator=g, device="cuda") + 0.5
    stream = lambda: B.StreamWeights(rn(6 * d, d), rn(6 * d), rn(3 * d, d), rn(3 * d), nw(), nw(), rn(d, d), rn(d),
                                     rn(mlp, d), rn(mlp), rn(d, mlp), rn(d))
    doubles = [(stream(), stream()) for _ in range(2)]
    singles = [B.BlockWeights(rn(3 * d, d), rn(3 * d), rn(3 * d + mlp, d), rn(3 * d + mlp), rn(d, d + mlp), rn(d),
                              nw(), nw()) for _ in range(2)]
    x = rn(S, d, s=1.0)
    tembs = rn(2, d, s=1.0)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_mixed_workspace_bytes(cfg, txt, len(doubles), len(singles)))
    wsm = B.alloc_workspace(B.mmdit_block_workspace_bytes(cfg))
    wsb = B.alloc_workspace(B.block_workspace_bytes(cfg))
    out = torch.empty(2, S, d, dtype=torch.bfloat16, device="cuda")
    st = B.Stack()
    for rep in range(2):
        st.replay_mixed(cfg, txt, doubles, singles, x, tembs, rc, rs, out, ws)
        for s in range(2):
            cur = x.clone()
            for t, i in doubles:
                B.mmdit_block_forward(cfg, txt, t, i, cur, tembs[s].contiguous(), rc, rs, y=cur, workspace=wsm)
            for b in singles:
                B.block_forward(cfg, b, cur, tembs[s].contiguous(), rc, rs, y=cur, workspace=wsb)
            torch.cuda.synchronize()
            assert torch.isfinite(out[s].float()).all()
            assert torch.equal(cur, out[s]), f"replay {rep} step {s}"
    st.close()


def test_mixed_stack_skipped_step(gpu_lib):
    B = gpu_lib
    doubles, singles = _weights(B, 1, 1)
    x, _ = DI.block_activations(MIX)
    tembs = np.stack([DI.step_temb(MIX, s) for s in range(3)])
    _, rc, rs = rope_dev(B, MIX)
    full = _run(B, doubles, singles, x, tembs, rc, rs)
    got = _run(B, doubles, singles, x, tembs, rc, rs, fresh=[1, 1, 0])
    assert np.array_equal(got[:2], full[:2])
    assert_parity(got[2], O.extrapolate_step(got[1], got[0], 2, 1, 0), "mixed stack skipped step")

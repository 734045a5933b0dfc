"""Capture safety of the block entry points on the caller's stream.

The Flux page ("ChituDiffusion: torch.compile and CUDA Graph on Flux.1-dev",
section 1.2) lists what a captured region may not do: allocate, synchronise
the host, or change shapes and addresses between replays.  The single-call
entry points only enqueue kernels on the caller's stream, so a caller may
capture them into its own graph; these tests capture them with PyTorch's
graph API, replay the graph several times with eager work and host
synchronisation between the replays, and check every replay against the
same call run eagerly, bitwise.  The stack replay is itself a graph launch
and refuses a capturing stream (DIT_ERR_CAPTURE), which is checked too.
"""
import numpy as np
import pytest

import dit_inputs as DI
from tests.parity import dev_bf16, dev_f32
from tests.test_gpu_block import DevBlock, cfg_of, rope_dev
from tests.test_gpu_mmdit import DevStream, MMDIT_CASES

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Capture fn() (which enqueues on the current stream) into a torch graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _inputs_series(shape, n):
    """n different x (the graph reads x's buffer; each replay gets new contents)."""
    xs = []
    for i in range(n):
        x = DI.draw(7000 + i, (shape.seq_len, shape.dim), 1.0)
        xs.append(x)
    return xs


@pytest.mark.parametrize("shape", [DI.TINY, DI.FLUX], ids=["tiny", "flux"])
def test_block_forward_captured_equals_eager(gpu_lib, shape):
    import torch
    B = gpu_lib
    print(f"capture block {shape.name}", flush=True)
    blk = DevBlock(B, shape, norm_weights="random")
    _, temb = DI.block_activations(shape)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.block_workspace_bytes(cfg))
    ws_e = B.alloc_workspace(B.block_workspace_bytes(cfg))
    x = torch.empty(shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    t = dev_bf16(temb)
    y = torch.empty_like(x)
    xs = _inputs_series(shape, 3)
    x.copy_(dev_bf16(xs[0]))
    g = _capture(lambda: B.block_forward(cfg, blk.dev, x, t, rc, rs, y=y, workspace=ws))
    for i, xv in enumerate(xs):
        x.copy_(dev_bf16(xv))
        g.replay()
        ye = B.block_forward(cfg, blk.dev, x, t, rc, rs, workspace=ws_e)  # eager, other workspace
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all()
        assert torch.equal(y, ye), f"replay {i}"
    del g


@pytest.mark.parametrize("case", [MMDIT_CASES[0], MMDIT_CASES[5]], ids=["mm300", "flux_double"])
def test_mmdit_block_forward_captured_equals_eager(gpu_lib, case):
    import torch
    B = gpu_lib
    shape, n_txt = case
    print(f"capture mmdit block {shape.name} T={n_txt}", flush=True)
    txt, img = DevStream(B, shape, 0), DevStream(B, shape, 1)
    _, temb = DI.block_activations(shape)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.mmdit_block_workspace_bytes(cfg))
    ws_e = B.alloc_workspace(B.mmdit_block_workspace_bytes(cfg))
    x = torch.empty(shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    t = dev_bf16(temb)
    y = torch.empty_like(x)
    xs = _inputs_series(shape, 3)
    x.copy_(dev_bf16(xs[0]))
    g = _capture(lambda: B.mmdit_block_forward(cfg, n_txt, txt.dev, img.dev, x, t, rc, rs, y=y, workspace=ws))
    for i, xv in enumerate(xs):
        x.copy_(dev_bf16(xv))
        g.replay()
        ye = B.mmdit_block_forward(cfg, n_txt, txt.dev, img.dev, x, t, rc, rs, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(y, ye), f"replay {i}"
    del g


def test_modulate_norm_and_gated_residual_captured_equal_eager(gpu_lib):
    import torch
    B = gpu_lib
    ch = DI.chain_inputs(4608, 3072)
    x = dev_bf16(ch["x"])
    h = dev_bf16(ch["h"])
    shift, scale, gate = dev_f32(ch["shift"]), dev_f32(ch["scale"]), dev_f32(ch["gate"])
    u = torch.empty_like(x)
    y = torch.empty_like(x)

    def body():
        B.modulate_norm(x, shift, scale, 1e-6, out=u)
        B.gated_residual(x, h, gate, out=y)

    g = _capture(body)
    for i in range(3):
        x.copy_(dev_bf16(DI.draw(7100 + i, (4608, 3072), 1.0)))
        g.replay()
        ue = B.modulate_norm(x, shift, scale, 1e-6)
        ye = B.gated_residual(x, h, gate)
        torch.cuda.synchronize()
        assert torch.equal(u, ue) and torch.equal(y, ye), f"replay {i}"
    del g


def test_stack_replay_refuses_a_capturing_stream(gpu_lib):
    """dit_stack_replay launches its own graph and stages its inputs, so it
    may not be captured into a caller's graph: on a capturing stream it
    returns DIT_ERR_CAPTURE and enqueues nothing, before its first capture
    and after it."""
    import torch
    B = gpu_lib
    shape = DI.BlockShape("stack_tiny", 3, 256, 256, 4, 64, 1024, (32, 32), (16, 16), 0)
    blocks = [DevBlock(B, shape, block=b) for b in range(2)]
    x, _ = DI.block_activations(shape)
    tembs = np.stack([DI.step_temb(shape, s) for s in range(2)])
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, len(blocks)))
    out = torch.zeros(2, shape.seq_len, shape.dim, dtype=torch.bfloat16, device="cuda")
    xd, td = dev_bf16(x), dev_bf16(tembs)
    st = B.Stack()
    marker = torch.zeros(4, device="cuda")
    codes = []

    def body():
        try:
            st.replay(cfg, [b.dev for b in blocks], xd, td, rc, rs, out, ws)
        except B.DitError as e:
            codes.append(e.code)
        marker.add_(1.0)  # keeps the captured graph non-empty

    g = _capture(body)  # before the stack's own first capture
    del g
    assert codes == [B.DIT_ERR_CAPTURE]
    assert torch.count_nonzero(out).item() == 0
    st.replay(cfg, [b.dev for b in blocks], xd, td, rc, rs, out, ws)  # captures and runs
    torch.cuda.synchronize()
    ref = out.clone()
    out.zero_()
    g = _capture(body)  # after it
    del g
    assert codes == [B.DIT_ERR_CAPTURE, B.DIT_ERR_CAPTURE]
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    st.replay(cfg, [b.dev for b in blocks], xd, td, rc, rs, out, ws)  # still usable
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    st.close()

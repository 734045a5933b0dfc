"""GPU parity of the two-stream (MMDiT) block and of the sequential block
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import dit_inputs as DI
from oracle import dit_oracle as O
from tests import bf16_boundaries as BB
from tests.parity import assert_attributed, assert_parity, dev_bf16, dev_f32, host
from tests.test_gpu_block import cfg_of, rope_dev, sample_rows

pytestmark = pytest.mark.gpu


class DevStream:
    """Seeded weights of one stream on the GPU plus the host copy for the oracle."""

    def __init__(self, B, shape, stream, norm_weights="random", w=None):
        self.w = w if w is not None else DI.stream_weights(shape, stream, norm_weights=norm_weights)
        w = self.w
        self.dev = B.StreamWeights(dev_bf16(w.w_mod), dev_bf16(w.b_mod), dev_bf16(w.w_qkv), dev_bf16(w.b_qkv),
                                   dev_f32(w.q_norm_w), dev_f32(w.k_norm_w), dev_bf16(w.w_o), dev_bf16(w.b_o),
                                   dev_bf16(w.w_fc1), dev_bf16(w.b_fc1), dev_bf16(w.w_fc2), dev_bf16(w.b_fc2))


def _shape(name, S, d, H, Dh, mlp, grid, text, axes):
    return DI.small_shape(seq_len=S, dim=d, num_heads=H, head_dim=Dh, mlp_hidden=mlp, grid=grid,
                          text_tokens=text, axes=axes, name=name)


# (shape, text tokens): several tiles, ragged streams, an empty text or image
# stream, both head dims, the Flux shape at full size and a ragged Flux-width
# case whose q|k|v linear runs on 256x256 tiles (q/k norm in the epilogue)
MMDIT_CASES = [
    (_shape("mm300", 300, 256, 2, 128, 512, (10, 12), 60, (64, 64)), 60),
    (DI.TINY, 37),
    (_shape("mm77_seq", 77, 128, 2, 64, 192, (7, 11), 0, (32, 32)), 0),
    (_shape("mm200_text_only", 200, 256, 2, 128, 512, (10, 10), 200, (64, 64)), 200),
    (_shape("mm_one_token", 1, 256, 4, 64, 256, (1, 1), 0, (32, 32)), 1),
    (DI.FLUX_DOUBLE, 512),
    (_shape("mm_flux_ragged4000", 4000, 3072, 24, 128, 12288, (60, 60), 400, (64, 64)), 400),
]


@pytest.mark.parametrize("shape,n_txt", MMDIT_CASES, ids=[f"{c[0].name}-T{c[1]}" for c in MMDIT_CASES])
def test_mmdit_block_forward(gpu_lib, shape, n_txt):
    import torch
    B = gpu_lib
    print(f"mmdit block {shape.name} S={shape.seq_len} T={n_txt}", flush=True)
    txt = DevStream(B, shape, 0) if n_txt > 0 else None
    img = DevStream(B, shape, 1) if n_txt < shape.seq_len else None
    x, temb = DI.block_activations(shape)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    y = B.mmdit_block_forward(cfg, n_txt, txt.dev if txt else None, img.dev if img else None, dev_bf16(x),
                              dev_bf16(temb), rc, rs)
    torch.cuda.synchronize()
    rows = sample_rows(shape.seq_len, extra=(n_txt - 1, n_txt))
    rows = rows[(rows >= 0) & (rows < shape.seq_len)]
    print(f"  comparing {len(rows)} rows", flush=True)
    ref = O.double_block_forward(shape, txt.w if txt else None, img.w if img else None, x, temb, pos,
                                 n_txt=n_txt, rows=rows)
    mref = BB.double_block_forward_bf16(shape, txt.w if txt else None, img.w if img else None, x, temb, pos,
                                        n_txt=n_txt, rows=rows)
    assert_attributed(host(y)[rows], ref, mref, f"mmdit y {shape.name} T={n_txt}")


SEQ_CASES = [DI.VIDEO, _shape("seq300", 300, 256, 2, 128, 512, (10, 12), 0, (64, 64))]


@pytest.mark.parametrize("shape", SEQ_CASES, ids=[s.name for s in SEQ_CASES])
def test_sequential_block_forward(gpu_lib, shape):
    """The sequential (Wan-style) block at the video shape (S = 16384,
    d = 1536, 12 heads, MLP 8960, 3D RoPE) on sampled rows (the oracle's
    attention over 16384 keys in float64 makes every row too slow for a
    test), and a ragged short case on every row."""
    import torch
    B = gpu_lib
    print(f"sequential block {shape.name} S={shape.seq_len}", flush=True)
    w = DevStream(B, shape, 1)
    x, temb = DI.block_activations(shape)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    y = B.sequential_block_forward(cfg, w.dev, dev_bf16(x), dev_bf16(temb), rc, rs)
    torch.cuda.synchronize()
    rows = sample_rows(shape.seq_len)
    print(f"  comparing {len(rows)} rows", flush=True)
    ref = O.sequential_block_forward(shape, w.w, x, temb, pos, rows=rows)
    mref = BB.double_block_forward_bf16(shape, None, w.w, x, temb, pos, n_txt=0, rows=rows)
    assert_attributed(host(y)[rows], ref, mref, f"sequential y {shape.name}")


def test_mmdit_in_place_deterministic_and_sequential_alias(gpu_lib):
    """In place (y = x) equals out of place bitwise; repeated calls agree;
    the sequential entry point equals the two-stream one with no text."""
    import torch
    B = gpu_lib
    shape = MMDIT_CASES[0][0]
    txt, img = DevStream(B, shape, 0), DevStream(B, shape, 1)
    x, temb = DI.block_activations(shape)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    ws = B.alloc_workspace(B.mmdit_block_workspace_bytes(cfg))
    xt, tt = dev_bf16(x), dev_bf16(temb)
    y1 = B.mmdit_block_forward(cfg, 60, txt.dev, img.dev, xt, tt, rc, rs, workspace=ws)
    y2 = B.mmdit_block_forward(cfg, 60, txt.dev, img.dev, xt, tt, rc, rs, workspace=ws)
    xi = xt.clone()
    B.mmdit_block_forward(cfg, 60, txt.dev, img.dev, xi, tt, rc, rs, y=xi, workspace=ws)
    s1 = B.sequential_block_forward(cfg, img.dev, xt, tt, rc, rs, workspace=ws)
    s2 = B.mmdit_block_forward(cfg, 0, None, img.dev, xt, tt, rc, rs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, xi)
    assert torch.equal(s1, s2)
    assert not torch.equal(s1, y1)


def test_mmdit_halves_match_oracle_halves(gpu_lib):
    """With W_fc2 = 0 and b_fc2 = 0 the block returns x' = x + gate1 * proj(o)
    (its attention half); with W_o = 0 and b_o = 0 it returns its MLP half.
    Each half is compared with the oracle on the same zeroed weights."""
    import torch
    B = gpu_lib
    shape = MMDIT_CASES[0][0]
    x, temb = DI.block_activations(shape)
    pos, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    for kill in (("w_fc2", "b_fc2"), ("w_o", "b_o")):
        ws_ = []
        for s in (0, 1):
            w = DI.stream_weights(shape, s, norm_weights="random")
            f = dict(w.__dict__)
            for k in kill:
                f[k] = 0 * f[k]
            ws_.append(DevStream(B, shape, s, w=DI.StreamWeights(**f)))
        y = B.mmdit_block_forward(cfg, 60, ws_[0].dev, ws_[1].dev, dev_bf16(x), dev_bf16(temb), rc, rs)
        torch.cuda.synchronize()
        ref = O.double_block_forward(shape, ws_[0].w, ws_[1].w, x, temb, pos, n_txt=60)
        assert_parity(host(y), ref, f"mmdit half without {kill[0]}")

"""dit_block_forward_noalloc (for callers that cannot allocate device memory)
against dit_block_forward on the same inputs, through the C ABI: two calls
in a row, the second with a smaller input, plus the size limit of the
built-in scratch array."""
import pytest

import dit_inputs as DI
from tests.parity import assert_parity, dev_bf16, host
from tests.test_gpu_block import DevBlock, cfg_of, rope_dev

pytestmark = pytest.mark.gpu


def _run_both(B, shape, seed_block):
    import torch
    print(f"noalloc vs workspace block forward: {shape.name} S={shape.seq_len} d={shape.dim}", flush=True)
    blk = DevBlock(B, shape, block=seed_block, norm_weights="random")
    x, temb = DI.block_activations(shape)
    _, rc, rs = rope_dev(B, shape)
    cfg = cfg_of(B, shape)
    xd, td = dev_bf16(x), dev_bf16(temb)
    y_ref = B.block_forward(cfg, blk.dev, xd, td, rc, rs)
    y = torch.full_like(xd, float("nan"))
    B.block_forward_noalloc(cfg, blk.dev, xd, td, rc, rs, y)
    torch.cuda.synchronize()
    return y, y_ref


def test_noalloc_matches_workspace_entry_point_twice(gpu_lib):
    """The Flux shape (243 MiB of the 256 MiB array), then the tiny shape in
    the same array: each equals dit_block_forward bitwise (same kernels, same
    order) and so meets the parity bar against it."""
    import torch
    B = gpu_lib
    assert B.block_noalloc_max_bytes() == 256 << 20
    for shape, sb in ((DI.FLUX, 0), (DI.TINY, 1)):
        cfg = cfg_of(B, shape)
        assert B.block_workspace_bytes(cfg) <= B.block_noalloc_max_bytes()
        y, y_ref = _run_both(B, shape, sb)
        assert torch.isfinite(y.float()).all()
        assert_parity(host(y), host(y_ref), f"noalloc vs workspace {shape.name}")
        assert torch.equal(y, y_ref)


def test_noalloc_rejects_configs_beyond_the_array(gpu_lib):
    import torch
    B = gpu_lib
    S, d, H, Dh, mlp = 8192, 3072, 24, 128, 12288
    cfg = B.make_config(S, d, H, Dh, mlp)
    assert B.block_workspace_bytes(cfg) > B.block_noalloc_max_bytes()
    x = torch.zeros(S, d, dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(d, dtype=torch.bfloat16, device="cuda")
    rc = torch.zeros(S, Dh // 2, dtype=torch.float32, device="cuda")
    w = B.BlockWeights(torch.zeros(3 * d, d, dtype=torch.bfloat16, device="cuda"), None,
                       torch.zeros(3 * d + mlp, d, dtype=torch.bfloat16, device="cuda"), None,
                       torch.zeros(d, d + mlp, dtype=torch.bfloat16, device="cuda"), None,
                       torch.ones(Dh, device="cuda"), torch.ones(Dh, device="cuda"))
    y = torch.empty_like(x)
    with pytest.raises(B.DitError) as e:
        B.block_forward_noalloc(cfg, w, x, t, rc, rc, y)
    assert e.value.code == B.DIT_ERR_WORKSPACE
    torch.cuda.synchronize()

"""CPU tests of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments with the documented codes before any HIP
call (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_block.h")
LIB = os.environ.get("DIT_LIB") or os.path.join(ROOT, "diffusion_transformer_dit_amd", "libdit_block.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from diffusion_transformer_dit_amd import build
        build.build()
    from diffusion_transformer_dit_amd import abi as binding
    return binding._lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    from diffusion_transformer_dit_amd import abi as binding
    assert "gfx950" in binding.version()


def cfg(**kw):
    from diffusion_transformer_dit_amd import abi as binding
    base = dict(seq_len=256, dim=256, num_heads=4, head_dim=64, mlp_hidden=1024)
    base.update(kw)
    return binding.make_config(**base)


def test_workspace_bytes(lib):
    from diffusion_transformer_dit_amd import abi as binding
    c = cfg()
    a = lambda n: (n + 255) // 256 * 256
    S, d, mlp = 256, 256, 1024
    want = a(3 * d * 4) + a(S * d * 2) + a(S * 3 * d * 2) + a(S * (d + mlp) * 2)
    assert binding.block_workspace_bytes(c) == want
    # stack: the block scratch, the carried activation, the staged temb, every
    # block's modulation vectors, the W_mod / b_mod pointer table and the probe
    # counters, all inside the caller's workspace
    for n in (1, 57):
        assert binding.stack_workspace_bytes(c, n) == (want + a(S * d * 2) + a(d * 2) + a(n * 3 * d * 4)
                                                       + a(2 * n * 8) + a(n * 7 * 2 * 8))
    assert binding.stack_workspace_bytes(c, 0) == 0
    assert binding.block_workspace_bytes(cfg(head_dim=96, num_heads=3, dim=288)) == 0
    assert binding.block_workspace_bytes(cfg(num_heads=3)) == 0


def test_invalid_arguments_are_rejected_before_hip(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert lib.dit_modulate_norm(None, P, P, P, 4, 8, 1e-6, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_modulate_norm(P, P, P, P, 4, 12, 1e-6, None) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_modulate_norm(P, P, P, P, -1, 8, 1e-6, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_modulate_norm(P, P, P, P, 4, 16384, 1e-6, None) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_gated_residual(P, None, P, P, 4, 8, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_attention(P, P, 64, 3, 96, 288, None) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_attention(P, P, 64, 2, 64, 100, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_linear1_gelu(P, P, None, P, P, 64, 100, 128, None) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_linear2_gated_residual(P, P, None, P, P, P, 64, 128, 96, None) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_modulation(P, P, None, P, 256, 12, None) == B.DIT_ERR_UNSUPPORTED
    dims = (ctypes.c_int32 * 2)(32, 30)
    assert lib.dit_rope_table(P, 16, 2, ctypes.cast(dims, ctypes.c_void_p), 64, 10000.0, P, P, None) \
        == B.DIT_ERR_INVALID_ARG
    assert "sum" in lib.dit_last_error().decode()


def test_misaligned_tensor_pointers_are_rejected(lib):
    from diffusion_transformer_dit_amd import abi as B
    P, Q = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)  # Q: 8-byte aligned only
    assert lib.dit_modulate_norm(Q, P, P, P, 4, 64, 1e-6, None) == B.DIT_ERR_INVALID_ARG
    assert "aligned" in lib.dit_last_error().decode()
    assert lib.dit_gated_residual(P, P, Q, P, 4, 64, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_linear1_gelu(P, P, Q, P, P, 64, 128, 128, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_linear2_gated_residual(P, P, P, P, P, Q, 64, 128, 128, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_attention(P, Q, 64, 2, 64, 128, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_qk_rmsnorm_rope(P, P, P, Q, P, 64, 2, 64, 1e-6, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_modulation(P, Q, None, P, 64, 64, None) == B.DIT_ERR_INVALID_ARG
    c = cfg()
    w = B.BlockWeightsC(0x1000, 0, 0x1008, 0, 0x1000, 0, 0x1000, 0x1000)
    need = B.block_workspace_bytes(c)
    assert lib.dit_block_forward(ctypes.byref(c), ctypes.byref(w), P, P, P, P, P, P, need, None) \
        == B.DIT_ERR_INVALID_ARG


def test_size_limits(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    # q|k|v beyond 4 GiB is supported (a Wan-size video sequence at width 8192 and more)
    ws = B.block_workspace_bytes(B.make_config(90000, 8192, 64, 128, 32768))
    assert ws >= 90000 * 3 * 8192 * 2 > 1 << 32
    # seq_len is capped at 2^24, dim at 8192
    assert lib.dit_attention(P, P, (1 << 24) + 1, 1, 128, 128, None) == B.DIT_ERR_UNSUPPORTED
    assert B.block_workspace_bytes(B.make_config((1 << 24) + 1, 256, 2, 128, 1024)) == 0
    assert lib.dit_attention(P, P, 64, 72, 128, 9216, None) == B.DIT_ERR_UNSUPPORTED


def test_split_attention_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    split = lambda S, n, ld=128, lses=P: lib.dit_attention_split(P, P, S, 1, 128, ld, n, P, lses, None)
    assert split(64, 0) == B.DIT_ERR_INVALID_ARG
    assert split(64, 65) == B.DIT_ERR_INVALID_ARG
    assert split(64, 4, ld=64) == B.DIT_ERR_INVALID_ARG          # ld_out < H*Dh
    assert split(64, 4, lses=ctypes.c_void_p(0x1002)) == B.DIT_ERR_INVALID_ARG
    assert split(64, 4, lses=None) == B.DIT_ERR_INVALID_ARG
    assert split(0, 4) == B.DIT_OK                              # empty: a no-op
    assert lib.dit_attention_split(P, P, 64, 1, 96, 128, 4, P, P, None) == B.DIT_ERR_UNSUPPORTED


def test_chunked_attention_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P, Q = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)
    assert lib.dit_attention_partial(P, 64, 2, 64, 10, 10, P, P, None) == B.DIT_ERR_INVALID_ARG  # empty range
    assert lib.dit_attention_partial(P, 64, 2, 64, 0, 65, P, P, None) == B.DIT_ERR_INVALID_ARG   # past the end
    assert lib.dit_attention_partial(P, 64, 2, 64, 0, 64, Q, P, None) == B.DIT_ERR_INVALID_ARG   # misaligned
    assert lib.dit_attention_partial(P, 64, 3, 96, 0, 64, P, P, None) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_attention_partial(None, 0, 2, 64, 0, 1, None, None, None) == B.DIT_OK         # empty input
    assert lib.dit_attention_merge(P, P, 0, 64, 2, 64, P, 128, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_attention_merge(P, P, 65, 64, 2, 64, P, 128, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_attention_merge(P, P, 2, 64, 2, 64, P, 100, None) == B.DIT_ERR_INVALID_ARG   # ld_out
    assert "ld_out" in lib.dit_last_error().decode()


def test_block_forward_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    c = cfg()
    w = B.BlockWeightsC(0x1000, 0, 0x1000, 0, 0x1000, 0, 0x1000, 0x1000)
    need = B.block_workspace_bytes(c)
    fwd = lambda cc, ww, ws_bytes, ws=P: lib.dit_block_forward(
        ctypes.byref(cc), ctypes.byref(ww), P, P, P, P, P, ws, ws_bytes, None)
    assert fwd(c, w, need - 1) == B.DIT_ERR_WORKSPACE
    assert fwd(c, w, need, None) == B.DIT_ERR_WORKSPACE
    assert fwd(c, w, need, ctypes.c_void_p(0x1010)) == B.DIT_ERR_WORKSPACE  # not 256-aligned
    bad = B.BlockWeightsC(0x1000, 0, 0, 0, 0x1000, 0, 0x1000, 0x1000)
    assert fwd(c, bad, need) == B.DIT_ERR_INVALID_ARG
    assert fwd(cfg(head_dim=32, num_heads=8), w, need) == B.DIT_ERR_UNSUPPORTED
    assert fwd(cfg(ln_eps=-1.0), w, need) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_block_forward(None, ctypes.byref(w), P, P, P, P, P, P, need, None) == B.DIT_ERR_INVALID_ARG


def test_mmdit_block_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    c = cfg()
    a = lambda n: (n + 255) // 256 * 256
    S, d, mlp = 256, 256, 1024
    need = B.mmdit_block_workspace_bytes(c)
    assert need == a(12 * d * 4) + a(S * d * 2) + a(S * 3 * d * 2) + a(S * d * 2) + a(S * d * 4) + a(S * mlp * 2)
    assert B.mmdit_block_workspace_bytes(cfg(num_heads=3)) == 0
    w = B.StreamWeightsC(*([0x1000] * 12))
    fwd = lambda cc, T, wt, wi, ws_bytes, ws=P: lib.dit_mmdit_block_forward(
        ctypes.byref(cc), T, wt, wi, P, P, P, P, P, ws, ws_bytes, None)
    W = ctypes.byref(w)
    assert fwd(c, 16, W, W, need - 1) == B.DIT_ERR_WORKSPACE
    assert fwd(c, 16, W, W, need, ctypes.c_void_p(0x1010)) == B.DIT_ERR_WORKSPACE
    assert fwd(c, -1, W, W, need) == B.DIT_ERR_INVALID_ARG
    assert fwd(c, S + 1, W, W, need) == B.DIT_ERR_INVALID_ARG
    assert fwd(c, 16, None, W, need) == B.DIT_ERR_INVALID_ARG      # text weights needed when txt_len > 0
    assert fwd(c, 0, W, None, need) == B.DIT_ERR_INVALID_ARG       # image weights needed when txt_len < S
    bad = B.StreamWeightsC(*([0x1000] * 6 + [0] + [0x1000] * 5))     # w_o missing
    assert fwd(c, 16, W, ctypes.byref(bad), need) == B.DIT_ERR_INVALID_ARG
    odd = B.StreamWeightsC(*([0x1000] * 11 + [0x1008]))              # b_fc2 not 16-byte aligned
    assert fwd(c, 16, W, ctypes.byref(odd), need) == B.DIT_ERR_INVALID_ARG
    assert fwd(cfg(head_dim=32, num_heads=8), 16, W, W, need) == B.DIT_ERR_UNSUPPORTED
    assert lib.dit_sequential_block_forward(ctypes.byref(c), None, P, P, P, P, P, P, need, None) == \
        B.DIT_ERR_INVALID_ARG
    assert lib.dit_sequential_block_forward(ctypes.byref(c), W, P, P, P, P, P, P, need - 1, None) == \
        B.DIT_ERR_WORKSPACE


def test_stack_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    h = ctypes.c_void_p()
    assert lib.dit_stack_create(ctypes.byref(h)) == B.DIT_OK and h.value
    c = cfg()
    w = (B.BlockWeightsC * 1)(B.BlockWeightsC(0x1000, 0, 0x1000, 0, 0x1000, 0, 0x1000, 0x1000))
    need = B.stack_workspace_bytes(c, 1)
    rep = lambda st, nb, ns, ws_bytes: lib.dit_stack_replay(
        st, ctypes.byref(c), ctypes.cast(w, ctypes.c_void_p), nb, P, P, ns, P, P, P, P, ws_bytes, None)
    assert rep(None, 1, 1, need) == B.DIT_ERR_INVALID_ARG
    assert rep(h, 0, 1, need) == B.DIT_ERR_INVALID_ARG
    assert rep(h, 1, -1, need) == B.DIT_ERR_INVALID_ARG
    assert rep(h, 1, 1, need - 256) == B.DIT_ERR_WORKSPACE
    assert lib.dit_stack_destroy(h) == B.DIT_OK
    assert lib.dit_stack_destroy(None) == B.DIT_OK


def test_stack_cached_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    h = ctypes.c_void_p()
    assert lib.dit_stack_create(ctypes.byref(h)) == B.DIT_OK and h.value
    c = cfg()
    w = (B.BlockWeightsC * 1)(B.BlockWeightsC(0x1000, 0, 0x1000, 0, 0x1000, 0, 0x1000, 0x1000))
    need = B.stack_workspace_bytes(c, 1)

    def rep(fresh, t, ns=3, ws_bytes=need, st=h):
        fr = None if fresh is None else ctypes.cast((ctypes.c_uint8 * len(fresh))(*fresh), ctypes.c_void_p)
        ts = None if t is None else ctypes.cast((ctypes.c_float * len(t))(*t), ctypes.c_void_p)
        return lib.dit_stack_replay_cached(st, ctypes.byref(c), ctypes.cast(w, ctypes.c_void_p), 1, P, P, ns, P, P,
                                           P, P, ws_bytes, fr, ts, None)
    assert rep(None, None) == B.DIT_ERR_INVALID_ARG                      # fresh missing
    assert rep([0, 1, 1], None) == B.DIT_ERR_INVALID_ARG                 # step 0 has no history
    assert rep([1, 0, 1], [1.0, 0.5, 0.5]) == B.DIT_ERR_INVALID_ARG      # not strictly monotonic
    assert rep([1, 0, 1], [0.0, 1.0, 0.5]) == B.DIT_ERR_INVALID_ARG
    assert rep([1, 0, 1], [0.0, float("nan"), 2.0]) == B.DIT_ERR_INVALID_ARG
    assert rep([1, 0, 1], [1.0, 0.5, 0.25], st=None) == B.DIT_ERR_INVALID_ARG
    assert rep([1, 0, 1], None, ws_bytes=need - 256) == B.DIT_ERR_WORKSPACE
    assert lib.dit_stack_destroy(h) == B.DIT_OK


def test_stack_mixed_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P = ctypes.c_void_p(0x1000)
    h = ctypes.c_void_p()
    assert lib.dit_stack_create(ctypes.byref(h)) == B.DIT_OK and h.value
    c = cfg()
    a = lambda n: (n + 255) // 256 * 256
    S, d = 256, 256
    need = B.stack_mixed_workspace_bytes(c, 16, 2, 1)
    # two two-stream blocks with both streams (6d vectors each) and one single-stream block (3d)
    assert need == (max(B.block_workspace_bytes(c), B.mmdit_block_workspace_bytes(c)) + a(S * d * 2) + a(d * 2)
                    + a((2 * 2 * 6 * d + 3 * d) * 4) + a(2 * 5 * 8) + a(7 * 2 * 8))
    # text only or image only: one stream per two-stream block
    assert B.stack_mixed_workspace_bytes(c, 0, 2, 1) < need
    assert B.stack_mixed_workspace_bytes(c, S + 1, 2, 1) == 0
    assert B.stack_mixed_workspace_bytes(c, 16, 0, 0) == 0
    sw = (B.StreamWeightsC * 2)(*([B.StreamWeightsC(*([0x1000] * 12))] * 2))
    bw = (B.BlockWeightsC * 1)(B.BlockWeightsC(0x1000, 0, 0x1000, 0, 0x1000, 0, 0x1000, 0x1000))
    V = lambda arr: ctypes.cast(arr, ctypes.c_void_p)

    def rep(T, txt, img, nd, singles, ns, ws_bytes=need):
        return lib.dit_stack_replay_mixed(h, ctypes.byref(c), T, txt, img, nd, singles, ns, P, P, 1, P, P, P, P,
                                          ws_bytes, None, None, None)
    assert rep(16, V(sw), V(sw), 0, None, 0) == B.DIT_ERR_INVALID_ARG        # no blocks
    assert rep(16, V(sw), V(sw), -1, V(bw), 1) == B.DIT_ERR_INVALID_ARG
    assert rep(16, None, V(sw), 2, V(bw), 1) == B.DIT_ERR_INVALID_ARG        # text weights needed
    assert rep(0, None, None, 2, V(bw), 1) == B.DIT_ERR_INVALID_ARG          # image weights needed
    assert rep(S + 1, V(sw), V(sw), 2, V(bw), 1) == B.DIT_ERR_INVALID_ARG
    assert rep(16, V(sw), V(sw), 2, None, 1) == B.DIT_ERR_INVALID_ARG        # singles NULL with n_single 1
    assert rep(16, V(sw), V(sw), 2, V(bw), 1, need - 256) == B.DIT_ERR_WORKSPACE
    # a mixed stack needs more than the single-stream stack's workspace
    assert rep(16, V(sw), V(sw), 2, V(bw), 1, B.stack_workspace_bytes(c, 3)) == B.DIT_ERR_WORKSPACE
    assert lib.dit_stack_destroy(h) == B.DIT_OK


def test_stack_probe_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    h = ctypes.c_void_p()
    assert lib.dit_stack_create(ctypes.byref(h)) == B.DIT_OK
    assert lib.dit_stack_set_probe(None, 1) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_stack_set_probe(h, 1 << 6) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_stack_set_probe(h, 0x3F) == B.DIT_OK
    buf = (ctypes.c_float * 6)()
    # no probed replay has run yet
    assert lib.dit_stack_probe_ms(h, ctypes.cast(buf, ctypes.c_void_p), 1) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_stack_destroy(h) == B.DIT_OK


def test_binding_declares_every_header_function(lib):
    from diffusion_transformer_dit_amd import abi as binding
    assert sorted(binding.SIGNATURES) == declared_functions()


def test_probe_and_graph_info_argument_checks(lib):
    from diffusion_transformer_dit_amd import abi as B
    P, Q = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x100000)
    assert lib.dit_probe_copy(P, Q, 0, None) == B.DIT_OK                     # nothing to copy
    assert lib.dit_probe_copy(None, Q, 64, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_probe_copy(P, Q, 24, None) == B.DIT_ERR_INVALID_ARG       # not a multiple of 16
    assert lib.dit_probe_copy(ctypes.c_void_p(0x1008), Q, 64, None) == B.DIT_ERR_INVALID_ARG  # misaligned
    assert lib.dit_probe_copy(P, ctypes.c_void_p(0x1010), 64, None) == B.DIT_ERR_INVALID_ARG  # overlap
    assert lib.dit_probe_mfma(None, 1, 1, 0, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_probe_mfma(P, 0, 1, 0, None) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_probe_mfma(P, 1, 0, 1, None) == B.DIT_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.dit_stack_create(ctypes.byref(h)) == B.DIT_OK
    k, n = ctypes.c_int(), ctypes.c_int()
    assert lib.dit_stack_graph_info(h, ctypes.byref(k), ctypes.byref(n)) == B.DIT_ERR_INVALID_ARG  # not captured
    assert lib.dit_stack_graph_info(None, ctypes.byref(k), ctypes.byref(n)) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_stack_destroy(h) == B.DIT_OK

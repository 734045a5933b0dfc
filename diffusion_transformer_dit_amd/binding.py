"""Thin ctypes binding of libdit_block (argument marshalling only).

Every function takes torch tensors that live on the GPU, checks dtype /
shape / contiguity, and passes raw pointers and the current HIP stream to the
C ABI declared in include/dit_block.h.  All arithmetic happens in the HIP
kernels; if the shared library is missing this module raises at import.
"""
from __future__ import annotations

import ctypes

import torch

from .abi import (DIT_ERR_CAPTURE, DIT_ERR_GRAPH_KEY, DIT_ERR_HIP, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED,  # noqa: F401
                  DIT_ERR_WORKSPACE, DIT_OK, DIT_STACK_CHAIN, ERROR_NAMES, F32, I32, I64, LIB_PATH, SIGNATURES, SZ,
                  VP, BlockConfig, BlockWeightsC, DitError, StreamWeightsC, _lib, block_noalloc_max_bytes,
                  block_workspace_bytes, load_library, make_config, mmdit_block_workspace_bytes,
                  stack_mixed_workspace_bytes, stack_workspace_bytes, version)
from .abi import check as _check

def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


BF16, F32T, I32T = torch.bfloat16, torch.float32, torch.int32


# --------------------------------------------------------------------- steps
def modulation(temb, w_mod, b_mod=None, out=None, stream=None):
    """mod = W_mod . SiLU(temb) + b_mod (fp32 [3d], shift | scale | gate)."""
    _need(temb, BF16, "temb", 1)
    _need(w_mod, BF16, "w_mod", 2)
    if b_mod is not None:
        _need(b_mod, BF16, "b_mod", 1)
    three_d, tdim = w_mod.shape
    if temb.numel() != tdim or three_d % 3:
        raise ValueError("shape mismatch between temb and w_mod")
    out = torch.empty(three_d, dtype=F32T, device=temb.device) if out is None else out
    _need(out, F32T, "out", 1)
    _check(_lib.dit_modulation(_p(temb), _p(w_mod), _p(b_mod), _p(out), three_d // 3, tdim, _stream(stream)))
    return out


def modulate_norm(x, shift, scale, eps=1e-6, out=None, stream=None):
    """out = LN(x) * (1 + scale) + shift, one pass."""
    _need(x, BF16, "x", 2)
    _need(shift, F32T, "shift", 1)
    _need(scale, F32T, "scale", 1)
    rows, cols = x.shape
    if shift.numel() != cols or scale.numel() != cols:
        raise ValueError("shift/scale length must equal x.shape[1]")
    out = torch.empty_like(x) if out is None else out
    _need(out, BF16, "out", 2)
    _check(_lib.dit_modulate_norm(_p(x), _p(shift), _p(scale), _p(out), rows, cols, eps, _stream(stream)))
    return out


def gated_residual(x, h, gate, out=None, stream=None):
    """y = x + gate * h."""
    _need(x, BF16, "x", 2)
    _need(h, BF16, "h", 2)
    _need(gate, F32T, "gate", 1)
    if h.shape != x.shape or gate.numel() != x.shape[1]:
        raise ValueError("shape mismatch")
    out = torch.empty_like(x) if out is None else out
    _need(out, BF16, "out", 2)
    _check(_lib.dit_gated_residual(_p(x), _p(h), _p(gate), _p(out), x.shape[0], x.shape[1], _stream(stream)))
    return out


def linear1_gelu(u, w1, b1, qkv, cat, mlp_hidden, stream=None):
    """qkv <- (u W1^T + b1)[:, :3d]; cat[:, d:] <- GELU_tanh((u W1^T + b1)[:, 3d:])."""
    _need(u, BF16, "u", 2)
    _need(w1, BF16, "w1", 2)
    _need(qkv, BF16, "qkv", 2)
    _need(cat, BF16, "cat", 2)
    if b1 is not None:
        _need(b1, BF16, "b1", 1)
    S, d = u.shape
    if w1.shape != (3 * d + mlp_hidden, d) or qkv.shape != (S, 3 * d) or cat.shape != (S, d + mlp_hidden):
        raise ValueError("shape mismatch")
    _check(_lib.dit_linear1_gelu(_p(u), _p(w1), _p(b1), _p(qkv), _p(cat), S, d, mlp_hidden, _stream(stream)))


def qk_rmsnorm_rope(qkv, q_norm_w, k_norm_w, rope_cos, rope_sin, num_heads, head_dim, eps=1e-6, stream=None):
    """In place on the q and k blocks of qkv: per-head RMSNorm, then RoPE."""
    _need(qkv, BF16, "qkv", 2)
    for t, n in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"), (rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _need(t, F32T, n)
    S = qkv.shape[0]
    if qkv.shape[1] != 3 * num_heads * head_dim or rope_cos.shape != (S, head_dim // 2) \
            or rope_sin.shape != (S, head_dim // 2) or q_norm_w.numel() != head_dim or k_norm_w.numel() != head_dim:
        raise ValueError("shape mismatch")
    _check(_lib.dit_qk_rmsnorm_rope(_p(qkv), _p(q_norm_w), _p(k_norm_w), _p(rope_cos), _p(rope_sin),
                                    S, num_heads, head_dim, eps, _stream(stream)))


def attention(qkv, out, num_heads, head_dim, stream=None):
    """out[:, :H*Dh] <- softmax(q k^T / sqrt(Dh)) v per head; q, k, v from qkv."""
    _need(qkv, BF16, "qkv", 2)
    _need(out, BF16, "out", 2)
    S = qkv.shape[0]
    if qkv.shape[1] != 3 * num_heads * head_dim or out.shape[0] != S:
        raise ValueError("shape mismatch")
    _check(_lib.dit_attention(_p(qkv), _p(out), S, num_heads, head_dim, out.shape[1], _stream(stream)))
    return out


def attention_partial(qkv, num_heads, head_dim, kv_begin, kv_end, o_part=None, lse=None, stream=None):
    """(o_part [S, H*Dh] fp32, lse [H, S] fp32): attention of every query over keys [kv_begin, kv_end)."""
    _need(qkv, BF16, "qkv", 2)
    S = qkv.shape[0]
    d = num_heads * head_dim
    if qkv.shape[1] != 3 * d:
        raise ValueError("shape mismatch")
    o_part = torch.empty(S, d, dtype=F32T, device=qkv.device) if o_part is None else o_part
    lse = torch.empty(num_heads, S, dtype=F32T, device=qkv.device) if lse is None else lse
    _need(o_part, F32T, "o_part", 2)
    _need(lse, F32T, "lse", 2)
    if o_part.shape != (S, d) or lse.shape != (num_heads, S):
        raise ValueError("output shape mismatch")
    _check(_lib.dit_attention_partial(_p(qkv), S, num_heads, head_dim, kv_begin, kv_end, _p(o_part), _p(lse),
                                      _stream(stream)))
    return o_part, lse


def attention_merge(o_parts, lses, out, num_heads, head_dim, stream=None):
    """out[:, :H*Dh] <- lse-weighted merge of o_parts [C, S, H*Dh] fp32 with lses [C, H, S] fp32."""
    _need(o_parts, F32T, "o_parts", 3)
    _need(lses, F32T, "lses", 3)
    _need(out, BF16, "out", 2)
    C, S, d = o_parts.shape
    if d != num_heads * head_dim or lses.shape != (C, num_heads, S) or out.shape[0] != S:
        raise ValueError("shape mismatch")
    _check(_lib.dit_attention_merge(_p(o_parts), _p(lses), C, S, num_heads, head_dim, _p(out), out.shape[1],
                                    _stream(stream)))
    return out


def attention_split(qkv, out, num_heads, head_dim, n_chunks, o_parts=None, lses=None, stream=None):
    """Attention over all keys, split into up to n_chunks key chunks (one
    launch of partials + the merge); out columns [0, H*Dh)."""
    _need(qkv, BF16, "qkv", 2)
    _need(out, BF16, "out", 2)
    S = qkv.shape[0]
    d = num_heads * head_dim
    if qkv.shape[1] != 3 * d or out.shape[0] != S or out.shape[1] < d:
        raise ValueError("qkv must be [S, 3*H*Dh], out [S, >= H*Dh]")
    if o_parts is None:
        o_parts = torch.empty(n_chunks, S, d, dtype=F32T, device=qkv.device)
    if lses is None:
        lses = torch.empty(n_chunks, num_heads, S, dtype=F32T, device=qkv.device)
    _need(o_parts, F32T, "o_parts", 3)
    _need(lses, F32T, "lses", 3)
    if o_parts.shape[0] < n_chunks or lses.shape[0] < n_chunks:
        raise ValueError("scratch too small for n_chunks")
    _check(_lib.dit_attention_split(_p(qkv), _p(out), S, num_heads, head_dim, out.stride(0), n_chunks, _p(o_parts),
                                    _p(lses), _stream(stream)))
    return out


def linear2_gated_residual(cat, w2, b2, x, gate, y, stream=None):
    """y <- x + gate * (cat W2^T + b2)."""
    for t, n in ((cat, "cat"), (w2, "w2"), (x, "x"), (y, "y")):
        _need(t, BF16, n, 2)
    _need(gate, F32T, "gate", 1)
    if b2 is not None:
        _need(b2, BF16, "b2", 1)
    S, n2 = cat.shape
    d = x.shape[1]
    if w2.shape != (d, n2) or x.shape != (S, d) or y.shape != (S, d) or gate.numel() != d:
        raise ValueError("shape mismatch")
    _check(_lib.dit_linear2_gated_residual(_p(cat), _p(w2), _p(b2), _p(x), _p(gate), _p(y),
                                           S, d, n2 - d, _stream(stream)))
    return y


def rope_table(positions, axes_dims, head_dim, base=10000.0, stream=None):
    """cos/sin [S, head_dim/2] fp32 from integer positions [S, n_axes] (int32, on the GPU)."""
    _need(positions, I32T, "positions", 2)
    S, n_axes = positions.shape
    dims = (ctypes.c_int32 * len(axes_dims))(*axes_dims)
    if len(axes_dims) != n_axes:
        raise ValueError("one axis dim per position column")
    c = torch.empty(S, head_dim // 2, dtype=F32T, device=positions.device)
    s = torch.empty_like(c)
    _check(_lib.dit_rope_table(_p(positions), S, n_axes, ctypes.cast(dims, VP), head_dim, base,
                               _p(c), _p(s), _stream(stream)))
    return c, s


# --------------------------------------------------------------------- block
class BlockWeights:
    """Device weights of one block (holds the tensors alive) and their C view."""

    def __init__(self, w_mod, b_mod, w1, b1, w2, b2, q_norm_w, k_norm_w):
        for t, n in ((w_mod, "w_mod"), (w1, "w1"), (w2, "w2")):
            _need(t, BF16, n, 2)
        for t, n in ((b_mod, "b_mod"), (b1, "b1"), (b2, "b2")):
            if t is not None:
                _need(t, BF16, n, 1)
        _need(q_norm_w, F32T, "q_norm_w", 1)
        _need(k_norm_w, F32T, "k_norm_w", 1)
        self.tensors = (w_mod, b_mod, w1, b1, w2, b2, q_norm_w, k_norm_w)
        self.c = BlockWeightsC(*[None if t is None else t.data_ptr() for t in self.tensors])


class StreamWeights:
    """Device weights of one stream of a two-stream (or sequential) block."""

    def __init__(self, w_mod, b_mod, w_qkv, b_qkv, q_norm_w, k_norm_w, w_o, b_o, w_fc1, b_fc1, w_fc2, b_fc2):
        for t, n in ((w_mod, "w_mod"), (w_qkv, "w_qkv"), (w_o, "w_o"), (w_fc1, "w_fc1"), (w_fc2, "w_fc2")):
            _need(t, BF16, n, 2)
        for t, n in ((b_mod, "b_mod"), (b_qkv, "b_qkv"), (b_o, "b_o"), (b_fc1, "b_fc1"), (b_fc2, "b_fc2")):
            if t is not None:
                _need(t, BF16, n, 1)
        _need(q_norm_w, F32T, "q_norm_w", 1)
        _need(k_norm_w, F32T, "k_norm_w", 1)
        self.tensors = (w_mod, b_mod, w_qkv, b_qkv, q_norm_w, k_norm_w, w_o, b_o, w_fc1, b_fc1, w_fc2, b_fc2)
        self.c = StreamWeightsC(*[None if t is None else t.data_ptr() for t in self.tensors])


def mmdit_block_forward(cfg, txt_len, txt: "StreamWeights | None", img: StreamWeights, x, temb, rope_cos,
                        rope_sin, y=None, workspace=None, stream=None):
    """One two-stream block forward: rows [0, txt_len) of x are the text
    tokens, the rest the image tokens; y may be x (in place)."""
    _need(x, BF16, "x", 2)
    _need(temb, BF16, "temb", 1)
    _need(rope_cos, F32T, "rope_cos", 2)
    _need(rope_sin, F32T, "rope_sin", 2)
    y = torch.empty_like(x) if y is None else y
    _need(y, BF16, "y", 2)
    if x.shape != (cfg.seq_len, cfg.dim) or y.shape != x.shape:
        raise ValueError("x / y shape does not match the config")
    if workspace is None:
        workspace = alloc_workspace(mmdit_block_workspace_bytes(cfg), x.device)
    _check(_lib.dit_mmdit_block_forward(ctypes.byref(cfg), int(txt_len),
                                        None if txt is None else ctypes.byref(txt.c),
                                        None if img is None else ctypes.byref(img.c), _p(x), _p(temb),
                                        _p(rope_cos), _p(rope_sin), _p(y), _p(workspace), workspace.numel(),
                                        _stream(stream)))
    return y


def sequential_block_forward(cfg, w: StreamWeights, x, temb, rope_cos, rope_sin, y=None, workspace=None,
                             stream=None):
    """One sequential (single-stream-sequence, Wan-style) block forward."""
    _need(x, BF16, "x", 2)
    _need(temb, BF16, "temb", 1)
    _need(rope_cos, F32T, "rope_cos", 2)
    _need(rope_sin, F32T, "rope_sin", 2)
    y = torch.empty_like(x) if y is None else y
    _need(y, BF16, "y", 2)
    if x.shape != (cfg.seq_len, cfg.dim) or y.shape != x.shape:
        raise ValueError("x / y shape does not match the config")
    if workspace is None:
        workspace = alloc_workspace(mmdit_block_workspace_bytes(cfg), x.device)
    _check(_lib.dit_sequential_block_forward(ctypes.byref(cfg), ctypes.byref(w.c), _p(x), _p(temb), _p(rope_cos),
                                             _p(rope_sin), _p(y), _p(workspace), workspace.numel(),
                                             _stream(stream)))
    return y


def alloc_workspace(nbytes: int, device="cuda"):
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def block_forward(cfg, weights: BlockWeights, x, temb, rope_cos, rope_sin, y=None, workspace=None, stream=None):
    """One block forward on the current stream; y may be x (in place)."""
    _need(x, BF16, "x", 2)
    _need(temb, BF16, "temb", 1)
    _need(rope_cos, F32T, "rope_cos", 2)
    _need(rope_sin, F32T, "rope_sin", 2)
    y = torch.empty_like(x) if y is None else y
    _need(y, BF16, "y", 2)
    if x.shape != (cfg.seq_len, cfg.dim) or y.shape != x.shape:
        raise ValueError("x / y shape does not match the config")
    if workspace is None:
        workspace = alloc_workspace(block_workspace_bytes(cfg), x.device)
    _check(_lib.dit_block_forward(ctypes.byref(cfg), ctypes.byref(weights.c), _p(x), _p(temb), _p(rope_cos),
                                  _p(rope_sin), _p(y), _p(workspace), workspace.numel(), _stream(stream)))
    return y


def probe_copy(src, dst, stream=None):
    """Ceiling probe: streaming copy of src into dst (same byte size, disjoint)."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous GPU tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(_lib.dit_probe_copy(_p(src), _p(dst), nbytes, _stream(stream)))
    return dst


def probe_mfma(out, n_workgroups, iters, vary_operands, stream=None):
    """Ceiling probe: n_workgroups x 4 waves x iters x 4 bf16 MFMAs of 32768 flop."""
    _need(out, F32T, "out", 1)
    if out.numel() < n_workgroups * 256:
        raise ValueError("out needs n_workgroups * 256 floats")
    _check(_lib.dit_probe_mfma(_p(out), n_workgroups, iters, 1 if vary_operands else 0, _stream(stream)))
    return out


def block_forward_noalloc(cfg, weights: BlockWeights, x, temb, rope_cos, rope_sin, y, stream=None):
    """block_forward with the library's built-in per-GPU scratch instead of a
    workspace (no allocation anywhere; y must be given)."""
    _need(x, BF16, "x", 2)
    _need(temb, BF16, "temb", 1)
    _need(rope_cos, F32T, "rope_cos", 2)
    _need(rope_sin, F32T, "rope_sin", 2)
    _need(y, BF16, "y", 2)
    if x.shape != (cfg.seq_len, cfg.dim) or y.shape != x.shape:
        raise ValueError("x / y shape does not match the config")
    _check(_lib.dit_block_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights.c), _p(x), _p(temb),
                                          _p(rope_cos), _p(rope_sin), _p(y), _stream(stream)))
    return y


class Stack:
    """A block stack captured once as a hipGraph and replayed per denoising step."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(_lib.dit_stack_create(ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _lib.dit_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    KERNELS = ("modulation", "modulate_norm", "linear1", "qk_rmsnorm_rope", "attention", "linear2")

    def set_probe(self, kernels):
        """Time the named block kernels inside every replay (before the first replay)."""
        mask = 0
        for k in kernels:
            mask |= 1 << self.KERNELS.index(k)
        _check(_lib.dit_stack_set_probe(self.handle, mask))
        self._probe = tuple(kernels)

    def graph_info(self):
        """(kernel nodes, all nodes) of the captured graph."""
        k, n = ctypes.c_int(), ctypes.c_int()
        _check(_lib.dit_stack_graph_info(self.handle, ctypes.byref(k), ctypes.byref(n)))
        return k.value, n.value

    def probe_ms(self, n_blocks):
        """{kernel: [mean ms per block]} over the probed steps since the previous
        read (synchronises the device; restarts the accumulation)."""
        buf = (ctypes.c_float * (n_blocks * 6))()
        _check(_lib.dit_stack_probe_ms(self.handle, ctypes.cast(buf, VP), n_blocks))
        return {k: [buf[b * 6 + self.KERNELS.index(k)] for b in range(n_blocks)] for k in self._probe}

    def replay(self, cfg, blocks, x_in, temb_steps, rope_cos, rope_sin, out, workspace, stream=None):
        _need(x_in, BF16, "x_in", 2)
        _need(temb_steps, BF16, "temb_steps", 2)
        _need(out, BF16, "out", 3)
        _need(workspace, torch.uint8, "workspace", 1)
        n_steps = temb_steps.shape[0]
        if out.shape != (n_steps, cfg.seq_len, cfg.dim):
            raise ValueError("out must be [n_steps, S, d]")
        arr = (BlockWeightsC * len(blocks))(*[b.c for b in blocks])
        self._keep = (blocks, arr)
        _check(_lib.dit_stack_replay(self.handle, ctypes.byref(cfg), ctypes.cast(arr, VP), len(blocks), _p(x_in),
                                     _p(temb_steps), n_steps, _p(rope_cos), _p(rope_sin), _p(out), _p(workspace),
                                     workspace.numel(), _stream(stream)))
        return out

    def replay_cached(self, cfg, blocks, x_in, temb_steps, rope_cos, rope_sin, out, workspace, fresh,
                      t_steps=None, stream=None):
        """Replay only the steps with fresh[s] true; a skipped step's output is
        the finite-difference prediction from the last two computed outputs
        (see dit_stack_replay_cached).  fresh: sequence of n_steps bools;
        t_steps: n_steps floats (strictly monotonic) or None for t_s = s."""
        _need(x_in, BF16, "x_in", 2)
        _need(temb_steps, BF16, "temb_steps", 2)
        _need(out, BF16, "out", 3)
        _need(workspace, torch.uint8, "workspace", 1)
        n_steps = temb_steps.shape[0]
        if out.shape != (n_steps, cfg.seq_len, cfg.dim):
            raise ValueError("out must be [n_steps, S, d]")
        if len(fresh) != n_steps or (t_steps is not None and len(t_steps) != n_steps):
            raise ValueError("fresh / t_steps must have one entry per step")
        fr = (ctypes.c_uint8 * max(n_steps, 1))(*[1 if f else 0 for f in fresh])
        ts = None if t_steps is None else (ctypes.c_float * max(n_steps, 1))(*[float(t) for t in t_steps])
        arr = (BlockWeightsC * len(blocks))(*[b.c for b in blocks])
        self._keep = (blocks, arr)
        _check(_lib.dit_stack_replay_cached(self.handle, ctypes.byref(cfg), ctypes.cast(arr, VP), len(blocks),
                                            _p(x_in), _p(temb_steps), n_steps, _p(rope_cos), _p(rope_sin), _p(out),
                                            _p(workspace), workspace.numel(), ctypes.cast(fr, VP),
                                            None if ts is None else ctypes.cast(ts, VP), _stream(stream)))
        return out

    def replay_mixed(self, cfg, txt_len, doubles, singles, x_in, temb_steps, rope_cos, rope_sin, out, workspace,
                     fresh=None, t_steps=None, stream=None):
        """A Flux-style stack: the two-stream blocks ``doubles`` (a list of
        (text StreamWeights or None, image StreamWeights or None)) then the
        single-stream blocks ``singles``; steps as in replay_cached (fresh
        None = every step computed)."""
        _need(x_in, BF16, "x_in", 2)
        _need(temb_steps, BF16, "temb_steps", 2)
        _need(out, BF16, "out", 3)
        _need(workspace, torch.uint8, "workspace", 1)
        n_steps = temb_steps.shape[0]
        if out.shape != (n_steps, cfg.seq_len, cfg.dim):
            raise ValueError("out must be [n_steps, S, d]")
        nd, ns = len(doubles), len(singles)
        empty = StreamWeightsC()
        txt = (StreamWeightsC * max(nd, 1))(*[(t.c if t is not None else empty) for t, _ in doubles])
        img = (StreamWeightsC * max(nd, 1))(*[(i.c if i is not None else empty) for _, i in doubles])
        sg = (BlockWeightsC * max(ns, 1))(*[b.c for b in singles])
        fr = None if fresh is None else (ctypes.c_uint8 * max(n_steps, 1))(*[1 if f else 0 for f in fresh])
        ts = None if t_steps is None else (ctypes.c_float * max(n_steps, 1))(*[float(t) for t in t_steps])
        if (fresh is not None and len(fresh) != n_steps) or (t_steps is not None and len(t_steps) != n_steps):
            raise ValueError("fresh / t_steps must have one entry per step")
        self._keep = (doubles, singles, txt, img, sg)
        no_txt = nd == 0 or all(t is None for t, _ in doubles)
        no_img = nd == 0 or all(i is None for _, i in doubles)
        _check(_lib.dit_stack_replay_mixed(self.handle, ctypes.byref(cfg), int(txt_len),
                                           None if no_txt else ctypes.cast(txt, VP),
                                           None if no_img else ctypes.cast(img, VP), nd,
                                           None if ns == 0 else ctypes.cast(sg, VP), ns, _p(x_in), _p(temb_steps),
                                           n_steps, _p(rope_cos), _p(rope_sin), _p(out), _p(workspace),
                                           workspace.numel(), None if fr is None else ctypes.cast(fr, VP),
                                           None if ts is None else ctypes.cast(ts, VP), _stream(stream)))
        return out


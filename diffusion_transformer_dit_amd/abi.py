"""ctypes declarations of libdit_block's C ABI (include/dit_block.h): status
codes, the config and weight structs, every entry point's signature and the
loader.  No torch here: the ABI checks in tests/test_abi.py use this module
alone (also against a build with host sanitizers), and binding.py builds
its tensor-level wrappers on it.

The library is diffusion_transformer_dit_amd/libdit_block.so, or the file
named by the DIT_LIB environment variable; loading fails loudly when it is
missing (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DIT_LIB") or os.path.join(_HERE, "libdit_block.so")

DIT_OK, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE, DIT_ERR_HIP, \
    DIT_ERR_CAPTURE, DIT_ERR_GRAPH_KEY = range(7)
DIT_STACK_CHAIN = 1

ERROR_NAMES = {1: "DIT_ERR_INVALID_ARG", 2: "DIT_ERR_UNSUPPORTED", 3: "DIT_ERR_WORKSPACE",
               4: "DIT_ERR_HIP", 5: "DIT_ERR_CAPTURE", 6: "DIT_ERR_GRAPH_KEY"}


class DitError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class BlockConfig(ctypes.Structure):
    _fields_ = [("seq_len", ctypes.c_int32), ("dim", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("mlp_hidden", ctypes.c_int32), ("temb_dim", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("qk_eps", ctypes.c_float), ("flags", ctypes.c_uint32)]


class BlockWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_mod", "b_mod", "w1", "b1", "w2", "b2", "q_norm_w", "k_norm_w")]


STREAM_FIELDS = ("w_mod", "b_mod", "w_qkv", "b_qkv", "q_norm_w", "k_norm_w", "w_o", "b_o",
                 "w_fc1", "b_fc1", "w_fc2", "b_fc2")


class StreamWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in STREAM_FIELDS]


VP, I64, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "dit_modulation": ([VP, VP, VP, VP, I64, I64, VP], ctypes.c_int),
    "dit_modulate_norm": ([VP, VP, VP, VP, I64, I64, F32, VP], ctypes.c_int),
    "dit_gated_residual": ([VP, VP, VP, VP, I64, I64, VP], ctypes.c_int),
    "dit_linear1_gelu": ([VP, VP, VP, VP, VP, I64, I64, I64, VP], ctypes.c_int),
    "dit_qk_rmsnorm_rope": ([VP, VP, VP, VP, VP, I64, I64, I64, F32, VP], ctypes.c_int),
    "dit_attention": ([VP, VP, I64, I64, I64, I64, VP], ctypes.c_int),
    "dit_linear2_gated_residual": ([VP, VP, VP, VP, VP, VP, I64, I64, I64, VP], ctypes.c_int),
    "dit_rope_table": ([VP, I64, I32, VP, I64, F32, VP, VP, VP], ctypes.c_int),
    "dit_block_workspace_bytes": ([VP], SZ),
    "dit_block_forward": ([VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP], ctypes.c_int),
    "dit_block_noalloc_max_bytes": ([], SZ),
    "dit_block_forward_noalloc": ([VP, VP, VP, VP, VP, VP, VP, VP], ctypes.c_int),
    "dit_mmdit_block_workspace_bytes": ([VP], SZ),
    "dit_mmdit_block_forward": ([VP, I64, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP], ctypes.c_int),
    "dit_sequential_block_forward": ([VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP], ctypes.c_int),
    "dit_stack_create": ([VP], ctypes.c_int),
    "dit_stack_destroy": ([VP], ctypes.c_int),
    "dit_stack_workspace_bytes": ([VP, ctypes.c_int], SZ),
    "dit_stack_replay": ([VP, VP, VP, ctypes.c_int, VP, VP, ctypes.c_int, VP, VP, VP, VP, SZ, VP], ctypes.c_int),
    "dit_attention_partial": ([VP, I64, I64, I64, I64, I64, VP, VP, VP], ctypes.c_int),
    "dit_attention_merge": ([VP, VP, I64, I64, I64, I64, VP, I64, VP], ctypes.c_int),
    "dit_attention_split": ([VP, VP, I64, I64, I64, I64, I64, VP, VP, VP], ctypes.c_int),
    "dit_stack_replay_cached": ([VP, VP, VP, ctypes.c_int, VP, VP, ctypes.c_int, VP, VP, VP, VP, SZ, VP, VP, VP],
                                ctypes.c_int),
    "dit_stack_mixed_workspace_bytes": ([VP, I64, ctypes.c_int, ctypes.c_int], SZ),
    "dit_stack_replay_mixed": ([VP, VP, I64, VP, VP, ctypes.c_int, VP, ctypes.c_int, VP, VP, ctypes.c_int, VP, VP,
                                VP, VP, SZ, VP, VP, VP], ctypes.c_int),
    "dit_stack_set_probe": ([VP, ctypes.c_uint32], ctypes.c_int),
    "dit_stack_probe_ms": ([VP, VP, ctypes.c_int], ctypes.c_int),
    "dit_stack_graph_info": ([VP, VP, VP], ctypes.c_int),
    "dit_probe_copy": ([VP, VP, SZ, VP], ctypes.c_int),
    "dit_probe_mfma": ([VP, I64, I64, I32, VP], ctypes.c_int),
    "dit_last_error": ([], ctypes.c_char_p),
    "dit_version": ([], ctypes.c_char_p),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m diffusion_transformer_dit_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = load_library()


def check(rc: int):
    if rc != DIT_OK:
        raise DitError(rc, _lib.dit_last_error().decode())


def version() -> str:
    return _lib.dit_version().decode()


def make_config(seq_len, dim, num_heads, head_dim, mlp_hidden, temb_dim=0, ln_eps=1e-6, qk_eps=1e-6, flags=0):
    return BlockConfig(seq_len, dim, num_heads, head_dim, mlp_hidden, temb_dim, ln_eps, qk_eps, flags)


def block_workspace_bytes(cfg: BlockConfig) -> int:
    return int(_lib.dit_block_workspace_bytes(ctypes.byref(cfg)))


def mmdit_block_workspace_bytes(cfg: BlockConfig) -> int:
    return int(_lib.dit_mmdit_block_workspace_bytes(ctypes.byref(cfg)))


def stack_workspace_bytes(cfg: BlockConfig, n_blocks: int) -> int:
    return int(_lib.dit_stack_workspace_bytes(ctypes.byref(cfg), int(n_blocks)))


def stack_mixed_workspace_bytes(cfg: BlockConfig, txt_len: int, n_double: int, n_single: int) -> int:
    return int(_lib.dit_stack_mixed_workspace_bytes(ctypes.byref(cfg), int(txt_len), int(n_double),
                                                    int(n_single)))


def block_noalloc_max_bytes() -> int:
    return int(_lib.dit_block_noalloc_max_bytes())

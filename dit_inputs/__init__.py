"""Seeded synthetic inputs for the Flux-style DiT blocks (single-stream,
two-stream and sequential).

This module is shared by the CPU oracle and by the GPU tests / bench.  It
holds no arithmetic of the block itself: only the workload shapes, the
seeded normal draws (rounded to bfloat16 so that bf16 and fp32 storage hold
the same numbers), and the integer token positions that feed the rotary
embedding.

Workload shapes follow the page "ChituDiffusion compile_graph" (chenyy20.com),
section 2 (one Flux single-stream block: S=4608, dim 3072, 24 heads x 128,
bf16), and the workload list of this project (tiny block, memory-bound chain,
Flux block, 57-block x 50-step replay, long-sequence video block, and the
two-stream block at the Flux shape with 512 text tokens).

Seeding recipe: ``seed = 1000*cfg_index + tensor_id`` (+100*block for the
stack, +50 for the image stream of a two-stream block, tensor id 10000+s for
the temb of denoising step s); draws are
``numpy.random.default_rng(seed).standard_normal(dtype=float32) * sigma``,
then rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

# tensor ids of the seeding recipe
TID = dict(x=1, temb=2, w_mod=3, b_mod=4, w1=5, b1=6, w2=7, b2=8,
           q_norm_w=9, k_norm_w=10, h=11, scale=12, shift=13, gate=14,
           # weights of one stream of a two-stream / sequential block (+50 for stream 1)
           w_mod6=15, b_mod6=16, w_qkv=17, b_qkv=18, w_o=19, b_o=20,
           w_fc1=21, b_fc1=22, w_fc2=23, b_fc2=24)


@dataclass(frozen=True)
class BlockShape:
    """Dimensions of one single-stream block and its token grid."""
    name: str
    cfg_index: int
    seq_len: int
    dim: int
    num_heads: int
    head_dim: int
    mlp_hidden: int
    # rotary embedding: dims of the head split per position axis, and the grid
    rope_axes_dims: tuple = ()
    grid: tuple = ()          # extent of each position axis for image/latent tokens
    text_tokens: int = 0      # tokens placed first, all at position 0 on every axis
    temb_dim: int = 0
    ln_eps: float = 1e-6
    qk_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def n1(self) -> int:       # linear1 output width: q | k | v | mlp
        return 3 * self.dim + self.mlp_hidden

    @property
    def n2(self) -> int:       # linear2 input width: attn_out | gelu(mlp)
        return self.dim + self.mlp_hidden

    @property
    def tdim(self) -> int:
        return self.temb_dim or self.dim


TINY = BlockShape("tiny", 0, 256, 256, 4, 64, 1024, (32, 32), (16, 16), 0)
CHAIN = BlockShape("chain", 1, 4608, 3072, 24, 128, 12288)
FLUX = BlockShape("flux", 2, 4608, 3072, 24, 128, 12288, (64, 64), (64, 64), 512)
STACK = BlockShape("stack", 3, 4608, 3072, 24, 128, 12288, (64, 64), (64, 64), 512)
VIDEO = BlockShape("video", 4, 16384, 1536, 12, 128, 8960, (32, 48, 48), (16, 32, 32), 0)
# two-stream block at the Flux shape: 512 text tokens then the 64x64 image grid
FLUX_DOUBLE = BlockShape("flux_double", 5, 4608, 3072, 24, 128, 12288, (64, 64), (64, 64), 512)
SHAPES = {s.name: s for s in (TINY, CHAIN, FLUX, STACK, VIDEO, FLUX_DOUBLE)}


def small_shape(seq_len=192, dim=256, num_heads=2, head_dim=128, mlp_hidden=512,
                grid=(8, 8), text_tokens=128, axes=(64, 64), name="small"):
    """A reduced block used by parity tests: several tiles plus ragged grids."""
    return BlockShape(name, 0, seq_len, dim, num_heads, head_dim, mlp_hidden,
                      axes, grid, text_tokens)


# ---------------------------------------------------------------- rounding
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even);
    return the raw 16-bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(a))


# ------------------------------------------------------------------ draws
def draw(seed: int, shape, sigma: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """Seeded N(mean, sigma^2) draw, rounded to bf16, returned as float32."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    if mean:
        a = a + np.float32(mean)
    return round_bf16(a)


def seed_of(shape: BlockShape, name: str, block: int = 0) -> int:
    return 1000 * shape.cfg_index + TID[name] + 100 * block


# -------------------------------------------------------------- positions
def positions(shape: BlockShape) -> np.ndarray:
    """Integer position of every token on each rotary axis, [S, n_axes] int32.

    The text tokens come first and sit at position 0 on every axis; the
    image (or latent video) tokens follow in row-major order over ``grid``.
    When the sequence is longer than text + grid (ragged test shapes), the
    grid is repeated.
    """
    n_axes = len(shape.rope_axes_dims)
    S = shape.seq_len
    pos = np.zeros((S, n_axes), dtype=np.int32)
    if n_axes == 0:
        return pos
    grid = np.stack(np.meshgrid(*[np.arange(g) for g in shape.grid], indexing="ij"),
                    axis=-1).reshape(-1, n_axes)
    n_img = S - shape.text_tokens
    reps = -(-n_img // grid.shape[0])
    pos[shape.text_tokens:] = np.tile(grid, (reps, 1))[:n_img]
    return pos


# ------------------------------------------------------------ block inputs
@dataclass
class BlockWeights:
    w_mod: np.ndarray   # [3d, temb_dim]
    b_mod: np.ndarray   # [3d]
    w1: np.ndarray      # [3d+mlp, d]
    b1: np.ndarray      # [3d+mlp]
    w2: np.ndarray      # [d, d+mlp]
    b2: np.ndarray      # [d]
    q_norm_w: np.ndarray  # [head_dim] float32
    k_norm_w: np.ndarray  # [head_dim] float32


def block_weights(shape: BlockShape, block: int = 0, norm_weights: str = "ones",
                  sigma: float = 0.02) -> BlockWeights:
    """Weights of one block: N(0, 0.02) bf16 values; RMSNorm weights are ones
    by default, or 1 + N(0, 0.1) (fp32, not rounded) with ``norm_weights='random'``."""
    d, t, n1, n2, dh = shape.dim, shape.tdim, shape.n1, shape.n2, shape.head_dim
    s = lambda name: seed_of(shape, name, block)
    if norm_weights == "ones":
        qw = np.ones(dh, np.float32)
        kw = np.ones(dh, np.float32)
    else:
        qw = (1.0 + 0.1 * np.random.default_rng(s("q_norm_w")).standard_normal(dh)).astype(np.float32)
        kw = (1.0 + 0.1 * np.random.default_rng(s("k_norm_w")).standard_normal(dh)).astype(np.float32)
    return BlockWeights(
        w_mod=draw(s("w_mod"), (3 * d, t), sigma), b_mod=draw(s("b_mod"), (3 * d,), sigma),
        w1=draw(s("w1"), (n1, d), sigma), b1=draw(s("b1"), (n1,), sigma),
        w2=draw(s("w2"), (d, n2), sigma), b2=draw(s("b2"), (d,), sigma),
        q_norm_w=qw, k_norm_w=kw)


@dataclass
class StreamWeights:
    """One stream of a two-stream block (or a sequential block)."""
    w_mod: np.ndarray     # [6d, temb_dim]
    b_mod: np.ndarray     # [6d]
    w_qkv: np.ndarray     # [3d, d]
    b_qkv: np.ndarray     # [3d]
    q_norm_w: np.ndarray  # [head_dim] float32
    k_norm_w: np.ndarray  # [head_dim] float32
    w_o: np.ndarray       # [d, d]
    b_o: np.ndarray       # [d]
    w_fc1: np.ndarray     # [mlp, d]
    b_fc1: np.ndarray     # [mlp]
    w_fc2: np.ndarray     # [d, mlp]
    b_fc2: np.ndarray     # [d]


def stream_weights(shape: BlockShape, stream: int = 0, block: int = 0, norm_weights: str = "ones",
                   sigma: float = 0.02) -> StreamWeights:
    """Weights of stream ``stream`` (0 text, 1 image) of a two-stream block:
    N(0, sigma) bf16 values, seeds offset by 50 per stream; RMSNorm weights as
    in block_weights."""
    d, t, m, dh = shape.dim, shape.tdim, shape.mlp_hidden, shape.head_dim
    s = lambda name: seed_of(shape, name, block) + 50 * stream
    if norm_weights == "ones":
        qw = np.ones(dh, np.float32)
        kw = np.ones(dh, np.float32)
    else:
        qw = (1.0 + 0.1 * np.random.default_rng(s("q_norm_w")).standard_normal(dh)).astype(np.float32)
        kw = (1.0 + 0.1 * np.random.default_rng(s("k_norm_w")).standard_normal(dh)).astype(np.float32)
    return StreamWeights(
        w_mod=draw(s("w_mod6"), (6 * d, t), sigma), b_mod=draw(s("b_mod6"), (6 * d,), sigma),
        w_qkv=draw(s("w_qkv"), (3 * d, d), sigma), b_qkv=draw(s("b_qkv"), (3 * d,), sigma),
        q_norm_w=qw, k_norm_w=kw,
        w_o=draw(s("w_o"), (d, d), sigma), b_o=draw(s("b_o"), (d,), sigma),
        w_fc1=draw(s("w_fc1"), (m, d), sigma), b_fc1=draw(s("b_fc1"), (m,), sigma),
        w_fc2=draw(s("w_fc2"), (d, m), sigma), b_fc2=draw(s("b_fc2"), (d,), sigma))


def block_activations(shape: BlockShape):
    """x [S, d] ~ N(0,1) and temb [temb_dim] ~ N(0,1), bf16 values."""
    x = draw(seed_of(shape, "x"), (shape.seq_len, shape.dim), 1.0)
    temb = draw(seed_of(shape, "temb"), (shape.tdim,), 1.0)
    return x, temb


def step_temb(shape: BlockShape, step: int) -> np.ndarray:
    """temb of denoising step ``step`` (tensor id 10000+step)."""
    return draw(1000 * shape.cfg_index + 10000 + step, (shape.tdim,), 1.0)


def chain_inputs(rows: int = 4608, cols: int = 3072, cfg_index: int = 1):
    """Memory-bound chain workload: x, h ~ N(0,1) [rows, cols] bf16 values;
    scale, shift, gate ~ N(0, 0.1) float32 (vectors of the modulation)."""
    b = 1000 * cfg_index
    x = draw(b + TID["x"], (rows, cols), 1.0)
    h = draw(b + TID["h"], (rows, cols), 1.0)
    vec = lambda tid: (np.random.default_rng(b + tid).standard_normal(cols, dtype=np.float32)
                       * np.float32(0.1))
    return dict(x=x, h=h, scale=vec(TID["scale"]), shift=vec(TID["shift"]),
                gate=vec(TID["gate"]))

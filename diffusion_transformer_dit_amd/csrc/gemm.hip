// bf16 GEMMs of the DiT blocks on gfx950 matrix cores, with the
// elementwise tails fused into the epilogue:
//   linear1:  z = u W1^T + b1; q|k|v columns -> qkv, mlp columns -> GELU -> cat
//             (optionally with the per-head q/k RMSNorm + RoPE)
//   linear2:  y = x + gate * (cat W2^T + b2)
// and the same epilogues for the two-stream block's linears, where one
// launch carries the text and the image stream's problems.
// Both operands are K-contiguous ([rows, K] row-major, the nn.Linear layout
// for the weight), C = A B^T.  The Flux page (ChituDiffusion, sections 2 and
// 3.2) finds these GEMMs dominating the block's timeline before and after
// fusion; the elementwise work around them is what its section 1.1 fuses.
//
// Two kernels.  The 256 x 256 tile runs the four-wave kernel further down
// (one wave per SIMD, 128 x 128 per wave, 64-wide K slices).  The other tiles
// run the ping-pong kernel: one workgroup of 8 wavefronts owns a BM x BN
// output tile; two groups of 4 waves each own half of it.  K is walked in BK = 32 slices
// through a ring of 4 LDS buffers filled by direct global->LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land in LDS without passing
// through registers), issued 3 slices ahead.  The two groups run half a slice
// apart ("ping-pong"): between two workgroup barriers one group multiplies its
// operands with v_mfma_f32_16x16x32_bf16 while the other group issues its
// share of the refill and reads its next operands from LDS, so each SIMD (one
// wave of each group) always has MFMA work while the other wave waits on
// memory.  Rows of a slice are 64 bytes (four 16-byte chunks); chunk
// positions are XOR-swizzled by row so that the operand reads are free of
// bank conflicts.  Accumulation is fp32.  Tiles are numbered so that the
// tiles one XCD runs at a time (blocks are dealt round-robin to the 8 XCDs)
// form a compact patch sharing A and B panels in that XCD's L2.
#include <type_traits>

#include "dit_common.hpp"
#include "launch.hpp"

namespace dit {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 32, NSTAGE = NSTAGE_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int ROW_BYTES = BK * 2;               // 64
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // one wave-load = 64 lanes x 16 bytes = 16 rows of a slice
  static constexpr int A_WL = BM / 16, B_WL = BN / 16, WL = A_WL + B_WL;
  static constexpr int L = (WL + NW - 1) / NW;           // wave-loads per wave per slice
  // waves with fewer real loads issue their spare ones into a 1 KB trash slot,
  // so that every wave has exactly L loads in flight per slice
  static constexpr int TRASH = NSTAGE * STAGE;
  static constexpr int LDS_BYTES = TRASH + ((WL % NW) ? 1024 : 0);
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "tile must be a multiple of 16 rows");
  static_assert(NSTAGE == 4, "the pipeline is written for a 4-slice ring");
  static_assert(NW == 8, "two groups of four waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring too large");
};

// Swizzle of 16-byte chunk positions inside a 64-byte row: chunk c of row r
// sits at position c ^ ((r >> 1) & 3).  A fragment read (row = lane & 15,
// chunk = lane >> 4) then touches every bank once per LDS cycle; measured
// with SQ_LDS_BANK_CONFLICT, other XOR patterns (including one that also
// folds in bit 3 of the row) leave one conflict cycle per two.
__device__ __forceinline__ int row_swz(int r) { return (r >> 1) & 3; }

// s_waitcnt vmcnt(VM) lgkmcnt(LGKM), expcnt unconstrained (gfx9 encoding;
// LGKM = 15 leaves lgkmcnt unconstrained).
template <int VM, int LGKM>
__device__ __forceinline__ void wait_cnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS; lane i writes
// lds_block + 16 i (lds_block must be the same for the whole wavefront).
__device__ __forceinline__ void load_lds_16(const bf16_t* src, unsigned char* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_block, 16, 0, 0);
}

// Epilogues act on 4 consecutive columns of one output row (the layout of
// the transposed MFMA product, see the kernel): col(col0) loads what depends
// only on the columns, pre(row, col0) what one row's 4 values need besides
// the accumulators (the residual of the gated epilogues), and
// store<Guard>(row, colb, lc, ...) finishes and writes them, at column
// colb + lc where colb (the 16-column block) is the same for the whole wave.
// Guard = false when the wave's whole sub-tile is inside M x N: the stores
// are then unconditional, with no branch around each one (a branch that may
// skip a store makes the compiler count fewer stores in flight and wait for
// earlier stores before later loads are used).
// Loaded values are kept as loaded (bf16 bits) and widened at the store, so
// that the loads of a batch are all issued before the first wait.
struct Cols4 {
  u32x2 a;  // bias (bf16 bits)
  f32x4 b;  // gate
};
struct NoPre {};
__device__ __forceinline__ f32x4 widen_bf4(const u32x2& w) {
  return f32x4{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
}
__device__ __forceinline__ u32x2 load_raw4(const bf16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ f32x4 load_bf4(const bf16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
}
__device__ __forceinline__ void store_bf4(bf16_t* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
}

// Columns [0, split) of z = acc + bias go to qkv (row stride ld_qkv);
// columns [split, N) go through GELU-tanh to cat at column gelu_col0 + (col -
// split) (row stride ld_cat).  d is the width of q (and of k) for the head
// norm of EpiLinear1QK.
struct EpiLinear1 {
  static constexpr bool kHeadNorm = false;
  static constexpr bool kRowStore = true;
  const bf16_t* bias;
  bf16_t* qkv;
  bf16_t* cat;
  int M, N, split, d, ld_qkv, ld_cat, gelu_col0;
  // columns past N (never stored) read the last 4 columns: no per-lane branch
  template <bool HasBias>
  __device__ __forceinline__ Cols4 col(int col0) const {
    Cols4 c;
    c.a = HasBias ? load_raw4(bias + min(col0, N - 4)) : u32x2{0u, 0u};
    return c;
  }
  using Pre = NoPre;
  __device__ __forceinline__ Pre pre(int, int) const { return {}; }
  template <bool Guard>
  __device__ __forceinline__ void store(int row, int colb, int lc, const Cols4& c, const Pre&, const f32x4& v) const {
    const int col0 = colb + lc;
    if (Guard && (row >= M || col0 >= N)) return;
    f32x4 z = v + widen_bf4(c.a);
    // split is a multiple of 64: the whole 16-column block is on one side, so
    // the branch is uniform and holds no memory access; the one store below
    // is unconditional
    const bool act = colb >= split;
    if (act) {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = gelu_tanh(z[i]);
    }
    bf16_t* dst = act ? cat + size_t(row) * ld_cat + gelu_col0 + (col0 - split) : qkv + size_t(row) * ld_qkv + col0;
    store_bf4(dst, z);
  }
  // A wave's whole sub-tile inside M x N with all its columns [colb0, colb0 +
  // 16 FN) on one side of split (act, uniform: the GELU side): one row
  // address per row block, the column blocks at immediate offsets from it,
  // so a store costs no address arithmetic.  One code path for both sides
  // (a uniform branch around the GELU): with two, the compiler moves every
  // accumulator out of the accumulation registers ahead of the branch.
  template <int FM, int FN>
  __device__ __forceinline__ void store_rows(int row0, int colb0, int lc, bool act, const u32x2 (&bv)[FN],
                                             const f32x4 (&acc)[FM][FN]) const {
    bf16_t* const base = (act ? cat + (gelu_col0 - split) : qkv) + colb0 + lc;
    const int ld = act ? ld_cat : ld_qkv;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      bf16_t* const rp = base + size_t(row0 + 16 * i) * ld;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        f32x4 z = acc[i][j] + widen_bf4(bv[j]);
        if (act) {
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = gelu_tanh(z[e]);
        }
        store_bf4(rp + 16 * j, z);
      }
    }
  }
};

// linear1 whose q and k columns also get the per-head RMSNorm (weights qw,
// kw over the head_dim dims of a head) and the RoPE rotation of adjacent dim
// pairs (tables [S, head_dim/2]) before they are stored, so q and k are
// rounded to bf16 once, after both: a wave that owns 128 columns (the tiles
// with WN == 128) holds whole heads of every row it covers, one head of 128
// or two of 64.
struct EpiLinear1QK : EpiLinear1 {
  static constexpr bool kHeadNorm = true;
  const float* qw;
  const float* kw;
  const float* rcos;
  const float* rsin;
  float eps;
  int head_dim;  // 64 or 128
  // Rows rw + fr + 16 i (i < FM) of the 128 columns starting at colw (< 2d,
  // a multiple of 64); lane columns 4*fk + 16 j + (0..3) of block j.  With
  // head_dim 64, blocks j < 4 and j >= 4 are two heads; the q | k boundary
  // (column d) may fall between them.  The RoPE tables and the output go
  // through buffer descriptors over the wave's rows that lie inside M (the
  // hardware range check covers the scalar offset too): table reads past M
  // return zero and stores past M are dropped, so no lane takes a branch; the
  // row block goes into the scalar offset and the column block into the
  // instruction's immediate, so no access costs address arithmetic.
  template <int FM, int FN>
  __device__ __forceinline__ void store_head(int rw, int fr, int colw, int fk, const f32x4 (&acc)[FM][FN]) const {
    static_assert(FN == 8, "128 columns per wave");
    const int hm = head_dim - 1;       // column inside the head = c & hm
    const int half = head_dim >> 1;    // RoPE table row length
    const float inv_hd = head_dim == 128 ? (1.0f / 128.0f) : (1.0f / 64.0f);
    f32x4 wv[FN];
    u32x2 bv[FN];  // bf16 bits, widened at use
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = j * 16 + 4 * fk;  // column inside the wave's 128
      const float* w = colw + c < d ? qw : kw;
      wv[j] = *reinterpret_cast<const f32x4*>(w + (c & hm));
    }
    if (bias) {  // one uniform branch around all the bias loads
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[j] = load_raw4(bias + colw + j * 16 + 4 * fk);
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[j] = u32x2{0u, 0u};
    }
    // the wave's rows inside M (none when rw >= M); the clamp compiles to a
    // vector instruction, so the result is made scalar again: a descriptor
    // built from a vector value costs a loop over lanes at every access
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16 * FM, M - rw)));
    const __amdgpu_buffer_rsrc_t out =
        __builtin_amdgcn_make_buffer_rsrc(qkv + size_t(rw) * ld_qkv + colw, 0, rows * ld_qkv * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t tcos =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rcos) + size_t(rw) * half, 0, rows * half * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t tsin =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rsin) + size_t(rw) * half, 0, rows * half * 4, 0x00020000);
    const int ovoff = (fr * ld_qkv + 4 * fk) * 2;  // bytes: row fr, lane column 4 fk
    const int tvoff = (fr * half + 2 * fk) * 4;     // bytes: table row fr, pair 2 fk
    // The RoPE table entries of row block i+1 are loaded before row block i
    // is stored (a wait for a load also waits for every store issued before
    // it).  Column block j's pair sits ((16 j) & hm) / 2 entries further.
    f32x2 cs[2][FN], sn[2][FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int so = ((j * 16) & hm) * 2;
      cs[0][j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(tcos, tvoff, so, 0));
      sn[0][j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(tsin, tvoff, so, 0));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i + 1 < FM) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int so = (16 * (i + 1) * half + ((j * 16) & hm) / 2) * 4;
          cs[(i + 1) & 1][j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(tcos, tvoff, so, 0));
          sn[(i + 1) & 1][j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(tsin, tvoff, so, 0));
        }
      }
      f32x4 z[FN];
      float s0 = 0.f, s1 = 0.f;  // sums of squares over blocks 0..3 and 4..7
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        z[j] = acc[i][j] + widen_bf4(bv[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j < 4) s0 = fmaf(z[j][e], z[j][e], s0);
          else s1 = fmaf(z[j][e], z[j][e], s1);
        }
      }
      // a row's 128 values sit in lanes fr + 16 fk, fk = 0..3
      s0 = xor32_sum(xor16_sum(s0));
      s1 = xor32_sum(xor16_sum(s1));
      if (head_dim == 128) s0 = s1 = s0 + s1;
      const float r0 = __frsqrt_rn(s0 * inv_hd + eps);
      const float r1 = __frsqrt_rn(s1 * inv_hd + eps);
      const int orow = 16 * i * ld_qkv * 2;  // row block i, bytes
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const float r = j < 4 ? r0 : r1;
        const f32x2 cj = cs[i & 1][j], sj = sn[i & 1][j];
        f32x4 n;
#pragma unroll
        for (int e = 0; e < 4; ++e) n[e] = z[j][e] * r * wv[j][e];
        f32x4 o;
        o[0] = n[0] * cj[0] - n[1] * sj[0];
        o[1] = n[0] * sj[0] + n[1] * cj[0];
        o[2] = n[2] * cj[1] - n[3] * sj[1];
        o[3] = n[2] * sj[1] + n[3] * cj[1];
        const u32x2 w = u32x2{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, out, ovoff + 32 * j, orow, 0);
      }
    }
  }
};

struct EpiLinear2 {
  static constexpr bool kHeadNorm = false;
  static constexpr bool kRowStore = false;
  const bf16_t* bias;
  const bf16_t* x;
  const float* gate;
  bf16_t* y;
  int M, N;
  // rows and columns past M and N (never stored) read the last ones: no per-lane branch
  template <bool HasBias>
  __device__ __forceinline__ Cols4 col(int col0) const {
    Cols4 c;
    const int cc = min(col0, N - 4);
    c.a = HasBias ? load_raw4(bias + cc) : u32x2{0u, 0u};
    c.b = *reinterpret_cast<const f32x4*>(gate + cc);
    return c;
  }
  using Pre = u32x2;  // the residual x (bf16 bits)
  __device__ __forceinline__ Pre pre(int row, int col0) const {
    return load_raw4(x + size_t(min(row, M - 1)) * N + min(col0, N - 4));
  }
  template <bool Guard>
  __device__ __forceinline__ void store(int row, int colb, int lc, const Cols4& c, const Pre& xr, const f32x4& v) const {
    const int col0 = colb + lc;
    if (Guard && (row >= M || col0 >= N)) return;
    const f32x4 xv = widen_bf4(xr), bv = widen_bf4(c.a);
    f32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = fmaf(c.b[i], v[i] + bv[i], xv[i]);
    store_bf4(y + size_t(row) * N + col0, z);
  }
};

// y = x + gate * (acc + bias) with the residual x and the output y of either
// storage type (bf16 or fp32): the two-stream block keeps its mid-block
// residual x' in fp32 between the attention and MLP halves.
__device__ __forceinline__ f32x4 load4(const bf16_t* p) { return load_bf4(p); }
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void store4(bf16_t* p, const f32x4& v) { store_bf4(p, v); }
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }

template <class XT, class YT>
struct EpiGated {
  static constexpr bool kHeadNorm = false;
  static constexpr bool kRowStore = false;
  const bf16_t* bias;
  const XT* x;
  const float* gate;
  YT* y;
  int M, N;
  // rows and columns past M and N (never stored) read the last ones: no per-lane branch
  template <bool HasBias>
  __device__ __forceinline__ Cols4 col(int col0) const {
    Cols4 c;
    const int cc = min(col0, N - 4);
    c.a = HasBias ? load_raw4(bias + cc) : u32x2{0u, 0u};
    c.b = *reinterpret_cast<const f32x4*>(gate + cc);
    return c;
  }
  // the residual x as loaded (bf16 bits or fp32)
  using Pre = std::conditional_t<std::is_same_v<XT, float>, f32x4, u32x2>;
  __device__ __forceinline__ Pre pre(int row, int col0) const {
    const XT* p = x + size_t(min(row, M - 1)) * N + min(col0, N - 4);
    if constexpr (std::is_same_v<XT, float>) return *reinterpret_cast<const f32x4*>(p);
    else return load_raw4(p);
  }
  template <bool Guard>
  __device__ __forceinline__ void store(int row, int colb, int lc, const Cols4& c, const Pre& xr, const f32x4& v) const {
    const int col0 = colb + lc;
    if (Guard && (row >= M || col0 >= N)) return;
    f32x4 xv;
    if constexpr (std::is_same_v<XT, float>) xv = xr;
    else xv = widen_bf4(xr);
    const f32x4 bv = widen_bf4(c.a);
    f32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = fmaf(c.b[i], v[i] + bv[i], xv[i]);
    store4(y + size_t(row) * N + col0, z);
  }
};

// A wave's stores: lane rows row0 + 16 i, columns col0 + 16 j + (0..3).  The
// column loads come first; the per-row loads of column block j+1 are issued
// before block j is stored.  The vector-memory counter counts loads and
// stores alike and completes in issue order, so a wait for a load issued
// after some stores would also wait for those stores to drain.
template <int FM, int FN, bool Guard, class Epi>
__device__ __forceinline__ void store_tile(const Epi& epi, int row0, int colb0, int lc, const f32x4 (&acc)[FM][FN]) {
  Cols4 c[FN];
  if (epi.bias) {  // one uniform branch around all the column loads
#pragma unroll
    for (int j = 0; j < FN; ++j) c[j] = epi.template col<true>(colb0 + 16 * j + lc);
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) c[j] = epi.template col<false>(colb0 + 16 * j + lc);
  }
  typename Epi::Pre p[2][FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) p[0][i] = epi.pre(row0 + 16 * i, colb0 + lc);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    if (j + 1 < FN) {
#pragma unroll
      for (int i = 0; i < FM; ++i) p[(j + 1) & 1][i] = epi.pre(row0 + 16 * i, colb0 + 16 * (j + 1) + lc);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
      epi.template store<Guard>(row0 + 16 * i, colb0 + 16 * j, lc, c[j], p[j & 1][i], acc[i][j]);
  }
}

// A wave's whole epilogue: the q/k head path for the tiles whose waves own
// whole heads; the row-address path of linear1 for a sub-tile inside the
// output whose columns lie on one side of split; otherwise store_tile, with
// unguarded stores when the wave's sub-tile lies inside the output.
template <int FM, int FN, class Epi>
__device__ __forceinline__ void wave_epilogue(const Epi& epi, int M, int N, int rw, int cw, int fr, int fk,
                                              const f32x4 (&acc)[FM][FN]) {
  rw = __builtin_amdgcn_readfirstlane(rw);  // the wave's first row and column: uniform
  cw = __builtin_amdgcn_readfirstlane(cw);
  const bool full = rw + 16 * FM <= M && cw + 16 * FN <= N;
  if constexpr (Epi::kHeadNorm && FN == 8) {
    if (cw < 2 * epi.d) {  // a whole head: q or k columns get normalised and rotated
      epi.template store_head<FM, FN>(rw, fr, cw, fk, acc);
      return;
    }
  }
  if constexpr (Epi::kRowStore) {
    if (full && (cw + 16 * FN <= epi.split || cw >= epi.split)) {
      u32x2 bv[FN];  // bias bf16 bits, one uniform branch around the loads
      if (epi.bias) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = load_raw4(epi.bias + cw + 16 * j + 4 * fk);
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = u32x2{0u, 0u};
      }
      epi.template store_rows<FM, FN>(rw + fr, cw, 4 * fk, cw >= epi.split, bv, acc);
      return;
    }
  }
  if (full) store_tile<FM, FN, false>(epi, rw + fr, cw, 4 * fk, acc);
  else store_tile<FM, FN, true>(epi, rw + fr, cw, 4 * fk, acc);
}

// One GEMM of a launch: C = A B^T with A [M, K], B [N, K], finished by epi.
template <class Epi>
struct GemmProblem {
  const bf16_t* A;
  const bf16_t* B;
  int M, N, K;
  Epi epi;
};

// NP independent GEMMs in one launch (e.g. the text and image streams of a
// two-stream block): problem i owns tile ids [first[i], first[i + 1]) of the
// XCD-remapped numbering, so the launch fills the chip once instead of
// leaving it half idle for the smaller problem.
template <class Epi, int NP>
struct GemmGroup {
  GemmProblem<Epi> p[NP];
  int first[NP];  // first[0] == 0
};

// Hardware deals block b to XCD b % 8; the remap makes consecutive ids run on
// one XCD, so that a problem's tiles stay together on an XCD.
__device__ __forceinline__ int xcd_block_id() {
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  return (nb & 7) == 0 ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
}

// Map a problem-local tile id to a (tile_m, tile_n) pair: consecutive ids
// form GROUP_M-tall column-major patches of tiles sharing A and B panels.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = GROUP_M * tiles_n;
  const int g = bid / group;
  const int first_m = g * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in = bid - g * group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

template <class C, class Epi, int NP>
__global__ void __launch_bounds__(C::NT, C::NW / 4)
gemm_bf16_tn_kernel(GemmGroup<Epi, NP> grp) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];
  int bid = xcd_block_id();
  int pi = 0;
#pragma unroll
  for (int i = 1; i < NP; ++i)
    if (bid >= grp.first[i]) pi = i;
  bid -= grp.first[pi];
  const bf16_t* __restrict__ A = grp.p[pi].A;
  const bf16_t* __restrict__ B = grp.p[pi].B;
  const int M = grp.p[pi].M, N = grp.p[pi].N, K = grp.p[pi].K;
  const Epi& epi = grp.p[pi].epi;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_coords<4>(bid, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  // Direct-to-LDS loads.  Wave w issues wave-loads j = w, w + NW, ...; lane i
  // of wave-load j writes LDS bytes [16 i, 16 i + 16) of the j-th 1 KB block
  // of the slice, i.e. row 16 j' + i/4 (j' = j inside A or B), chunk position
  // i % 4, which holds global chunk (i % 4) ^ swz(row) of that row.
  const int lrow = lane >> 2;                       // row inside the 16-row block
  const int lchunk = (lane & 3) ^ row_swz(lrow);    // global chunk this lane fetches
  const bf16_t* gsrc[C::L];
  uint32_t ldst[C::L];  // LDS byte offset inside a slice buffer, or TRASH for a spare load
#pragma unroll
  for (int i = 0; i < C::L; ++i) {
    const int j = wave + i * C::NW;
    if (j < C::A_WL) {
      const int r = min(m0 + 16 * j + lrow, M - 1);  // rows past M are clamped; never stored
      gsrc[i] = A + size_t(r) * K + lchunk * 8;
      ldst[i] = uint32_t(j) * 1024u;
    } else if (j < C::WL) {
      const int jb = j - C::A_WL;
      const int r = min(n0 + 16 * jb + lrow, N - 1);
      gsrc[i] = B + size_t(r) * K + lchunk * 8;
      ldst[i] = uint32_t(C::A_BYTES) + uint32_t(jb) * 1024u;
    } else {
      gsrc[i] = gsrc[0];  // any valid address; lands in the trash slot
      ldst[i] = C::TRASH;
    }
  }
  // the trash slot is shared by all stages: its offset does not move with the stage
  auto issue = [&](int kt, int stage) {
    const uint32_t sbase = uint32_t(stage) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::L; ++i)
      load_lds_16(gsrc[i] + kt * C::BK, smem + (ldst[i] == uint32_t(C::TRASH) ? ldst[i] : sbase + ldst[i]));
  };

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA operand reads: lane holds row (lane & 15) of a 16-row fragment and
  // the 8 K-values of chunk (lane >> 4) of the 32-wide slice.
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const uint32_t swz = uint32_t((fk ^ row_swz(fr)) << 4);
  const uint32_t a_off = uint32_t(wm * C::WM + fr) * C::ROW_BYTES + swz;
  const uint32_t b_off = C::A_BYTES + uint32_t(wn * C::WN + fr) * C::ROW_BYTES + swz;

  bf16x8 frag[C::FM + C::FN];
  auto read_frags = [&](int stage) {
    const unsigned char* s = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) frag[i] = *reinterpret_cast<const bf16x8*>(s + a_off + i * 16 * C::ROW_BYTES);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      frag[C::FM + j] = *reinterpret_cast<const bf16x8*>(s + b_off + j * 16 * C::ROW_BYTES);
  };
  auto mfmas = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag[C::FM + j], frag[i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Workgroup barrier after this wave's loads of all but the `ahead` most
  // recent slices have landed and its LDS reads are complete.
  auto sync = [&](int ahead) {
    if (ahead >= 2) wait_cnt<2 * C::L, 0>();
    else if (ahead == 1) wait_cnt<C::L, 0>();
    else wait_cnt<0, 0>();
    block_barrier();
  };

  const int KT = K / C::BK;  // >= 2: K is a multiple of 64
  const int group = wave >> 2;
  // prologue: every wave issues its share of slices 0..2; slice s lives in buffer s % 4
  issue(0, 0);
  issue(1, 1);
  if (KT > 2) issue(2, 2);
  // Iteration k, two phases.  Phase 1: group 0 refills (slice k+3 into the
  // buffer of slice k-1, which both groups have finished reading) and reads
  // slice k; group 1 multiplies slice k-1.  Phase 2: group 0 multiplies
  // slice k; group 1 refills and reads slice k.  Before a group reads slice
  // k, every wave's loads of slice k have landed (barrier of phase 1).
  for (int k = 0; k <= KT; ++k) {
    const int ahead = min(2, KT - 1 - k);
    sync(ahead);
    if (group == 0) {
      if (k < KT) {
        if (k + 3 < KT) issue(k + 3, (k + 3) & 3);
        read_frags(k & 3);
      }
    } else if (k >= 1) {
      mfmas();
    }
    // phase 2 needs no wait: every wave's loads of slice k landed before the
    // phase-1 barrier, and no slot is refilled before the next one
    block_barrier();
    if (k < KT) {
      if (group == 0) {
        mfmas();
      } else {
        if (k + 3 < KT) issue(k + 3, (k + 3) & 3);
        read_frags(k & 3);
      }
    }
  }

  // The MFMAs compute the transposed product C^T = B A^T per 16x16 block, so
  // lane l holds row (l & 15) of the block and its 4 consecutive columns
  // 4*(l >> 4) + (0..3): one 8-byte store per block and lane.
  wave_epilogue<C::FM, C::FN>(epi, M, N, m0 + wm * C::WM, n0 + wn * C::WN, fr, fk, acc);
}

// ------------------------------------------------------------ four-wave kernel
// One wave per SIMD: 4 waves in a 2 x 2 grid, each owning a (BM/2) x (BN/2)
// sub-tile whose fp32 accumulators live in the accumulation registers.  K is
// walked in slices of 64 (128-byte rows: every refill request covers a whole
// 128-byte cache line, half as many L2 requests as 64-byte rows need) through
// two LDS slots.  A wave streams its own MFMAs and, between them, reads the
// next half-slice's operands from LDS and issues its share of the refill, so
// a 128 x 128 sub-tile reads 0.25 operand fragments per MFMA and one
// workgroup barrier is needed per slice.  Same K order, MFMA and operand
// pairing as the ping-pong kernel, so both produce bitwise the same results.
template <int BM_, int BN_>
struct Tile4Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, NSTAGE = 2;
  static constexpr int WAVES_M = 2, WAVES_N = 2, NW = 4, NT = 256;
  static constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  static constexpr int ROW_BYTES = BK * 2;  // 128
  static constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // one wave-load = 64 lanes x 16 bytes = 8 rows of a slice
  static constexpr int A_WL = BM / 8, B_WL = BN / 8, WL = A_WL + B_WL;
  static constexpr int LA = A_WL / NW, LB = B_WL / NW, L = LA + LB;  // wave-loads per wave per slice
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static_assert(A_WL % NW == 0 && B_WL % NW == 0, "every wave issues the same number of loads");
  static_assert(FM * FN * 4 <= 256, "the accumulators fill at most the 256 accumulation registers");
  static_assert(L <= FM * FN, "at most one refill per MFMA");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring too large");
};

// Where a half-slice's operand reads and refills go between its FM x FN
// MFMAs: read r (the FN B fragments, then the FM A fragments of the next
// half) after MFMA (r NM) / NR + 1, refill l after MFMA (l NM) / L + NM /
// (2 L) + 1, so that no two follow the same MFMA (128 x 128 sub-tiles: reads
// after MFMAs 1, 5, 9, ..., refills after 3, 7, 11, ...).  -1: nothing.
template <class C>
struct Tile4Sched {
  static constexpr int NM = C::FM * C::FN, NR = C::FM + C::FN;
  struct Tab {
    int read[NM];
    int load[NM];
  };
  static constexpr Tab make() {
    Tab t{};
    for (int m = 0; m < NM; ++m) t.read[m] = t.load[m] = -1;
    for (int r = 0; r < NR; ++r) t.read[(r * NM) / NR + 1] = r;
    for (int l = 0; l < C::L; ++l) t.load[(l * NM) / C::L + NM / (2 * C::L) + 1] = l;
    return t;
  }
  static constexpr bool valid() {
    const Tab t = make();
    int nr = 0, nl = 0;
    for (int m = 0; m < NM; ++m) {
      nr += t.read[m] >= 0;
      nl += t.load[m] >= 0;
    }
    return nr == NR && nl == C::L && (((NR - 1) * NM) / NR + 1) < NM &&
           (((C::L - 1) * NM) / C::L + NM / (2 * C::L) + 1) < NM;
  }
  static_assert(valid(), "every read and refill has its own MFMA");
  static constexpr Tab tab = make();
};

// 16-byte chunk c of a 128-byte row r sits at position c ^ ((r >> 1) & 7): the
// 16 rows of a fragment read then cover the 64 banks once per 16 lanes.
__device__ __forceinline__ int row_swz8(int r) { return (r >> 1) & 7; }

// Buffer descriptor over `bytes` bytes from `base` (raw, 32-bit data format):
// loads at offsets past the range read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel_rsrc(const bf16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), 0, int(bytes), 0x00020000);
}

// acc += B-fragment x A-fragment (the transposed product, as in the ping-pong
// kernel) with the accumulator pinned to an accumulation register: written as
// the instruction itself so that the compiler neither copies the 256
// accumulators between register files nor spills them.  Each accumulator is
// written once per 64 MFMAs here, so no dependent pair is adjacent; the reads
// after the last one are preceded by explicit wait states (mfma_drain).
__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8& b, const bf16x8& a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}
// the first product of a tile: acc = B-fragment x A-fragment (zero accumulator input)
__device__ __forceinline__ void mfma_first(f32x4& acc, const bf16x8& b, const bf16x8& a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(b), "v"(a));
}
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

template <class C, class Epi, int NP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm4w_kernel(GemmGroup<Epi, NP> grp) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];
  int bid = xcd_block_id();
  int pi = 0;
#pragma unroll
  for (int i = 1; i < NP; ++i)
    if (bid >= grp.first[i]) pi = i;
  bid -= grp.first[pi];
  const bf16_t* __restrict__ A = grp.p[pi].A;
  const bf16_t* __restrict__ B = grp.p[pi].B;
  const int M = grp.p[pi].M, N = grp.p[pi].N, K = grp.p[pi].K;
  const Epi& epi = grp.p[pi].epi;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the LDS slot addresses are scalar
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_coords<4>(bid, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  // Refill loads through buffer descriptors over the tile's A and B row
  // panels (rows past M or N read as zero and are never stored).  Wave w
  // issues wave-loads j = w + 4 i (A for i < LA, then B): lane l fetches row
  // 8 j + l/8 of its panel, global chunk (l % 8) ^ swz8(row), into LDS bytes
  // [16 l, 16 l + 16) of the j-th 1 KB block of the slice.  The per-lane
  // offset is the same for every load; the row block and the slice go into
  // the scalar offset.
  const int lrow = lane >> 3;
  const __amdgpu_buffer_rsrc_t ra = panel_rsrc(A + size_t(m0) * K, uint32_t(min(C::BM, M - m0)) * uint32_t(K) * 2u);
  const __amdgpu_buffer_rsrc_t rb = panel_rsrc(B + size_t(n0) * K, uint32_t(min(C::BN, N - n0)) * uint32_t(K) * 2u);
  const int kb = K * 2;  // bytes per row
  const int voff0 = (8 * wave + lrow) * kb;
  const int blk_stride = 32 * kb;  // 32 rows: the next load of the same wave
  // row 8 (w + 4 i) + lrow has swz8 = (4 (w + 4 i) + (lrow >> 1)) & 7 = (4 w + (lrow >> 1)) & 7,
  // the same for every load of the wave
  const int voff = voff0 + (((lane & 7) ^ ((4 * wave + (lrow >> 1)) & 7)) * 16);
  auto issue1 = [&](int i, int kt, uint32_t sbase) {
    const bool isa = i < C::LA;
    const int ii = isa ? i : i - C::LA;
    const int soff = ii * blk_stride + kt * (C::BK * 2);
    unsigned char* dst = smem + sbase + (isa ? 0u : uint32_t(C::A_BYTES)) + uint32_t(wave + 4 * ii) * 1024u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? ra : rb, (lds_ptr_t)dst, 16, voff, soff, 0, 0);
  };

  f32x4 acc[C::FM][C::FN];  // born in the accumulation registers by the first MFMAs

  // Fragment reads: lane holds row (lane & 15) of a 16-row block and the 8
  // K-values of chunk 4 h + (lane >> 4) of half-slice h.
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const uint32_t a_row = uint32_t(wm * C::WM + fr) * C::ROW_BYTES;
  const uint32_t b_row = C::A_BYTES + uint32_t(wn * C::WN + fr) * C::ROW_BYTES;
  // position of chunk 4 h + fk in row fr (+ 16 i: bits 1..3 of the row do not change)
  const uint32_t sw0 = uint32_t(((0 + fk) ^ row_swz8(fr)) << 4), sw1 = uint32_t(((4 + fk) ^ row_swz8(fr)) << 4);
  bf16x8 fa[2][C::FM], fb[2][C::FN];
  // half-slice h of the slice in the LDS slot at sb into buffer buf: B first
  auto read_b = [&](int buf, int j, const unsigned char* sb, uint32_t sw) {
    fb[buf][j] = *reinterpret_cast<const bf16x8*>(sb + b_row + sw + j * 16 * C::ROW_BYTES);
  };
  auto read_a = [&](int buf, int i, const unsigned char* sb, uint32_t sw) {
    fa[buf][i] = *reinterpret_cast<const bf16x8*>(sb + a_row + sw + i * 16 * C::ROW_BYTES);
  };

  const int KT = K / C::BK;  // >= 1
  // prologue: slices 0 and 1 in flight (a slice past the end re-fetches the
  // last one into a slot nobody reads), half-slice 0 of slice 0 in registers
#pragma unroll
  for (int i = 0; i < C::L; ++i) issue1(i, 0, 0);
#pragma unroll
  for (int i = 0; i < C::L; ++i) issue1(i, min(1, KT - 1), C::STAGE);
  wait_cnt<C::L, 15>();
  block_barrier();
#pragma unroll
  for (int j = 0; j < C::FN; ++j) read_b(0, j, smem, sw0);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) read_a(0, i, smem, sw0);

  // Slice k in slot k & 1.  Phase 0: multiply half 0 (buffer 0) while
  // reading half 1 of the same slot into buffer 1.  Then this wave's loads
  // of slice k+1 have landed and its reads are done; a barrier makes that
  // hold for every wave.  Phase 1: multiply half 1 while reading half 0 of
  // slice k+1 (the other slot) and refilling slot k & 1 with slice k+2.
  auto phase = [&](int k, auto ph_c, auto first_c) {
    constexpr int cur = decltype(ph_c)::value, nxt = cur ^ 1;
    constexpr bool first = decltype(first_c)::value;
    const uint32_t slot = uint32_t(k & 1) * C::STAGE;
    const unsigned char* sb = smem + (cur == 0 ? slot : slot ^ uint32_t(C::STAGE));
    const uint32_t sw = cur == 0 ? sw1 : sw0;
    const int kl = min(k + 2, KT - 1);
    // The FM x FN MFMAs of the half, row block by row block, with the
    // half's operand reads for the next half and, in phase 1, its refills
    // between them one instruction at a time (the table above).
    using S = Tile4Sched<C>;
#pragma unroll
    for (int m = 0; m < S::NM; ++m) {
      const int g = m / C::FN, j = m % C::FN;
      if constexpr (first) mfma_first(acc[g][j], fb[cur][j], fa[cur][g]);
      else mfma_acc(acc[g][j], fb[cur][j], fa[cur][g]);
      const int r = S::tab.read[m];
      if (r >= 0) {
        if (r < C::FN) read_b(nxt, r, sb, sw);
        else read_a(nxt, r - C::FN, sb, sw);
      }
      if constexpr (cur == 1) {
        const int l = S::tab.load[m];
        if (l >= 0) issue1(l, kl, slot);
      }
    }
  };
  auto slice = [&](int k, auto first_c) {
    phase(k, std::integral_constant<int, 0>{}, first_c);
    wait_cnt<0, 0>();
    block_barrier();
    phase(k, std::integral_constant<int, 1>{}, std::false_type{});
  };
  slice(0, std::true_type{});
  for (int k = 1; k < KT; ++k) slice(k, std::false_type{});
  mfma_drain();
  wait_cnt<0, 0>();  // the tail's re-fetches land before the workgroup ends

  wave_epilogue<C::FM, C::FN>(epi, M, N, m0 + wm * C::WM, n0 + wn * C::WN, fr, fk, acc);
}

// ------------------------------------------------------------------ tile choice
using T288x192 = TileCfg<288, 192, 2, 4, 4>;  // 8 waves of 144 x 48; groups own 144-row halves
using T256 = Tile4Cfg<256, 256>;              // 4 waves of 128 x 128, 64-wide K slices
using T288x192w4 = Tile4Cfg<288, 192>;        // 4 waves of 144 x 96, 64-wide K slices
using T256x192w4 = Tile4Cfg<256, 192>;        // 4 waves of 128 x 96 (N = 1536 in 8 tiles: two full rounds at S = 16384)
using T256pp = TileCfg<256, 256, 4, 2, 4>;    // the same tile on the ping-pong kernel (8 waves of 64 x 128)
// The four-wave kernel's refills have one phase of lead (two 64 KB slots),
// the ping-pong kernel's three 32-wide slices.  For long K both operands
// stream from HBM (fc2 of the two-stream block: K = 12288, 402 against
// 347 us) and the deeper prefetch wins.  An epilogue that loads a residual
// per output (the gated ones) has its latency hidden only with two waves per
// SIMD (two-stream output projection: 132 against 115 us), so the gated
// epilogues on 256x256 tiles stay on the ping-pong kernel.  Otherwise the
// four-wave kernel's larger sub-tiles and whole-line refills win: the linear1
// epilogues at K = d on 256x256 tiles, linear2 on 288x192 tiles (one full
// round at the Flux shape, K = 15360: 365 against 393-402 us) and every
// epilogue on 256x192 tiles (the video shape's N = 1536 GEMMs: block -2.5 to
// -2.9 %).
constexpr int kFourWaveMaxK = 4096;
template <class Epi>
constexpr bool four_wave(int K) {
  return std::is_same_v<typename Epi::Pre, NoPre> && K <= kFourWaveMaxK;
}
using T128x256 = TileCfg<128, 256, 4, 2, 4>;  // 8 waves of 32 x 128 (whole heads per wave, small M)
using T128 = TileCfg<128, 128, 4, 2, 4>;      // 8 waves of 32 x 64

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
      n = p.multiProcessorCount;
    if (n <= 0) n = 256;
  }
  return n;
}

void prepare_device() { (void)num_cus(); }

enum TileKind { K288x192 = 0, K256 = 1, K128 = 2, K128x256 = 3, K256x192 = 4 };

// Pick the tile that minimises rounds-of-workgroups x tile area / efficiency
// (a proxy for the time of the busiest CU) over the tiles of all problems of
// one launch.  head_tiles restricts the choice to the tiles whose waves own
// 128 columns (whole heads: the fused q/k RMSNorm + RoPE epilogue).
static TileKind choose_tile(const int* Ms, const int* Ns, int np, bool head_tiles = false) {
  const int cus = num_cus();
  struct Opt { TileKind k; int bm, bn; double eff; bool heads; } opts[] = {
      // per-tile efficiency measured on the ping-pong kernel at the Flux
      // shape (288x192 waves hold a thinner 144 x 48 sub-tile and run at 0.87
      // of the 256x256 rate) and, for 256x192 (64 x 96 per wave), at the
      // video shape's N = 1536 GEMMs; the four-wave configs of these tiles
      // only widen the margin of the choices they win
      {K288x192, 288, 192, 0.87, false}, {K256, 256, 256, 1.0, true}, {K128, 128, 128, 0.6, false},
      {K128x256, 128, 256, 0.75, true}, {K256x192, 256, 192, 0.82, false}};
  TileKind best = head_tiles ? K128x256 : K128;
  double best_cost = 1e300;
  for (const Opt& o : opts) {
    if (head_tiles && !o.heads) continue;
    long long tiles = 0;
    for (int i = 0; i < np; ++i) tiles += (long long)((Ms[i] + o.bm - 1) / o.bm) * ((Ns[i] + o.bn - 1) / o.bn);
    const long long rounds = (tiles + cus - 1) / cus;
    const double cost = double(rounds) * o.bm * o.bn / o.eff;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = o.k;
    }
  }
  return best;
}
static TileKind choose_tile(int M, int N) { return choose_tile(&M, &N, 1); }

template <class C, class Epi>
static hipError_t launch_tile(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& e,
                              hipStream_t st) {
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  GemmGroup<Epi, 1> g;
  g.p[0] = GemmProblem<Epi>{A, B, M, N, K, e};
  g.first[0] = 0;
  if constexpr (C::NW == 4)
    gemm4w_kernel<C, Epi, 1><<<tiles, C::NT, 0, st>>>(g);
  else
    gemm_bf16_tn_kernel<C, Epi, 1><<<tiles, C::NT, 0, st>>>(g);
  return hipGetLastError();
}

// One launch for np (1 or 2) problems on the tile config C; problems with
// no rows or columns get no tiles.
template <class C, class Epi>
static hipError_t launch_tile_group(const GemmProblem<Epi>* ps, int np, hipStream_t st) {
  GemmGroup<Epi, 2> g;
  int n = 0, tiles = 0;
  for (int i = 0; i < np; ++i) {
    if (ps[i].M == 0 || ps[i].N == 0) continue;
    g.p[n] = ps[i];
    g.first[n] = tiles;
    tiles += ((ps[i].M + C::BM - 1) / C::BM) * ((ps[i].N + C::BN - 1) / C::BN);
    ++n;
  }
  if (n == 0) return hipSuccess;
  if (n == 1) return launch_tile<C>(g.p[0].A, g.p[0].B, g.p[0].M, g.p[0].N, g.p[0].K, g.p[0].epi, st);
  if constexpr (C::NW == 4)
    gemm4w_kernel<C, Epi, 2><<<tiles, C::NT, 0, st>>>(g);
  else
    gemm_bf16_tn_kernel<C, Epi, 2><<<tiles, C::NT, 0, st>>>(g);
  return hipGetLastError();
}

template <class Epi>
static TileKind choose_group_tile(const GemmProblem<Epi>* ps, int np) {
  int Ms[2], Ns[2];
  for (int i = 0; i < np; ++i) {
    Ms[i] = ps[i].M;
    Ns[i] = ps[i].N;
  }
  return choose_tile(Ms, Ns, np);
}

template <class Epi>
static hipError_t launch_gemm_group(const GemmProblem<Epi>* ps, int np, hipStream_t st) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  switch (choose_group_tile(ps, np)) {
    case K288x192: return launch_tile_group<T288x192>(ps, np, st);
    case K256:
      if constexpr (std::is_same_v<typename Epi::Pre, NoPre>)  // the four-wave kernel is built only for these
        if (four_wave<Epi>(ps[0].K)) return launch_tile_group<T256>(ps, np, st);
      return launch_tile_group<T256pp>(ps, np, st);
    case K256x192: return launch_tile_group<T256x192w4>(ps, np, st);
    default: return launch_tile_group<T128>(ps, np, st);
  }
}

template <class Epi>
static hipError_t launch_gemm(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& e,
                              hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (choose_tile(M, N)) {
    case K288x192:
      if constexpr (std::is_same_v<Epi, EpiLinear2>) return launch_tile<T288x192w4>(A, B, M, N, K, e, st);
      return launch_tile<T288x192>(A, B, M, N, K, e, st);
    case K256:
      if constexpr (std::is_same_v<typename Epi::Pre, NoPre>)
        if (four_wave<Epi>(K)) return launch_tile<T256>(A, B, M, N, K, e, st);
      return launch_tile<T256pp>(A, B, M, N, K, e, st);
    case K256x192: return launch_tile<T256x192w4>(A, B, M, N, K, e, st);
    default: return launch_tile<T128>(A, B, M, N, K, e, st);
  }
}

hipError_t launch_linear1(const bf16_t* u, const bf16_t* w1, const bf16_t* b1, bf16_t* qkv,
                          bf16_t* cat, int S, int d, int mlp, hipStream_t st) {
  EpiLinear1 e{b1, qkv, cat, S, 3 * d + mlp, 3 * d, d, 3 * d, d + mlp, d};
  return launch_gemm(u, w1, S, 3 * d + mlp, d, e, st);
}

bool linear1_fuses_qk(int S, int d, int mlp, int DH) {
  (void)mlp;
  return (DH == 128 || DH == 64) && S > 0 && d % 64 == 0;
}

hipError_t launch_linear1_qk(const bf16_t* u, const bf16_t* w1, const bf16_t* b1, bf16_t* qkv, bf16_t* cat,
                             int S, int d, int mlp, int DH, const float* qw, const float* kw, const float* rcos,
                             const float* rsin, float eps, hipStream_t st) {
  if (!linear1_fuses_qk(S, d, mlp, DH)) return hipErrorInvalidValue;
  EpiLinear1QK e;
  static_cast<EpiLinear1&>(e) = EpiLinear1{b1, qkv, cat, S, 3 * d + mlp, 3 * d, d, 3 * d, d + mlp, d};
  e.qw = qw;
  e.kw = kw;
  e.rcos = rcos;
  e.rsin = rsin;
  e.eps = eps;
  e.head_dim = DH;
  const int N = 3 * d + mlp;
  if (choose_tile(&S, &N, 1, true) == K256)
    return four_wave<EpiLinear1QK>(d) ? launch_tile<T256>(u, w1, S, N, d, e, st) : launch_tile<T256pp>(u, w1, S, N, d, e, st);
  return launch_tile<T128x256>(u, w1, S, N, d, e, st);
}

hipError_t launch_linear2(const bf16_t* cat, const bf16_t* w2, const bf16_t* b2, const bf16_t* x,
                          const float* gate, bf16_t* y, int S, int d, int mlp, hipStream_t st) {
  EpiLinear2 e{b2, x, gate, y, S, d};
  return launch_gemm(cat, w2, S, d, d + mlp, e, st);
}

// ------------------------------------------------ grouped linears (1 or 2 problems)
static EpiLinear1 bias_act_epi(const BiasActArgs& a) {
  return EpiLinear1{a.b, a.plain, a.gelu, a.M, a.N, a.n_plain, a.qk_dim, a.ld_plain, a.ld_gelu, a.gelu_col0};
}

hipError_t launch_bias_act_group(const BiasActArgs* a, int np, hipStream_t st) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  GemmProblem<EpiLinear1> ps[2];
  for (int i = 0; i < np; ++i) ps[i] = GemmProblem<EpiLinear1>{a[i].A, a[i].W, a[i].M, a[i].N, a[i].K, bias_act_epi(a[i])};
  return launch_gemm_group(ps, np, st);
}

bool bias_act_fuses_qk(const BiasActArgs* a, int np, int DH) {
  if ((DH != 128 && DH != 64) || np < 1 || np > 2) return false;
  for (int i = 0; i < np; ++i)
    if (a[i].qk_dim % 64 != 0 || 2 * a[i].qk_dim > a[i].n_plain) return false;
  return true;
}

hipError_t launch_bias_act_qk_group(const BiasActArgs* a, const QKNormArgs* q, int np, int DH, hipStream_t st) {
  if (!bias_act_fuses_qk(a, np, DH)) return hipErrorInvalidValue;
  GemmProblem<EpiLinear1QK> ps[2];
  int Ms[2], Ns[2];
  for (int i = 0; i < np; ++i) {
    EpiLinear1QK e;
    static_cast<EpiLinear1&>(e) = bias_act_epi(a[i]);
    e.qw = q[i].qw;
    e.kw = q[i].kw;
    e.rcos = q[i].rcos;
    e.rsin = q[i].rsin;
    e.eps = q[i].eps;
    e.head_dim = DH;
    ps[i] = GemmProblem<EpiLinear1QK>{a[i].A, a[i].W, a[i].M, a[i].N, a[i].K, e};
    Ms[i] = a[i].M;
    Ns[i] = a[i].N;
  }
  if (choose_tile(Ms, Ns, np, true) == K256)
    return four_wave<EpiLinear1QK>(ps[0].K) ? launch_tile_group<T256>(ps, np, st) : launch_tile_group<T256pp>(ps, np, st);
  return launch_tile_group<T128x256>(ps, np, st);
}

hipError_t launch_gated_group(const GatedArgs* a, int np, hipStream_t st) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  GemmProblem<EpiLinear2> ps[2];
  for (int i = 0; i < np; ++i)
    ps[i] = GemmProblem<EpiLinear2>{a[i].A, a[i].W, a[i].M, a[i].N, a[i].K,
                                    EpiLinear2{a[i].b, a[i].x, a[i].gate, a[i].y, a[i].M, a[i].N}};
  return launch_gemm_group(ps, np, st);
}

template <class XT, class YT>
static hipError_t gated_typed_group(const GatedArgs* a, int np, const XT* const* xs, YT* const* ys,
                                    hipStream_t st) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  GemmProblem<EpiGated<XT, YT>> ps[2];
  for (int i = 0; i < np; ++i)
    ps[i] = GemmProblem<EpiGated<XT, YT>>{a[i].A, a[i].W, a[i].M, a[i].N, a[i].K,
                                          EpiGated<XT, YT>{a[i].b, xs[i], a[i].gate, ys[i], a[i].M, a[i].N}};
  return launch_gemm_group(ps, np, st);
}

hipError_t launch_gated_f32out_group(const GatedArgs* a, float* const* y32, int np, hipStream_t st) {
  const bf16_t* xs[2] = {a[0].x, np > 1 ? a[1].x : nullptr};
  return gated_typed_group<bf16_t, float>(a, np, xs, y32, st);
}

hipError_t launch_gated_f32in_group(const GatedArgs* a, const float* const* x32, int np, hipStream_t st) {
  bf16_t* ys[2] = {a[0].y, np > 1 ? a[1].y : nullptr};
  return gated_typed_group<float, bf16_t>(a, np, x32, ys, st);
}

}  // namespace dit

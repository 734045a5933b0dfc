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
// Design: one workgroup of 8 wavefronts owns a BM x BN output tile; two
// groups of 4 waves each own half of it.  K is walked in BK = 32 slices
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
// only on the columns, store() finishes and writes one row's 4 values.
struct Cols4 {
  f32x4 a, b;
};
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
  const bf16_t* bias;
  bf16_t* qkv;
  bf16_t* cat;
  int M, N, split, d, ld_qkv, ld_cat, gelu_col0;
  __device__ __forceinline__ Cols4 col(int col0) const {
    Cols4 c;
    c.a = (bias && col0 < N) ? load_bf4(bias + col0) : f32x4{0.f, 0.f, 0.f, 0.f};
    return c;
  }
  __device__ __forceinline__ void store(int row, int col0, const Cols4& c, const f32x4& v) const {
    if (row >= M || col0 >= N) return;  // N and split are multiples of 64
    f32x4 z = v + c.a;
    if (col0 < split) {
      store_bf4(qkv + size_t(row) * ld_qkv + col0, z);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = gelu_tanh(z[i]);
      store_bf4(cat + size_t(row) * ld_cat + gelu_col0 + (col0 - split), z);
    }
  }
};

// linear1 whose q and k columns also get the per-head RMSNorm (weights qw,
// kw over the 128 dims of a head) and the RoPE rotation of adjacent dim
// pairs (tables [S, 64]) before they are stored: the whole head of a row is
// in one wave when the wave owns 128 columns (the 256x256 tile).
struct EpiLinear1QK : EpiLinear1 {
  static constexpr bool kHeadNorm = true;
  const float* qw;
  const float* kw;
  const float* rcos;
  const float* rsin;
  float eps;
  // Rows row_base + 16 i (i < FM) of the 128-column head starting at column
  // colw (< 2d); lane columns 4*fk + 16 j + (0..3) of block j.
  template <int FM, int FN>
  __device__ __forceinline__ void store_head(int row_base, int colw, int fk, const f32x4 (&acc)[FM][FN]) const {
    static_assert(FN == 8, "one head of 128 columns per wave");
    const float* w = colw < d ? qw : kw;
    f32x4 wv[FN], bv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = j * 16 + 4 * fk;  // column inside the head
      wv[j] = *reinterpret_cast<const f32x4*>(w + c);
      bv[j] = bias ? load_bf4(bias + colw + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = row_base + 16 * i;
      const int rc = min(row, M - 1);
      f32x4 z[FN];
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        z[j] = acc[i][j] + bv[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(z[j][e], z[j][e], ss);
      }
      // the row's 128 values sit in lanes fr + 16 fk, fk = 0..3
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float r = __frsqrt_rn(ss * (1.0f / 128.0f) + eps);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = j * 16 + 4 * fk;
        const f32x2 cs = *reinterpret_cast<const f32x2*>(rcos + size_t(rc) * 64 + c / 2);
        const f32x2 sn = *reinterpret_cast<const f32x2*>(rsin + size_t(rc) * 64 + c / 2);
        f32x4 n;
#pragma unroll
        for (int e = 0; e < 4; ++e) n[e] = z[j][e] * r * wv[j][e];
        f32x4 o;
        o[0] = n[0] * cs[0] - n[1] * sn[0];
        o[1] = n[0] * sn[0] + n[1] * cs[0];
        o[2] = n[2] * cs[1] - n[3] * sn[1];
        o[3] = n[2] * sn[1] + n[3] * cs[1];
        if (row < M) store_bf4(qkv + size_t(row) * ld_qkv + colw + c, o);
      }
    }
  }
};

struct EpiLinear2 {
  static constexpr bool kHeadNorm = false;
  const bf16_t* bias;
  const bf16_t* x;
  const float* gate;
  bf16_t* y;
  int M, N;
  __device__ __forceinline__ Cols4 col(int col0) const {
    Cols4 c;
    c.a = (bias && col0 < N) ? load_bf4(bias + col0) : f32x4{0.f, 0.f, 0.f, 0.f};
    c.b = col0 < N ? *reinterpret_cast<const f32x4*>(gate + col0) : f32x4{0.f, 0.f, 0.f, 0.f};
    return c;
  }
  __device__ __forceinline__ void store(int row, int col0, const Cols4& c, const f32x4& v) const {
    if (row >= M || col0 >= N) return;
    const size_t o = size_t(row) * N + col0;
    const f32x4 xv = load_bf4(x + o);
    f32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = fmaf(c.b[i], v[i] + c.a[i], xv[i]);
    store_bf4(y + o, z);
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
  const bf16_t* bias;
  const XT* x;
  const float* gate;
  YT* y;
  int M, N;
  __device__ __forceinline__ Cols4 col(int col0) const {
    Cols4 c;
    c.a = (bias && col0 < N) ? load_bf4(bias + col0) : f32x4{0.f, 0.f, 0.f, 0.f};
    c.b = col0 < N ? *reinterpret_cast<const f32x4*>(gate + col0) : f32x4{0.f, 0.f, 0.f, 0.f};
    return c;
  }
  __device__ __forceinline__ void store(int row, int col0, const Cols4& c, const f32x4& v) const {
    if (row >= M || col0 >= N) return;
    const size_t o = size_t(row) * N + col0;
    const f32x4 xv = load4(x + o);
    f32x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = fmaf(c.b[i], v[i] + c.a[i], xv[i]);
    store4(y + o, z);
  }
};

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
  if constexpr (Epi::kHeadNorm && C::WN == 128) {
    const int colw = n0 + wn * C::WN;  // a whole head: q or k columns get normalised and rotated
    if (colw < 2 * epi.d) {
      epi.template store_head<C::FM, C::FN>(m0 + wm * C::WM + fr, colw, fk, acc);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int col0 = n0 + wn * C::WN + j * 16 + 4 * fk;
    const Cols4 c = epi.col(col0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) epi.store(m0 + wm * C::WM + i * 16 + fr, col0, c, acc[i][j]);
  }
}

// ------------------------------------------------------------------ tile choice
using T288x192 = TileCfg<288, 192, 2, 4, 4>;  // 8 waves of 144 x 48; groups own 144-row halves
using T256 = TileCfg<256, 256, 4, 2, 4>;      // 8 waves of 64 x 128; groups own 128-row halves
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

enum TileKind { K288x192 = 0, K256 = 1, K128 = 2 };

// Pick the tile that minimises rounds-of-workgroups x tile area / efficiency
// (a proxy for the time of the busiest CU) over the tiles of all problems of
// one launch.
static TileKind choose_tile(const int* Ms, const int* Ns, int np) {
  const int cus = num_cus();
  struct Opt { TileKind k; int bm, bn; double eff; } opts[] = {
      // per-tile efficiency measured at the Flux shape (288x192 waves hold a
      // thinner 144 x 48 sub-tile and run at 0.87 of the 256x256 rate)
      {K288x192, 288, 192, 0.87}, {K256, 256, 256, 1.0}, {K128, 128, 128, 0.6}};
  TileKind best = K128;
  double best_cost = 1e300;
  for (const Opt& o : opts) {
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
    case K256: return launch_tile_group<T256>(ps, np, st);
    default: return launch_tile_group<T128>(ps, np, st);
  }
}

template <class Epi>
static hipError_t launch_gemm(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& e,
                              hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (choose_tile(M, N)) {
    case K288x192: return launch_tile<T288x192>(A, B, M, N, K, e, st);
    case K256: return launch_tile<T256>(A, B, M, N, K, e, st);
    default: return launch_tile<T128>(A, B, M, N, K, e, st);
  }
}

hipError_t launch_linear1(const bf16_t* u, const bf16_t* w1, const bf16_t* b1, bf16_t* qkv,
                          bf16_t* cat, int S, int d, int mlp, hipStream_t st) {
  EpiLinear1 e{b1, qkv, cat, S, 3 * d + mlp, 3 * d, d, 3 * d, d + mlp, d};
  return launch_gemm(u, w1, S, 3 * d + mlp, d, e, st);
}

bool linear1_fuses_qk(int S, int d, int mlp, int DH) {
  return DH == 128 && S > 0 && choose_tile(S, 3 * d + mlp) == K256;
}

hipError_t launch_linear1_qk(const bf16_t* u, const bf16_t* w1, const bf16_t* b1, bf16_t* qkv, bf16_t* cat,
                             int S, int d, int mlp, const float* qw, const float* kw, const float* rcos,
                             const float* rsin, float eps, hipStream_t st) {
  if (!linear1_fuses_qk(S, d, mlp, 128)) return hipErrorInvalidValue;
  EpiLinear1QK e;
  static_cast<EpiLinear1&>(e) = EpiLinear1{b1, qkv, cat, S, 3 * d + mlp, 3 * d, d, 3 * d, d + mlp, d};
  e.qw = qw;
  e.kw = kw;
  e.rcos = rcos;
  e.rsin = rsin;
  e.eps = eps;
  return launch_tile<T256>(u, w1, S, 3 * d + mlp, d, e, st);
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
  if (DH != 128 || np < 1 || np > 2) return false;
  int Ms[2], Ns[2];
  for (int i = 0; i < np; ++i) {
    if (a[i].qk_dim % 128 != 0 || 2 * a[i].qk_dim > a[i].n_plain) return false;
    Ms[i] = a[i].M;
    Ns[i] = a[i].N;
  }
  return choose_tile(Ms, Ns, np) == K256;
}

hipError_t launch_bias_act_qk_group(const BiasActArgs* a, const QKNormArgs* q, int np, hipStream_t st) {
  if (!bias_act_fuses_qk(a, np, 128)) return hipErrorInvalidValue;
  GemmProblem<EpiLinear1QK> ps[2];
  for (int i = 0; i < np; ++i) {
    EpiLinear1QK e;
    static_cast<EpiLinear1&>(e) = bias_act_epi(a[i]);
    e.qw = q[i].qw;
    e.kw = q[i].kw;
    e.rcos = q[i].rcos;
    e.rsin = q[i].rsin;
    e.eps = q[i].eps;
    ps[i] = GemmProblem<EpiLinear1QK>{a[i].A, a[i].W, a[i].M, a[i].N, a[i].K, e};
  }
  return launch_tile_group<T256>(ps, np, st);
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

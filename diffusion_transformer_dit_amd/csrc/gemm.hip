// bf16 GEMMs of the single-stream block on gfx950 matrix cores, with the
// elementwise tails fused into the epilogue:
//   linear1:  z = u W1^T + b1; q|k|v columns -> qkv, mlp columns -> GELU -> cat
//   linear2:  y = x + gate * (cat W2^T + b2)
// Both operands are K-contiguous ([rows, K] row-major, the nn.Linear layout
// for the weight), C = A B^T.  The Flux page (ChituDiffusion, sections 2 and
// 3.2) finds these GEMMs dominating the block's timeline before and after
// fusion; the elementwise work around them is what its section 1.1 fuses.
//
// Design: one workgroup of 4 wavefronts owns a BM x BN output tile; K is
// walked in BK = 64 slices staged through LDS (double buffered, 16-byte
// chunks, XOR-swizzled so that both the 16-byte stores and the MFMA operand
// reads are bank-conflict free).  Each wave computes a WM x WN sub-tile with
// v_mfma_f32_16x16x32_bf16, fp32 accumulators; the next slice's global loads
// are in flight while the current slice is multiplied.  Tiles are numbered
// so that the tiles resident on one XCD (blocks are dealt round-robin over
// the 8 XCDs) form a compact 2D patch sharing A and B panels in that XCD's L2.
#include "dit_common.hpp"
#include "launch.hpp"

namespace dit {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_LD = BM * 8 / NT;  // 16-byte chunks per thread per slice
  static constexpr int B_LD = BN * 8 / NT;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile rows must split over threads");
};

// Byte offset of 16-byte chunk `c` (0..7) of row `r` inside an LDS slice whose
// rows are 64 bf16 (128 bytes): chunk positions are XOR-swizzled by row.
__device__ __forceinline__ uint32_t lds_off(int r, int c) {
  return uint32_t(r) * 128u + (uint32_t(c ^ (r & 7)) << 4);
}

struct EpiLinear1 {
  const bf16_t* bias;
  bf16_t* qkv;
  bf16_t* cat;
  int M, N, split, d, ld_qkv, ld_cat;
  __device__ __forceinline__ void operator()(int row0, int col, const f32x4& v) const {
    if (col >= N) return;
    const float b = bias ? bf2f(bias[col]) : 0.f;
    if (col < split) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (row0 + i < M) qkv[size_t(row0 + i) * ld_qkv + col] = bf16_t(f2bf_bits(v[i] + b));
    } else {
      const int cc = d + (col - split);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (row0 + i < M) cat[size_t(row0 + i) * ld_cat + cc] = bf16_t(f2bf_bits(gelu_tanh(v[i] + b)));
    }
  }
};

struct EpiLinear2 {
  const bf16_t* bias;
  const bf16_t* x;
  const float* gate;
  bf16_t* y;
  int M, N;
  __device__ __forceinline__ void operator()(int row0, int col, const f32x4& v) const {
    if (col >= N) return;
    const float b = bias ? bf2f(bias[col]) : 0.f;
    const float g = gate[col];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (row0 + i < M) {
        const size_t o = size_t(row0 + i) * N + col;
        y[o] = bf16_t(f2bf_bits(bf2f(x[o]) + g * (v[i] + b)));
      }
    }
  }
};

// Map the linear block id to a (tile_m, tile_n) pair.  Hardware deals block b
// to XCD b % 8; consecutive ids on one XCD are regrouped into GROUP_M-tall
// column-major patches of tiles.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int group = GROUP_M * tiles_n;
  const int g = bid / group;
  const int first_m = g * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in = bid - g * group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

template <class C, class Epi>
__global__ void __launch_bounds__(C::NT, 1)
gemm_bf16_tn_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, int M, int N,
                    int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_coords<4>(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  // global -> LDS chunk assignment: chunk q = tid + i*NT, row q/8, column chunk q%8.
  const int lc = tid & 7;
  const int lr = tid >> 3;
  constexpr int RSTEP = C::NT / 8;
  const bf16_t* ga[C::A_LD];
  const bf16_t* gb[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int r = min(m0 + lr + i * RSTEP, M - 1);  // rows past M are clamped; never stored
    ga[i] = A + size_t(r) * K + lc * 8;
  }
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    const int r = min(n0 + lr + i * RSTEP, N - 1);
    gb[i] = B + size_t(r) * K + lc * 8;
  }
  uint32_t la[C::A_LD], lb[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) la[i] = lds_off(lr + i * RSTEP, lc);
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) lb[i] = C::A_BYTES + lds_off(lr + i * RSTEP, lc);

  u32x4 ra[C::A_LD], rb[C::B_LD];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i] + kt * C::BK);
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i] + kt * C::BK);
  };
  auto lstore = [&](int stage) {
    unsigned char* s = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) *reinterpret_cast<u32x4*>(s + la[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) *reinterpret_cast<u32x4*>(s + lb[i]) = rb[i];
  };

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand read offsets: lane holds row (lane & 15) of a 16-row fragment and
  // the 8 K-values of chunk (lane >> 4) of the current 32-wide K step.
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const uint32_t a_row = uint32_t(wm * C::WM + fr) * 128u;
  const uint32_t b_row = C::A_BYTES + uint32_t(wn * C::WN + fr) * 128u;

  const int KT = K / C::BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const unsigned char* s = smem + cur * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const uint32_t sw = uint32_t(((ks * 4 + fk) ^ (fr & 7)) << 4);
      bf16x8 a[C::FM], b[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(s + a_row + i * 16 * 128 + sw);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(s + b_row + j * 16 * 128 + sw);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // C fragment layout (16x16): lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      epi(m0 + wm * C::WM + i * 16 + 4 * fk, n0 + wn * C::WN + j * 16 + fr, acc[i][j]);
}

// ------------------------------------------------------------------ tile choice
using T288x192 = TileCfg<288, 192, 2, 2>;
using T256 = TileCfg<256, 256, 2, 2>;
using T128 = TileCfg<128, 128, 2, 2>;

static int num_cus() {
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

// Pick the tile that minimises rounds-of-workgroups x tile area (a proxy for
// the time of the busiest CU); small tiles pay a fixed efficiency penalty.
static TileKind choose_tile(int M, int N) {
  const int cus = num_cus();
  struct Opt { TileKind k; int bm, bn; double eff; } opts[] = {
      {K288x192, 288, 192, 1.0}, {K256, 256, 256, 1.0}, {K128, 128, 128, 0.75}};
  TileKind best = K128;
  double best_cost = 1e300;
  for (const Opt& o : opts) {
    const long long tiles = (long long)((M + o.bm - 1) / o.bm) * ((N + o.bn - 1) / o.bn);
    const long long rounds = (tiles + cus - 1) / cus;
    const double cost = double(rounds) * o.bm * o.bn / o.eff;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = o.k;
    }
  }
  return best;
}

template <class C, class Epi>
static hipError_t launch_tile(const bf16_t* A, const bf16_t* B, int M, int N, int K, const Epi& e,
                              hipStream_t st) {
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  gemm_bf16_tn_kernel<C, Epi><<<tiles, C::NT, 0, st>>>(A, B, M, N, K, e);
  return hipGetLastError();
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
  EpiLinear1 e{b1, qkv, cat, S, 3 * d + mlp, 3 * d, d, 3 * d, d + mlp};
  return launch_gemm(u, w1, S, 3 * d + mlp, d, e, st);
}

hipError_t launch_linear2(const bf16_t* cat, const bf16_t* w2, const bf16_t* b2, const bf16_t* x,
                          const float* gate, bf16_t* y, int S, int d, int mlp, hipStream_t st) {
  EpiLinear2 e{b2, x, gate, y, S, d};
  return launch_gemm(cat, w2, S, d, d + mlp, e, st);
}

}  // namespace dit

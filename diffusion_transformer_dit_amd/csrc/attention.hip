// Exact softmax attention of the single-stream block (no mask, scale
// 1/sqrt(Dh)) on gfx950 matrix cores: the flash / sdpa backends of the Flux
// page (ChituDiffusion, sections 2 and 4) and the fp32 softmax the Wan2.1
// video page (mhpq.cn, section 5.1) recommends, as one LDS-tiled online-
// softmax kernel.
//
// One workgroup = 8 wavefronts = 256 queries of one head, one workgroup per
// CU (4 wavefronts = 128 queries, two per CU, when the 8-wave grid would
// leave CUs idle); each wave owns 32 queries.  K and V stream through LDS in
// tiles of 64 tokens, double buffered, filled by direct buffer->LDS loads (buffer_load_dwordx4 ... lds,
// no VALU address work per load) issued one tile ahead.  Both tiles keep the
// token-major layout of qkv (rows of Dh bf16) with 16-byte chunks
// XOR-swizzled by row.  Per tile and wave, in two halves of 32 keys:
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16 (Q stays in registers), so
//                 every lane holds scores of ONE query: a row max needs one
//                 exchange between lanes l and l^32 (v_permlane32_swap);
//   online softmax in fp32 with exp2 and the 1/sqrt(Dh)*log2(e) scale folded
//                 into one FMA, against a running max that is only
//                 recomputed when the probabilities grow past 2^8; P is
//                 packed to bf16 (v_cvt_pk_bf16_f32) and the denominator
//                 sums the packed values, so the output is a convex
//                 combination of V rows with exactly the weights applied;
//   O^T += V^T P^T, where the P^T operand comes straight from the S^T
//                 accumulator registers and the V^T operand is read from the
//                 token-major V tile with ds_read_b64_tr_b16 (a transposing
//                 LDS read: lane i of a 16-lane group receives element i of
//                 four consecutive rows).  The key order inside each 16-key
//                 MFMA step is permuted identically on both operands, which
//                 leaves the contraction unchanged.
// The MFMAs of one half are issued between the softmax instructions of the
// other, so a wave's matrix-core work overlaps its own VALU work.
#include <type_traits>

#include "dit_common.hpp"
#include "launch.hpp"
#include "mod_gemv.hpp"

namespace dit {

constexpr int ATT_BN = 64;  // keys per tile
// VALU (and transcendental) instructions of a half's softmax issued after
// each MFMA of the other half's QK product, and after each MFMA of its PV
// product (the interleave of the tile body below)
constexpr int kValuPerQK = 9, kValuPerPV = 12;

template <int DH>
struct AttCfg {
  static constexpr int ROW = DH * 2;                // bytes per token row
  static constexpr int TILE = ATT_BN * ROW;         // one K or V tile
  static constexpr int STAGE = 2 * TILE;            // K tile then V tile
  static constexpr int KCH = DH / 8;                // 16-byte chunks per row
  static_assert(KCH == 8 || KCH == 16, "head_dim 64 or 128");
};

// Chunk swizzles.  K is read 16 rows x one chunk per 256 bytes of LDS banks,
// so the 16 rows of a read phase must land on 16 distinct chunk positions;
// V is read 4 rows x one 64-byte group, so the 4 rows must land on distinct
// 64-byte bank groups.
template <int KCH>
__device__ __forceinline__ int k_swz(int row) { return KCH == 16 ? (row & 15) : ((row >> 1) & 7); }
template <int KCH>
__device__ __forceinline__ int v_swz(int row) { return KCH == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;

// Buffer descriptor over `bytes` bytes from `base` (raw, 32-bit data format):
// loads at offsets past the range read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
// 16 bytes per lane from a buffer straight into LDS: lane i writes lds_block + 16 i
__device__ __forceinline__ void buffer_load_lds_16(__amdgpu_buffer_rsrc_t r, unsigned char* lds_block, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_block, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ u32x2 read_tr16(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p));
}
// pairwise sum of 16 values (a tree of depth 4 instead of a serial chain)
__device__ __forceinline__ float sum16(const float* e) {
  float s8[8], s4[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = e[2 * i] + e[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = s8[2 * i] + s8[2 * i + 1];
  return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}
// P in bf16 for the PV product: packs the 16 probabilities of a lane
// (p[0] = keys of the first 16-key step, p[1] of the second) and returns the
// sum of the ROUNDED values, so that the denominator is the sum of the exact
// weights the matrix cores multiply V by.  The sum is taken on the packed
// pairs by v_dot2c_f32_bf16 against (1, 1): one instruction per pair.
__device__ __forceinline__ float pack_p(const float* e, u32x4* p) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w = pack_bf2(e[8 * half + 2 * t], e[8 * half + 2 * t + 1]);
      p[half][t] = w;
      s[t & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, s[t & 1], false);
    }
  return s[0] + s[1];
}
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// Online-softmax state of one lane after a range of keys: the O^T
// accumulators (registers 4g..4g+3 of oacc[b] hold dims b*32 + 8g + 4hh +
// (0..3) of the lane's query, hh = lane / 32), the running max of the raw
// scores (the same in lanes l and l^32) and this lane's share of the
// softmax denominator (lanes l and l^32 hold the two halves).
template <int DH>
struct AttState {
  f32x16 oacc[DH / 32];
  float m_run, l_run;
};

// One wave's 32 queries (this lane's query row qc, clamped to S - 1 by the
// caller) of head `head` against the keys [kv_begin, kv_end), streamed
// through the two K/V stages in `smem`.  Ends after a workgroup barrier with
// every LDS read done, so the caller may start another range at once.
template <int DH, int NW>
__device__ __forceinline__ void att_range(const bf16_t* __restrict__ qkv, unsigned char* smem, int H, int head,
                                          int qc, int kv_begin, int kv_end, float c_log2, AttState<DH>& state) {
  using C = AttCfg<DH>;
  constexpr int LPW = ATT_BN * C::KCH / 64 / NW;  // 1 KB wave-loads per wave per tile
  constexpr int KCH = C::KCH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS targets stay scalar
  const int d = H * DH;
  const int ld = 3 * d;
  const bf16_t* Qg = qkv + head * DH;

  const int ql = lane & 31;  // query column of this lane
  const int hh = lane >> 5;  // lane half

  // Q^T operand: 8 dims (16*s + 8*hh ..) of this lane's query for each K-step s.
  bf16x8 qf[DH / 16];
#pragma unroll
  for (int s = 0; s < DH / 16; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(Qg + size_t(qc) * ld + 16 * s + 8 * hh);

  // ---- tile loads: wave-load w of a tile fills LDS chunks [64w, 64w + 64);
  // chunk p holds row p / KCH, global chunk (p % KCH) ^ swz(row).
  // Byte offsets of this lane's chunks inside a tile (rows = tokens of the
  // tile).  Each tile gets a descriptor whose range ends with the tile or
  // with the key range, whichever comes first, so the rows of a ragged last
  // tile past it read as zero: their scores are masked to -inf and their V
  // rows meet zero probabilities.  (The range is at most 64 rows, so its
  // 32-bit byte count cannot wrap even when q|k|v spans more than 4 GiB.)
  int koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int p = (wave * LPW + i) * 64 + lane;
    const int row = p / KCH, cp = p % KCH;
    koff[i] = (row * ld + d + head * DH + 8 * (cp ^ k_swz<KCH>(row))) * 2;
    voff[i] = (row * ld + 2 * d + head * DH + 8 * (cp ^ v_swz<KCH>(row))) * 2;
  }
  auto issue = [&](int t0, int stage) {
    unsigned char* sK = smem + stage * C::STAGE;
    unsigned char* sV = sK + C::TILE;
    const uint32_t rows = uint32_t(min(kv_end - t0, ATT_BN));
    const __amdgpu_buffer_rsrc_t r = make_rsrc(qkv + size_t(t0) * ld, rows * uint32_t(ld) * 2u);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int w = wave * LPW + i;
      buffer_load_lds_16(r, sK + w * 1024, koff[i]);
      buffer_load_lds_16(r, sV + w * 1024, voff[i]);
    }
  };

  // LDS read offsets of this lane (bytes within a stage).
  // K (A operand of S^T): row kb*32 + ql, chunk 2s + hh.
  int kaddr[DH / 16];
#pragma unroll
  for (int s = 0; s < DH / 16; ++s) kaddr[s] = ql * C::ROW + (((2 * s + hh) ^ k_swz<KCH>(ql)) << 4);
  // V (A operand of O^T via the transposing read): lane j of 16-lane group g
  // points at row 4*(g >> 1) + (j >> 2) (+ 16m, + 8 for the second read) and
  // dims 32b + 16*(g & 1) + 4*(j & 3).
  const int g = lane >> 4, j = lane & 15;
  const int vrow = 4 * (g >> 1) + (j >> 2);
  int vaddr[DH / 32];
#pragma unroll
  for (int b = 0; b < DH / 32; ++b) {
    const int dim = 32 * b + 16 * (g & 1) + 4 * (j & 3);
    vaddr[b] = C::TILE + vrow * C::ROW + (((dim >> 3) ^ v_swz<KCH>(vrow)) << 4) + 2 * (dim & 7);
  }

  f32x16 (&oacc)[DH / 32] = state.oacc;
#pragma unroll
  for (int b = 0; b < DH / 32; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float& m_run = state.m_run;  // running max of raw scores of this lane's query
  float& l_run = state.l_run;  // this lane's share of the running softmax denominator
  m_run = -1e30f;
  l_run = 0.f;

  const int ntiles = (kv_end - kv_begin + ATT_BN - 1) / ATT_BN;
  issue(kv_begin, 0);
  wait_all();
  __syncthreads();

  // S^T of one 32-key half kb of a staged tile: accumulator register i holds
  // key 32*kb + 8*(i/4) + 4*hh + (i%4) of the tile for this lane's query.
  auto scores = [&](const unsigned char* st, int kb) {
    bf16x8 kf[DH / 16];
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(st + kb * 32 * C::ROW + kaddr[s]);
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
    return sacc;
  };
  // keys at or past kv_end (ragged last tile only) score -inf
  auto mask_tail = [&](f32x16& sacc, int key0, int kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (key0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3) >= kv_end) sacc[i] = -INFINITY;
  };
  // Online-softmax update for one half, in two parts so that the common
  // path has no branch: softmax_exp packs the bf16 probabilities against
  // the running max into pk and returns this lane's sum of them;
  // softmax_fix then handles the rare case where the max must move.  The
  // max of the scores is only taken when some lane's 16 probabilities sum
  // past 2^8 (or overflow), i.e. a score rose well above the running max
  // (always on the first tile).  Keeping a stale max is exact: numerator and
  // denominator share it, and values up to 2^8 cannot overflow the fp32 sums.
  auto softmax_exp = [&](const f32x16& sacc, u32x4 (&pk)[2]) {
    float e[16];
    const float mc = m_run * c_log2;
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = exp2_fast(fmaf(sacc[i], c_log2, -mc));
    return pack_p(e, pk);
  };
  auto softmax_fix = [&](const f32x16& sacc, u32x4 (&pk)[2], float hs) {
    if (__builtin_amdgcn_ballot_w64(!(hs <= 256.0f))) {
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = xor32_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast((m_run - m_new) * c_log2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DH / 32; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
      hs = softmax_exp(sacc, pk);
    }
    l_run += hs;
  };
  // O^T += V^T P^T over the two 16-key steps of half kb; step m covers keys
  // 16m + 4hh + (0..3) and 16m + 8 + 4hh + (0..3) of the tile.
  auto pv = [&](const unsigned char* st, int kb, const u32x4 (&pk)[2]) {
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      const int m = 2 * kb + mh;
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pk[mh]);
#pragma unroll
      for (int b = 0; b < DH / 32; ++b) {
        const u32x2 lo = read_tr16(st + vaddr[b] + (16 * m) * C::ROW);
        const u32x2 hi = read_tr16(st + vaddr[b] + (16 * m + 8) * C::ROW);
        u32x4 av;
        av[0] = lo[0];
        av[1] = lo[1];
        av[2] = hi[0];
        av[3] = hi[1];
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pf, oacc[b], 0, 0, 0);
      }
    }
  };
  // One K/V tile; the stage is a compile-time constant (the loop below runs
  // tiles in pairs), so every LDS read address is a per-lane base plus an
  // immediate offset, with no per-tile address arithmetic.  The scores of
  // the second half are issued before the softmax of the first, and the PV
  // product of the first half before the softmax of the second, so that the
  // matrix cores work on one half while the VALU exponentiates the other;
  // the arithmetic, and its order on every accumulator, is that of the
  // plain sequence (scores, softmax, PV per half).
  auto tile = [&](int jt, auto stage_c, auto ragged_c) {
    constexpr int cur = decltype(stage_c)::value;
    constexpr bool ragged = decltype(ragged_c)::value;
    if (jt + 1 < ntiles) issue(kv_begin + (jt + 1) * ATT_BN, cur ^ 1);
    const unsigned char* st = smem + cur * C::STAGE;
    const int key0 = kv_begin + jt * ATT_BN;
    f32x16 s0 = scores(st, 0);
    if constexpr (ragged) mask_tail(s0, key0, 0);
    f32x16 s1 = scores(st, 1);
    u32x4 p0[2], p1[2];
    float hs = softmax_exp(s0, p0);
    // issue order: the 16 K reads and half 0's MFMAs, then half 1's MFMAs
    // each followed by a share of half 0's exponentials
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x402, kValuPerQK, 0);  // VALU + transcendental
    }
    softmax_fix(s0, p0, hs);
    if constexpr (ragged) mask_tail(s1, key0, 1);
    pv(st, 0, p0);
    hs = softmax_exp(s1, p1);
    // half 0's PV MFMAs, each after its two V reads and followed by a
    // share of half 1's exponentials
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS transposing reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x402, kValuPerPV, 0);  // VALU + transcendental
    }
    softmax_fix(s1, p1, hs);
    pv(st, 1, p1);
    wait_all();
    __syncthreads();
  };
  // every tile but a ragged last one takes the unmasked path
  const int nfull = (kv_end - kv_begin) / ATT_BN;
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  using F = std::false_type;
  int jt = 0;
  for (; jt + 1 < nfull; jt += 2) {
    tile(jt, Z{}, F{});
    tile(jt + 1, O{}, F{});
  }
  if (jt < nfull) {
    tile(jt, Z{}, F{});
    if (jt + 1 < ntiles) tile(jt + 1, O{}, std::true_type{});
  } else if (jt < ntiles) {
    tile(jt, Z{}, std::true_type{});
  }
}

// bf16 output row of the lane's query: registers 4g..4g+3 of oacc[b] hold
// dims b*32 + 8g + 4hh + (0..3), scaled by the reciprocal denominator.
template <int DH>
__device__ __forceinline__ void att_store_bf16(const f32x16 (&oacc)[DH / 32], float inv, bf16_t* orow, int hh) {
#pragma unroll
  for (int b = 0; b < DH / 32; ++b)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      u32x2 w;
      w[0] = pack_bf2(oacc[b][4 * gg] * inv, oacc[b][4 * gg + 1] * inv);
      w[1] = pack_bf2(oacc[b][4 * gg + 2] * inv, oacc[b][4 * gg + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + b * 32 + 8 * gg + 4 * hh) = w;
    }
}

// PARTIAL: attend to keys [kv_begin, kv_end) only and write the chunk's
// normalised output in fp32 to out_f32 [S, H*DH] and its log-sum-exp (natural
// log) to lse [H, S], the per-hop step of ring attention; otherwise write
// bf16 to out (row stride ld_out) over all keys.
// With PARTIAL, blockIdx.z selects one of gridDim.z consecutive key chunks
// of kv_chunk tokens inside [kv_begin, kv_end) and its output slices
// (out_f32 + z*S*H*DH, lse + z*H*S): a split of the keys over more
// workgroups when one workgroup per query block and head cannot fill the chip.
// NW waves per workgroup (32 NW queries): 8 (one workgroup per CU) or 4 (two).
template <int DH, bool PARTIAL, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
attention_fwd_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out, float* __restrict__ out_f32,
                     float* __restrict__ lse, int S, int H, int ld_out, float c_log2, int kv_begin,
                     int kv_end, int kv_chunk, int xcd_remap) {
  using C = AttCfg<DH>;
  constexpr int BM = 32 * NW;                      // queries per workgroup
  if constexpr (PARTIAL) {
    const int z = blockIdx.z;
    kv_begin += z * kv_chunk;
    kv_end = min(kv_end, kv_begin + kv_chunk);
    out_f32 += size_t(z) * S * H * DH;
    lse += size_t(z) * H * S;
  }
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * C::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // (query block, head) from the linear block id; with xcd_remap the ids are
  // remapped so that the workgroups one XCD runs at a time (blocks are dealt
  // round-robin to the 8 XCDs) are consecutive query blocks of the same few
  // heads, whose K and V then stay in that XCD's 4 MB L2 (the launchers set
  // it when one head's K and V fit in 4 MB: +2-3 % at the Flux shape, -1.5 %
  // at S = 16384 where they do not).
  int bid = blockIdx.x + blockIdx.y * gridDim.x;
  const int nb = gridDim.x * gridDim.y;
  if (xcd_remap && (nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int qblock = bid % gridDim.x;
  const int head = bid / gridDim.x;
  const int d = H * DH;
  const int q = qblock * BM + wave * 32 + (lane & 31);
  const int hh = lane >> 5;
  AttState<DH> st;
  att_range<DH, NW>(qkv, smem, H, head, min(q, S - 1), kv_begin, kv_end, c_log2, st);
  const f32x16 (&oacc)[DH / 32] = st.oacc;
  const float m_run = st.m_run, l_run = st.l_run;

  const float l_tot = xor32_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (q < S) {
    if constexpr (PARTIAL) {
      float* orow = out_f32 + size_t(q) * d + head * DH;
#pragma unroll
      for (int b = 0; b < DH / 32; ++b)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          // registers 4gg..4gg+3 hold dims b*32 + 8gg + 4hh + (0..3)
          const f32x4 w = {oacc[b][4 * gg] * inv, oacc[b][4 * gg + 1] * inv, oacc[b][4 * gg + 2] * inv,
                           oacc[b][4 * gg + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + b * 32 + 8 * gg + 4 * hh) = w;
        }
      // scores in exp2 units are s * log2(e)/sqrt(Dh): lse = (m c + log2 l) ln 2
      if (hh == 0) lse[size_t(head) * S + q] = (m_run * c_log2 + __log2f(l_tot)) * 0.6931471805599453f;
    } else {
      att_store_bf16<DH>(oacc, inv, out + size_t(q) * ld_out + head * DH, hh);
    }
  }
}

// The attention of attention_fwd_kernel<DH, false, 8> in workgroups
// [0, n_qb * H) and, in the workgroups after them, the modulation GEMVs of
// one or two matrices (the next block's, in a block stack).  Those
// workgroups are dispatched after every attention workgroup, so they run on
// the CUs that the attention's last, partial round of workgroups leaves idle
// (432 workgroups on 256 CUs at the Flux shape).  The GEMV rows' arithmetic
// is that of mod_gemv_multi_kernel.
template <int DH, int NCH>
__global__ void __launch_bounds__(512, 1)
attention_mod_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out, int S, int H, int ld_out,
                     float c_log2, int xcd_remap, int n_qb, const bf16_t* __restrict__ temb, ModTab2 tab,
                     float* __restrict__ mods, int rows_per_mat, int mod_rows, int mod_cols, int mod_rpw) {
  using C = AttCfg<DH>;
  static_assert(NCH * 512 * 4 <= 2 * C::STAGE, "SiLU(temb) must fit the K/V stages");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * C::STAGE];
  const int n_att = n_qb * H;
  if (int(blockIdx.x) >= n_att) {
    mod_gemv_rows<NCH>(temb, tab, mods, rows_per_mat, mod_rows, mod_cols, mod_rpw,
                       (int(blockIdx.x) - n_att) * 8 + int(threadIdx.x >> 6), reinterpret_cast<float*>(smem));
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int bid = blockIdx.x;
  if (xcd_remap && (n_att & 7) == 0) bid = (bid & 7) * (n_att >> 3) + (bid >> 3);
  const int qblock = bid % n_qb;
  const int head = bid / n_qb;
  const int q = qblock * 256 + wave * 32 + (lane & 31);
  const int hh = lane >> 5;
  AttState<DH> st;
  att_range<DH, 8>(qkv, smem, H, head, min(q, S - 1), 0, S, c_log2, st);
  const float l_tot = xor32_sum(st.l_run);
  const float inv = 1.0f / l_tot;
  if (q < S) att_store_bf16<DH>(st.oacc, inv, out + size_t(q) * ld_out + head * DH, hh);
}

// Merge of the partial results of disjoint key chunks: with
// lse = ln sum_c exp(lse_c), out = sum_c exp(lse_c - lse) o_c.  One thread
// owns 8 consecutive dims of one (token, head); the chunk weights are
// recomputed by each of the head's DH/8 threads, and the partial outputs are
// read four chunks at a time (all four loads in flight before the sums).
__global__ void __launch_bounds__(256)
attention_merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lses, int n_chunks, int S,
                       int H, int DH, bf16_t* __restrict__ out, int ld_out) {
  const int d = H * DH;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)S * (d / 8);
  if (gid >= total) return;
  const int t = int(gid / (d / 8));
  const int c8 = int(gid % (d / 8)) * 8;  // first of the 8 dims
  const int h = c8 / DH;
  const float* lrow = lses + size_t(h) * S + t;  // chunk c at lrow[c * H * S]
  const size_t lstep = size_t(H) * S;
  float mx = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) mx = fmaxf(mx, lrow[c * lstep]);
  float z = 0.f;
  for (int c = 0; c < n_chunks; ++c) z += exp2_fast((lrow[c * lstep] - mx) * kLog2e);
  const float lz = mx + __log2f(z) * 0.6931471805599453f;
  const float* orow = o_parts + size_t(t) * d + c8;  // chunk c at orow[c * S * d]
  const size_t ostep = size_t(S) * d;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n_chunks; c0 += 4) {
    f32x4 o0[4], o1[4];
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i < n_chunks) {
        const float* p = orow + (c0 + i) * ostep;
        o0[i] = *reinterpret_cast<const f32x4*>(p);
        o1[i] = *reinterpret_cast<const f32x4*>(p + 4);
        w[i] = exp2_fast((lrow[(c0 + i) * lstep] - lz) * kLog2e);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i < n_chunks) {
        acc0 += w[i] * o0[i];
        acc1 += w[i] * o1[i];
      }
  }
  // two 8-byte stores: ld_out need only be a multiple of 4
  u32x2 w0, w1;
  w0[0] = pack_bf2(acc0[0], acc0[1]);
  w0[1] = pack_bf2(acc0[2], acc0[3]);
  w1[0] = pack_bf2(acc1[0], acc1[1]);
  w1[1] = pack_bf2(acc1[2], acc1[3]);
  u32x2* dst = reinterpret_cast<u32x2*>(out + size_t(t) * ld_out + c8);
  dst[0] = w0;
  dst[1] = w1;
}

// one head's K and V fit in an XCD's 4 MB L2
static int att_remap(int S, int DH) { return (long long)S * DH * 2 * 2 <= (4ll << 20) ? 1 : 0; }

// One launch of n_chunks key chunks (1 for a plain attention) of `chunk`
// keys inside [kv_begin, kv_end).  Eight-wave workgroups (one per CU) load
// each K/V tile once for 256 queries instead of 128, which halves the tile
// loads a wave issues; they are used when their grid still gives every CU a
// workgroup, else the 4-wave kernel keeps twice as many workgroups in flight
// (a few heads, short sequences).
template <bool PARTIAL>
static hipError_t launch_fwd(const bf16_t* qkv, bf16_t* out, float* o_part, float* lse, int S, int H, int DH,
                             int ld_out, int kv_begin, int kv_end, int chunk, int n_chunks, hipStream_t st) {
  if (DH != 128 && DH != 64) return hipErrorInvalidValue;
  const float c = kLog2e / sqrtf(float(DH));
  const int rm = att_remap(chunk, DH);
  const bool wide = (long long)((S + 255) / 256) * H * n_chunks >= num_cus();
  const int nw = wide ? 8 : 4;
  dim3 grid((S + 32 * nw - 1) / (32 * nw), H, n_chunks), block(64 * nw);
#define DIT_ATT_LAUNCH(D, W)                                                                                    \
  attention_fwd_kernel<D, PARTIAL, W><<<grid, block, 0, st>>>(qkv, out, o_part, lse, S, H, ld_out, c, kv_begin, \
                                                              kv_end, chunk, rm)
  if (DH == 128) {
    if (wide) DIT_ATT_LAUNCH(128, 8);
    else DIT_ATT_LAUNCH(128, 4);
  } else {
    if (wide) DIT_ATT_LAUNCH(64, 8);
    else DIT_ATT_LAUNCH(64, 4);
  }
#undef DIT_ATT_LAUNCH
  return hipGetLastError();
}

// The attention launch carries the GEMV when it runs 8-wave workgroups, at
// least one per CU (unless their count is a multiple of the CU count, the
// last round then leaves CUs idle for the GEMV), and the GEMV's row length
// is one of the instantiated ones (16-byte chunks per lane: temb widths up
// to 8192).
static bool mod_nch_supported(int nch) {
  return nch == 1 || nch == 2 || nch == 3 || nch == 4 || nch == 6 || nch == 8 || nch == 10 || nch == 12 ||
         nch == 16;
}

bool attention_hosts_modulation(int S, int H, int DH, int mod_cols) {
  if (S <= 0 || (DH != 128 && DH != 64) || mod_cols <= 0 || mod_cols % 8 != 0) return false;
  if (!mod_nch_supported((mod_cols / 8 + 63) / 64)) return false;
  return (long long)((S + 255) / 256) * H >= num_cus();
}

template <int DH>
static hipError_t launch_att_mod(dim3 grid, int nch, const bf16_t* qkv, bf16_t* out, int S, int H, int ld_out,
                                 float c, int rm, int n_qb, const bf16_t* temb, const ModTab2& tab, float* mods,
                                 int rows_per_mat, int mod_rows, int mod_cols, int rpw, hipStream_t st) {
  switch (nch) {
#define DIT_ATT_MOD(N)                                                                                            \
  case N:                                                                                                         \
    attention_mod_kernel<DH, N><<<grid, dim3(512), 0, st>>>(qkv, out, S, H, ld_out, c, rm, n_qb, temb, tab, mods, \
                                                            rows_per_mat, mod_rows, mod_cols, rpw);               \
    break;
    DIT_ATT_MOD(1) DIT_ATT_MOD(2) DIT_ATT_MOD(3) DIT_ATT_MOD(4) DIT_ATT_MOD(6) DIT_ATT_MOD(8) DIT_ATT_MOD(10)
    DIT_ATT_MOD(12) DIT_ATT_MOD(16)
#undef DIT_ATT_MOD
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_mod(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out,
                                const bf16_t* temb, const bf16_t* w0, const bf16_t* b0, const bf16_t* w1,
                                const bf16_t* b1, int n_mats, float* mods, int rows_per_mat, int mod_cols,
                                hipStream_t st) {
  if (!attention_hosts_modulation(S, H, DH, mod_cols) || rows_per_mat <= 0 || n_mats < 1 || n_mats > 2)
    return hipErrorInvalidValue;
  const float c = kLog2e / sqrtf(float(DH));
  const int rm = att_remap(S, DH);
  const int n_qb = (S + 255) / 256;
  const int n_att = n_qb * H;
  const int mod_rows = n_mats * rows_per_mat;
  // 9 rows per wave: one block's GEMV (3 x 3072 rows) is 128 workgroups at the Flux width
  const int rpw = 9;
  const int n_mod = (mod_rows + 8 * rpw - 1) / (8 * rpw);
  ModTab2 tab;
  tab.ws[0] = w0;
  tab.ws[1] = w1;
  tab.bs[0] = b0;
  tab.bs[1] = b1;
  const int nch = (mod_cols / 8 + 63) / 64;
  const dim3 grid(n_att + n_mod);
  if (DH == 128)
    return launch_att_mod<128>(grid, nch, qkv, out, S, H, ld_out, c, rm, n_qb, temb, tab, mods, rows_per_mat,
                               mod_rows, mod_cols, rpw, st);
  return launch_att_mod<64>(grid, nch, qkv, out, S, H, ld_out, c, rm, n_qb, temb, tab, mods, rows_per_mat, mod_rows,
                            mod_cols, rpw, st);
}

hipError_t launch_attention(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out,
                            hipStream_t st) {
  if (S == 0) return hipSuccess;
  return launch_fwd<false>(qkv, out, nullptr, nullptr, S, H, DH, ld_out, 0, S, S, 1, st);
}

// n_chunks key chunks of ceil((kv_end - kv_begin) / n_chunks) tokens in one
// launch (every chunk non-empty: callers pass n_chunks from attention_chunks)
static hipError_t launch_partials(const bf16_t* qkv, int S, int H, int DH, int kv_begin, int kv_end, int n_chunks,
                                  float* o_part, float* lse, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const int chunk = (kv_end - kv_begin + n_chunks - 1) / n_chunks;
  return launch_fwd<true>(qkv, nullptr, o_part, lse, S, H, DH, 0, kv_begin, kv_end, chunk, n_chunks, st);
}

hipError_t launch_attention_partial(const bf16_t* qkv, int S, int H, int DH, int kv_begin, int kv_end,
                                    float* o_part, float* lse, hipStream_t st) {
  return launch_partials(qkv, S, H, DH, kv_begin, kv_end, 1, o_part, lse, st);
}

int attention_chunks(int S, int n_chunks) {
  if (S <= 0 || n_chunks <= 1) return 1;
  const int chunk = (S + n_chunks - 1) / n_chunks;
  return (S + chunk - 1) / chunk;
}

hipError_t launch_attention_split(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out, int n_chunks,
                                  float* o_parts, float* lses, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const int n = attention_chunks(S, n_chunks);
  hipError_t e = launch_partials(qkv, S, H, DH, 0, S, n, o_parts, lses, st);
  if (e != hipSuccess) return e;
  return launch_attention_merge(o_parts, lses, n, S, H, DH, out, ld_out, st);
}

hipError_t launch_attention_merge(const float* o_parts, const float* lses, int n_chunks, int S, int H, int DH,
                                  bf16_t* out, int ld_out, hipStream_t st) {
  if (S == 0) return hipSuccess;
  const long long total = (long long)S * (H * DH / 8);
  attention_merge_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(o_parts, lses, n_chunks, S, H, DH, out,
                                                                           ld_out);
  return hipGetLastError();
}

}  // namespace dit

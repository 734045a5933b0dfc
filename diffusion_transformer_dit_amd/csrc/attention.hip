// Exact softmax attention of the single-stream block (no mask, scale
// 1/sqrt(Dh)) on gfx950 matrix cores: the flash / sdpa backends of the Flux
// page (ChituDiffusion, sections 2 and 4) and the fp32 softmax the Wan2.1
// video page (mhpq.cn, section 5.1) recommends, as one LDS-tiled online-
// softmax kernel.
//
// One workgroup = 4 wavefronts = 128 queries of one head; each wave owns 32
// queries.  Keys/values stream through LDS in tiles of 64 tokens (double
// buffered; the next tile's global loads are in flight during the current
// tile's math).  Per tile and wave:
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16 (Q stays in registers), so
//                 every lane holds scores of ONE query: the row max / sum need
//                 one cross-lane step (lanes l and l^32) instead of a 32-lane
//                 reduction;
//   online softmax in fp32 with exp2 and the 1/sqrt(Dh)*log2(e) scale folded;
//   O^T += V^T P^T, where the P^T operand comes straight from the S^T
//                 accumulator registers (rounded to bf16) and V^T is read from
//                 an LDS copy of V stored transposed (8-byte units of 4 keys,
//                 XOR-swizzled).  The key order inside each 16-key MFMA step
//                 is permuted identically on both operands, which leaves the
//                 contraction unchanged.
#include "dit_common.hpp"
#include "launch.hpp"

namespace dit {

constexpr int ATT_BM = 128;  // queries per workgroup
constexpr int ATT_BN = 64;   // keys per tile

template <int DH>
struct AttCfg {
  static constexpr int K_BYTES = ATT_BN * DH * 2;  // K tile, rows of DH bf16
  static constexpr int V_BYTES = ATT_BN * DH * 2;  // V^T tile, rows of ATT_BN bf16
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int KCH = DH / 8;                    // 16-byte chunks per K row
  static constexpr int K_LD = ATT_BN * KCH / 256;       // K chunks per thread
  static constexpr int V_GROUPS = (DH / 8) * (ATT_BN / 4);  // (8 dims x 4 keys) groups
};

__device__ __forceinline__ uint32_t bf_at(const u32x4& v, int e) {
  return (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
}

template <int DH>
__global__ void __launch_bounds__(256, 2)
attention_fwd_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out, int S, int H,
                     int ld_out, float c_log2) {
  using C = AttCfg<DH>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int head = blockIdx.y;
  const int d = H * DH;
  const size_t ld = size_t(3) * d;
  const bf16_t* Qg = qkv + head * DH;
  const bf16_t* Kg = qkv + d + head * DH;
  const bf16_t* Vg = qkv + 2 * d + head * DH;

  const int ql = lane & 31;  // query column of this lane
  const int hh = lane >> 5;  // lane half
  const int q = blockIdx.x * ATT_BM + wave * 32 + ql;
  const int qc = min(q, S - 1);

  // Q^T operand: 8 dims (16*s + 8*hh ..) of this lane's query for each K-step s.
  bf16x8 qf[DH / 16];
#pragma unroll
  for (int s = 0; s < DH / 16; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(Qg + size_t(qc) * ld + 16 * s + 8 * hh);

  // ---- K/V tile loaders
  u32x4 rk[C::K_LD];
  u32x4 rv[4];
  const int vu = tid & 15;        // key group (keys 4*vu .. 4*vu+3)
  const int ve = tid >> 4;        // dim group (dims 8*ve .. 8*ve+7)
  const bool v_active = ve < DH / 8;
  auto gload = [&](int t0) {
#pragma unroll
    for (int i = 0; i < C::K_LD; ++i) {
      const int qd = tid + i * 256;
      const int key = qd / C::KCH, c = qd % C::KCH;
      const int tok = min(t0 + key, S - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(Kg + size_t(tok) * ld + 8 * c);
    }
    if (v_active) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int tok = min(t0 + 4 * vu + kk, S - 1);
        rv[kk] = *reinterpret_cast<const u32x4*>(Vg + size_t(tok) * ld + 8 * ve);
      }
    }
  };
  auto lstore = [&](int stage) {
    unsigned char* sK = smem + stage * C::STAGE;
    unsigned char* sV = sK + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::K_LD; ++i) {
      const int qd = tid + i * 256;
      const int key = qd / C::KCH, c = qd % C::KCH;
      *reinterpret_cast<u32x4*>(sK + key * (DH * 2) + ((c ^ (key & 7)) << 4)) = rk[i];
    }
    if (v_active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = 8 * ve + e;
        u32x2 w;
        w[0] = bf_at(rv[0], e) | (bf_at(rv[1], e) << 16);
        w[1] = bf_at(rv[2], e) | (bf_at(rv[3], e) << 16);
        *reinterpret_cast<u32x2*>(sV + dim * (ATT_BN * 2) + ((vu ^ (dim & 15)) << 3)) = w;
      }
    }
  };

  f32x16 oacc[DH / 32];
#pragma unroll
  for (int b = 0; b < DH / 32; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
  float m_run = -1e30f;  // running max of raw scores of this lane's query
  float l_run = 0.f;     // this lane's share of the running softmax denominator

  const int ntiles = (S + ATT_BN - 1) / ATT_BN;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int jt = 0; jt < ntiles; ++jt) {
    const int cur = jt & 1;
    if (jt + 1 < ntiles) gload((jt + 1) * ATT_BN);
    const unsigned char* sK = smem + cur * C::STAGE;
    const unsigned char* sV = sK + C::K_BYTES;

    // The tile is processed as two halves of 32 keys: S^T for keys
    // [32*kb, 32*kb+32), online softmax, then O^T += V^T P^T for those keys.
    const int key0 = jt * ATT_BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
      {
        const int key = kb * 32 + ql;
#pragma unroll
        for (int s = 0; s < DH / 16; ++s) {
          const int c = 2 * s + hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + key * (DH * 2) + ((c ^ (key & 7)) << 4));
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
        }
      }
      // accumulator row of register i: key 32*kb + 8*(i/4) + 4*hh + (i%4)
      if (key0 + ATT_BN > S) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3) >= S) sacc[i] = -INFINITY;
      }
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescale: the running max only moves (and O, l are rescaled) when
      // a score exceeds it by more than 2^8 in exp2 units for some lane of the
      // wave; otherwise the stale max stays, which is exact because numerator
      // and denominator use the same max and 2^8 cannot overflow fp32 sums.
      if (__builtin_amdgcn_ballot_w64((mx - m_run) * c_log2 > 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast((m_run - m_new) * c_log2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DH / 32; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
      }
      const float mc = m_run * c_log2;
      bf16x8 pf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = exp2_fast(fmaf(sacc[8 * half + j], c_log2, -mc));
          l_run += p[j];
        }
        u32x4 pk = pack8(p);
        pf[half] = __builtin_bit_cast(bf16x8, pk);
      }
      // O^T += V^T P^T over the two 16-key steps m of this half: lane supplies
      // keys 16m + 4hh + (0..3) and 16m + 8 + 4hh + (0..3), i.e. 8-byte units
      // 4m+hh and 4m+2+hh of the V^T row.
#pragma unroll
      for (int b = 0; b < DH / 32; ++b) {
        const int dim = b * 32 + ql;
        const unsigned char* row = sV + dim * (ATT_BN * 2);
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) {
          const int m = 2 * kb + mh;
          const int u1 = 4 * m + hh, u2 = 4 * m + 2 + hh;
          u32x4 av;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row + ((u1 ^ (dim & 15)) << 3));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + ((u2 ^ (dim & 15)) << 3));
          av[0] = lo[0];
          av[1] = lo[1];
          av[2] = hi[0];
          av[3] = hi[1];
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pf[mh],
                                                            oacc[b], 0, 0, 0);
        }
      }
    }
    if (jt + 1 < ntiles) lstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q < S) {
    bf16_t* orow = out + size_t(q) * ld_out + head * DH;
#pragma unroll
    for (int b = 0; b < DH / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // registers 4g..4g+3 hold dims b*32 + 8g + 4hh + (0..3)
        u32x2 w;
        w[0] = pack_bf2(oacc[b][4 * g] * inv, oacc[b][4 * g + 1] * inv);
        w[1] = pack_bf2(oacc[b][4 * g + 2] * inv, oacc[b][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + b * 32 + 8 * g + 4 * hh) = w;
      }
  }
}

hipError_t launch_attention(const bf16_t* qkv, bf16_t* out, int S, int H, int DH, int ld_out,
                            hipStream_t st) {
  if (S == 0) return hipSuccess;
  dim3 grid((S + ATT_BM - 1) / ATT_BM, H), block(256);
  const float c = kLog2e / sqrtf(float(DH));
  if (DH == 128)
    attention_fwd_kernel<128><<<grid, block, 0, st>>>(qkv, out, S, H, ld_out, c);
  else if (DH == 64)
    attention_fwd_kernel<64><<<grid, block, 0, st>>>(qkv, out, S, H, ld_out, c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dit

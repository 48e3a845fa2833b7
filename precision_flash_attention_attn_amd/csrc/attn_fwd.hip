// Forward flash attention for gfx950: tiled, online safe softmax, BF16 MFMA
// with FP32 accumulation, three modes (plain BF16 output, FP32 output,
// repeated-maximum-aware safe softmax).
//
// Method: "Why Low-Precision Transformer Training Fails: An Analysis on Flash
// Attention" (arXiv 2510.04212), paper-graph-ui summary, section 3.4.4 (the
// definitions P-bar = exp(S - rowmax S), O-bar = P-bar V, O = O-bar/rowsum P-bar
// and the BF16 rounding of the FP32-accumulated product) and section 3.4.5
// (the modified safe softmax inside the tiled forward pass).
//
// Work decomposition: one workgroup of 4 waves per (batch*head, block of 128
// queries); each wave owns 32 queries.  Keys stream in tiles of 64 through a
// double-buffered LDS stage.  Per tile and wave:
//   S^T (64 keys x 32 queries) = K_tile Q^T   (MFMA, A = K rows from LDS,
//                                              B = the wave's Q held in VGPRs)
//   online max / top-2 / shift / exp on the accumulators (VALU)
//   O^T (d x 32 queries) += V_tile^T P-bar^T   (MFMA, A = V read transposed from
//                                              LDS, B = P-bar packed to BF16 in
//                                              place from the S accumulators)
// The K rows of each 32-key block are fed to the MFMA in the order sigma (see
// sigma32) so that the accumulator registers of a lane already hold the 8
// consecutive keys the P-bar V step needs as its B operand: P-bar never goes
// through LDS.
#include "pfa_common.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int32_t* flags;
  int BH, N, n_qblocks;
  float scale, beta, eps;
};

// Row order of K inside a 32-key block: MFMA accumulator row i of lane half h
// holds key sigma(i); chosen so that registers 0..7 of lane l hold keys
// 8*(l/32) + 0..7 and registers 8..15 hold keys 16 + 8*(l/32) + 0..7.
__device__ __forceinline__ int sigma32(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return ((a >> 1) << 4) | (h << 3) | ((a & 1) << 2) | b;
}

// Longest-first order for causal work; when the number of (batch, head)
// slices is a multiple of 8, each XCD (workgroup id mod 8) works on a fixed
// set of slices so their K/V stay in that XCD's L2.
__device__ __forceinline__ void map_block(int bid, int BH, int nqb, int& bh, int& qb) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, idx = bid >> 3, hp = BH >> 3;
    bh = xcd * hp + idx % hp;
    qb = nqb - 1 - idx / hp;
  } else {
    bh = bid % BH;
    qb = nqb - 1 - bid / BH;
  }
}

template <int D, int MODE, bool CAUSAL, bool FLAGS>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdParams p) {
  constexpr int BM = 128, BN = 64, NT = 256;
  constexpr int CH = D / 8;    // 16-byte chunks per K/V row
  constexpr int DC = D / 16;   // contraction steps of K Q^T
  constexpr int KB = BN / 32;  // 32-key blocks per tile
  constexpr int KC = BN / 16;  // 16-key contraction steps of V^T P^T
  constexpr int DB = D / 32;   // 32-feature blocks of O
  constexpr bool TIE = MODE == kTieAware;
  constexpr bool HP = MODE == kFp32Out;
  constexpr bool SUNITS = FLAGS || TIE;  // scores kept as S = scale*dot (else the raw dot)
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int ROWS_PER_PASS = NT / CH;
  constexpr int PASSES = BN / ROWS_PER_PASS;

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5;
  const int N = p.N;
  int bh, qb;
  map_block(blockIdx.x, p.BH, p.n_qblocks, bh, qb);
  const size_t base = (size_t)bh * N * D;
  const uint16_t* __restrict__ Q = p.q + base;
  const uint16_t* __restrict__ K = p.k + base;
  const uint16_t* __restrict__ V = p.v + base;
  const int q0 = qb * BM;
  const int qw0 = q0 + 32 * w;
  const int myq = qw0 + (lane & 31);

  // This wave's queries as the B operand of K Q^T: chunk 2c + hi of row myq.
  u32x4 qreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c)
    qreg[c] = (myq < N) ? ldg_b128(Q + (size_t)myq * D + (2 * c + hi) * 8) : u32x4{0, 0, 0, 0};

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  const int st_row = tid / CH, st_chunk = tid % CH;
  u32x4 kst[PASSES], vst[PASSES];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int key = j * BN + ps * ROWS_PER_PASS + st_row;
      if (key < N) {
        kst[ps] = ldg_b128(K + (size_t)key * D + st_chunk * 8);
        vst[ps] = ldg_b128(V + (size_t)key * D + st_chunk * 8);
      } else {
        kst[ps] = u32x4{0, 0, 0, 0};
        vst[ps] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kl = smem + buf * 2 * TILE_BYTES;
    char* vl = kl + TILE_BYTES;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int row = ps * ROWS_PER_PASS + st_row;
      lds_write_b128(kl, swz<CH>(row, st_chunk), kst[ps]);
      lds_write_b128(vl, swz<CH>(row, st_chunk), vst[ps]);
    }
  };

  const float scale = p.scale;
  const float cexp = SUNITS ? kLog2e : scale * kLog2e;
  float M = kNegInf, M2 = kNegInf, m = kNegInf, lsum = 0.f;
  bool flag = false;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // per-lane LDS offsets that do not depend on the tile
  const int krow = sigma32(lane & 31);
  const int g = lane >> 4, s = lane & 15;
  const int tr_row = 8 * (g >> 1) + (s >> 2);   // + 16*kc + 4*half
  const int tr_col = 16 * (g & 1) + 4 * (s & 3);  // + 32*db

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);
    const int kv0 = j * BN;
    const bool wave_active = (qw0 < N) && (!CAUSAL || kv0 <= qw0 + 31);
    if (wave_active) {
      const char* kl = smem + buf * 2 * TILE_BYTES;
      const char* vl = kl + TILE_BYTES;
      f32x16 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const u32x4 a = lds_read_b128(kl, swz<CH>(kb * 32 + krow, 2 * c + hi));
          sacc[kb] = mfma_bf16(a, qreg[c], sacc[kb]);
        }
      }
      // scores: scale, mask, tile top-2 (or max)
      const bool need_mask = (CAUSAL && kv0 + BN - 1 > qw0) || (kv0 + BN > N);
      float t1 = kNegInf, t2 = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sv = sacc[kb][r];
          if (SUNITS) sv *= scale;
          if (need_mask) {
            const int key = kv0 + 32 * kb + 16 * (r >> 3) + 8 * hi + (r & 7);
            if (key >= N || (CAUSAL && key > myq)) sv = kNegInf;
          }
          sacc[kb][r] = sv;
          if (FLAGS) t2 = med3(t1, t2, sv);
          t1 = fmaxf(t1, sv);
        }
      }
      // combine the two lane halves that share a query
      const float o1 = xchg32(t1);
      if (FLAGS) {
        const float o2 = xchg32(t2);
        t2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
      }
      t1 = fmaxf(t1, o1);
      // running row maximum and second largest (multiset), tie flag, shift
      if (FLAGS) M2 = fmaxf(fminf(M, t1), fmaxf(M2, t2));
      M = fmaxf(M, t1);
      if (FLAGS) flag = (M2 != kNegInf) && (M - M2 <= p.eps);
      float m_new = M;
      if (TIE && flag) m_new = (M > 0.f) ? p.beta * M : ((M < 0.f) ? 0.f : M);
      float alpha;
      float mb;
      if (m_new == kNegInf) {  // no unmasked key seen yet for this row
        alpha = 1.f;
        mb = 0.f;
      } else {
        alpha = (m == kNegInf) ? 0.f : fast_exp2((m - m_new) * cexp);
        mb = m_new * cexp;
        m = m_new;
      }
      // probabilities, rounded to BF16 (or split hi + lo), row sums
      uint32_t pk[KB][8];
      uint32_t pl[KB][8];
      float lt = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pa = fast_exp2(fmaf(sacc[kb][2 * i], cexp, -mb));
          const float pb = fast_exp2(fmaf(sacc[kb][2 * i + 1], cexp, -mb));
          const uint32_t u = pack_bf16(pa, pb);
          pk[kb][i] = u;
          const float ha = bf16lo_to_f32(u), hb = bf16hi_to_f32(u);
          if (HP) {
            const uint32_t ul = pack_bf16(pa - ha, pb - hb);
            pl[kb][i] = ul;
            lt += (ha + bf16lo_to_f32(ul)) + (hb + bf16hi_to_f32(ul));
          } else {
            lt += ha + hb;
          }
        }
      }
      lsum = lsum * alpha + lt;
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      // O^T += V^T P-bar^T
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int kb = kc >> 1, o4 = 4 * (kc & 1);
        const u32x4 bop = u32x4{pk[kb][o4], pk[kb][o4 + 1], pk[kb][o4 + 2], pk[kb][o4 + 3]};
        u32x4 bop_lo;
        if (HP) bop_lo = u32x4{pl[kb][o4], pl[kb][o4 + 1], pl[kb][o4 + 2], pl[kb][o4 + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int row = 16 * kc + tr_row, col = 32 * db + tr_col;
          const u32x2 a0 = lds_read_tr(vl, swz_elem<CH>(row, col));
          const u32x2 a1 = lds_read_tr(vl, swz_elem<CH>(row + 4, col));
          const u32x4 aop = u32x4{a0.x, a0.y, a1.x, a1.y};
          oacc[db] = mfma_bf16(aop, bop, oacc[db]);
          if (HP) oacc[db] = mfma_bf16(aop, bop_lo, oacc[db]);
        }
      }
    }
    if (j + 1 < n_tiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // epilogue: O = bf16(bf16(O-bar) / l)   or   O = O-bar / l (FP32 output)
  const float ltot = lsum + xchg32(lsum);
  if (myq < N) {
    const size_t orow = base + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * hi;
        const float v0 = oacc[db][4 * rr], v1 = oacc[db][4 * rr + 1];
        const float v2 = oacc[db][4 * rr + 2], v3 = oacc[db][4 * rr + 3];
        if (HP) {
          f32x4 out = {v0 / ltot, v1 / ltot, v2 / ltot, v3 / ltot};
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + orow + d0) = out;
        } else {
          const float r0 = round_bf16(v0) / ltot, r1 = round_bf16(v1) / ltot;
          const float r2 = round_bf16(v2) / ltot, r3 = round_bf16(v3) / ltot;
          u32x2 out = {pack_bf16(r0, r1), pack_bf16(r2, r3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + orow + d0) = out;
        }
      }
    }
    if (hi == 0) {
      const float m_s = SUNITS ? m : m * scale;
      p.lse[(size_t)bh * N + myq] = m_s + logf(ltot);
      if (FLAGS && p.flags) p.flags[(size_t)bh * N + myq] = flag ? 1 : 0;
    }
  }
}

template <int D, int MODE, bool CAUSAL, bool FLAGS>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.flags = a.flags;
  p.BH = a.B * a.H;
  p.N = a.N;
  p.n_qblocks = (a.N + 127) / 128;
  p.scale = a.scale;
  p.beta = a.beta;
  p.eps = a.eps;
  const unsigned grid = (unsigned)(p.BH * p.n_qblocks);
  hipLaunchKernelGGL((fwd_kernel<D, MODE, CAUSAL, FLAGS>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_m(const FwdArgs& a, hipStream_t stream) {
  const bool flags = MODE == kTieAware || a.flags != nullptr;
  if (a.causal) {
    if (MODE == kTieAware || flags) return launch_t<D, MODE, true, true>(a, stream);
    return launch_t<D, MODE, true, (MODE == kTieAware)>(a, stream);
  }
  if (MODE == kTieAware || flags) return launch_t<D, MODE, false, true>(a, stream);
  return launch_t<D, MODE, false, (MODE == kTieAware)>(a, stream);
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  switch (a.mode) {
    case kBf16Out: return launch_m<D, kBf16Out>(a, stream);
    case kFp32Out: return launch_m<D, kFp32Out>(a, stream);
    default: return launch_m<D, kTieAware>(a, stream);
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace pfa

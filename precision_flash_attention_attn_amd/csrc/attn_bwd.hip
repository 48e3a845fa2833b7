// Backward flash attention for gfx950.
//
// Method: "Why Low-Precision Transformer Training Fails: An Analysis on Flash
// Attention" (arXiv 2510.04212), paper-graph-ui summary, section 3.4.2 (the
// backward computes delta = rowsum(dO o O) and dS = P o (dP - delta)) and
// section 3.4.3 (dS = alpha P o (dP - delta), dQ = dS K).  dK = alpha dS^T Q and
// dV = P^T dO are the matching gradients of the same products.
//
// Three kernels on the caller's stream:
//   bwd_pre      delta = rowsum(dO o O) in FP32 (O, dO BF16, or FP32 in the
//                FP32-output mode); clears the FP32 dQ accumulator.
//   bwd_main     one workgroup of 4 waves per (batch*head, block of 128 keys);
//                each wave owns 32 keys, keeps K^T and V^T operands in VGPRs and
//                accumulates dK^T, dV^T in MFMA accumulators while query tiles
//                of 64 stream through LDS:
//                  S = Q K^T, dP = dO V^T          (A from LDS, B from VGPRs)
//                  P = exp(S - LSE), dS = P o (dP - delta)          (VALU)
//                  dV^T += dO^T P, dK^T += Q^T dS  (A read transposed from LDS,
//                                                   B = P, dS packed in place)
//                  dQ += dS K                      (dS through LDS; FP32
//                                                   atomic adds to the accumulator)
//   bwd_dq_cvt   dQ = bf16(scale * accumulator).
#include "pfa_common.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

// ---------------------------------------------------------------------------
// delta = rowsum(dO o O); dQ accumulator := 0
template <int D, bool F32IO>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const void* __restrict__ o,
                                                      const void* __restrict__ dout,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, size_t rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const int t = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * RPB + t / TPR;
  const int c = t % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = row * D + c * 8;
    if (F32IO) {
      const f32x4* op = reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + off);
      const f32x4* dp = reinterpret_cast<const f32x4*>(static_cast<const float*>(dout) + off);
      const f32x4 o0 = op[0], o1 = op[1], d0 = dp[0], d1 = dp[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += o0[i] * d0[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += o1[i] * d1[i];
    } else {
      const u32x4 ov = ldg_b128(static_cast<const uint16_t*>(o) + off);
      const u32x4 dv = ldg_b128(static_cast<const uint16_t*>(dout) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += bf16lo_to_f32(ov[i]) * bf16lo_to_f32(dv[i]);
        acc += bf16hi_to_f32(ov[i]) * bf16hi_to_f32(dv[i]);
      }
    }
    f32x4* z = reinterpret_cast<f32x4*>(dq_acc + off);
    z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int sh = TPR / 2; sh >= 1; sh >>= 1) acc += __shfl_xor(acc, sh, 64);
  if (row < rows && c == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
__device__ __forceinline__ int sigma32(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return ((a >> 1) << 4) | (h << 3) | ((a & 1) << 2) | b;
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* dout;
  const float* lse;
  const float* delta;
  float* dq_acc;
  uint16_t* dk;
  uint16_t* dv;
  int BH, N, n_kvblocks;
  float scale;
};

__device__ __forceinline__ void map_kv_block(int bid, int BH, int nkb, int& bh, int& kb) {
  // heaviest key blocks (the first ones, under a causal mask) first; slices
  // grouped per XCD when their number is a multiple of 8
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, idx = bid >> 3, hp = BH >> 3;
    bh = xcd * hp + idx % hp;
    kb = idx / hp;
  } else {
    bh = bid % BH;
    kb = bid / BH;
  }
}

template <int D, bool CAUSAL, bool F32DO>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdParams p) {
  constexpr int BKV = 128, BQ = 64, NT = 256;
  constexpr int CH = D / 8;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int QROWS_PER_PASS = NT / CH;
  constexpr int QPASSES = BQ / QROWS_PER_PASS;
  constexpr int KPASSES = BKV / QROWS_PER_PASS;
  constexpr int KBLK_BYTES = BKV * D * 2;
  constexpr int QT_BYTES = BQ * D * 2;
  constexpr int DS_BYTES = BKV * BQ * 2;
  // dQ blocks (32 queries x 32 features) per wave
  constexpr int NDQ = (2 * DB) / 4;

  __shared__ __attribute__((aligned(16))) char s_k[KBLK_BYTES];
  __shared__ __attribute__((aligned(16))) char s_q[QT_BYTES];
  __shared__ __attribute__((aligned(16))) char s_do[QT_BYTES];
  __shared__ __attribute__((aligned(16))) char s_ds[DS_BYTES];
  __shared__ __attribute__((aligned(16))) float s_lse[BQ];
  __shared__ __attribute__((aligned(16))) float s_delta[BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5;
  const int N = p.N;
  int bh, kvb;
  map_kv_block(blockIdx.x, p.BH, p.n_kvblocks, bh, kvb);
  const size_t base = (size_t)bh * N * D;
  const size_t rbase = (size_t)bh * N;
  const uint16_t* __restrict__ Q = p.q + base;
  const uint16_t* __restrict__ K = p.k + base;
  const uint16_t* __restrict__ V = p.v + base;
  const int kv0 = kvb * BKV;
  const int kw0 = kv0 + 32 * w;
  const int mykey = kw0 + (lane & 31);

  // K and V of this wave's keys as B operands (columns = keys)
  u32x4 kreg[DC], vreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const bool ok = mykey < N;
    kreg[c] = ok ? ldg_b128(K + (size_t)mykey * D + (2 * c + hi) * 8) : u32x4{0, 0, 0, 0};
    vreg[c] = ok ? ldg_b128(V + (size_t)mykey * D + (2 * c + hi) * 8) : u32x4{0, 0, 0, 0};
  }
  // the workgroup's K block in LDS (B operand of dQ = dS K)
  const int st_row = tid / CH, st_chunk = tid % CH;
#pragma unroll
  for (int ps = 0; ps < KPASSES; ++ps) {
    const int row = ps * QROWS_PER_PASS + st_row, key = kv0 + row;
    const u32x4 val = key < N ? ldg_b128(K + (size_t)key * D + st_chunk * 8) : u32x4{0, 0, 0, 0};
    lds_write_b128(s_k, swz<CH>(row, st_chunk), val);
  }

  // query tile staging (prefetched into registers one tile ahead)
  u32x4 qst[QPASSES], dost[QPASSES], dost2[QPASSES];
  float lse_st = 0.f, delta_st = 0.f;
  const float l2e = kLog2e;
  auto load_qtile = [&](int qt0) {
#pragma unroll
    for (int ps = 0; ps < QPASSES; ++ps) {
      const int qrow = qt0 + ps * QROWS_PER_PASS + st_row;
      if (qrow < N) {
        qst[ps] = ldg_b128(Q + (size_t)qrow * D + st_chunk * 8);
        if (F32DO) {
          const float* dp = static_cast<const float*>(p.dout) + base + (size_t)qrow * D + st_chunk * 8;
          dost[ps] = ldg_b128(dp);
          dost2[ps] = ldg_b128(dp + 4);
        } else {
          dost[ps] = ldg_b128(static_cast<const uint16_t*>(p.dout) + base + (size_t)qrow * D + st_chunk * 8);
        }
      } else {
        qst[ps] = u32x4{0, 0, 0, 0};
        dost[ps] = u32x4{0, 0, 0, 0};
        if (F32DO) dost2[ps] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < BQ) {
      const int qrow = qt0 + tid;
      lse_st = qrow < N ? p.lse[rbase + qrow] * l2e : __builtin_inff();
      delta_st = qrow < N ? p.delta[rbase + qrow] : 0.f;
    }
  };
  auto store_qtile = [&]() {
#pragma unroll
    for (int ps = 0; ps < QPASSES; ++ps) {
      const int row = ps * QROWS_PER_PASS + st_row;
      lds_write_b128(s_q, swz<CH>(row, st_chunk), qst[ps]);
      u32x4 dv;
      if (F32DO) {
        // whole-vector reinterpretation (bit-casting single vector elements is avoided)
        const f32x4 a = __builtin_bit_cast(f32x4, dost[ps]);
        const f32x4 b = __builtin_bit_cast(f32x4, dost2[ps]);
        dv = u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
                   pack_bf16(b[2], b[3])};
      } else {
        dv = dost[ps];
      }
      lds_write_b128(s_do, swz<CH>(row, st_chunk), dv);
    }
    if (tid < BQ) {
      s_lse[tid] = lse_st;
      s_delta[tid] = delta_st;
    }
  };

  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  const int arow = sigma32(lane & 31);
  const int g = lane >> 4, s = lane & 15;
  const int tr_row = 8 * (g >> 1) + (s >> 2);
  const int tr_col = 16 * (g & 1) + 4 * (s & 3);
  const float sl2 = p.scale * kLog2e;

  const int qt_begin = CAUSAL ? kv0 : 0;
  if (qt_begin < N) {
    load_qtile(qt_begin);
    store_qtile();
  }
  __syncthreads();

  for (int qt0 = qt_begin; qt0 < N; qt0 += BQ) {
    const bool has_next = qt0 + BQ < N;
    if (has_next) load_qtile(qt0 + BQ);
    // 1. S = Q K^T and dP = dO V^T (rows: queries in sigma order; columns: this wave's keys)
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sacc[qb] = f32x16{};
      dpacc[qb] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const int off = swz<CH>(32 * qb + arow, 2 * c + hi);
        sacc[qb] = mfma_bf16(lds_read_b128(s_q, off), kreg[c], sacc[qb]);
        dpacc[qb] = mfma_bf16(lds_read_b128(s_do, off), vreg[c], dpacc[qb]);
      }
    }
    // 2. P = exp(S - LSE), dS = P o (dP - delta), packed to BF16
    const bool need_mask = (CAUSAL && qt0 < kw0 + 31) || (kv0 + BKV > N);
    uint32_t pP[2][8], pS[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qi = 32 * qb + 16 * hh + 8 * hi;  // 8 consecutive queries of the tile
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(s_lse + qi);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(s_lse + qi + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(s_delta + qi);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(s_delta + qi + 4);
        float pv[8], dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * hh + e;
          const float lse2 = e < 4 ? l0[e] : l1[e - 4];
          const float dl = e < 4 ? d0[e] : d1[e - 4];
          float pr = fast_exp2(fmaf(sacc[qb][r], sl2, -lse2));
          if (need_mask) {
            const int qrow = qt0 + qi + e;
            if (mykey >= N || (CAUSAL && mykey > qrow)) pr = 0.f;
          }
          pv[e] = pr;
          dsv[e] = pr * (dpacc[qb][r] - dl);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pP[qb][4 * hh + e] = pack_bf16(pv[2 * e], pv[2 * e + 1]);
          pS[qb][4 * hh + e] = pack_bf16(dsv[2 * e], dsv[2 * e + 1]);
        }
      }
    }
    // 3. dV^T += dO^T P, dK^T += Q^T dS; 4. dS^T to LDS for dQ
#pragma unroll
    for (int qc = 0; qc < 4; ++qc) {
      const int qb = qc >> 1, o4 = 4 * (qc & 1);
      const u32x4 bP = u32x4{pP[qb][o4], pP[qb][o4 + 1], pP[qb][o4 + 2], pP[qb][o4 + 3]};
      const u32x4 bS = u32x4{pS[qb][o4], pS[qb][o4 + 1], pS[qb][o4 + 2], pS[qb][o4 + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 16 * qc + tr_row, col = 32 * db + tr_col;
        const u32x2 a0 = lds_read_tr(s_do, swz_elem<CH>(row, col));
        const u32x2 a1 = lds_read_tr(s_do, swz_elem<CH>(row + 4, col));
        dvacc[db] = mfma_bf16(u32x4{a0.x, a0.y, a1.x, a1.y}, bP, dvacc[db]);
        const u32x2 b0 = lds_read_tr(s_q, swz_elem<CH>(row, col));
        const u32x2 b1 = lds_read_tr(s_q, swz_elem<CH>(row + 4, col));
        dkacc[db] = mfma_bf16(u32x4{b0.x, b0.y, b1.x, b1.y}, bS, dkacc[db]);
      }
      lds_write_b128(s_ds, swz<8>(32 * w + (lane & 31), 2 * qc + hi), bS);
    }
    __syncthreads();
    if (has_next) store_qtile();
    // 5. dQ (queries x features) += dS K over the workgroup's 128 keys
#pragma unroll
    for (int t = 0; t < NDQ; ++t) {
      const int blk = w * NDQ + t;        // 2*DB blocks: qb = blk % 2, db = blk / 2
      const int qb = blk & 1, db = blk >> 1;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kc = 0; kc < BKV / 16; ++kc) {
        const int row = 16 * kc + tr_row;
        const u32x2 a0 = lds_read_tr(s_ds, swz_elem<8>(row, 32 * qb + tr_col));
        const u32x2 a1 = lds_read_tr(s_ds, swz_elem<8>(row + 4, 32 * qb + tr_col));
        const u32x2 b0 = lds_read_tr(s_k, swz_elem<CH>(row, 32 * db + tr_col));
        const u32x2 b1 = lds_read_tr(s_k, swz_elem<CH>(row + 4, 32 * db + tr_col));
        acc = mfma_bf16(u32x4{a0.x, a0.y, a1.x, a1.y}, u32x4{b0.x, b0.y, b1.x, b1.y}, acc);
      }
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = qt0 + 32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (qrow < N) unsafeAtomicAdd(p.dq_acc + base + (size_t)qrow * D + d, acc[r]);
      }
    }
    __syncthreads();
  }

  // epilogue: dK = scale * dK^T acc, dV; lane holds key mykey, features 32db + 8(r/4) + 4hi + r%4
  if (mykey < N) {
    const size_t krow = base + (size_t)mykey * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * hi;
        const u32x2 kv = {pack_bf16(p.scale * dkacc[db][4 * rr], p.scale * dkacc[db][4 * rr + 1]),
                          pack_bf16(p.scale * dkacc[db][4 * rr + 2], p.scale * dkacc[db][4 * rr + 3])};
        const u32x2 vv = {pack_bf16(dvacc[db][4 * rr], dvacc[db][4 * rr + 1]),
                          pack_bf16(dvacc[db][4 * rr + 2], dvacc[db][4 * rr + 3])};
        *reinterpret_cast<u32x2*>(p.dk + krow + d0) = kv;
        *reinterpret_cast<u32x2*>(p.dv + krow + d0) = vv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_cvt_kernel(const float* __restrict__ acc,
                                                         uint16_t* __restrict__ dq, float scale,
                                                         size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(acc)[2 * i];
  const f32x4 b = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
  const u32x4 out = {pack_bf16(scale * a[0], scale * a[1]), pack_bf16(scale * a[2], scale * a[3]),
                     pack_bf16(scale * b[0], scale * b[1]), pack_bf16(scale * b[2], scale * b[3])};
  reinterpret_cast<u32x4*>(dq)[i] = out;
}

template <int D>
hipError_t prep_d(const BwdArgs& a, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
  if (a.mode == kFp32Out)
    hipLaunchKernelGGL((bwd_pre_kernel<D, true>), dim3(grid), dim3(256), 0, stream, a.o, a.dout,
                       a.delta, a.dq_acc, rows);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<D, false>), dim3(grid), dim3(256), 0, stream, a.o, a.dout,
                       a.delta, a.dq_acc, rows);
  return hipGetLastError();
}

template <int D>
hipError_t main_d(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = a.dout;
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq_acc = a.dq_acc;
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.BH = a.B * a.H;
  p.N = a.N;
  p.n_kvblocks = (a.N + 127) / 128;
  p.scale = a.scale;
  const unsigned grid = (unsigned)(p.BH * p.n_kvblocks);
  const bool f32io = a.mode == kFp32Out;
  if (a.causal) {
    if (f32io) hipLaunchKernelGGL((bwd_main_kernel<D, true, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_main_kernel<D, true, false>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (f32io) hipLaunchKernelGGL((bwd_main_kernel<D, false, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_main_kernel<D, false, false>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? prep_d<64>(a, stream) : prep_d<128>(a, stream);
}

hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? main_d<64>(a, stream) : main_d<128>(a, stream);
}

hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream) {
  const size_t n8 = (size_t)a.B * a.H * a.N * a.d / 8;
  hipLaunchKernelGGL(bwd_dq_cvt_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     a.dq_acc, static_cast<uint16_t*>(a.dq), a.scale, n8);
  return hipGetLastError();
}

}  // namespace pfa

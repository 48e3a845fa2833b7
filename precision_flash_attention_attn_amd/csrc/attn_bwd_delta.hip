// Alternative sources of delta for the backward, from the isolation
// experiments of "Why Low-Precision Transformer Training Fails: An Analysis on
// Flash Attention" (arXiv 2510.04212), paper-graph-ui summary, section 3.2
// and section 3.4.2:
//
//   kDeltaDpP    delta = rowsum(dP o P), P = exp(S - LSE), dP = dO V^T: the
//                formulation that needs no stored O (equal to rowsum(dO o O)
//                in exact arithmetic);
//   kDeltaOhp    delta = rowsum(dO o O_hp), O_hp = P V recomputed inside the
//                backward with FP32 accumulation (P split into BF16 hi + lo,
//                both products on MFMA, as in the FP32-output forward);
//   kDeltaErr    delta_lp - delta_hp per row: rowsum(dO o O) with the stored
//                O minus the kDeltaOhp value (the error of delta that
//                section 3.4.4 traces back to the rounding of O).
//
// P is exp(S - LSE) renormalised by its own FP32 row sum: the LSE of the
// forward carries the rounding of its row sum of BF16 P-bar, and the point of
// these sources is a delta free of the forward's low precision.
//
// Work decomposition as in the dQ kernel: one workgroup of 4 waves per
// (batch*head, block of 128 queries), each wave owning 32 queries; key tiles
// of 64 stream through double-buffered LDS stages (K and V in separate
// arrays).  Per tile and wave:
//   S^T = K_tile Q^T                                  (MFMA, A = K rows, B = Q)
//   P = exp(S - LSE), zero where masked               (VALU)
//   kDeltaDpP:  dP^T = V_tile dO^T (MFMA); acc += P dP (VALU)
//   otherwise:  O_hp^T += V^T P_hi^T + V^T P_lo^T     (MFMA, A = V read
//               transposed, B = P packed in place from the accumulators)
#include "pfa_common.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

struct DeltaParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;        // stored O (kDeltaErr): BF16, or FP32 in the FP32-output mode
  const void* dout;     // dO as given: BF16, or FP32 in the FP32-output mode
  const float* lse;
  float* delta;
  int BH, N, n_qblocks;
  float scale;
};

__device__ __forceinline__ int sigma32(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return ((a >> 1) << 4) | (h << 3) | ((a & 1) << 2) | b;
}

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

// 8 consecutive values of row `row` of a [*, D] tensor starting at column c0,
// as FP32 (BF16 widened exactly, or FP32).
template <bool F32>
__device__ __forceinline__ void load8(const void* base, size_t off, float (&x)[8]) {
  if (F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  } else {
    const u32x4 u = ldg_b128(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo_to_f32(u[i]);
      x[2 * i + 1] = bf16hi_to_f32(u[i]);
    }
  }
}

template <int D, bool CAUSAL, int SRC, bool F32IO>
struct DeltaKernel {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int CH = D / 8;
  static constexpr int DC = D / 16;
  static constexpr int KB = BN / 32;
  static constexpr int KC = BN / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BN * D * 2;
  static constexpr int LOADS = TILE / (NT * 16);
  static constexpr int ROWB = CH * 16;
  static constexpr bool DP = SRC == kDeltaDpP;

  const DeltaParams& p;
  char* kb0;
  char* kb1;
  char* vb0;
  char* vb1;
  int tid, lane, w, hi, N, bh, qw0, myq, q0;
  size_t base;
  __amdgpu_buffer_rsrc_t krs, vrs;
  int voff[LOADS];
  int kbase, vbase0, vbase1;
  u32x4 qreg[DC];
  u32x4 doreg[DC];      // kDeltaDpP: this lane's dO fragments (BF16)
  f32x16 oacc[DB];      // otherwise: O_hp^T accumulators
  float lse2, acc, psum;

  __device__ DeltaKernel(const DeltaParams& p_, char* k0, char* k1, char* v0, char* v1)
      : p(p_), kb0(k0), kb1(k1), vb0(v0), vb1(v1) {}

  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int j, char* dst0) {
    const int kv0 = j * BN;
    if (kv0 + BN <= N) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) buf2lds_b128(rs, voff[i], kv0 * D * 2, dst0 + (w * LOADS + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int row = ((w * LOADS + i) * 64 + lane) / CH;
        const int off = voff[i] + (min(kv0 + row, N - 1) - row) * D * 2;
        buf2lds_b128(rs, off, 0, dst0 + (w * LOADS + i) * 1024);
      }
    }
  }

  template <int B>
  __device__ __forceinline__ void issue_tile(int j) {
    issue(krs, j, B ? kb1 : kb0);
    issue(vrs, j, B ? vb1 : vb0);
  }

  template <int B, bool MASK>
  __device__ __forceinline__ void compute_tile(int j) {
    const int kv0 = j * BN;
    if (MASK && !(qw0 < N && (!CAUSAL || kv0 <= qw0 + 31))) return;   // no visible key
    const char* kl = B ? kb1 : kb0;
    const char* vl = B ? vb1 : vb0;
    int kbs = kbase;
    asm volatile("" : "+v"(kbs));
    f32x16 sacc[KB], pacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
      if (DP) pacc[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        sacc[kb] = mfma_bf16(lds_read_b128(kl, (kbs ^ (32 * c)) + kb * 32 * ROWB), qreg[c], sacc[kb]);
        if (DP)
          pacc[kb] = mfma_bf16(lds_read_b128(vl, (kbs ^ (32 * c)) + kb * 32 * ROWB), doreg[c], pacc[kb]);
      }
    }
    const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - (kv0 + 8 * hi);
    const float c1 = p.scale * kLog2e;
    uint32_t ph[KB][8], pl[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float pr[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          pr[e] = fast_exp2(fmaf(sacc[kb][r], c1, -lse2));
          if (MASK) {
            const int off = 32 * kb + 16 * (r >> 3) + (r & 7);
            pr[e] = off > lim ? 0.f : pr[e];
          }
          psum += pr[e];
          if (DP) acc = fmaf(pr[e], pacc[kb][r], acc);
        }
        if (!DP) {
          const uint32_t u = pack_bf16(pr[0], pr[1]);
          ph[kb][i] = u;
          pl[kb][i] = pack_bf16(pr[0] - bf16lo_to_f32(u), pr[1] - bf16hi_to_f32(u));
        }
      }
    if (!DP) {
      int v0s = vbase0, v1s = vbase1;
      asm volatile("" : "+v"(v0s), "+v"(v1s));
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int kb = kc >> 1, o4 = 4 * (kc & 1);
        const u32x4 bh_ = u32x4{ph[kb][o4], ph[kb][o4 + 1], ph[kb][o4 + 2], ph[kb][o4 + 3]};
        const u32x4 bl_ = u32x4{pl[kb][o4], pl[kb][o4 + 1], pl[kb][o4 + 2], pl[kb][o4 + 3]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 a0 = lds_read_tr(vl, (v0s ^ (64 * db)) + kc * 16 * ROWB);
          const u32x2 a1 = lds_read_tr(vl, (v1s ^ (64 * db)) + kc * 16 * ROWB);
          const u32x4 aop = u32x4{a0.x, a0.y, a1.x, a1.y};
          oacc[db] = mfma_bf16(aop, bh_, oacc[db]);
          oacc[db] = mfma_bf16(aop, bl_, oacc[db]);
        }
      }
    }
  }

  template <int B, bool MASK>
  __device__ __forceinline__ void step(int j, int n_tiles) {
    if (j + 1 < n_tiles) issue_tile<1 - B>(j + 1);
    compute_tile<B, MASK>(j);
    wait_all_and_barrier();
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    hi = lane >> 5;
    N = p.N;
    int qb;
    map_block(blockIdx.x, p.BH, p.n_qblocks, bh, qb);
    base = (size_t)bh * N * D;
    krs = make_rsrc(p.k + base, N * D * 2);
    vrs = make_rsrc(p.v + base, N * D * 2);
    q0 = qb * BM;
    qw0 = q0 + 32 * w;
    myq = qw0 + (lane & 31);
    const bool valid = myq < N;
    const size_t qrow = base + (size_t)(valid ? myq : 0) * D;

#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int col = (2 * c + hi) * 8;
      qreg[c] = valid ? ldg_b128(p.q + qrow + col) : u32x4{0, 0, 0, 0};
      if (DP) {
        float x[8];
        load8<F32IO>(p.dout, qrow + col, x);
        doreg[c] = valid ? u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                                 pack_bf16(x[6], x[7])}
                         : u32x4{0, 0, 0, 0};
      }
    }
    lse2 = valid ? p.lse[(size_t)bh * N + myq] * kLog2e : __builtin_inff();
    acc = 0.f;
    psum = 0.f;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (w * LOADS + i) * 64 + lane;
      const int row = slot / CH, pchunk = slot % CH;
      voff[i] = (row * D + (pchunk ^ swz_pattern<CH>(row)) * 8) * 2;
    }
    kbase = swz<CH>(sigma32(lane & 31), hi);
    const int g = lane >> 4, s = lane & 15;
    const int tr_row = 8 * (g >> 1) + (s >> 2);
    const int tr_col = 16 * (g & 1) + 4 * (s & 3);
    vbase0 = swz_elem<CH>(tr_row, tr_col);
    vbase1 = swz_elem<CH>(tr_row + 4, tr_col);
    if (!DP) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    }

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int n_tiles = (kv_end + BN - 1) / BN;
    const int n_plain = CAUSAL ? min(q0, N) / BN : N / BN;
    issue_tile<0>(0);
    wait_all_and_barrier();
    int j = 0;
    for (; j + 2 <= n_plain; j += 2) {
      step<0, false>(j, n_tiles);
      step<1, false>(j + 1, n_tiles);
    }
    for (; j < n_tiles; j += 2) {
      step<0, true>(j, n_tiles);
      if (j + 1 < n_tiles) step<1, true>(j + 1, n_tiles);
    }

    // this lane holds query myq; the other lane half holds the rest of the row
    float part = 0.f, lp = 0.f;
    if (DP) {
      part = acc;
    } else {
      // O_hp^T: lane holds features 32db + 8(r/4) + 4hi + r%4 of query myq
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * db + 8 * rr + 4 * hi;
          float g4[4], o4[4];
          if (F32IO) {
            const f32x4 gv = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.dout) + qrow + d0);
#pragma unroll
            for (int t = 0; t < 4; ++t) g4[t] = gv[t];
          } else {
            const u32x2 gv = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.dout) + qrow + d0);
            g4[0] = bf16lo_to_f32(gv.x);
            g4[1] = bf16hi_to_f32(gv.x);
            g4[2] = bf16lo_to_f32(gv.y);
            g4[3] = bf16hi_to_f32(gv.y);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) part = fmaf(g4[t], oacc[db][4 * rr + t], part);
          if (SRC == kDeltaErr) {
            // minus the stored-O term, so the sum is delta_lp - delta_hp
            if (F32IO) {
              const f32x4 ov = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + qrow + d0);
#pragma unroll
              for (int t = 0; t < 4; ++t) o4[t] = ov[t];
            } else {
              const u32x2 ov = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.o) + qrow + d0);
              o4[0] = bf16lo_to_f32(ov.x);
              o4[1] = bf16hi_to_f32(ov.x);
              o4[2] = bf16lo_to_f32(ov.y);
              o4[3] = bf16hi_to_f32(ov.y);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) lp = fmaf(g4[t], o4[t], lp);
          }
        }
    }
    float a, b, sa, sb;
    pair32(part, a, b);
    pair32(psum, sa, sb);
    float res = (a + b) / (sa + sb);
    if (SRC == kDeltaErr) {
      float la, lb;
      pair32(lp, la, lb);
      res = (la + lb) - res;
    }
    if (valid && hi == 0) p.delta[(size_t)bh * N + myq] = res;
  }
};

template <int D, bool CAUSAL, int SRC, bool F32IO>
__global__ __launch_bounds__(256, 2) void bwd_delta_kernel(DeltaParams p) {
  using Kt = DeltaKernel<D, CAUSAL, SRC, F32IO>;
  __shared__ __attribute__((aligned(1024))) char k0[Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[Kt::TILE];
  Kt k(p, k0, k1, v0, v1);
  k.run();
}

template <int D, int SRC, bool F32IO>
hipError_t delta_s(const BwdArgs& a, const DeltaParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)(p.BH * p.n_qblocks);
  if (a.causal)
    hipLaunchKernelGGL((bwd_delta_kernel<D, true, SRC, F32IO>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<D, false, SRC, F32IO>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t delta_d(const BwdArgs& a, int src, float* out, hipStream_t stream) {
  DeltaParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.delta = out;
  p.BH = a.B * a.H;
  p.N = a.N;
  p.n_qblocks = (a.N + 127) / 128;
  p.scale = a.scale;
  const bool f32 = a.mode == kFp32Out;
  switch (src) {
    case kDeltaDpP: return f32 ? delta_s<D, kDeltaDpP, true>(a, p, stream) : delta_s<D, kDeltaDpP, false>(a, p, stream);
    case kDeltaOhp: return f32 ? delta_s<D, kDeltaOhp, true>(a, p, stream) : delta_s<D, kDeltaOhp, false>(a, p, stream);
    default: return f32 ? delta_s<D, kDeltaErr, true>(a, p, stream) : delta_s<D, kDeltaErr, false>(a, p, stream);
  }
}

}  // namespace

hipError_t launch_bwd_delta(const BwdArgs& a, int src, float* out, hipStream_t stream) {
  return a.d == 64 ? delta_d<64>(a, src, out, stream) : delta_d<128>(a, src, out, stream);
}

}  // namespace pfa

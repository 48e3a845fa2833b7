// dQ of the backward for gfx950, without atomics.
//
// Method: "Why Low-Precision Transformer Training Fails: An Analysis on Flash
// Attention" (arXiv 2510.04212), paper-graph-ui summary, section 3.4.3: the
// score gradient dS = alpha P o (dP - delta) with dP = dO V^T, and dQ = dS K.
//
// Same work decomposition as the forward kernel: one workgroup of 4 waves per
// (batch*head, block of 128 queries), two workgroups per CU, each wave owning
// 32 queries; key tiles of 64 stream through a double-buffered LDS stage
// filled by direct global->LDS loads.  Per tile and wave:
//   S^T  = K_tile Q^T      dP^T = V_tile dO^T    (MFMA, A = K or V rows from
//                                                 LDS, B = this wave's Q or dO)
//   P = exp(S - LSE), dS = P o (dP - delta)        (VALU; LSE and delta are one
//                                                 value per query, i.e. per lane)
//   dQ^T += K_tile^T dS^T                          (MFMA, A = K read transposed
//                                                 from LDS, B = dS packed to BF16
//                                                 in place from the accumulators)
// The K and V rows of each 32-key block are taken in the order sigma, so the
// accumulators of a lane hold the 8 consecutive keys the last product needs.
#include "pfa_common.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

struct DqParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;   // BF16 dO (the pre-pass copy in the FP32-output mode); unused with DELTA
  const float* lse;
  float* delta;           // read (without DELTA) or written (DELTA)
  uint16_t* dq;
  int BH, N, n_qblocks;
  float scale;
  // DELTA: the kernel forms delta = rowsum(dO o O) itself from O and the
  // caller's dO (FP32 both when f32io, else BF16) and writes it to `delta`;
  // with f32io it also writes the BF16 copy of dO that the dK/dV kernel reads.
  const void* o;
  const void* dout_in;
  uint16_t* dout16;
  int f32io;
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

template <int D, bool CAUSAL, bool DELTA>
struct DqKernel {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int CH = D / 8;
  static constexpr int DC = D / 16;
  static constexpr int KB = BN / 32;
  static constexpr int KC = BN / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BN * D * 2;
  static constexpr int LOADS = TILE / (NT * 16);
  static constexpr int ROWB = CH * 16;

  const DqParams& p;
  // The two stage buffers are separate LDS arrays: the compiler can then tell
  // that the direct loads into one never alias reads of the other, and does
  // not wait for the loads in flight before reading the current buffer.
  char* sm0;
  char* sm1;
  int tid, lane, w, hi, N, bh, qw0, myq, q0;
  size_t base;
  __amdgpu_buffer_rsrc_t krs, vrs;   // this slice of K and V
  int voff[LOADS];
  int kofs[DC];
  int tofs[2][DB];
  u32x4 qreg[DC];
  u32x4 doreg[DC];
  f32x16 dqacc[DB];
  float lse2, dlt;

  __device__ DqKernel(const DqParams& p_, char* s0, char* s1) : p(p_), sm0(s0), sm1(s1) {}

  template <int BUF>
  __device__ __forceinline__ void issue_tile(int j) {
    const int kv0 = j * BN;
    char* kl = BUF ? sm1 : sm0;
    if (kv0 + BN <= N) {
      // whole tile inside the slice: per-lane offsets fixed, tile offset scalar
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        char* dst = kl + (w * LOADS + i) * 1024;
        buf2lds_b128(krs, voff[i], kv0 * D * 2, dst);
        buf2lds_b128(vrs, voff[i], kv0 * D * 2, dst + TILE);
      }
    } else {
      // ragged last tile: rows past the end repeat row N-1 (masked later)
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int slot = (w * LOADS + i) * 64 + lane;
        const int row = slot / CH;
        const int off = voff[i] + (min(kv0 + row, N - 1) - row) * D * 2;
        char* dst = kl + (w * LOADS + i) * 1024;
        buf2lds_b128(krs, off, 0, dst);
        buf2lds_b128(vrs, off, 0, dst + TILE);
      }
    }
  }

  // Tile j for this wave; MASK tiles handle keys after a query of the workgroup
  // (causal) or past the sequence end, the others are fully visible.
  template <int BUF, bool MASK>
  __device__ __forceinline__ void compute_tile(int j) {
    const int kv0 = j * BN;
    if (MASK && !(qw0 < N && (!CAUSAL || kv0 <= qw0 + 31))) return;  // no key of this tile is visible
    tile<BUF, MASK>(kv0);
  }

  template <int BUF, bool MASK>
  __device__ __forceinline__ void tile(int kv0) {
    const char* kl = BUF ? sm1 : sm0;
    const char* vl = kl + TILE;
    f32x16 sacc[KB], pacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x16{};
      pacc[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        sacc[kb] = mfma_bf16(lds_read_b128(kl, kofs[c] + kb * 32 * ROWB), qreg[c], sacc[kb]);
        pacc[kb] = mfma_bf16(lds_read_b128(vl, kofs[c] + kb * 32 * ROWB), doreg[c], pacc[kb]);
      }
    }
    const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - (kv0 + 8 * hi);
    const float c1 = p.scale * kLog2e;
    uint32_t pk[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float d2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          float pr = fast_exp2(fmaf(sacc[kb][r], c1, -lse2));
          if (MASK) {
            const int off = 32 * kb + 16 * (r >> 3) + (r & 7);
            pr = off > lim ? 0.f : pr;
          }
          d2[e] = pr * (pacc[kb][r] - dlt);
        }
        pk[kb][i] = pack_bf16(d2[0], d2[1]);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int kb = kc >> 1, o4 = 4 * (kc & 1);
      const u32x4 bop = u32x4{pk[kb][o4], pk[kb][o4 + 1], pk[kb][o4 + 2], pk[kb][o4 + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a0 = lds_read_tr(kl, tofs[0][db] + kc * 16 * ROWB);
        const u32x2 a1 = lds_read_tr(kl, tofs[1][db] + kc * 16 * ROWB);
        dqacc[db] = mfma_bf16(u32x4{a0.x, a0.y, a1.x, a1.y}, bop, dqacc[db]);
      }
    }
  }

  // DELTA: dO of this lane's query into doreg (converted to BF16 from an FP32
  // dO, whose BF16 copy is stored as well) and delta = rowsum(dO o O), summed
  // in the order of the pre-pass kernel -- a partial sum per 8-feature chunk,
  // then a butterfly over the chunks (c + c^8, then ^4, ^2, ^1 at d = 128) --
  // so that it is bit for bit the pre-pass's delta.  The lane holds chunks
  // 2c + hi: every butterfly step but the last pairs two of its own chunks.
  __device__ __forceinline__ float own_delta(bool valid) {
    float part[DC];
    const size_t row = base + (size_t)myq * D;
    // all of the lane's loads first, then the sums: one wait for the lot
    if (p.f32io) {
      f32x4 oa[DC][2], da[DC][2];
      if (valid) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int col = (2 * c + hi) * 8;
          const f32x4* op = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + row + col);
          const f32x4* dp = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.dout_in) + row + col);
          oa[c][0] = op[0];
          oa[c][1] = op[1];
          da[c][0] = dp[0];
          da[c][1] = dp[1];
        }
      } else {
#pragma unroll
        for (int c = 0; c < DC; ++c) oa[c][0] = oa[c][1] = da[c][0] = da[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += oa[c][0][i] * da[c][0][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += oa[c][1][i] * da[c][1][i];
        part[c] = acc;
        const f32x4 d0 = da[c][0], d1 = da[c][1];
        doreg[c] = u32x4{pack_bf16(d0[0], d0[1]), pack_bf16(d0[2], d0[3]), pack_bf16(d1[0], d1[1]),
                         pack_bf16(d1[2], d1[3])};
        if (valid) *reinterpret_cast<u32x4*>(p.dout16 + row + (2 * c + hi) * 8) = doreg[c];
      }
    } else {
      u32x4 ov[DC];
      if (valid) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int col = (2 * c + hi) * 8;
          ov[c] = ldg_b128(static_cast<const uint16_t*>(p.o) + row + col);
          doreg[c] = ldg_b128(static_cast<const uint16_t*>(p.dout_in) + row + col);
        }
      } else {
#pragma unroll
        for (int c = 0; c < DC; ++c) ov[c] = doreg[c] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc += bf16lo_to_f32(ov[c][i]) * bf16lo_to_f32(doreg[c][i]);
          acc += bf16hi_to_f32(ov[c][i]) * bf16hi_to_f32(doreg[c][i]);
        }
        part[c] = acc;
      }
    }
#pragma unroll
    for (int m = DC / 2; m >= 1; m >>= 1) {
      float nxt[DC];
#pragma unroll
      for (int c = 0; c < DC; ++c) nxt[c] = part[c] + part[c ^ m];
#pragma unroll
      for (int c = 0; c < DC; ++c) part[c] = nxt[c];
    }
    const float dl = part[0] + xchg32(part[0]);
    if (valid && hi == 0) p.delta[(size_t)bh * N + myq] = dl;
    return dl;
  }

  template <int BUF, bool MASK>
  __device__ __forceinline__ void step(int j, int n_tiles) {
    if (j + 1 < n_tiles) issue_tile<1 - BUF>(j + 1);
    compute_tile<BUF, MASK>(j);
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
    const uint16_t* Q = p.q + base;
    krs = make_rsrc(p.k + base, N * D * 2);
    vrs = make_rsrc(p.v + base, N * D * 2);
    q0 = qb * BM;
    qw0 = q0 + 32 * w;
    myq = qw0 + (lane & 31);
    const bool valid = myq < N;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (w * LOADS + i) * 64 + lane;
      const int row = slot / CH, pchunk = slot % CH;
      voff[i] = (row * D + (pchunk ^ swz_pattern<CH>(row)) * 8) * 2;
    }
    // the first K/V tile's loads go out first: the wait for this lane's rows
    // (and, with DELTA, for O before delta is summed) then overlaps them
    issue_tile<0>(0);

#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int col = (2 * c + hi) * 8;
      qreg[c] = valid ? ldg_b128(Q + (size_t)myq * D + col) : u32x4{0, 0, 0, 0};
      if (!DELTA) doreg[c] = valid ? ldg_b128(p.dout + base + (size_t)myq * D + col) : u32x4{0, 0, 0, 0};
    }
    if (DELTA) dlt = own_delta(valid);
    else dlt = valid ? p.delta[(size_t)bh * N + myq] : 0.f;
    lse2 = valid ? p.lse[(size_t)bh * N + myq] * kLog2e : __builtin_inff();
    const int krow = sigma32(lane & 31);
#pragma unroll
    for (int c = 0; c < DC; ++c) kofs[c] = swz<CH>(krow, 2 * c + hi);
    const int g = lane >> 4, s = lane & 15;
    const int tr_row = 8 * (g >> 1) + (s >> 2);
    const int tr_col = 16 * (g & 1) + 4 * (s & 3);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db) tofs[hh][db] = swz_elem<CH>(tr_row + 4 * hh, 32 * db + tr_col);
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int n_tiles = (kv_end + BN - 1) / BN;
    wait_all_and_barrier();
    // Leading tiles that need no mask for any wave of the workgroup (all keys
    // before the first query, none past N) run unmasked, in pairs so that the
    // buffer index stays a compile-time constant; the rest run masked.
    const int n_plain = CAUSAL ? min(q0, N) / BN : N / BN;
    int j = 0;
    for (; j + 2 <= n_plain; j += 2) {
      step<0, false>(j, n_tiles);
      step<1, false>(j + 1, n_tiles);
    }
    for (; j < n_tiles; j += 2) {
      step<0, true>(j, n_tiles);
      if (j + 1 < n_tiles) step<1, true>(j + 1, n_tiles);
    }
    // dQ = scale * dQ^T; lane holds query myq, features 32db + 8(r/4) + 4hi + r%4
    if (!valid) return;
    const size_t orow = base + (size_t)myq * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * hi;
        const u32x2 out = {pack_bf16(sc * dqacc[db][4 * rr], sc * dqacc[db][4 * rr + 1]),
                           pack_bf16(sc * dqacc[db][4 * rr + 2], sc * dqacc[db][4 * rr + 3])};
        *reinterpret_cast<u32x2*>(p.dq + orow + d0) = out;
      }
  }
};

template <int D, bool CAUSAL, bool DELTA>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(DqParams p) {
  using Kt = DqKernel<D, CAUSAL, DELTA>;
  __shared__ __attribute__((aligned(1024))) char s0[2 * Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char s1[2 * Kt::TILE];
  Kt k(p, s0, s1);
  k.run();
}

template <int D, bool DELTA>
hipError_t dq_d(const BwdArgs& a, hipStream_t stream) {
  DqParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = a.mode == kFp32Out ? a.dout16 : static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.BH = a.B * a.H;
  p.N = a.N;
  p.n_qblocks = (a.N + 127) / 128;
  p.scale = a.scale;
  p.o = a.o;
  p.dout_in = a.dout;
  p.dout16 = a.dout16;
  p.f32io = a.mode == kFp32Out ? 1 : 0;
  const unsigned grid = (unsigned)(p.BH * p.n_qblocks);
  if (a.causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, DELTA>), dim3(grid), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, false, DELTA>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? dq_d<64, false>(a, stream) : dq_d<128, false>(a, stream);
}

hipError_t launch_bwd_dq_delta(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? dq_d<64, true>(a, stream) : dq_d<128, true>(a, stream);
}

}  // namespace pfa

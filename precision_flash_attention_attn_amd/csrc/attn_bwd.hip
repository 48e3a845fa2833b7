// Backward flash attention for gfx950: delta pre-pass and the dK/dV kernel.
//
// Method: "Why Low-Precision Transformer Training Fails: An Analysis on Flash
// Attention" (arXiv 2510.04212), paper-graph-ui summary, section 3.4.2 (the
// backward computes delta = rowsum(dO o O) and dS = P o (dP - delta)) and
// section 3.4.3 (dS = alpha P o (dP - delta), dQ = dS K).  dK = alpha dS^T Q and
// dV = P^T dO are the matching gradients of the same products.
//
//   bwd_pre      delta = rowsum(dO o O) in FP32 (O, dO BF16, or FP32 in the
//                FP32-output mode, where it also writes a BF16 copy of dO for
//                the MFMA operands of the gradient kernels).
//   bwd_dkdv     one workgroup per (batch*head, block of 128 keys at d = 128,
//                64 at d = 64); query tiles stream through a double-buffered
//                LDS stage.  Split geometry: tiles of 64 queries, two waves per
//                32 keys each take one 32-query half and accumulate partial
//                dK^T, dV^T, summed through LDS at the end.  Unsplit geometry
//                (d = 128 with B*H >= 32): tiles of 32 queries, one wave per 32
//                keys, two workgroups per CU.  Per wave and tile:
//                  S = Q K^T, dP = dO V^T          (A from LDS; B = K^T from the
//                                                   key block in LDS, V^T in VGPRs)
//                  P = exp(S - LSE), dS = P o (dP - delta)          (VALU)
//                  dV^T += dO^T P, dK^T += Q^T dS  (A read transposed from LDS,
//                                                   B = P, dS packed in place)
// dQ is computed by its own kernel (attn_bwd_dq.hip), so no atomics are used
// and every gradient is bitwise reproducible.
#include "pfa_common.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

// ---------------------------------------------------------------------------
// delta = rowsum(dO o O); in the FP32-output mode also a BF16 copy of dO for
// the gradient kernels' MFMA operands.
template <int D, bool F32IO>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const void* __restrict__ o,
                                                      const void* __restrict__ dout,
                                                      float* __restrict__ delta,
                                                      uint16_t* __restrict__ dout16, size_t rows) {
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
      *reinterpret_cast<u32x4*>(dout16 + off) =
          u32x4{pack_bf16(d0[0], d0[1]), pack_bf16(d0[2], d0[3]), pack_bf16(d1[0], d1[1]),
                pack_bf16(d1[2], d1[3])};
    } else {
      const u32x4 ov = ldg_b128(static_cast<const uint16_t*>(o) + off);
      const u32x4 dv = ldg_b128(static_cast<const uint16_t*>(dout) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += bf16lo_to_f32(ov[i]) * bf16lo_to_f32(dv[i]);
        acc += bf16hi_to_f32(ov[i]) * bf16hi_to_f32(dv[i]);
      }
    }
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

struct DkdvParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;   // BF16 dO (the pre-pass copy in the FP32-output mode)
  const float* lse;
  const float* delta;
  uint16_t* dk;
  uint16_t* dv;
  int BH, N, n_kvblocks;
  float scale;
};

__device__ __forceinline__ void map_kv_block(int bid, int BH, int& bh, int& kb) {
  // under a causal mask the first key blocks see the most queries: they go first;
  // slices are grouped per XCD when their number is a multiple of 8
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, idx = bid >> 3, hp = BH >> 3;
    bh = xcd * hp + idx % hp;
    kb = idx / hp;
  } else {
    bh = bid % BH;
    kb = bid / BH;
  }
}

template <int D, bool CAUSAL, bool SPLIT>
struct DkdvKernel {
  // d = 128: 128 keys, 8 waves, one workgroup per CU; d = 64: 64 keys, 4
  // waves, three workgroups per CU (the short sequences of the d = 64 shapes
  // need the smaller blocks to fill the CUs).
  // Two geometries.  SPLIT: 64-query tiles, the two waves of a 32-key group
  // take one half each and sum their partial gradients at the end (d = 128:
  // 128 keys, 8 waves, one workgroup per CU; d = 64: 64 keys, 4 waves, three
  // workgroups per CU -- the short sequences of the d = 64 shapes need the
  // smaller blocks to fill the CUs).  Not SPLIT (d = 128 only): 32-query
  // tiles, one wave per 32 keys takes the whole tile, two workgroups per CU,
  // so the two waves on a SIMD belong to different workgroups and share no
  // barrier.  The launcher picks the second when B*H >= 32 (measured: it is
  // 2-11% faster there, 2-4% slower with 8 or 16 slices).
  static_assert(SPLIT || D == 128, "the unsplit geometry is built for d = 128");
  static constexpr int BKV = D == 128 ? 128 : 64, BQ = SPLIT ? 64 : 32;
  static constexpr int KG = BKV / 32;                // key groups of 32
  static constexpr int NT = (SPLIT ? 2 : 1) * KG * 64;
  static constexpr int MIN_WG = D == 128 ? (SPLIT ? 1 : 2) : 3;
  static constexpr int CH = D / 8;
  static constexpr int DC = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = CH * 16;
  static constexpr int QT = BQ * D * 2;              // bytes of a Q (or dO) tile
  static constexpr int KBLK = BKV * D * 2;           // bytes of the key block
  static constexpr int STAT = 2 * BQ * 4;            // LSE and delta of a query tile
  static constexpr int BUFB = STAT + 2 * QT;         // one tile buffer: LSE, delta, Q, dO
  static constexpr int LOADS = QT / (NT * 16);       // direct loads per thread per tile
  static constexpr int KLOADS = KBLK / (NT * 16);    // direct loads per thread for the key block

  const DkdvParams& p;
  // Separate LDS arrays for the key block and the two stage buffers: the
  // compiler can then tell that the direct loads into one buffer never alias
  // reads of the other and does not wait for the loads in flight.
  char* kls;
  char* sm0;
  char* sm1;
  int tid, lane, w, hi, kb, qh, N, bh, kv0, kw0, mykey, qt_begin;
  size_t base;
  __amdgpu_buffer_rsrc_t qrs, dors, lrs, drs;   // this slice of Q, dO, LSE, delta
  int voff[LOADS];   // byte offset in a tile of this lane's direct loads
  // LDS offsets of the operand reads at contraction step 0 (feature block 0):
  // Q / dO rows of this wave's query half, K rows of its keys, and the two
  // transpose reads.  Step c (block db) is the offset XOR 32c (XOR 64db), as
  // the swizzle only permutes chunks inside a row.
  int abase, kbase, tbase[2];
  u32x4 vreg[DC];
  f32x16 dvacc[DB], dkacc[DB];

  __device__ DkdvKernel(const DkdvParams& p_, char* kl_, char* s0, char* s1)
      : p(p_), kls(kl_), sm0(s0), sm1(s1) {}

  // Direct loads of the query tile at qt0 (Q, dO, LSE, delta) into buffer BUF.
  template <int BUF>
  __device__ __forceinline__ void issue_tile(int qt0) {
    char* bl = BUF ? sm1 : sm0;
    if (qt0 + BQ <= N) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        char* dst = bl + STAT + (w * LOADS + i) * 1024;
        buf2lds_b128(qrs, voff[i], qt0 * D * 2, dst);
        buf2lds_b128(dors, voff[i], qt0 * D * 2, dst + QT);
      }
      if (w < 2 && lane < BQ)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w == 0 ? lrs : drs,
                                                 (__attribute__((address_space(3))) void*)(bl + w * BQ * 4),
                                                 4, lane * 4, qt0 * 4, 0, 0);
    } else {
      // ragged last tile: rows past the end repeat row N-1 (masked later)
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int row = ((w * LOADS + i) * 64 + lane) / CH;
        const int off = voff[i] + (min(qt0 + row, N - 1) - row) * D * 2;
        char* dst = bl + STAT + (w * LOADS + i) * 1024;
        buf2lds_b128(qrs, off, 0, dst);
        buf2lds_b128(dors, off, 0, dst + QT);
      }
      if (w < 2 && lane < BQ)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w == 0 ? lrs : drs,
                                                 (__attribute__((address_space(3))) void*)(bl + w * BQ * 4),
                                                 4, min(qt0 + lane, N - 1) * 4, 0, 0, 0);
    }
  }

  // One query tile for this wave.  MASK tiles handle queries before a key of
  // the block (causal) and queries or keys past the end; the others need no mask.
  template <int BUF, bool MASK>
  __device__ __forceinline__ void compute_tile(int qt0) {
    const char* kl = kls;
    const char* sb = BUF ? sm1 : sm0;
    const float* sl = reinterpret_cast<const float*>(sb);
    const float* tl = sl + BQ;
    const char* ql = sb + STAT;
    const char* dl = ql + QT;
    const int qw = qt0 + 32 * qh;   // first query of this wave's half
    if (MASK && CAUSAL && qw + 31 < kw0) return;   // every query of the half precedes every key
    // The per-step offsets are rebuilt from the bases in every tile (one XOR
    // each): kept live across the loop they would push the kernel past 256
    // VGPRs.  The empty asm hides the bases' values so the XORs stay here.
    int ab = abase, kbs = kbase, t0 = tbase[0], t1 = tbase[1];
    asm volatile("" : "+v"(ab), "+v"(kbs), "+v"(t0), "+v"(t1));
    // S = Q K^T and dP = dO V^T; rows: queries (sigma order), columns: keys
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    // Wave priority 1 while the MFMA phases issue, 0 for the VALU phase: the
    // other wave on the SIMD then fills the matrix core's gaps with its
    // softmax work rather than competing with these products for issue.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      sacc = mfma_bf16(lds_read_b128(ql, ab ^ (32 * c)), lds_read_b128(kl, kbs ^ (32 * c)), sacc);
      pacc = mfma_bf16(lds_read_b128(dl, ab ^ (32 * c)), vreg[c], pacc);
    }
    __builtin_amdgcn_s_setprio(0);
    // P = exp(S - LSE) and dS = P o (dP - delta), packed to BF16
    const float c1 = p.scale * kLog2e;
    uint32_t pP[8], pS[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int qi = 32 * qh + 16 * hh + 8 * hi;  // 8 consecutive queries of the tile
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(sl + qi);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(sl + qi + 4);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(tl + qi);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(tl + qi + 4);
      // query qt0 + qi + e is visible to this key when e >= vis, and exists when e < qend
      const int vis = CAUSAL ? mykey - (qt0 + qi) : -8;
      const int qend = N - (qt0 + qi);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float pr[2], ds[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 8 * hh + e + u;
          const float lse = (e + u) < 4 ? l0[e + u] : l1[e + u - 4];
          const float dlt = (e + u) < 4 ? d0[e + u] : d1[e + u - 4];
          float pv = fast_exp2(fmaf(sacc[r], c1, -lse * kLog2e));
          if (MASK) pv = ((e + u) >= vis && (e + u) < qend && mykey < N) ? pv : 0.f;
          pr[u] = pv;
          ds[u] = pv * (pacc[r] - dlt);
        }
        pP[4 * hh + e / 2] = pack_bf16(pr[0], pr[1]);
        pS[4 * hh + e / 2] = pack_bf16(ds[0], ds[1]);
      }
    }
    __builtin_amdgcn_s_setprio(1);
    // dV^T += dO^T P, dK^T += Q^T dS over the half's 32 queries (two 16-query steps)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int o4 = 4 * h2;
      const u32x4 bP = u32x4{pP[o4], pP[o4 + 1], pP[o4 + 2], pP[o4 + 3]};
      const u32x4 bS = u32x4{pS[o4], pS[o4 + 1], pS[o4 + 2], pS[o4 + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a0 = lds_read_tr(dl, (t0 ^ (64 * db)) + h2 * 16 * ROWB);
        const u32x2 a1 = lds_read_tr(dl, (t1 ^ (64 * db)) + h2 * 16 * ROWB);
        dvacc[db] = mfma_bf16(u32x4{a0.x, a0.y, a1.x, a1.y}, bP, dvacc[db]);
        const u32x2 b0 = lds_read_tr(ql, (t0 ^ (64 * db)) + h2 * 16 * ROWB);
        const u32x2 b1 = lds_read_tr(ql, (t1 ^ (64 * db)) + h2 * 16 * ROWB);
        dkacc[db] = mfma_bf16(u32x4{b0.x, b0.y, b1.x, b1.y}, bS, dkacc[db]);
      }
    }
  }

  // Tile t of the loop (query tile qt_begin + t * BQ): start the loads of tile
  // t + 1 into the other buffer, compute tile t, then wait for both.
  template <int BUF, bool MASK>
  __device__ __forceinline__ void step(int t, int n_tiles) {
    if (t + 1 < n_tiles) issue_tile<1 - BUF>(qt_begin + (t + 1) * BQ);
    compute_tile<BUF, MASK>(qt_begin + t * BQ);
    __builtin_amdgcn_s_setprio(0);
    wait_all_and_barrier();
  }

  // Sum the partial accumulators of waves w and w + KG (same keys, other query
  // half) through LDS and store the gradient from waves 0..KG-1.  The exchange
  // area (DB x 16 floats x 64 lanes per key group) of key groups 0, 1 is in
  // buffer 0, of groups 2, 3 in buffer 1.
  __device__ __forceinline__ void reduce_store(f32x16* acc, uint16_t* out, float mul) {
    if constexpr (!SPLIT) {
      if (mykey < N) {
        const size_t krow = base + (size_t)mykey * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * hi;
            const u32x2 v = {pack_bf16(mul * acc[db][4 * j], mul * acc[db][4 * j + 1]),
                             pack_bf16(mul * acc[db][4 * j + 2], mul * acc[db][4 * j + 3])};
            *reinterpret_cast<u32x2*>(out + krow + d0) = v;
          }
      }
      return;
    }
    f32x4* red = reinterpret_cast<f32x4*>(kb < 2 ? sm0 : sm1);
    const int kg = kb & 1;
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          red[((kg * DB + db) * 4 + j) * 64 + lane] =
              f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
    }
    __syncthreads();
    if (qh == 0 && mykey < N) {
      const size_t krow = base + (size_t)mykey * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 o = red[((kg * DB + db) * 4 + j) * 64 + lane];
          const int d0 = 32 * db + 8 * j + 4 * hi;
          const u32x2 v = {pack_bf16(mul * (acc[db][4 * j] + o[0]), mul * (acc[db][4 * j + 1] + o[1])),
                           pack_bf16(mul * (acc[db][4 * j + 2] + o[2]), mul * (acc[db][4 * j + 3] + o[3]))};
          *reinterpret_cast<u32x2*>(out + krow + d0) = v;
        }
    }
    __syncthreads();
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    hi = lane >> 5;
    kb = SPLIT ? w % KG : w;
    qh = SPLIT ? w / KG : 0;
    N = p.N;
    int kvb;
    map_kv_block(blockIdx.x, p.BH, bh, kvb);
    base = (size_t)bh * N * D;
    const uint16_t* K = p.k + base;
    const uint16_t* V = p.v + base;
    qrs = make_rsrc(p.q + base, N * D * 2);
    dors = make_rsrc(p.dout + base, N * D * 2);
    lrs = make_rsrc(p.lse + (size_t)bh * N, N * 4);
    drs = make_rsrc(p.delta + (size_t)bh * N, N * 4);
    kv0 = kvb * BKV;
    kw0 = kv0 + 32 * kb;
    mykey = kw0 + (lane & 31);

    // the key block into LDS (rows = keys, swizzled), V of this wave's keys into VGPRs
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int slot = (w * KLOADS + i) * 64 + lane;
      const int row = slot / CH, pchunk = slot % CH;
      const int key = min(kv0 + row, N - 1);
      g2lds_b128(K + (size_t)key * D + (pchunk ^ swz_pattern<CH>(row)) * 8,
                 kls + (w * KLOADS + i) * 1024);
    }
#pragma unroll
    for (int c = 0; c < DC; ++c)
      vreg[c] = mykey < N ? ldg_b128(V + (size_t)mykey * D + (2 * c + hi) * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (w * LOADS + i) * 64 + lane;
      const int row = slot / CH, pchunk = slot % CH;
      voff[i] = (row * D + (pchunk ^ swz_pattern<CH>(row)) * 8) * 2;
    }
    const int arow = 32 * qh + sigma32(lane & 31);
    abase = swz<CH>(arow, hi);
    kbase = swz<CH>(32 * kb + (lane & 31), hi);
    const int g = lane >> 4, s = lane & 15;
    const int tr_row = 32 * qh + 8 * (g >> 1) + (s >> 2);
    const int tr_col = 16 * (g & 1) + 4 * (s & 3);
    tbase[0] = swz_elem<CH>(tr_row, tr_col);
    tbase[1] = swz_elem<CH>(tr_row + 4, tr_col);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dvacc[db] = f32x16{};
      dkacc[db] = f32x16{};
    }

    // Query tiles qt_begin + t * BQ, t < n_tiles.  Under a causal mask the first
    // two overlap the key block and need the mask; a ragged last tile needs it
    // for the queries past N.  The tiles in between run unmasked, in pairs so
    // that the buffer index stays a compile-time constant.
    qt_begin = CAUSAL ? kv0 : 0;
    const int n_tiles = (N - qt_begin + BQ - 1) / BQ;
    const int n_full = (N - qt_begin) / BQ;
    // tiles that overlap the key block need the causal mask: BKV / BQ of them (an even count)
    const int n_lead = CAUSAL ? min(BKV / BQ < 2 ? 2 : BKV / BQ, n_tiles) : 0;
    if (n_tiles > 0) issue_tile<0>(qt_begin);
    wait_all_and_barrier();
    int t = 0;
    for (; t + 2 <= n_lead; t += 2) {
      step<0, true>(t, n_tiles);
      step<1, true>(t + 1, n_tiles);
    }
    if (t == n_lead)
      for (; t + 2 <= n_full; t += 2) {
        step<0, false>(t, n_tiles);
        step<1, false>(t + 1, n_tiles);
      }
    for (; t < n_tiles; t += 2) {
      step<0, true>(t, n_tiles);
      if (t + 1 < n_tiles) step<1, true>(t + 1, n_tiles);
    }
    reduce_store(dvacc, p.dv, 1.f);
    reduce_store(dkacc, p.dk, p.scale);
  }
};

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__((DkdvKernel<D, CAUSAL, SPLIT>::NT),
                             (DkdvKernel<D, CAUSAL, SPLIT>::MIN_WG)) void bwd_dkdv_kernel(DkdvParams p) {
  using Kt = DkdvKernel<D, CAUSAL, SPLIT>;
  constexpr int RED = 2 * (D / 32) * 4 * 64 * 16;   // exchange area of two key groups
  static_assert(!SPLIT || RED <= Kt::BUFB, "the exchange area must fit one tile buffer");
  __shared__ __attribute__((aligned(1024))) char kl[Kt::KBLK];
  __shared__ __attribute__((aligned(1024))) char s0[Kt::BUFB];
  __shared__ __attribute__((aligned(1024))) char s1[Kt::BUFB];
  Kt k(p, kl, s0, s1);
  k.run();
}

template <int D>
hipError_t prep_d(const BwdArgs& a, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  constexpr int RPB = 256 / (D / 8);
  const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
  if (a.mode == kFp32Out)
    hipLaunchKernelGGL((bwd_pre_kernel<D, true>), dim3(grid), dim3(256), 0, stream, a.o, a.dout,
                       a.delta, a.dout16, rows);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<D, false>), dim3(grid), dim3(256), 0, stream, a.o, a.dout,
                       a.delta, nullptr, rows);
  return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t dkdv_launch(DkdvParams p, const BwdArgs& a, hipStream_t stream) {
  using Kt = DkdvKernel<D, true, SPLIT>;
  p.n_kvblocks = (a.N + Kt::BKV - 1) / Kt::BKV;
  const unsigned grid = (unsigned)(p.BH * p.n_kvblocks);
  if (a.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, SPLIT>), dim3(grid), dim3(Kt::NT), 0, stream, p);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, SPLIT>), dim3(grid), dim3(Kt::NT), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_d(const BwdArgs& a, hipStream_t stream) {
  DkdvParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = a.mode == kFp32Out ? a.dout16 : static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.BH = a.B * a.H;
  p.N = a.N;
  p.scale = a.scale;
  if constexpr (D == 128)
    if (p.BH >= 32) return dkdv_launch<D, false>(p, a, stream);
  return dkdv_launch<D, true>(p, a, stream);
}

}  // namespace

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? prep_d<64>(a, stream) : prep_d<128>(a, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? dkdv_d<64>(a, stream) : dkdv_d<128>(a, stream);
}

}  // namespace pfa

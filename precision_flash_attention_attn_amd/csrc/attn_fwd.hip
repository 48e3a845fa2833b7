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
// Work decomposition: one workgroup per (batch*head, block of queries): 8
// waves over 256 queries and one workgroup per CU at d = 128 with fewer than
// 32 (batch, head) slices, else 4 waves over 128 queries and two workgroups
// per CU (two waves per SIMD either way); each wave owns 32 queries, and every
// K/V tile staged in LDS serves the whole block.  Keys stream in
// tiles of 64 through double-buffered LDS stages filled by direct
// global->LDS loads.  Per tile and wave:
//   S^T (64 keys x 32 queries) = K_tile Q^T   (MFMA, A = K rows from LDS,
//                                              B = the wave's Q held in VGPRs)
//   online row maximum / top-2 / shift / exp on the accumulators (VALU)
//   O^T (d x 32 queries) += V_tile^T P-bar^T   (MFMA, A = V read transposed from
//                                              LDS, B = P-bar packed to BF16 in
//                                              place from the S accumulators)
// The K rows of each 32-key block are fed to the MFMA in the order sigma (see
// sigma32) so that the accumulator registers of a lane already hold the 8
// consecutive keys the P-bar V step needs as its B operand: P-bar never goes
// through LDS.
//
// Scores are kept as the raw dot products q.k in the accumulators.  S =
// fp32(dot * scale) is monotone in the dot, so the row maximum and the second
// largest score of S are the scaled maximum and second largest dot; only those
// two are scaled, which gives bit for bit the S-based tie test of the pages.
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
  // +inf and -inf, passed in so that max(a, b) = med3(a, b, +inf) and
  // min(a, b) = med3(a, b, -inf) stay single v_med3_f32 instructions (a
  // literal infinity is folded back into fmaxf/fminf, which the compiler
  // surrounds with NaN-quieting copies of both operands)
  float pinf, ninf;
  // Per-head selection: when `filter` is set, only heads h (of H) whose bit
  // is set in hmask run; the others' workgroups exit at once.  o_f32: write
  // O as FP32 (the BF16 result widened exactly in the BF16 modes).
  int H, filter, o_f32;
  uint64_t hmask[4];
  int32_t* pbar_one;     // diagnostic variant: per-row count of P-bar entries equal to 1
  float* o_one;          // diagnostic variant: the part of O from those entries (NULL: skip)
  float one_thr;         // the smallest FP32 d with bf16(fp32(exp(d))) = 1 (P-bar rounds to 1)
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

// DIAG (a diagnostic variant, always with FLAGS): also count, per row, the
// P-bar entries that round to 1 in BF16 -- the P-bar = 1 additions the pages'
// cumulative-error trace singles out (section 3.4.4, "Why P-bar = 1 is the
// critical condition") -- and accumulate the part of O-bar they carry (their
// V rows, rescaled with O-bar), kept apart from the rest.  The decision
// follows the method's definition of P-bar rather than the fast exponent of
// the product: S = fp32(dot * scale), d = fp32(S - m), and P-bar rounds to 1
// exactly when fp32(exp(d)) >= 1 - 2^-9 (exp correctly rounded), i.e.
// d >= one_thr.  The same entries are
// counted in every mode (in the FP32-output mode they enter the product as
// hi + lo within 2^-9 of 1).
// Largest element of x: one v_max3_f32 per two elements.
template <int N>
struct MaxAll {
  static __device__ __forceinline__ float run(const float (&x)[N]) {
    float r = x[0];
    int i = 1;
#pragma unroll
    for (; i + 1 < N; i += 2) r = __builtin_fmaxf(__builtin_fmaxf(r, x[i]), x[i + 1]);
    if (i < N) r = __builtin_fmaxf(r, x[i]);
    return r;
  }
};

// Largest (t1) and second largest (t2) element of x, as a multiset: t2 = t1
// when the maximum occurs twice.  Each group of three gives its maximum
// (v_max3_f32) and median (v_med3_f32); the second largest element is then
// the larger of the largest median and the second largest group maximum,
// found the same way one level up.  About 1.3 instructions per element
// instead of 2 for a running pair.  hv, lv: +inf and -inf (see FwdParams).
template <int N>
struct Top2 {
  static constexpr int G = N / 3, R = N % 3, M = G + (R ? 1 : 0), NB = G + (R == 2 ? 1 : 0);
  static __device__ __forceinline__ void run(const float (&x)[N], float& t1, float& t2, float hv, float lv) {
    float a[M], b[NB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      a[g] = __builtin_fmaxf(__builtin_fmaxf(x[3 * g], x[3 * g + 1]), x[3 * g + 2]);
      b[g] = med3(x[3 * g], x[3 * g + 1], x[3 * g + 2]);
    }
    if (R == 2) {
      a[G] = med3(x[N - 2], x[N - 1], hv);
      b[G] = med3(x[N - 2], x[N - 1], lv);
    } else if (R == 1) {
      a[G] = x[N - 1];
    }
    float s2;
    Top2<M>::run(a, t1, s2, hv, lv);
    t2 = __builtin_fmaxf(s2, MaxAll<NB>::run(b));
  }
};
template <>
struct Top2<1> {
  static __device__ __forceinline__ void run(const float (&x)[1], float& t1, float& t2, float, float lv) {
    t1 = x[0];
    t2 = lv;
  }
};
template <>
struct Top2<2> {
  static __device__ __forceinline__ void run(const float (&x)[2], float& t1, float& t2, float hv, float lv) {
    t1 = med3(x[0], x[1], hv);
    t2 = med3(x[0], x[1], lv);
  }
};
template <>
struct Top2<3> {
  static __device__ __forceinline__ void run(const float (&x)[3], float& t1, float& t2, float, float) {
    t1 = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), x[2]);
    t2 = med3(x[0], x[1], x[2]);
  }
};

template <int D, int MODE, bool CAUSAL, bool FLAGS, bool DIAG, bool WIDE>
struct FwdKernel {
  // WIDE (d = 128 with fewer than 32 (batch, head) slices): 8 waves over 256
  // queries, one workgroup per CU, every K/V tile serving 256 queries.
  // Otherwise 4 waves over 128 queries, two workgroups per CU, whose waves
  // share a SIMD without sharing a barrier; with 32 or more slices, or the
  // short sequences of the d = 64 shapes, that balances better (measured at
  // d = 128: 4-11% faster from 32 slices up, 2.4% slower at B1 H16 N8192).
  // Two waves per SIMD either way.
  static_assert(!WIDE || D == 128, "the 256-query geometry is built for d = 128");
  static constexpr int BM = WIDE ? 256 : 128, BN = 64, NT = BM * 2;
  // The diagnostic variant keeps a second O-bar accumulator: one workgroup
  // per CU, so each wave may hold up to 512 registers.
  static constexpr int MIN_WG = (WIDE || DIAG) ? 1 : 2;
  static constexpr int CH = D / 8;    // 16-byte chunks per K/V row
  static constexpr int DC = D / 16;   // contraction steps of K Q^T
  static constexpr int KB = BN / 32;  // 32-key blocks per tile
  static constexpr int KC = BN / 16;  // 16-key contraction steps of V^T P^T
  static constexpr int DB = D / 32;   // 32-feature blocks of O
  static constexpr bool TIE = MODE == kTieAware;
  static constexpr bool HP = MODE == kFp32Out;
  static constexpr int TILE = BN * D * 2;            // bytes of one K (or V) tile
  static constexpr int LOADS = TILE / (NT * 16);     // direct loads per thread per tile and tensor
  static constexpr int ROWB = CH * 16;               // bytes per LDS row

  const FwdParams& p;
  // K and V tiles are staged in two buffers each, four separate LDS arrays:
  // the compiler can then tell that the direct loads into one never alias
  // reads of another, and does not wait for loads in flight before a read.
  char* kb0;
  char* kb1;
  char* vb0;
  char* vb1;
  int tid, lane, w, hi, N, bh, qw0, myq, q0;
  size_t base;
  __amdgpu_buffer_rsrc_t krs, vrs;  // this slice of K and V
  int voff[LOADS];       // byte offset in a tile, (row * D + swizzled chunk * 8) * 2, of this lane's direct loads
  // LDS byte offsets of the K operand read (32-key block 0, contraction step
  // 0) and of the two V transpose reads (16-key step 0, feature block 0);
  // step c (block db) is the offset XOR 32c (XOR 64db), as the swizzle only
  // permutes the chunks inside a row.
  int kbase, vbase0, vbase1;
  u32x4 qreg[DC];
  f32x16 oacc[DB];
  f32x16 scur[KB];       // raw dot products of the tile whose P-bar is next
  float Mraw, M2raw, m, mb, alpha, lsum;
  bool flag;
  int n_one;             // DIAG: this lane's count of P-bar == 1
  f32x16 oone[DIAG ? DB : 1];  // DIAG: O-bar^T of the P-bar == 1 entries alone

  __device__ FwdKernel(const FwdParams& p_, char* k0, char* k1, char* v0, char* v1)
      : p(p_), kb0(k0), kb1(k1), vb0(v0), vb1(v1) {}

  // Direct loads of rows j*BN .. j*BN + 63 of X (K or V) into dst; rows past
  // the end of a ragged last tile repeat row N-1 (their scores are masked).
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
  template <int B> __device__ __forceinline__ void issue_k(int j) { issue(krs, j, B ? kb1 : kb0); }
  template <int B> __device__ __forceinline__ void issue_v(int j) { issue(vrs, j, B ? vb1 : vb0); }

  // S^T (64 keys x 32 queries) = K_tile Q^T from K buffer B.
  template <int B>
  __device__ __forceinline__ void qk(f32x16 (&s)[KB]) {
    const char* kl = B ? kb1 : kb0;
    int kbs = kbase;
    asm volatile("" : "+v"(kbs));   // keep the per-step XORs here, not in live registers
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c)
        s[kb] = mfma_bf16(lds_read_b128(kl, (kbs ^ (32 * c)) + kb * 32 * ROWB), qreg[c], s[kb]);
    }
  }

  // Keys after the query (causal) or past the sequence end get -inf.
  __device__ __forceinline__ void mask(f32x16 (&s)[KB], int kv0) {
    const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - (kv0 + 8 * hi);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * kb + 16 * (r >> 3) + (r & 7);
        s[kb][r] = off > lim ? kNegInf : s[kb][r];
      }
  }

  // Running maximum (and second largest, as a multiset) of the raw dot
  // products, then the S-unit maximum, tie flag and shift (section 3.4.5):
  // sets m, mb = m log2 e and alpha = exp(m_old - m) for the tile s.
  __device__ __forceinline__ void update_max(const f32x16 (&s)[KB]) {
    // No contraction here: the compiler would otherwise fuse m - Mraw*scale
    // (and Ms - M2raw*scale) into one fma with the unrounded product, so an
    // unchanged maximum would give alpha = exp2(rounding residue) != 1 (and
    // l and O-bar would drift by an ulp per tile), and the tie test would
    // not use the rounded S values it is defined on.
#pragma clang fp contract(off)
    const float hv = p.pinf, lv = p.ninf;
    float x[16 * KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[16 * kb + r] = s[kb][r];
    float t1, t2 = kNegInf;
    if (FLAGS) Top2<16 * KB>::run(x, t1, t2, hv, lv);
    else t1 = MaxAll<16 * KB>::run(x);
    // combine the two lane halves that share a query
    float a1, b1;
    pair32(t1, a1, b1);
    const float tmax = med3(a1, b1, hv);
    if (FLAGS) {
      float a2, b2;
      pair32(t2, a2, b2);
      t2 = med3(med3(a1, b1, lv), med3(a2, b2, hv), hv);
      M2raw = med3(med3(Mraw, tmax, lv), med3(M2raw, t2, hv), hv);
    }
    Mraw = med3(Mraw, tmax, hv);
    const float Ms = Mraw * p.scale;
    if (FLAGS) flag = (M2raw != kNegInf) && (Ms - M2raw * p.scale <= p.eps);
    float m_new = Ms;
    if (TIE && flag) m_new = (Ms > 0.f) ? p.beta * Ms : ((Ms < 0.f) ? 0.f : Ms);
    alpha = 1.f;
    if (m_new != kNegInf) {
      alpha = (m == kNegInf) ? 0.f : fast_exp2((m - m_new) * kLog2e);
      mb = m_new * kLog2e;
      m = m_new;
    }
  }

  // O-bar *= alpha, skipped when no query of the wave changed its maximum.
  __device__ __forceinline__ void rescale() {
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      if (DIAG)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oone[db][r] *= alpha;
    }
  }

  // DIAG: 1 when the score with raw dot product x gives a P-bar that rounds to
  // 1 in BF16 under the current shift m (see the DIAG note above).
  __device__ __forceinline__ uint32_t is_one(float x) {
#pragma clang fp contract(off)
    const float sv = x * p.scale;
    const float dv = sv - m;
    return dv >= p.one_thr ? 1u : 0u;
  }

  // P-bar = exp(S - m) rounded to BF16 (plus the BF16 remainder in the FP32
  // output mode), and l = l alpha + its row sum.
  __device__ __forceinline__ void softmax(const f32x16 (&s)[KB], uint32_t (&pk)[KB][8], uint32_t (&pl)[KB][8],
                                          uint32_t (&po)[KB][8]) {
    const float c1 = p.scale * kLog2e;
    float lt = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pa = fast_exp2(fmaf(s[kb][2 * i], c1, -mb));
        const float pb = fast_exp2(fmaf(s[kb][2 * i + 1], c1, -mb));
        const uint32_t u = pack_bf16(pa, pb);
        pk[kb][i] = u;
        lt = add_bf16_pair(u, lt);
        uint32_t ul = 0;
        if (HP) {
          ul = pack_bf16(pa - bf16lo_to_f32(u), pb - bf16hi_to_f32(u));
          pl[kb][i] = ul;
          lt = add_bf16_pair(ul, lt);
        }
        if (DIAG) {
          // the entries whose P-bar rounds to 1, as a BF16 pair of 1.0 / 0 values
          const uint32_t ia = is_one(s[kb][2 * i]), ib = is_one(s[kb][2 * i + 1]);
          n_one += (int)(ia + ib);
          po[kb][i] = (ia ? 0x3f80u : 0u) | (ib ? 0x3f800000u : 0u);
        }
      }
    lsum = fmaf(lsum, alpha, lt);
  }

  // O^T += V^T P-bar^T from V buffer B.
  template <int B>
  __device__ __forceinline__ void pv(const uint32_t (&pk)[KB][8], const uint32_t (&pl)[KB][8],
                                     const uint32_t (&po)[KB][8]) {
    const char* vl = B ? vb1 : vb0;
    int v0s = vbase0, v1s = vbase1;
    asm volatile("" : "+v"(v0s), "+v"(v1s));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int kb = kc >> 1, o4 = 4 * (kc & 1);
      const u32x4 bop = u32x4{pk[kb][o4], pk[kb][o4 + 1], pk[kb][o4 + 2], pk[kb][o4 + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a0 = lds_read_tr(vl, (v0s ^ (64 * db)) + kc * 16 * ROWB);
        const u32x2 a1v = lds_read_tr(vl, (v1s ^ (64 * db)) + kc * 16 * ROWB);
        const u32x4 aop = u32x4{a0.x, a0.y, a1v.x, a1v.y};
        oacc[db] = mfma_bf16(aop, bop, oacc[db]);
        if (HP) {
          const u32x4 bl = u32x4{pl[kb][o4], pl[kb][o4 + 1], pl[kb][o4 + 2], pl[kb][o4 + 3]};
          oacc[db] = mfma_bf16(aop, bl, oacc[db]);
        }
        if (DIAG) {
          const u32x4 bo = u32x4{po[kb][o4], po[kb][o4 + 1], po[kb][o4 + 2], po[kb][o4 + 3]};
          oone[db] = mfma_bf16(aop, bo, oone[db]);
        }
      }
    }
  }

  // Loop step j (P = j mod 2): tile j is finished (P-bar, O-bar update) while
  // the scores of tile j + 1 are computed and reduced, so the MFMA and VALU
  // work of consecutive tiles can interleave.  K runs one tile ahead of V:
  // K(j+1) sits in K buffer 1-P, V(j) in V buffer P; the loads of V(j+1) and
  // K(j+2) go into the buffers that step j-1 finished with.
  template <int P, bool MASKN>
  __device__ __forceinline__ void step(int j, int n_tiles) {
    issue_v<1 - P>(j + 1);
    if (j + 2 < n_tiles) issue_k<P>(j + 2);
    rescale();
    f32x16 sn[KB];
    qk<1 - P>(sn);
    uint32_t pk[KB][8], pl[KB][8], po[KB][8];
    softmax(scur, pk, pl, po);
    pv<P>(pk, pl, po);
    if (MASKN) mask(sn, (j + 1) * BN);
    update_max(sn);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) scur[kb] = sn[kb];
    wait_all_and_barrier();
  }

  // The last tile (P = its index mod 2): nothing left to overlap.
  template <int P>
  __device__ __forceinline__ void last() {
    rescale();
    uint32_t pk[KB][8], pl[KB][8], po[KB][8];
    softmax(scur, pk, pl, po);
    pv<P>(pk, pl, po);
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    hi = lane >> 5;
    N = p.N;
    int qb;
    map_block(blockIdx.x, p.BH, p.n_qblocks, bh, qb);
    if (p.filter) {
      const int h = bh % p.H;
      if (!((p.hmask[h >> 6] >> (h & 63)) & 1)) return;   // the whole workgroup: bh is uniform
    }
    base = (size_t)bh * N * D;
    const uint16_t* Q = p.q + base;
    krs = make_rsrc(p.k + base, N * D * 2);
    vrs = make_rsrc(p.v + base, N * D * 2);
    q0 = qb * BM;
    qw0 = q0 + 32 * w;
    myq = qw0 + (lane & 31);

#pragma unroll
    for (int c = 0; c < DC; ++c)
      qreg[c] = (myq < N) ? ldg_b128(Q + (size_t)myq * D + (2 * c + hi) * 8) : u32x4{0, 0, 0, 0};
    // direct-load slots: wave w, load i covers LDS slots (w*LOADS + i)*64 + lane
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
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    if (DIAG)
#pragma unroll
      for (int db = 0; db < DB; ++db) oone[db] = f32x16{};
    Mraw = kNegInf;
    M2raw = kNegInf;
    m = kNegInf;
    mb = 0.f;
    lsum = 0.f;
    flag = false;
    n_one = 0;

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int n_tiles = (kv_end + BN - 1) / BN;
    // Tiles 0 .. n_plain-1 need no mask for any wave of the workgroup (all
    // keys before the first query, none past N).
    const int n_plain = CAUSAL ? min(q0, N) / BN : N / BN;

    // prologue: scores and maximum of tile 0
    issue_k<0>(0);
    issue_v<0>(0);
    if (n_tiles > 1) issue_k<1>(1);
    wait_all_and_barrier();
    qk<0>(scur);
    mask(scur, 0);
    update_max(scur);
    // Step 0 loads K(2) into the buffer that holds K(0): every wave must have
    // read K(0) first.  (Later steps are covered by the barrier that ends the
    // step before.)
    if (n_tiles > 2) __syncthreads();

    // steps 0 .. n_tiles-2, in pairs so that buffer indices are compile-time
    // constants; a step masks the scores of its next tile unless that tile is
    // one of the plain ones.
    const int n_steps = n_tiles - 1;
    const int n_plain_steps = min(n_plain - 1, n_steps);
    int j = 0;
    for (; j + 2 <= n_plain_steps; j += 2) {
      step<0, false>(j, n_tiles);
      step<1, false>(j + 1, n_tiles);
    }
    for (; j + 2 <= n_steps; j += 2) {
      step<0, true>(j, n_tiles);
      step<1, true>(j + 1, n_tiles);
    }
    if (j < n_steps) {
      step<0, true>(j, n_tiles);
      ++j;
    }
    if (j & 1) last<1>();
    else last<0>();
    epilogue();
  }

  // O = bf16(bf16(O-bar) / l)   or   O = O-bar / l (FP32 output)
  __device__ __forceinline__ void epilogue() {
    float la, lb;
    pair32(lsum, la, lb);
    const float ltot = la + lb;
    int ones = 0;
    if (DIAG) {
      float na, nb;
      pair32(__int_as_float(n_one), na, nb);
      ones = __float_as_int(na) + __float_as_int(nb);
    }
    if (myq >= N) return;
    const size_t orow = base + (size_t)myq * D;
    if (DIAG && p.o_one) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * db + 8 * rr + 4 * hi;
          const f32x4 out = {oone[db][4 * rr] / ltot, oone[db][4 * rr + 1] / ltot,
                             oone[db][4 * rr + 2] / ltot, oone[db][4 * rr + 3] / ltot};
          *reinterpret_cast<f32x4*>(p.o_one + orow + d0) = out;
        }
    }
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
          if (p.o_f32) {
            f32x4 wide = {bf16lo_to_f32(out.x), bf16hi_to_f32(out.x), bf16lo_to_f32(out.y),
                          bf16hi_to_f32(out.y)};
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + orow + d0) = wide;
          } else {
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + orow + d0) = out;
          }
        }
      }
    }
    if (hi == 0) {
      p.lse[(size_t)bh * N + myq] = m + logf(ltot);
      if (FLAGS && p.flags) p.flags[(size_t)bh * N + myq] = flag ? 1 : 0;
      if (DIAG) p.pbar_one[(size_t)bh * N + myq] = ones;
    }
  }
};

template <int D, int MODE, bool CAUSAL, bool FLAGS, bool DIAG, bool WIDE>
__global__ __launch_bounds__((FwdKernel<D, MODE, CAUSAL, FLAGS, DIAG, WIDE>::NT),
                             (FwdKernel<D, MODE, CAUSAL, FLAGS, DIAG, WIDE>::MIN_WG)) void fwd_kernel(FwdParams p) {
  using Kt = FwdKernel<D, MODE, CAUSAL, FLAGS, DIAG, WIDE>;
  __shared__ __attribute__((aligned(1024))) char k0[Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[Kt::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[Kt::TILE];
  Kt k(p, k0, k1, v0, v1);
  k.run();
}

template <int D, int MODE, bool CAUSAL, bool FLAGS, bool DIAG, bool WIDE>
hipError_t launch_g(FwdParams p, hipStream_t stream) {
  using Kt = FwdKernel<D, MODE, CAUSAL, FLAGS, DIAG, WIDE>;
  p.n_qblocks = (p.N + Kt::BM - 1) / Kt::BM;
  const unsigned grid = (unsigned)(p.BH * p.n_qblocks);
  hipLaunchKernelGGL((fwd_kernel<D, MODE, CAUSAL, FLAGS, DIAG, WIDE>), dim3(grid), dim3(Kt::NT), 0, stream, p);
  return hipGetLastError();
}

template <int D, int MODE, bool CAUSAL, bool FLAGS, bool DIAG = false>
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
  p.scale = a.scale;
  p.beta = a.beta;
  p.eps = a.eps;
  p.pinf = __builtin_inff();
  p.ninf = -__builtin_inff();
  p.H = a.H;
  p.filter = a.filter;
  p.o_f32 = a.o_f32;
  for (int i = 0; i < 4; ++i) p.hmask[i] = a.hmask[i];
  p.pbar_one = a.pbar_one;
  p.o_one = a.o_one;
  p.one_thr = a.one_thr;
  // the 256-query geometry for fewer than 32 slices at d = 128 (see FwdKernel);
  // the diagnostic variant always runs 128-query workgroups
  if constexpr (D == 128 && !DIAG)
    if (p.BH < 32) return launch_g<D, MODE, CAUSAL, FLAGS, DIAG, true>(p, stream);
  return launch_g<D, MODE, CAUSAL, FLAGS, DIAG, false>(p, stream);
}

template <int D, int MODE>
hipError_t launch_m(const FwdArgs& a, hipStream_t stream) {
  // the tie-aware shift needs the running second maximum; the plain modes
  // track it only when the caller asks for the tie flags
  const bool flags = MODE == kTieAware || a.flags != nullptr;
  if (a.pbar_one) {
    if (a.causal) return launch_t<D, MODE, true, true, true>(a, stream);
    return launch_t<D, MODE, false, true, true>(a, stream);
  }
  if (a.causal) {
    if (flags) return launch_t<D, MODE, true, true>(a, stream);
    return launch_t<D, MODE, true, (MODE == kTieAware)>(a, stream);
  }
  if (flags) return launch_t<D, MODE, false, true>(a, stream);
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

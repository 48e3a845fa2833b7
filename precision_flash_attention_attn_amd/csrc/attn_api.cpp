// C ABI of the precision flash attention library: argument checks, then the
// kernel launches on the caller's stream.  Every check runs before any HIP
// call, so invalid arguments return an error without touching the device.
#include <cmath>
#include <cstdint>

#include "pfa_attn.h"
#include "pfa_internal.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_sizes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return PFA_ERR_INVALID;
  const int64_t bh = int64_t(B) * H;
  if (bh * N * d >= kMaxElems) return PFA_ERR_INVALID;
  // launch sizes: the largest grid has (B*H) * ceil(N/64) workgroups of up to
  // 512 threads, and a launch may hold fewer than 2^32 threads
  if (bh * ((int64_t(N) + 63) / 64) >= (int64_t(1) << 23)) return PFA_ERR_INVALID;
  if (d != 64 && d != 128) return PFA_ERR_UNSUPPORTED;
  // tiles are staged with 32-bit byte offsets inside one (batch, head) slice
  if (int64_t(N) * d >= (int64_t(1) << 29)) return PFA_ERR_UNSUPPORTED;
  return PFA_OK;
}

// The smallest FP32 value t for which P-bar = bf16(fp32(exp(t))) is 1 (BF16
// round to nearest even): the FP32 value must be at least 1 - 2^-9, the
// halfway point below 1 that goes to the even 1.0.  exp is taken correctly
// rounded to FP32 (double exp, then rounded): the candidates near t are 2^-32
// apart, and none of their exponentials lies near an FP32 halfway point.
float pbar_one_threshold() {
  const float target = 1.0f - 1.0f / 512.0f;
  const auto rn = [](float t) { return static_cast<float>(std::exp(static_cast<double>(t))); };
  float t = static_cast<float>(std::log(static_cast<double>(target)));
  while (rn(t) < target) t = std::nextafter(t, 0.0f);
  while (rn(std::nextafter(t, -1.0f)) >= target) t = std::nextafter(t, -1.0f);
  return t;
}

int check_common(int B, int H, int N, int d, float scale, int mode) {
  const int s = check_sizes(B, H, N, d);
  if (s != PFA_OK) return s;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PFA_ERR_INVALID;
  if (mode != PFA_BF16_OUT && mode != PFA_FP32_OUT && mode != PFA_TIE_AWARE_SOFTMAX)
    return PFA_ERR_INVALID;
  return PFA_OK;
}

}  // namespace

extern "C" {

namespace {

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* tie_flags,
             int32_t* pbar_one, float* o_one, int B, int H, int N, int d, int causal, float scale,
             int mode, const pfa_tie_opts* opts, void* stream) {
  int st = check_common(B, H, N, d, scale, mode);
  if (st != PFA_OK) return st;
  if (!q || !k || !v || !o || !lse) return PFA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return PFA_ERR_INVALID;
  if (tie_flags && !aligned4(tie_flags)) return PFA_ERR_INVALID;
  float beta = 2.0f, eps = 1e-3f;
  if (opts) {
    beta = opts->beta;
    eps = opts->eps;
  }
  if (!std::isfinite(beta) || !(beta > 1.0f)) return PFA_ERR_INVALID;
  if (!std::isfinite(eps) || !(eps >= 0.0f)) return PFA_ERR_INVALID;

  pfa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.flags = tie_flags;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.causal = causal ? 1 : 0;
  a.mode = mode;
  a.scale = scale;
  a.beta = beta;
  a.eps = eps;
  a.pbar_one = pbar_one;
  a.o_one = o_one;
  if (pbar_one) {
    static const float thr = pbar_one_threshold();
    a.one_thr = thr;
  }
  const hipError_t e = pfa::launch_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

}  // namespace

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* tie_flags,
             int B, int H, int N, int d, int causal, float scale, int mode,
             const pfa_tie_opts* opts, void* stream) {
  return fwd_impl(q, k, v, o, lse, tie_flags, nullptr, nullptr, B, H, N, d, causal, scale, mode, opts,
                  stream);
}

int attn_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse,
                  int32_t* tie_flags, int32_t* pbar_one, float* o_one, int B, int H, int N, int d,
                  int causal, float scale, int mode, const pfa_tie_opts* opts, void* stream) {
  if (!pbar_one || !aligned4(pbar_one)) return PFA_ERR_INVALID;
  if (o_one && !aligned16(o_one)) return PFA_ERR_INVALID;
  return fwd_impl(q, k, v, o, lse, tie_flags, pbar_one, o_one, B, H, N, d, causal, scale, mode, opts,
                  stream);
}

int attn_fwd_heads(const void* q, const void* k, const void* v, float* o, float* lse,
                   int32_t* tie_flags, int B, int H, int N, int d, int causal, float scale,
                   const int32_t* head_modes, const pfa_tie_opts* opts, void* stream) {
  int st = check_common(B, H, N, d, scale, PFA_BF16_OUT);
  if (st != PFA_OK) return st;
  if (H > 256) return PFA_ERR_UNSUPPORTED;
  if (!head_modes) return PFA_ERR_INVALID;
  uint64_t masks[3][4] = {};
  for (int h = 0; h < H; ++h) {
    const int m = head_modes[h];
    if (m != PFA_BF16_OUT && m != PFA_FP32_OUT && m != PFA_TIE_AWARE_SOFTMAX) return PFA_ERR_INVALID;
    masks[m][h >> 6] |= uint64_t(1) << (h & 63);
  }
  if (!q || !k || !v || !o || !lse) return PFA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return PFA_ERR_INVALID;
  if (tie_flags && !aligned4(tie_flags)) return PFA_ERR_INVALID;
  float beta = 2.0f, eps = 1e-3f;
  if (opts) {
    beta = opts->beta;
    eps = opts->eps;
  }
  if (!std::isfinite(beta) || !(beta > 1.0f)) return PFA_ERR_INVALID;
  if (!std::isfinite(eps) || !(eps >= 0.0f)) return PFA_ERR_INVALID;
  for (int m = 0; m < 3; ++m) {
    if (!(masks[m][0] | masks[m][1] | masks[m][2] | masks[m][3])) continue;
    pfa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.flags = tie_flags;
    a.B = B;
    a.H = H;
    a.N = N;
    a.d = d;
    a.causal = causal ? 1 : 0;
    a.mode = m;
    a.scale = scale;
    a.beta = beta;
    a.eps = eps;
    a.filter = 1;
    a.o_f32 = 1;
    for (int i = 0; i < 4; ++i) a.hmask[i] = masks[m][i];
    const hipError_t e = pfa::launch_fwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PFA_ERR_HIP;
  }
  return PFA_OK;
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, int mode) {
  if (check_sizes(B, H, N, d) != PFA_OK) return 0;
  if (mode != PFA_BF16_OUT && mode != PFA_FP32_OUT && mode != PFA_TIE_AWARE_SOFTMAX) return 0;
  const size_t rows = size_t(B) * H * N;
  return pfa::bwd_delta_bytes(rows) + pfa::bwd_dout16_bytes(rows, d, mode);
}

namespace {

// Shared checks of the backward entry points; fills the workspace pointers.
int bwd_args(pfa::BwdArgs& a, void* workspace, size_t workspace_bytes, float* delta, int B, int H,
             int N, int d, int causal, float scale, int mode) {
  const int st = check_common(B, H, N, d, scale, mode);
  if (st != PFA_OK) return st;
  if (!workspace || !aligned16(workspace)) return PFA_ERR_INVALID;
  if (delta && !aligned4(delta)) return PFA_ERR_INVALID;
  const size_t need = attn_bwd_workspace_bytes(B, H, N, d, mode);
  if (need == 0 || workspace_bytes < need) return PFA_ERR_INVALID;
  a = pfa::BwdArgs{};
  const size_t rows = size_t(B) * H * N;
  a.delta = delta ? delta : static_cast<float*>(workspace);
  a.dout16 = mode == PFA_FP32_OUT
                 ? reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + pfa::bwd_delta_bytes(rows))
                 : nullptr;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.causal = causal ? 1 : 0;
  a.mode = mode;
  a.scale = scale;
  return PFA_OK;
}

bool ok16(const void* p) { return p && aligned16(p); }

int status_of(hipError_t e) { return e == hipSuccess ? PFA_OK : PFA_ERR_HIP; }

// The backward with delta = rowsum(dO o O): the dQ kernel first, which also
// forms delta (and the BF16 dO of the FP32-output mode) for the dK/dV kernel,
// so no pre-pass over O and dO is needed.
int bwd_standard(const pfa::BwdArgs& a, hipStream_t s) {
  hipError_t e = pfa::launch_bwd_dq_delta(a, s);
  if (e == hipSuccess) e = pfa::launch_bwd_dkdv(a, s);
  return status_of(e);
}

}  // namespace

int attn_bwd_prep(const void* o, const void* dout, float* delta, void* workspace,
                  size_t workspace_bytes, int B, int H, int N, int d, int mode, void* stream) {
  pfa::BwdArgs a;
  const int st = bwd_args(a, workspace, workspace_bytes, delta, B, H, N, d, 1, 1.0f, mode);
  if (st != PFA_OK) return st;
  if (!ok16(o) || !ok16(dout)) return PFA_ERR_INVALID;
  a.o = o;
  a.dout = dout;
  return status_of(pfa::launch_bwd_prep(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                  const float* delta, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  int B, int H, int N, int d, int causal, float scale, int mode, void* stream) {
  pfa::BwdArgs a;
  const int st = bwd_args(a, workspace, workspace_bytes, const_cast<float*>(delta), B, H, N, d,
                          causal, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(dout) || !ok16(dk) || !ok16(dv)) return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dk = dk;
  a.dv = dv;
  return status_of(pfa::launch_bwd_dkdv(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const float* delta, void* dq, void* workspace, size_t workspace_bytes, int B, int H,
                int N, int d, int causal, float scale, int mode, void* stream) {
  pfa::BwdArgs a;
  const int st = bwd_args(a, workspace, workspace_bytes, const_cast<float*>(delta), B, H, N, d,
                          causal, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(dout) || !ok16(dq)) return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  return status_of(pfa::launch_bwd_dq(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, float* delta, void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d, int causal, float scale, int mode, void* stream) {
  pfa::BwdArgs a;
  const int st = bwd_args(a, workspace, workspace_bytes, delta, B, H, N, d, causal, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(o) || !ok16(dout) || !ok16(dq)) return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  return status_of(pfa::launch_bwd_dq_delta(a, static_cast<hipStream_t>(stream)));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, void* workspace,
             size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale, int mode,
             void* stream) {
  pfa::BwdArgs a;
  int st = bwd_args(a, workspace, workspace_bytes, delta, B, H, N, d, causal, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(o) || !ok16(dout) || !ok16(dq) || !ok16(dk) ||
      !ok16(dv))
    return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  return bwd_standard(a, static_cast<hipStream_t>(stream));
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                     int d, int causal, float scale, int mode, void* stream) {
  // every argument check before the first HIP call
  const int st = check_common(B, H, N, d, scale, mode);
  if (st != PFA_OK) return st;
  if (attn_bwd_workspace_bytes(B, H, N, d, mode) > pfa::kNoallocScratchBytes) return PFA_ERR_SCRATCH;
  if (delta && !aligned4(delta)) return PFA_ERR_INVALID;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(o) || !ok16(dout) || !ok16(dq) || !ok16(dk) ||
      !ok16(dv))
    return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  void* ws = nullptr;
  const int sst = pfa::noalloc_scratch(stream, &ws);
  if (sst != PFA_OK) return sst;
  pfa::BwdArgs a;
  // the same workspace layout as attn_bwd, in the scratch
  const int st2 = bwd_args(a, ws, pfa::kNoallocScratchBytes, delta, B, H, N, d, causal, scale, mode);
  if (st2 != PFA_OK) return st2;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  return bwd_standard(a, static_cast<hipStream_t>(stream));
}

size_t attn_bwd_noalloc_max_bytes(void) { return pfa::kNoallocScratchBytes; }

int attn_bwd_delta(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* delta, void* workspace, size_t workspace_bytes, int B,
                   int H, int N, int d, int causal, float scale, int mode, int delta_src,
                   void* stream) {
  if (delta_src != PFA_DELTA_DO_O && delta_src != PFA_DELTA_DP_P && delta_src != PFA_DELTA_DO_OHP)
    return PFA_ERR_INVALID;
  pfa::BwdArgs a;
  const int st = bwd_args(a, workspace, workspace_bytes, delta, B, H, N, d, causal, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(o) || !ok16(dout)) return PFA_ERR_INVALID;
  if (delta_src != PFA_DELTA_DO_O) {
    if (!ok16(q) || !ok16(k) || !ok16(v)) return PFA_ERR_INVALID;
    if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the pre-pass also leaves the BF16 copy of dO that the FP32-output mode's
  // gradient kernels read; its delta is then replaced
  hipError_t e = hipSuccess;
  if (delta_src == PFA_DELTA_DO_O || mode == PFA_FP32_OUT) e = pfa::launch_bwd_prep(a, s);
  if (e == hipSuccess && delta_src != PFA_DELTA_DO_O) e = pfa::launch_bwd_delta(a, delta_src, a.delta, s);
  return status_of(e);
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, float* delta, void* workspace,
                size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
                int mode, int delta_src, void* stream) {
  if (delta_src != PFA_DELTA_DO_O && delta_src != PFA_DELTA_DP_P && delta_src != PFA_DELTA_DO_OHP)
    return PFA_ERR_INVALID;
  pfa::BwdArgs a;
  int st = bwd_args(a, workspace, workspace_bytes, delta, B, H, N, d, causal, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(o) || !ok16(dout) || !ok16(dq) || !ok16(dk) ||
      !ok16(dv))
    return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse)) return PFA_ERR_INVALID;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (delta_src == PFA_DELTA_DO_O) return bwd_standard(a, s);
  if (mode == PFA_FP32_OUT) e = pfa::launch_bwd_prep(a, s);
  if (e == hipSuccess) e = pfa::launch_bwd_delta(a, delta_src, a.delta, s);
  if (e == hipSuccess) e = pfa::launch_bwd_dkdv(a, s);
  if (e == hipSuccess) e = pfa::launch_bwd_dq(a, s);
  return status_of(e);
}

int attn_delta_error(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* err, int B, int H, int N, int d, int causal,
                     float scale, int mode, void* stream) {
  const int st = check_common(B, H, N, d, scale, mode);
  if (st != PFA_OK) return st;
  if (!ok16(q) || !ok16(k) || !ok16(v) || !ok16(o) || !ok16(dout)) return PFA_ERR_INVALID;
  if (!lse || !aligned4(lse) || !err || !aligned4(err)) return PFA_ERR_INVALID;
  pfa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.causal = causal ? 1 : 0;
  a.mode = mode;
  a.scale = scale;
  return status_of(pfa::launch_bwd_delta(a, pfa::kDeltaErr, err, static_cast<hipStream_t>(stream)));
}

const char* attn_strerror(int status) {
  switch (status) {
    case PFA_OK: return "ok";
    case PFA_ERR_INVALID: return "invalid argument";
    case PFA_ERR_UNSUPPORTED: return "unsupported configuration (head dimension must be 64 or 128)";
    case PFA_ERR_HIP: return "HIP launch failure";
    case PFA_ERR_SCRATCH:
      return "workspace larger than the static scratch of attn_bwd_noalloc (see attn_bwd_noalloc_max_bytes)";
    default: return "unknown status";
  }
}

const char* attn_version(void) { return "pfa_attn 0.1.0 gfx950"; }

}  // extern "C"

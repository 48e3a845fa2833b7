// Host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pfa {

enum Mode { kBf16Out = 0, kFp32Out = 1, kTieAware = 2 };

// Sources of delta (the C ABI's pfa_delta_src), plus the error export.
enum DeltaSrc { kDeltaDoO = 0, kDeltaDpP = 1, kDeltaOhp = 2, kDeltaErr = 3 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t* flags;
  int B, H, N, d;
  int causal;
  int mode;
  float scale, beta, eps;
  // per-head selection (attn_fwd_heads): run only heads whose bit is set;
  // o_f32: O is FP32 whatever the mode
  int filter = 0, o_f32 = 0;
  uint64_t hmask[4] = {0, 0, 0, 0};
  int32_t* pbar_one = nullptr;   // attn_fwd_diag: per-row count of P-bar == 1
  float* o_one = nullptr;        // attn_fwd_diag: the part of O from those entries (optional)
  float one_thr = 0.f;           // smallest FP32 d with exp(d) >= 1 - 2^-9
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;     // where delta is written (caller's buffer or workspace)
  uint16_t* dout16; // BF16 copy of an FP32 dO in the workspace (FP32-output mode)
  int B, H, N, d;
  int causal;
  int mode;
  float scale;
};

// Workspace of the backward: the FP32 delta row vector, then (FP32-output
// mode only) a BF16 copy of dO; 256-byte aligned parts.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t bwd_delta_bytes(size_t rows) { return align256(rows * 4); }
inline size_t bwd_dout16_bytes(size_t rows, int d, int mode) {
  return mode == kFp32Out ? align256(rows * (size_t)d * 2) : 0;
}

// Size of the static device scratch of attn_bwd_noalloc (per device).
constexpr size_t kNoallocScratchBytes = size_t(72) << 20;

// Device address of the static scratch on the stream's device (the current
// device for a NULL stream), looked up once per device.  Returns a PFA_*
// status.
int noalloc_scratch(void* stream, void** ptr);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// The backward's kernels on one stream: delta = rowsum(dO o O); dK and dV;
// dQ.
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
// dQ that also forms delta = rowsum(dO o O) (bit for bit the pre-pass's) and,
// in the FP32-output mode, the BF16 copy of dO: it replaces the pre-pass when
// it runs before the dK/dV kernel.
hipError_t launch_bwd_dq_delta(const BwdArgs& a, hipStream_t stream);
// delta from another source (kDeltaDpP, kDeltaOhp) or delta_lp - delta_hp
// (kDeltaErr), written to `out` [B,H,N].
hipError_t launch_bwd_delta(const BwdArgs& a, int src, float* out, hipStream_t stream);

}  // namespace pfa

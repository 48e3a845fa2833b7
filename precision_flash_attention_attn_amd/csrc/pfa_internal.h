// Host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pfa {

enum Mode { kBf16Out = 0, kFp32Out = 1, kTieAware = 2 };

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
  float* dq_acc;    // FP32 dQ accumulator in the workspace
  int B, H, N, d;
  int causal;
  int mode;
  float scale;
};

// Workspace layout of the backward: [dQ accumulator | delta], 256-byte aligned parts.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline size_t bwd_dq_acc_bytes(size_t rows, int d) { return align256(rows * (size_t)d * 4); }
inline size_t bwd_delta_bytes(size_t rows) { return align256(rows * 4); }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// The backward in three stages on one stream: delta and the cleared dQ
// accumulator; dK, dV and the dQ accumulation; dQ conversion to BF16.
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream);

}  // namespace pfa

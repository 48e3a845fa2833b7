/*
 * pfa_attn.h -- C ABI of the precision flash attention library (MI355X, gfx950).
 *
 * Tiled flash attention with the online safe softmax, forward and backward,
 * BF16 inputs with FP32 accumulation, in three modes:
 *
 *   PFA_BF16_OUT            plain BF16 flash attention.  The unnormalised
 *                           product O-bar = P-bar V is accumulated in FP32 over
 *                           all key tiles, rounded to BF16 once, and the output
 *                           O = O-bar / rowsum(P-bar) is rounded to BF16.
 *                           P-bar = exp(S - rowmax S) is rounded to BF16 before
 *                           the product, so P-bar is exactly 1 at every row
 *                           maximum ("Why Low-Precision Transformer Training
 *                           Fails", arXiv 2510.04212, as summarised on
 *                           paper-graph-ui, section 3.4.4).
 *   PFA_FP32_OUT            remedy 1: O is kept in FP32 and P-bar enters the
 *                           product at high precision (a two-term BF16
 *                           expansion hi + lo).  Section 3.4.2 reports that an
 *                           FP32 O stabilises training and section 3.4.4 that
 *                           an FP32 P-bar V product alone suffices.  dO is
 *                           FP32 in this mode.
 *   PFA_TIE_AWARE_SOFTMAX   remedy 2: the repeated-maximum-aware safe softmax of
 *                           section 3.4.5.  With rm the row maximum and
 *                           rs = #{t : rm - S_t <= eps}, the shift is beta*rm
 *                           when rm > 0 and rs > 1, 0 when rm < 0 and rs > 1,
 *                           and rm otherwise, so no P-bar equals 1 on rows with
 *                           repeated maxima.  Output as in PFA_BF16_OUT.
 *
 * Scores are S = scale * Q K^T; with causal != 0, key t is masked for query
 * T when t > T.  The tie test uses this S (FP32, base e) and eps in FP32.
 *
 * Layout: every tensor is contiguous [B, H, N, d] (d fastest), row vectors
 * [B, H, N] for LSE, delta and tie flags.  Q, K, V, dQ, dK, dV are BF16; O and
 * dO are BF16 except in PFA_FP32_OUT, where they are FP32.  All pointers are
 * DEVICE pointers owned by the caller, 16-byte aligned.  The library allocates
 * no memory, keeps no state between calls (attn_bwd_noalloc's static scratch
 * aside, see there) and launches only on the given stream (a hipStream_t;
 * NULL is the default stream).  Calls are asynchronous: a device fault
 * surfaces at the caller's next synchronisation.
 *
 * Supported: d in {64, 128}; any N >= 1 (ragged tails are masked) with
 * N*d < 2^29 (byte offsets inside one (batch, head) slice stay 32-bit);
 * B, H >= 1; B*H*N*d < 2^40; B*H*ceil(N/64) < 2^23 (the largest launch then
 * stays under 2^32 threads).
 *
 * Errors: arguments are checked before anything is launched; a failed check
 * returns a negative status and writes nothing.  PFA_ERR_INVALID for a NULL
 * required pointer, misaligned pointer, non-positive or oversized B/H/N,
 * non-finite or non-positive scale, unknown mode, beta <= 1 or non-finite,
 * eps < 0 or non-finite, a too small workspace.  PFA_ERR_UNSUPPORTED for
 * d not in {64, 128} or N*d >= 2^29.  PFA_ERR_HIP if a launch fails.
 *
 * Numerical note (tie-aware mode): when (beta - 1) * rm exceeds the FP32
 * exponent range (about 87) on a tied row, every P-bar underflows, the row sum
 * is 0 and that row of O is NaN.  The pages name this underflow as the reason
 * the shift is applied only to tied rows; it is reported, not an error code.
 */
#ifndef PFA_ATTN_H
#define PFA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pfa_mode { PFA_BF16_OUT = 0, PFA_FP32_OUT = 1, PFA_TIE_AWARE_SOFTMAX = 2 };

enum pfa_status {
  PFA_OK = 0,
  PFA_ERR_INVALID = -1,
  PFA_ERR_UNSUPPORTED = -2,
  PFA_ERR_HIP = -3,
  PFA_ERR_SCRATCH = -4
};

/* Parameters of the repeated-maximum-aware softmax (section 3.4.5): beta > 1
 * (the pages use 2, and recommend 2 to 8), eps >= 0 (the pages' example is
 * 1e-3).  NULL selects {2.0f, 1e-3f}. */
typedef struct pfa_tie_opts {
  float beta;
  float eps;
} pfa_tie_opts;

/*
 * Forward pass.  Defines: P-bar = exp(S - m), O-bar = P-bar V,
 * O = O-bar / rowsum(P-bar)  (section 3.4.4), m chosen per mode as above.
 *
 *   q, k, v    in   BF16 [B,H,N,d]
 *   o          out  BF16 [B,H,N,d] (PFA_FP32_OUT: FP32)
 *   lse        out  FP32 [B,H,N], m + log(rowsum P-bar): the log of the
 *                   softmax normaliser, used by the backward
 *   tie_flags  out  INT32 [B,H,N] or NULL: 1 where at least two unmasked
 *                   scores lie within eps of the row maximum (rs > 1), else 0.
 *                   The same function of S in every mode.
 *   opts       in   tie parameters (NULL = defaults); eps also sets the flag
 *                   threshold in the plain modes.
 *   stream     in   hipStream_t
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int32_t* tie_flags, int B, int H, int N, int d, int causal, float scale,
             int mode, const pfa_tie_opts* opts, void* stream);

/*
 * attn_fwd plus two diagnostics of the P-bar = 1 additions at which the pages'
 * cumulative error of O-bar jumps (section 3.4.4, "How the error accumulates
 * across token positions" and "Why P-bar = 1 is the critical condition"):
 *
 *   pbar_one  out  INT32 [B,H,N], device, required: per row, the number of
 *                  entries whose P-bar rounds to 1 in BF16.  Decided on the
 *                  method's definition: S = fp32(fp32(q.k) * scale),
 *                  d = fp32(S - m) with m the shift in force for the entry's
 *                  key tile, and P-bar = bf16(fp32(exp(d))) is 1 exactly
 *                  when exp(d), correctly rounded to FP32, is at least
 *                  1 - 2^-9.  The same entries in every mode (in
 *                  PFA_FP32_OUT they enter the product as hi + lo, within
 *                  2^-9 of 1).
 *   o_one     out  FP32 [B,H,N,d], device, 16-byte aligned, or NULL: the part
 *                  of O those entries carry, (sum of their V rows, rescaled
 *                  with O-bar from tile to tile) / rowsum(P-bar), kept apart
 *                  from the rest of O.
 *
 * Same outputs as attn_fwd otherwise; runs a separate kernel variant, so
 * attn_fwd pays nothing for it.  Errors as attn_fwd, plus PFA_ERR_INVALID for
 * a NULL or misaligned pbar_one or a misaligned o_one.
 */
int attn_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse,
                  int32_t* tie_flags, int32_t* pbar_one, float* o_one, int B, int H, int N, int d,
                  int causal, float scale, int mode, const pfa_tie_opts* opts, void* stream);

/*
 * Forward with a mode per head: the pages' localisation experiment computes O
 * in FP32 on selected heads only (section 3.2, "Failure is localized to
 * specific attention heads"); the tie-aware softmax can be selected the same
 * way.  head_modes: HOST array of H pfa_mode values.  o: FP32 [B,H,N,d] for
 * every head -- heads in PFA_BF16_OUT or PFA_TIE_AWARE_SOFTMAX hold their BF16
 * result widened exactly, so each head's O equals attn_fwd's in its own mode.
 * lse, tie_flags, opts as attn_fwd.  The backward takes this O with mode
 * PFA_FP32_OUT (dO FP32).  One kernel launch per mode present.  Errors as
 * attn_fwd, plus PFA_ERR_INVALID for a NULL head_modes or an unknown mode in
 * it, PFA_ERR_UNSUPPORTED for H > 256.
 */
int attn_fwd_heads(const void* q, const void* k, const void* v, float* o, float* lse,
                   int32_t* tie_flags, int B, int H, int N, int d, int causal, float scale,
                   const int32_t* head_modes, const pfa_tie_opts* opts, void* stream);

/* Bytes of device workspace the backward needs: room for the FP32 delta row
 * vector [B,H,N] (used when the caller passes no delta buffer) and, in
 * PFA_FP32_OUT, a BF16 copy of dO for the MFMA operands; 256-byte aligned
 * parts.  0 on invalid sizes. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, int mode);

/*
 * Backward pass (section 3.4.2 and 3.4.3):
 *   delta = rowsum(dO o O); P = exp(S - LSE); dV = P^T dO; dP = dO V^T;
 *   dS = P o (dP - delta); dQ = scale * dS K; dK = scale * dS^T Q.
 * The tie-aware softmax changes only the forward: given its O and LSE the
 * backward is that of PFA_BF16_OUT.
 *
 *   q, k, v         in   BF16 [B,H,N,d]
 *   o, dout         in   BF16 [B,H,N,d] (PFA_FP32_OUT: FP32)
 *   lse             in   FP32 [B,H,N] from attn_fwd
 *   dq, dk, dv      out  BF16 [B,H,N,d]
 *   delta           out  FP32 [B,H,N] or NULL: delta as used, for diagnostics
 *   workspace       in   device memory of at least attn_bwd_workspace_bytes;
 *                        contents on entry are ignored
 * No atomics are used: dQ, dK and dV are bitwise reproducible.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
             int causal, float scale, int mode, void* stream);

/*
 * The backward in stages, for callers that schedule or time them separately.
 * Two orders give bit for bit the result of attn_bwd, each on one stream:
 *   attn_bwd_prep, attn_bwd_dkdv, attn_bwd_dq   (three kernels), or
 *   attn_bwd_dq_delta, attn_bwd_dkdv            (two kernels; what attn_bwd runs).
 *
 * Stage 1, attn_bwd_prep: delta = rowsum(dO o O) in FP32 -- the term the
 * pages single out as computed apart in the backward (section 3.4.2) -- into
 * `delta` (or into the workspace when delta is NULL).  o, dout: BF16 (FP32 in
 * PFA_FP32_OUT).
 */
int attn_bwd_prep(const void* o, const void* dout, float* delta, void* workspace,
                  size_t workspace_bytes, int B, int H, int N, int d, int mode, void* stream);

/* Stage 2, attn_bwd_dkdv: P = exp(S - LSE), dP = dO V^T, dS = P o (dP - delta);
 * writes dV = P^T dO and dK = scale dS^T Q (BF16) (sections 3.4.2, 3.4.3).
 * delta: the vector stage 1 wrote (NULL = the workspace copy).  In
 * PFA_FP32_OUT stages 2 and 3 take dO from the BF16 copy stage 1 left in the
 * workspace, so they need the same workspace, after stage 1. */
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                  const float* delta, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  int B, int H, int N, int d, int causal, float scale, int mode, void* stream);

/* Stage 3, attn_bwd_dq: recomputes P and dS per query block and writes
 * dQ = scale dS K (BF16) (section 3.4.3).  delta as in stage 2. */
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const float* delta, void* dq, void* workspace, size_t workspace_bytes, int B, int H,
                int N, int d, int causal, float scale, int mode, void* stream);

/* Stages 1 and 3 in one kernel, attn_bwd_dq_delta: dQ as attn_bwd_dq, with
 * delta = rowsum(dO o O) (section 3.4.2) formed per query row on the way --
 * summed in the order attn_bwd_prep uses, so the value is bit for bit the
 * same -- and written to `delta` (or the workspace when delta is NULL); in
 * PFA_FP32_OUT also the BF16 copy of dO in the workspace.  attn_bwd_dkdv with
 * the same delta and workspace, after it on the same stream, completes the
 * backward.  o, dout: BF16 (FP32 in PFA_FP32_OUT).  Errors as attn_bwd. */
int attn_bwd_dq_delta(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, float* delta, void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d, int causal, float scale, int mode, void* stream);

/*
 * Where the backward takes delta from: the isolation experiments of section
 * 3.2 (and the error analysis of section 3.4.2) swap the standard term for
 * equivalents that avoid the BF16 O of the forward.
 *   PFA_DELTA_DO_O    rowsum(dO o O) with the stored O (the standard backward)
 *   PFA_DELTA_DP_P    rowsum(dP o P), P = exp(S - LSE), dP = dO V^T with dO in
 *                     BF16 (as the gradient kernels use it); FP32 products and
 *                     sums.  Equal to the first in exact arithmetic.
 *   PFA_DELTA_DO_OHP  rowsum(dO o O_hp): O = P V recomputed in the backward with
 *                     FP32 accumulation, P split into BF16 hi + lo parts (both
 *                     products on MFMA); dO as given (FP32 in PFA_FP32_OUT).
 * The last two cost one more pass over the keys per query block.
 */
enum pfa_delta_src { PFA_DELTA_DO_O = 0, PFA_DELTA_DP_P = 1, PFA_DELTA_DO_OHP = 2 };

/* Stage 1 with a choice of delta source: writes delta (into `delta`, or the
 * workspace when NULL) and, in PFA_FP32_OUT, the BF16 copy of dO stages 2 and
 * 3 read.  PFA_DELTA_DO_O is exactly attn_bwd_prep (q, k, v, lse unused and
 * may be NULL); the other sources need q, k, v and lse.  Errors as
 * attn_bwd_prep, plus PFA_ERR_INVALID for an unknown delta_src. */
int attn_bwd_delta(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* delta, void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, int causal, float scale, int mode, int delta_src,
                   void* stream);

/* attn_bwd with delta taken from delta_src: attn_bwd_delta followed by
 * stages 2 and 3.  With PFA_DELTA_DO_O it is attn_bwd. */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, float* delta, void* workspace,
                size_t workspace_bytes, int B, int H, int N, int d, int causal, float scale,
                int mode, int delta_src, void* stream);

/* Diagnostic export of the error of delta (section 3.4.4): per row,
 * err = rowsum(dO o O) - rowsum(dO o O_hp), the stored-O delta minus the
 * PFA_DELTA_DO_OHP value, both with dO as given.  err: FP32 [B,H,N], device.
 * Needs no workspace.  Errors as attn_fwd's argument checks. */
int attn_delta_error(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* err, int B, int H, int N, int d, int causal,
                     float scale, int mode, void* stream);

/*
 * attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels, with the backward's workspace taken from a static device
 * array inside the library instead of a caller buffer.  Arguments as attn_bwd
 * without workspace/workspace_bytes.
 *
 * Limit: attn_bwd_workspace_bytes(B, H, N, d, mode) must not exceed
 * attn_bwd_noalloc_max_bytes() (72 MiB: about 18.8 million rows in the BF16
 * modes, 290 thousand rows at d = 128 in PFA_FP32_OUT); larger problems
 * return PFA_ERR_SCRATCH before anything is launched.  Other errors as
 * attn_bwd.  The call allocates nothing: each GPU holds its own copy of the
 * array (loaded with the library's code, kept until the process ends), whose
 * device address is looked up on the first call on that GPU.  Every call on a
 * GPU shares that GPU's array and leaves its contents behind (the backward
 * overwrites all it reads): calls that overlap on one GPU (concurrent streams
 * or host threads) race and give wrong results; serialise them.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
                     int d, int causal, float scale, int mode, void* stream);

/* Bytes of the static scratch attn_bwd_noalloc uses per GPU. */
size_t attn_bwd_noalloc_max_bytes(void);

/* Static text for a status code. */
const char* attn_strerror(int status);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PFA_ATTN_H */

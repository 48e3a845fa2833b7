// Shared device helpers for the gfx950 (CDNA4) attention kernels.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, one wave64):
//   A (32 x 16, rows i, contraction k): lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32, contraction k, cols j): lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32): lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// (checked on the hardware with exact small-integer products).
//
// LDS transpose read ds_read_b64_tr_b16, per group of 16 lanes: if lane s of
// the group points at 4 consecutive 16-bit values R[s][0..3], lane j of the
// group receives R[4 e + j / 4][j % 4] in element e.  Pointing lane s at row
// (kbase + s / 4), columns (cbase + 4 (s % 4)) .. +3 of a row-major matrix
// gives lane j the column cbase + j, rows kbase .. kbase + 3: a 4 x 16 block
// read transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two FP32 values -> packed BF16 pair (lo = a, hi = b), round to nearest even
// (one v_cvt_pk_bf16_f32).  Written as a vector conversion the compiler knows,
// not inline assembly, so its hazard checks see the instruction (a
// transcendental result read by the next VALU instruction needs a wait state).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 r = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Round an FP32 value to BF16 precision (nearest even), result as FP32.
__device__ __forceinline__ float round_bf16(float x) { return bf16lo_to_f32(pack_bf16(x, 0.f)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float med3(float a, float b, float c) { return __builtin_amdgcn_fmed3f(a, b, c); }


// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xchg32(float x) { return __shfl_xor(x, 32, 64); }

// The value of x in this lane and in the lane 32 positions away, in an order
// that depends on the lane (v_permlane32_swap): use only symmetric functions
// of the pair (max, min, sum).
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __uint_as_float(r0);
  b = __uint_as_float(r1);
}

// Two transpose reads of 4 x 16 blocks from a row-major LDS tile whose rows
// are `row_bytes` long and whose 16-byte chunks are XOR-swizzled by row.
__device__ __forceinline__ u32x2 lds_read_tr(const char* lds_base, int byte_off) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_base + byte_off));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 lds_read_b128(const char* lds_base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(lds_base + byte_off);
}

__device__ __forceinline__ void lds_write_b128(char* lds_base, int byte_off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(lds_base + byte_off) = v;
}

// XOR pattern applied to the 16-byte chunk index of a row of a row-major BF16
// tile in LDS (CHUNKS = 16-byte chunks per row: 16 for 128 features, 8 for
// 64).  Two read patterns must both be free of bank conflicts:
//  * 16 lanes reading one chunk from each of 16 different rows (MFMA operands
//    read with ds_read_b128): the pattern is a permutation of the rows mod 16;
//  * the transpose read: 4 consecutive rows (4-aligned) x 4 consecutive chunks
//    (4-aligned): the pattern sends each of the 4 rows to its own 64-byte
//    quad of banks.
// 16 chunks: bits 0-1 of the row select the quad, bits 2-3 the chunk within it.
// 8 chunks (two rows share a 256-byte bank line): bit 1 of the row selects the
// quad, bits 2-3 the chunk.
template <int CHUNKS>
__device__ __forceinline__ int swz_pattern(int row) {
  if (CHUNKS == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Swizzled byte offset of 16-byte chunk `chunk` of row `row`.
template <int CHUNKS>
__device__ __forceinline__ int swz(int row, int chunk) {
  return (row * CHUNKS + (chunk ^ swz_pattern<CHUNKS>(row))) * 16;
}

// Byte offset of element (row, col) of a swizzled row-major BF16 tile.
template <int CHUNKS>
__device__ __forceinline__ int swz_elem(int row, int col) {
  return swz<CHUNKS>(row, col >> 3) + (col & 7) * 2;
}

__device__ __forceinline__ u32x4 ldg_b128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at lds_wave_base + 16 * l.  lds_wave_base must be the
// same for the whole wave.  Completion is tracked by vmcnt.
__device__ __forceinline__ void g2lds_b128(const void* gptr, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Buffer resource for raw byte-offset loads from base .. base + bytes - 1
// (stride 0, 32-bit data format word of the gfx9 family).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Direct buffer -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds)
// from byte offset voff + soff of the resource: lane l's bytes land at
// lds_wave_base + 16 * l.  soff and lds_wave_base must be wave-uniform.
__device__ __forceinline__ void buf2lds_b128(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                             char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base,
                                           16, voff, soff, 0, 0);
}

// Wait for every outstanding memory operation of this wave (including direct
// loads into LDS), then the workgroup barrier.
__device__ __forceinline__ void wait_all_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Sum of the two BF16 values packed in u, accumulated onto acc in FP32.
__device__ __forceinline__ float add_bf16_pair(uint32_t u, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

}  // namespace pfa

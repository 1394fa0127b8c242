// Internal definitions shared by the HIP translation units of liblq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lq.h"

namespace lq {

// NF4 levels and the 15 decision points between them, passed by value to the
// kernels that need them (built once on the host, see codebook.cpp).
struct NF4Table {
  float cb[16];
  float thr[15];
  float pad;
};

// host: built on first use, immutable afterwards; LQ_CB_NF4 or
// LQ_CB_NF4_SYMMETRIC
const NF4Table& nf4_table(int32_t codebook);

// Multi-adapter rank layout, passed to the kernels by value.  Adapter a owns
// the concatenated rank columns roff[a] .. roff[a+1]-1 and the scale scale[a]
// (its alpha_a / r_a); its B (N x r_a, row-major) starts at element N roff[a]
// of the concatenated B, so rank column c of output row n is element
// col_base[c] + n col_stride[c].  Uniform ranks are the case roff[a] = a r.
constexpr int kMaxRankCols = 64;
struct MultiTab {
  int32_t n_ad;
  int32_t rc;  // total rank columns
  int32_t roff[kMaxRankCols + 1];
  float scale[kMaxRankCols];
  int32_t col_base[kMaxRankCols];
  int32_t col_stride[kMaxRankCols];
  float oscale = 1.0f;  // skinny products: every stored result times this (dropout's 1 / (1 - p))
};

// Per-thread error reporting used by the ABI layer.
void set_error(const char* fmt, ...);
int hip_fail(hipError_t e, const char* where);

// Event brackets around a kernel launch (no-ops unless lq_timing_enable).
void timing_begin(const char* name, hipStream_t st);
void timing_end(hipStream_t st);
bool timing_enabled();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float32 -> bfloat16 (finite inputs).  gfx950 has a
// native packed conversion with the default rounding mode (nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Second-level step fl32(c2 / 127) with IEEE division (correctly rounded).
__device__ __forceinline__ float dq_step(float c2) { return c2 / 127.0f; }

// Value of a non-negative E4M3 code q (0..126): 4 exponent bits with bias 7,
// 3 mantissa bits, subnormals m * 2^-9.  Exact: a small integer times a power
// of two.
__device__ __forceinline__ float e4m3_value(uint32_t q) {
  const uint32_t e = (q >> 3) & 15u, m = q & 7u;
  const uint32_t mant = e ? (m | 8u) : m;              // (8 + m) or m
  const uint32_t ex = (e ? e : 1u) + 127u - 10u;       // 2^(e - 10), subnormal 2^-9
  return (float)mant * __uint_as_float(ex << 23);
}

// The value the 8-bit second-level constant stands for: the integer itself
// (LQ_DQ_INT8) or the E4M3 value of the byte (LQ_DQ_FP8).
template <bool FP8>
__device__ __forceinline__ float dq_value(uint32_t q) {
  return FP8 ? e4m3_value(q) : (float)q;
}

// The same with the format a uniform argument: LQ_DQ_INT8 or LQ_DQ_FP8.
__device__ __forceinline__ float dq_q_rt(int32_t dq, uint32_t q) {
  return dq == LQ_DQ_FP8 ? dq_value<true>(q) : dq_value<false>(q);
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace lq

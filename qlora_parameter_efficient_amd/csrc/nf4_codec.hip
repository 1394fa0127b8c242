// NF4 quantisation with blockwise absmax and 8-bit double quantisation, and
// the standalone dequantiser.
//
// "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ..."
// (llms.blog), sections "1. 4-bit NormalFloat (NF4) Quantization" (absmax per
// block, normalise, nearest level) and "2. Double Quantization (DQ)"
// (c1_8bit = round(c1 / c2 * 127) over 256 first-level constants);
// "Large Language Model Fine-tuning and LoRA" (aicomputerinstitute.com),
// section "Quantizing the frozen weights" (block size 64, DQ block 256).
//
// Both kernels are HBM-bound streaming passes.  Bit-exactness rests on: exact
// float32 max, correctly rounded float32 division (HIP's default), no fused
// multiply-add anywhere in the arithmetic (only lone products and quotients),
// rintf (ties to even) for the 8-bit integer constant or an exact bit-level
// E4M3 rounding for the FP8 one, and RNE for bf16 stores.
#include "common.h"
#include "nf4_deq.h"

namespace lq {
namespace {

constexpr int kGroupElems = LQ_NF4_BLOCK * LQ_NF4_DQ_BLOCK;  // 16384
constexpr int kQuantThreads = 256;
constexpr int kChunk = 8;            // elements per thread per step
constexpr int kSteps = kGroupElems / (kQuantThreads * kChunk);  // 8

template <typename T>
__device__ __forceinline__ void load8(const T* W, int64_t e0, int64_t n, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* W, int64_t e0, int64_t n,
                                                float (&v)[8]) {
  if (e0 + 8 <= n) {
    u32x4 q = *reinterpret_cast<const u32x4*>(W + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = lo_bf16(q[i]);
      v[2 * i + 1] = hi_bf16(q[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < n) ? bf16_to_f32(W[e0 + i]) : 0.0f;
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* W, int64_t e0, int64_t n, float (&v)[8]) {
  if (e0 + 8 <= n) {
    f32x4 a = *reinterpret_cast<const f32x4*>(W + e0);
    f32x4 b = *reinterpret_cast<const f32x4*>(W + e0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < n) ? W[e0 + i] : 0.0f;
  }
}

// code = number of thresholds strictly below x.  The 15 thresholds ascend, so
// the count is found by a four-level binary search (x > th[c + 2^k - 1]
// decides bit k of c), the same count as comparing against all 15; every
// level is a compare and selects, no branches.  NaN gives 0.
struct Thr {  // named scalars, so that every select below is a register select
  float t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11, t12, t13, t14;
};

// each threshold held in a register the compiler cannot see through, so that
// it keeps the selects as register selects instead of indexing memory
__device__ __forceinline__ float in_reg(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ Thr make_thr(const NF4Table& tab) {
  return Thr{in_reg(tab.thr[0]),  in_reg(tab.thr[1]),  in_reg(tab.thr[2]),  in_reg(tab.thr[3]),
             in_reg(tab.thr[4]),  in_reg(tab.thr[5]),  in_reg(tab.thr[6]),  in_reg(tab.thr[7]),
             in_reg(tab.thr[8]),  in_reg(tab.thr[9]),  in_reg(tab.thr[10]), in_reg(tab.thr[11]),
             in_reg(tab.thr[12]), in_reg(tab.thr[13]), in_reg(tab.thr[14])};
}

// value select (operands by value: a ternary on two lvalues would select
// addresses and load)
__device__ __forceinline__ float fsel(bool c, float a, float b) { return c ? a : b; }

__device__ __forceinline__ uint32_t nf4_code(float x, const Thr t) {
  const bool b3 = x > t.t7;
  const bool b2 = x > fsel(b3, t.t11, t.t3);
  const bool b1 = x > fsel(b3, fsel(b2, t.t13, t.t9), fsel(b2, t.t5, t.t1));
  const float l0h = fsel(b2, fsel(b1, t.t14, t.t12), fsel(b1, t.t10, t.t8));
  const float l0l = fsel(b2, fsel(b1, t.t6, t.t4), fsel(b1, t.t2, t.t0));
  const bool b0 = x > fsel(b3, l0h, l0l);
  return (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// Nearest non-negative E4M3 code to y in [0, 448], ties to the even code.
// Below 2^-6 the codes are the subnormals m * 2^-9, so the code is rint(y *
// 512) (8 is the first normal, 2^-6); above, the float32 exponent and the top
// three mantissa bits form the code, rounded half-even on the dropped bits
// (a carry out of the mantissa steps the exponent, as the encoding does).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  if (y < 0.015625f) return (uint32_t)__builtin_rintf(y * 512.0f);
  const uint32_t b = __float_as_uint(y);
  const uint32_t e = (b >> 23) - 127u + 7u;
  const uint32_t mant = (b >> 20) & 7u;
  const uint32_t rest = b & 0xFFFFFu;
  const uint32_t up = (rest > 0x80000u || (rest == 0x80000u && (mant & 1u))) ? 1u : 0u;
  return ((e << 3) | mant) + up;
}

// One workgroup per group of 256 blocks (16384 elements).  Step s, thread t
// handles elements [g0 + (s*256 + t)*8, +8): eight consecutive threads cover
// one 64-element block, whose absmax is reduced across those lanes.
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void nf4_quantize_kernel(
    const T* __restrict__ W, int64_t n, int32_t double_quant, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ q8, float* __restrict__ c2out, float* __restrict__ absmax,
    NF4Table tab) {
  __shared__ float c1s[LQ_NF4_DQ_BLOCK];
  __shared__ float wmax[kQuantThreads / 64];
  const int t = threadIdx.x;
  const Thr th = make_thr(tab);
  const int64_t g0 = (int64_t)blockIdx.x * kGroupElems;
  const int64_t nb_total = (n + LQ_NF4_BLOCK - 1) / LQ_NF4_BLOCK;

  // all steps' loads are issued before any arithmetic
  float vall[kSteps][8];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int64_t e0 = g0 + (int64_t)(s * kQuantThreads + t) * kChunk;
    if (e0 < n) {
      load8<T>(W, e0, n, vall[s]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) vall[s][i] = 0.0f;
    }
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int chunk = s * kQuantThreads + t;
    const int64_t e0 = g0 + (int64_t)chunk * kChunk;
    const float (&v)[8] = vall[s];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    // max over the 8 lanes of this block (lanes 8k .. 8k+7)
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const float c1 = m;
    if ((t & 7) == 0) c1s[chunk >> 3] = c1;
    const int64_t byte0 = e0 >> 1;
    if (e0 + 8 <= n) {
      // whole chunk, no per-element branches: the eight divisions interleave.
      // c1 == 0 (an all-zero block) encodes every element as level 7 (the
      // zero of the default codebook; the level nearest zero otherwise).
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t code = nf4_code(v[i] / c1, th);
        packed |= (c1 != 0.0f ? code : 7u) << (4 * i);
      }
      *reinterpret_cast<uint32_t*>(codes + byte0) = packed;
    } else if (e0 < n) {
      uint32_t packed = 0;
      for (int i = 0; i < 8; ++i) {
        uint32_t code = 7u;
        if (e0 + i >= n) code = 0u;  // padding nibble past the end stays 0
        else if (c1 != 0.0f) code = nf4_code(v[i] / c1, th);
        packed |= code << (4 * i);
      }
      const int64_t nbytes = (n - e0 + 1) >> 1;
      for (int64_t b = 0; b < nbytes; ++b) codes[byte0 + b] = (uint8_t)(packed >> (8 * b));
    }
  }
  __syncthreads();

  const int64_t blk = (int64_t)blockIdx.x * LQ_NF4_DQ_BLOCK + t;
  const float c1 = c1s[t];
  if (!double_quant) {
    if (blk < nb_total) absmax[blk] = c1;
    return;
  }
  // c2 = max c1 over the group (blocks past the end hold 0)
  float m = c1;
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  if (t == 0) c2out[blockIdx.x] = c2;
  if (blk < nb_total) {
    uint32_t q = 0;
    if (c2 != 0.0f) {
      const float ratio = c1 / c2;
      const float scaled = ratio * 127.0f;
      q = double_quant == LQ_DQ_FP8 ? e4m3_code(scaled) : (uint32_t)__builtin_rintf(scaled);
    }
    q8[blk] = (uint8_t)q;
  }
}

template <bool BF16OUT>
__global__ __launch_bounds__(kDeqThreads) void nf4_dequantize_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ q8,
    const float* __restrict__ c2, const float* __restrict__ absmax, int32_t double_quant,
    int64_t n, void* __restrict__ out, NF4Table tab) {
  nf4_deq_span<BF16OUT>(threadIdx.x, blockIdx.x, codes, q8, c2, absmax, double_quant, n, out, tab);
}

}  // namespace

int launch_nf4_quantize(const void* W, lq_dtype wdt, int64_t n, int32_t double_quant,
                        int32_t codebook, uint8_t* codes, uint8_t* q8, float* c2, float* absmax,
                        hipStream_t stream) {
  const int64_t groups = cdiv(n, kGroupElems);
  const NF4Table& tab = nf4_table(codebook);
  if (wdt == LQ_BF16) {
    hipLaunchKernelGGL(nf4_quantize_kernel<uint16_t>, dim3((unsigned)groups), dim3(kQuantThreads),
                       0, stream, (const uint16_t*)W, n, double_quant, codes, q8, c2, absmax, tab);
  } else {
    hipLaunchKernelGGL(nf4_quantize_kernel<float>, dim3((unsigned)groups), dim3(kQuantThreads), 0,
                       stream, (const float*)W, n, double_quant, codes, q8, c2, absmax, tab);
  }
  return hip_fail(hipGetLastError(), "nf4_quantize launch");
}

int launch_nf4_dequantize(const uint8_t* codes, const uint8_t* q8, const float* c2,
                          const float* absmax, int32_t double_quant, int32_t codebook, int64_t n,
                          void* out, lq_dtype odt, hipStream_t stream) {
  const int64_t blocks = cdiv(n, kDeqSpan);
  const NF4Table& tab = nf4_table(codebook);
  if (odt == LQ_BF16) {
    hipLaunchKernelGGL(nf4_dequantize_kernel<true>, dim3((unsigned)blocks), dim3(kDeqThreads), 0,
                       stream, codes, q8, c2, absmax, double_quant, n, out, tab);
  } else {
    hipLaunchKernelGGL(nf4_dequantize_kernel<false>, dim3((unsigned)blocks), dim3(kDeqThreads), 0,
                       stream, codes, q8, c2, absmax, double_quant, n, out, tab);
  }
  return hip_fail(hipGetLastError(), "nf4_dequantize launch");
}

}  // namespace lq

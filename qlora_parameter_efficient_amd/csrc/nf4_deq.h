// NF4 -> bf16 / float32 dequantisation of one 32768-element span, shared by
// the standalone dequantiser and the large-M prep kernel.
//
// ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ...",
// sections "1. 4-bit NormalFloat (NF4) Quantization" and "2. Double
// Quantization (DQ)": w = cb[code] * a', a' = q * (c2 / 127) with q the
// integer or the E4M3 value of the 8-bit constant.)
//
// 256 threads cover 32768 elements (two groups of 256 blocks); thread t owns
// the 16 chunks of 8 elements t + 256 i, so consecutive lanes read
// consecutive code words and write consecutive 16-byte (bf16) or 32-byte
// (float32) pieces.  All code words and block constants are loaded before any
// arithmetic; the second-level steps fl32(c2 / 127) of the span's groups come
// from a small LDS table.  A partial last chunk (n not a multiple of 8) is
// finished element by element.  Bit-exact: lone float32 products, RNE stores.
#pragma once

#include "common.h"

namespace lq {

constexpr int kDeqThreads = 256;
constexpr int kDeqChunks = 16;                                       // chunks of 8 per thread
constexpr int64_t kDeqSpan = (int64_t)kDeqThreads * kDeqChunks * 8;  // 32768 elements
constexpr int64_t kDeqGroup = (int64_t)LQ_NF4_BLOCK * LQ_NF4_DQ_BLOCK;  // 16384

// t in [0, 256); every thread of the workgroup calls it (it synchronises).
template <bool BF16OUT>
__device__ __forceinline__ void nf4_deq_span(int t, int64_t span, const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ q8,
                                             const float* __restrict__ c2,
                                             const float* __restrict__ absmax,
                                             int32_t double_quant, int64_t n,
                                             void* __restrict__ out, const NF4Table& tab) {
  __shared__ float cbs[16];
  __shared__ float steps[4];
  const int64_t base = span * kDeqSpan;
  const int64_t g_lo = base / kDeqGroup;
  const int64_t ngroups = (n + kDeqGroup - 1) / kDeqGroup;
  if (t < 16) cbs[t] = tab.cb[t];
  if (double_quant && t < 3 && g_lo + t < ngroups) steps[t] = dq_step(c2[g_lo + t]);
  uint32_t cw[kDeqChunks], qv[kDeqChunks];
#pragma unroll
  for (int i = 0; i < kDeqChunks; ++i) {
    int64_t e = base + 8 * (int64_t)(t + kDeqThreads * i);
    e = e < n ? e : 0;  // chunks past the end are not stored
    const int64_t blk = e / LQ_NF4_BLOCK;
    cw[i] = e + 8 <= n ? *reinterpret_cast<const uint32_t*>(codes + (e >> 1)) : 0u;
    qv[i] = double_quant ? (uint32_t)q8[blk] : __float_as_uint(absmax[blk]);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kDeqChunks; ++i) {
    const int64_t e = base + 8 * (int64_t)(t + kDeqThreads * i);
    if (e >= n) continue;
    const float qf = double_quant == LQ_DQ_FP8 ? dq_value<true>(qv[i]) : dq_value<false>(qv[i]);
    const float a = double_quant ? qf * steps[e / kDeqGroup - g_lo] : __uint_as_float(qv[i]);
    if (e + 8 <= n) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = cbs[(cw[i] >> (4 * j)) & 15u] * a;
      if (BF16OUT) {
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + e) =
            u32x4{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                  pack_bf16x2(w[6], w[7])};
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e);
        dst[0] = f32x4{w[0], w[1], w[2], w[3]};
        dst[1] = f32x4{w[4], w[5], w[6], w[7]};
      }
    } else {
      for (int64_t k = e; k < n; ++k) {
        const uint32_t byte = codes[k >> 1];
        const uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
        const float w = cbs[code] * a;
        if (BF16OUT) reinterpret_cast<uint16_t*>(out)[k] = f32_to_bf16(w);
        else reinterpret_cast<float*>(out)[k] = w;
      }
    }
  }
}

}  // namespace lq

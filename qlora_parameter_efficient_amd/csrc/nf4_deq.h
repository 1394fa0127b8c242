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
// (float32) pieces.  A whole span takes the straight-line path: the level
// table (both levels of every code byte) is built in LDS and synchronised
// before any load is issued, then every code word, block constant and the two
// groups' c2 are loaded, and chunk i is finished and stored as soon as its own
// loads have returned (no barrier or branch between the loads and the stores,
// so the stores of the first chunks overlap the arrival of the later ones).
// The last, partial span keeps a general path: second-level steps in a small
// LDS table, a partial last chunk (n not a multiple of 8) finished element by
// element.  Bit-exact either way: lone float32 products, RNE stores.
#pragma once

#include "device_util.h"

namespace lq {

constexpr int kDeqThreads = 256;
constexpr int kDeqChunks = 16;                                       // chunks of 8 per thread
constexpr int64_t kDeqSpan = (int64_t)kDeqThreads * kDeqChunks * 8;  // 32768 elements
constexpr int64_t kDeqGroup = (int64_t)LQ_NF4_BLOCK * LQ_NF4_DQ_BLOCK;  // 16384

// A whole span (base + kDeqSpan <= n) with the constants' format DQ as a
// template parameter; lut is the level table, built and synchronised by the
// caller before this is called.
template <bool BF16OUT, int DQ>
__device__ __forceinline__ void nf4_deq_full(int t, int64_t base, const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ q8,
                                             const float* __restrict__ c2,
                                             const float* __restrict__ absmax,
                                             void* __restrict__ out, const float2* lut) {
  uint32_t cw[kDeqChunks], qv[kDeqChunks];
  float c2v[2] = {1.0f, 1.0f};
  if (DQ != LQ_DQ_NONE) {
    // chunks 0-7 lie in the span's first group, 8-15 in its second (loaded
    // first: the loads return in order, and chunk 0 needs both)
    c2v[0] = c2[base / kDeqGroup];
    c2v[1] = c2[base / kDeqGroup + 1];
  }
#pragma unroll
  for (int i = 0; i < kDeqChunks; ++i) {
    const int64_t e = base + 8 * (int64_t)(t + kDeqThreads * i);
    cw[i] = *reinterpret_cast<const uint32_t*>(codes + (e >> 1));
    qv[i] = DQ != LQ_DQ_NONE ? (uint32_t)q8[e / LQ_NF4_BLOCK]
                             : __float_as_uint(absmax[e / LQ_NF4_BLOCK]);
    // issue order kept: chunk by chunk, every load before the first wait
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < kDeqChunks; ++i) {
    const int64_t e = base + 8 * (int64_t)(t + kDeqThreads * i);
    const float a = DQ != LQ_DQ_NONE
                        ? dq_value<DQ == LQ_DQ_FP8>(qv[i]) * dq_step(c2v[i >= kDeqChunks / 2])
                        : __uint_as_float(qv[i]);
    const LutFetch f = lut_fetch(cw[i], lut);
    if (BF16OUT) {
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + e) = lut_finish(f, a);
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e);
      dst[0] = f32x4{f.v[0].x * a, f.v[0].y * a, f.v[1].x * a, f.v[1].y * a};
      dst[1] = f32x4{f.v[2].x * a, f.v[2].y * a, f.v[3].x * a, f.v[3].y * a};
    }
    // chunk by chunk, so that no later chunk's data is waited for early
    __builtin_amdgcn_sched_barrier(0);
  }
}

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
  __shared__ float2 lut[256];
  const int64_t base = span * kDeqSpan;
  if (base + kDeqSpan <= n) {  // uniform
    build_lut(lut, tab);
    __syncthreads();
    if (double_quant == LQ_DQ_INT8)
      nf4_deq_full<BF16OUT, LQ_DQ_INT8>(t, base, codes, q8, c2, absmax, out, lut);
    else if (double_quant == LQ_DQ_FP8)
      nf4_deq_full<BF16OUT, LQ_DQ_FP8>(t, base, codes, q8, c2, absmax, out, lut);
    else
      nf4_deq_full<BF16OUT, LQ_DQ_NONE>(t, base, codes, q8, c2, absmax, out, lut);
    return;
  }
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

// LoRA-input dropout: the adapter branch sees D(X) = X * keep / (1 - p), the
// base product the undropped X ("Lesson 26: LoRA / QLoRA theory", section
// "Putting It Together": the adapter configuration's lora_dropout).  The mask
// is drawn by the caller and passed packed one bit per element of X, bit j of
// byte i for element 8 i + j.
//
// The dropout forward and backward reuse the library's product kernels and
// add three small streaming kernels around them:
//   keep_apply_kernel   X_d = X * keep (bf16; each element is X or 0), the
//                       operand of every adapter-side reduction
//   t_finish_kernel     T *= 1 / (1 - p) in place and, for the fused forward,
//                       Tm = bf16(s T) padded to the expand's rank width
//   dx_fixup_kernel     dX += s ((U' A) * keep) for the backward, with
//                       U' = U / (1 - p) already scaled
// The 1/(1 - p) factor is applied to the float32 rank-r factors (T, U), never
// to a bf16 activation, so no extra rounding touches X.

#include <hip/hip_runtime.h>

#include "common.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kKeepThreads = 256;
constexpr int kKeepChunks = 4;  // 8-element chunks per thread

// 16-bit lane masks of one 8-element chunk from its mask byte
__device__ __forceinline__ u32x4 keep_lanes(uint32_t b) {
  u32x4 m;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (b >> (2 * i)) & 1u ? 0x0000FFFFu : 0u;
    const uint32_t hi = (b >> (2 * i + 1)) & 1u ? 0xFFFF0000u : 0u;
    m[i] = lo | hi;
  }
  return m;
}

__global__ __launch_bounds__(kKeepThreads) void keep_apply_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ keep, int64_t n8,
    uint16_t* __restrict__ Xd) {
  const int64_t c0 = (int64_t)blockIdx.x * kKeepThreads * kKeepChunks + threadIdx.x;
  u32x4 v[kKeepChunks];
  uint32_t b[kKeepChunks];
#pragma unroll
  for (int u = 0; u < kKeepChunks; ++u) {
    const int64_t c = c0 + (int64_t)u * kKeepThreads;
    const int64_t cc = c < n8 ? c : 0;
    v[u] = *reinterpret_cast<const u32x4*>(X + 8 * cc);
    b[u] = keep[cc];
  }
#pragma unroll
  for (int u = 0; u < kKeepChunks; ++u) {
    const int64_t c = c0 + (int64_t)u * kKeepThreads;
    if (c < n8) *reinterpret_cast<u32x4*>(Xd + 8 * c) = v[u] & keep_lanes(b[u]);
  }
}

__global__ __launch_bounds__(256) void t_finish_kernel(float* __restrict__ T, int64_t M, int r,
                                                       float inv_keep, float s,
                                                       uint16_t* __restrict__ Tm, int rp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int w = Tm ? rp : r;
  if (i >= M * w) return;
  const int64_t m = i / w;
  const int c = (int)(i - m * w);
  if (c < r) {
    const float t = T[m * r + c] * inv_keep;
    T[m * r + c] = t;
    if (Tm) Tm[m * rp + c] = f32_to_bf16(s * t);
  } else {
    Tm[m * rp + c] = 0;
  }
}

// One workgroup: 32 rows x 256 columns.  Thread t owns the 8 columns
// 8 (t % 32) and the rows 4 (t / 32) .. +3 of the tile; it accumulates
// sum_j U'[m][j] A[j][k] in float32 for its 4 x 8 outputs, one A row chunk
// (16 bytes, shared through L1 by the tile's eight row groups) per j.
constexpr int kFixRows = 32, kFixCols = 256;

__global__ __launch_bounds__(256) void dx_fixup_kernel(uint16_t* __restrict__ dX,
                                                       const float* __restrict__ U,
                                                       const uint16_t* __restrict__ A,
                                                       const uint8_t* __restrict__ keep,
                                                       int64_t M, int64_t K, int r, float s,
                                                       int col_tiles) {
  const int t = threadIdx.x;
  const int64_t m0 = (int64_t)(blockIdx.x / col_tiles) * kFixRows + 4 * (t >> 5);
  const int64_t k = (int64_t)(blockIdx.x % col_tiles) * kFixCols + 8 * (t & 31);
  if (k >= K) return;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
  int64_t mr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mr[i] = m0 + i < M ? m0 + i : M - 1;  // clamped reads
  for (int j = 0; j < r; ++j) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(A + (int64_t)j * K + k);
    float af[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      af[2 * d] = lo_bf16(a[d]);
      af[2 * d + 1] = hi_bf16(a[d]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = U[mr[i] * r + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] += u * af[e];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + i;
    if (m >= M) break;
    const int64_t off = m * K + k;
    const uint32_t b = keep[off >> 3];
    const u32x4 x = *reinterpret_cast<const u32x4*>(dX + off);
    float o[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      o[2 * d] = lo_bf16(x[d]) + (((b >> (2 * d)) & 1u) ? s * acc[i][2 * d] : 0.0f);
      o[2 * d + 1] = hi_bf16(x[d]) + (((b >> (2 * d + 1)) & 1u) ? s * acc[i][2 * d + 1] : 0.0f);
    }
    *reinterpret_cast<u32x4*>(dX + off) =
        u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
              pack_bf16x2(o[6], o[7])};
  }
}

}  // namespace

namespace dispatch {

int launch_keep_apply(const void* X, const uint8_t* keep, int64_t M, int64_t K, void* Xd,
                      hipStream_t st) {
  const int64_t n8 = M * K / 8;
  if (n8 == 0) return LQ_OK;
  const int64_t blocks = cdiv(n8, (int64_t)kKeepThreads * kKeepChunks);
  hipLaunchKernelGGL(keep_apply_kernel, dim3((unsigned)blocks), dim3(kKeepThreads), 0, st,
                     (const uint16_t*)X, keep, n8, (uint16_t*)Xd);
  return hip_fail(hipGetLastError(), "keep_apply launch");
}

int launch_t_finish(float* T, int64_t M, int64_t r, float inv_keep, float s, void* Tm, int rp,
                    hipStream_t st) {
  const int64_t n = M * (Tm ? rp : r);
  if (n == 0) return LQ_OK;
  hipLaunchKernelGGL(t_finish_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, st, T, M,
                     (int)r, inv_keep, s, (uint16_t*)Tm, rp);
  return hip_fail(hipGetLastError(), "t_finish launch");
}

int launch_dx_fixup(void* dX, const float* U, const void* A, const uint8_t* keep, int64_t M,
                    int64_t K, int64_t r, float s, hipStream_t st) {
  if (M == 0) return LQ_OK;
  const int col_tiles = (int)cdiv(K, kFixCols);
  const int64_t blocks = cdiv(M, kFixRows) * col_tiles;
  hipLaunchKernelGGL(dx_fixup_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint16_t*)dX, U,
                     (const uint16_t*)A, keep, M, K, (int)r, s, col_tiles);
  return hip_fail(hipGetLastError(), "dx_fixup launch");
}

}  // namespace dispatch
}  // namespace lq

// Deployment merge W_final = deq(W0) + s B A, written as a dense bf16 N x K
// matrix ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations
// ...", section "1. Static Weight Merging"; "Large Language Model Fine-tuning
// and LoRA", section "Merging adapters vs keeping them separate": a one-time
// product of 2 d_out r d_in FLOPs, the result keeping W0's shape).
//
// HBM-bound: the kernel reads W0 (NF4 or bf16) and writes the merged matrix
// once.  A workgroup owns a 32 x 256 tile: its four waves form s B A for the
// tile on MFMA (the rank r is the reduction, so one or a few instructions per
// 32 x 32 block) into an LDS tile, then every thread takes 32 consecutive
// elements of one row, dequantises them (to the same bf16 value the fused
// GEMM multiplies by), adds the low-rank term in float32 and stores the bf16
// result with 16-byte writes.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;
constexpr int kTN = 32, kTK = 256;
constexpr int kSPitch = kTK + 4;

struct MergeParams {
  WeightArgs W;
  const uint16_t* A;  // r x K
  const uint16_t* B;  // N x r
  int32_t r;
  float s;
  int32_t k_tiles;
  int32_t pad;
  uint16_t* out;      // N x K
  NF4Table tab;
};

template <int WK>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  __shared__ float S[kTN * kSPitch];
  __shared__ float2 lut[256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t N = p.W.N, K = p.W.K;
  const int tk = blockIdx.x % p.k_tiles, tn = blockIdx.x / p.k_tiles;
  const int64_t n0 = (int64_t)tn * kTN, k0 = (int64_t)tk * kTK;
  const int r = p.r;
  if (WK != 0) build_lut(lut, p.tab);

  // low-rank term: C[k][n] = sum_j A[j][k] B[n][j]  (A operand rows = k)
  const int64_t kw = k0 + 64 * wave;
  if (kw < K) {
    f32x16 acc[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ks][v] = 0.0f;
    const uint16_t* brow = p.B + (n0 + l32) * r;
    for (int c = 0; c * 16 < r; ++c) {
      uint32_t bv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * c + 8 * h + 2 * e;
        const uint32_t lo = (j < r) ? brow[j] : 0u;
        const uint32_t hi = (j + 1 < r) ? brow[j + 1] : 0u;
        bv[e] = lo | (hi << 16);
      }
      const u32x4 bf{bv[0], bv[1], bv[2], bv[3]};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int64_t k = kw + 32 * ks + l32;
        uint32_t av[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * c + 8 * h + 2 * e;
          const uint32_t lo = (j < r) ? p.A[(int64_t)j * K + k] : 0u;
          const uint32_t hi = (j + 1 < r) ? p.A[(int64_t)(j + 1) * K + k] : 0u;
          av[e] = lo | (hi << 16);
        }
        acc[ks] = mfma32(u32x4{av[0], av[1], av[2], av[3]}, bf, acc[ks]);
      }
    }
    // lane: n = n0 + l32, k = kw + 32 ks + 8 q + 4 h + i
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = 64 * wave + 32 * ks + 8 * q + 4 * h;
        *reinterpret_cast<f32x4*>(&S[l32 * kSPitch + kk]) =
            f32x4{p.s * acc[ks][4 * q], p.s * acc[ks][4 * q + 1], p.s * acc[ks][4 * q + 2],
                  p.s * acc[ks][4 * q + 3]};
      }
  }
  __syncthreads();

  const int row = tid >> 3, kc = (tid & 7) * 32;
  const int64_t n = n0 + row, k = k0 + kc;
  if (k >= K) return;
  const float* srow = &S[row * kSPitch + kc];
  float w[32];
  if (WK == 0) {
    const u32x4* src = reinterpret_cast<const u32x4*>(p.W.dense + n * K + k);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 v = src[d];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[8 * d + 2 * i] = lo_bf16(v[i]);
        w[8 * d + 2 * i + 1] = hi_bf16(v[i]);
      }
    }
  } else {
    const int64_t e = n * K + k;
    const u32x4 cw = *reinterpret_cast<const u32x4*>(p.W.codes + (e >> 1));
    ScaleCache sc;
    sc.init();
    const float a = sc.scale(p.W, e >> 6);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 v = deq8(cw[d], a, lut);  // bf16 values the GEMM would use
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[8 * d + 2 * i] = lo_bf16(v[i]);
        w[8 * d + 2 * i + 1] = hi_bf16(v[i]);
      }
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(p.out + n * K + k);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(w[8 * d + 2 * i] + srow[8 * d + 2 * i],
                         w[8 * d + 2 * i + 1] + srow[8 * d + 2 * i + 1]);
    dst[d] = o;
  }
}

}  // namespace

namespace dispatch {

int bf16_merge(const lq_weight& W, const void* A, const void* B, int64_t r, float s, void* Wout,
               hipStream_t st) {
  MergeParams p;
  p.W = weight_args(W);
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.r = (int32_t)r;
  p.s = s;
  p.k_tiles = (int32_t)cdiv(W.K, kTK);
  p.pad = 0;
  p.out = (uint16_t*)Wout;
  p.tab = nf4_table();
  const unsigned blocks = (unsigned)(p.k_tiles * (W.N / kTN));
  if (W.kind == LQ_WEIGHT_DENSE)
    hipLaunchKernelGGL(merge_kernel<0>, dim3(blocks), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(merge_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, p);
  return hip_fail(hipGetLastError(), "merge launch");
}

}  // namespace dispatch
}  // namespace lq

// Decode-sized forward (M <= 16) and the skinny rank-r products.
//
// Decode: Y = X deq(W0)^T + s T B^T with T = X A^T computed first by the
// skinny kernel.  With at most 16 activation rows the layer is bound by
// streaming W0 from HBM (4.127 bits per weight in NF4 with double
// quantisation: "Large Language Model Fine-tuning and LoRA", section
// "Quantizing the frozen weights"), so the kernel is organised around that
// stream: a workgroup owns 16 output rows n and its four waves split K; each
// lane loads 16 code bytes (32 weights, half a block) per step, dequantises
// them in registers through the LDS level table and feeds four
// v_mfma_f32_16x16x32_bf16 (X padded to 16 rows).  The four partial sums are
// combined through LDS; the rank-r expand is a few scalar FMAs per output.
//
// Skinny: out[m][j] = sum_k Z[m][k] G[j][k] for j < r <= 64, G = A (r x K)
// or B^T (B is K x r here, i.e. the reduction runs over B's rows).  Each wave
// takes 32 rows of Z straight into MFMA registers; the small G tile of each
// step is staged in LDS (transposed for B).
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;

template <int RP, bool GT>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const uint16_t* __restrict__ Z,
                                                          int64_t M, int64_t K,
                                                          const uint16_t* __restrict__ G, int r,
                                                          float* __restrict__ out) {
  constexpr int JT = RP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t gl[RP * kPitch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t mrow = ((int64_t)blockIdx.x * 4 + wave) * 32 + l32;
  const int64_t mr = mrow < M ? mrow : M - 1;
  f32x16 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.0f;
  for (int64_t k0 = 0; k0 < K; k0 += 64) {
    __syncthreads();
    for (int e = tid; e < RP * 64; e += kThreads) {
      int j, kk;
      uint16_t v = 0;
      if (GT) {  // G[j][k] = B[k][j], read B rows coalesced
        kk = e / RP;
        j = e - kk * RP;
        if (j < r && k0 + kk < K) v = G[(k0 + kk) * r + j];
      } else {
        j = e / 64;
        kk = e - j * 64;
        if (j < r && k0 + kk < K) v = G[(int64_t)j * K + k0 + kk];
      }
      gl[j * kPitch + kk] = v;
    }
    __syncthreads();
    const uint16_t* zrow = Z + mr * K + k0 + 32 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok = k0 + 32 * h + 8 * s < K;
      const u32x4 zf = ok ? *reinterpret_cast<const u32x4*>(zrow + 8 * s) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 gf =
            *reinterpret_cast<const u32x4*>(gl + (32 * jt + l32) * kPitch + 32 * h + 8 * s);
        acc[jt] = mfma32(gf, zf, acc[jt]);
      }
    }
  }
  if (mrow >= M) return;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 32 * jt + 8 * q + 4 * h + i;
        if (j < r) out[mrow * r + j] = acc[jt][4 * q + i];
      }
}

int launch_skinny(const uint16_t* Z, int64_t M, int64_t K, const uint16_t* G, bool gt, int64_t r,
                  float* out, hipStream_t st) {
  const unsigned blocks = (unsigned)cdiv(M, 128);
  if (r <= 32) {
    if (gt)
      hipLaunchKernelGGL((skinny_kernel<32, true>), dim3(blocks), dim3(kThreads), 0, st, Z, M, K, G,
                         (int)r, out);
    else
      hipLaunchKernelGGL((skinny_kernel<32, false>), dim3(blocks), dim3(kThreads), 0, st, Z, M, K,
                         G, (int)r, out);
  } else {
    if (gt)
      hipLaunchKernelGGL((skinny_kernel<64, true>), dim3(blocks), dim3(kThreads), 0, st, Z, M, K, G,
                         (int)r, out);
    else
      hipLaunchKernelGGL((skinny_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, st, Z, M, K,
                         G, (int)r, out);
  }
  return hip_fail(hipGetLastError(), "skinny launch");
}

// ------------------------------------------------------------ decode GEMV

struct GemvParams {
  const uint16_t* X;  // M x K
  int64_t M;
  WeightArgs W;
  const float* T;     // M x r
  const uint16_t* B;  // N x r
  int32_t r;
  float s;
  uint16_t* Y;        // M x N
  NF4Table tab;
};

template <int WK>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
  __shared__ float2 lut[256];
  __shared__ f32x4 part[4][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  if (WK != 0) {
    build_lut(lut, p.tab);
    __syncthreads();
  }
  const int64_t n = n0 + l16;  // A-operand row of this lane (N % 32 == 0)
  const bool mrow = l16 < M;   // B-operand column (activation row) of this lane
  const int64_t xm = mrow ? l16 : 0;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  ScaleCache sc;
  sc.init();
  // K is split into 32-element granules (half an NF4 block); a step covers four
  // consecutive granules, one per quarter-wave q, and steps go round-robin to
  // the four waves.  Lanes past the end feed zeros to the MFMA.
  const int64_t G = K / 32;
  const int64_t steps = (G + 3) / 4;
  for (int64_t t = wave; t < steps; t += 4) {
    const int64_t g = 4 * t + q;
    const bool ok = g < G;
    const int64_t k = ok ? 32 * g : 0;
    u32x4 wf[4];
    if (WK == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wf[i] = ok ? *reinterpret_cast<const u32x4*>(p.W.dense + n * K + k + 8 * i)
                   : u32x4{0, 0, 0, 0};
    } else {
      const int64_t e = n * K + k;
      u32x4 cw = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      float a = 0.0f;
      if (ok) {
        cw = *reinterpret_cast<const u32x4*>(p.W.codes + (e >> 1));
        a = sc.scale(p.W, e >> 6);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = deq8(cw[i], a, lut);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 xf = (mrow && ok) ? *reinterpret_cast<const u32x4*>(p.X + xm * K + k + 8 * i)
                                    : u32x4{0, 0, 0, 0};
      acc = mfma16(wf[i], xf, acc);
    }
  }
  // acc lane l: rows n0 + 4 q + i, column m = l16 (16x16 accumulator layout)
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = part[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const f32x4 o = part[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += o[i];
  }
  if (!mrow) return;
  const int64_t m = l16;
  const int r = p.r;
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t nn = n0 + 4 * q + i;
    float d = 0.0f;
    for (int j = 0; j < r; ++j) d = fmaf(p.T[m * r + j], bf16_to_f32(p.B[nn * r + j]), d);
    y[i] = sum[i] + p.s * d;
  }
  *reinterpret_cast<u32x2*>(p.Y + m * N + n0 + 4 * q) =
      u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
}

}  // namespace

namespace dispatch {

int t_only(const void* X, int64_t M, int64_t K, const void* A, int64_t r, float* T,
           hipStream_t st) {
  return launch_skinny((const uint16_t*)X, M, K, (const uint16_t*)A, false, r, T, st);
}

int u_only(const void* dY, int64_t M, int64_t N, const void* B, int64_t r, float* U,
           hipStream_t st) {
  return launch_skinny((const uint16_t*)dY, M, N, (const uint16_t*)B, true, r, U, st);
}

int decode_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
               int64_t r, float s, void* Y, float* T, hipStream_t st) {
  int e = t_only(X, M, W.K, A, r, T, st);
  if (e) return e;
  GemvParams p;
  p.X = (const uint16_t*)X;
  p.M = M;
  p.W = weight_args(W);
  p.T = T;
  p.B = (const uint16_t*)B;
  p.r = (int32_t)r;
  p.s = s;
  p.Y = (uint16_t*)Y;
  p.tab = nf4_table();
  const unsigned blocks = (unsigned)(W.N / 16);
  if (W.kind == LQ_WEIGHT_DENSE)
    hipLaunchKernelGGL(gemv_kernel<0>, dim3(blocks), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(gemv_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, p);
  return hip_fail(hipGetLastError(), "gemv launch");
}

}  // namespace dispatch
}  // namespace lq

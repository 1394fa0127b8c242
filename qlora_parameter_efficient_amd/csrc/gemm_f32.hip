// float32 path: a strided, LDS-tiled GEMM  C = alpha * P Q (+ C)  with an
// optional NF4 operand dequantised on the fly, and the LoRA forward /
// backward / merge composed from it.  Used when the call's dtype is LQ_F32
// (small layers checked at 1e-5); the bf16 path lives in lora_bf16.hip.
//
// Formulas: "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations
// ..." (llms.blog) -- forward h = W0 x + (alpha/r) B A x; section "Gradient
// Dynamics and Backpropagation Mechanics" for dA, dB, dx; section
// "1. Static Weight Merging" for W0 + (alpha/r) B A.
#include "common.h"
#include "dispatch.h"

namespace lq {
namespace {

// Matrix accessor: element (a, b) lives at flattened index a * rs + b * cs.
struct Acc {
  const float* f32;      // dense float32 source (kind 0)
  const uint8_t* codes;  // NF4 source (kind 1)
  const uint8_t* q8;
  const float* c2;
  const float* absmax;
  int64_t rs, cs;
  int32_t kind;
  int32_t double_quant;
  int32_t codebook;
};

__device__ __forceinline__ float acc_load(const Acc& m, int64_t a, int64_t b, const float* cbs) {
  const int64_t e = a * m.rs + b * m.cs;
  if (m.kind == 0) return m.f32[e];
  const uint32_t byte = m.codes[e >> 1];
  const uint32_t code = (e & 1) ? (byte >> 4) : (byte & 15u);
  const int64_t blk = e / LQ_NF4_BLOCK;
  float s;
  if (m.double_quant)
    s = dq_q_rt(m.double_quant, m.q8[blk]) * dq_step(m.c2[blk / LQ_NF4_DQ_BLOCK]);
  else s = m.absmax[blk];
  return cbs[code] * s;
}

constexpr int TS = 16;

// C[I x J] (row-major, ldc) = alpha * sum_k P(i, k) Q(k, j)  (+ C if accumulate)
__global__ __launch_bounds__(TS* TS) void gemm_f32_kernel(Acc P, Acc Q, float* __restrict__ C,
                                                         int64_t ldc, int64_t I, int64_t J,
                                                         int64_t Kd, float alpha, int accumulate,
                                                         NF4Table tab) {
  __shared__ float sp[TS][TS + 1];
  __shared__ float sq[TS][TS + 1];
  __shared__ float cbs[16];
  const int tx = threadIdx.x % TS, ty = threadIdx.x / TS;
  if (threadIdx.x < 16) cbs[threadIdx.x] = tab.cb[threadIdx.x];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.y * TS + ty;
  const int64_t j = (int64_t)blockIdx.x * TS + tx;
  float sum = 0.0f;
  for (int64_t k0 = 0; k0 < Kd; k0 += TS) {
    const int64_t pi = (int64_t)blockIdx.y * TS + ty, pk = k0 + tx;
    sp[ty][tx] = (pi < I && pk < Kd) ? acc_load(P, pi, pk, cbs) : 0.0f;
    const int64_t qk = k0 + ty, qj = (int64_t)blockIdx.x * TS + tx;
    sq[ty][tx] = (qk < Kd && qj < J) ? acc_load(Q, qk, qj, cbs) : 0.0f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TS; ++k) sum = fmaf(sp[ty][k], sq[k][tx], sum);
    __syncthreads();
  }
  if (i < I && j < J) {
    float v = alpha * sum;
    if (accumulate) v += C[i * ldc + j];
    C[i * ldc + j] = v;
  }
}

Acc dense(const float* p, int64_t rs, int64_t cs) {
  Acc a{};
  a.f32 = p;
  a.rs = rs;
  a.cs = cs;
  a.kind = 0;
  return a;
}

Acc weight_acc(const lq_weight& w, int64_t rs, int64_t cs) {
  if (w.kind == LQ_WEIGHT_DENSE) return dense((const float*)w.dense, rs, cs);
  Acc a{};
  a.codes = w.codes;
  a.q8 = w.q8;
  a.c2 = w.c2;
  a.absmax = w.absmax;
  a.double_quant = w.double_quant;
  a.codebook = w.codebook;
  a.rs = rs;
  a.cs = cs;
  a.kind = 1;
  return a;
}

int gemm(const Acc& P, const Acc& Q, float* C, int64_t ldc, int64_t I, int64_t J, int64_t Kd,
         float alpha, int accumulate, hipStream_t stream) {
  if (I == 0 || J == 0) return LQ_OK;
  dim3 grid((unsigned)cdiv(J, TS), (unsigned)cdiv(I, TS));
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(TS * TS), 0, stream, P, Q, C, ldc, I, J, Kd, alpha,
                     accumulate, nf4_table(P.kind ? P.codebook : Q.codebook));
  return hip_fail(hipGetLastError(), "gemm_f32 launch");
}

__global__ void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

int launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
  if (n == 0) return LQ_OK;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, p, n);
  return hip_fail(hipGetLastError(), "zero launch");
}

// Y = X W0^T + s (X A^T) B^T; T (M x r) is float32 scratch (T_out or ws).
int f32_lora_fwd(const float* X, int64_t M, const lq_weight& W, const float* A, const float* B,
                 int64_t r, float s, float* Y, float* T, hipStream_t st) {
  const int64_t N = W.N, K = W.K;
  int rc;
  if ((rc = gemm(dense(X, K, 1), dense(A, 1, K), T, r, M, r, K, 1.0f, 0, st))) return rc;
  if ((rc = gemm(dense(X, K, 1), weight_acc(W, 1, K), Y, N, M, N, K, 1.0f, 0, st))) return rc;
  return gemm(dense(T, r, 1), dense(B, 1, r), Y, N, M, N, r, s, 1, st);
}

// ws holds U (M x r) and, when T_saved is NULL, T (M x r).
int f32_lora_bwd(const float* dY, const float* X, int64_t M, const lq_weight& W, const float* A,
                 const float* B, int64_t r, float s, const float* T_saved, float* dX, float* dA,
                 float* dB, int accumulate, float* ws, hipStream_t st) {
  const int64_t N = W.N, K = W.K;
  int rc;
  float* U = ws;
  const float* T = T_saved;
  const bool grads = dA != nullptr;  // dX only when both gradients are NULL
  if (!T && grads) {
    float* Tw = ws + M * r;
    if ((rc = gemm(dense(X, K, 1), dense(A, 1, K), Tw, r, M, r, K, 1.0f, 0, st))) return rc;
    T = Tw;
  }
  if ((rc = gemm(dense(dY, N, 1), dense(B, r, 1), U, r, M, r, N, 1.0f, 0, st))) return rc;
  if (dX) {
    if ((rc = gemm(dense(dY, N, 1), weight_acc(W, K, 1), dX, K, M, K, N, 1.0f, 0, st))) return rc;
    if ((rc = gemm(dense(U, r, 1), dense(A, K, 1), dX, K, M, K, r, s, 1, st))) return rc;
  }
  if (!grads) return LQ_OK;
  if (M == 0) {
    if (!accumulate) {
      if ((rc = launch_zero_f32(dA, r * K, st))) return rc;
      return launch_zero_f32(dB, N * r, st);
    }
    return LQ_OK;
  }
  if ((rc = gemm(dense(U, 1, r), dense(X, K, 1), dA, K, r, K, M, s, accumulate, st))) return rc;
  return gemm(dense(dY, 1, N), dense(T, r, 1), dB, r, N, r, M, s, accumulate, st);
}

int f32_lora_merge(const lq_weight& W, const float* A, const float* B, int64_t r, float s,
                   float* Wout, hipStream_t st) {
  const int64_t N = W.N, K = W.K;
  int rc;
  if (W.kind == LQ_WEIGHT_DENSE) {
    hipError_t e = hipMemcpyAsync(Wout, W.dense, sizeof(float) * N * K, hipMemcpyDeviceToDevice, st);
    if ((rc = hip_fail(e, "merge copy"))) return rc;
  } else {
    if ((rc = launch_nf4_dequantize(W.codes, W.q8, W.c2, W.absmax, W.double_quant, W.codebook,
                                    N * K, Wout, LQ_F32, st)))
      return rc;
  }
  return gemm(dense(B, r, 1), dense(A, K, 1), Wout, K, N, K, r, s, 1, st);
}

}  // namespace lq

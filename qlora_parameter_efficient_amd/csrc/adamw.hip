// AdamW step on the LoRA factors, many tensors per launch.
//
// Each trainable parameter carries a float32 master weight and float32 AdamW
// moments m and v, plus a 16-bit working weight for the forward and backward
// products ("Large Language Model Fine-tuning and LoRA", section "The real
// memory ledger"; "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical
// Foundations ...", section "The Memory Bottleneck of Full Fine-Tuning").  The
// update is decoupled-weight-decay Adam (Loshchilov and Hutter, 2019):
//   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps),
// with g = grad_scale * gradient, and the working weight is bf16 RNE(p).
//
// The step is a pure stream: 16 bytes read and 14 written per parameter with
// a float32 gradient and a bf16 working copy.  The adapters of a whole model
// are many small tensors (two per adapted linear), so one launch takes a
// table of up to kAdamTensors of them, passed by value; each workgroup owns
// one contiguous span of one tensor and finds its tensor from the table's
// running block counts.  Loads are 16-byte vectors when the tensor's pointers
// allow, and every load of a thread is issued before the arithmetic.

#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "dispatch.h"

namespace lq {
namespace {

using dispatch::kAdamTensors;

constexpr int kAdamThreads = 256;
constexpr int kAdamVec = 4;                                  // elements per vector
constexpr int kAdamIters = 2;                                // vectors per thread
constexpr int kAdamSpan = kAdamThreads * kAdamVec * kAdamIters;  // 2048 per workgroup

struct AdamTab {
  float* master[kAdamTensors];
  float* m[kAdamTensors];
  float* v[kAdamTensors];
  const void* g[kAdamTensors];
  uint16_t* w[kAdamTensors];
  int64_t n[kAdamTensors];
  int32_t blk0[kAdamTensors + 1];  // first workgroup of each tensor; blk0[count] = grid
  int32_t count;
  uint32_t vec;                    // bit i: tensor i takes the 16-byte vector path
  float keep;                      // 1 - lr wd
  float b1, omb1, b2, omb2;        // beta1, 1 - beta1, beta2, 1 - beta2
  float step_size;                 // lr / (1 - beta1^t)
  float inv_sqrt_bc2;              // 1 / sqrt(1 - beta2^t)
  float eps, gscale;
};

struct Upd {
  float p, m, v;
};

__device__ __forceinline__ Upd adam_one(const AdamTab& t, float p, float m, float v, float g) {
  g *= t.gscale;
  p *= t.keep;
  m = t.b1 * m + t.omb1 * g;
  v = t.b2 * v + t.omb2 * (g * g);
  const float denom = sqrtf(v) * t.inv_sqrt_bc2 + t.eps;
  p -= t.step_size * (m / denom);
  return {p, m, v};
}

template <bool BF16G>
__device__ __forceinline__ float load_g(const void* g, int64_t i) {
  if (BF16G) return bf16_to_f32(((const uint16_t*)g)[i]);
  return ((const float*)g)[i];
}

template <bool BF16G>
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(AdamTab t) {
  const int b = blockIdx.x;
  int ti = 0;
  while (ti + 1 < t.count && b >= t.blk0[ti + 1]) ++ti;  // uniform over the workgroup
  const int64_t n = t.n[ti];
  float* __restrict__ P = t.master[ti];
  float* __restrict__ Mo = t.m[ti];
  float* __restrict__ Vo = t.v[ti];
  const void* G = t.g[ti];
  uint16_t* __restrict__ W = t.w[ti];
  const int64_t base = (int64_t)(b - t.blk0[ti]) * kAdamSpan;

  if ((t.vec >> ti) & 1u) {
    f32x4 p[kAdamIters], m[kAdamIters], v[kAdamIters], g[kAdamIters];
    bool ok[kAdamIters];
#pragma unroll
    for (int u = 0; u < kAdamIters; ++u) {
      const int64_t i = base + (int64_t)(u * kAdamThreads + threadIdx.x) * kAdamVec;
      ok[u] = i + kAdamVec <= n;
      if (ok[u]) {
        p[u] = *(const f32x4*)(P + i);
        m[u] = *(const f32x4*)(Mo + i);
        v[u] = *(const f32x4*)(Vo + i);
        if (BF16G) {
          const u32x2 q = *(const u32x2*)((const uint16_t*)G + i);
          g[u] = f32x4{lo_bf16(q[0]), hi_bf16(q[0]), lo_bf16(q[1]), hi_bf16(q[1])};
        } else {
          g[u] = *(const f32x4*)((const float*)G + i);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kAdamIters; ++u) {
      const int64_t i = base + (int64_t)(u * kAdamThreads + threadIdx.x) * kAdamVec;
      if (ok[u]) {
        f32x4 po, mo, vo;
#pragma unroll
        for (int e = 0; e < kAdamVec; ++e) {
          const Upd r = adam_one(t, p[u][e], m[u][e], v[u][e], g[u][e]);
          po[e] = r.p;
          mo[e] = r.m;
          vo[e] = r.v;
        }
        *(f32x4*)(P + i) = po;
        *(f32x4*)(Mo + i) = mo;
        *(f32x4*)(Vo + i) = vo;
        if (W) *(u32x2*)(W + i) = u32x2{pack_bf16x2(po[0], po[1]), pack_bf16x2(po[2], po[3])};
      } else {
        // the ragged end of the tensor, element by element
        for (int e = 0; e < kAdamVec; ++e) {
          if (i + e >= n) break;
          const Upd r = adam_one(t, P[i + e], Mo[i + e], Vo[i + e], load_g<BF16G>(G, i + e));
          P[i + e] = r.p;
          Mo[i + e] = r.m;
          Vo[i + e] = r.v;
          if (W) W[i + e] = f32_to_bf16(r.p);
        }
      }
    }
  } else {
    // pointers not 16-byte aligned: coalesced scalar accesses
    for (int k = threadIdx.x; k < kAdamSpan; k += kAdamThreads) {
      const int64_t i = base + k;
      if (i >= n) break;
      const Upd r = adam_one(t, P[i], Mo[i], Vo[i], load_g<BF16G>(G, i));
      P[i] = r.p;
      Mo[i] = r.m;
      Vo[i] = r.v;
      if (W) W[i] = f32_to_bf16(r.p);
    }
  }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

namespace dispatch {

int adamw_step(const lq_adamw_tensor* ts, int32_t n_tensors, bool bf16_grad, const AdamHyper& h,
               hipStream_t st) {
  AdamTab t{};
  // Scalars in double on the host, then one rounding each, as the kernel's
  // float32 arithmetic uses them.
  t.keep = (float)(1.0 - (double)h.lr * (double)h.weight_decay);
  t.b1 = h.beta1;
  t.omb1 = (float)(1.0 - (double)h.beta1);
  t.b2 = h.beta2;
  t.omb2 = (float)(1.0 - (double)h.beta2);
  const double bc1 = 1.0 - std::pow((double)h.beta1, (double)h.step);
  const double bc2 = 1.0 - std::pow((double)h.beta2, (double)h.step);
  t.step_size = (float)((double)h.lr / bc1);
  t.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  t.eps = h.eps;
  t.gscale = h.grad_scale;

  int32_t i = 0;
  while (i < n_tensors) {
    t.count = 0;
    t.vec = 0;
    int64_t blocks = 0;
    for (; i < n_tensors && t.count < kAdamTensors; ++i) {
      const lq_adamw_tensor& x = ts[i];
      if (x.n == 0) continue;
      const int64_t nb = cdiv(x.n, kAdamSpan);
      if (blocks + nb > (int64_t)INT32_MAX / 2) break;  // launch what is gathered first
      const int c = t.count++;
      t.master[c] = x.master;
      t.m[c] = x.m;
      t.v[c] = x.v;
      t.g[c] = x.grad;
      t.w[c] = (uint16_t*)x.weight;
      t.n[c] = x.n;
      t.blk0[c] = (int32_t)blocks;
      blocks += nb;
      const bool vec = aligned(x.master, 16) && aligned(x.m, 16) && aligned(x.v, 16) &&
                       aligned(x.grad, bf16_grad ? 8 : 16) && aligned(x.weight, 8);
      if (vec) t.vec |= 1u << c;
    }
    if (t.count == 0) continue;
    t.blk0[t.count] = (int32_t)blocks;
    if (bf16_grad)
      hipLaunchKernelGGL(adamw_kernel<true>, dim3((unsigned)blocks), dim3(kAdamThreads), 0, st, t);
    else
      hipLaunchKernelGGL(adamw_kernel<false>, dim3((unsigned)blocks), dim3(kAdamThreads), 0, st, t);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "adamw_kernel launch");
  }
  return LQ_OK;
}

}  // namespace dispatch
}  // namespace lq

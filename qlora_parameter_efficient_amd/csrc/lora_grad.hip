// Adapter gradients, reduced over the batch rows:
//   dA = s (dY B)^T X   (r x K)      dB = s dY^T (X A^T)   (N x r)
// ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ..."
// (llms.blog), section "Gradient Dynamics and Backpropagation Mechanics",
// summed over the rows of the batch.)
//
// Both have the form out[j][c] = s * sum_m V[m][j] Z[m][c] with V = U or T
// (M x r float32, from the dX / forward kernels) and Z = X or dY (M x C bf16).
// They are skinny (r <= 64 outputs per column) and HBM-bound on Z.  Each
// workgroup streams a 64-row slab of Z at a time with coalesced 16-byte
// loads, transposes it in registers into LDS so the row index m becomes the
// MFMA reduction index, and accumulates a 128-column x r block; the rows are
// split over several workgroups, whose partial sums land in a workspace and
// are added in a fixed order by a second small kernel (deterministic, no
// atomics), which also applies s and the accumulate flag.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileC = 128;

struct GradParams {
  const uint16_t* Z;   // M x C bf16
  const float* V;      // M x r float32
  int64_t M, C;
  int32_t r;
  int32_t splits;
  int64_t rows_per_split;  // multiple of 64
  float* P;            // splits x r x C partial sums
};

template <int RP>
__global__ __launch_bounds__(kThreads) void grad_kernel(GradParams p) {
  constexpr int JT = RP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t zt[2][kTileC * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][RP * kPitch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int c_tiles = (int)cdiv(p.C, kTileC);
  const int tile = xcd_tile(blockIdx.x, c_tiles * p.splits);
  const int tc = tile % c_tiles, split = tile / c_tiles;
  const int64_t c0 = (int64_t)tc * kTileC;
  const int64_t mbeg = (int64_t)split * p.rows_per_split;
  int64_t mend = mbeg + p.rows_per_split;
  mend = mend < p.M ? mend : p.M;
  const int steps = mend > mbeg ? (int)cdiv(mend - mbeg, 64) : 0;
  const int r = p.r;

  f32x16 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.0f;

  // staging: thread covers columns c0 + 8 (tid & 15) .. +7 of rows 4 (tid >> 4) .. +3
  const int cc = tid & 15, mg = tid >> 4;
  const int64_t ccol = c0 + 8 * cc;
  auto load = [&](int64_t m0r, uint32_t (&raw)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0r + 4 * mg + i;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (m < mend && ccol < p.C) v = *reinterpret_cast<const u32x4*>(p.Z + m * p.C + ccol);
#pragma unroll
      for (int d = 0; d < 4; ++d) raw[4 * i + d] = v[d];
    }
  };
  auto store = [&](const uint32_t (&raw)[16], uint16_t* dst) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x2 ev{pair_lo(raw[d], raw[4 + d]), pair_lo(raw[8 + d], raw[12 + d])};
      const u32x2 od{pair_hi(raw[d], raw[4 + d]), pair_hi(raw[8 + d], raw[12 + d])};
      *reinterpret_cast<u32x2*>(dst + (8 * cc + 2 * d) * kPitch + 4 * mg) = ev;
      *reinterpret_cast<u32x2*>(dst + (8 * cc + 2 * d + 1) * kPitch + 4 * mg) = od;
    }
  };
  // V^T tile: thread owns row m = tid % 64, columns j = tid / 64 + 4 i; the
  // values are loaded with the Z prefetch and stored after the MFMAs.
  const int vm = tid & 63, vj0 = tid >> 6;
  auto load_v = [&](int64_t m0r, float (&vv)[RP / 4]) {
    const bool ok = m0r + vm < mend;
    const float* row = p.V + (m0r + vm) * r;
#pragma unroll
    for (int i = 0; i < RP / 4; ++i) {
      const int j = vj0 + 4 * i;
      vv[i] = (ok && j < r) ? row[j] : 0.0f;
    }
  };
  auto store_v = [&](const float (&vv)[RP / 4], uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < RP / 4; ++i) dst[(vj0 + 4 * i) * kPitch + vm] = f32_to_bf16(vv[i]);
  };

  uint32_t raw[16];
  float vv[RP / 4];
  if (steps > 0) {
    load(mbeg, raw);
    load_v(mbeg, vv);
    store(raw, zt[0]);
    store_v(vv, vt[0]);
  }
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < steps;
    const int64_t m1 = mbeg + (int64_t)(st + 1) * 64;
    if (more) {
      load(m1, raw);
      load_v(m1, vv);
    }
    const uint16_t* z = zt[buf];
    const uint16_t* v = vt[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 zf =
          *reinterpret_cast<const u32x4*>(z + (32 * wave + l32) * kPitch + 32 * h + 8 * s);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 vf =
            *reinterpret_cast<const u32x4*>(v + (32 * jt + l32) * kPitch + 32 * h + 8 * s);
        acc[jt] = mfma32(zf, vf, acc[jt]);
      }
    }
    if (more) {
      store(raw, zt[buf ^ 1]);
      store_v(vv, vt[buf ^ 1]);
    }
    __syncthreads();
  }
  // acc[jt] lane l: rows c = c0 + 32 wave + 8q + 4h + i, column j = 32 jt + l32
  float* P = p.P + (int64_t)split * r * p.C;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 32 * jt + l32;
    if (j >= r) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t c = c0 + 32 * wave + 8 * q + 4 * h;
      if (c + 4 <= p.C) {
        *reinterpret_cast<f32x4*>(P + (int64_t)j * p.C + c) =
            f32x4{acc[jt][4 * q], acc[jt][4 * q + 1], acc[jt][4 * q + 2], acc[jt][4 * q + 3]};
      } else {
        for (int i = 0; i < 4; ++i)
          if (c + i < p.C) P[(int64_t)j * p.C + c + i] = acc[jt][4 * q + i];
      }
    }
  }
}

// out = s * sum_split P[split] (+ out if accumulate); layout jc: out[j][c]
// (dA, r x K) or cj: out[c][j] (dB, N x r).
__global__ void grad_reduce_kernel(const float* __restrict__ P, int splits, int r, int64_t C,
                                   float s, int accumulate, int transpose,
                                   float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)r * C;
  if (idx >= total) return;
  int64_t j, c;
  if (transpose) {  // idx runs over out[c][j]
    c = idx / r;
    j = idx - c * r;
  } else {
    j = idx / C;
    c = idx - j * C;
  }
  float sum = 0.0f;
  for (int t = 0; t < splits; ++t) sum += P[(int64_t)t * total + j * C + c];
  float v = s * sum;
  if (accumulate) v += out[idx];
  out[idx] = v;
}

int pick_splits(int64_t M, int64_t C) {
  const int64_t c_tiles = cdiv(C, kTileC);
  int64_t want = cdiv(512, c_tiles);
  const int64_t max_split = cdiv(M, 256);
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  return (int)want;
}

int run_grad(const uint16_t* Z, const float* V, int64_t M, int64_t C, int r, float s,
             int accumulate, int transpose, float* out, float* P, hipStream_t st) {
  const int splits = pick_splits(M, C);
  GradParams p;
  p.Z = Z;
  p.V = V;
  p.M = M;
  p.C = C;
  p.r = r;
  p.splits = splits;
  p.rows_per_split = cdiv(cdiv(M, splits), 64) * 64;
  p.P = P;
  const int blocks = (int)cdiv(C, kTileC) * splits;
  if (r <= 32)
    hipLaunchKernelGGL(grad_kernel<32>, dim3(blocks), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(grad_kernel<64>, dim3(blocks), dim3(kThreads), 0, st, p);
  int e = hip_fail(hipGetLastError(), "grad_kernel launch");
  if (e) return e;
  const int64_t total = (int64_t)r * C;
  hipLaunchKernelGGL(grad_reduce_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, st, P,
                     splits, r, C, s, accumulate, transpose, out);
  return hip_fail(hipGetLastError(), "grad_reduce launch");
}

}  // namespace

namespace dispatch {

int bf16_fwd(const void*, int64_t, const lq_weight&, const void*, const void*, int64_t, float,
             void*, float*, hipStream_t);
int bf16_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
            int64_t r, float s, void* dX, float* U_out, hipStream_t st);
int t_only(const void* X, int64_t M, int64_t K, const void* A, int64_t r, float* T,
           hipStream_t st);
int u_only(const void* dY, int64_t M, int64_t N, const void* B, int64_t r, float* U,
           hipStream_t st);

size_t grad_partial_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t sa = pick_splits(M, K), sb = pick_splits(M, N);
  return (size_t)(sa * r * K + sb * r * N) * 4 + 512;
}

int bf16_bwd(const void* dY, const void* X, int64_t M, const lq_weight& W, const void* A,
             const void* B, int64_t r, float s, const float* T_saved, void* dX, float* dA,
             float* dB, int accumulate, void* ws, hipStream_t st) {
  const int64_t N = W.N, K = W.K;
  float* U = (float*)ws;
  float* Tw = U + M * r;
  uintptr_t pa = ((uintptr_t)(Tw + M * r) + 255) & ~(uintptr_t)255;
  float* PA = (float*)pa;
  float* PB = PA + (int64_t)pick_splits(M, K) * r * K;
  int e;
  if (M == 0) {
    if (accumulate) return LQ_OK;
    if ((e = launch_zero_f32(dA, r * K, st))) return e;
    return launch_zero_f32(dB, N * r, st);
  }
  const float* T = T_saved;
  if (!T) {
    if ((e = t_only(X, M, K, A, r, Tw, st))) return e;
    T = Tw;
  }
  if (dX) {
    if ((e = bf16_dx(dY, M, W, A, B, r, s, dX, U, st))) return e;
  } else {
    if ((e = u_only(dY, M, N, B, r, U, st))) return e;
  }
  if ((e = run_grad((const uint16_t*)X, U, M, K, (int)r, s, accumulate, 0, dA, PA, st))) return e;
  return run_grad((const uint16_t*)dY, T, M, N, (int)r, s, accumulate, 1, dB, PB, st);
}

}  // namespace dispatch
}  // namespace lq

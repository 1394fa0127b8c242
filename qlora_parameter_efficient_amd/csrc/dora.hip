// DoRA on the adapted linear layer: W' = diag(m / c) (W0 + s B A) with
// c_n = ||W0[n] + s B[n] A||_2, one trained magnitude m_n per output row
// ("Large Language Model Fine-tuning and LoRA", section "Choosing what to
// adapt": a magnitude vector of size d_out and a low-rank update of the
// direction; "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations
// ...", section "Advanced Variants: DoRA and LoRA+": W = m (V + dW) / ||V +
// dW||, its norm read as the per-row vector norm).
//
// Forward: Y = Z * g (per output column), Z = X (W0 + s B A)^T the plain
// layer, g = m / c.  The row norms come from the expansion
//   c_n^2 = ||W0[n]||^2 + 2 s <(W0 A^T)[n], B[n]> + s^2 B[n] (A A^T) B[n]^T,
// whose pieces are a row sum of squares of the bf16 W0 the products use and
// two rank-r shrinks (W0 A^T and A A^T) run by the library's shrink kernels.
// Backward (exact chain rule through c): with G' = dY * g and
// h_n = sum_m dY[m][n] Z[m][n],
//   dm = h / c,  kappa = -h m / c^3,  dW = G'^T X + diag(kappa) (W0 + s B A)
//   dX = G' W,   dA = s B^T dW,   dB = s dW A^T;
// the G' terms are the plain backward with dY := G'; the kappa terms add
//   dA += s (kappa B)^T W0 + s^2 ((kappa B)^T B) A
//   dB += s kappa * (W0 A^T + s B (A A^T)).
#include <hip/hip_runtime.h>

#include "common.h"
#include "dispatch.h"

namespace lq {
namespace {

// sum_k W[n][k]^2 of a bf16 N x K matrix (K % 8 == 0): one wave per row.
__global__ __launch_bounds__(256) void rowsumsq_kernel(const uint16_t* __restrict__ W, int64_t N,
                                                       int64_t K, float* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  if (n >= N) return;
  const uint16_t* row = W + n * K;
  float acc = 0.0f;
  for (int64_t k = 8 * lane; k < K; k += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + k);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = lo_bf16(v[d]), b = hi_bf16(v[d]);
      acc += a * a + b * b;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) out[n] = acc;
}

// c_n and g_n = m_n / c_n from the expansion of ||W0[n] + s B[n] A||^2.
// RP lanes per row (RP = 16, 32 or 64 >= r, a power of two): lane i forms
// b_i (Gram b)_i and P0[n][i] b_i, and the row's lanes add them with
// shuffles.  Gram is staged in LDS.
template <int RP>
__global__ __launch_bounds__(256) void dora_norm_kernel(const float* __restrict__ w0sq,
                                                        const float* __restrict__ P0,
                                                        const float* __restrict__ Gram,
                                                        const uint16_t* __restrict__ B,
                                                        const float* __restrict__ m, int64_t N,
                                                        int r, float s, float* __restrict__ c,
                                                        float* __restrict__ g) {
  __shared__ float G[kMaxRankCols * kMaxRankCols];
  for (int i = threadIdx.x; i < r * r; i += 256) G[i] = Gram[i];
  __syncthreads();
  const int i = threadIdx.x % RP;
  const int64_t n = (int64_t)blockIdx.x * (256 / RP) + threadIdx.x / RP;
  const int64_t nn = n < N ? n : N - 1;
  const uint16_t* b = B + nn * r;
  float cross = 0.0f, quad = 0.0f;
  if (i < r) {
    const float bi = bf16_to_f32(b[i]);
    float gb = 0.0f;
    for (int j = 0; j < r; ++j) gb += G[i * r + j] * bf16_to_f32(b[j]);
    quad = bi * gb;
    cross = P0[nn * r + i] * bi;
  }
#pragma unroll
  for (int o = RP / 2; o >= 1; o >>= 1) {
    quad += __shfl_xor(quad, o);
    cross += __shfl_xor(cross, o);
  }
  if (i == 0 && n < N) {
    const float c2 = w0sq[n] + 2.0f * s * cross + s * s * quad;
    const float cn = sqrtf(fmaxf(c2, 0.0f));
    c[n] = cn;
    g[n] = m[n] / cn;
  }
}

// Partial Gram matrices A A^T over 256-column chunks of A (r x K, bf16): the
// chunk is staged in LDS, and each thread forms whole entries of the r x r
// partial.
constexpr int kGramCols = 256;

__global__ __launch_bounds__(256) void gram_part_kernel(const uint16_t* __restrict__ A, int r,
                                                        int64_t K, float* __restrict__ part) {
  __shared__ uint16_t As[kMaxRankCols][kGramCols + 2];
  const int64_t k0 = (int64_t)blockIdx.x * kGramCols;
  const int64_t cols = K - k0 < kGramCols ? K - k0 : kGramCols;
  for (int e = threadIdx.x; e < r * kGramCols; e += 256) {
    const int j = e / kGramCols, k = e % kGramCols;
    As[j][k] = k < cols ? A[(int64_t)j * K + k0 + k] : (uint16_t)0;
  }
  __syncthreads();
  float* out = part + (int64_t)blockIdx.x * r * r;
  for (int p = threadIdx.x; p < r * r; p += 256) {
    const int i = p / r, j = p - i * r;
    float acc = 0.0f;
    for (int k = 0; k < kGramCols; ++k) acc += bf16_to_f32(As[i][k]) * bf16_to_f32(As[j][k]);
    out[p] = acc;
  }
}

// g = m / c from saved row norms (the same division the norm kernel does).
__global__ __launch_bounds__(256) void dora_g_kernel(const float* __restrict__ m,
                                                     const float* __restrict__ c, int64_t N,
                                                     float* __restrict__ g) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n < N) g[n] = m[n] / c[n];
}

// Y[m][n] = bf16(Z[m][n] g[n]), 16-byte chunks (N % 8 == 0).
constexpr int kScaleChunks = 4;

__global__ __launch_bounds__(256) void col_scale_kernel(const uint16_t* __restrict__ Z,
                                                        const float* __restrict__ g, int64_t n8,
                                                        int64_t N, uint16_t* __restrict__ Y) {
  const int64_t c0 = (int64_t)blockIdx.x * 256 * kScaleChunks + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kScaleChunks; ++u) {
    const int64_t c = c0 + (int64_t)u * 256;
    if (c >= n8) return;
    const int64_t e = 8 * c;
    const int64_t n = e % N;
    const u32x4 z = *reinterpret_cast<const u32x4*>(Z + e);
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(g + n);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + n + 4);
    *reinterpret_cast<u32x4*>(Y + e) =
        u32x4{pack_bf16x2(lo_bf16(z[0]) * g0[0], hi_bf16(z[0]) * g0[1]),
              pack_bf16x2(lo_bf16(z[1]) * g0[2], hi_bf16(z[1]) * g0[3]),
              pack_bf16x2(lo_bf16(z[2]) * g1[0], hi_bf16(z[2]) * g1[1]),
              pack_bf16x2(lo_bf16(z[3]) * g1[2], hi_bf16(z[3]) * g1[3])};
  }
}

// G'[m][n] = bf16(dY[m][n] g[n]) and the partial column sums
// hpart[t][n] = sum over the 16 rows of tile t of dY[m][n] Z[m][n].
// A workgroup covers 2048 columns (8 per thread) of one 16-row tile.
constexpr int kHRows = 16, kHCols = 2048;

__global__ __launch_bounds__(256) void dora_gprep_kernel(const uint16_t* __restrict__ dY,
                                                         const uint16_t* __restrict__ Z,
                                                         const float* __restrict__ g, int64_t M,
                                                         int64_t N, int col_groups,
                                                         uint16_t* __restrict__ Gp,
                                                         float* __restrict__ hpart) {
  const int64_t t = blockIdx.x / col_groups;
  const int64_t n = (int64_t)(blockIdx.x % col_groups) * kHCols + 8 * threadIdx.x;
  if (n >= N) return;
  float gg[8], h[8];
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(g + n);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + n + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gg[e] = g0[e];
    gg[4 + e] = g1[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = 0.0f;
  const int64_t m0 = t * kHRows;
  const int64_t m1 = m0 + kHRows < M ? m0 + kHRows : M;
  for (int64_t mb = m0; mb < m1; mb += 4) {
    u32x4 a[4], z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb + i < m1 ? mb + i : m1 - 1;
      a[i] = *reinterpret_cast<const u32x4*>(dY + m * N + n);
      z[i] = *reinterpret_cast<const u32x4*>(Z + m * N + n);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (mb + i >= m1) break;
      float o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float a0 = lo_bf16(a[i][d]), a1 = hi_bf16(a[i][d]);
        h[2 * d] += a0 * lo_bf16(z[i][d]);
        h[2 * d + 1] += a1 * hi_bf16(z[i][d]);
        o[2 * d] = a0 * gg[2 * d];
        o[2 * d + 1] = a1 * gg[2 * d + 1];
      }
      *reinterpret_cast<u32x4*>(Gp + (mb + i) * N + n) =
          u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                pack_bf16x2(o[6], o[7])};
    }
  }
  float* hp = hpart + t * N + n;
  *reinterpret_cast<f32x4*>(hp) = f32x4{h[0], h[1], h[2], h[3]};
  *reinterpret_cast<f32x4*>(hp + 4) = f32x4{h[4], h[5], h[6], h[7]};
}

// h_n from the tile partials, dm = h / c, kappa = -h g / c^2,
// KB[n][j] = kappa_n B[n][j].  A workgroup owns 64 columns; its four thread
// groups add every fourth tile, then the four sums are added in a fixed order.
__global__ __launch_bounds__(256) void dora_hfin_kernel(const float* __restrict__ hpart,
                                                        int tiles, int64_t N,
                                                        const float* __restrict__ c,
                                                        const float* __restrict__ g,
                                                        const uint16_t* __restrict__ B, int r,
                                                        float* __restrict__ dm, int accumulate,
                                                        float* __restrict__ kappa,
                                                        float* __restrict__ KB) {
  __shared__ float part[4][64];
  __shared__ float ks[64];
  const int q = threadIdx.x >> 6, col = threadIdx.x & 63;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t n = n0 + col;
  float h0 = 0.0f, h1 = 0.0f, h2 = 0.0f, h3 = 0.0f;
  if (n < N) {
    int t = q;
    for (; t + 12 < tiles; t += 16) {  // four independent chains of loads
      h0 += hpart[(int64_t)t * N + n];
      h1 += hpart[(int64_t)(t + 4) * N + n];
      h2 += hpart[(int64_t)(t + 8) * N + n];
      h3 += hpart[(int64_t)(t + 12) * N + n];
    }
    for (; t < tiles; t += 4) h0 += hpart[(int64_t)t * N + n];
  }
  part[q][col] = (h0 + h1) + (h2 + h3);
  __syncthreads();
  if (q == 0) {
    float k = 0.0f;
    if (n < N) {
      const float hs = ((part[0][col] + part[1][col]) + part[2][col]) + part[3][col];
      const float cn = c[n];
      const float d = hs / cn;
      dm[n] = accumulate ? dm[n] + d : d;
      k = -hs * g[n] / (cn * cn);
      kappa[n] = k;
    }
    ks[col] = k;
  }
  __syncthreads();
  // KB for the workgroup's 64 rows: 64 r consecutive floats
  const int64_t rows = N - n0 < 64 ? N - n0 : 64;
  for (int64_t i = threadIdx.x; i < rows * r; i += 256)
    KB[n0 * r + i] = ks[i / r] * bf16_to_f32(B[n0 * r + i]);
}

// R[j][i] = sum_n KB[n][j] B[n][i] in two steps: each workgroup stages 64
// rows of KB and B in LDS and writes the partial r x r sum of its rows; a
// second kernel adds the partials in block order.
constexpr int kRRows = 64;

__global__ __launch_bounds__(256) void dora_rpart_kernel(const float* __restrict__ KB,
                                                         const uint16_t* __restrict__ B,
                                                         int64_t N, int r,
                                                         float* __restrict__ Rpart) {
  __shared__ float Ks[kRRows][kMaxRankCols + 1];
  __shared__ float Bs[kRRows][kMaxRankCols + 1];
  const int64_t n0 = (int64_t)blockIdx.x * kRRows;
  const int64_t rows = N - n0 < kRRows ? N - n0 : kRRows;
  for (int i = threadIdx.x; i < kRRows * r; i += 256) {
    const bool ok = i / r < rows;
    Ks[i / r][i % r] = ok ? KB[n0 * r + i] : 0.0f;
    Bs[i / r][i % r] = ok ? bf16_to_f32(B[n0 * r + i]) : 0.0f;
  }
  __syncthreads();
  float* out = Rpart + (int64_t)blockIdx.x * r * r;
  for (int p = threadIdx.x; p < r * r; p += 256) {
    const int j = p / r, i = p - j * r;
    float acc = 0.0f;
    for (int k = 0; k < kRRows; ++k) acc += Ks[k][j] * Bs[k][i];
    out[p] = acc;
  }
}

// Sums blocks partial r x r matrices in a fixed order (also the Gram partials).
__global__ __launch_bounds__(256) void dora_rsum_kernel(const float* __restrict__ Rpart,
                                                        int blocks, int r,
                                                        float* __restrict__ R) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= r * r) return;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  const int64_t rr = (int64_t)r * r;
  int b = 0;
  for (; b + 3 < blocks; b += 4) {  // four independent chains of loads
    a0 += Rpart[b * rr + p];
    a1 += Rpart[(b + 1) * rr + p];
    a2 += Rpart[(b + 2) * rr + p];
    a3 += Rpart[(b + 3) * rr + p];
  }
  for (; b < blocks; ++b) a0 += Rpart[b * rr + p];
  R[p] = (a0 + a1) + (a2 + a3);
}

// The remaining kappa terms: index space r K (dA) then N r (dB).
//   dA[j][k] += s^2 sum_i R[j][i] A[i][k]
//   dB[n][j] += s kappa_n (P0[n][j] + s sum_i B[n][i] Gram[i][j])
__global__ __launch_bounds__(256) void dora_fix_kernel(float* __restrict__ dA,
                                                       float* __restrict__ dB,
                                                       const float* __restrict__ R,
                                                       const uint16_t* __restrict__ A,
                                                       const float* __restrict__ kappa,
                                                       const float* __restrict__ P0,
                                                       const uint16_t* __restrict__ B,
                                                       const float* __restrict__ Gram, int64_t N,
                                                       int64_t K, int r, float s) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t na = (int64_t)r * K;
  if (idx < na) {
    const int64_t j = idx / K, k = idx - j * K;
    float v = 0.0f;
    for (int i = 0; i < r; ++i) v += R[j * r + i] * bf16_to_f32(A[(int64_t)i * K + k]);
    dA[idx] += s * s * v;
    return;
  }
  const int64_t i2 = idx - na;
  if (i2 >= N * r) return;
  const int64_t n = i2 / r;
  const int j = (int)(i2 - n * r);
  float v = 0.0f;
  for (int i = 0; i < r; ++i) v += bf16_to_f32(B[n * r + i]) * Gram[i * r + j];
  dB[i2] += s * kappa[n] * (P0[i2] + s * v);
}

}  // namespace

namespace dispatch {

int dora_weight_side(const void* Wd, int64_t N, int64_t K, const void* A, const void* B,
                     int64_t r, float s, const float* m, const DoraSide& d, hipStream_t st) {
  int e;
  hipLaunchKernelGGL(rowsumsq_kernel, dim3((unsigned)cdiv(N, 4)), dim3(256), 0, st,
                     (const uint16_t*)Wd, N, K, d.w0sq);
  if ((e = hip_fail(hipGetLastError(), "rowsumsq launch"))) return e;
  if ((e = t_only(Wd, N, K, A, r, d.P0, st, nullptr, 0))) return e;      // W0 A^T
  const int gblocks = dora_gblocks(K);  // A A^T: chunk partials, then their sum
  hipLaunchKernelGGL(gram_part_kernel, dim3((unsigned)gblocks), dim3(256), 0, st,
                     (const uint16_t*)A, (int)r, K, d.Gpart);
  if ((e = hip_fail(hipGetLastError(), "gram_part launch"))) return e;
  hipLaunchKernelGGL(dora_rsum_kernel, dim3((unsigned)cdiv(r * r, 256)), dim3(256), 0, st,
                     d.Gpart, gblocks, (int)r, d.Gram);
  if ((e = hip_fail(hipGetLastError(), "gram sum launch"))) return e;
  const unsigned nb16 = (unsigned)cdiv(N, 16), nb8 = (unsigned)cdiv(N, 8),
                 nb4 = (unsigned)cdiv(N, 4);
  const uint16_t* Bh = (const uint16_t*)B;
  if (r <= 16)
    hipLaunchKernelGGL(dora_norm_kernel<16>, dim3(nb16), dim3(256), 0, st, d.w0sq, d.P0, d.Gram,
                       Bh, m, N, (int)r, s, d.c, d.g);
  else if (r <= 32)
    hipLaunchKernelGGL(dora_norm_kernel<32>, dim3(nb8), dim3(256), 0, st, d.w0sq, d.P0, d.Gram,
                       Bh, m, N, (int)r, s, d.c, d.g);
  else
    hipLaunchKernelGGL(dora_norm_kernel<64>, dim3(nb4), dim3(256), 0, st, d.w0sq, d.P0, d.Gram,
                       Bh, m, N, (int)r, s, d.c, d.g);
  return hip_fail(hipGetLastError(), "dora_norm launch");
}

int dora_g_from_c(const float* m, const DoraSide& d, int64_t N, hipStream_t st) {
  hipLaunchKernelGGL(dora_g_kernel, dim3((unsigned)cdiv(N, 256)), dim3(256), 0, st, m, d.c, N,
                     d.g);
  return hip_fail(hipGetLastError(), "dora_g launch");
}

int launch_col_scale(const void* Z, const float* g, int64_t M, int64_t N, void* Y,
                     hipStream_t st) {
  const int64_t n8 = M * N / 8;
  if (n8 == 0) return LQ_OK;
  hipLaunchKernelGGL(col_scale_kernel, dim3((unsigned)cdiv(n8, 256 * kScaleChunks)), dim3(256), 0,
                     st, (const uint16_t*)Z, g, n8, N, (uint16_t*)Y);
  return hip_fail(hipGetLastError(), "col_scale launch");
}

int dora_tiles(int64_t M) { return (int)cdiv(M, kHRows); }

int dora_rblocks(int64_t N) { return (int)cdiv(N, kRRows); }

int dora_gblocks(int64_t K) { return (int)cdiv(K, kGramCols); }

int dora_grad_side(const void* dY, const void* Z, const float* m, const void* B, int64_t M,
                   int64_t N, int64_t r, const DoraSide& d, const DoraGrad& q, float* dm,
                   int accumulate, hipStream_t st) {
  (void)m;
  const int col_groups = (int)cdiv(N, kHCols);
  const int tiles = dora_tiles(M);
  int e;
  hipLaunchKernelGGL(dora_gprep_kernel, dim3((unsigned)(tiles * col_groups)), dim3(256), 0, st,
                     (const uint16_t*)dY, (const uint16_t*)Z, d.g, M, N, col_groups, q.Gp,
                     q.hpart);
  if ((e = hip_fail(hipGetLastError(), "dora_gprep launch"))) return e;
  hipLaunchKernelGGL(dora_hfin_kernel, dim3((unsigned)cdiv(N, 64)), dim3(256), 0, st, q.hpart,
                     tiles, N, d.c, d.g, (const uint16_t*)B, (int)r, dm, accumulate, q.kappa, q.KB);
  return hip_fail(hipGetLastError(), "dora_hfin launch");
}

int dora_fix(const void* Wd, const void* A, const void* B, int64_t N, int64_t K, int64_t r,
             float s, const DoraSide& d, const DoraGrad& q, float* dA, float* dB, hipStream_t st) {
  int e;
  const int rblocks = dora_rblocks(N);
  hipLaunchKernelGGL(dora_rpart_kernel, dim3((unsigned)rblocks), dim3(256), 0, st, q.KB,
                     (const uint16_t*)B, N, (int)r, q.Rpart);
  if ((e = hip_fail(hipGetLastError(), "dora_rpart launch"))) return e;
  hipLaunchKernelGGL(dora_rsum_kernel, dim3((unsigned)cdiv(r * r, 256)), dim3(256), 0, st,
                     q.Rpart, rblocks, (int)r, q.R);
  if ((e = hip_fail(hipGetLastError(), "dora_rsum launch"))) return e;
  // dA += s (kappa B)^T W0: the gradient reduction over the N rows of W0
  if ((e = grad_one(Wd, q.KB, N, K, (int)r, s, dA, q.part, st))) return e;
  const int64_t total = r * K + N * r;
  hipLaunchKernelGGL(dora_fix_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, st, dA, dB,
                     q.R, (const uint16_t*)A, q.kappa, d.P0, (const uint16_t*)B, d.Gram, N, K,
                     (int)r, s);
  return hip_fail(hipGetLastError(), "dora_fix launch");
}

}  // namespace dispatch
}  // namespace lq

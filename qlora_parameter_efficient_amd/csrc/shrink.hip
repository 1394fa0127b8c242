// Skinny rank-r products of the adapted linear layer, float32 results:
//   T = X A^T   (forward, M x r; kept for the backward)
//   U = dY B    (backward, M x r; feeds dX and dA)
// ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ...": the
// forward-pass equation applies A to x first; section "Gradient Dynamics and
// Backpropagation Mechanics": dY B appears in both dL/dA and dL/dx.)
//
// Both read their M x K activation operand once and are bound by that stream.
// A workgroup owns 16 rows; its waves (8 in the standalone kernel, 4 in the
// prep kernel that also writes the bf16 weight copy) split the reduction into
// contiguous ranges of 32-wide units and add their partial sums through LDS in
// a fixed order at the end.  Each unit is one v_mfma_f32_16x16x32_bf16
// per 16 rank columns, the activation rows as the A operand (lane (g, l16):
// row l16, 16 bytes at reduction 8 g, loaded straight from global memory) and
// the rank-side matrix as the B operand:
//   * G = A (r x K, reduction contiguous): lane (g, l16) loads row l16 of A
//     (clamped to r - 1; those result columns are never stored);
//   * G = B^T (B is K x r, rank contiguous): the 32 R rows of B that a round
//     of R units needs are one contiguous block of memory, loaded with
//     16-byte loads, stored to a per-wave LDS tile in storage order and read
//     back with the transposing ds_read_b64_tr_b16 (inside each 16-lane group
//     lane c addresses row c / 4, columns 4 (c % 4) .. +3; lane i receives
//     column i of the four rows).  8-byte aligned reads need r % 4 == 0.
// The loads of the next round are issued before the products of the current
// one; reduction units past the wave's range (clamped loads) are masked to
// zero.
#include "device_util.h"
#include "dispatch.h"
#include "nf4_deq.h"

namespace lq {
namespace {

constexpr int kSW = 8;  // waves per workgroup of the standalone kernel
constexpr int kSThreads = 64 * kSW;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 tr_read(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 16 rows (rb * 16 ..) of out with NW waves; every thread of the workgroup
// (64 NW of them) calls it.
// row_ad (optional, multi-adapter): result column j of row m is kept, times
// the adapter's scale, only inside the columns of the row's adapter row_ad[m]
// (mt), else written as 0.
template <int JT, bool GT, int NW>
__device__ __forceinline__ void shrink_rows(int64_t rb, const uint16_t* __restrict__ Z, int64_t M,
                                            int64_t K, const uint16_t* __restrict__ G, int r,
                                            float* __restrict__ out,
                                            const int32_t* __restrict__ row_ad,
                                            const MultiTab& mt) {
  constexpr int RC = 16 * JT;    // rank columns, padded
  constexpr int R = 8 / JT;      // units per round
  constexpr int NB = R * JT;     // GT: 1 KB pieces of B per round (32 R rows of up to RC)
  __shared__ __attribute__((aligned(16))) uint16_t gtile[GT ? NW : 1][GT ? NB * 512 : 8];
  __shared__ f32x4 red[NW][JT][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;

  const int64_t m0 = rb * 16;
  int64_t mr = m0 + l16;
  mr = mr < M ? mr : M - 1;
  const int64_t UT = K >> 5;
  const int64_t u0 = UT * wave / NW, u1 = UT * (wave + 1) / NW;
  const uint16_t* zrow = Z + mr * K + 8 * g;
  const uint16_t* arow[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    int j = 16 * jt + l16;
    j = j < r ? j : r - 1;
    arow[jt] = G + (int64_t)j * K + 8 * g;
  }
  const int64_t gbytes = K * r * 2;  // GT: bytes of B
  const char* gb = reinterpret_cast<const char*>(G);

  struct Round {
    u32x4 z[R];
    u32x4 a[GT ? 1 : R][JT];
    u32x4 b[GT ? NB : 1];
  };
  auto load = [&](Round& d, int64_t u) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      int64_t uq = u + q;
      uq = uq < u1 ? uq : u1 - 1;
      d.z[q] = *reinterpret_cast<const u32x4*>(zrow + 32 * uq);
      if (!GT)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
          d.a[q][jt] = *reinterpret_cast<const u32x4*>(arow[jt] + 32 * uq);
    }
    if (GT) {
      const int64_t base = u * 32 * r * 2;
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        int64_t off = base + 1024 * t + 16 * lane;
        off = off <= gbytes - 16 ? off : gbytes - 16;
        d.b[t] = *reinterpret_cast<const u32x4*>(gb + off);
      }
    }
  };

  f32x4 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const Round& d, int64_t u) {
    uint16_t* tl = gtile[GT ? wave : 0];
    if (GT) {
      // the wave's own tile; its LDS operations run in order, so these stores
      // land before the reads below and after the previous round's reads
#pragma unroll
      for (int t = 0; t < NB; ++t) *reinterpret_cast<u32x4*>(tl + 512 * t + 8 * lane) = d.b[t];
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const u32x4 zq = sel4(u + q < u1, d.z[q]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        u32x4 gf;
        if (GT) {
          const uint16_t* p = tl + (32 * q + 8 * g + (l16 >> 2)) * r + 16 * jt + 4 * (l16 & 3);
          const u32x2 lo = tr_read(p), hi = tr_read(p + 4 * r);
          gf = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          gf = d.a[q][jt];
        }
        acc[jt] = mfma16(zq, gf, acc[jt]);
      }
    }
  };

  if (u0 < u1) {
    Round d0, d1;
    load(d0, u0);
    for (int64_t u = u0; u < u1; u += 2 * R) {
      if (u + R < u1) load(d1, u + R);
      compute(d0, u);
      if (u + R < u1) {
        if (u + 2 * R < u1) load(d0, u + 2 * R);
        compute(d1, u + R);
      }
    }
  }

#pragma unroll
  for (int jt = 0; jt < JT; ++jt) red[wave][jt][lane] = acc[jt];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      f32x4 s = red[0][jt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w][jt][lane];
      const int j = 16 * jt + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * g + i;
        if (m < M && j < r) {
          float v = s[i];
          if (row_ad) {
            int a = row_ad[m];  // clamped: ids are in range by precondition
            a = a < 0 ? 0 : (a >= mt.n_ad ? mt.n_ad - 1 : a);
            v = (j >= mt.roff[a] && j < mt.roff[a + 1]) ? v * mt.scale[a] : 0.0f;
          }
          out[m * r + j] = v * mt.oscale;
        }
      }
    }
  }
}

template <int JT, bool GT>
__global__ __launch_bounds__(kSThreads) void shrink_kernel(const uint16_t* __restrict__ Z,
                                                           int64_t M, int64_t K,
                                                           const uint16_t* __restrict__ G,
                                                           int r, float* __restrict__ out,
                                                           int32_t* __restrict__ zero, int nzero,
                                                           const int32_t* __restrict__ row_ad,
                                                           MultiTab mt) {
  // side job: clear the next kernel's flag words (a kernel store, so it also
  // replays correctly inside a captured graph)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += kSThreads) zero[i] = 0;
  shrink_rows<JT, GT, kSW>(blockIdx.x, Z, M, K, G, r, out, row_ad, mt);
}

// Prep of the large-M path in one launch: workgroups below nd write the bf16
// copy of the NF4 weight (32768 elements each), the others compute 16 rows of
// T or U with four waves; the two HBM streams overlap.
struct PrepArgs {
  const uint8_t* codes;
  const uint8_t* q8;
  const float* c2;
  const float* absmax;
  int32_t dq;
  int32_t nd;  // dequantising workgroups
  int64_t n;   // weight elements
  uint16_t* wout;
  NF4Table tab;
};

template <int JT, bool GT>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs pa, const uint16_t* __restrict__ Z,
                                                   int64_t M, int64_t K,
                                                   const uint16_t* __restrict__ G, int r,
                                                   float* __restrict__ out,
                                                   int32_t* __restrict__ zero, int nzero,
                                                   const int32_t* __restrict__ row_ad,
                                                   MultiTab mt) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0;
  if ((int)blockIdx.x < pa.nd)
    nf4_deq_span<true>(threadIdx.x, blockIdx.x, pa.codes, pa.q8, pa.c2, pa.absmax, pa.dq, pa.n,
                       pa.wout, pa.tab);
  else
    shrink_rows<JT, GT, 4>((int64_t)blockIdx.x - pa.nd, Z, M, K, G, r, out, row_ad, mt);
}

// Wide shrink (out = Z G^T with G = A, 16 < r <= 64) for many rows: a
// workgroup of four waves owns 128 rows and all RC = 32 JC rank columns.  Per
// 64-wide reduction step the rank tile (RC rows of 128 bytes) is staged in LDS
// once and shared by the four waves -- the rows-per-workgroup of the kernel
// above would re-read all of A for every 16 rows.  Each wave loads its 32
// activation rows straight into MFMA registers: lane (h, l32) takes row l32
// and the 64 contiguous bytes 64 h .. of the step, so substep s of
// v_mfma_f32_32x32x16_bf16 reduces elements 32 h + 8 s .. + 7 on both operands
// (the rank tile is read with the same relabelling).  Rank-tile chunk c of
// row j sits at chunk c ^ (j & 7) in LDS, so the 32 lanes of one read hit
// distinct bank groups.  The next step's tiles are loaded into registers
// before the current step's products.
constexpr int kWRows = 128;

template <int JC>
__global__ __launch_bounds__(256) void shrink_wide_kernel(const uint16_t* __restrict__ Z,
                                                          int64_t M, int64_t K,
                                                          const uint16_t* __restrict__ G, int r,
                                                          float* __restrict__ out,
                                                          int32_t* __restrict__ zero, int nzero,
                                                          const int32_t* __restrict__ row_ad,
                                                          MultiTab mt) {
  constexpr int RC = 32 * JC;
  constexpr int GL = RC * 8 / 256;  // 16-byte rank-tile loads per thread per step
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][RC * 64];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.x * kWRows + 32 * wave;
  const int64_t mz = m0 + l32 < M ? m0 + l32 : M - 1;
  const uint16_t* zrow = Z + mz * K + 32 * h;
  // rank-tile loads: piece e = tid + 256 i -> row e / 8 (clamped to r - 1), chunk e % 8
  const uint16_t* grow[GL];
  uint32_t gst[GL];
#pragma unroll
  for (int i = 0; i < GL; ++i) {
    const int e = tid + 256 * i, row = e >> 3, ch = e & 7;
    grow[i] = G + (int64_t)(row < r ? row : r - 1) * K + 8 * ch;
    gst[i] = (uint32_t)(row * 64 + 8 * (ch ^ (row & 7)));
  }
  f32x16 acc[JC];
#pragma unroll
  for (int jc = 0; jc < JC; ++jc)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jc][v] = 0.0f;
  const int64_t steps = K / 64;
  u32x4 zc[4], zn[4], gc[GL];
  auto zload = [&](int64_t kt, u32x4 (&z)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) z[s] = *reinterpret_cast<const u32x4*>(zrow + kt * 64 + 8 * s);
  };
  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < GL; ++i) gc[i] = *reinterpret_cast<const u32x4*>(grow[i] + kt * 64);
  };
  auto gstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < GL; ++i) *reinterpret_cast<u32x4*>(&gt[b][gst[i]]) = gc[i];
  };
  zload(0, zc);
  gload(0);
  gstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < steps; ++kt) {
    const int b = (int)(kt & 1);
    const bool more = kt + 1 < steps;
    if (more) {
      zload(kt + 1, zn);
      gload(kt + 1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int jc = 0; jc < JC; ++jc) {
        const int j = 32 * jc + l32;
        const u32x4 gf = *reinterpret_cast<const u32x4*>(&gt[b][j * 64 + 8 * ((4 * h + s) ^ (j & 7))]);
        acc[jc] = mfma32(zc[s], gf, acc[jc]);
      }
    }
    if (more) {
      gstore(b ^ 1);  // the other buffer: its last reads were the previous step's
#pragma unroll
      for (int s = 0; s < 4; ++s) zc[s] = zn[s];
    }
    __syncthreads();
  }
  // acc[jc] lane l: rows m0 + 8 (v / 4) + 4 h + v % 4, column 32 jc + l32
#pragma unroll
  for (int jc = 0; jc < JC; ++jc) {
    const int j = 32 * jc + l32;
    if (j >= r) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = m0 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (m >= M) continue;
      float val = acc[jc][v];
      if (row_ad) {
        int a = row_ad[m];  // clamped: ids are in range by precondition
        a = a < 0 ? 0 : (a >= mt.n_ad ? mt.n_ad - 1 : a);
        val = (j >= mt.roff[a] && j < mt.roff[a + 1]) ? val * mt.scale[a] : 0.0f;
      }
      out[m * r + j] = val * mt.oscale;
    }
  }
}

bool wide_ok(bool gt, int64_t M, int64_t r) { return !gt && r > 16 && M >= kWRows; }

int launch_wide(const uint16_t* Z, int64_t M, int64_t K, const uint16_t* G, int64_t r, float* out,
                int32_t* zero, int nzero, const int32_t* row_ad, const MultiTab& mt,
                hipStream_t st) {
  const dim3 grid((unsigned)cdiv(M, kWRows)), block(256);
  if (r <= 32)
    hipLaunchKernelGGL((shrink_wide_kernel<1>), grid, block, 0, st, Z, M, K, G, (int)r, out, zero,
                       nzero, row_ad, mt);
  else
    hipLaunchKernelGGL((shrink_wide_kernel<2>), grid, block, 0, st, Z, M, K, G, (int)r, out, zero,
                       nzero, row_ad, mt);
  return hip_fail(hipGetLastError(), "shrink_wide launch");
}

template <bool GT>
int launch(const uint16_t* Z, int64_t M, int64_t K, const uint16_t* G, int64_t r, float* out,
           int32_t* zero, int nzero, const int32_t* row_ad, const MultiTab& mt, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(M, 16)), block(kSThreads);
  switch ((r + 15) / 16) {
    case 1:
      hipLaunchKernelGGL((shrink_kernel<1, GT>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero, row_ad, mt);
      break;
    case 2:
      hipLaunchKernelGGL((shrink_kernel<2, GT>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero, row_ad, mt);
      break;
    default:
      hipLaunchKernelGGL((shrink_kernel<4, GT>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero, row_ad, mt);
      break;
  }
  return hip_fail(hipGetLastError(), "shrink launch");
}

}  // namespace

namespace dispatch {

bool shrink_eligible(bool gt, int64_t r) { return !gt || r % 4 == 0; }

int launch_shrink(const void* Z, int64_t M, int64_t K, const void* G, bool gt, int64_t r,
                  float* out, int32_t* zero, int nzero, hipStream_t st, const int32_t* row_ad,
                  const MultiTab* mt) {
  const MultiTab none{};
  const MultiTab& t = mt ? *mt : none;
  if (wide_ok(gt, M, r))
    return launch_wide((const uint16_t*)Z, M, K, (const uint16_t*)G, r, out, zero, nzero, row_ad,
                       t, st);
  if (gt)
    return launch<true>((const uint16_t*)Z, M, K, (const uint16_t*)G, r, out, zero, nzero, row_ad,
                        t, st);
  return launch<false>((const uint16_t*)Z, M, K, (const uint16_t*)G, r, out, zero, nzero, row_ad,
                       t, st);
}

int launch_prep(const lq_weight& W, void* wout, const void* Z, int64_t M, int64_t K, const void* G,
                bool gt, int64_t r, float* out, int32_t* zero, int nzero, hipStream_t st,
                const int32_t* row_ad, const MultiTab* mt) {
  const MultiTab none{};
  const MultiTab& mtab = mt ? *mt : none;
  PrepArgs pa;
  pa.codes = W.codes;
  pa.q8 = W.q8;
  pa.c2 = W.c2;
  pa.absmax = W.absmax;
  pa.dq = W.double_quant;
  pa.n = W.N * W.K;
  pa.nd = (int32_t)cdiv(pa.n, kDeqSpan);
  pa.wout = (uint16_t*)wout;
  pa.tab = nf4_table(W.codebook);
  if (wide_ok(gt, M, r)) {
    // wide rank: the prep launch only dequantises (and clears the flags); the
    // shrink runs as the wide kernel, which shares the rank tile across 128 rows
    hipLaunchKernelGGL((prep_kernel<1, false>), dim3((unsigned)pa.nd), dim3(256), 0, st, pa,
                       (const uint16_t*)Z, (int64_t)0, K, (const uint16_t*)G, (int)r, out, zero,
                       nzero, row_ad, mtab);
    int e = hip_fail(hipGetLastError(), "prep launch");
    if (e) return e;
    return launch_wide((const uint16_t*)Z, M, K, (const uint16_t*)G, r, out, nullptr, 0, row_ad,
                       mtab, st);
  }
  const dim3 grid((unsigned)(pa.nd + cdiv(M, 16))), block(256);
  const uint16_t* Zh = (const uint16_t*)Z;
  const uint16_t* Gh = (const uint16_t*)G;
  switch ((r + 15) / 16) {
    case 1:
      if (gt)
        hipLaunchKernelGGL((prep_kernel<1, true>), grid, block, 0, st, pa, Zh, M, K, Gh, (int)r,
                           out, zero, nzero, row_ad, mtab);
      else
        hipLaunchKernelGGL((prep_kernel<1, false>), grid, block, 0, st, pa, Zh, M, K, Gh, (int)r,
                           out, zero, nzero, row_ad, mtab);
      break;
    case 2:
      if (gt)
        hipLaunchKernelGGL((prep_kernel<2, true>), grid, block, 0, st, pa, Zh, M, K, Gh, (int)r,
                           out, zero, nzero, row_ad, mtab);
      else
        hipLaunchKernelGGL((prep_kernel<2, false>), grid, block, 0, st, pa, Zh, M, K, Gh, (int)r,
                           out, zero, nzero, row_ad, mtab);
      break;
    default:
      if (gt)
        hipLaunchKernelGGL((prep_kernel<4, true>), grid, block, 0, st, pa, Zh, M, K, Gh, (int)r,
                           out, zero, nzero, row_ad, mtab);
      else
        hipLaunchKernelGGL((prep_kernel<4, false>), grid, block, 0, st, pa, Zh, M, K, Gh, (int)r,
                           out, zero, nzero, row_ad, mtab);
      break;
  }
  return hip_fail(hipGetLastError(), "prep launch");
}

}  // namespace dispatch
}  // namespace lq

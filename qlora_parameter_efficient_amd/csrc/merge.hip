// Deployment merge W_final = deq(W0) + s B A, written as a dense bf16 N x K
// matrix ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations
// ...", section "1. Static Weight Merging"; "Large Language Model Fine-tuning
// and LoRA", section "Merging adapters vs keeping them separate": a one-time
// product of 2 d_out r d_in FLOPs, the result keeping W0's shape).
//
// HBM-bound: the kernel reads W0 (NF4 or bf16) and writes the merged matrix
// once.  A workgroup owns a 128 x 256 block: it stages A's rows for the
// block's 256 columns (storage order in LDS) and B's rows for its 128 rows
// once, then walks four 32-row slices.  Every thread owns four 16-byte output
// chunks of a slice (8 consecutive elements of one row; chunk t + 256 i, so
// consecutive lanes write consecutive bytes); it issues the loads of the codes
// and block constants of all its chunks of all slices up front (bf16 weights:
// one slice ahead).  Per slice the four waves form the low-rank term
// s (B A)^T on MFMA -- A's columns read with the transposing LDS read as the A
// operand, B's rows as the B operand, r the reduction -- into an LDS float32
// tile; then each thread dequantises its chunks (to the same
// bf16 values the fused GEMM multiplies by), adds the low-rank term in
// float32 and stores the bf16 result.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;
constexpr int kTN = 32, kTK = 256;     // slice: 32 rows x 256 columns
constexpr int kSlices = 4;             // slices per workgroup (128 rows)
constexpr int kSPitch = kTK + 4;       // float32 S tile pitch
constexpr int kAPitch = kTK + 32;      // bf16 A tile pitch: rows 64 bytes apart modulo 256
constexpr int kMergeTab = 520;         // second-level steps of 128 rows (K <= 65536)

struct MergeParams {
  WeightArgs W;
  const uint16_t* A;  // r x K
  const uint16_t* B;  // N x r
  int32_t r;
  float s;
  int32_t k_tiles;
  int32_t n_blocks;
  uint16_t* out;      // N x K
  NF4Table tab;
};

typedef short s16x4m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr_m(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4m* lds_ptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p)));
}

template <int WK>
struct MergeStage {
  u32x4 wd[WK == kDense ? 4 : 1];
  uint32_t wc[4], q8[4];
};

template <int WK, int RP>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  __shared__ __attribute__((aligned(16))) float S[kTN * kSPitch];
  __shared__ __attribute__((aligned(16))) uint16_t At[RP * kAPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[kSlices * kTN * RP];
  __shared__ float2 lut[256];
  __shared__ float stab[WK == kNF4DQ ? kMergeTab : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t N = p.W.N, K = p.W.K;
  const int tk = blockIdx.x % p.k_tiles, tb = blockIdx.x / p.k_tiles;
  const int64_t nb = (int64_t)tb * kSlices * kTN, k0 = (int64_t)tk * kTK;
  const int slices = (int)((N - nb) / kTN < kSlices ? (N - nb) / kTN : kSlices);
  const int r = p.r;

  auto load_slice = [&](int sl, MergeStage<WK>& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 5, c = ch & 31;
      int64_t k = k0 + 8 * c;
      k = k < K ? k : K - 8;
      const int64_t e = (nb + (int64_t)sl * kTN + row) * K + k;
      if (WK == kDense) {
        st.wd[i] = *reinterpret_cast<const u32x4*>(p.W.dense + e);
      } else {
        st.wc[i] = *reinterpret_cast<const uint32_t*>(p.W.codes + (e >> 1));
        st.q8[i] = WK == kNF4DQ ? (uint32_t)p.W.q8[e >> 6] : __float_as_uint(p.W.absmax[e >> 6]);
      }
    }
  };
  // Loads, in the order they are waited for (they return in order): A's and
  // B's rows and the c2 of the block's groups first, then the weight (NF4:
  // the codes and constants of all slices, 4 slices x 4 chunks; dense: one
  // slice ahead).  Staging A, B and the steps in LDS then waits for the
  // first only, and the weight is still in flight during the first slice's
  // low-rank product.
  // A rows j < RP for columns k0 .. k0+255, B rows nb .. nb+127 (zero past r / K)
  // (clamped addresses, zeros selected)
  constexpr int NA = RP * (kTK / 8) / kThreads;  // 16-byte chunks of A per thread
  u32x4 av[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int idx = tid + kThreads * i, j = idx / (kTK / 8), c = idx % (kTK / 8);
    int64_t k = k0 + 8 * c;
    k = k < K ? k : K - 8;
    av[i] = *reinterpret_cast<const u32x4*>(p.A + (int64_t)(j < r ? j : 0) * K + k);
  }
  constexpr int NB = kSlices * kTN * RP / kThreads;  // elements of B per thread
  uint16_t bv[NB];
  const int64_t nmax = (int64_t)slices * kTN;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int idx = tid + kThreads * i, n = idx / RP, j = idx % RP;
    const bool ok = j < r && n < nmax;
    bv[i] = p.B[(nb + (ok ? n : 0)) * r + (ok ? j : 0)];
  }
  // second-level steps of groups g_lo .. g_hi (at most kMergeTab)
  const int64_t g_lo = (nb * K) >> 14;
  constexpr int NC = (kMergeTab + kThreads - 1) / kThreads;
  float c2v[NC];
  int ng = 0;
  if (WK == kNF4DQ) {
    const int64_t g_hi = ((nb + (int64_t)slices * kTN - 1) * K + K - 1) >> 14;
    ng = (int)(g_hi - g_lo + 1);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int gi = tid + kThreads * i;
      c2v[i] = p.W.c2[g_lo + (gi < ng ? gi : 0)];
    }
  }
  constexpr int NS = WK == kDense ? 2 : kSlices;
  MergeStage<WK> st[NS];
  if (WK == kDense) {
    load_slice(0, st[0]);
  } else {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) load_slice(sl < slices ? sl : 0, st[sl]);
  }

  if (WK != kDense) build_lut(lut, p.tab);
  if (WK == kNF4DQ) {
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (tid + kThreads * i < ng) stab[tid + kThreads * i] = dq_step(c2v[i]);
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int idx = tid + kThreads * i, j = idx / (kTK / 8), c = idx % (kTK / 8);
    *reinterpret_cast<u32x4*>(At + j * kAPitch + 8 * c) = sel4(j < r && k0 + 8 * c < K, av[i]);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int idx = tid + kThreads * i, n = idx / RP, j = idx % RP;
    Bt[idx] = (j < r && n < nmax) ? bv[i] : (uint16_t)0;
  }
  __syncthreads();

  const int c16 = lane & 15, g = lane >> 4;
  // slice sl: prefetch slice sl + 1 into nxt, finish slice sl from cur
  auto slice = [&](int sl, const MergeStage<WK>& sc, MergeStage<WK>& nxt) {
    if (WK == kDense && sl + 1 < slices) load_slice(sl + 1, nxt);
    // S[n][k] = s sum_j B[n][j] A[j][k] for this slice's 32 rows; wave w takes
    // column blocks 2w, 2w+1 (rows k of the transposed product)
    {
      const uint16_t* brow = Bt + (sl * kTN + l32) * RP;
      f32x16 acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[kb][v] = 0.0f;
#pragma unroll
      for (int jc = 0; jc < RP / 16; ++jc) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(brow + 16 * jc + 8 * h);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint16_t* q = At + (16 * jc + 8 * h + (c16 >> 2)) * kAPitch + 64 * wave + 32 * kb +
                              16 * (g & 1) + 4 * (c16 & 3);
          const u32x2 lo = lds_tr_m(q), hi = lds_tr_m(q + 4 * kAPitch);
          acc[kb] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, bf, acc[kb]);
        }
      }
      // lane: rows k = 64 w + 32 kb + 8 q + 4 h + i, column n = l32
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(&S[l32 * kSPitch + 64 * wave + 32 * kb + 8 * q + 4 * h]) =
              f32x4{p.s * acc[kb][4 * q], p.s * acc[kb][4 * q + 1], p.s * acc[kb][4 * q + 2],
                    p.s * acc[kb][4 * q + 3]};
    }
    __syncthreads();
    // dequantise, add, round, store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 5, c = ch & 31;
      const int64_t k = k0 + 8 * c;
      const int64_t n = nb + (int64_t)sl * kTN + row;
      const float* srow = &S[row * kSPitch + 8 * c];
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(srow);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(srow + 4);
      float w[8];
      if (WK == kDense) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w[2 * d] = lo_bf16(sc.wd[i][d]);
          w[2 * d + 1] = hi_bf16(sc.wd[i][d]);
        }
      } else {
        float a;
        if (WK == kNF4DQ) {
          const int64_t e = n * K + (k < K ? k : K - 8);
          a = dq_q_rt(p.W.dq, sc.q8[i]) * stab[(e >> 14) - g_lo];
        } else {
          a = __uint_as_float(sc.q8[i]);
        }
        const u32x4 v = deq8(sc.wc[i], a, lut);  // bf16 values the GEMM would use
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w[2 * d] = lo_bf16(v[d]);
          w[2 * d + 1] = hi_bf16(v[d]);
        }
      }
      if (k < K) {
        const u32x4 o{pack_bf16x2(w[0] + s0[0], w[1] + s0[1]),
                      pack_bf16x2(w[2] + s0[2], w[3] + s0[3]),
                      pack_bf16x2(w[4] + s1[0], w[5] + s1[1]),
                      pack_bf16x2(w[6] + s1[2], w[7] + s1[3])};
        *reinterpret_cast<u32x4*>(p.out + n * K + k) = o;
      }
    }
    __syncthreads();  // S is rewritten by the next slice
  };
  if (WK == kDense) {
    for (int sl = 0; sl < slices; sl += 2) {
      slice(sl, st[0], st[1]);
      if (sl + 1 < slices) slice(sl + 1, st[1], st[0]);
    }
  } else {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      if (sl < slices) slice(sl, st[sl], st[sl]);
  }
}

template <int WK>
int launch_merge(const MergeParams& p, unsigned blocks, hipStream_t st) {
  if (p.r <= 16)
    hipLaunchKernelGGL((merge_kernel<WK, 16>), dim3(blocks), dim3(kThreads), 0, st, p);
  else if (p.r <= 32)
    hipLaunchKernelGGL((merge_kernel<WK, 32>), dim3(blocks), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((merge_kernel<WK, 64>), dim3(blocks), dim3(kThreads), 0, st, p);
  return hip_fail(hipGetLastError(), "merge launch");
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
  p.n_blocks = (int32_t)cdiv(W.N, kSlices * kTN);
  p.out = (uint16_t*)Wout;
  p.tab = nf4_table(W.codebook);
  const unsigned blocks = (unsigned)(p.k_tiles * p.n_blocks);
  switch (weight_format(W)) {
    case kDense:
      return launch_merge<kDense>(p, blocks, st);
    case kNF4DQ:
      return launch_merge<kNF4DQ>(p, blocks, st);
    default:
      return launch_merge<kNF4>(p, blocks, st);
  }
}

}  // namespace dispatch
}  // namespace lq

// Forward of the adapted linear layer for a few rows (16 < M <= 64) with an
// NF4 weight:
//
//   Y = X Wd^T + s T B^T,   T = X A^T   ("Low-Rank Adaptation (LoRA) and QLoRA:
//   Mathematical Foundations ..." (llms.blog), the forward-pass equation with
//   alpha/r; Wd the NF4 weight dequantised to bf16 right before the multiply,
//   "LoRA and QLoRA fine-tuning under the hood", section 3.4).
//
// With so few rows the layer is bound by streaming the 4-bit weight, so the
// weight is streamed exactly once: it is cut into pieces of 128 rows (outputs
// n) x 512 columns (reduction k), one per workgroup (256 pieces for 4096^2):
//   * small_fwd_kernel: a workgroup loads its piece's codes (32 bytes per row
//     and 64-column chunk), the block constants of its rows and the matching
//     512 columns of X straight into LDS, all at the start; then per 64-column
//     chunk it dequantises the codes in registers (the level table of each
//     block built by the quad of lanes that share it, looked up with
//     v_perm_b32) into a bf16 tile (128 rows x 64 columns, two of them
//     alternating) and multiplies it with the X rows
//     (v_mfma_f32_32x32x16_bf16, weight rows as the MFMA rows).  It writes its
//     float32 partial sums of X Wd^T for its column range.  The pieces of row
//     slab 0 also form the partial sums of T over their column range from the
//     X rows already in LDS.
//   * small_fwd_reduce_kernel: adds the partial sums of the column ranges in a
//     fixed order (so the result does not depend on scheduling), forms T and
//     s T B^T in float32, writes Y (bf16) and T.
// Compared with 16-row decode chunks, each of which streams the weight again,
// every code is read and dequantised once per call.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kSfThreads = 512;
constexpr int kSfRows = 128;                 // weight rows (outputs) per workgroup
constexpr int kSfCols = 512;                 // reduction columns per workgroup
constexpr int kSfChunk = 64;                 // columns per dequantised tile (one NF4 block per row)
constexpr int kSfNC = kSfCols / kSfChunk;    // 8
constexpr int kSfMaxM = 64;

struct SfParams {
  const uint16_t* X;  // M x K
  WeightArgs W;       // NF4, N x K
  const uint16_t* A;  // r x K
  float* part;        // KS x M x N partial sums of X Wd^T
  float* tpart;       // KS x M x r partial sums of T
  int64_t M, N, K;
  int32_t NS;         // row slabs (N / 128)
  int32_t KS;         // column ranges (K / 512)
  int32_t r;
  NF4Table tab;
};

__device__ __forceinline__ uint32_t sf_lds(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 (4) bytes per lane from global memory (base + off) straight into LDS at
// m0 + 16 (4) * lane.  The compiler does not track these loads: the kernel
// waits for them itself (vmcnt, counting its own issue order) before the
// barrier that publishes them.
__device__ __forceinline__ void sf_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void sf_dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// wait until at most n vector-memory loads of this wave are outstanding
// (n is a constant once the chunk loop is unrolled)
__device__ __forceinline__ void sf_wait(int n) {
  switch (n) {
#define SF_W(k) \
  case k:       \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
    SF_W(0) SF_W(1) SF_W(2) SF_W(3) SF_W(4) SF_W(5) SF_W(6) SF_W(7)
    SF_W(8) SF_W(9) SF_W(10) SF_W(11) SF_W(12) SF_W(13) SF_W(14)
#undef SF_W
    default:
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

__device__ __forceinline__ u32x4 sf_read16(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x4* lp;
  return *(lp)(uintptr_t)addr;
}

__device__ __forceinline__ void sf_write16(uint32_t addr, const u32x4& v) {
  typedef __attribute__((address_space(3))) u32x4* lp;
  *(lp)(uintptr_t)addr = v;
}

// 16-byte chunk swizzle of 128-byte rows: the operand reads of 16
// consecutive rows (one chunk each) land on 16 distinct bank groups
__device__ __forceinline__ int sf_swz(int x) { return (x & 7) ^ ((x >> 3) & 1); }

// One workgroup (8 waves) per (row slab ns, column range ks); MT = 32-row
// groups of X rows held.  Each XCD takes a contiguous run of pieces, in
// column-range order: the slabs of one column range share the X columns.
//
// Loads, all issued at the start as direct-to-LDS loads:
//   first the block constants of the piece's rows (8-bit constants: waves 0-3
//   the two words of each row, waves 4 and 5 the rows' c2; or float32 absmax:
//   two instructions in every wave), then per chunk and wave:
//   waves 0-3: 32 rows of codes (32 bytes each);  MT = 2: also X rows
//              32 + 8 w .. + 7 (the chunk's 64 columns)
//   waves 4-7: X rows 8 (w - 4) .. + 7
// so each wave knows how many of its loads are younger than a chunk's and
// waits for that chunk alone.
// Chunk loop: the products of chunk c (tile c & 1) and the dequantisation of
// chunk c + 1 (into the other tile) have no dependence and interleave; one
// barrier per chunk, after the wait for chunk c + 2's loads.
template <int MT, int WK, bool FP8>
__global__ __launch_bounds__(kSfThreads) void small_fwd_kernel(SfParams p) {
  constexpr int DR = 32 * MT;  // X rows held
  __shared__ __attribute__((aligned(1024))) char codes[kSfNC][kSfRows * 32];
  __shared__ __attribute__((aligned(1024))) char xs[kSfNC][DR * 128];
  __shared__ __attribute__((aligned(1024))) char wt[2][kSfRows * 128];
  // per row: two words of 8-bit constants and c2, or eight float32 absmax
  __shared__ __attribute__((aligned(16))) uint32_t cst[kSfRows * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int tile = xcd_tile((int)blockIdx.x, p.NS * p.KS);
  const int ks = tile / p.NS, ns = tile - ks * p.NS;
  const int64_t n0 = (int64_t)ns * kSfRows, k0 = (int64_t)ks * kSfCols;
  const int64_t KB = K / 64;
  const int r = p.r;
  float cbq[4];
  quad_levels(p.tab, lane, cbq);

  // slab 0: this lane's A operands for the shrink over chunk `wave` of the
  // range (rank 32 q + l32, zero past r), ordinary loads issued before the
  // direct-to-LDS loads so that those stay exactly counted
  constexpr int RQ = 2;
  const bool tslab = ns == 0;
  u32x4 af[RQ][4];
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int s = 0; s < 4; ++s) af[q][s] = u32x4{0u, 0u, 0u, 0u};
  if (tslab) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int j = 32 * q + l32;
      if (j < r) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          af[q][s] = *reinterpret_cast<const u32x4*>(p.A + (int64_t)j * K + k0 + 64 * wave +
                                                     16 * s + 8 * h);
      }
    }
  }

  // ---- constants
  const uint32_t cbase = sf_lds(cst);
  if (WK == kNF4DQ) {
    if (wave < 4) {  // the row's two words of 8-bit constants (blocks 8 ks .. + 7)
      const int row = 32 * wave + (lane >> 1);
      sf_dma4(p.W.q8, (uint32_t)((n0 + row) * KB + 8 * ks + 4 * (lane & 1)), cbase + 256 * wave);
    } else if (wave < 6) {  // the row's c2 (its eight blocks share one group)
      const int row = 64 * (wave - 4) + lane;
      sf_dma4(p.W.c2, (uint32_t)((((n0 + row) * KB + 8 * ks) >> 8) * 4),
              cbase + 1024 + 256 * (wave - 4));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // absmax of rows 16 w + 8 i + lane / 8, block lane % 8
      const int row = 16 * wave + 8 * i + (lane >> 3);
      sf_dma4(p.W.absmax, (uint32_t)(((n0 + row) * KB + 8 * ks + (lane & 7)) * 4),
              cbase + (16 * wave + 8 * i) * 32);
    }
  }

  // ---- codes and X, chunk by chunk
  auto issue_x = [&](int c, int g) {  // X rows 8 g .. 8 g + 7 of chunk c
    const int row = 8 * g + (lane >> 3);
    const int64_t m = row < M ? row : M - 1;  // rows past M are never stored
    const int lc = (lane & 7) ^ sf_swz(row);
    sf_dma16(p.X, (uint32_t)((m * K + k0 + kSfChunk * c + 8 * lc) * 2),
             sf_lds(xs[c]) + 8 * g * 128);
  };
#pragma unroll
  for (int c = 0; c < kSfNC; ++c) {
    if (wave < 4) {  // codes of rows 32 w .. + 31: two lanes per row
      const int row = 32 * wave + (lane >> 1);
      sf_dma16(p.W.codes,
               (uint32_t)((((n0 + row) * K + k0 + kSfChunk * c) >> 1) + 16 * (lane & 1)),
               sf_lds(codes[c]) + 32 * wave * 32);
      if (MT == 2) issue_x(c, 4 + wave);
    } else {
      issue_x(c, wave - 4);
    }
  }
  // loads per chunk issued by this wave
  const int per = (wave < 4 && MT == 2) ? 2 : 1;

  // ---- dequantisation: thread t takes row t / 4 of the piece, codes
  // 16 (t % 4) .. + 15 of the chunk -> bf16 chunks 2 (t % 4), + 1 of the
  // tile row (128-byte rows, chunk swizzle as the X rows)
  const int dr = tid >> 2, dq = tid & 3;
  float step = 0.0f;  // fl32(c2 / 127) of this thread's row, once the constants are in
  auto dequant = [&](int c) {
    float a;
    if (WK == kNF4DQ) {
      const uint32_t qw = cst[2 * dr + (c >> 2)];
      a = dq_value<FP8>((qw >> (8 * (c & 3))) & 0xFFu) * step;
    } else {
      a = __uint_as_float(cst[8 * dr + c]);
    }
    typedef __attribute__((address_space(3))) const u32x2* lp;
    const u32x2 w = *(lp)(uintptr_t)(sf_lds(codes[c]) + dr * 32 + 8 * dq);
    const PermTable pt = perm_table_quad(cbq, a);
    const uint32_t wb = sf_lds(wt[c & 1]) + dr * 128;
#pragma unroll
    for (int d = 0; d < 2; ++d)
      sf_write16(wb + (((2 * dq + d) ^ sf_swz(dr)) << 4), perm_deq8(w[d], pt));
  };

  // ---- products: wave w takes the 32 weight rows 32 (w % 4) ..; MT = 1:
  // substeps 2 (w / 4), + 1 of each chunk (the two halves are added at the
  // end), MT = 2: X rows 32 (w / 4) .. + 31, all four substeps
  const int ct = wave & 3, wq = wave >> 2;
  const int mrow = MT == 2 ? 32 * wq + l32 : l32;
  const uint32_t wrd = (uint32_t)((32 * ct + l32) * 128);
  const uint32_t xrd = (uint32_t)(mrow * 128);
  const int sw = sf_swz(l32);
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  auto products = [&](int c) {
    const uint32_t wb = sf_lds(wt[c & 1]) + wrd, xb = sf_lds(xs[c]) + xrd;
#pragma unroll
    for (int i = 0; i < (MT == 2 ? 4 : 2); ++i) {
      const int s = MT == 2 ? i : 2 * wq + i;
      const uint32_t co = (uint32_t)(((2 * s + h) ^ sw) << 4);
      acc = mfma32(sf_read16(wb + co), sf_read16(xb + co), acc);
    }
  };

  sf_wait((kSfNC - 2) * per);  // constants and chunks 0, 1 have landed (this wave's loads)
  __syncthreads();
  if (WK == kNF4DQ) step = dq_step(__uint_as_float(cst[256 + dr]));
  dequant(0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kSfNC; ++c) {
    products(c);
    if (c + 1 < kSfNC) dequant(c + 1);
    if (c + 2 < kSfNC) sf_wait((kSfNC - 3 - c) * per);  // chunk c + 2 has landed
    __syncthreads();
  }

  // ---- partial sums of X Wd^T: lane (h, l32) holds row m = mrow, outputs
  // 32 ct + 8 q + 4 h .. + 3
  float* comb = reinterpret_cast<float*>(wt[0]);  // MT = 1: the second half's sums
  if (MT == 1 && wq == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) comb[(ct * 16 + v) * 64 + lane] = acc[v];
  }
  if (MT == 1) __syncthreads();
  if (MT == 2 || wq == 0) {
    if (MT == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] += comb[(ct * 16 + v) * 64 + lane];
    }
    if (mrow < M) {
      float* out = p.part + ((int64_t)ks * M + mrow) * N + n0 + 32 * ct + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(out + 8 * q) =
            f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
  }
  if (!tslab) return;

  // ---- slab 0: partial sums of T over the range.  Wave w multiplies chunk w
  // of X (still in LDS) by its A operands: per 32-rank block q and 32-row
  // group g an accumulator holding T[32 g + l32][32 q + 8 (v / 4) + 4 h + v % 4]
  // (the A rows are the MFMA rows); the eight waves' sums are then added in
  // wave order through LDS, one (q, g) at a time.
  __syncthreads();  // the combination buffer (MT = 1) has been read
  const int nq = (r + 31) / 32;
  float* red = reinterpret_cast<float*>(wt[0]);  // 8 waves x 1024 floats
  for (int q = 0; q < nq; ++q) {
    for (int g = 0; g < MT; ++g) {
      f32x16 ta;
#pragma unroll
      for (int v = 0; v < 16; ++v) ta[v] = 0.0f;
      const uint32_t xb = sf_lds(xs[wave]) + (uint32_t)((32 * g + l32) * 128);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        ta = mfma32(q ? af[1][s] : af[0][s], sf_read16(xb + (uint32_t)(((2 * s + h) ^ sw) << 4)), ta);
#pragma unroll
      for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = ta[v];
      __syncthreads();
      // thread t < 1024 / 2: two outputs (v, lane) of the 32 x 32 block
      for (int e = tid; e < 1024; e += kSfThreads) {
        const int v = e >> 6, ln = e & 63;
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) t += red[(w * 16 + v) * 64 + ln];
        const int m = 32 * g + (ln & 31);
        const int j = 32 * q + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
        if (m < M && j < r) p.tpart[((int64_t)ks * M + m) * r + j] = t;
      }
      __syncthreads();
    }
  }
}

// Row m, outputs 4 t .. 4 t + 3 of a 1024-output block:
//   T[m][j] = sum over column ranges (in order) of the T partial sums,
//   Y[m][n..] = sum over column ranges (in order) of the partial sums
//               + s sum_j T[m][j] B[n..][j]   (float32, then bf16)
// Block column 0 also writes T.  The partial sums of Y are loaded before the
// barrier that publishes T.
__global__ __launch_bounds__(256) void small_fwd_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ tpart, int KS, int64_t M,
    int64_t N, const uint16_t* __restrict__ B, int r, float s, float* __restrict__ T,
    uint16_t* __restrict__ Y) {
  __shared__ float ts[64];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.y;
  const int64_t n = 4 * ((int64_t)blockIdx.x * 256 + tid);
  const bool live = n < N;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (live) {
#pragma unroll 8
    for (int t = 0; t < KS; ++t)
      acc += *reinterpret_cast<const f32x4*>(part + ((int64_t)t * M + m) * N + n);
  }
  if (tid < r) {
    float u = 0.0f;
    for (int t = 0; t < KS; ++t) u += tpart[((int64_t)t * M + m) * r + tid];
    ts[tid] = u;
    if (blockIdx.x == 0 && T) T[m * r + tid] = u;
  }
  __syncthreads();
  if (!live) return;
  f32x4 e = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* brow = B + (n + i) * r;
    float d = 0.0f;
    int j = 0;
    if ((r & 7) == 0) {
      for (; j < r; j += 8) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(brow + j);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          d = fmaf(ts[j + 2 * w], lo_bf16(b[w]), d);
          d = fmaf(ts[j + 2 * w + 1], hi_bf16(b[w]), d);
        }
      }
    }
    for (; j < r; ++j) d = fmaf(ts[j], bf16_to_f32(brow[j]), d);
    e[i] = d;
  }
  *reinterpret_cast<u32x2*>(Y + m * N + n) =
      u32x2{pack_bf16x2(acc[0] + s * e[0], acc[1] + s * e[1]),
            pack_bf16x2(acc[2] + s * e[2], acc[3] + s * e[3])};
}

size_t sf_align(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

namespace dispatch {

size_t small_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t KS = K / kSfCols;
  return sf_align((size_t)(KS * M * N) * 4) + (size_t)(KS * M * r) * 4;
}

// Whole pieces (N % 128, K % 512), every byte offset of the codes and of X
// below 2^32.
bool small_fwd_eligible(const lq_weight& W, int64_t M, int64_t r) {
  return W.kind == LQ_WEIGHT_NF4 && M > 16 && M <= kSfMaxM && r >= 1 && r <= 64 &&
         W.N % kSfRows == 0 && W.K % kSfCols == 0 && (double)W.N * W.K / 2 < 4294967296.0 &&
         (double)M * W.K * 2 < 4294967296.0;
}

template <int MT, int WK, bool FP8>
static void launch_sf(const SfParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((small_fwd_kernel<MT, WK, FP8>), grid, dim3(kSfThreads), 0, st, p);
}

int small_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
              int64_t r, float s, void* Y, float* T_out, void* ws, hipStream_t st) {
  SfParams p;
  p.X = (const uint16_t*)X;
  p.W = weight_args(W);
  p.A = (const uint16_t*)A;
  p.M = M;
  p.N = W.N;
  p.K = W.K;
  p.NS = (int32_t)(W.N / kSfRows);
  p.KS = (int32_t)(W.K / kSfCols);
  p.r = (int32_t)r;
  p.part = (float*)ws;
  p.tpart = (float*)((char*)ws + sf_align((size_t)(p.KS * M * W.N) * 4));
  p.tab = nf4_table(W.codebook);
  const dim3 grid((unsigned)(p.NS * p.KS));
  timing_begin("small_fwd", st);
  const bool fp8 = W.double_quant == LQ_DQ_FP8;
  if (M <= 32) {
    if (!W.double_quant) launch_sf<1, kNF4, false>(p, grid, st);
    else if (fp8) launch_sf<1, kNF4DQ, true>(p, grid, st);
    else launch_sf<1, kNF4DQ, false>(p, grid, st);
  } else {
    if (!W.double_quant) launch_sf<2, kNF4, false>(p, grid, st);
    else if (fp8) launch_sf<2, kNF4DQ, true>(p, grid, st);
    else launch_sf<2, kNF4DQ, false>(p, grid, st);
  }
  timing_end(st);
  int e = hip_fail(hipGetLastError(), "small forward launch");
  if (e) return e;
  const dim3 rgrid((unsigned)cdiv(W.N, 1024), (unsigned)M);
  hipLaunchKernelGGL(small_fwd_reduce_kernel, rgrid, dim3(256), 0, st, (const float*)p.part,
                     (const float*)p.tpart, (int)p.KS, M, W.N, (const uint16_t*)B, (int)r, s,
                     T_out, (uint16_t*)Y);
  return hip_fail(hipGetLastError(), "small forward reduce launch");
}

}  // namespace dispatch
}  // namespace lq

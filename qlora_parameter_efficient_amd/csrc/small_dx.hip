// dX of the adapted linear layer for a few rows (M <= 64) with an NF4 weight:
//
//   dX = dY Wd + s U A,   U = dY B   ("Low-Rank Adaptation (LoRA) and QLoRA:
//   Mathematical Foundations ..." (llms.blog), section "Gradient Dynamics and
//   Backpropagation Mechanics": dL/dx; Wd the NF4 weight dequantised to bf16
//   right before the multiply, "LoRA and QLoRA fine-tuning under the hood",
//   section 3.4).
//
// With so few rows the product is bound by streaming the 4-bit weight, and the
// large-tile path (one bf16 copy of W0, then 256 x 128 output tiles of which
// only M rows are used) streams it through far too few workgroups.  Here the
// weight is cut into pieces of 128 columns x 512 rows, one per workgroup (256
// pieces for 4096^2), each streamed once:
//   * small_dx_kernel: a workgroup loads its piece's codes (64 bytes per row)
//     and the matching 512 columns of dY straight into LDS, then per 64-row
//     chunk dequantises the codes through the LDS level table into a bf16 tile
//     (64 rows x 128 columns, two of them alternating) and multiplies it, read
//     transposed with ds_read_b64_tr_b16, with the dY rows
//     (v_mfma_f32_32x32x16_bf16; the weight columns are the MFMA rows).  It
//     writes its float32 partial sums of dX for its row range, and its partial
//     sums of U for one rank column (column j goes to the workgroups of column
//     slab j, j + slabs, ...), from the dY rows already in LDS.
//   * small_dx_reduce_kernel: adds the partial sums of the row ranges in a
//     fixed order (so the result does not depend on scheduling), forms U and
//     s (U A) in float32, writes U and dX (bf16).
//
// LDS bank layout (64 banks of 4 bytes: a 256-byte period).  Tile row n holds
// its 16-byte chunk c at c ^ 5 (n & 3): the dequantising stores (16 lanes: 4
// rows x 4 chunks c = 4 q + d) and the transposing reads (32 lanes: 4 rows x
// 4 consecutive chunks) each land on 16 distinct 16-byte bank groups.  dY row
// m holds its chunk c of each 64-column group at c ^ ((m >> 1) & 7), so the 32
// rows that one operand read covers fall on distinct groups per 16 lanes.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kSdxThreads = 512;
constexpr int kSdxCols = 128;   // weight columns per workgroup
constexpr int kSdxRows = 512;   // weight rows per workgroup
constexpr int kSdxChunk = 64;   // weight rows per dequantised tile
constexpr int kSdxNC = kSdxRows / kSdxChunk;
constexpr int kSdxMaxM = 64;

struct SdxParams {
  const uint16_t* dY;  // M x N
  WeightArgs W;        // NF4, N x K
  const uint16_t* B;   // N x r
  float* part;         // S x M x K partial sums of dY Wd
  float* upart;        // S x M x r partial sums of U
  int64_t M, N, K;
  int32_t S;           // row ranges
  int32_t KS;          // column slabs
  int32_t r;
  NF4Table tab;
};

__device__ __forceinline__ uint32_t sdx_lds(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 (4) bytes per lane from global memory (base + off) straight into LDS at
// m0 + 16 (4) * lane.  The compiler does not track these loads: the kernel
// waits for them itself (vmcnt, counting its own issue order) before the
// barrier that publishes them.
__device__ __forceinline__ void sdx_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void sdx_dma4(const void* base, uint32_t off, uint32_t lds) {
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
__device__ __forceinline__ void sdx_wait(int n) {
  switch (n) {
#define SDX_W(k) \
  case k:        \
    asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
    SDX_W(0) SDX_W(1) SDX_W(2) SDX_W(3) SDX_W(4) SDX_W(5) SDX_W(6) SDX_W(7)
    SDX_W(8) SDX_W(9) SDX_W(10) SDX_W(11) SDX_W(12) SDX_W(13) SDX_W(14)
#undef SDX_W
    default:
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

__device__ __forceinline__ u32x4 sdx_read16(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x4* lp;
  return *(lp)(uintptr_t)addr;
}

__device__ __forceinline__ u32x2 sdx_read8(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x2* lp;
  return *(lp)(uintptr_t)addr;
}

__device__ __forceinline__ void sdx_write16(uint32_t addr, const u32x4& v) {
  typedef __attribute__((address_space(3))) u32x4* lp;
  *(lp)(uintptr_t)addr = v;
}

typedef short sdx_s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 sdx_read_tr(uint32_t addr) {
  typedef __attribute__((address_space(3))) sdx_s16x4* lp;
  const sdx_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// byte offset of logical 16-byte chunk c of tile row n (256-byte rows)
__device__ __forceinline__ uint32_t sdx_tile_off(int n, int c) {
  return (uint32_t)(n * 256 + ((c ^ (5 * (n & 3))) << 4));
}

// byte offset of logical 16-byte chunk c (0..7) of dY row m in a chunk's
// block (128-byte rows)
__device__ __forceinline__ uint32_t sdx_dy_off(int m, int c) {
  return (uint32_t)(m * 128 + ((c ^ ((m >> 1) & 7)) << 4));
}

__device__ __forceinline__ f32x16 sdx_mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One workgroup (8 waves) per (column slab ks, row range ns); MT = 32-row
// groups of dY rows.  Workgroups are placed so that each XCD takes a
// contiguous run of pieces: the two slabs that share a 128-byte line of codes,
// and the slabs that share the same dY columns, meet in one L2.
//
// Loads, all issued at the start as direct-to-LDS loads, per chunk and wave:
//   waves 0-3: 16 rows of codes (64 bytes each);  MT = 2: also dY rows
//              32 + 8 w .. + 7 (the chunk's 64 columns)
//   waves 4-7: dY rows 8 (w - 4) .. + 7;  waves 6, 7: also the block constants
//              of the chunk's rows (8-bit constants and c2, or absmax)
// so each wave knows how many of its loads are younger than a chunk's and
// waits for that chunk alone.  A ragged last row range repeats its last
// chunk's loads in place of the missing chunks, keeping the counts fixed.
// Chunk loop: the products of chunk c (tile c & 1) and the dequantisation of
// chunk c + 1 (into the other tile) have no dependence and interleave; one
// barrier per chunk, after the wait for chunk c + 2's loads.
template <int MT, bool DQ>
__global__ __launch_bounds__(kSdxThreads) void small_dx_kernel(SdxParams p) {
  constexpr int DR = 32 * MT;  // dY rows held
  __shared__ __attribute__((aligned(1024))) char codes[kSdxNC][kSdxChunk * 64];
  __shared__ __attribute__((aligned(1024))) char dyt[kSdxNC][DR * 128];
  __shared__ __attribute__((aligned(1024))) char wt[2][kSdxChunk * 256];
  __shared__ uint32_t scl[kSdxNC][128];
  __shared__ float2 lut[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int tile = xcd_tile((int)blockIdx.x, p.S * p.KS);
  const int ks = tile % p.KS, ns = tile / p.KS;
  const int64_t n0 = (int64_t)ns * kSdxRows;
  const int nrows = (int)((N - n0) < kSdxRows ? (N - n0) : kSdxRows);  // multiple of 64
  const int nch = nrows / kSdxChunk;
  const int64_t KB = K / 64;
  const bool ulive = ks < p.r;  // this slab forms U partial sums (rank column ks)

  // B's rank column ks over the row range, for U (an ordinary load, issued
  // before the direct-to-LDS loads so that their counting stays exact)
  // (unconditional, from a clamped in-range address, so that nothing waits
  // for it before its use)
  const uint16_t braw =
      p.B[(n0 + (tid < nrows ? tid : nrows - 1)) * p.r + (ks < p.r ? ks : p.r - 1)];

  auto issue_dy = [&](int c, int64_t nb, int g) {  // dY rows 8 g .. 8 g + 7
    int64_t m = 8 * g + (lane >> 3);
    m = m < M ? m : M - 1;  // rows past M are never used
    const int lc = (lane & 7) ^ (int)(((8 * g + (lane >> 3)) >> 1) & 7);
    const uint32_t off = (uint32_t)((m * N + nb + 8 * lc) * 2);
    sdx_dma16(p.dY, off, sdx_lds(dyt[c]) + 8 * g * 128);
  };
#pragma unroll
  for (int c = 0; c < kSdxNC; ++c) {
    const int cc = c < nch ? c : nch - 1;
    const int64_t nb = n0 + (int64_t)kSdxChunk * cc;  // first row of the chunk
    if (wave < 4) {
      const uint32_t off = (uint32_t)((((nb + 16 * wave + (lane >> 2)) * K) >> 1) +
                                      (int64_t)ks * 64 + 16 * (lane & 3));
      sdx_dma16(p.W.codes, off, sdx_lds(codes[c]) + 16 * wave * 64);
      if (MT == 2) issue_dy(c, nb, 4 + wave);
    } else {
      issue_dy(c, nb, wave - 4);
      if (wave >= 6) {
        const uint32_t dst = sdx_lds(scl[c]) + (wave - 6) * 256;
        if (DQ) {
          const int64_t b0 = (nb + lane) * KB + 2 * ks;  // the row's first block
          if (wave == 6)
            sdx_dma4(p.W.q8, (uint32_t)(b0 & ~(int64_t)3), dst);
          else
            sdx_dma4(p.W.c2, (uint32_t)((b0 >> 8) * 4), dst);
        } else {
          const int64_t row = nb + 32 * (wave - 6) + (lane >> 1);
          sdx_dma4(p.W.absmax, (uint32_t)((row * KB + 2 * ks + (lane & 1)) * 4), dst);
        }
      }
    }
  }
  // loads per chunk issued by this wave
  const int per = (wave < 4) ? (MT == 2 ? 2 : 1) : (wave >= 6 ? 2 : 1);
  build_lut(lut, p.tab);

  // ---- dequantisation: thread t takes row t / 8 of a chunk, codes
  // 16 (t % 8) .. + 15 of the slab (block 2 ks + (t % 8) / 4 of the row) ->
  // bf16 chunks 2 (t % 8), + 1 of the tile row
  const int dr = tid >> 3, dq = tid & 7;
  auto dequant = [&](int c) {
    const int64_t n = n0 + (int64_t)kSdxChunk * c + dr;
    float a;
    if (DQ) {
      const uint32_t qw = scl[c][dr];
      const int bo = (int)((n * KB + 2 * ks) & 3) + (dq >> 2);
      a = dq_q_rt(p.W.dq, (qw >> (8 * bo)) & 0xFFu) * dq_step(__uint_as_float(scl[c][64 + dr]));
    } else {
      a = __uint_as_float(scl[c][2 * dr + (dq >> 2)]);
    }
    const u32x2 w = sdx_read8(sdx_lds(codes[c]) + dr * 64 + 8 * dq);
    const uint32_t wb = sdx_lds(wt[c & 1]);
    sdx_write16(wb + sdx_tile_off(dr, 2 * dq), deq8(w[0], a, lut));
    sdx_write16(wb + sdx_tile_off(dr, 2 * dq + 1), deq8(w[1], a, lut));
  };

  // ---- products: wave w takes the 32 columns 32 (w % 4) .. of the slab;
  // MT = 1: substeps 2 (w / 4), + 1 of each chunk (the two halves are added at
  // the end), MT = 2: dY rows 32 (w / 4) .. + 31, all four substeps.  Weight
  // tile read transposed: in each 16-lane group, lane (row nlo, column group)
  // addresses 4 columns of one of 4 rows and receives one column of the 4 rows.
  const int ct = wave & 3, wq = wave >> 2;
  const int gc = l32 & 15, half = l32 >> 4, nlo = gc >> 2;
  const int col = 32 * ct + 16 * half + 4 * (gc & 3);
  // rows 16 s + 8 h + nlo (+ 4): row & 3 = nlo in every substep
  const uint32_t wrd = sdx_tile_off(8 * h + nlo, col >> 3) + (col & 7) * 2;
  const int mrow = MT == 2 ? 32 * wq + l32 : l32;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  auto products = [&](int c) {
    const uint32_t wb = sdx_lds(wt[c & 1]), dbase = sdx_lds(dyt[c]);
#pragma unroll
    for (int i = 0; i < (MT == 2 ? 4 : 2); ++i) {
      const int s = MT == 2 ? i : 2 * wq + i;
      const uint32_t ad = wb + wrd + (uint32_t)(16 * s * 256);
      const u32x2 lo = sdx_read_tr(ad), hi = sdx_read_tr(ad + 4 * 256);
      acc = sdx_mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]},
                       sdx_read16(dbase + sdx_dy_off(mrow, 2 * s + h)), acc);
    }
  };

  sdx_wait((kSdxNC - 2) * per);  // chunks 0 and 1 have landed (this wave's loads)
  __syncthreads();
  if (nch > 0) dequant(0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kSdxNC; ++c) {
    if (c < nch) products(c);
    if (c + 1 < nch) dequant(c + 1);
    if (c + 2 < kSdxNC) sdx_wait((kSdxNC - 3 - c) * per);  // chunk c + 2 has landed
    __syncthreads();
  }

  // ---- partial sums of dY Wd: lane (h, l32) holds row m, columns
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
    const int64_t m = mrow;
    if (m < M) {
      float* out = p.part + ((int64_t)ns * M + m) * K + (int64_t)ks * kSdxCols + 32 * ct + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(out + 8 * q) =
            f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
  }

  // ---- partial sums of U = dY B for rank columns ks, ks + KS, ...: B's
  // column over the row range in LDS, then thread (m, g) sums the n of group
  // g from the dY rows in LDS, and the groups are added in order
  if (!ulive) return;
  constexpr int NG = kSdxThreads / DR;  // n groups
  constexpr int GN = kSdxRows / NG;     // n per group
  float* bcol = reinterpret_cast<float*>(wt[1]);
  float* ured = bcol + kSdxRows;
  const int um = tid % DR, ug = tid / DR;
  for (int j = ks; j < p.r; j += p.KS) {
    __syncthreads();  // the previous column is no longer read
    const float bval = tid >= nrows ? 0.0f
                       : j == ks  ? bf16_to_f32(braw)
                                  : bf16_to_f32(p.B[(n0 + tid) * p.r + j]);
    bcol[tid] = bval;
    __syncthreads();
    float u = 0.0f;
    for (int n = GN * ug; n < GN * ug + GN && n < nrows; n += 8) {
      const u32x4 v = sdx_read16(sdx_lds(dyt[n / kSdxChunk]) + sdx_dy_off(um, (n % kSdxChunk) / 8));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u = fmaf(__uint_as_float(v[e] << 16), bcol[n + 2 * e], u);
        u = fmaf(__uint_as_float(v[e] & 0xFFFF0000u), bcol[n + 2 * e + 1], u);
      }
    }
    ured[ug * DR + um] = u;
    __syncthreads();
    if (tid < M) {
      float t = 0.0f;
      for (int g = 0; g < NG; ++g) t += ured[g * DR + tid];
      p.upart[((int64_t)ns * M + tid) * p.r + j] = t;
    }
  }
}

// Row m, columns 4 t .. 4 t + 3 of a 1024-column block:
//   U[m][j] = sum over row ranges (in order) of the U partial sums,
//   dX[m][k..] = sum over row ranges (in order) of the partial sums
//                + s sum_j U[m][j] A[j][k..]   (float32, then bf16)
// Block column 0 also writes U.  Every load that does not need U (the partial
// sums and the first 16 rows of A) is issued before the barrier that
// publishes U.
__global__ __launch_bounds__(256) void small_dx_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ upart, int S, int64_t M, int64_t K,
    const uint16_t* __restrict__ A, int r, float s, float* __restrict__ U,
    uint16_t* __restrict__ dX) {
  __shared__ float us[64];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.y;
  const int64_t k = 4 * ((int64_t)blockIdx.x * 256 + tid);
  const bool live = k < K;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  u32x2 av[16];
  if (live) {
#pragma unroll 8
    for (int t = 0; t < S; ++t)
      acc += *reinterpret_cast<const f32x4*>(part + ((int64_t)t * M + m) * K + k);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      av[j] = j < r ? *reinterpret_cast<const u32x2*>(A + (int64_t)j * K + k) : u32x2{0u, 0u};
  }
  if (tid < r) {
    float u = 0.0f;
    for (int t = 0; t < S; ++t) u += upart[((int64_t)t * M + m) * r + tid];
    us[tid] = u;
    if (blockIdx.x == 0 && U) U[m * r + tid] = u;
  }
  __syncthreads();
  if (!live) return;
  f32x4 e = {0.0f, 0.0f, 0.0f, 0.0f};
  auto add = [&](float u, const u32x2& a) {
    e[0] = fmaf(u, __uint_as_float(a[0] << 16), e[0]);
    e[1] = fmaf(u, __uint_as_float(a[0] & 0xFFFF0000u), e[1]);
    e[2] = fmaf(u, __uint_as_float(a[1] << 16), e[2]);
    e[3] = fmaf(u, __uint_as_float(a[1] & 0xFFFF0000u), e[3]);
  };
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < r) add(us[j], av[j]);
  for (int j = 16; j < r; ++j) add(us[j], *reinterpret_cast<const u32x2*>(A + (int64_t)j * K + k));
  *reinterpret_cast<u32x2*>(dX + m * K + k) =
      u32x2{pack_bf16x2(acc[0] + s * e[0], acc[1] + s * e[1]),
            pack_bf16x2(acc[2] + s * e[2], acc[3] + s * e[3])};
}

int64_t sdx_ranges(int64_t N) { return cdiv(N, kSdxRows); }
size_t sdx_align(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

namespace dispatch {

size_t small_dx_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t S = sdx_ranges(N);
  return sdx_align((size_t)(S * M * K) * 4) + (size_t)(S * M * r) * 4;
}

// The partial sums go into the large-tile dX workspace, so that path's
// conditions (which also keep every byte offset of the codes and of dY below
// 2^32) and its workspace size bound this one.
bool small_dx_eligible(const lq_weight& W, int64_t M, int64_t r) {
  return W.kind == LQ_WEIGHT_NF4 && M >= 1 && M <= kSdxMaxM && r >= 1 && r <= 64 &&
         W.K % kSdxCols == 0 && W.N % kSdxChunk == 0 && big_dx_eligible(M, W.N, W.K) &&
         small_dx_ws_bytes(M, W.N, W.K, r) <= big_dx_ws_bytes(M, W.N, W.K);
}

int small_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
             int64_t r, float s, float* U, void* dX, void* ws, hipStream_t st) {
  SdxParams p;
  p.dY = (const uint16_t*)dY;
  p.W = weight_args(W);
  p.B = (const uint16_t*)B;
  p.M = M;
  p.N = W.N;
  p.K = W.K;
  p.S = (int32_t)sdx_ranges(W.N);
  p.KS = (int32_t)(W.K / kSdxCols);
  p.r = (int32_t)r;
  p.part = (float*)ws;
  p.upart = (float*)((char*)ws + sdx_align((size_t)(p.S * M * W.K) * 4));
  p.tab = nf4_table(W.codebook);
  const dim3 grid((unsigned)(p.S * p.KS));
  timing_begin("small_dx", st);
  if (M <= 32) {
    if (W.double_quant)
      hipLaunchKernelGGL((small_dx_kernel<1, true>), grid, dim3(kSdxThreads), 0, st, p);
    else
      hipLaunchKernelGGL((small_dx_kernel<1, false>), grid, dim3(kSdxThreads), 0, st, p);
  } else {
    if (W.double_quant)
      hipLaunchKernelGGL((small_dx_kernel<2, true>), grid, dim3(kSdxThreads), 0, st, p);
    else
      hipLaunchKernelGGL((small_dx_kernel<2, false>), grid, dim3(kSdxThreads), 0, st, p);
  }
  timing_end(st);
  int e = hip_fail(hipGetLastError(), "small dX launch");
  if (e) return e;
  const dim3 rgrid((unsigned)cdiv(W.K, 1024), (unsigned)M);
  hipLaunchKernelGGL(small_dx_reduce_kernel, rgrid, dim3(256), 0, st, (const float*)p.part,
                     (const float*)p.upart, (int)p.S, M, W.K, (const uint16_t*)A, (int)r, s, U,
                     (uint16_t*)dX);
  return hip_fail(hipGetLastError(), "small dX reduce launch");
}

}  // namespace dispatch
}  // namespace lq

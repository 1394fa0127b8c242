// bf16 MFMA kernels of the adapted linear layer on gfx950.
//
//   forward   Y  = X deq(W0)^T + s (X A^T) B^T
//   backward  dX = dY deq(W0)   + s (dY B) A
//
// ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ..."
// (llms.blog): the forward-pass equation with alpha/r after B, and section
// "Gradient Dynamics and Backpropagation Mechanics" for dL/dx; W0 is read
// only by these two products.  NF4 weights are dequantised to bf16 right
// before the multiply, section "1. 4-bit NormalFloat (NF4) Quantization";
// "LoRA and QLoRA fine-tuning under the hood", section 3.4: dequantise in
// on-chip memory so the dense W0 never reaches VRAM.)
//
// Structure shared by both kernels.  A workgroup of 256 threads (4 waves)
// owns a 128-wide slice of the weight-side output dimension (n for the
// forward, k for dX) and 128 * MS activation rows; wave w owns rows
// 32 MS w .. +32 MS.  The reduction runs in steps of 128.  Each step the whole
// workgroup stages one LDS tile holding the 128 weight rows -- NF4 codes
// dequantised through a byte-indexed level table, and for dX transposed in
// registers so the reduction index n is contiguous -- plus the RP rows of the
// rank-r shrink operand (A for the forward, B^T for dX).  Each wave streams
// its own activation rows straight from global memory into MFMA registers, so
// every weight element is dequantised once per 128 * MS activation rows and
// activations never pass through LDS.
//
// Software pipeline per step: issue the next step's global loads (activation
// fragments into the idle half of a ping-pong register pair, weight codes
// into staging registers), run the 8 MFMA substeps on the current LDS tile
// with each substep's LDS fragment reads issued one substep ahead, then
// dequantise / transpose the staged next tile into the other LDS buffer, one
// barrier.  All loads are issued from clamped addresses; lanes out of range
// select zeros instead of branching.
//
// The LoRA branch is fused: the shrink (X A^T, or dY B) runs as extra MFMA
// rows in the same substeps on the activation registers already loaded (r
// padded to 32 or 64), and the expand (. B^T, or . A) runs in the epilogue on
// the finished accumulators, with s folded into the bf16 rounding of T.  The
// output tile is computed transposed (weight side = MFMA rows), so each lane
// ends up holding four consecutive outputs of one row and stores 8 bytes.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileI = 128;   // weight-side outputs per workgroup
constexpr int kBK = 64;       // reduction elements per step
constexpr int kLP = kBK + 8;  // LDS row pitch (bf16): 144 bytes, conflict-free 16-byte reads

__device__ __forceinline__ u32x4 sel4(bool ok, const u32x4& v) {
  return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

// Four consecutive bf16 of a row (8 bytes) or zeros, with element masking.
__device__ __forceinline__ u32x2 load4_masked(const uint16_t* row, int j0, int jmax) {
  if (j0 + 4 <= jmax && ((reinterpret_cast<uintptr_t>(row + j0) & 7) == 0))
    return *reinterpret_cast<const u32x2*>(row + j0);
  uint16_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (j0 + i < jmax) ? row[j0 + i] : (uint16_t)0;
  return u32x2{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
}

// bf16 MFMA B operand of the expand for chunk c from a shrink accumulator:
// lane (h) gets T[.][16c + 4h + 0..3] and T[.][16c + 8 + 4h + 0..3], scaled by s.
__device__ __forceinline__ u32x4 t_operand(const f32x16& t, int cc, float s) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(s * t[8 * cc + 2 * e], s * t[8 * cc + 2 * e + 1]);
  return o;
}

// R x 8 bf16 patch, rows[i][d] = elements (2d, 2d+1) of row i (R = 4 or 8),
// stored transposed: output row c (c = 0..7) holds element c of rows 0..R-1.
template <int R>
__device__ __forceinline__ void store_transposed(const uint32_t (&rows)[R][4], uint16_t* dst,
                                                 int pitch) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t ev[R / 2], od[R / 2];
#pragma unroll
    for (int e = 0; e < R / 2; ++e) {
      ev[e] = pair_lo(rows[2 * e][d], rows[2 * e + 1][d]);
      od[e] = pair_hi(rows[2 * e][d], rows[2 * e + 1][d]);
    }
    if (R == 8) {
      *reinterpret_cast<u32x4*>(dst + (2 * d) * pitch) = u32x4{ev[0], ev[1], ev[2], ev[3]};
      *reinterpret_cast<u32x4*>(dst + (2 * d + 1) * pitch) = u32x4{od[0], od[1], od[2], od[3]};
    } else {
      *reinterpret_cast<u32x2*>(dst + (2 * d) * pitch) = u32x2{ev[0], ev[1]};
      *reinterpret_cast<u32x2*>(dst + (2 * d + 1) * pitch) = u32x2{od[0], od[1]};
    }
  }
}

// Activation tile of one step, 128 MS rows x 64: thread t loads chunks
// c = t + 256 i (row c / 8, 16-byte chunk c % 8), so eight consecutive lanes
// read one row's 128 contiguous bytes.  Offsets are per-thread constants
// (rows past the end clamped: their outputs are never stored); the step only
// moves the uniform base pointer.
template <int MS>
struct ActStage {
  u32x4 v[4 * MS];
};

template <int MS>
__device__ __forceinline__ void act_offsets(uint32_t (&off)[4 * MS], int64_t ld, int64_t m0,
                                            int64_t rows) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4 * MS; ++i) {
    int64_t m = m0 + (tid >> 3) + 32 * i;
    m = m < rows ? m : rows - 1;
    off[i] = (uint32_t)((m * ld + 8 * (tid & 7)) * 2);
  }
}

template <int MS>
__device__ __forceinline__ void act_load(ActStage<MS>& st, const char* base,
                                         const uint32_t (&off)[4 * MS]) {
#pragma unroll
  for (int i = 0; i < 4 * MS; ++i) st.v[i] = *reinterpret_cast<const u32x4*>(base + off[i]);
}

// part (0..3) of storing an activation stage: chunks i = MS part .. +MS
template <int MS>
__device__ __forceinline__ void act_part(const ActStage<MS>& st, uint16_t* tile, int part) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < MS; ++j) {
    const int i = MS * part + j;
    *reinterpret_cast<u32x4*>(tile + ((tid >> 3) + 32 * i) * kLP + 8 * (tid & 7)) = st.v[i];
  }
}

// One MFMA step over the tiles in LDS: weight tile rows 32 ns + l32 (4 output
// subtiles, then JT shrink subtiles at rows 128 + 32 jt + l32) against the
// activation tile rows of this wave (32 MS wave + 32 ms + l32).  Reduction
// elements of substep s for lane half h: 32 h + 8 s .. +7.  LDS fragment reads
// run one substep ahead; after the MFMAs of substep s, part(s) stores one
// quarter of the next step's tiles.
template <int MS, int JT, typename Part>
__device__ __forceinline__ void mfma_step(const uint16_t* wtile, const uint16_t* atile, int wave,
                                          int l32, int h, f32x16 (&acc)[4][MS],
                                          f32x16 (&tacc)[JT > 0 ? JT : 1][MS], Part&& part) {
  constexpr int NR = 4 + JT;
  const uint16_t* wbase = wtile + l32 * kLP + 32 * h;
  const uint16_t* abase = atile + (32 * MS * wave + l32) * kLP + 32 * h;
  u32x4 wf[2][NR], af[2][MS];
#pragma unroll
  for (int ns = 0; ns < NR; ++ns) wf[0][ns] = *reinterpret_cast<const u32x4*>(wbase + 32 * ns * kLP);
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) af[0][ms] = *reinterpret_cast<const u32x4*>(abase + 32 * ms * kLP);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = s & 1;
    if (s < 3) {
#pragma unroll
      for (int ns = 0; ns < NR; ++ns)
        wf[c ^ 1][ns] = *reinterpret_cast<const u32x4*>(wbase + 32 * ns * kLP + 8 * (s + 1));
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        af[c ^ 1][ms] = *reinterpret_cast<const u32x4*>(abase + 32 * ms * kLP + 8 * (s + 1));
    }
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[ns][ms] = mfma32(wf[c][ns], af[c][ms], acc[ns][ms]);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) tacc[jt][ms] = mfma32(wf[c][4 + jt], af[c][ms], tacc[jt][ms]);
    part(s);
  }
}

template <int N1, int N2>
__device__ __forceinline__ void zero_acc(f32x16 (&a)[N1][N2]) {
#pragma unroll
  for (int i = 0; i < N1; ++i)
#pragma unroll
    for (int j = 0; j < N2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) a[i][j][v] = 0.0f;
}

// ------------------------------------------------------------------ forward

struct FwdParams {
  const uint16_t* X;
  int64_t M;
  WeightArgs W;
  const uint16_t* A;        // r x K            (single adapter)
  const uint16_t* B;        // N x r            (single adapter)
  const uint16_t* Tm;       // M x RP bf16, s-scaled and adapter-masked (multi)
  const uint16_t* Bstack;   // n_ad x N x r     (multi)
  int32_t r;
  int32_t n_ad;
  float s;
  int32_t m_tiles;
  int32_t n_tiles;
  int32_t pad;
  uint16_t* Y;
  float* T_out;
  NF4Table tab;
};

constexpr int kFwdTab = 1024;  // second-level steps of one tile's 128 rows (K <= 65536)

// Weight formats, fixed at compile time: dense bf16, NF4 with 8-bit double
// quantised constants, NF4 with float32 absmax.
constexpr int kDense = 0, kNF4DQ = 1, kNF4 = 2;

// Block constant as loaded (8-bit value, or float32 absmax bits) and its
// second-level group relative to the step table; turned into the scale a'
// only when the tile is written, a step after the load was issued.
struct RawScale {
  uint32_t q;
  int32_t gi;
};

template <int WK>
__device__ __forceinline__ RawScale load_raw_scale(const uint8_t* q8, const float* absmax,
                                                   uint32_t qoff, int32_t gi) {
  RawScale r;
  r.gi = gi;
  r.q = WK == kNF4DQ ? (uint32_t)q8[qoff] : __float_as_uint(absmax[qoff]);
  return r;
}

template <int WK>
__device__ __forceinline__ float raw_scale_value(const RawScale& r, const float* tab) {
  if (WK == kNF4DQ) return (float)r.q * tab[r.gi];
  return __uint_as_float(r.q);
}

// Weight staging for one forward step: rows n0 .. n0+127, columns kb .. kb+63.
// NF4: thread t takes row t/2, half a block (16 code bytes).  Dense: thread t
// takes four 16-byte chunks (row t/8 + 32 i).  The JT = RP/32 shrink operand
// tiles (A rows, RP x 64; thread t takes row t/8 + 32 i) ride along as tile
// rows 128 ...  Stages are loaded two steps ahead and written to LDS a
// quarter per MFMA substep.  Per-thread offsets are fixed; rows past the end
// are clamped (they only feed outputs that are never stored).
template <int WK, int JT>
struct FwdStage {
  u32x4 w[WK == kDense ? 4 : 1];
  RawScale sc;
  u32x4 at[JT > 0 ? JT : 1];
};

struct FwdOffsets {
  uint32_t w[4];       // dense: byte offsets of the 4 chunks; NF4: w[0] code byte offset
  uint32_t q;          // NF4: block index at k = 0
  uint32_t e;          // NF4: element index at k = 0 (for the group of each step)
  uint32_t a[2];       // A rows
};

template <int WK, int JT>
__device__ __forceinline__ void fwd_stage_load(FwdStage<WK, JT>& st, const FwdParams& p,
                                               const FwdOffsets& o, int64_t kb, int64_t g_lo) {
  if (WK == kDense) {
    const char* base = reinterpret_cast<const char*>(p.W.dense + kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.w[i] = *reinterpret_cast<const u32x4*>(base + o.w[i]);
  } else {
    st.w[0] = *reinterpret_cast<const u32x4*>(p.W.codes + (kb >> 1) + o.w[0]);
    const uint32_t qoff = o.q + (uint32_t)(kb >> 6);
    const int32_t gi = (int32_t)((((int64_t)o.e + kb) >> 14) - g_lo);
    st.sc = load_raw_scale<WK>(p.W.q8, p.W.absmax, qoff, gi);
  }
  const char* abase = reinterpret_cast<const char*>(p.A + kb);
#pragma unroll
  for (int i = 0; i < JT; ++i) st.at[i] = *reinterpret_cast<const u32x4*>(abase + o.a[i]);
}

// part (0..3) of writing a staged forward weight tile; a = its block scale
template <int WK, int JT>
__device__ __forceinline__ void fwd_stage_part(const FwdStage<WK, JT>& st, uint16_t* tile,
                                               const float2* lut, float a, int part) {
  const int tid = threadIdx.x;
  if (WK == kDense) {
    *reinterpret_cast<u32x4*>(tile + ((tid >> 3) + 32 * part) * kLP + 8 * (tid & 7)) = st.w[part];
  } else {
    *reinterpret_cast<u32x4*>(tile + (tid >> 1) * kLP + 32 * (tid & 1) + 8 * part) =
        deq8(st.w[0][part], a, lut);
  }
  if (part < JT)
    *reinterpret_cast<u32x4*>(tile + (kTileI + (tid >> 3) + 32 * part) * kLP + 8 * (tid & 7)) =
        st.at[part];
}

template <int WK, int MS, int RP, bool MULTI>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdParams p) {
  constexpr int JT = MULTI ? 0 : RP / 32;
  constexpr int WROWS = kTileI + 32 * JT;
  constexpr int AROWS = 128 * MS;
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][WROWS * kLP];
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][AROWS * kLP];
  __shared__ float2 lut[256];
  __shared__ float stab[WK == kNF4DQ ? kFwdTab : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles);
  const int tile_n = tile % p.n_tiles, tile_m = tile / p.n_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t n0 = (int64_t)tile_n * kTileI, m0 = (int64_t)tile_m * AROWS;
  const int64_t mw = m0 + wave * 32 * MS;  // this wave's first row
  const int KT = (int)(K / kBK);

  // groups of this tile's rows, for the second-level step table
  const int64_t nlast = (n0 + kTileI < N ? n0 + kTileI : N) - 1;
  const int64_t g_lo = (n0 * K) >> 14;
  if (WK != kDense) build_lut(lut, p.tab);
  if (WK == kNF4DQ) build_steps(stab, p.W, g_lo, (int)(((nlast * K + K - 1) >> 14) - g_lo + 1));

  FwdOffsets o;
  if (WK == kDense) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t n = n0 + (tid >> 3) + 32 * i;
      n = n < N ? n : N - 1;
      o.w[i] = (uint32_t)((n * K + 8 * (tid & 7)) * 2);
    }
  } else {
    int64_t n = n0 + (tid >> 1);
    n = n < N ? n : N - 1;
    const int64_t e = n * K + 32 * (tid & 1);
    o.w[0] = (uint32_t)(e >> 1);
    o.q = (uint32_t)(e >> 6);
    o.e = (uint32_t)e;
  }
#pragma unroll
  for (int i = 0; i < JT; ++i) {
    int j = (tid >> 3) + 32 * i;
    j = j < p.r ? j : p.r - 1;
    o.a[i] = (uint32_t)((j * K + 8 * (tid & 7)) * 2);
  }
  uint32_t xo[4 * MS];
  act_offsets<MS>(xo, K, m0, M);
  const char* xbase = reinterpret_cast<const char*>(p.X);

  f32x16 acc[4][MS];
  f32x16 tacc[JT > 0 ? JT : 1][MS];
  zero_acc(acc);
  zero_acc(tacc);

  FwdStage<WK, JT> s0, s1;
  ActStage<MS> x0, x1;

  fwd_stage_load<WK, JT>(s0, p, o, 0, g_lo);
  act_load<MS>(x0, xbase, xo);
  __syncthreads();  // level and step tables ready
  {
    const float a = WK != kDense ? raw_scale_value<WK>(s0.sc, stab) : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      fwd_stage_part<WK, JT>(s0, wt[0], lut, a, q);
      act_part<MS>(x0, xt[0], q);
    }
  }
  const int64_t kb1 = (int64_t)(KT > 1 ? 1 : 0) * kBK;
  fwd_stage_load<WK, JT>(s1, p, o, kb1, g_lo);
  act_load<MS>(x1, xbase + 2 * kb1, xo);
  __syncthreads();

  // step kt: loads stage kt+2 into (snxt, xnxt), runs the MFMAs of step kt on
  // LDS buffer kt & 1, writes stage kt+1 (scur, xcur) into the other buffer
  auto step = [&](int kt, const FwdStage<WK, JT>& scur, const ActStage<MS>& xcur,
                  FwdStage<WK, JT>& snxt, ActStage<MS>& xnxt) {
    const int64_t k2 = (int64_t)(kt + 2 < KT ? kt + 2 : KT - 1) * kBK;
    fwd_stage_load<WK, JT>(snxt, p, o, k2, g_lo);
    act_load<MS>(xnxt, xbase + 2 * k2, xo);
    const float a = WK != kDense ? raw_scale_value<WK>(scur.sc, stab) : 0.0f;
    const int b = kt & 1;
    uint16_t* wn = wt[b ^ 1];
    uint16_t* xn = xt[b ^ 1];
    mfma_step<MS, JT>(wt[b], xt[b], wave, l32, h, acc, tacc, [&](int q) {
      fwd_stage_part<WK, JT>(scur, wn, lut, a, q);
      act_part<MS>(xcur, xn, q);
    });
    __syncthreads();
  };

  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(kt, s1, x1, s0, x0);
    step(kt + 1, s0, x0, s1, x1);
  }
  if (kt < KT) step(kt, s1, x1, s0, x0);

  // ---------------------------------------------------------------- epilogue
  const int r = p.r;
  if (!MULTI) {
    // T = X A^T for this wave's rows: lane holds T[row l32][32jt + 8q + 4h + i]
    if (p.T_out && tile_n == 0) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int64_t m = mw + 32 * ms + l32;
        if (m < M) {
#pragma unroll
          for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = 32 * jt + 8 * q + 4 * h + i;
                if (j < r) p.T_out[m * r + j] = tacc[jt][ms][4 * q + i];
              }
        }
      }
    }
    const int chunks = (r + 15) >> 4;
#pragma unroll
    for (int c = 0; c < 2 * JT; ++c) {
      if (c < chunks) {
        u32x4 bfr[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          int64_t n = n0 + 32 * ns + l32;
          n = n < N ? n : N - 1;
          const uint16_t* brow = p.B + n * r;
          const u32x2 lo = load4_masked(brow, 16 * c + 4 * h, r);
          const u32x2 hi = load4_masked(brow, 16 * c + 8 + 4 * h, r);
          bfr[ns] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          const u32x4 tb = t_operand(tacc[c >> 1][ms], c & 1, p.s);
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) acc[ns][ms] = mfma32(bfr[ns], tb, acc[ns][ms]);
        }
      }
    }
  } else {
    const int rc = r * p.n_ad;
    const int chunks = (rc + 15) >> 4;
#pragma unroll
    for (int c = 0; c < RP / 16; ++c) {
      if (c < chunks) {
        u32x4 bfr[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          int64_t n = n0 + 32 * ns + l32;
          n = n < N ? n : N - 1;
          uint32_t v[4];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int j0 = 16 * c + 8 * half + 4 * h;
            uint16_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 + i;
              e[i] = 0;
              if (j < rc) {
                const int a = j / r, jj = j - a * r;
                e[i] = p.Bstack[((int64_t)a * N + n) * r + jj];
              }
            }
            v[2 * half] = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
            v[2 * half + 1] = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
          }
          bfr[ns] = u32x4{v[0], v[1], v[2], v[3]};
        }
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          int64_t m = mw + 32 * ms + l32;
          m = m < M ? m : M - 1;
          const uint16_t* trow = p.Tm + m * RP;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(trow + 16 * c + 4 * h);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(trow + 16 * c + 8 + 4 * h);
          const u32x4 tb{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) acc[ns][ms] = mfma32(bfr[ns], tb, acc[ns][ms]);
        }
      }
    }
  }

  // Y[m][n0 + 32ns + 8q + 4h + 0..3] = acc[ns][ms][4q + 0..3]
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int64_t m = mw + 32 * ms + l32;
    if (m >= M) continue;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + 32 * ns + 8 * q + 4 * h;
        if (n < N) {
          const u32x2 o{pack_bf16x2(acc[ns][ms][4 * q], acc[ns][ms][4 * q + 1]),
                        pack_bf16x2(acc[ns][ms][4 * q + 2], acc[ns][ms][4 * q + 3])};
          *reinterpret_cast<u32x2*>(p.Y + m * N + n) = o;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dX

struct BwdParams {
  const uint16_t* dY;  // M x N
  int64_t M;
  WeightArgs W;
  const uint16_t* A;   // r x K
  const uint16_t* B;   // N x r
  int32_t r;
  float s;
  int32_t m_tiles;
  int32_t k_tiles;
  uint16_t* dX;        // M x K
  float* U_out;        // M x r
  NF4Table tab;
};

constexpr int kDxTab = 512;  // second-level steps of one step's 64 x 128 tile (K <= 65536)

// Weight staging for one dX step: W rows n0r .. n0r+63 (reduction) and
// columns k0 .. k0+127 (outputs), stored transposed: tile[k][n].  Thread t
// covers columns k0 + 8 (t & 15) .. +7 of rows n0r + 4 (t >> 4) .. +3 and
// transposes that 4 x 8 patch in registers.  B^T (RP x 64) rides along as
// tile rows 128 ..: its RP 8 x 8 patches (B rows n0r + 8 (t & 7) .., columns
// 8 (t / 8) ..) go to the first RP / 4 lanes of every wave.  The step's
// second-level constants (at most kDxTab groups) are loaded with the stage and
// turned into that stage's step table while the previous step runs.  Offsets
// are per-thread constants; columns past K are clamped (their outputs are
// never stored) and N % 64 == 0 keeps every reduction step full.
template <int WK, int RP>
struct BwdStage {
  uint32_t w[4][WK == kDense ? 4 : 1];
  RawScale sc[WK == kDense ? 1 : 4];
  uint32_t b[8][4];
  float c2[kDxTab / kThreads];
};

struct BwdOffsets {
  uint32_t w[4];   // per patch row: dense byte offset, NF4 code byte offset
  uint32_t q[4];   // NF4: block index of the patch row (relative to the step's first row)
  uint32_t e[4];   // NF4: element index (relative to the step's first row)
  uint32_t b[8];   // B^T patch rows: byte offsets (relative to the step's first row)
  int bt;          // B^T patch index of this lane, or -1
};

template <int RP>
__device__ __forceinline__ int bt_task(int tid) {
  // RP patches: RP / 4 lanes in each of the 4 waves
  const int lane = tid & 63, wave = tid >> 6;
  return lane < RP / 4 ? wave * (RP / 4) + lane : -1;
}

template <int WK, int RP>
__device__ __forceinline__ void bwd_stage_load(BwdStage<WK, RP>& st, const BwdParams& p,
                                               const BwdOffsets& o, int64_t n0r, int64_t k0) {
  const int tid = threadIdx.x;
  const int64_t K = p.W.K;
  const int64_t eb = n0r * K;  // first element of the step's rows
  if (WK == kDense) {
    const char* base = reinterpret_cast<const char*>(p.W.dense + eb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(base + o.w[i]);
#pragma unroll
      for (int d = 0; d < 4; ++d) st.w[i][d] = v[d];
    }
  } else {
    const uint8_t* cb = p.W.codes + (eb >> 1);
    const int64_t g_lo = (eb + k0) >> 14;
    const int64_t elo = eb & 16383;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.w[i][0] = *reinterpret_cast<const uint32_t*>(cb + o.w[i]);
      const int32_t gi = (int32_t)(((elo + o.e[i]) >> 14) - ((elo + k0) >> 14));
      st.sc[i] = load_raw_scale<WK>(p.W.q8 + (eb >> 6), p.W.absmax + (eb >> 6), o.q[i], gi);
    }
    if (WK == kNF4DQ) {
      const int64_t ng = (p.W.N * K + 16383) >> 14;  // number of groups
#pragma unroll
      for (int i = 0; i < kDxTab / kThreads; ++i) {
        const int64_t g = g_lo + tid + kThreads * i;
        st.c2[i] = p.W.c2[g < ng ? g : ng - 1];
      }
    }
  }
  if (o.bt >= 0) {
    const char* base = reinterpret_cast<const char*>(p.B + n0r * p.r);
    const int jb = 8 * (o.bt >> 3);
    const int r = p.r;
    if ((r & 7) == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 v = sel4(jb < r, *reinterpret_cast<const u32x4*>(base + o.b[i]));
#pragma unroll
        for (int d = 0; d < 4; ++d) st.b[i][d] = v[d];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t* row = reinterpret_cast<const uint16_t*>(base + o.b[i]);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int j = jb + 2 * d;
          const uint32_t lo = j < r ? row[j - jb] : 0u;
          const uint32_t hi = j + 1 < r ? row[j + 1 - jb] : 0u;
          st.b[i][d] = lo | (hi << 16);
        }
      }
    }
  }
}

// part (0..3): dequantise row `part` of the weight patch; the last part
// transposes and stores the weight patch and the B^T patch.
template <int WK, int RP>
__device__ __forceinline__ void bwd_stage_part(const BwdStage<WK, RP>& st, uint32_t (&rows)[4][4],
                                               uint16_t* tile, const float2* lut, const float* tab,
                                               int bt, int part) {
  const int tid = threadIdx.x;
  if (WK == kDense) {
#pragma unroll
    for (int d = 0; d < 4; ++d) rows[part][d] = st.w[part][d];
  } else {
    const u32x4 v = deq8(st.w[part][0], raw_scale_value<WK>(st.sc[part], tab), lut);
#pragma unroll
    for (int d = 0; d < 4; ++d) rows[part][d] = v[d];
  }
  if (part == 3) {
    store_transposed<4>(rows, tile + (8 * (tid & 15)) * kLP + 4 * (tid >> 4), kLP);
    if (bt >= 0) store_transposed<8>(st.b, tile + (kTileI + 8 * (bt >> 3)) * kLP + 8 * (bt & 7), kLP);
  }
}

template <int WK, int RP>
__device__ __forceinline__ void bwd_stage_steps(const BwdStage<WK, RP>& st, float* tab) {
  if (WK == kNF4DQ) {
#pragma unroll
    for (int i = 0; i < kDxTab / kThreads; ++i) tab[threadIdx.x + kThreads * i] = dq_step(st.c2[i]);
  }
}

template <int WK, int MS, int RP>
__global__ __launch_bounds__(kThreads) void dx_kernel(BwdParams p) {
  constexpr int JT = RP / 32;
  constexpr int WROWS = kTileI + RP;
  constexpr int AROWS = 128 * MS;
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][WROWS * kLP];
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][AROWS * kLP];
  __shared__ float2 lut[256];
  __shared__ float stab[2][WK == kNF4DQ ? kDxTab : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.k_tiles);
  const int tile_k = tile % p.k_tiles, tile_m = tile / p.k_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t k0 = (int64_t)tile_k * kTileI, m0 = (int64_t)tile_m * AROWS;
  const int64_t mw = m0 + wave * 32 * MS;
  const int RT = (int)(N / kBK);

  if (WK != kDense) build_lut(lut, p.tab);

  BwdOffsets o;
  {
    int64_t k = k0 + 8 * (tid & 15);
    k = k < K ? k : K - 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e = (int64_t)(4 * (tid >> 4) + i) * K + k;  // relative to the step's rows
      o.w[i] = WK == kDense ? (uint32_t)(e * 2) : (uint32_t)(e >> 1);
      o.q[i] = (uint32_t)(e >> 6);
      o.e[i] = (uint32_t)e;
    }
    o.bt = bt_task<RP>(tid);
    const int bt = o.bt < 0 ? 0 : o.bt;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int jb = 8 * (bt >> 3);
      const int jc = jb < p.r ? jb : 0;
      o.b[i] = (uint32_t)(((8 * (bt & 7) + i) * p.r + jc) * 2);
    }
  }
  uint32_t go[4 * MS];
  act_offsets<MS>(go, N, m0, M);
  const char* gbase = reinterpret_cast<const char*>(p.dY);

  f32x16 acc[4][MS];
  f32x16 uacc[JT][MS];
  zero_acc(acc);
  zero_acc(uacc);

  BwdStage<WK, RP> s0, s1;
  ActStage<MS> g0, g1;
  uint32_t rows[4][4];

  // stage s uses step-table slot s & 1
  bwd_stage_load<WK, RP>(s0, p, o, 0, k0);
  act_load<MS>(g0, gbase, go);
  bwd_stage_steps<WK, RP>(s0, stab[0]);
  __syncthreads();  // level table and stage-0 step table ready
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bwd_stage_part<WK, RP>(s0, rows, wt[0], lut, stab[0], o.bt, q);
    act_part<MS>(g0, gt[0], q);
  }
  const int64_t n1 = (int64_t)(RT > 1 ? 1 : 0) * kBK;
  bwd_stage_load<WK, RP>(s1, p, o, n1, k0);
  act_load<MS>(g1, gbase + 2 * n1, go);
  bwd_stage_steps<WK, RP>(s1, stab[1]);
  __syncthreads();

  // step rt: loads stage rt+2 into (snxt, gnxt), runs the MFMAs of step rt on
  // buffer rt & 1, writes stage rt+1 (scur, gcur) into the other buffer and
  // the step table of stage rt+2 into slot rt & 1
  auto step = [&](int rt, const BwdStage<WK, RP>& scur, const ActStage<MS>& gcur,
                  BwdStage<WK, RP>& snxt, ActStage<MS>& gnxt) {
    const int64_t n2 = (int64_t)(rt + 2 < RT ? rt + 2 : RT - 1) * kBK;
    bwd_stage_load<WK, RP>(snxt, p, o, n2, k0);
    act_load<MS>(gnxt, gbase + 2 * n2, go);
    const int b = rt & 1;
    uint16_t* wn = wt[b ^ 1];
    uint16_t* gn = gt[b ^ 1];
    const float* tcur = stab[b ^ 1];
    mfma_step<MS, JT>(wt[b], gt[b], wave, l32, h, acc, uacc, [&](int q) {
      bwd_stage_part<WK, RP>(scur, rows, wn, lut, tcur, o.bt, q);
      act_part<MS>(gcur, gn, q);
      if (q == 3) bwd_stage_steps<WK, RP>(snxt, stab[b]);
    });
    __syncthreads();
  };

  int rt = 0;
  for (; rt + 1 < RT; rt += 2) {
    step(rt, s1, g1, s0, g0);
    step(rt + 1, s0, g0, s1, g1);
  }
  if (rt < RT) step(rt, s1, g1, s0, g0);

  const int r = p.r;
  if (p.U_out && tile_k == 0) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int64_t m = mw + 32 * ms + l32;
      if (m < M) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 32 * jt + 8 * q + 4 * h + i;
              if (j < r) p.U_out[m * r + j] = uacc[jt][ms][4 * q + i];
            }
      }
    }
  }
  // expand: dX^T[k][m] += sum_j A[j][k] (s U[m][j])
  const int chunks = (r + 15) >> 4;
#pragma unroll
  for (int c = 0; c < RP / 16; ++c) {
    if (c < chunks) {
      u32x4 afr[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        int64_t k = k0 + 32 * ks + l32;
        k = k < K ? k : K - 1;
        uint32_t v[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint16_t e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 16 * c + 8 * half + 4 * h + i;
            e[i] = (j < r) ? p.A[(int64_t)j * K + k] : (uint16_t)0;
          }
          v[2 * half] = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
          v[2 * half + 1] = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
        }
        afr[ks] = u32x4{v[0], v[1], v[2], v[3]};
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const u32x4 ub = t_operand(uacc[c >> 1][ms], c & 1, p.s);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[ks][ms] = mfma32(afr[ks], ub, acc[ks][ms]);
      }
    }
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int64_t m = mw + 32 * ms + l32;
    if (m >= M) continue;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + 32 * ks + 8 * q + 4 * h;
        if (k < K) {
          const u32x2 o{pack_bf16x2(acc[ks][ms][4 * q], acc[ks][ms][4 * q + 1]),
                        pack_bf16x2(acc[ks][ms][4 * q + 2], acc[ks][ms][4 * q + 3])};
          *reinterpret_cast<u32x2*>(p.dX + m * K + k) = o;
        }
      }
    }
  }
}

// -------------------------------------------------- multi-adapter helpers

// row_ad[m] = adapter of the segment holding row m.  Offsets are clamped to
// [0, T] so that metadata breaking the documented preconditions cannot write
// outside row_ad.
__global__ void rowmap_kernel(const int32_t* __restrict__ off, const int32_t* __restrict__ ids,
                              int64_t T, int32_t* __restrict__ row_ad) {
  const int seg = blockIdx.x;
  int64_t lo = off[seg], hi = off[seg + 1];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  const int a = ids[seg];
  for (int64_t m = lo + threadIdx.x; m < hi; m += blockDim.x) row_ad[m] = a;
}

// Tm[m][c] = s * sum_k X[m][k] Acat[c][k] if adapter(m) == c / r else 0, for
// c < n_ad * r (Acat = A_stack viewed as (n_ad r) x K), zero up to RP; bf16.
// Each wave takes 32 rows; lane (h, l32) reads row l32, 32 contiguous columns
// per 64-step (the same relabelling of the reduction index on both operands).
template <int RP>
__global__ __launch_bounds__(kThreads) void multi_shrink_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Acat,
    int rc, int r, const int32_t* __restrict__ row_ad, float s, uint16_t* __restrict__ Tm) {
  constexpr int JT = RP / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t mw = ((int64_t)blockIdx.x * 4 + wave) * 32;
  const int64_t m = mw + l32;
  const uint16_t* xrow = X + (m < M ? m : M - 1) * K + 32 * h;
  const uint16_t* arow[JT];
  bool aok[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 32 * jt + l32;
    aok[jt] = j < rc;
    arow[jt] = Acat + (int64_t)(j < rc ? j : 0) * K + 32 * h;
  }
  f32x16 t[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) t[jt][v] = 0.0f;
  for (int64_t kb = 0; kb < K; kb += 64) {
    u32x4 xf[4], af[JT][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xf[q] = *reinterpret_cast<const u32x4*>(xrow + kb + 8 * q);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        af[jt][q] = sel4(aok[jt], *reinterpret_cast<const u32x4*>(arow[jt] + kb + 8 * q));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) t[jt] = mfma32(af[jt][q], xf[q], t[jt]);
  }
  if (m >= M) return;
  const int a = row_ad[m];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = 32 * jt + 8 * q + 4 * h;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + i;
        v[i] = (c < rc && c / r == a) ? s * t[jt][4 * q + i] : 0.0f;
      }
      *reinterpret_cast<u32x2*>(Tm + m * RP + c0) = u32x2{pack_bf16x2(v[0], v[1]),
                                                          pack_bf16x2(v[2], v[3])};
    }
}

// ------------------------------------------------------------ launchers

template <int WK, int MS, int RP, bool MULTI>
int launch_fwd(const FwdParams& p0, hipStream_t st) {
  FwdParams p = p0;
  p.n_tiles = (int)cdiv(p.W.N, kTileI);
  p.m_tiles = (int)cdiv(p.M, 128 * MS);
  const int blocks = p.n_tiles * p.m_tiles;
  hipLaunchKernelGGL((fwd_kernel<WK, MS, RP, MULTI>), dim3(blocks), dim3(kThreads), 0, st, p);
  return hip_fail(hipGetLastError(), "fwd_kernel launch");
}

// two activation m-subtiles per wave (256-row tiles) once there are enough
// rows for every CU, otherwise one
inline bool big_tiles(int64_t M) { return M >= 2048; }

template <int WK, bool MULTI>
int fwd_pick(const FwdParams& p, int rp, hipStream_t st) {
  const bool big = big_tiles(p.M);
  if (rp <= 32)
    return big ? launch_fwd<WK, 2, 32, MULTI>(p, st) : launch_fwd<WK, 1, 32, MULTI>(p, st);
  return big ? launch_fwd<WK, 2, 64, MULTI>(p, st) : launch_fwd<WK, 1, 64, MULTI>(p, st);
}

template <bool MULTI>
int fwd_dispatch(const FwdParams& p, const lq_weight& W, int rp, hipStream_t st) {
  if (W.kind == LQ_WEIGHT_DENSE) return fwd_pick<kDense, MULTI>(p, rp, st);
  if (W.double_quant) return fwd_pick<kNF4DQ, MULTI>(p, rp, st);
  return fwd_pick<kNF4, MULTI>(p, rp, st);
}

template <int WK, int MS, int RP>
int launch_dx(const BwdParams& p0, hipStream_t st) {
  BwdParams p = p0;
  p.k_tiles = (int)cdiv(p.W.K, kTileI);
  p.m_tiles = (int)cdiv(p.M, 128 * MS);
  const int blocks = p.k_tiles * p.m_tiles;
  hipLaunchKernelGGL((dx_kernel<WK, MS, RP>), dim3(blocks), dim3(kThreads), 0, st, p);
  return hip_fail(hipGetLastError(), "dx_kernel launch");
}

template <int WK>
int dx_pick(const BwdParams& p, hipStream_t st) {
  const bool big = big_tiles(p.M);
  if (p.r <= 32) return big ? launch_dx<WK, 2, 32>(p, st) : launch_dx<WK, 1, 32>(p, st);
  return big ? launch_dx<WK, 2, 64>(p, st) : launch_dx<WK, 1, 64>(p, st);
}

}  // namespace

namespace dispatch {

int bf16_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
             int64_t r, float s, void* Y, float* T_out, hipStream_t st) {
  FwdParams p{};
  p.X = (const uint16_t*)X;
  p.M = M;
  p.W = weight_args(W);
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.r = (int32_t)r;
  p.n_ad = 1;
  p.s = s;
  p.Y = (uint16_t*)Y;
  p.T_out = T_out;
  p.tab = nf4_table();
  return fwd_dispatch<false>(p, W, (int)r, st);
}

// dX and U = dY B (written to U_out) in one kernel.
int bf16_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
            int64_t r, float s, void* dX, float* U_out, hipStream_t st) {
  BwdParams p{};
  p.dY = (const uint16_t*)dY;
  p.M = M;
  p.W = weight_args(W);
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.r = (int32_t)r;
  p.s = s;
  p.dX = (uint16_t*)dX;
  p.U_out = U_out;
  p.tab = nf4_table();
  if (W.kind == LQ_WEIGHT_DENSE) return dx_pick<kDense>(p, st);
  if (W.double_quant) return dx_pick<kNF4DQ>(p, st);
  return dx_pick<kNF4>(p, st);
}

size_t multi_ws_bytes(int64_t T_tokens, int64_t r, int32_t n_adapters) {
  const int64_t rp = (r * n_adapters <= 32) ? 32 : 64;
  return (size_t)T_tokens * 4 + (size_t)T_tokens * rp * 2 + 256;
}

int bf16_fwd_multi(const void* X, int64_t T_tokens, const lq_weight& W, const void* A_stack,
                   const void* B_stack, int32_t n_adapters, int64_t r, float s,
                   const int32_t* seg_offsets, const int32_t* seg_adapter, int32_t n_seg, void* Y,
                   void* ws, hipStream_t st) {
  const int rc = (int)(r * n_adapters);
  const int rp = rc <= 32 ? 32 : 64;
  int32_t* row_ad = (int32_t*)ws;
  uintptr_t tm_addr = ((uintptr_t)ws + (size_t)T_tokens * 4 + 255) & ~(uintptr_t)255;
  uint16_t* Tm = (uint16_t*)tm_addr;
  const int64_t K = W.K;
  hipLaunchKernelGGL(rowmap_kernel, dim3(n_seg), dim3(256), 0, st, seg_offsets, seg_adapter,
                     T_tokens, row_ad);
  int e = hip_fail(hipGetLastError(), "rowmap launch");
  if (e) return e;
  const unsigned sblocks = (unsigned)cdiv(T_tokens, 128);
  if (rp == 32)
    hipLaunchKernelGGL(multi_shrink_kernel<32>, dim3(sblocks), dim3(kThreads), 0, st,
                       (const uint16_t*)X, T_tokens, K, (const uint16_t*)A_stack, rc, (int)r,
                       row_ad, s, Tm);
  else
    hipLaunchKernelGGL(multi_shrink_kernel<64>, dim3(sblocks), dim3(kThreads), 0, st,
                       (const uint16_t*)X, T_tokens, K, (const uint16_t*)A_stack, rc, (int)r,
                       row_ad, s, Tm);
  if ((e = hip_fail(hipGetLastError(), "multi shrink launch"))) return e;
  FwdParams p{};
  p.X = (const uint16_t*)X;
  p.M = T_tokens;
  p.W = weight_args(W);
  p.Tm = Tm;
  p.Bstack = (const uint16_t*)B_stack;
  p.r = (int32_t)r;
  p.n_ad = n_adapters;
  p.s = s;
  p.Y = (uint16_t*)Y;
  p.tab = nf4_table();
  return fwd_dispatch<true>(p, W, rp, st);
}

}  // namespace dispatch
}  // namespace lq

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
// forward, k for dX) and 128 * MS activation rows.  Each reduction step of 64
// the whole workgroup stages the weight tile into LDS -- dequantising NF4
// codes through a byte-indexed level table, and for dX transposing it so the
// reduction index (n) is contiguous -- while each wave streams its own
// activation rows straight from global memory into MFMA registers.  So every
// weight element is dequantised once per 128 * MS activation rows, and the
// activations never pass through LDS.  Weight tiles are double-buffered: one
// barrier per step.
//
// The LoRA branch is fused: the rank-r shrink (X A^T, or dY B) runs in the
// same reduction loop on the activation registers already loaded (r padded to
// 32 or 64 rows of MFMA), and the expand (. B^T, or . A) runs in the epilogue
// on the finished accumulators, with s folded into the bf16 rounding of T.
// The output tile is computed transposed (weight side = MFMA rows), so each
// lane ends up holding four consecutive outputs of one row and stores 8 bytes.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileI = 128;  // weight-side outputs per workgroup

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

// Weight-side staging for the forward: rows n0 .. n0+127, columns k0 .. k0+63.
template <int WK>
struct FwdStage {
  // WK == 0: dense bf16, four 16-byte chunks per thread
  // WK == 1: NF4, 16 code bytes (32 weights, half a block) per thread
  u32x4 raw[WK == 0 ? 4 : 1];
  float a;
};

template <int WK>
__device__ __forceinline__ void fwd_stage_load(FwdStage<WK>& st, const FwdParams& p, int64_t n0,
                                               int64_t k0, ScaleCache& sc) {
  const int tid = threadIdx.x;
  const int64_t N = p.W.N, K = p.W.K;
  if (WK == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int64_t n = n0 + (c >> 3);
      if (n < N)
        st.raw[i] = *reinterpret_cast<const u32x4*>(p.W.dense + n * K + k0 + 8 * (c & 7));
      else
        st.raw[i] = u32x4{0, 0, 0, 0};
    }
  } else {
    const int64_t n = n0 + (tid >> 1);
    if (n < N) {
      const int64_t e = n * K + k0 + 32 * (tid & 1);
      st.raw[0] = *reinterpret_cast<const u32x4*>(p.W.codes + (e >> 1));
      st.a = sc.scale(p.W, e >> 6);
    } else {
      st.raw[0] = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      st.a = 0.0f;
    }
  }
}

template <int WK>
__device__ __forceinline__ void fwd_stage_store(const FwdStage<WK>& st, uint16_t* wl,
                                                const float2* lut) {
  const int tid = threadIdx.x;
  if (WK == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(wl + (c >> 3) * kPitch + 8 * (c & 7)) = st.raw[i];
    }
  } else {
    uint16_t* dst = wl + (tid >> 1) * kPitch + 32 * (tid & 1);
#pragma unroll
    for (int d = 0; d < 4; ++d)
      *reinterpret_cast<u32x4*>(dst + 8 * d) = deq8(st.raw[0][d], st.a, lut);
  }
}

// Activation fragments: lane (h, l32) of a wave holds row l32 of each of its
// m-subtiles, reduction elements k0 + 32h + 8s .. +7 for substep s.
template <int MS>
__device__ __forceinline__ void load_act(u32x4 (&f)[MS][4], const uint16_t* base, int64_t ld,
                                         int64_t row0, int64_t rows, int64_t col0, int64_t cols,
                                         int lane) {
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    int64_t row = row0 + 32 * ms + l32;
    const bool ok = row < rows;
    row = ok ? row : rows - 1;
    const uint16_t* src = base + row * ld + col0 + 32 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool cok = ok && (col0 + 32 * h + 8 * s < cols);
      f[ms][s] = cok ? *reinterpret_cast<const u32x4*>(src + 8 * s) : u32x4{0, 0, 0, 0};
    }
  }
}

// Rows of A (r x K) as MFMA A-operand rows j = 32 jt + l32 (zero past r).
template <int JT>
__device__ __forceinline__ void load_a_rows(u32x4 (&f)[JT][4], const uint16_t* A, int64_t K,
                                            int r, int64_t k0, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 32 * jt + l32;
    const uint16_t* src = A + (int64_t)j * K + k0 + 32 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      f[jt][s] = (j < r) ? *reinterpret_cast<const u32x4*>(src + 8 * s) : u32x4{0, 0, 0, 0};
  }
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

template <int WK, int MS, int RP, bool MULTI>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdParams p) {
  constexpr int JT = RP / 32;
  constexpr int BJ = 4 * 32 * MS;
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][kTileI * kPitch];
  __shared__ float2 lut[256];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles);
  const int tile_n = tile % p.n_tiles, tile_m = tile / p.n_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t n0 = (int64_t)tile_n * kTileI, m0 = (int64_t)tile_m * BJ;
  const int64_t mw = m0 + wave * 32 * MS;  // this wave's first row
  const int KT = (int)(K / 64);

  if (WK != 0) build_lut(lut, p.tab);

  f32x16 acc[4][MS];
  f32x16 tacc[JT][MS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][ms][v] = 0.0f;
#pragma unroll
  for (int i = 0; i < JT; ++i)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) tacc[i][ms][v] = 0.0f;

  ScaleCache sc;
  sc.init();
  FwdStage<WK> st;
  u32x4 xf[MS][4], xn[MS][4];
  u32x4 af[JT][4], an[JT][4];

  fwd_stage_load<WK>(st, p, n0, 0, sc);
  load_act<MS>(xf, p.X, K, mw, M, 0, K, lane);
  if (!MULTI) load_a_rows<JT>(af, p.A, K, p.r, 0, lane);
  __syncthreads();  // LUT ready
  fwd_stage_store<WK>(st, wl[0], lut);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    const int64_t k1 = (int64_t)(kt + 1) * 64;
    if (more) {
      fwd_stage_load<WK>(st, p, n0, k1, sc);
      load_act<MS>(xn, p.X, K, mw, M, k1, K, lane);
      if (!MULTI) load_a_rows<JT>(an, p.A, K, p.r, k1, lane);
    }
    const uint16_t* w = wl[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 wf[4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
        wf[ns] = *reinterpret_cast<const u32x4*>(w + (32 * ns + l32) * kPitch + 32 * h + 8 * s);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) acc[ns][ms] = mfma32(wf[ns], xf[ms][s], acc[ns][ms]);
      if (!MULTI) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) tacc[jt][ms] = mfma32(af[jt][s], xf[ms][s], tacc[jt][ms]);
      }
    }
    if (more) fwd_stage_store<WK>(st, wl[buf ^ 1], lut);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s) xf[ms][s] = xn[ms][s];
      if (!MULTI) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
          for (int s = 0; s < 4; ++s) af[jt][s] = an[jt][s];
      }
    }
  }

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
    for (int c = 0; c < RP / 16; ++c) {
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

// Weight-side staging for dX: rows n0r .. n0r+63 (reduction), columns
// k0 .. k0+127 (outputs), written transposed: wt[k][n].  Thread t covers
// columns k0 + 8 (t & 15) .. +7 of rows n0r + 4 (t >> 4) .. +3.
template <int WK>
struct BwdStage {
  uint32_t raw[WK == 0 ? 16 : 4];
  float a[WK == 0 ? 1 : 4];
};

template <int WK>
__device__ __forceinline__ void bwd_stage_load(BwdStage<WK>& st, const BwdParams& p, int64_t n0r,
                                               int64_t k0, ScaleCache& sc) {
  const int tid = threadIdx.x;
  const int64_t N = p.W.N, K = p.W.K;
  const int64_t k = k0 + 8 * (tid & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0r + 4 * (tid >> 4) + i;
    const bool ok = n < N && k < K;
    if (WK == 0) {
      u32x4 v = ok ? *reinterpret_cast<const u32x4*>(p.W.dense + n * K + k) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int d = 0; d < 4; ++d) st.raw[4 * i + d] = v[d];
    } else {
      const int64_t e = n * K + k;
      st.raw[i] = ok ? *reinterpret_cast<const uint32_t*>(p.W.codes + (e >> 1)) : 0x77777777u;
      st.a[i] = ok ? sc.scale(p.W, e >> 6) : 0.0f;
    }
  }
}

template <int WK>
__device__ __forceinline__ void bwd_stage_store(const BwdStage<WK>& st, uint16_t* wt,
                                                const float2* lut) {
  const int tid = threadIdx.x;
  uint32_t row[4][4];  // [n][dword]: dword d holds k = 2d, 2d + 1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (WK == 0) {
#pragma unroll
      for (int d = 0; d < 4; ++d) row[i][d] = st.raw[4 * i + d];
    } else {
      const u32x4 v = deq8(st.raw[i], st.a[i], lut);
#pragma unroll
      for (int d = 0; d < 4; ++d) row[i][d] = v[d];
    }
  }
  const int kc = tid & 15, ng = tid >> 4;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // column k = 2d: (row0, row1), (row2, row3)
    const u32x2 ev{pair_lo(row[0][d], row[1][d]), pair_lo(row[2][d], row[3][d])};
    const u32x2 od{pair_hi(row[0][d], row[1][d]), pair_hi(row[2][d], row[3][d])};
    *reinterpret_cast<u32x2*>(wt + (8 * kc + 2 * d) * kPitch + 4 * ng) = ev;
    *reinterpret_cast<u32x2*>(wt + (8 * kc + 2 * d + 1) * kPitch + 4 * ng) = od;
  }
}

// B^T tile for the shrink U = dY B: bt[j][n] = B[n0r + n][j], rows j >= r zero.
template <int RP>
__device__ __forceinline__ void stage_bt(uint16_t* bt, const uint16_t* B, int64_t N, int r,
                                         int64_t n0r) {
  for (int e = threadIdx.x; e < 64 * RP; e += kThreads) {
    const int n = e / RP, j = e - n * RP;
    uint16_t v = 0;
    if (j < r && n0r + n < N) v = B[(n0r + n) * r + j];
    bt[j * kPitch + n] = v;
  }
}

template <int WK, int MS, int RP>
__global__ __launch_bounds__(kThreads) void dx_kernel(BwdParams p) {
  constexpr int JT = RP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][kTileI * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t bt[2][RP * kPitch];
  __shared__ float2 lut[256];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.k_tiles);
  const int tile_k = tile % p.k_tiles, tile_m = tile / p.k_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t k0 = (int64_t)tile_k * kTileI, m0 = (int64_t)tile_m * (128 * MS);
  const int64_t mw = m0 + wave * 32 * MS;
  const int RT = (int)((N + 63) / 64);

  if (WK != 0) build_lut(lut, p.tab);

  f32x16 acc[4][MS];
  f32x16 uacc[JT][MS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][ms][v] = 0.0f;
#pragma unroll
  for (int i = 0; i < JT; ++i)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) uacc[i][ms][v] = 0.0f;

  ScaleCache sc;
  sc.init();
  BwdStage<WK> st;
  u32x4 gf[MS][4], gn[MS][4];

  bwd_stage_load<WK>(st, p, 0, k0, sc);
  load_act<MS>(gf, p.dY, N, mw, M, 0, N, lane);
  stage_bt<RP>(bt[0], p.B, N, p.r, 0);
  __syncthreads();  // LUT ready
  bwd_stage_store<WK>(st, wt[0], lut);
  __syncthreads();

  for (int rt = 0; rt < RT; ++rt) {
    const int buf = rt & 1;
    const bool more = rt + 1 < RT;
    const int64_t n1 = (int64_t)(rt + 1) * 64;
    if (more) {
      bwd_stage_load<WK>(st, p, n1, k0, sc);
      load_act<MS>(gn, p.dY, N, mw, M, n1, N, lane);
    }
    const uint16_t* w = wt[buf];
    const uint16_t* b = bt[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 wf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        wf[ks] = *reinterpret_cast<const u32x4*>(w + (32 * ks + l32) * kPitch + 32 * h + 8 * s);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) acc[ks][ms] = mfma32(wf[ks], gf[ms][s], acc[ks][ms]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 bf =
            *reinterpret_cast<const u32x4*>(b + (32 * jt + l32) * kPitch + 32 * h + 8 * s);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) uacc[jt][ms] = mfma32(bf, gf[ms][s], uacc[jt][ms]);
      }
    }
    if (more) {
      bwd_stage_store<WK>(st, wt[buf ^ 1], lut);
      stage_bt<RP>(bt[buf ^ 1], p.B, N, p.r, n1);
    }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s) gf[ms][s] = gn[ms][s];
    }
  }

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

// row_ad[m] = adapter of the segment holding row m.
// Offsets are clamped to [0, T] so that metadata breaking the documented
// preconditions cannot write outside row_ad.
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
template <int RP>
__global__ __launch_bounds__(kThreads) void multi_shrink_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Acat,
    int rc, int r, const int32_t* __restrict__ row_ad, float s, uint16_t* __restrict__ Tm) {
  constexpr int JT = RP / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t mw = ((int64_t)blockIdx.x * 4 + wave) * 32;
  f32x16 t[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) t[jt][v] = 0.0f;
  u32x4 xf[1][4], af[JT][4];
  for (int64_t k0 = 0; k0 < K; k0 += 64) {
    load_act<1>(xf, X, K, mw, M, k0, K, lane);
    load_a_rows<JT>(af, Acat, K, rc, k0, lane);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) t[jt] = mfma32(af[jt][s4], xf[0][s4], t[jt]);
  }
  const int64_t m = mw + l32;
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

template <int WK, bool MULTI>
int fwd_pick(const FwdParams& p, int rp, hipStream_t st) {
  // two activation m-subtiles per wave when there are enough rows to keep
  // every CU busy with 256-row tiles, otherwise one
  const bool big = p.M >= 2048;
  if (rp <= 32) {
    return big ? launch_fwd<WK, 2, 32, MULTI>(p, st) : launch_fwd<WK, 1, 32, MULTI>(p, st);
  }
  return big ? launch_fwd<WK, 2, 64, MULTI>(p, st) : launch_fwd<WK, 1, 64, MULTI>(p, st);
}

template <bool MULTI>
int fwd_dispatch(const FwdParams& p, const lq_weight& W, int rp, hipStream_t st) {
  if (W.kind == LQ_WEIGHT_DENSE) return fwd_pick<0, MULTI>(p, rp, st);
  return fwd_pick<1, MULTI>(p, rp, st);
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
  const bool big = p.M >= 2048;
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
  if (W.kind == LQ_WEIGHT_DENSE) return dx_pick<0>(p, st);
  return dx_pick<1>(p, st);
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

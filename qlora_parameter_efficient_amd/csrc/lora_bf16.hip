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
constexpr int kBK = 128;      // reduction elements per step
constexpr int kLP = kBK + 8;  // LDS row pitch (bf16): 272 bytes, conflict-free 16-byte reads

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

// 8 x 8 bf16 patch, rows[i][d] = elements (2d, 2d+1) of row i, stored
// transposed: output row c holds element c of rows 0..7 (16 bytes).
__device__ __forceinline__ void store_transposed8(const uint32_t (&rows)[8][4], uint16_t* dst,
                                                  int pitch) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 ev{pair_lo(rows[0][d], rows[1][d]), pair_lo(rows[2][d], rows[3][d]),
                   pair_lo(rows[4][d], rows[5][d]), pair_lo(rows[6][d], rows[7][d])};
    const u32x4 od{pair_hi(rows[0][d], rows[1][d]), pair_hi(rows[2][d], rows[3][d]),
                   pair_hi(rows[4][d], rows[5][d]), pair_hi(rows[6][d], rows[7][d])};
    *reinterpret_cast<u32x4*>(dst + (2 * d) * pitch) = ev;
    *reinterpret_cast<u32x4*>(dst + (2 * d + 1) * pitch) = od;
  }
}

// Activation fragments of one step for a wave: for each m-subtile, lane
// (h, l32) holds row l32, reduction elements kb + 64 h + 8 sg .. +7 for
// substeps sg = 0..7 (one contiguous 128-byte run per lane).
template <int MS>
struct ActRegs {
  u32x4 f[MS][8];
};

template <int MS>
__device__ __forceinline__ void load_act(ActRegs<MS>& a, const uint16_t* const (&rowp)[MS],
                                         int64_t kb, int64_t kmax, int h) {
  const int64_t k = kb + 64 * h;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
    for (int sg = 0; sg < 8; ++sg) {
      const bool ok = k + 8 * sg < kmax;
      const int64_t kk = ok ? k + 8 * sg : 0;
      a.f[ms][sg] = sel4(ok, *reinterpret_cast<const u32x4*>(rowp[ms] + kk));
    }
  }
}

// One MFMA step over the tile in LDS: 4 weight-side subtiles (rows 32 ns + l32)
// plus JT shrink subtiles (tile rows 128 + 32 jt + l32), against the MS
// activation subtiles.  LDS fragment reads run one substep ahead; after the
// MFMAs of substep sg, part(sg) stores one eighth of the next tile.
template <int MS, int JT, typename Part>
__device__ __forceinline__ void mfma_step(const uint16_t* tile, int l32, int h,
                                          const ActRegs<MS>& cur, f32x16 (&acc)[4][MS],
                                          f32x16 (&tacc)[JT > 0 ? JT : 1][MS], Part&& part) {
  constexpr int NR = 4 + JT;
  const uint16_t* wbase = tile + l32 * kLP + 64 * h;
  u32x4 wf[2][NR];
#pragma unroll
  for (int ns = 0; ns < NR; ++ns) wf[0][ns] = *reinterpret_cast<const u32x4*>(wbase + 32 * ns * kLP);
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) {
    const int c = sg & 1;
    if (sg < 7) {
#pragma unroll
      for (int ns = 0; ns < NR; ++ns)
        wf[c ^ 1][ns] = *reinterpret_cast<const u32x4*>(wbase + 32 * ns * kLP + 8 * (sg + 1));
    }
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[ns][ms] = mfma32(wf[c][ns], cur.f[ms][sg], acc[ns][ms]);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        tacc[jt][ms] = mfma32(wf[c][4 + jt], cur.f[ms][sg], tacc[jt][ms]);
    part(sg);
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

// Staging for one forward step: weight rows n0 .. n0+127, columns kb .. kb+127.
// NF4: thread t takes row t/2, one whole 64-element block (32 code bytes).
// Dense: thread t takes eight 16-byte chunks.  The JT = RP/32 shrink operand
// tiles (A rows, RP x 128) ride along as tile rows 128 ...  Stages are loaded
// two steps ahead and written to LDS one eighth per MFMA substep.
template <int WK, int JT>
struct FwdStage {
  u32x4 w[WK == 0 ? 8 : 2];
  ScaleRef sr;
  bool wok;
  u32x4 a[JT > 0 ? 2 * JT : 1];
};

template <int WK, int JT>
__device__ __forceinline__ void fwd_stage_load(FwdStage<WK, JT>& st, const FwdParams& p,
                                               int64_t n0, int64_t kb, int64_t g_lo) {
  const int tid = threadIdx.x;
  const int64_t N = p.W.N, K = p.W.K;
  if (WK == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i;
      const int64_t n = n0 + (c >> 4), k = kb + 8 * (c & 15);
      const bool ok = n < N && k < K;
      const int64_t nn = n < N ? n : N - 1, kk = k < K ? k : 0;
      st.w[i] = sel4(ok, *reinterpret_cast<const u32x4*>(p.W.dense + nn * K + kk));
    }
  } else {
    const int64_t n = n0 + (tid >> 1), k = kb + 64 * (tid & 1);
    st.wok = n < N && k < K;
    const int64_t e = (n < N ? n : N - 1) * K + (k < K ? k : 0);
    const u32x4* src = reinterpret_cast<const u32x4*>(p.W.codes + (e >> 1));
    st.w[0] = src[0];
    st.w[1] = src[1];
    st.sr = load_scale_ref(p.W, e >> 6, g_lo);
  }
#pragma unroll
  for (int i = 0; i < 2 * JT; ++i) {
    const int c = tid + kThreads * i;
    const int j = c >> 4;
    const int64_t k = kb + 8 * (c & 15);
    const bool ok = j < p.r && k < K;
    const int jj = j < p.r ? j : 0;
    const int64_t kk = k < K ? k : 0;
    st.a[i] = sel4(ok, *reinterpret_cast<const u32x4*>(p.A + (int64_t)jj * K + kk));
  }
}

// part sg (0..7) of writing a staged forward tile; a = the thread's block scale
template <int WK, int JT>
__device__ __forceinline__ void fwd_stage_part(const FwdStage<WK, JT>& st, uint16_t* tile,
                                               const float2* lut, float a, int sg) {
  const int tid = threadIdx.x;
  if (WK == 0) {
    const int c = tid + kThreads * sg;
    *reinterpret_cast<u32x4*>(tile + (c >> 4) * kLP + 8 * (c & 15)) = st.w[sg];
  } else {
    const u32x4 v = deq8(st.w[sg >> 2][sg & 3], a, lut);
    *reinterpret_cast<u32x4*>(tile + (tid >> 1) * kLP + 64 * (tid & 1) + 8 * sg) = sel4(st.wok, v);
  }
  if (sg < 2 * JT) {
    const int c = tid + kThreads * sg;
    *reinterpret_cast<u32x4*>(tile + (kTileI + (c >> 4)) * kLP + 8 * (c & 15)) = st.a[sg];
  }
}

template <int WK, int MS, int RP, bool MULTI>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdParams p) {
  constexpr int JT = MULTI ? 0 : RP / 32;
  constexpr int ROWS = kTileI + 32 * JT;
  __shared__ __attribute__((aligned(16))) uint16_t tl[2][ROWS * kLP];
  __shared__ float2 lut[256];
  __shared__ float stab[WK != 0 ? kFwdTab : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.n_tiles);
  const int tile_n = tile % p.n_tiles, tile_m = tile / p.n_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t n0 = (int64_t)tile_n * kTileI, m0 = (int64_t)tile_m * (128 * MS);
  const int64_t mw = m0 + wave * 32 * MS;  // this wave's first row
  const int KT = (int)((K + kBK - 1) / kBK);

  // groups of this tile's rows, for the second-level step table
  const int64_t nlast = (n0 + kTileI < N ? n0 + kTileI : N) - 1;
  const int64_t g_lo = (n0 * K) >> 14;
  if (WK != 0) {
    build_lut(lut, p.tab);
    if (p.W.dq) build_steps(stab, p.W, g_lo, (int)(((nlast * K + K - 1) >> 14) - g_lo + 1));
  }

  f32x16 acc[4][MS];
  f32x16 tacc[JT > 0 ? JT : 1][MS];
  zero_acc(acc);
  zero_acc(tacc);

  const uint16_t* xrow[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int64_t m = mw + 32 * ms + l32;
    xrow[ms] = p.X + (m < M ? m : M - 1) * K;
  }

  FwdStage<WK, JT> s0, s1;
  ActRegs<MS> xa, xb;

  fwd_stage_load<WK, JT>(s0, p, n0, 0, g_lo);
  load_act<MS>(xa, xrow, 0, K, h);
  __syncthreads();  // level and step tables ready
  {
    const float a = WK != 0 ? scale_from(p.W, s0.sr, stab) : 0.0f;
#pragma unroll
    for (int sg = 0; sg < 8; ++sg) fwd_stage_part<WK, JT>(s0, tl[0], lut, a, sg);
  }
  fwd_stage_load<WK, JT>(s1, p, n0, (KT > 1 ? 1 : 0) * (int64_t)kBK, g_lo);
  __syncthreads();

  // step kt: loads stage kt+2 into snxt and activations kt+1 into nxt, runs
  // the MFMAs of step kt, writes stage kt+1 (scur) into the other buffer
  auto step = [&](int kt, const ActRegs<MS>& cur, ActRegs<MS>& nxt, const FwdStage<WK, JT>& scur,
                  FwdStage<WK, JT>& snxt) {
    const int64_t k1 = (int64_t)(kt + 1 < KT ? kt + 1 : KT - 1) * kBK;
    const int64_t k2 = (int64_t)(kt + 2 < KT ? kt + 2 : KT - 1) * kBK;
    fwd_stage_load<WK, JT>(snxt, p, n0, k2, g_lo);
    load_act<MS>(nxt, xrow, k1, K, h);
    const float a = WK != 0 ? scale_from(p.W, scur.sr, stab) : 0.0f;
    uint16_t* nt = tl[(kt & 1) ^ 1];
    mfma_step<MS, JT>(tl[kt & 1], l32, h, cur, acc, tacc,
                      [&](int sg) { fwd_stage_part<WK, JT>(scur, nt, lut, a, sg); });
    __syncthreads();
  };

  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(kt, xa, xb, s1, s0);
    step(kt + 1, xb, xa, s0, s1);
  }
  if (kt < KT) step(kt, xa, xb, s1, s0);

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

constexpr int kDxTab = 1024;  // second-level steps of one step's 128 x 128 tile (K <= 65536)

// Staging for one dX step: W rows n0r .. n0r+127 (reduction) and columns
// k0 .. k0+127 (outputs), stored transposed: tile[k][n].  Thread t covers
// columns k0 + 8 (t & 15) .. +7 of rows n0r + 8 (t >> 4) .. +7 and transposes
// that 8 x 8 patch in registers.  B^T (RP x 128) rides along as tile rows
// 128 ..: thread t < 2 RP takes B rows n0r + 8 (t & 15) .. +7, columns
// 8 (t >> 4) .. +7 (zero past r), transposed the same way.  The step's
// second-level constants (at most kDxTab groups) are loaded with the stage and
// turned into the step table of its LDS slot while the previous step runs.
template <int WK, int RP>
struct BwdStage {
  uint32_t w[8][WK == 0 ? 4 : 1];
  ScaleRef sr[WK == 0 ? 1 : 8];
  bool ok[8];
  uint32_t b[8][4];
  float c2[WK == 0 ? 1 : kDxTab / kThreads];
};

__device__ __forceinline__ int64_t dx_group_base(int64_t n0r, int64_t k0, int64_t K) {
  return (n0r * K + k0) >> 14;
}

template <int WK, int RP>
__device__ __forceinline__ void bwd_stage_load(BwdStage<WK, RP>& st, const BwdParams& p,
                                               int64_t n0r, int64_t k0) {
  const int tid = threadIdx.x;
  const int64_t N = p.W.N, K = p.W.K;
  const int64_t k = k0 + 8 * (tid & 15);
  const int64_t kk = k < K ? k : K - 8;  // stays at or after k0, so groups stay >= g_lo
  const int64_t g_lo = dx_group_base(n0r, k0, K);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0r + 8 * (tid >> 4) + i;
    st.ok[i] = n < N && k < K;
    const int64_t nn = n < N ? n : N - 1;
    if (WK == 0) {
      const u32x4 v = sel4(st.ok[i], *reinterpret_cast<const u32x4*>(p.W.dense + nn * K + kk));
#pragma unroll
      for (int d = 0; d < 4; ++d) st.w[i][d] = v[d];
    } else {
      const int64_t e = nn * K + kk;
      st.w[i][0] = *reinterpret_cast<const uint32_t*>(p.W.codes + (e >> 1));
      st.sr[i] = load_scale_ref(p.W, e >> 6, g_lo);
    }
  }
  if (WK != 0 && p.W.dq) {
    const int64_t ng = (N * K + 16383) >> 14;  // number of groups
#pragma unroll
    for (int i = 0; i < kDxTab / kThreads; ++i) {
      const int64_t g = g_lo + tid + kThreads * i;
      st.c2[i] = p.W.c2[g < ng ? g : ng - 1];
    }
  }
  const int jb = 8 * (tid >> 4);
  if (jb < RP) {
    const int r = p.r;
    const bool vec = (r & 7) == 0 && jb + 8 <= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = n0r + 8 * (tid & 15) + i;
      const bool nok = n < N;
      const uint16_t* row = p.B + (nok ? n : N - 1) * r;
      if (vec) {
        const u32x4 q = sel4(nok, *reinterpret_cast<const u32x4*>(row + jb));
#pragma unroll
        for (int d = 0; d < 4; ++d) st.b[i][d] = q[d];
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int j = jb + 2 * d;
          const uint32_t lo = (nok && j < r) ? row[j] : 0u;
          const uint32_t hi = (nok && j + 1 < r) ? row[j + 1] : 0u;
          st.b[i][d] = lo | (hi << 16);
        }
      }
    }
  }
}

// second-level step table of a loaded stage (written by every thread)
template <int WK, int RP>
__device__ __forceinline__ void bwd_stage_steps(const BwdStage<WK, RP>& st, float* tab) {
  if (WK != 0) {
#pragma unroll
    for (int i = 0; i < kDxTab / kThreads; ++i) tab[threadIdx.x + kThreads * i] = dq_step(st.c2[i]);
  }
}

// part sg (0..7): dequantise row sg of the patch; the last part transposes and
// stores the weight patch and the B^T patch.
template <int WK, int RP>
__device__ __forceinline__ void bwd_stage_part(const BwdStage<WK, RP>& st, uint32_t (&rows)[8][4],
                                               uint16_t* tile, const float2* lut,
                                               const WeightArgs& w, const float* tab, int sg) {
  const int tid = threadIdx.x;
  if (WK == 0) {
#pragma unroll
    for (int d = 0; d < 4; ++d) rows[sg][d] = st.w[sg][d];
  } else {
    const float a = scale_from(w, st.sr[sg], tab);
    const u32x4 v = sel4(st.ok[sg], deq8(st.w[sg][0], a, lut));
#pragma unroll
    for (int d = 0; d < 4; ++d) rows[sg][d] = v[d];
  }
  if (sg == 7) {
    store_transposed8(rows, tile + (8 * (tid & 15)) * kLP + 8 * (tid >> 4), kLP);
    const int jb = 8 * (tid >> 4);
    if (jb < RP) store_transposed8(st.b, tile + (kTileI + jb) * kLP + 8 * (tid & 15), kLP);
  }
}

template <int WK, int MS, int RP>
__global__ __launch_bounds__(kThreads) void dx_kernel(BwdParams p) {
  constexpr int JT = RP / 32;
  constexpr int ROWS = kTileI + RP;
  __shared__ __attribute__((aligned(16))) uint16_t tl[2][ROWS * kLP];
  __shared__ float2 lut[256];
  __shared__ float stab[2][WK != 0 ? kDxTab : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.k_tiles);
  const int tile_k = tile % p.k_tiles, tile_m = tile / p.k_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t k0 = (int64_t)tile_k * kTileI, m0 = (int64_t)tile_m * (128 * MS);
  const int64_t mw = m0 + wave * 32 * MS;
  const int RT = (int)((N + kBK - 1) / kBK);

  if (WK != 0) build_lut(lut, p.tab);

  f32x16 acc[4][MS];
  f32x16 uacc[JT][MS];
  zero_acc(acc);
  zero_acc(uacc);

  const uint16_t* grow[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int64_t m = mw + 32 * ms + l32;
    grow[ms] = p.dY + (m < M ? m : M - 1) * N;
  }

  BwdStage<WK, RP> s0, s1;
  ActRegs<MS> ga, gb;
  uint32_t rows[8][4];

  // stage s uses step-table slot s & 1
  bwd_stage_load<WK, RP>(s0, p, 0, k0);
  load_act<MS>(ga, grow, 0, N, h);
  bwd_stage_steps<WK, RP>(s0, stab[0]);
  __syncthreads();  // level table and stage-0 step table ready
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) bwd_stage_part<WK, RP>(s0, rows, tl[0], lut, p.W, stab[0], sg);
  bwd_stage_load<WK, RP>(s1, p, (RT > 1 ? 1 : 0) * (int64_t)kBK, k0);
  bwd_stage_steps<WK, RP>(s1, stab[1]);
  __syncthreads();

  // step rt: loads stage rt+2 into snxt and activations rt+1 into nxt, runs
  // the MFMAs of step rt, writes stage rt+1 (scur) into the other buffer and
  // the step table of stage rt+2 into slot (rt+2) & 1 = rt & 1
  auto step = [&](int rt, const ActRegs<MS>& cur, ActRegs<MS>& nxt, const BwdStage<WK, RP>& scur,
                  BwdStage<WK, RP>& snxt) {
    const int64_t n1 = (int64_t)(rt + 1 < RT ? rt + 1 : RT - 1) * kBK;
    const int64_t n2 = (int64_t)(rt + 2 < RT ? rt + 2 : RT - 1) * kBK;
    bwd_stage_load<WK, RP>(snxt, p, n2, k0);
    load_act<MS>(nxt, grow, n1, N, h);
    uint16_t* nt = tl[(rt & 1) ^ 1];
    const float* tcur = stab[(rt & 1) ^ 1];
    mfma_step<MS, JT>(tl[rt & 1], l32, h, cur, acc, uacc, [&](int sg) {
      bwd_stage_part<WK, RP>(scur, rows, nt, lut, p.W, tcur, sg);
      if (sg == 7) bwd_stage_steps<WK, RP>(snxt, stab[rt & 1]);
    });
    __syncthreads();
  };

  int rt = 0;
  for (; rt + 1 < RT; rt += 2) {
    step(rt, ga, gb, s1, s0);
    step(rt + 1, gb, ga, s0, s1);
  }
  if (rt < RT) step(rt, ga, gb, s1, s0);

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
// Each wave takes 32 rows; A_stack rows are read straight from L2.
template <int RP>
__global__ __launch_bounds__(kThreads) void multi_shrink_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Acat,
    int rc, int r, const int32_t* __restrict__ row_ad, float s, uint16_t* __restrict__ Tm) {
  constexpr int JT = RP / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t mw = ((int64_t)blockIdx.x * 4 + wave) * 32;
  const int64_t m = mw + l32;
  const uint16_t* xrow[1] = {X + (m < M ? m : M - 1) * K};
  const uint16_t* arow[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 32 * jt + l32;
    arow[jt] = Acat + (int64_t)(j < rc ? j : 0) * K;
  }
  f32x16 t[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) t[jt][v] = 0.0f;
  for (int64_t kb = 0; kb < K; kb += kBK) {
    ActRegs<1> xf;
    load_act<1>(xf, xrow, kb, K, h);
    ActRegs<JT> af;
    load_act<JT>(af, arow, kb, K, h);
#pragma unroll
    for (int sg = 0; sg < 8; ++sg)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const bool jok = 32 * jt + l32 < rc;
        t[jt] = mfma32(sel4(jok, af.f[jt][sg]), xf.f[0][sg], t[jt]);
      }
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

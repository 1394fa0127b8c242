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
// 32 MS w .. +32 MS.  The reduction runs in steps of 64.  Each step the whole
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
// into staging registers), run the 4 MFMA substeps on the current LDS tile
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

// Activation fragments of one step loaded straight into MFMA operand
// registers: lane (h, l32) of wave w takes row mw + 32 ms + l32 (clamped; its
// outputs are never stored) and the reduction elements kb + 32 h .. +31, one
// 16-byte fragment per substep (the same labels as the weight tile reads).
template <int MS>
struct FragStage {
  u32x4 v[MS][4];
};

template <int MS>
__device__ __forceinline__ void frag_offsets(uint32_t (&off)[MS], int64_t ld, int64_t mw,
                                             int64_t rows, int l32, int h) {
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    int64_t m = mw + 32 * ms + l32;
    m = m < rows ? m : rows - 1;
    off[ms] = (uint32_t)((m * ld + 32 * h) * 2);
  }
}

template <int MS>
__device__ __forceinline__ void frag_load(FragStage<MS>& st, const char* base,
                                          const uint32_t (&off)[MS]) {
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      st.v[ms][s] = *reinterpret_cast<const u32x4*>(base + off[ms] + 16 * s);
}

// mfma_step with the activation operands taken from registers.  Substep s
// issues its LDS reads first -- the weight fragments of substep s + 1 and
// pre(s + 1), the table reads of the next part of the staged tile -- then,
// behind a scheduling fence, its MFMAs and post(s), which finishes the part
// whose reads were issued a substep earlier.  Every LDS read therefore has a
// full substep of MFMAs to land, and the in-order LDS return queue never
// makes a product wait for reads issued after its own.
template <int MS, int JT, typename Pre, typename Post>
__device__ __forceinline__ void mfma_step_rx(const uint16_t* wtile, const FragStage<MS>& xf,
                                             int l32, int h, f32x16 (&acc)[4][MS],
                                             f32x16 (&tacc)[JT > 0 ? JT : 1][MS], Pre&& pre,
                                             Post&& post) {
  constexpr int NR = 4 + JT;
  const uint16_t* wbase = wtile + l32 * kLP + 32 * h;
  u32x4 wf[2][NR];
#pragma unroll
  for (int ns = 0; ns < NR; ++ns) wf[0][ns] = *reinterpret_cast<const u32x4*>(wbase + 32 * ns * kLP);
  pre(0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = s & 1;
    if (s < 3) {
#pragma unroll
      for (int ns = 0; ns < NR; ++ns)
        wf[c ^ 1][ns] = *reinterpret_cast<const u32x4*>(wbase + 32 * ns * kLP + 8 * (s + 1));
      pre(s + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[ns][ms] = mfma32(wf[c][ns], xf.v[ms][s], acc[ns][ms]);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) tacc[jt][ms] = mfma32(wf[c][4 + jt], xf.v[ms][s], tacc[jt][ms]);
    post(s);
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
  const uint16_t* Tm;       // M x RP bf16, scaled and adapter-masked (multi)
  const uint16_t* Bstack;   // concatenated B of the adapters (multi), read through col_*
  int32_t r;
  int32_t n_ad;
  float s;
  int32_t m_tiles;
  int32_t n_tiles;
  int32_t pad;
  uint16_t* Y;
  float* T_out;
  NF4Table tab;
  int32_t rc;               // multi: total rank columns
  int32_t col_base[kMaxRankCols];    // multi: rank column c of row n is Bstack[col_base[c]
  int32_t col_stride[kMaxRankCols];  //        + n col_stride[c]]
};

constexpr int kFwdTab = 1024;  // second-level steps of one tile's 128 rows (K <= 65536)

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

// Marks v as produced here.  The compiler otherwise converts a freshly loaded
// constant right after its load, which waits for that load (a full memory
// latency) in the middle of the step that issued it.
__device__ __forceinline__ uint32_t pin(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float pin(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ u32x4 pin(u32x4 v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int WK>
__device__ __forceinline__ float raw_scale_value(const RawScale& r, const float* tab, int32_t dq) {
  if (WK == kNF4DQ) return dq_q_rt(dq, pin(r.q)) * tab[r.gi];
  return __uint_as_float(pin(r.q));
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

// part (0..3) of writing a staged forward weight tile: fwd_stage_fetch issues
// the level-table reads of the part, fwd_stage_finish scales (a = the block
// scale), rounds and stores it (and the part's shrink-operand rows).
template <int WK, int JT>
__device__ __forceinline__ LutFetch fwd_stage_fetch(const FwdStage<WK, JT>& st, const float2* lut,
                                                    int part) {
  if (WK == kDense) return LutFetch{};
  return lut_fetch(st.w[0][part], lut);
}

template <int WK, int JT>
__device__ __forceinline__ void fwd_stage_finish(const FwdStage<WK, JT>& st, const LutFetch& f,
                                                 uint16_t* tile, float a, int part) {
  const int tid = threadIdx.x;
  if (WK == kDense) {
    *reinterpret_cast<u32x4*>(tile + ((tid >> 3) + 32 * part) * kLP + 8 * (tid & 7)) = st.w[part];
  } else {
    *reinterpret_cast<u32x4*>(tile + (tid >> 1) * kLP + 32 * (tid & 1) + 8 * part) =
        lut_finish(f, a);
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
  uint32_t xo[MS];
  frag_offsets<MS>(xo, K, mw, M, l32, h);
  const char* xbase = reinterpret_cast<const char*>(p.X);

  f32x16 acc[4][MS];
  f32x16 tacc[JT > 0 ? JT : 1][MS];
  zero_acc(acc);
  zero_acc(tacc);

  FwdStage<WK, JT> s0, s1;
  FragStage<MS> x0, x1, x2;

  fwd_stage_load<WK, JT>(s0, p, o, 0, g_lo);
  frag_load<MS>(x0, xbase, xo);
  frag_load<MS>(x1, xbase + 2 * ((int64_t)(KT > 1 ? 1 : 0) * kBK), xo);
  __syncthreads();  // level and step tables ready
  {
    const float a = WK != kDense ? raw_scale_value<WK>(s0.sc, stab, p.W.dq) : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      fwd_stage_finish<WK, JT>(s0, fwd_stage_fetch<WK, JT>(s0, lut, q), wt[0], a, q);
  }
  const int64_t kb1 = (int64_t)(KT > 1 ? 1 : 0) * kBK;
  fwd_stage_load<WK, JT>(s1, p, o, kb1, g_lo);
  __syncthreads();

  // step kt: loads weight stage kt+2 into snxt and the activation fragments
  // of step kt+2 into xnxt, runs the MFMAs of step kt (LDS buffer kt & 1,
  // fragments xcur), writes weight stage kt+1 (scur) into the other buffer.
  // Weight stages rotate over two register sets, activation fragments over
  // three, so the main loop is unrolled by six.
  auto step = [&](int kt, const FwdStage<WK, JT>& scur, const FragStage<MS>& xcur,
                  FwdStage<WK, JT>& snxt, FragStage<MS>& xnxt) {
    const int64_t k2 = (int64_t)(kt + 2 < KT ? kt + 2 : KT - 1) * kBK;
    fwd_stage_load<WK, JT>(snxt, p, o, k2, g_lo);
    frag_load<MS>(xnxt, xbase + 2 * k2, xo);
    const float a = WK != kDense ? raw_scale_value<WK>(scur.sc, stab, p.W.dq) : 0.0f;
    const int b = kt & 1;
    uint16_t* wn = wt[b ^ 1];
    LutFetch lf[2];
    mfma_step_rx<MS, JT>(
        wt[b], xcur, l32, h, acc, tacc,
        [&](int q) { lf[q & 1] = fwd_stage_fetch<WK, JT>(scur, lut, q); },
        [&](int q) { fwd_stage_finish<WK, JT>(scur, lf[q & 1], wn, a, q); });
    __syncthreads();
  };

  for (int kt = 0; kt < KT; kt += 6) {
    step(kt, s1, x0, s0, x2);
    if (kt + 1 < KT) step(kt + 1, s0, x1, s1, x0);
    if (kt + 2 < KT) step(kt + 2, s1, x2, s0, x1);
    if (kt + 3 < KT) step(kt + 3, s0, x0, s1, x2);
    if (kt + 4 < KT) step(kt + 4, s1, x1, s0, x0);
    if (kt + 5 < KT) step(kt + 5, s0, x2, s1, x1);
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
    const int rc = p.rc;
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
              e[i] = j < rc ? p.Bstack[p.col_base[j] + n * p.col_stride[j]] : (uint16_t)0;
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

// dX weight tile of one step: W rows n0r .. n0r+63 (the reduction) by
// columns k0 .. k0+127 (the outputs), kept in LDS in storage order (row n, k
// contiguous), and B rows n0r .. n0r+63 as columns 128 .. 128+RP of the same
// tile rows.  The MFMA operands (one column, eight consecutive rows) are read
// with the gfx950 transposing LDS read ds_read_b64_tr_b16: inside each group
// of 16 lanes, lane c addresses row c / 4, columns 4 (c % 4) .. +3 of a 4 x 16
// block, and lane i receives column i of rows 0..3.  16-byte chunk q of row n
// is stored at chunk q ^ (n & 3); with a row pitch of 20 (RP = 32) or 28
// (RP = 64) chunks, both the 16-byte stores and the transposing reads of 16
// lanes land on 16 distinct 16-byte bank groups.
template <int RP>
struct DxPitch {
  static constexpr int P = RP == 32 ? 160 : 224;  // elements
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
  return __builtin_bit_cast(u32x2, v);
}

// mfma_step with the weight operands read transposed from a storage-order
// tile of pitch P: subtile ns covers columns 32 ns .. +31, substep s rows
// 32 h + 8 s .. +7 (lane half h), the same reduction labels as the
// activation operand.
template <int MS, int JT, int P, typename Part>
__device__ __forceinline__ void mfma_step_tr(const uint16_t* wtile, const uint16_t* atile, int wave,
                                             int lane, f32x16 (&acc)[4][MS],
                                             f32x16 (&tacc)[JT][MS], Part&& part) {
  constexpr int NR = 4 + JT;
  const int c = lane & 15, g = lane >> 4, h = lane >> 5, l32 = lane & 31;
  const uint16_t* wbase = wtile + (32 * h + (c >> 2)) * P +
                          8 * ((2 * (g & 1) + ((c >> 1) & 1)) ^ (c >> 2)) + 4 * (c & 1);
  const uint16_t* abase = atile + (32 * MS * wave + l32) * kLP + 32 * h;
  auto wread = [&](int ns, int s) {
    const uint16_t* q = wbase + 8 * s * P + 32 * ns;
    const u32x2 lo = lds_read_tr(q), hi = lds_read_tr(q + 4 * P);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  u32x4 wf[2][NR], af[2][MS];
#pragma unroll
  for (int ns = 0; ns < NR; ++ns) wf[0][ns] = wread(ns, 0);
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) af[0][ms] = *reinterpret_cast<const u32x4*>(abase + 32 * ms * kLP);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cb = s & 1;
    if (s < 3) {
#pragma unroll
      for (int ns = 0; ns < NR; ++ns) wf[cb ^ 1][ns] = wread(ns, s + 1);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        af[cb ^ 1][ms] = *reinterpret_cast<const u32x4*>(abase + 32 * ms * kLP + 8 * (s + 1));
    }
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[ns][ms] = mfma32(wf[cb][ns], af[cb][ms], acc[ns][ms]);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) tacc[jt][ms] = mfma32(wf[cb][4 + jt], af[cb][ms], tacc[jt][ms]);
    part(s);
  }
}

// Staging of one dX step, loaded two steps ahead.  NF4: thread t takes row
// t / 4 and the 32 columns k0 + 32 (t % 4) .. (16 code bytes, half a block:
// one block constant, and for double quantisation its group's c2).  Dense:
// thread t takes the 16-byte chunk t % 16 of rows t / 16 + 16 i.  B: thread t
// takes row t / 4, columns 8 (t % 4 + 4 i) .. +7 (whole 16-byte chunks when
// r % 8 == 0 (BV), element loads otherwise).  Columns past K are clamped
// (their outputs are never stored) and N % 64 == 0 keeps every step full.
template <int WK, int RP>
struct DxStage {
  u32x4 w[WK == kDense ? 4 : 1];
  uint32_t q;
  float c2;
  u32x4 b[RP / 32];
};

struct DxOffsets {
  uint32_t w[4];  // dense: byte offsets of the 4 chunks; NF4: w[0] code byte offset
  uint32_t e;     // NF4: element index of the thread's first code
  uint32_t b[2];  // B: element offset of each chunk (row * r + 8 chunk)
  uint32_t st[4]; // LDS element offsets of the 4 weight parts
  uint32_t sb;    // LDS element offset of the B chunks
};

template <int WK, int RP, bool BV>
__device__ __forceinline__ void dx_stage_load(DxStage<WK, RP>& st, const BwdParams& p,
                                              const DxOffsets& o, int64_t n0r) {
  const int64_t K = p.W.K;
  const int64_t eb = n0r * K;  // first element of the step's rows
  if (WK == kDense) {
    const char* base = reinterpret_cast<const char*>(p.W.dense + eb);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.w[i] = *reinterpret_cast<const u32x4*>(base + o.w[i]);
  } else {
    st.w[0] = *reinterpret_cast<const u32x4*>(p.W.codes + (eb >> 1) + o.w[0]);
    const uint32_t blk = o.e >> 6;
    if (WK == kNF4DQ) {
      st.q = p.W.q8[(eb >> 6) + blk];
      const int64_t g = (eb >> 14) + (((eb & 16383) + o.e) >> 14);
      st.c2 = p.W.c2[g];
    } else {
      st.q = __float_as_uint(p.W.absmax[(eb >> 6) + blk]);
    }
  }
  const int r = p.r;
  const uint16_t* bb = p.B + n0r * r;
  const int cb = threadIdx.x & 3;
#pragma unroll
  for (int i = 0; i < RP / 32; ++i) {
    const int j0 = 8 * (cb + 4 * i);
    if (BV) {
      st.b[i] = *reinterpret_cast<const u32x4*>(bb + o.b[i]);  // chunks past r masked when stored
    } else {
      uint32_t v[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int j = j0 + 2 * d;
        const uint32_t lo = bb[o.b[i] + (j < r ? 2 * d : 0)];
        const uint32_t hi = bb[o.b[i] + (j + 1 < r ? 2 * d + 1 : 0)];
        v[d] = (j < r ? lo : 0u) | ((j + 1 < r ? hi : 0u) << 16);
      }
      st.b[i] = u32x4{v[0], v[1], v[2], v[3]};
    }
  }
}

template <int WK, int RP>
__device__ __forceinline__ float dx_scale(const DxStage<WK, RP>& st, int32_t dq) {
  if (WK == kNF4DQ) return dq_q_rt(dq, pin(st.q)) * dq_step(pin(st.c2));
  return __uint_as_float(pin(st.q));
}

// part (0..3) of writing a staged dX tile (a = its block scale)
template <int WK, int RP>
__device__ __forceinline__ void dx_stage_part(const DxStage<WK, RP>& st, const DxOffsets& o,
                                              uint16_t* tile, const float2* lut, float a, int r,
                                              int part) {
  if (WK == kDense) {
    *reinterpret_cast<u32x4*>(tile + o.st[part]) = st.w[part];
  } else {
    *reinterpret_cast<u32x4*>(tile + o.st[part]) = deq8(st.w[0][part], a, lut);
  }
  if (part < RP / 32)
    *reinterpret_cast<u32x4*>(tile + o.sb + 32 * part) =
        sel4(8 * ((threadIdx.x & 3) + 4 * part) < r, pin(st.b[part]));
}

template <int WK, int MS, int RP, bool BV>
__global__ __launch_bounds__(kThreads) void dx_kernel(BwdParams p) {
  constexpr int JT = RP / 32;
  constexpr int P = DxPitch<RP>::P;
  constexpr int AROWS = 128 * MS;
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][kBK * P];
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][AROWS * kLP];
  __shared__ float2 lut[256];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = xcd_tile(blockIdx.x, p.m_tiles * p.k_tiles);
  const int tile_k = tile % p.k_tiles, tile_m = tile / p.k_tiles;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t k0 = (int64_t)tile_k * kTileI, m0 = (int64_t)tile_m * AROWS;
  const int64_t mw = m0 + wave * 32 * MS;
  const int RT = (int)(N / kBK);

  if (WK != kDense) build_lut(lut, p.tab);

  DxOffsets o;
  {
    const int r = p.r;
    const int nt = tid >> 2, ct = tid & 3;
    if (WK == kDense) {
      const int c = tid & 15, nr = tid >> 4;
      int64_t k = k0 + 8 * c;
      k = k < K ? k : K - 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o.w[i] = (uint32_t)(((int64_t)(nr + 16 * i) * K + k) * 2);
        o.st[i] = (uint32_t)((nr + 16 * i) * P + 8 * (c ^ (nr & 3)));
      }
    } else {
      int64_t k = k0 + 32 * ct;
      k = k < K ? k : K - 32;
      const int64_t e = (int64_t)nt * K + k;
      o.w[0] = (uint32_t)(e >> 1);
      o.e = (uint32_t)e;
#pragma unroll
      for (int q = 0; q < 4; ++q) o.st[q] = (uint32_t)(nt * P + 8 * ((4 * ct + q) ^ (nt & 3)));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int j0 = 8 * (ct + 4 * i);
      j0 = j0 < r ? j0 : 0;
      o.b[i] = (uint32_t)(nt * r + j0);
    }
    o.sb = (uint32_t)(nt * P + 128 + 8 * (ct ^ (nt & 3)));
  }
  uint32_t go[4 * MS];
  act_offsets<MS>(go, N, m0, M);
  const char* gbase = reinterpret_cast<const char*>(p.dY);

  f32x16 acc[4][MS];
  f32x16 uacc[JT][MS];
  zero_acc(acc);
  zero_acc(uacc);

  DxStage<WK, RP> s0, s1;
  ActStage<MS> g0, g1;

  dx_stage_load<WK, RP, BV>(s0, p, o, 0);
  act_load<MS>(g0, gbase, go);
  __syncthreads();  // level table ready
  {
    const float a = WK != kDense ? dx_scale<WK, RP>(s0, p.W.dq) : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dx_stage_part<WK, RP>(s0, o, wt[0], lut, a, p.r, q);
      act_part<MS>(g0, gt[0], q);
    }
  }
  const int64_t n1 = (int64_t)(RT > 1 ? 1 : 0) * kBK;
  dx_stage_load<WK, RP, BV>(s1, p, o, n1);
  act_load<MS>(g1, gbase + 2 * n1, go);
  __syncthreads();

  // step rt: loads stage rt+2 into (snxt, gnxt), runs the MFMAs of step rt on
  // buffer rt & 1 and writes stage rt+1 (scur, gcur) into the other buffer
  auto step = [&](int rt, const DxStage<WK, RP>& scur, const ActStage<MS>& gcur,
                  DxStage<WK, RP>& snxt, ActStage<MS>& gnxt) {
    const int64_t n2 = (int64_t)(rt + 2 < RT ? rt + 2 : RT - 1) * kBK;
    dx_stage_load<WK, RP, BV>(snxt, p, o, n2);
    act_load<MS>(gnxt, gbase + 2 * n2, go);
    const float a = WK != kDense ? dx_scale<WK, RP>(scur, p.W.dq) : 0.0f;
    const int b = rt & 1;
    uint16_t* wn = wt[b ^ 1];
    uint16_t* gn = gt[b ^ 1];
    mfma_step_tr<MS, JT, P>(wt[b], gt[b], wave, lane, acc, uacc, [&](int q) {
      dx_stage_part<WK, RP>(scur, o, wn, lut, a, p.r, q);
      act_part<MS>(gcur, gn, q);
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

// Tm[m][c] = scale[a] * sum_k X[m][k] Acat[c][k] if column c belongs to the
// row's adapter a = row_ad[m] (mt), else 0, for c < rc (Acat = the adapters' A
// stacked by rows, rc x K), zero up to RP; bf16.
// Each wave takes 32 rows; lane (h, l32) reads row l32, 32 contiguous columns
// per 64-step (the same relabelling of the reduction index on both operands).
template <int RP>
__global__ __launch_bounds__(kThreads) void multi_shrink_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, const uint16_t* __restrict__ Acat,
    int rc, const int32_t* __restrict__ row_ad, MultiTab mt, uint16_t* __restrict__ Tm) {
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
  int a = row_ad[m];  // clamped: ids are in range by precondition
  a = a < 0 ? 0 : (a >= mt.n_ad ? mt.n_ad - 1 : a);
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = 32 * jt + 8 * q + 4 * h;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + i;
        v[i] = (c < rc && c >= mt.roff[a] && c < mt.roff[a + 1]) ? mt.scale[a] * t[jt][4 * q + i]
                                                                 : 0.0f;
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
  timing_begin("fwd_kernel", st);
  hipLaunchKernelGGL((fwd_kernel<WK, MS, RP, MULTI>), dim3(blocks), dim3(kThreads), 0, st, p);
  timing_end(st);
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

template <int WK, int MS, int RP, bool BV>
int launch_dx(const BwdParams& p0, hipStream_t st) {
  BwdParams p = p0;
  p.k_tiles = (int)cdiv(p.W.K, kTileI);
  p.m_tiles = (int)cdiv(p.M, 128 * MS);
  const int blocks = p.k_tiles * p.m_tiles;
  timing_begin("dx_kernel", st);
  hipLaunchKernelGGL((dx_kernel<WK, MS, RP, BV>), dim3(blocks), dim3(kThreads), 0, st, p);
  timing_end(st);
  return hip_fail(hipGetLastError(), "dx_kernel launch");
}

template <int WK, int RP>
int dx_pick_ms(const BwdParams& p, hipStream_t st) {
  const bool big = big_tiles(p.M), bv = p.r % 8 == 0;
  if (big) return bv ? launch_dx<WK, 2, RP, true>(p, st) : launch_dx<WK, 2, RP, false>(p, st);
  return bv ? launch_dx<WK, 1, RP, true>(p, st) : launch_dx<WK, 1, RP, false>(p, st);
}

template <int WK>
int dx_pick(const BwdParams& p, hipStream_t st) {
  return p.r <= 32 ? dx_pick_ms<WK, 32>(p, st) : dx_pick_ms<WK, 64>(p, st);
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
  p.tab = nf4_table(W.codebook);
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
  p.tab = nf4_table(W.codebook);
  if (W.kind == LQ_WEIGHT_DENSE) return dx_pick<kDense>(p, st);
  if (W.double_quant) return dx_pick<kNF4DQ>(p, st);
  return dx_pick<kNF4>(p, st);
}

int launch_rowmap(const int32_t* seg_off, const int32_t* seg_ad, int32_t n_seg, int64_t T,
                  int32_t* row_ad, hipStream_t st) {
  hipLaunchKernelGGL(rowmap_kernel, dim3(n_seg), dim3(256), 0, st, seg_off, seg_ad, T, row_ad);
  return hip_fail(hipGetLastError(), "rowmap launch");
}

size_t multi_ws_bytes(int64_t T_tokens, int64_t r, int32_t n_adapters) {
  const int64_t rp = (r * n_adapters <= 32) ? 32 : 64;
  return (size_t)T_tokens * 4 + (size_t)T_tokens * rp * 2 + 256;
}

int bf16_fwd_given_t(const void* X, int64_t M, const lq_weight& W, const void* B, int64_t r,
                     const void* Tm, void* Y, hipStream_t st) {
  FwdParams p{};
  p.X = (const uint16_t*)X;
  p.M = M;
  p.W = weight_args(W);
  p.Tm = (const uint16_t*)Tm;
  p.Bstack = (const uint16_t*)B;
  p.r = (int32_t)r;
  p.n_ad = 1;
  p.s = 1.0f;
  p.rc = (int32_t)r;
  for (int c = 0; c < kMaxRankCols; ++c) {  // B[n][c] = B[c + n r]; unused columns at 0
    p.col_base[c] = c < r ? c : 0;
    p.col_stride[c] = c < r ? (int32_t)r : 0;
  }
  p.Y = (uint16_t*)Y;
  p.tab = nf4_table(W.codebook);
  return fwd_dispatch<true>(p, W, r <= 32 ? 32 : 64, st);
}

int bf16_fwd_multi(const void* X, int64_t T_tokens, const lq_weight& W, const void* A_cat,
                   const void* B_cat, const MultiTab& mt, const int32_t* seg_offsets,
                   const int32_t* seg_adapter, int32_t n_seg, void* Y, void* ws, hipStream_t st) {
  const int rc = mt.rc;
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
                       (const uint16_t*)X, T_tokens, K, (const uint16_t*)A_cat, rc, row_ad, mt,
                       Tm);
  else
    hipLaunchKernelGGL(multi_shrink_kernel<64>, dim3(sblocks), dim3(kThreads), 0, st,
                       (const uint16_t*)X, T_tokens, K, (const uint16_t*)A_cat, rc, row_ad, mt,
                       Tm);
  if ((e = hip_fail(hipGetLastError(), "multi shrink launch"))) return e;
  FwdParams p{};
  p.X = (const uint16_t*)X;
  p.M = T_tokens;
  p.W = weight_args(W);
  p.Tm = Tm;
  p.Bstack = (const uint16_t*)B_cat;
  p.r = rc;
  p.n_ad = mt.n_ad;
  p.s = 1.0f;
  p.rc = rc;
  for (int c = 0; c < kMaxRankCols; ++c) {
    p.col_base[c] = mt.col_base[c];
    p.col_stride[c] = mt.col_stride[c];
  }
  p.Y = (uint16_t*)Y;
  p.tab = nf4_table(W.codebook);
  return fwd_dispatch<true>(p, W, rp, st);
}

}  // namespace dispatch
}  // namespace lq

// Decode-sized forward (M <= 16) and the skinny rank-r products.
//
// Decode: Y = X deq(W0)^T + s T B^T, with the partial sums of T = X A^T
// formed first by tpart_kernel.  With at most 16 activation rows the layer is
// bound by streaming W0 from HBM (4.127 bits per weight in NF4 with double
// quantisation: "Large Language Model Fine-tuning and LoRA", section
// "Quantizing the frozen weights"), so gemv_kernel is organised around that
// stream: a workgroup owns 16 output rows n and its sixteen waves split K;
// each lane loads 16 code bytes (32 weights, half a block) per granule,
// dequantises them in registers through the LDS level table and feeds four
// v_mfma_f32_16x16x32_bf16 (X padded to 16 rows).  The wave partial sums are
// combined through LDS; the rank-r expand is r scalar FMAs per output.
//
// Skinny: out[m][j] = sum_k Z[m][k] G[j][k] for j < r <= 64, G = A (r x K)
// or B^T (B is K x r here, i.e. the reduction runs over B's rows).  Each wave
// takes 32 rows of Z straight into MFMA registers; the small G tile of each
// step is staged in LDS (transposed for B).
#include <atomic>
#include <climits>
#include <cstring>
#include <map>
#include <mutex>

#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;

template <int RP, bool GT>
__global__ __launch_bounds__(kThreads) void skinny_kernel(const uint16_t* __restrict__ Z,
                                                          int64_t M, int64_t K,
                                                          const uint16_t* __restrict__ G, int r,
                                                          float* __restrict__ out,
                                                          int32_t* __restrict__ zero, int nzero) {
  constexpr int JT = RP / 32;
  __shared__ __attribute__((aligned(16))) uint16_t gl[RP * kPitch];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // side job: clear the next kernel's flag words (a kernel store, so it also
  // replays correctly inside a captured graph)
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += kThreads) zero[i] = 0;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t mrow = ((int64_t)blockIdx.x * 4 + wave) * 32 + l32;
  const int64_t mr = mrow < M ? mrow : M - 1;
  f32x16 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.0f;
  for (int64_t k0 = 0; k0 < K; k0 += 64) {
    __syncthreads();
    for (int e = tid; e < RP * 64; e += kThreads) {
      int j, kk;
      uint16_t v = 0;
      if (GT) {  // G[j][k] = B[k][j], read B rows coalesced
        kk = e / RP;
        j = e - kk * RP;
        if (j < r && k0 + kk < K) v = G[(k0 + kk) * r + j];
      } else {
        j = e / 64;
        kk = e - j * 64;
        if (j < r && k0 + kk < K) v = G[(int64_t)j * K + k0 + kk];
      }
      gl[j * kPitch + kk] = v;
    }
    __syncthreads();
    const uint16_t* zrow = Z + mr * K + k0 + 32 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok = k0 + 32 * h + 8 * s < K;
      const u32x4 zf = ok ? *reinterpret_cast<const u32x4*>(zrow + 8 * s) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 gf =
            *reinterpret_cast<const u32x4*>(gl + (32 * jt + l32) * kPitch + 32 * h + 8 * s);
        acc[jt] = mfma32(gf, zf, acc[jt]);
      }
    }
  }
  if (mrow >= M) return;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 32 * jt + 8 * q + 4 * h + i;
        if (j < r) out[mrow * r + j] = acc[jt][4 * q + i];
      }
}

int launch_skinny(const uint16_t* Z, int64_t M, int64_t K, const uint16_t* G, bool gt, int64_t r,
                  float* out, int32_t* zero, int nzero, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(M, 128)), block(kThreads);
  if (r <= 32) {
    if (gt)
      hipLaunchKernelGGL((skinny_kernel<32, true>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero);
    else
      hipLaunchKernelGGL((skinny_kernel<32, false>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero);
  } else {
    if (gt)
      hipLaunchKernelGGL((skinny_kernel<64, true>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero);
    else
      hipLaunchKernelGGL((skinny_kernel<64, false>), grid, block, 0, st, Z, M, K, G, (int)r, out,
                         zero, nzero);
  }
  return hip_fail(hipGetLastError(), "skinny launch");
}

// ------------------------------------------------------------ decode GEMV

struct GemvParams {
  const uint16_t* X;  // M x K
  int64_t M;
  WeightArgs W;
  const float* Tp;    // kTParts x M x r partial sums of X A^T
  const uint16_t* B;  // N x r
  float* T_out;       // M x r or NULL (written by workgroup 0)
  int32_t r;
  float s;
  uint16_t* Y;        // M x N
  NF4Table tab;
};

// Granule = 32 consecutive weights of one row (16 code bytes, half an NF4
// block).  A workgroup of 16 waves owns 16 output rows; lane (q, l16) of wave
// w takes row n0 + l16 and granules 4 t + q for t = w, w + 16, ..., CH of them
// per round, all loads issued from clamped addresses before any is used.
// Each granule feeds four v_mfma_f32_16x16x32_bf16 (X padded to 16 rows, the
// 32 reduction elements of a lane relabelled so that they are contiguous) on
// its own accumulator chain.  The inputs of the rank-r expand (the T partial
// sums and this workgroup's 16 rows of B) are loaded into registers before
// the weight stream and only summed and staged in LDS after it; the 16 wave
// partials are added through LDS.
// The activations are staged in LDS once per workgroup (XS > 0: up to XS
// elements of one chunk's rows; 16384 keeps two workgroups per compute unit,
// 65536 one).  Loaded per lane
// straight from global memory, the lanes of a 16-lane group whose row is past
// M would all load row 0 again (16 times the bytes of X through each compute
// unit's load path at M = 1), and at M = 16 the per-lane 16-byte pieces are
// scattered over 16 rows.  Staged row m, 16-byte chunk c sits at chunk
// c ^ (m & 15) of its row (needs K % 128 == 0), so the 16 rows read by one
// lane group hit 16 distinct bank groups.
constexpr int kGemvWaves = 16;

template <int WK, int XS>
__global__ __launch_bounds__(64 * kGemvWaves) void gemv_kernel(GemvParams p) {
  // 16-row chunk blockIdx.y of a call with up to 64 rows: its rows of X, Y and
  // T_out, and its own partial sums of T
  {
    const int64_t m0 = 16 * (int64_t)blockIdx.y;
    p.X += m0 * p.W.K;
    p.Y += m0 * p.W.N;
    if (p.T_out) p.T_out += m0 * p.r;
    p.Tp += (int64_t)blockIdx.y * kTParts * 16 * p.r;
    p.M = p.M - m0 < 16 ? p.M - m0 : 16;
  }
  constexpr bool XL = XS > 0;
  constexpr int CH = 2;
  constexpr int NT = 64 * kGemvWaves;
  constexpr int XC = XL ? XS / 8 / NT : 1;  // 16-byte X chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? XS : 8];
  __shared__ float2 lut[256];
  __shared__ f32x4 part[kGemvWaves][64];
  __shared__ float tT[16 * 64];
  __shared__ float tB[16 * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int r = p.r;

  // XL: the chunks of X, issued first so that the wait before their LDS store
  // does not wait for the weight stream (clamped to the last chunk; a clamped
  // thread stores the same value to the same place as the last chunk's owner)
  const int64_t nxc = M * K / 8, rowc = K / 8;
  u32x4 xc[XC];
  uint32_t xsto[XC];
  if (XL) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      int64_t c = tid + (int64_t)NT * i;
      c = c < nxc ? c : nxc - 1;
      xc[i] = *reinterpret_cast<const u32x4*>(p.X + 8 * c);
      const int64_t m = c / rowc, ch = c - m * rowc;
      xsto[i] = (uint32_t)(m * K + 8 * (ch ^ (m & 15)));
    }
  }

  // expand inputs: element tid of T (M x r <= 1024) and of B rows n0.. (16 x r),
  // loaded without branches (clamped index; threads past the end load a valid
  // element and drop it), so that no wait for them is placed before the
  // weight stream
  const int ET = (int)M * r, EB = 16 * r;
  const int te = tid < ET ? tid : ET - 1, tb = tid < EB ? tid : EB - 1;
  float tp[kTParts];
#pragma unroll
  for (int b = 0; b < kTParts; ++b) tp[b] = p.Tp[b * ET + te];
  const uint16_t braw = p.B[n0 * r + tb];

  const int64_t n = n0 + l16;  // A-operand row of this lane (N % 16 == 0)
  const bool mrow = l16 < M;   // B-operand column (activation row) of this lane
  const int64_t xm = mrow ? l16 : 0;
  f32x4 acc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t G = K / 32;
  const int64_t steps = (G + 3) / 4;
  u32x4 wraw[CH][WK == kDense ? 4 : 1];
  uint32_t sq[CH];
  float sc2[CH];
  u32x4 xf[CH][4];
  int64_t kx[CH];
  bool ok[CH];
  // one round of granule loads (clamped addresses; granules past the end masked)
  auto load = [&](int64_t base) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t t = base + kGemvWaves * i;
      const int64_t g = 4 * t + q;
      ok[i] = t < steps && g < G;
      const int64_t k = ok[i] ? 32 * g : 0;
      const int64_t e = n * K + k;
      if (WK == kDense) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          wraw[i][d] = *reinterpret_cast<const u32x4*>(p.W.dense + e + 8 * d);
      } else {
        wraw[i][0] = *reinterpret_cast<const u32x4*>(p.W.codes + (e >> 1));
        if (WK == kNF4DQ) {
          sq[i] = p.W.q8[e >> 6];
          sc2[i] = p.W.c2[e >> 14];
        } else {
          sq[i] = __float_as_uint(p.W.absmax[e >> 6]);
        }
      }
      // every lane loads (lanes without an activation row read row 0 and are
      // masked at the product): no branch, so no wait at a join
      kx[i] = xm * K + k;
      if (!XL)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          xf[i][d] = *reinterpret_cast<const u32x4*>(p.X + kx[i] + 8 * d);
      else  // staged: the chunk index of k, before the row swizzle
        kx[i] = k >> 3;
      ok[i] = ok[i] && mrow;
    }
  };
  // The first round's loads go out before the level table is built, so that
  // their memory latency overlaps the table and its barrier (every wave
  // issues them; a wave with no granule loads clamped addresses and masks).
  load(wave);
  if (WK != kDense) build_lut(lut, p.tab);
  if (XL) {
    // every thread stores: no branch, so the loads of X stay ahead of the
    // weight stream
#pragma unroll
    for (int i = 0; i < XC; ++i) *reinterpret_cast<u32x4*>(xs + xsto[i]) = xc[i];
  }
  if (XL || WK != kDense) __syncthreads();  // level table, staged X
  for (int64_t base = wave; base < steps; base += kGemvWaves * CH) {
    if (base != wave) load(base);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (XL)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          xf[i][d] = *reinterpret_cast<const u32x4*>(
              xs + xm * K + 8 * ((kx[i] + d) ^ (xm & 15)));
      if (WK == kDense) {
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[i] = mfma16(wraw[i][d], sel4(ok[i], xf[i][d]), acc[i]);
      } else {
        const float a =
            WK == kNF4DQ ? dq_q_rt(p.W.dq, sq[i]) * dq_step(sc2[i]) : __uint_as_float(sq[i]);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          acc[i] = mfma16(deq8(wraw[i][0][d], a, lut), sel4(ok[i], xf[i][d]), acc[i]);
      }
    }
  }
  // stage the expand inputs (their loads finished long ago)
  if (tid < ET) {
    float t = 0.0f;
#pragma unroll
    for (int b = 0; b < kTParts; ++b) t += tp[b];
    const int m = tid / r, j = tid - m * r;
    tT[m * 64 + j] = t;
    if (blockIdx.x == 0 && p.T_out) p.T_out[tid] = t;
  }
  if (tid < EB) {
    const int nn = tid / r, j = tid - nn * r;
    tB[nn * 64 + j] = bf16_to_f32(braw);
  }
  // acc lane l: rows n0 + 4 q + i, column m = l16 (16x16 accumulator layout)
  f32x4 a0 = acc[0];
#pragma unroll
  for (int i = 1; i < CH; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) a0[v] += acc[i][v];
  part[wave][lane] = a0;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = part[0][lane];
#pragma unroll
  for (int w = 1; w < kGemvWaves; ++w) {
    const f32x4 o = part[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += o[i];
  }
  if (!mrow) return;
  const int m = l16;
  float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < r; ++j) {
    const float t = tT[m * 64 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = fmaf(t, tB[(4 * q + i) * 64 + j], d[i]);
  }
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = sum[i] + p.s * d[i];
  *reinterpret_cast<u32x2*>(p.Y + m * N + n0 + 4 * q) =
      u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
}

// ------------------------------------------------------------ decode, one launch
//
// dq_kernel runs the decode forward (M <= 16) in one launch.  Workgroup b owns
// output rows 16 b .. 16 b + 15 and streams their NF4 codes as gemv_kernel
// does (each lane two 32-weight granules per round, every load issued before
// any is used, dequantised in registers through the LDS level table into
// v_mfma_f32_16x16x32_bf16, activations staged in LDS).  T = X A^T is formed
// in the same launch: the first P workgroups ("producers") also reduce one
// contiguous range of the reduction each (one granule per wave, A fragments
// loaded with the first weight loads, activations from LDS) and publish their
// partial sums; after its own weight stream every workgroup adds the P
// partials in producer order and applies the rank-r expand.
// Publication without fences: every published float travels as one 64-bit
// word (call tag, value), written and read with relaxed agent-scope atomics
// (single-copy atomic, coherent across the XCDs).  A reader accepts a word
// only when its tag is this call's, so it never needs the writer's other
// stores to be visible and no ordering between words is required.  The call
// tag is epoch + 1, with the epoch a word of the stream's slot in library
// memory that every workgroup reads as its first load.  Each workgroup counts
// itself in (one of eight counters, by XCD) once that load has returned;
// workgroup 0 reads the counters after its weight stream and, at its end
// (re-reading while they are short), returns them to zero and advances the
// epoch.  So every workgroup of a call sees
// the same tag, each call (also each replay of a captured graph) has a new
// one, and nothing needs clearing between calls.  Every wait is bounded; a
// workgroup that gives up on the partials counts the give-up
// (lq_debug_wait_giveups) and computes T itself from X and A (the same value
// up to summation order), so a call stays correct even then.  The bound set
// by lq_debug_set_wait_limit applies to that wait only; workgroup 0's wait
// before it advances the epoch keeps the default bound, since advancing early
// would hand a late workgroup the next call's tag.
constexpr int kDecSlots = 32;        // streams with their own slot, per device
constexpr int kDecMaxP = 16;         // producer workgroups at most
constexpr int kDecMaxT = 16 * 64;    // elements of T at most (M <= 16, r <= 64)
struct DecSlot {
  uint32_t epoch;
  uint32_t pad[31];
  uint32_t started[8][32];  // workgroups counted in this call, by XCD (one line each)
  uint64_t part[kDecMaxP * kDecMaxT];  // (tag, partial sum of T) of producer p, element e
};
__device__ DecSlot g_dec_slot[kDecSlots];
// waits for T words that gave up since the host last read the count
__device__ unsigned long long g_dec_giveups;

struct DecParams {
  const uint16_t* X;  // M x K, M <= 16
  int64_t M;
  WeightArgs W;
  const uint16_t* A;  // r x K
  const uint16_t* B;  // N x r
  float* T_out;       // M x r or NULL
  int32_t r;
  float s;
  uint16_t* Y;        // M x N
  NF4Table tab;
  int32_t P;          // producer workgroups
  int32_t slot;
  int32_t spin;       // bound of a wait for a word, in polls (< 0: give up at once)
};

__device__ __forceinline__ uint64_t tagged(uint32_t tag, float v) {
  return ((uint64_t)tag << 32) | __float_as_uint(v);
}

// T straight from X and A in float32 by the 64 lanes of one wave (the fallback
// of a wait that gave up): element e = m r + j goes to T[64 m + j]
__device__ __forceinline__ void dec_t_direct(const DecParams& p, float* T) {
  const int lane = threadIdx.x & 63;
  const int64_t K = p.W.K;
  for (int e = lane; e < (int)p.M * p.r; e += 64) {
    const int m = e / p.r, j = e - m * p.r;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k)
      acc = fmaf(bf16_to_f32(p.X[m * K + k]), bf16_to_f32(p.A[(int64_t)j * K + k]), acc);
    T[64 * m + j] = acc;
  }
}

// The body of the one-launch decode.  lb is the workgroup's block within its
// layer (output rows 16 lb ..), pbase the index of the layer's first producer
// in the slot's partial-sum words; blockIdx.x and gridDim.x keep their
// call-wide meaning (counting in, the workgroup that moves the epoch on).
template <int WK, int XS, int JT, bool SS>
__device__ __forceinline__ void dq_body(const DecParams& p, const int lb, const int pbase) {
  constexpr bool XL = XS > 0;
  constexpr int CH = 2;
  constexpr int NT = 64 * kGemvWaves;
  constexpr int XC = XL ? XS / 8 / NT : 1;  // 16-byte X chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? XS : 8];
  __shared__ float2 lut[256];
  __shared__ f32x4 part[kGemvWaves][64];
  __shared__ float tB[16 * 64];
  __shared__ float tT[16 * 64];
  // SS (NF4, K <= 4096): the block scales a' of the workgroup's 16 rows, formed
  // once per block by the workgroup (row stride 65 words: the 16 rows one
  // lane group reads sit in distinct banks)
  __shared__ float sa[SS ? 16 * 65 : 1];
  DecSlot* sl = g_dec_slot + p.slot;
  // the call tag: this call's epoch + 1, read before anything else
  const uint32_t tag =
      __hip_atomic_load(&sl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  asm volatile("" ::: "memory");  // keep the epoch load first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t N = p.W.N, K = p.W.K, M = p.M;
  const int64_t n0 = (int64_t)lb * 16;
  const int r = p.r, ET = (int)M * r;
  const int64_t G = K / 32;

  // X chunks first, as gemv_kernel (clamped, branchless)
  const int64_t nxc = M * K / 8, rowc = K / 8;
  u32x4 xc[XC];
  uint32_t xsto[XC];
  if (XL) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      int64_t c = tid + (int64_t)NT * i;
      c = c < nxc ? c : nxc - 1;
      xc[i] = *reinterpret_cast<const u32x4*>(p.X + 8 * c);
      const int64_t m = c / rowc, ch = c - m * rowc;
      xsto[i] = (uint32_t)(m * K + 8 * (ch ^ (m & 15)));
    }
  }
  // producers: granule g0 + wave of the range [g0, g1) (at most one per wave)
  const bool producer = lb < p.P;
  const int64_t g0 = producer ? (int64_t)lb * G / p.P : 0;
  const int64_t g1 = producer ? (int64_t)(lb + 1) * G / p.P : 0;
  const bool twave = producer && g0 + wave < g1;  // wave-uniform
  u32x4 af[JT];
  if (twave) {
    const int64_t k = 32 * (g0 + wave) + 8 * q;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int j = 16 * jt + l16;
      af[jt] = *reinterpret_cast<const u32x4*>(p.A + (int64_t)(j < r ? j : 0) * K + k);
    }
  }
  const int EB = 16 * r;
  const int tb = tid < EB ? tid : EB - 1;
  const uint16_t braw = p.B[n0 * r + tb];
  // SS: thread t < 16 KB loads the constants of block t of the 16 rows (row
  // t / KB, block t % KB; consecutive threads read consecutive bytes)
  const int KB = (int)(K / 64);
  uint32_t sraw = 0;
  float sc2raw = 1.0f;
  if (SS) {
    const int tq = tid < 16 * KB ? tid : 16 * KB - 1;
    const int64_t e = n0 * KB + tq;
    if (WK == kNF4DQ) {
      sraw = p.W.q8[e];
      sc2raw = p.W.c2[e >> 8];
    } else {
      sraw = __float_as_uint(p.W.absmax[e]);
    }
  }

  const int64_t n = n0 + l16;
  const bool mrow = l16 < M;
  const int64_t xm = mrow ? l16 : 0;
  f32x4 acc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t steps = (G + 3) / 4;
  u32x4 wraw[CH][WK == kDense ? 4 : 1];
  uint32_t sq[CH];
  float sc2[CH];
  u32x4 xf[CH][4];
  int64_t kx[CH];
  bool ok[CH];
  auto load = [&](int64_t base) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t t = base + kGemvWaves * i;
      const int64_t g = 4 * t + q;
      ok[i] = t < steps && g < G;
      const int64_t k = ok[i] ? 32 * g : 0;
      const int64_t e = n * K + k;
      if (WK == kDense) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          wraw[i][d] = *reinterpret_cast<const u32x4*>(p.W.dense + e + 8 * d);
      } else {
        wraw[i][0] = *reinterpret_cast<const u32x4*>(p.W.codes + (e >> 1));
        if (SS) {
        } else if (WK == kNF4DQ) {
          sq[i] = p.W.q8[e >> 6];
          sc2[i] = p.W.c2[e >> 14];
        } else {
          sq[i] = __float_as_uint(p.W.absmax[e >> 6]);
        }
      }
      kx[i] = xm * K + k;
      if (!XL)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          xf[i][d] = *reinterpret_cast<const u32x4*>(p.X + kx[i] + 8 * d);
      else
        kx[i] = k >> 3;
      ok[i] = ok[i] && mrow;
    }
  };
  load(wave);
  if (WK != kDense) build_lut(lut, p.tab);
  if (XL) {
#pragma unroll
    for (int i = 0; i < XC; ++i) *reinterpret_cast<u32x4*>(xs + xsto[i]) = xc[i];
  }
  if (tid < EB) {
    const int nn = tid / r, j = tid - nn * r;
    tB[nn * 64 + j] = bf16_to_f32(braw);
  }
  if (SS && tid < 16 * KB) {
    const int rr = tid / KB;
    sa[rr * 65 + (tid - rr * KB)] =
        WK == kNF4DQ ? dq_q_rt(p.W.dq, sraw) * dq_step(sc2raw) : __uint_as_float(sraw);
  }
  __syncthreads();  // level table, staged X, B rows, block scales
  // count this workgroup in: its epoch load, issued before the loads waited
  // for above, has returned (loads complete in order)
  if (tid == 0)
    __hip_atomic_fetch_add(&sl->started[blockIdx.x & 7][0], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);

  // ---- producers: the partial sums of T over [g0, g1), added over the waves
  // through LDS one rank tile at a time; lane (q, l16) of a wave holds
  // T[m = l16][j = 16 jt + 4 q + i]
  if (producer) {
    f32x4 ta[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) ta[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (twave) {
      // granules g0 + wave, g0 + wave + 16, ... (the first one's A fragments
      // were loaded up front)
      for (int64_t g = g0 + wave; g < g1; g += kGemvWaves) {
        const int64_t k = 32 * g + 8 * q;
        u32x4 x;
        if (XL)
          x = *reinterpret_cast<const u32x4*>(xs + xm * K + 8 * ((k >> 3) ^ (xm & 15)));
        else
          x = *reinterpret_cast<const u32x4*>(p.X + xm * K + k);
        x = sel4(mrow, x);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const int j = 16 * jt + l16;
          const u32x4 a = g == g0 + wave
                              ? af[jt]
                              : *reinterpret_cast<const u32x4*>(p.A + (int64_t)(j < r ? j : 0) * K + k);
          ta[jt] = mfma16(sel4(j < r, a), x, ta[jt]);
        }
      }
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      part[wave][lane] = ta[jt];
      __syncthreads();
      if (wave == 0 && mrow) {
        f32x4 s4 = part[0][lane];
        for (int w = 1; w < kGemvWaves; ++w) {
          const f32x4 o = part[w][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] += o[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * jt + 4 * q + i;
          if (j < r)
            __hip_atomic_store(&sl->part[(pbase + lb) * kDecMaxT + l16 * r + j],
                               tagged(tag, s4[i]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
    }
  }

  // ---- the weight stream
  for (int64_t base = wave; base < steps; base += kGemvWaves * CH) {
    if (base != wave) load(base);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (XL)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          xf[i][d] = *reinterpret_cast<const u32x4*>(
              xs + xm * K + 8 * ((kx[i] + d) ^ (xm & 15)));
      if (WK == kDense) {
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[i] = mfma16(wraw[i][d], sel4(ok[i], xf[i][d]), acc[i]);
      } else {
        // SS: the granule's block within its row, (4 t + q) / 2
        // (granules past the row's end read the last block's scale: their
        // activations are masked, and an unwritten scale could be NaN)
        const int sblk = (int)((4 * (base + kGemvWaves * i) + q) >> 1);
        const float a = SS ? sa[l16 * 65 + (sblk < KB ? sblk : KB - 1)]
                        : WK == kNF4DQ ? dq_q_rt(p.W.dq, sq[i]) * dq_step(sc2[i])
                                       : __uint_as_float(sq[i]);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          acc[i] = mfma16(deq8(wraw[i][0][d], a, lut), sel4(ok[i], xf[i][d]), acc[i]);
      }
    }
  }
  f32x4 a0 = acc[0];
#pragma unroll
  for (int i = 1; i < CH; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) a0[v] += acc[i][v];
  part[wave][lane] = a0;

  // workgroup 0, wave 0: read the eight started counters now (lane x reads
  // counter x & 7), while the T words, the expand and the stores are still
  // ahead; the values are used at the end
  const bool ep = blockIdx.x == 0 && wave == 0;
  uint32_t cv = 0;
  if (ep)
    cv = __hip_atomic_load(&sl->started[lane & 7][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- T: thread e < M r reads element e's P partial words (all loads in
  // flight together), re-reads any that is not yet this call's (bounded), and
  // adds them in producer order
  bool got = p.spin >= 0;
  if (tid < ET && got) {
    uint64_t v[kDecMaxP];
#pragma unroll
    for (int b = 0; b < kDecMaxP; ++b)
      if (b < p.P)
        v[b] = __hip_atomic_load(&sl->part[(pbase + b) * kDecMaxT + tid], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    float t = 0.0f;
#pragma unroll
    for (int b = 0; b < kDecMaxP; ++b) {
      if (b < p.P) {
        int it = 0;
        while ((uint32_t)(v[b] >> 32) != tag && got) {
          if (++it > p.spin) got = false;
          __builtin_amdgcn_s_sleep(1);
          v[b] = __hip_atomic_load(&sl->part[(pbase + b) * kDecMaxT + tid],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        t += __uint_as_float((uint32_t)v[b]);
      }
    }
    tT[64 * (tid / r) + tid % r] = t;
  }
  const bool gave_up = __syncthreads_or(!got);
  if (wave != 0) return;
  if (gave_up) {
    if (lane == 0)
      __hip_atomic_fetch_add(&g_dec_giveups, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    dec_t_direct(p, tT);
  }
  if (lb == 0 && p.T_out)
    for (int e = lane; e < ET; e += 64) p.T_out[e] = tT[64 * (e / r) + e % r];
  f32x4 sum = part[0][lane];
#pragma unroll
  for (int w = 1; w < kGemvWaves; ++w) {
    const f32x4 o = part[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += o[i];
  }
  if (mrow) {
    const int m = l16;
    float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < r; ++j) {
      const float t = tT[m * 64 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = fmaf(t, tB[(4 * q + i) * 64 + j], d[i]);
    }
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = sum[i] + p.s * d[i];
    *reinterpret_cast<u32x2*>(p.Y + m * N + n0 + 4 * q) =
        u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  }
  // ---- workgroup 0, last: once every workgroup has read the epoch (the
  // counters read above, re-read while short), move it on
  if (ep) {
    uint32_t c = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) c += (uint32_t)__shfl((int)cv, x);
    if (lane == 0) {
      int it = 0;
      while (c < gridDim.x && ++it <= dispatch::kDefaultWaitPolls) {
        __builtin_amdgcn_s_sleep(1);
        c = 0;
#pragma unroll
        for (int x = 0; x < 8; ++x)
          c += __hip_atomic_load(&sl->started[x][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int x = 0; x < 8; ++x)
        __hip_atomic_store(&sl->started[x][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&sl->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int WK, int XS, int JT, bool SS>
__global__ __launch_bounds__(64 * kGemvWaves) void dq_kernel(DecParams p) {
  dq_body<WK, XS, JT, SS>(p, (int)blockIdx.x, 0);
}

// Several adapted layers that read the same activations (the query, key and
// value projections of an attention block, the gate and up projections of its
// MLP) in one launch.  The layers' 16-row blocks are numbered one after the
// other (layer g owns blocks blk0 .. blk0 + N_g / 16 - 1) and the grid has at
// most one workgroup per compute unit: workgroup w takes a contiguous range of
// blocks in turn (consecutive weight rows, mostly of one layer), and the code
// loads (and constants and B rows) of its next block are issued before it
// works on the current one, so that their memory latency overlaps the
// dequantisation, the expand and the stores of the current block.  A layer's
// T is read once per workgroup, at its first block of that layer.  Each
// block's work is the single-layer decode's with 8 waves (each two granules
// per lane more, so that the registers of two blocks in flight fit): the
// waves split the reduction, dequantised codes feed 16 x 16 x 32 MFMAs, wave
// partials are added through LDS, then the rank-r expand.  The
// first nprod workgroups also form partial sums of T, producer pbase + i of
// layer g reducing its share of that layer's A, published as tagged words
// in the stream's slot before their first block; a workgroup reads a
// layer's words after the stream of its first block of that layer.  All
// layers share X, K, r, the weight format and the call's tag.
constexpr int kDecMaxGroup = kDecodeMaxGroup;
struct DecLayer {
  WeightArgs W;
  const uint16_t* A;
  const uint16_t* B;
  float* T_out;
  uint16_t* Y;
  float s;
  int32_t blk0, P, pbase;
};
struct DecGroupParams {
  DecParams c;  // X, M, r, tab, slot, spin, and layer 0's weight (K, format)
  DecLayer l[kDecMaxGroup];
  int32_t n;        // layers
  int32_t nblocks;  // 16-row blocks of all layers
  int32_t nprod;    // producers of all layers
};

// Index of the layer whose range holds v (blocks, or producers when prod);
// wave-uniform.  The kernel keeps layer indexes and reads a layer's fields
// from the argument block where it needs them.
__device__ __forceinline__ int dec_layer_at(const DecGroupParams& gp, int v, bool prod) {
  int g = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxGroup; ++i)
    if (i < gp.n && v >= (prod ? gp.l[i].pbase : gp.l[i].blk0)) g = i;
  return g;
}

// waves of a grouped-decode workgroup, and granules per lane and round (one
// round covers K = 4096): 256 registers per lane with one workgroup per
// compute unit
constexpr int kDecGWaves = 8, kDecGCH = 4;

template <int WK, bool SS>
struct DecBlockLoads {
  u32x4 w[kDecGCH][WK == kDense ? 4 : 1];  // one round of this lane's granules
  uint32_t sq[kDecGCH];                    // their block constants (not SS)
  float sc2[kDecGCH];
  // SS: the constants of blocks tid and tid + 64 kDecGWaves of the 16 rows
  uint32_t sraw[2];
  float sc2raw[2];
  uint16_t braw[2];  // elements tid and tid + 64 kDecGWaves of its 16 rows of B
};

template <int WK, int XS, int JT, bool SS>
__global__ __launch_bounds__(64 * kDecGWaves) void dqg_kernel(DecGroupParams gp) {
  constexpr bool XL = XS > 0;
  constexpr int CH = kDecGCH;
  constexpr int NT = 64 * kDecGWaves;
  constexpr int XC = XL ? XS / 8 / NT : 1;
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? XS : 8];
  __shared__ float2 lut[256];
  __shared__ f32x4 part[kDecGWaves][64];
  __shared__ float tB[16 * 64];
  __shared__ float tT[16 * 64];
  __shared__ float sa[SS ? 16 * 65 : 1];
  const DecParams& c = gp.c;
  DecSlot* sl = g_dec_slot + c.slot;
  const uint32_t tag =
      __hip_atomic_load(&sl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  asm volatile("" ::: "memory");  // keep the epoch load first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t K = c.W.K, M = c.M;
  const int r = c.r, ET = (int)M * r;
  const int64_t G = K / 32;
  const int64_t steps = (G + 3) / 4;
  const int KB = (int)(K / 64);
  const int EB = 16 * r;
  // B elements and (SS) block constants: two per thread (16 r and 16 K / 64
  // are at most 1024)
  int tb[2], tq[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + NT * u;
    tb[u] = e < EB ? e : EB - 1;
    tq[u] = SS ? (e < 16 * KB ? e : 16 * KB - 1) : 0;
  }
  const bool mrow = l16 < M;
  const int64_t xm = mrow ? l16 : 0;

  // X chunks first (clamped, branchless), staged in LDS below
  const int64_t nxc = M * K / 8, rowc = K / 8;
  u32x4 xc[XC];
  uint32_t xsto[XC];
  if (XL) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      int64_t ci = tid + (int64_t)NT * i;
      ci = ci < nxc ? ci : nxc - 1;
      xc[i] = *reinterpret_cast<const u32x4*>(c.X + 8 * ci);
      const int64_t m = ci / rowc, ch = ci - m * rowc;
      xsto[i] = (uint32_t)(m * K + 8 * (ch ^ (m & 15)));
    }
  }
  // producer role: granules [g0, g1) of its layer's reduction, one per wave
  // (the first one's A fragments loaded now)
  const bool producer = (int)blockIdx.x < gp.nprod;
  const DecLayer& PL = gp.l[dec_layer_at(gp, producer ? (int)blockIdx.x : 0, true)];
  const int lp = (int)blockIdx.x - PL.pbase;
  const int64_t g0 = producer ? (int64_t)lp * G / PL.P : 0;
  const int64_t g1 = producer ? (int64_t)(lp + 1) * G / PL.P : 0;
  const bool twave = producer && g0 + wave < g1;  // wave-uniform
  u32x4 af[JT];
  if (twave) {
    const int64_t k = 32 * (g0 + wave) + 8 * q;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int j = 16 * jt + l16;
      af[jt] = *reinterpret_cast<const u32x4*>(PL.A + (int64_t)(j < r ? j : 0) * K + k);
    }
  }

  // loads of one round (granule steps base, base + 16) of block bid
  auto issue_round = [&](DecBlockLoads<WK, SS>& o, int gi, int bid, int64_t base) {
    const DecLayer& L = gp.l[gi];
    const int64_t n = (int64_t)(bid - L.blk0) * 16 + l16;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t t = base + kDecGWaves * i;
      const int64_t g = 4 * t + q;
      const bool ok = t < steps && g < G;
      const int64_t e = n * K + (ok ? 32 * g : 0);
      if (WK == kDense) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o.w[i][d] = *reinterpret_cast<const u32x4*>(L.W.dense + e + 8 * d);
      } else {
        o.w[i][0] = *reinterpret_cast<const u32x4*>(L.W.codes + (e >> 1));
        if (SS) {
        } else if (WK == kNF4DQ) {
          o.sq[i] = L.W.q8[e >> 6];
          o.sc2[i] = L.W.c2[e >> 14];
        } else {
          o.sq[i] = __float_as_uint(L.W.absmax[e >> 6]);
        }
      }
    }
  };
  // the block's B rows and (SS) the constants of its 16 rows
  auto issue_consts = [&](DecBlockLoads<WK, SS>& o, int gi, int bid) {
    const DecLayer& L = gp.l[gi];
    const int64_t n0 = (int64_t)(bid - L.blk0) * 16;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      o.braw[u] = L.B[n0 * r + tb[u]];
      if (SS) {
        const int64_t e = n0 * KB + tq[u];
        if (WK == kNF4DQ) {
          o.sraw[u] = L.W.q8[e];
          o.sc2raw[u] = L.W.c2[e >> 8];
        } else {
          o.sraw[u] = __float_as_uint(L.W.absmax[e]);
        }
      }
    }
  };

  // this workgroup's blocks: a contiguous range (consecutive rows, mostly of
  // one layer, so that a layer's T is read once per workgroup)
  const int bend = (int)(((int64_t)blockIdx.x + 1) * gp.nblocks / gridDim.x);
  int bid = (int)((int64_t)blockIdx.x * gp.nblocks / gridDim.x);
  int gi = dec_layer_at(gp, bid < bend ? bid : 0, false);
  int tlayer = -1;  // the layer whose T is in tT
  DecBlockLoads<WK, SS> cur;
  issue_round(cur, gi, bid, wave);
  issue_consts(cur, gi, bid);
  if (WK != kDense) build_lut(lut, c.tab);
  if (XL) {
#pragma unroll
    for (int i = 0; i < XC; ++i) *reinterpret_cast<u32x4*>(xs + xsto[i]) = xc[i];
  }
  __syncthreads();  // level table, staged X
  // count this workgroup in: its epoch load, issued before the loads waited
  // for above, has returned (loads complete in order)
  if (tid == 0)
    __hip_atomic_fetch_add(&sl->started[blockIdx.x & 7][0], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);

  // ---- producers: partial sums of their layer's T over [g0, g1), added
  // over the waves through LDS one rank tile at a time
  if (producer) {
    f32x4 ta[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) ta[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (twave) {
      for (int64_t g = g0 + wave; g < g1; g += kDecGWaves) {
        const int64_t k = 32 * g + 8 * q;
        u32x4 x;
        if (XL)
          x = *reinterpret_cast<const u32x4*>(xs + xm * K + 8 * ((k >> 3) ^ (xm & 15)));
        else
          x = *reinterpret_cast<const u32x4*>(c.X + xm * K + k);
        x = sel4(mrow, x);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const int j = 16 * jt + l16;
          const u32x4 a =
              g == g0 + wave
                  ? af[jt]
                  : *reinterpret_cast<const u32x4*>(PL.A + (int64_t)(j < r ? j : 0) * K + k);
          ta[jt] = mfma16(sel4(j < r, a), x, ta[jt]);
        }
      }
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      part[wave][lane] = ta[jt];
      __syncthreads();
      if (wave == 0 && mrow) {
        f32x4 s4 = part[0][lane];
        for (int w = 1; w < kDecGWaves; ++w) {
          const f32x4 o = part[w][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] += o[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * jt + 4 * q + i;
          if (j < r)
            __hip_atomic_store(&sl->part[blockIdx.x * kDecMaxT + l16 * r + j],
                               tagged(tag, s4[i]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
    }
  }

  // ---- the blocks
  for (; bid < bend; ++bid) {
    const int nb = bid + 1;
    const bool more = nb < bend;
    const int gn = dec_layer_at(gp, more ? nb : bid, false);
    DecBlockLoads<WK, SS> nxt;
    if (more) {
      issue_round(nxt, gn, nb, wave);
      issue_consts(nxt, gn, nb);
    }
    const DecLayer& L = gp.l[gi];
    const int lb = bid - L.blk0;
    const int64_t N = L.W.N, n0 = (int64_t)lb * 16;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + NT * u;
      if (e < EB) {
        const int nn = e / r, j = e - nn * r;
        tB[nn * 64 + j] = bf16_to_f32(cur.braw[u]);
      }
      if (SS && e < 16 * KB) {
        const int rr = e / KB;
        sa[rr * 65 + (e - rr * KB)] =
            WK == kNF4DQ ? dq_q_rt(L.W.dq, cur.sraw[u]) * dq_step(cur.sc2raw[u])
                         : __uint_as_float(cur.sraw[u]);
      }
    }
    __syncthreads();  // B rows, block scales

    f32x4 acc[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t base = wave; base < steps; base += kDecGWaves * CH) {
      if (base != wave) issue_round(cur, gi, bid, base);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int64_t t = base + kDecGWaves * i;
        const int64_t g = 4 * t + q;
        const bool ok = t < steps && g < G && mrow;
        const int64_t kk = ok ? 32 * g : 0;
        u32x4 xf[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
          xf[d] = XL ? *reinterpret_cast<const u32x4*>(
                           xs + xm * K + 8 * (((kk >> 3) + d) ^ (xm & 15)))
                     : *reinterpret_cast<const u32x4*>(c.X + xm * K + kk + 8 * d);
        if (WK == kDense) {
#pragma unroll
          for (int d = 0; d < 4; ++d) acc[i] = mfma16(cur.w[i][d], sel4(ok, xf[d]), acc[i]);
        } else {
          // (granules past the row's end read the last block's scale: their
          // activations are masked, and an unwritten scale could be NaN)
          const int sblk = (int)((4 * t + q) >> 1);
          const float a = SS ? sa[l16 * 65 + (sblk < KB ? sblk : KB - 1)]
                          : WK == kNF4DQ ? dq_q_rt(L.W.dq, cur.sq[i]) * dq_step(cur.sc2[i])
                                         : __uint_as_float(cur.sq[i]);
#pragma unroll
          for (int d = 0; d < 4; ++d)
            acc[i] = mfma16(deq8(cur.w[i][0][d], a, lut), sel4(ok, xf[d]), acc[i]);
        }
      }
    }
    f32x4 a0 = acc[0];
#pragma unroll
    for (int i = 1; i < CH; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) a0[v] += acc[i][v];
    part[wave][lane] = a0;

    // T of this block's layer, unless the previous block's layer was the same
    // (tT holds it then): thread t reads the P words of elements t and
    // t + 64 kDecGWaves (below M r; all of an element's words in flight),
    // re-reads any that is not yet this call's (bounded), adds them in
    // producer order
    const bool tnew = gi != tlayer;  // wave-uniform
    bool got = c.spin >= 0;
    for (int e = tid; e < ET && got && tnew; e += NT) {
      uint64_t v[kDecMaxP];
#pragma unroll
      for (int b = 0; b < kDecMaxP; ++b)
        if (b < L.P)
          v[b] = __hip_atomic_load(&sl->part[(L.pbase + b) * kDecMaxT + e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      float tsum = 0.0f;
#pragma unroll
      for (int b = 0; b < kDecMaxP; ++b) {
        if (b < L.P) {
          int it = 0;
          while ((uint32_t)(v[b] >> 32) != tag && got) {
            if (++it > c.spin) got = false;
            __builtin_amdgcn_s_sleep(1);
            v[b] = __hip_atomic_load(&sl->part[(L.pbase + b) * kDecMaxT + e], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
          tsum += __uint_as_float((uint32_t)v[b]);
        }
      }
      tT[64 * (e / r) + e % r] = tsum;
    }
    const bool gave_up = __syncthreads_or(!got);
    tlayer = gi;
    if (wave == 0) {
      if (gave_up && tnew) {
        if (lane == 0)
          __hip_atomic_fetch_add(&g_dec_giveups, 1ull, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        DecParams fp = c;
        fp.A = L.A;
        dec_t_direct(fp, tT);
      }
      if (lb == 0 && L.T_out)
        for (int e = lane; e < ET; e += 64) L.T_out[e] = tT[64 * (e / r) + e % r];
      f32x4 sum = part[0][lane];
#pragma unroll
      for (int w = 1; w < kDecGWaves; ++w) {
        const f32x4 o = part[w][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += o[i];
      }
      if (mrow) {
        const int m = l16;
        float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int j = 0; j < r; ++j) {
          const float t = tT[m * 64 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] = fmaf(t, tB[(4 * q + i) * 64 + j], d[i]);
        }
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = sum[i] + L.s * d[i];
        *reinterpret_cast<u32x2*>(L.Y + m * N + n0 + 4 * q) =
            u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      }
    }
    __syncthreads();  // part, tT, tB and sa are rewritten for the next block
    if (more) {
      cur = nxt;
      gi = gn;
    }
  }

  // ---- workgroup 0, last: once every workgroup has read the epoch, move it on
  if (blockIdx.x == 0 && tid == 0) {
    uint32_t cnt = 0;
    int it = 0;
    for (;;) {
      cnt = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x)
        cnt += __hip_atomic_load(&sl->started[x][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (cnt >= gridDim.x || ++it > dispatch::kDefaultWaitPolls) break;
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
      __hip_atomic_store(&sl->started[x][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&sl->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Partial sums of T = X A^T for one 16-row chunk (blockIdx.y) of up to 64
// rows, kTParts x 16 x r floats per chunk: workgroup b reduces granules
// [b G / kTParts, (b + 1) G / kTParts) of the G = K / 32 granules of 32
// reduction elements; its four waves take every fourth granule and run
// v_mfma_f32_16x16x32_bf16 with A rows as the A operand (16 per tile, JT
// tiles) and the activation rows as the B operand; the wave partials are added
// through LDS and Tp[b] (M x r) is written.  The decode GEMV adds the
// kTParts partials in a fixed order.
template <int JT>
__global__ __launch_bounds__(kThreads) void tpart_kernel(const uint16_t* __restrict__ X, int64_t M,
                                                         int64_t K, const uint16_t* __restrict__ A,
                                                         int r, float* __restrict__ Tp) {
  constexpr int CH = 4;
  __shared__ f32x4 part[4][JT][64];
  {  // 16-row chunk blockIdx.y (the decode GEMV reads this chunk's partials)
    const int64_t m0 = 16 * (int64_t)blockIdx.y;
    X += m0 * K;
    M = M - m0 < 16 ? M - m0 : 16;
    Tp += (int64_t)blockIdx.y * kTParts * 16 * r;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, q = lane >> 4;
  const bool mrow = l16 < M;
  const int64_t xm = mrow ? l16 : 0;
  const int64_t G = K / 32;
  const int64_t g0 = (int64_t)blockIdx.x * G / kTParts, g1 = (int64_t)(blockIdx.x + 1) * G / kTParts;
  f32x4 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t gb = g0 + wave; gb < g1; gb += 4 * CH) {
    u32x4 af[CH][JT], xf[CH];
    bool ok[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t g = gb + 4 * i;
      ok[i] = g < g1;
      const int64_t k = 32 * (ok[i] ? g : g0) + 8 * q;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const int j = 16 * jt + l16;
        af[i][jt] = *reinterpret_cast<const u32x4*>(A + (int64_t)(j < r ? j : 0) * K + k);
      }
      // every lane loads (rows past M read row 0, masked below): no branch
      xf[i] = *reinterpret_cast<const u32x4*>(X + xm * K + k);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const u32x4 x = sel4(ok[i] && mrow, xf[i]);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        acc[jt] = mfma16(sel4(16 * jt + l16 < r, af[i][jt]), x, acc[jt]);
    }
  }
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) part[wave][jt][lane] = acc[jt];
  __syncthreads();
  // thread -> (jt, lane) of the sum; lane holds rows j = 16 jt + 4 q + i, column m = l16
  if (tid < JT * 64) {
    const int jt = tid >> 6, ln = tid & 63;
    f32x4 s4 = part[0][jt][ln];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 o = part[w][jt][ln];
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[i] += o[i];
    }
    const int m = ln & 15, qq = ln >> 4;
    if (m < M) {
      float* out = Tp + (int64_t)blockIdx.x * M * r + m * r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * jt + 4 * qq + i;
        if (j < r) out[j] = s4[i];
      }
    }
  }
}

}  // namespace

namespace dispatch {

int t_only(const void* X, int64_t M, int64_t K, const void* A, int64_t r, float* T,
           hipStream_t st, int32_t* zero, int nzero, float oscale) {
  MultiTab sc{};
  sc.oscale = oscale;
  if (shrink_eligible(false, r))
    return launch_shrink(X, M, K, A, false, r, T, zero, nzero, st, nullptr, &sc);
  const int e = launch_skinny((const uint16_t*)X, M, K, (const uint16_t*)A, false, r, T, zero,
                              nzero, st);
  if (e || oscale == 1.0f) return e;
  return launch_t_finish(T, M, r, oscale, 0.0f, nullptr, 0, st);
}

int u_only(const void* dY, int64_t M, int64_t N, const void* B, int64_t r, float* U,
           hipStream_t st, int32_t* zero, int nzero, float oscale) {
  MultiTab sc{};
  sc.oscale = oscale;
  if (shrink_eligible(true, r))
    return launch_shrink(dY, M, N, B, true, r, U, zero, nzero, st, nullptr, &sc);
  const int e = launch_skinny((const uint16_t*)dY, M, N, (const uint16_t*)B, true, r, U, zero,
                              nzero, st);
  if (e || oscale == 1.0f) return e;
  return launch_t_finish(U, M, r, oscale, 0.0f, nullptr, 0, st);
}

// Slot of a stream on the current device: one per (device, stream) pair,
// given out in order of first use; past kDecSlots streams on one device the
// slots are shared (stream index modulo kDecSlots), so two such streams must
// not run decode calls at the same time.
static int stream_slot(hipStream_t st) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, int> slots;
  static std::map<int, int> used;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_pair(dev, st);
  auto it = slots.find(key);
  if (it != slots.end()) return it->second;
  const int id = used[dev]++ % kDecSlots;
  slots.emplace(key, id);
  return id;
}

// producers: enough that each reduces at most one granule per wave (up to
// kDecMaxP; past that a wave takes several), and at most the grid
static int dec_producers(int64_t N, int64_t K) {
  int64_t P = cdiv(K / 32, kGemvWaves);
  P = P < kDecMaxP ? P : kDecMaxP;
  return (int)(P < N / 16 ? P : N / 16);
}

size_t decode1_floats(int64_t, int64_t, int64_t, int64_t) { return 0; }

int take_decode_giveups(uint64_t* n) {
  unsigned long long v = 0, z = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dec_giveups), sizeof(v));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_dec_giveups), &z, sizeof(z));
  *n = v;
  return hip_fail(e, "decode give-up count");
}

template <int WK, int XS, int JT, bool SS>
static void dec_launch(const DecParams* p, const DecGroupParams* gp, unsigned blocks,
                       hipStream_t st) {
  const dim3 grid(blocks);
  if (gp)
    hipLaunchKernelGGL((dqg_kernel<WK, XS, JT, SS>), grid, dim3(64 * kDecGWaves), 0, st, *gp);
  else
    hipLaunchKernelGGL((dq_kernel<WK, XS, JT, SS>), grid, dim3(64 * kGemvWaves), 0, st, *p);
}

// Picks the instance of the one-launch decode for the weight format, the size
// of the activations and the rank, and launches it over `blocks` workgroups
// (the single-layer kernel when gp is NULL, else the grouped one).
static int dec_select_launch(const lq_weight& W, int64_t M, int64_t r, const DecParams* p,
                             const DecGroupParams* gp, unsigned blocks, hipStream_t st) {
  const int64_t mk = M * W.K;
  const int xs = W.K % 128 ? 0 : mk <= 16384 ? 1 : mk <= 65536 ? 2 : 0;
  const int jt = r <= 16 ? 0 : r <= 32 ? 1 : 2;
  // block scales staged per workgroup for an NF4 weight with K <= 4096
  const bool ss = W.kind == LQ_WEIGHT_NF4 && W.K <= 4096;
  const int sel = ((weight_format(W) * 3 + xs) * 3 + jt) * 2 + (ss ? 1 : 0);
#define LQ_DEC(WKv, XSv, JTv, SSv, idx)                \
  case idx:                                            \
    dec_launch<WKv, XSv, JTv, SSv>(p, gp, blocks, st); \
    break;
#define LQ_DEC3(WKv, XSv, base)                                                    \
  LQ_DEC(WKv, XSv, 1, false, 2 * (base)) LQ_DEC(WKv, XSv, 2, false, 2 * (base) + 2) \
  LQ_DEC(WKv, XSv, 4, false, 2 * (base) + 4)
#define LQ_DEC3S(WKv, XSv, base)                                                   \
  LQ_DEC3(WKv, XSv, base)                                                          \
  LQ_DEC(WKv, XSv, 1, true, 2 * (base) + 1) LQ_DEC(WKv, XSv, 2, true, 2 * (base) + 3) \
  LQ_DEC(WKv, XSv, 4, true, 2 * (base) + 5)
  switch (sel) {
    LQ_DEC3(kDense, 0, 0)
    LQ_DEC3(kDense, 16384, 3)
    LQ_DEC3(kDense, 65536, 6)
    LQ_DEC3S(kNF4DQ, 0, 9)
    LQ_DEC3S(kNF4DQ, 16384, 12)
    LQ_DEC3S(kNF4DQ, 65536, 15)
    LQ_DEC3S(kNF4, 0, 18)
    LQ_DEC3S(kNF4, 16384, 21)
    LQ_DEC3S(kNF4, 65536, 24)
    default: break;
  }
#undef LQ_DEC3S
#undef LQ_DEC3
#undef LQ_DEC
  return hip_fail(hipGetLastError(), "decode launch");
}

int decode_fwd1(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
                int64_t r, float s, void* Y, float* T_out, float*, hipStream_t st) {
  DecParams p;
  p.X = (const uint16_t*)X;
  p.M = M;
  p.W = weight_args(W);
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.T_out = T_out;
  p.r = (int32_t)r;
  p.s = s;
  p.Y = (uint16_t*)Y;
  p.tab = nf4_table(W.codebook);
  p.P = dec_producers(W.N, W.K);
  p.slot = stream_slot(st);
  p.spin = wait_limit();
  return dec_select_launch(W, M, r, &p, nullptr, (unsigned)(W.N / 16), st);
}

int decode_fwd_group(const void* X, int64_t M, int32_t n, const lq_weight* W,
                     const void* const* A, const void* const* B, int64_t r, const float* s,
                     void* const* Y, float* const* T_out, hipStream_t st) {
  DecGroupParams gp;
  memset(&gp, 0, sizeof(gp));
  gp.c.X = (const uint16_t*)X;
  gp.c.M = M;
  gp.c.r = (int32_t)r;
  gp.c.tab = nf4_table(W[0].codebook);
  gp.c.slot = stream_slot(st);
  gp.c.spin = wait_limit();
  gp.c.W = weight_args(W[0]);
  gp.n = n;
  // producers per layer: at most kDecMaxP in all
  const int pmax = kDecMaxP / n;
  int32_t blk = 0, pb = 0;
  for (int g = 0; g < n; ++g) {
    DecLayer& L = gp.l[g];
    L.W = weight_args(W[g]);
    L.A = (const uint16_t*)A[g];
    L.B = (const uint16_t*)B[g];
    L.T_out = T_out ? T_out[g] : nullptr;
    L.Y = (uint16_t*)Y[g];
    L.s = s[g];
    const int pg = dec_producers(W[g].N, W[g].K);
    L.P = pg < pmax ? pg : pmax;
    L.blk0 = blk;
    L.pbase = pb;
    blk += (int32_t)(W[g].N / 16);
    pb += L.P;
  }
  for (int g = n; g < kDecMaxGroup; ++g) gp.l[g].blk0 = gp.l[g].pbase = INT32_MAX;
  gp.nblocks = blk;
  gp.nprod = pb;
  // one workgroup per compute unit at most (a workgroup of this kernel fills
  // one), each taking every grid-th block
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  const int grid = blk < cus ? blk : cus;
  return dec_select_launch(W[0], M, r, nullptr, &gp, (unsigned)(grid > pb ? grid : pb), st);
}

int decode_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
               int64_t r, float s, void* Y, float* T_out, float* Tp, hipStream_t st) {
  const int jt = (int)((r + 15) / 16);
  const uint16_t* Xh = (const uint16_t*)X;
  const uint16_t* Ah = (const uint16_t*)A;
  const unsigned chunks = (unsigned)((M + 15) / 16);  // 16-row chunks, grid dimension y
  const dim3 tg(kTParts, chunks), tb(kThreads);
  switch (jt) {
    case 1:
      hipLaunchKernelGGL(tpart_kernel<1>, tg, tb, 0, st, Xh, M, W.K, Ah, (int)r, Tp);
      break;
    case 2:
      hipLaunchKernelGGL(tpart_kernel<2>, tg, tb, 0, st, Xh, M, W.K, Ah, (int)r, Tp);
      break;
    case 3:
      hipLaunchKernelGGL(tpart_kernel<3>, tg, tb, 0, st, Xh, M, W.K, Ah, (int)r, Tp);
      break;
    default:
      hipLaunchKernelGGL(tpart_kernel<4>, tg, tb, 0, st, Xh, M, W.K, Ah, (int)r, Tp);
      break;
  }
  int e = hip_fail(hipGetLastError(), "tpart launch");
  if (e) return e;
  GemvParams p;
  p.X = Xh;
  p.M = M;
  p.W = weight_args(W);
  p.Tp = Tp;
  p.B = (const uint16_t*)B;
  p.T_out = T_out;
  p.r = (int32_t)r;
  p.s = s;
  p.Y = (uint16_t*)Y;
  p.tab = nf4_table(W.codebook);
  const dim3 grid((unsigned)(W.N / 16), chunks), block(64 * kGemvWaves);
  // staged X (one chunk's rows): 16384 elements keep two workgroups per
  // compute unit; 65536 allows one, and still measured faster than loading X
  // per lane with grids of up to six workgroups per compute unit
  const int64_t mk = (M < 16 ? M : 16) * W.K;
  const int xs = W.K % 128 ? 0 : mk <= 16384 ? 1 : mk <= 65536 ? 2 : 0;
  switch (weight_format(W) * 3 + xs) {
    case kDense * 3 + 0: hipLaunchKernelGGL((gemv_kernel<kDense, 0>), grid, block, 0, st, p); break;
    case kDense * 3 + 1: hipLaunchKernelGGL((gemv_kernel<kDense, 16384>), grid, block, 0, st, p); break;
    case kDense * 3 + 2: hipLaunchKernelGGL((gemv_kernel<kDense, 65536>), grid, block, 0, st, p); break;
    case kNF4DQ * 3 + 0: hipLaunchKernelGGL((gemv_kernel<kNF4DQ, 0>), grid, block, 0, st, p); break;
    case kNF4DQ * 3 + 1: hipLaunchKernelGGL((gemv_kernel<kNF4DQ, 16384>), grid, block, 0, st, p); break;
    case kNF4DQ * 3 + 2: hipLaunchKernelGGL((gemv_kernel<kNF4DQ, 65536>), grid, block, 0, st, p); break;
    case kNF4 * 3 + 0: hipLaunchKernelGGL((gemv_kernel<kNF4, 0>), grid, block, 0, st, p); break;
    case kNF4 * 3 + 1: hipLaunchKernelGGL((gemv_kernel<kNF4, 16384>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((gemv_kernel<kNF4, 65536>), grid, block, 0, st, p); break;
  }
  return hip_fail(hipGetLastError(), "gemv launch");
}

}  // namespace dispatch
}  // namespace lq

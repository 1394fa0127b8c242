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

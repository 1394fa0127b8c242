// Adapter gradients, reduced over the batch rows:
//   dA = s (dY B)^T X   (r x K)      dB = s dY^T (X A^T)   (N x r)
// ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ..."
// (llms.blog), section "Gradient Dynamics and Backpropagation Mechanics",
// summed over the rows of the batch.)
//
// Both have the form out[j][c] = s * sum_m V[m][j] Z[m][c] with V = U or T
// (M x r float32, from the dX / forward kernels) and Z = X or dY (M x C bf16).
// They are skinny (r <= 64 outputs per column) and HBM-bound on Z.  Both run
// in one launch (the grid holds the dA tiles, then the dB tiles).  Each
// workgroup issues the coalesced 16-byte loads of up to four 64-row slabs of
// Z (and the matching rows of V) at once, stores each slab in LDS in storage
// order, reads it back as MFMA operands with the row index m as the reduction
// index, and accumulates a 128-column x r block;
// the rows are split over several workgroups, whose partial sums land in a
// workspace and are added in a fixed order by one small finishing kernel for
// both outputs (deterministic, no atomics), which also applies s and the
// accumulate flag.
#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileC = 128;
constexpr int kChunk = 4;  // 64-row steps whose loads are in flight together

// One reduction job: out[j][c] = s * sum_m V[m][j] Z[m][c] over a range of
// rows, for one 128-column tile of Z.
struct GradJob {
  const uint16_t* Z;   // M x C bf16
  const float* V;      // M x r float32
  int64_t C;
  int32_t c_tiles;
  int32_t splits;
  int64_t rows_per_split;  // multiple of 64
  float* P;            // splits x r x C partial sums
};

struct GradParams {
  GradJob job[2];
  int64_t M;
  int32_t r;
  int32_t blocks0;     // workgroups of job 0; the rest belong to job 1
};

// LDS tile of one 64-row step in storage order: row m holds Z[m][c0 .. c0+127]
// then V[m][0 .. RP-1] (bf16), 16-byte chunk q at q ^ (m & 3), pitch 20 or 28
// chunks.  MFMA operands (one column, eight consecutive rows m) come from the
// transposing LDS read ds_read_b64_tr_b16 (in each 16-lane group lane c
// addresses row c / 4, columns 4 (c % 4) ..; lane i receives column i of the
// four rows), so neither operand is transposed in registers.
template <int RP>
struct GradPitch {
  static constexpr int P = RP == 32 ? 160 : 224;
};

typedef short s16x4g __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4g* lds_ptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p)));
}

template <int RP, bool V4>
__global__ __launch_bounds__(kThreads) void grad_kernel(GradParams p) {
  constexpr int JT = RP / 32;
  constexpr int PT = GradPitch<RP>::P;
  constexpr int NV = RP / 16;  // float4 chunks of V per thread per step (64 rows x RP / 4)
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][64 * PT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const bool second = (int)blockIdx.x >= p.blocks0;
  const GradJob& jb = second ? p.job[1] : p.job[0];
  const int bid = second ? (int)blockIdx.x - p.blocks0 : (int)blockIdx.x;
  const int tl = xcd_tile(bid, jb.c_tiles * jb.splits);
  const int tc = tl % jb.c_tiles, split = tl / jb.c_tiles;
  const int64_t C = jb.C, M = p.M;
  const int64_t c0 = (int64_t)tc * kTileC;
  const int64_t mbeg = (int64_t)split * jb.rows_per_split;
  int64_t mend = mbeg + jb.rows_per_split;
  mend = mend < M ? mend : M;
  const int steps = mend > mbeg ? (int)cdiv(mend - mbeg, 64) : 0;
  const int r = p.r;

  f32x16 acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.0f;

  // Z staging: chunk zc = tid & 15 of rows zr + 16 i (columns past C clamped,
  // zeroed when stored); V staging: row vr = tid / 4, float4 chunks
  // vc = tid % 4 + 4 i (j = 4 vc ..); rows past mend are zeroed when stored.
  const int zc = tid & 15, zr = tid >> 4;
  int64_t zcol = c0 + 8 * zc;
  const bool zok = zcol < C;
  zcol = zok ? zcol : C - 8;
  const int vr = tid >> 2;
  uint32_t zst[4], vst[NV];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = zr + 16 * i;
    zst[i] = (uint32_t)(m * PT + 8 * (zc ^ (m & 3)));
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vc = (tid & 3) + 4 * i;  // float4 chunk: half of 16-byte chunk 16 + vc / 2
    vst[i] = (uint32_t)(vr * PT + 8 * ((16 + (vc >> 1)) ^ (vr & 3)) + 4 * (vc & 1));
  }
  struct Stage {
    u32x4 z[4];
    f32x4 v[NV];
  };
  auto load = [&](int64_t m0r, Stage& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t m = m0r + zr + 16 * i;
      m = m < mend ? m : mend - 1;
      st.z[i] = *reinterpret_cast<const u32x4*>(jb.Z + m * C + zcol);
    }
    int64_t m = m0r + vr;
    m = m < mend ? m : mend - 1;
    const float* row = jb.V + m * r;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j0 = 4 * ((tid & 3) + 4 * i);
      if (V4) {
        st.v[i] = *reinterpret_cast<const f32x4*>(row + (j0 < r ? j0 : 0));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) st.v[i][e] = row[j0 + e < r ? j0 + e : 0];
      }
    }
  };
  auto store = [&](int64_t m0r, const Stage& st, uint16_t* t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = zok && m0r + zr + 16 * i < mend;
      *reinterpret_cast<u32x4*>(t + zst[i]) = sel4(ok, st.z[i]);
    }
    const bool vok = m0r + vr < mend;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j0 = 4 * ((tid & 3) + 4 * i);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (vok && j0 + e < r) ? st.v[i][e] : 0.0f;
      *reinterpret_cast<u32x2*>(t + vst[i]) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  };
  // operand reads: lane (g = lane / 16, c = lane % 16)
  const int c = lane & 15, g = lane >> 4;
  const int rbase = (32 * h + (c >> 2)) * PT + 8 * ((2 * (g & 1) + ((c >> 1) & 1)) ^ (c >> 2)) + 4 * (c & 1);
  auto frag = [&](const uint16_t* t, int col32, int s) {
    const uint16_t* q = t + rbase + 8 * s * PT + 32 * col32;
    const u32x2 lo = lds_tr(q), hi = lds_tr(q + 4 * PT);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // chunks of kChunk steps: all their loads are issued together
  for (int s0 = 0; s0 < steps; s0 += kChunk) {
    Stage st[kChunk];
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int sq = s0 + q < steps ? s0 + q : steps - 1;
      load(mbeg + (int64_t)sq * 64, st[q]);
    }
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      if (s0 + q < steps) {  // uniform
        uint16_t* t = tile[q & 1];
        store(mbeg + (int64_t)(s0 + q) * 64, st[q], t);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 zf = frag(t, wave, s);
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) acc[jt] = mfma32(zf, frag(t, 4 + jt, s), acc[jt]);
        }
      }
    }
    __syncthreads();
  }
  // acc[jt] lane l: rows c = c0 + 32 wave + 8q + 4h + i, column j = 32 jt + l32
  float* P = jb.P + (int64_t)split * r * C;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 32 * jt + l32;
    if (j >= r) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t c = c0 + 32 * wave + 8 * q + 4 * h;
      if (c + 4 <= C) {
        *reinterpret_cast<f32x4*>(P + (int64_t)j * C + c) =
            f32x4{acc[jt][4 * q], acc[jt][4 * q + 1], acc[jt][4 * q + 2], acc[jt][4 * q + 3]};
      } else {
        for (int i = 0; i < 4; ++i)
          if (c + i < C) P[(int64_t)j * C + c + i] = acc[jt][4 * q + i];
      }
    }
  }
}

// Both reductions' finishing pass: out = s * sum_split P[split] (+ out if
// accumulate), the split partials added in a fixed order (four interleaved
// chains, then their pairwise sum).  Index space: dA
// (r x K, out[j][c]) then dB (N x r, out[c][j]).
struct ReduceParams {
  const float* P[2];
  float* out[2];
  int64_t C[2];
  int32_t splits[2];
  int32_t r;
  float s;
  int32_t accumulate;
};

__global__ void grad_reduce_kernel(ReduceParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t0 = (int64_t)p.r * p.C[0];
  const int jb = idx < t0 ? 0 : 1;
  const int64_t total = (int64_t)p.r * p.C[jb];
  const int64_t i = jb ? idx - t0 : idx;
  if (i >= total) return;
  const int64_t C = p.C[jb];
  int64_t j, c;
  if (jb) {  // out[c][j]
    c = i / p.r;
    j = i - c * p.r;
  } else {   // out[j][c]
    j = i / C;
    c = i - j * C;
  }
  const float* P = p.P[jb] + j * C + c;
  const int ns = p.splits[jb];
  // four independent chains, added in a fixed order (split t goes to chain
  // t % 4); eight splits' loads are issued together before any is added
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int t = 0;
  for (; t + 7 < ns; t += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = P[(int64_t)(t + u) * total];
    s0 += v[0];
    s1 += v[1];
    s2 += v[2];
    s3 += v[3];
    s0 += v[4];
    s1 += v[5];
    s2 += v[6];
    s3 += v[7];
  }
  for (; t + 3 < ns; t += 4) {
    s0 += P[(int64_t)t * total];
    s1 += P[(int64_t)(t + 1) * total];
    s2 += P[(int64_t)(t + 2) * total];
    s3 += P[(int64_t)(t + 3) * total];
  }
  for (; t < ns; ++t) s0 += P[(int64_t)t * total];
  const float sum = (s0 + s1) + (s2 + s3);
  float v = p.s * sum;
  if (p.accumulate) v += p.out[jb][i];
  p.out[jb][i] = v;
}

int pick_splits(int64_t M, int64_t C) {
  const int64_t c_tiles = cdiv(C, kTileC);
  int64_t want = cdiv(512, c_tiles);
  const int64_t max_split = cdiv(M, 256);
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  return (int)want;
}

GradJob make_job(const uint16_t* Z, const float* V, int64_t M, int64_t C, float* P) {
  GradJob j;
  j.Z = Z;
  j.V = V;
  j.C = C;
  j.c_tiles = (int)cdiv(C, kTileC);
  j.splits = pick_splits(M, C);
  j.rows_per_split = cdiv(cdiv(M, j.splits), 64) * 64;
  j.P = P;
  return j;
}

// dA = s U^T X (r x K) and dB = s dY^T T (N x r) in one launch plus one
// finishing launch.
int run_grads(const uint16_t* X, const float* U, const uint16_t* dY, const float* T, int64_t M,
              int64_t N, int64_t K, int r, float s, int accumulate, float* dA, float* dB,
              float* PA, float* PB, hipStream_t st) {
  GradParams p;
  p.job[0] = make_job(X, U, M, K, PA);
  p.job[1] = make_job(dY, T, M, N, PB);
  p.M = M;
  p.r = r;
  p.blocks0 = p.job[0].c_tiles * p.job[0].splits;
  const int blocks = p.blocks0 + p.job[1].c_tiles * p.job[1].splits;
  const bool v4 = r % 4 == 0;
  if (r <= 32) {
    if (v4)
      hipLaunchKernelGGL((grad_kernel<32, true>), dim3(blocks), dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((grad_kernel<32, false>), dim3(blocks), dim3(kThreads), 0, st, p);
  } else {
    if (v4)
      hipLaunchKernelGGL((grad_kernel<64, true>), dim3(blocks), dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((grad_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, st, p);
  }
  int e = hip_fail(hipGetLastError(), "grad_kernel launch");
  if (e) return e;
  ReduceParams q;
  q.P[0] = PA;
  q.P[1] = PB;
  q.out[0] = dA;
  q.out[1] = dB;
  q.C[0] = K;
  q.C[1] = N;
  q.splits[0] = p.job[0].splits;
  q.splits[1] = p.job[1].splits;
  q.r = r;
  q.s = s;
  q.accumulate = accumulate;
  const int64_t total = (int64_t)r * (K + N);
  hipLaunchKernelGGL(grad_reduce_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, st, q);
  return hip_fail(hipGetLastError(), "grad_reduce launch");
}

}  // namespace

namespace dispatch {

size_t grad_one_bytes(int64_t M, int64_t C, int64_t r) {
  return (size_t)(pick_splits(M, C) * r * C) * 4 + 512;
}

int grad_one(const void* Z, const float* V, int64_t M, int64_t C, int r, float s, float* out,
             float* part, hipStream_t st) {
  GradParams p;
  p.job[0] = make_job((const uint16_t*)Z, V, M, C, part);
  p.job[1] = p.job[0];  // unused: every workgroup belongs to job 0
  p.M = M;
  p.r = r;
  p.blocks0 = p.job[0].c_tiles * p.job[0].splits;
  const int blocks = p.blocks0;
  const bool v4 = r % 4 == 0;
  if (r <= 32) {
    if (v4)
      hipLaunchKernelGGL((grad_kernel<32, true>), dim3(blocks), dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((grad_kernel<32, false>), dim3(blocks), dim3(kThreads), 0, st, p);
  } else {
    if (v4)
      hipLaunchKernelGGL((grad_kernel<64, true>), dim3(blocks), dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((grad_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, st, p);
  }
  int e = hip_fail(hipGetLastError(), "grad_kernel launch");
  if (e) return e;
  ReduceParams q;
  q.P[0] = part;
  q.P[1] = part;
  q.out[0] = out;
  q.out[1] = out;
  q.C[0] = C;
  q.C[1] = 0;  // empty second part: the grid's rounding threads return at once
  q.splits[0] = p.job[0].splits;
  q.splits[1] = 0;
  q.r = r;
  q.s = s;
  q.accumulate = 1;
  const int64_t total = (int64_t)r * C;  // job 0's index space only
  hipLaunchKernelGGL(grad_reduce_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, st, q);
  return hip_fail(hipGetLastError(), "grad_reduce launch");
}

size_t grad_partial_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t sa = pick_splits(M, K), sb = pick_splits(M, N);
  return (size_t)(sa * r * K + sb * r * N) * 4 + 512;
}

int bf16_bwd(const void* dY, const void* X, int64_t M, const lq_weight& W, const void* A,
             const void* B, int64_t r, float s, const float* T_saved, void* dX, float* dA,
             float* dB, int accumulate, void* ws, void* big_ws, hipStream_t st) {
  const int64_t N = W.N, K = W.K;
  float* U = (float*)ws;
  float* Tw = U + M * r;
  uintptr_t pa = ((uintptr_t)(Tw + M * r) + 255) & ~(uintptr_t)255;
  float* PA = (float*)pa;
  float* PB = PA + (int64_t)pick_splits(M, K) * r * K;
  int e;
  const bool grads = dA != nullptr;  // dX only when both gradients are NULL
  if (M == 0) {
    if (accumulate || !grads) return LQ_OK;
    if ((e = launch_zero_f32(dA, r * K, st))) return e;
    return launch_zero_f32(dB, N * r, st);
  }
  // dX (and U = dY B on the way): for an NF4 weight at large M by the
  // product that dequantises in its K loop (no workspace), unless the
  // large-tile path has its workspace and would run 256 x 256 tiles; by the
  // large-tile path when it has its workspace (for an NF4 weight and at most
  // 64 rows, by the weight-streaming kernel, its partial sums in that
  // workspace), else by the fused kernel
  auto run_dx = [&](float* Uo) {
    if (big_ws && small_dx_eligible(W, M, r)) return small_dx(dY, M, W, A, B, r, s, U, dX, big_ws, st);
    if (inloop_dx_eligible(W, M, r) && !(big_ws && big_wide_tiles(M, W.K)))
      return inloop_dx(dY, M, W, A, B, r, s, dX, Uo, st);
    return big_ws ? big_dx(dY, M, W, A, B, r, s, dX, U, big_ws, st)
                  : bf16_dx(dY, M, W, A, B, r, s, dX, Uo, st);
  };
  if (!grads) return run_dx(nullptr);
  const float* T = T_saved;
  if (!T) {
    if ((e = t_only(X, M, K, A, r, Tw, st, nullptr, 0))) return e;
    T = Tw;
  }
  if (dX) {
    if ((e = run_dx(U))) return e;
  } else {
    if ((e = u_only(dY, M, N, B, r, U, st, nullptr, 0))) return e;
  }
  return run_grads((const uint16_t*)X, U, (const uint16_t*)dY, T, M, N, K, (int)r, s, accumulate,
                   dA, dB, PA, PB, st);
}

// Backward of the dropout forward Y = X W0^T + s (D(X) A^T) B^T with
// D(X) = X * keep * inv_keep:
//   dX = dY W0 + s ((U' A) * keep),  U' = inv_keep (dY B)
//   dA = s U'^T (X * keep),  dB = s dY^T T   (T = D(X) A^T, as the forward left it)
// dX's base term comes from the product kernels run with s = 0 (which also
// give U), its adapter term from the fix-up kernel.
int bf16_bwd_dropout(const void* dY, const void* X, const uint8_t* keep, float inv_keep,
                     int64_t M, const lq_weight& W, const void* A, const void* B, int64_t r,
                     float s, const float* T_saved, void* dX, float* dA, float* dB,
                     int accumulate, void* Xd, void* ws, void* big_ws, hipStream_t st) {
  const int64_t N = W.N, K = W.K;
  float* U = (float*)ws;
  float* Tw = U + M * r;
  uintptr_t pa = ((uintptr_t)(Tw + M * r) + 255) & ~(uintptr_t)255;
  float* PA = (float*)pa;
  float* PB = PA + (int64_t)pick_splits(M, K) * r * K;
  int e;
  const bool grads = dA != nullptr;
  if (M == 0) {
    if (accumulate || !grads) return LQ_OK;
    if ((e = launch_zero_f32(dA, r * K, st))) return e;
    return launch_zero_f32(dB, N * r, st);
  }
  // U' = inv_keep U: in the shrink's stores, except after the fused dX kernel
  if (dX && big_ws) {
    e = big_dx(dY, M, W, A, B, r, 0.0f, dX, U, big_ws, st, inv_keep);
  } else if (dX) {
    if (!(e = bf16_dx(dY, M, W, A, B, r, 0.0f, dX, U, st)))
      e = launch_t_finish(U, M, r, inv_keep, 0.0f, nullptr, 0, st);
  } else {
    e = u_only(dY, M, N, B, r, U, st, nullptr, 0, inv_keep);
  }
  if (e) return e;
  if (dX && (e = launch_dx_fixup(dX, U, A, keep, M, K, r, s, st))) return e;
  if (!grads) return LQ_OK;
  if ((e = launch_keep_apply(X, keep, M, K, Xd, st))) return e;
  const float* T = T_saved;
  if (!T) {
    if ((e = t_only(Xd, M, K, A, r, Tw, st, nullptr, 0, inv_keep))) return e;
    T = Tw;
  }
  return run_grads((const uint16_t*)Xd, U, (const uint16_t*)dY, T, M, N, K, (int)r, s, accumulate,
                   dA, dB, PA, PB, st);
}

}  // namespace dispatch
}  // namespace lq

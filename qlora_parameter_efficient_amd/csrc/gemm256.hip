// Large-M products of the adapted linear layer on gfx950.
//
//   forward  Y  = X Wd^T + (s T) B^T      T = X A^T  (M x r, float32)
//   dX       dX = dY Wd  + (s U) A        U = dY B   (M x r, float32)
//
// ("Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations ..."
// (llms.blog): the forward-pass equation with alpha/r after B, and section
// "Gradient Dynamics and Backpropagation Mechanics" for dL/dx.)  Wd is the
// bf16 weight: the dense W0, or the NF4 weight dequantised to bf16 by the
// dequantisation kernel just before the product ("Large Language Model
// Fine-tuning and LoRA", section on QLoRA: every forward and backward
// multiply runs in bf16 on dequantised blocks).  T and U come from the skinny
// kernels; this kernel does the two large products and the rank-r expand.
//
// Tiles.  A workgroup of 256 threads (4 waves, one per SIMD) owns a 256 x 256
// output tile: i (the weight side: n for the forward, k for dX) by j (the
// activation rows m).  Wave (wi, wj) owns the 128 x 128 block at
// (128 wi, 128 wj): sixteen 32 x 32 MFMA accumulators (256 registers).  The
// output is computed transposed (weight side = MFMA rows), so each lane holds
// four consecutive outputs of one row.
//
// Reduction.  Steps of 64, four 16-wide MFMA substeps each.  Both operand
// tiles of a step (32 KB each) go from global memory straight into LDS with
// gfx950's global_load_lds_dwordx4: lane L of an instruction lands at LDS
// base + 16 L, and the lanes' global addresses are chosen so that every
// instruction reads whole 128-byte lines and the tile comes out swizzled for
// conflict-free operand reads.  Two LDS stages: the loads of step t + 1 are
// issued before the MFMAs of step t; one wait and one barrier per step.
//   * Row tiles (activations, and the forward's weight): 256 rows x 128 bytes;
//     16-byte chunk c of row x sits at chunk c ^ f(x), f(x) = (x & 7) ^ (x >> 3
//     & 1), so the 16-byte operand reads of 16 consecutive rows hit 16
//     distinct bank groups.
//   * dX weight tile: 64 reduction rows n x 256 outputs (512 bytes per row) in
//     storage order; chunk c of row n sits at c ^ 2 (n & 3) ^ 8 (c >> 1 & 1).
//     Operands (one output column, 8 consecutive n) are read with the
//     transposing ds_read_b64_tr_b16; 32 lanes of one read then cover 16
//     distinct bank groups.
// The reduction index of substep s, lane half h is 16 s + 8 h + 0..7 on both
// operands.
//
// Split K.  When there are fewer tiles than compute units, each tile's
// reduction is split between two workgroups.  The first to finish publishes
// its float32 accumulators to a per-tile slot and a ready flag; the second
// adds them to its own and finishes the tile.  The second only ever waits for
// a workgroup that is already past its main loop, so the wait cannot
// deadlock; it is also bounded, and a timeout is recorded in an error word.
// The flags return to zero before the kernel ends, ready for the next call.
//
// Epilogue.  The expand adds (s V) E as extra MFMAs on the finished
// accumulators (V = T or U rounded to bf16 after scaling by s, E = B or A),
// then the tile is staged in LDS as bf16 and written with 16-byte stores that
// cover whole output lines.
#include <type_traits>

#include "device_util.h"
#include "dispatch.h"

namespace lq {
namespace {

constexpr int kGT = 256;                     // tile edge
constexpr int kGK = 64;                      // reduction elements per step
constexpr int kGThreads = 256;
constexpr int kTileBytes = kGT * kGK * 2;    // weight tile of one step: 32 KB

// JM = 32-row activation subtiles per wave: the tile is 256 x 64 JM (JM = 4:
// 256 x 256, JM = 2: 256 x 128 for problems with too few 256 x 256 tiles)
template <int JM>
struct Shape {
  static constexpr int TJ = 64 * JM;                      // activation rows per tile
  static constexpr int PBytes = TJ * kGK * 2;             // activation tile of one step
  static constexpr int Stage = kTileBytes + PBytes;       // LDS stage
  static constexpr int Slot = kGT * TJ;                   // split-K partial (floats)
  static constexpr int NST = 2;                           // LDS stages (3 measured no faster)
  static constexpr int DMA = 8 + 2 * JM;                  // loads per wave per step
};
constexpr int kSpinLimit = 1 << 22;          // split-K wait bound (s_sleep 2 each)

struct G256Params {
  const uint16_t* P;  // activations, M x KR (X or dY)
  const uint16_t* Q;  // bf16 weight: forward NI x KR, dX KR x NI
  const float* V;     // M x r: T (forward) or U (dX)
  const uint16_t* E;  // forward: B (NI x r); dX: A (r x NI)
  uint16_t* Y;        // M x NI
  float* part;        // split-K slots, Shape<JM>::Slot floats per tile
  int32_t* flags;     // split-K (arrivals, ready) per tile, zero between calls
  int32_t* err;       // set to 1 if a split-K wait gave up
  int64_t M, NI, KR;
  int32_t r;
  float s;
  int32_t ti, tj, splits, ksteps;
  int32_t tpx;  // split K: tiles per XCD
  int32_t multi;  // multi-adapter forward: E is the concatenated B, read through col_*
  int32_t col_base[kMaxRankCols];
  int32_t col_stride[kMaxRankCols];
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory (base + off) straight into LDS at
// m0 + 16 * lane.  Issued from asm so that the compiler's wait insertion does
// not make later LDS reads of the other stage wait for it; the kernel waits
// for these loads itself (vmcnt) before the barrier that publishes a stage.
// The instruction has no register results, and its address operands are read
// when it issues.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// wait until at most N of this wave's loads are outstanding
template <int N>
__device__ __forceinline__ void wait_dma_but() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 read_tr(uint32_t addr) {
  typedef __attribute__((address_space(3))) s16x4* lds_ptr;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 read16(uint32_t addr) {
  typedef __attribute__((address_space(3))) const u32x4* lds_ptr;
  return *(lds_ptr)(uintptr_t)addr;
}

// swizzle of the 128-byte-row tiles
__device__ __forceinline__ int rswz(int x) { return (x & 7) ^ ((x >> 3) & 1); }

// physical chunk of logical chunk c in row n of the dX weight tile, and back
__device__ __forceinline__ int tphys(int c, int n) { return c ^ (2 * (n & 3)) ^ (8 * ((c >> 1) & 1)); }
__device__ __forceinline__ int tlogical(int p, int n) {
  return p ^ (2 * (n & 3)) ^ (8 * (((p >> 1) & 1) ^ (n & 1)));
}

// s * v[0..7] rounded to bf16 (MFMA operand), v a float32 row of length r
// starting at rank j0; ranks past r are zero.
__device__ __forceinline__ u32x4 v_operand(const float* row, int j0, int r, float s) {
  float e[8];
  if (j0 + 8 <= r && ((reinterpret_cast<uintptr_t>(row + j0) & 15) == 0)) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + j0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + j0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = a[i];
      e[4 + i] = b[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (j0 + i < r) ? row[j0 + i] : 0.0f;
  }
  return u32x4{pack_bf16x2(s * e[0], s * e[1]), pack_bf16x2(s * e[2], s * e[3]),
               pack_bf16x2(s * e[4], s * e[5]), pack_bf16x2(s * e[6], s * e[7])};
}

// bf16 row segment [j0, j0 + 8) of a row of length r (zeros past r)
__device__ __forceinline__ u32x4 e_operand_row(const uint16_t* row, int j0, int r) {
  if (j0 + 8 <= r && ((reinterpret_cast<uintptr_t>(row + j0) & 15) == 0))
    return *reinterpret_cast<const u32x4*>(row + j0);
  uint16_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (j0 + i < r) ? row[j0 + i] : (uint16_t)0;
  return u32x4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
               (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
}

// Multi-adapter forward: rank column c of output row n is element
// col_base[c] + n col_stride[c] of the concatenated B; columns j0 .. j0 + 7,
// zeros past rc.  One 16-byte load when the eight columns are contiguous in
// one adapter and aligned.
__device__ __forceinline__ u32x4 e_operand_multi(const uint16_t* Bc, const int32_t* cb,
                                                 const int32_t* cs, int64_t n, int j0, int rc) {
  if (j0 + 8 <= rc && cb[j0 + 7] == cb[j0] + 7 && cs[j0] == cs[j0 + 7] && cs[j0] % 8 == 0 &&
      cb[j0] % 8 == 0)
    return *reinterpret_cast<const u32x4*>(Bc + cb[j0] + n * cs[j0]);
  uint16_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = j0 + i;
    v[i] = c < rc ? Bc[cb[c] + n * cs[c]] : (uint16_t)0;
  }
  return u32x4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
               (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
}

// bf16 column segment: A[j0 + i][k] for i < 8 (A is r x ld), zeros past r
__device__ __forceinline__ u32x4 e_operand_col(const uint16_t* A, int64_t ld, int64_t k, int j0,
                                               int r) {
  uint16_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (j0 + i < r) ? A[(int64_t)(j0 + i) * ld + k] : (uint16_t)0;
  return u32x4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
               (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
}

template <bool TR, int JM>
__global__ __launch_bounds__(kGThreads) void g256_kernel(G256Params p) {
  using S = Shape<JM>;
  __shared__ __attribute__((aligned(1024))) char smem[S::NST * S::Stage];
  __shared__ int s_first, s_ready;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave & 1, wj = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;

  // tile and split of this workgroup.  Workgroup b runs on XCD b % 8; each
  // XCD is given a contiguous range of tiles (in groups of four activation
  // tiles, so that the tiles sharing an L2 share operand rows), and the two
  // splits of a tile are workgroups b and b + 8, on the same XCD.
  const int ntiles = p.ti * p.tj;
  int t, split;
  if (p.splits == 2) {
    const int b = blockIdx.x;
    t = (b & 7) * p.tpx + (b >> 4);
    split = (b >> 3) & 1;
    if (t >= ntiles) return;  // padding of the grid to whole groups of 16
  } else {
    t = xcd_tile(blockIdx.x, ntiles);
    split = 0;
  }
  constexpr int GJ = 4;
  const int grp = t / (GJ * p.ti);
  const int in = t - grp * GJ * p.ti;
  const int gj = (p.tj - grp * GJ) < GJ ? (p.tj - grp * GJ) : GJ;
  const int tile_j = grp * GJ + in % gj;
  const int tile_i = in / gj;
  const int tile = tile_j * p.ti + tile_i;
  const int64_t i0 = (int64_t)tile_i * kGT, j0 = (int64_t)tile_j * S::TJ;
  const int64_t M = p.M, NI = p.NI, KR = p.KR;
  const int KT = (int)(KR / kGK);
  const int kt0 = split * p.ksteps;
  const int kt1 = (kt0 + p.ksteps) < KT ? (kt0 + p.ksteps) : KT;

  const uint32_t sbase = lds_addr(smem);
  // stage b: weight tile at sbase + b * S::Stage, activation tile + kTileBytes

  // split K: per tile (arrivals, ready, XCD of split 0, XCD of split 1)
  int32_t* fl = p.flags + 4 * tile;
  const int xcc = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 15u);
  if (p.splits > 1 && tid == 0)
    __hip_atomic_store(fl + 2 + split, xcc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- per-thread DMA offsets (bytes, relative to the step's base pointer)
  uint32_t poff[2 * JM], qoff[8];
#pragma unroll
  for (int u = 0; u < 2 * JM; ++u) {
    const int row = 16 * JM * wave + 8 * u + (lane >> 3);
    int64_t m = j0 + row;
    m = m < M ? m : M - 1;
    poff[u] = (uint32_t)((m * KR + 8 * ((lane & 7) ^ rswz(row))) * 2);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (!TR) {
      const int row = 64 * wave + 8 * u + (lane >> 3);
      const int c = (lane & 7) ^ rswz(row);
      const int64_t n = i0 + row;
      qoff[u] = (uint32_t)((n * KR + 8 * c) * 2);
    } else {
      const int nr = 16 * wave + 2 * u + (lane >> 5);
      const int cq = tlogical(lane & 31, nr);
      qoff[u] = (uint32_t)(((int64_t)nr * NI + i0 + 8 * cq) * 2);
    }
  }
  const char* pbase0 = reinterpret_cast<const char*>(p.P);
  const char* qbase0 = reinterpret_cast<const char*>(p.Q);

  // loads of one step, in four parts (u = 2 part, 2 part + 1)
  auto issue_part = [&](int kt, int b, int part) {
    const uint32_t st = sbase + b * S::Stage;
    const char* qb = TR ? qbase0 + (int64_t)kt * kGK * NI * 2 : qbase0 + (int64_t)kt * kGK * 2;
    const char* pb = pbase0 + (int64_t)kt * kGK * 2;
#pragma unroll
    for (int u = 2 * part; u < 2 * part + 2; ++u) {
      const uint32_t qd = TR ? st + (16 * wave + 2 * u) * 512 : st + (64 * wave + 8 * u) * 128;
      dma16(qb, qoff[u], qd);
      if (u < 2 * JM) dma16(pb, poff[u], st + kTileBytes + (16 * JM * wave + 8 * u) * 128);
    }
  };
  auto issue = [&](int kt, int b) {
#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(kt, b, part);
  };

  // ---- per-lane LDS read offsets
  // activation operand ms: row 32 JM wj + 32 ms + l32, chunk 2 s + h
  const int sw = rswz(l32);
  const uint32_t prow = (uint32_t)((32 * JM * wj + l32) * 128);
  uint32_t pcx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) pcx[s] = (uint32_t)(((2 * s + h) ^ sw) << 4);
  // weight operand
  const uint32_t qrow = (uint32_t)((128 * wi + l32) * 128);  // !TR
  uint32_t qtr[4];                                           // TR: per ns, excluding the row term
  uint32_t qtr_row = 0;
  if (TR) {
    const int gc = l32 & 15, half = l32 >> 4;
    const int nlo = gc >> 2;  // row within the 4-row block
    qtr_row = (uint32_t)((8 * h + nlo) * 512);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = 128 * wi + 32 * ns + 16 * half + 4 * (gc & 3);
      qtr[ns] = (uint32_t)(tphys(col >> 3, nlo) * 16 + (col & 7) * 2);
    }
  }

  auto load_frags = [&](uint32_t st, int s, u32x4 (&wf)[4], u32x4 (&xf)[JM]) {
    const uint32_t pt = st + kTileBytes;
#pragma unroll
    for (int ms = 0; ms < JM; ++ms) xf[ms] = read16(pt + prow + ms * 32 * 128 + pcx[s]);
    if (!TR) {
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) wf[ns] = read16(st + qrow + ns * 32 * 128 + pcx[s]);
    } else {
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const uint32_t a = st + qtr_row + (uint32_t)(16 * s * 512) + qtr[ns];
        const u32x2 lo = read_tr(a), hi = read_tr(a + 4 * 512);
        wf[ns] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  };

  f32x16 acc[4][JM];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < JM; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // one step on LDS stage B (compile-time, so that every operand address is a
  // per-lane base plus an immediate): the loads of step kt + NST - 1 go into
  // the stage read one step earlier (all at once for 256 x 128 tiles, a
  // quarter per substep for 256 x 256, which measured slightly faster there),
  // then four substeps whose LDS reads run one substep ahead; before the
  // barrier, wait until the loads of step kt + 1 have landed (those of later
  // steps stay in flight)
  constexpr int NST = S::NST;
  auto step = [&](int kt, auto stage) {
    constexpr int B = decltype(stage)::value;
    const bool more = kt + NST - 1 < kt1;
    if (more && JM == 2) issue(kt + NST - 1, (B + NST - 1) % NST);
    const uint32_t st = sbase + B * S::Stage;
    u32x4 wf[2][4], xf[2][JM];
    load_frags(st, 0, wf[0], xf[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = s & 1;
      if (more && JM == 4) issue_part(kt + NST - 1, (B + NST - 1) % NST, s);
      if (s < 3) load_frags(st, s + 1, wf[c ^ 1], xf[c ^ 1]);
      __builtin_amdgcn_sched_barrier(0);  // next substep's reads before these products
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int ms = 0; ms < JM; ++ms) acc[ns][ms] = mfma32(wf[c][ns], xf[c][ms], acc[ns][ms]);
    }
    if (NST > 2 && more)
      wait_dma_but<S::DMA>();
    else
      wait_dma();
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (kt0 < kt1) {
    issue(kt0, 0);
    if (NST > 2 && kt0 + 1 < kt1) {
      issue(kt0 + 1, 1);
      wait_dma_but<S::DMA>();
    } else {
      wait_dma();
    }
    __syncthreads();
    int kt = kt0;
    if (NST == 2) {
      for (; kt + 1 < kt1; kt += 2) {
        step(kt, I0{});
        step(kt + 1, I1{});
      }
      if (kt < kt1) step(kt, I0{});
    } else {
      for (; kt + 2 < kt1; kt += 3) {
        step(kt, I0{});
        step(kt + 1, I1{});
        step(kt + 2, I2{});
      }
      if (kt < kt1) step(kt, I0{});
      if (kt + 1 < kt1) step(kt + 1, I1{});
    }
  }

  // ---- split-K: the second workgroup of a tile to finish completes it.
  // Only relaxed device-scope atomics touch the flags, so no whole-L2
  // write-back or invalidation is needed.  When the partner is known to run on
  // this XCD (its XCD published at its start), the partial sums stay in the
  // shared L2: plain stores, a wait for their completion, then the ready flag
  // (1).  Otherwise (partner elsewhere or not started) they are published with
  // a device-scope release (ready = 2) and read after an acquire.
  if (p.splits > 1) {
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(fl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int partner = __hip_atomic_load(fl + 3 - split, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
      s_first = old == 0 ? (partner == xcc + 1 ? 1 : 2) : 0;
    }
    __syncthreads();
    const int mode = s_first;
    f32x4* slot = reinterpret_cast<f32x4*>(p.part + (int64_t)tile * S::Slot);
    if (mode) {
#pragma unroll
      for (int a = 0; a < 4 * JM; ++a)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x16& x = acc[a / JM][a % JM];
          slot[((wave * 4 * JM + a) * 4 + v4) * 64 + lane] =
              f32x4{x[4 * v4], x[4 * v4 + 1], x[4 * v4 + 2], x[4 * v4 + 3]};
        }
      if (mode == 1)
        wait_dma();  // the stores have reached the L2 shared with the partner
      else
        __threadfence();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(fl + 1, mode, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (tid == 0) {
      int it = 0, rd;
      while ((rd = __hip_atomic_load(fl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
        if (++it > kSpinLimit) {
          __hip_atomic_store(p.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      s_ready = rd;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_store(fl + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (s_ready == 2) __threadfence();
#pragma unroll
    for (int a = 0; a < 4 * JM; ++a)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x4 y = slot[((wave * 4 * JM + a) * 4 + v4) * 64 + lane];
        f32x16& x = acc[a / JM][a % JM];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * v4 + e] += y[e];
      }
  }

  // ---- expand: acc += E-operand x (s V)-operand over rank chunks of 16
  const int r = p.r;
  for (int c = 0; c < r; c += 16) {
    const int jr = c + 8 * h;
    u32x4 ef[4], vf[JM];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int64_t i = i0 + 128 * wi + 32 * ns + l32;
      ef[ns] = TR       ? e_operand_col(p.E, NI, i, jr, r)
               : p.multi ? e_operand_multi(p.E, p.col_base, p.col_stride, i, jr, r)
                         : e_operand_row(p.E + i * r, jr, r);
    }
#pragma unroll
    for (int ms = 0; ms < JM; ++ms) {
      int64_t m = j0 + 32 * JM * wj + 32 * ms + l32;
      m = m < M ? m : M - 1;
      vf[ms] = v_operand(p.V + m * r, jr, r, p.s);
    }
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int ms = 0; ms < JM; ++ms) acc[ns][ms] = mfma32(ef[ns], vf[ms], acc[ns][ms]);
  }

  // ---- store: bf16 tile in LDS (row j, 512 bytes; chunk c at c ^ (j & 15)),
  // then whole 512-byte output rows with 16-byte stores
  __syncthreads();  // every wave is done with the stages (and the split-K slot)
#pragma unroll
  for (int ms = 0; ms < JM; ++ms) {
    const int j = 32 * JM * wj + 32 * ms + l32;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 128 * wi + 32 * ns + 8 * q + 4 * h;  // 4 outputs i .. i + 3
        const int chunk = (i >> 3) ^ (j & 15);
        const uint32_t a = sbase + (uint32_t)(j * 512 + chunk * 16 + (i & 7) * 2);
        typedef __attribute__((address_space(3))) u32x2* lds_ptr;
        *(lds_ptr)(uintptr_t)a = u32x2{pack_bf16x2(acc[ns][ms][4 * q], acc[ns][ms][4 * q + 1]),
                                       pack_bf16x2(acc[ns][ms][4 * q + 2], acc[ns][ms][4 * q + 3])};
      }
  }
  __syncthreads();
  const int cl = tid & 31;  // chunk of the row
#pragma unroll 4
  for (int it = 0; it < 8 * JM; ++it) {
    const int j = 8 * it + (tid >> 5);
    const int64_t m = j0 + j;
    const u32x4 v = read16(sbase + (uint32_t)(j * 512 + ((cl ^ (j & 15)) << 4)));
    if (m < M) *reinterpret_cast<u32x4*>(p.Y + m * NI + i0 + 8 * cl) = v;
  }
}

}  // namespace

namespace dispatch {

namespace {

// Any M: with the bf16 weight copy in the workspace this path measured faster
// than the fused kernels at every M tried (W0 4096^2 NF4: forward 53 vs 56-98
// us at M = 32..1536, dX 52-82 vs 65-104 us at M = 1..1536), and equal at
// M = 2048.
bool g256_fits(int64_t M, int64_t NI, int64_t KR) {
  return M >= 1 && NI % kGT == 0 && KR % kGK == 0 &&
         (double)NI * KR * 2 < 4294967296.0 && (double)M * KR * 2 < 4294967296.0;
}

// Tile shape and split: 256 x 256 tiles when there are enough of them to fill
// the chip, else 256 x 128; K split in two when even those leave most compute
// units idle.
struct G256Plan {
  int jm, splits;
  int64_t ti, tj, tiles;
};

G256Plan g256_plan(int64_t M, int64_t NI) {
  G256Plan pl;
  pl.ti = NI / kGT;
  pl.jm = pl.ti * cdiv(M, 256) >= 192 ? 4 : 2;
  pl.tj = cdiv(M, 64 * pl.jm);
  pl.tiles = pl.ti * pl.tj;
  pl.splits = pl.tiles <= 160 ? 2 : 1;
  return pl;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// error word, then four flag words per tile
size_t g256_flag_bytes(int64_t M, int64_t NI) {
  return 256 + align256((size_t)g256_plan(M, NI).tiles * 16);
}

size_t g256_ws_bytes(int64_t M, int64_t NI) {
  const G256Plan pl = g256_plan(M, NI);
  const size_t slots = pl.splits > 1 ? (size_t)pl.tiles * kGT * 64 * pl.jm * 4 : 0;
  return g256_flag_bytes(M, NI) + slots;
}

template <bool TR, int JM>
void launch_shape(const G256Params& p, unsigned blocks, hipStream_t st) {
  hipLaunchKernelGGL((g256_kernel<TR, JM>), dim3(blocks), dim3(kGThreads), 0, st, p);
}

int launch_g256(bool tr, const void* P, const void* Q, const float* V, const void* E, int64_t M,
                int64_t NI, int64_t KR, int64_t r, float s, void* Y, void* ws, hipStream_t st,
                const MultiTab* mt = nullptr) {
  const G256Plan pl = g256_plan(M, NI);
  G256Params p{};
  p.P = (const uint16_t*)P;
  p.Q = (const uint16_t*)Q;
  p.V = V;
  p.E = (const uint16_t*)E;
  p.Y = (uint16_t*)Y;
  p.M = M;
  p.NI = NI;
  p.KR = KR;
  p.r = (int32_t)r;
  p.s = s;
  if (mt) {
    p.multi = 1;
    for (int c = 0; c < kMaxRankCols; ++c) {
      p.col_base[c] = mt->col_base[c];
      p.col_stride[c] = mt->col_stride[c];
    }
  }
  p.ti = (int32_t)pl.ti;
  p.tj = (int32_t)pl.tj;
  p.splits = pl.splits;
  p.ksteps = (int32_t)cdiv(KR / kGK, p.splits);
  char* w = (char*)ws;
  p.err = (int32_t*)w;
  p.flags = (int32_t*)(w + 256);
  p.part = (float*)(w + g256_flag_bytes(M, NI));
  p.tpx = (int32_t)cdiv(pl.tiles, 8);
  const unsigned blocks = (unsigned)(p.splits == 2 ? 16 * (int64_t)p.tpx : pl.tiles);
  timing_begin(tr ? "g256_dx" : "g256_fwd", st);
  if (tr) {
    if (pl.jm == 4) launch_shape<true, 4>(p, blocks, st);
    else launch_shape<true, 2>(p, blocks, st);
  } else {
    if (pl.jm == 4) launch_shape<false, 4>(p, blocks, st);
    else launch_shape<false, 2>(p, blocks, st);
  }
  timing_end(st);
  return hip_fail(hipGetLastError(), "g256 launch");
}

// the NF4 weight dequantised to bf16 into the workspace at q (when the prep
// kernel cannot take the shrink as well)
int bf16_weight(const lq_weight& W, void* q, hipStream_t st) {
  return launch_nf4_dequantize(W.codes, W.q8, W.c2, W.absmax, W.double_quant, W.codebook,
                               W.N * W.K, q, LQ_BF16, st);
}

}  // namespace

bool big_fwd_eligible(int64_t M, int64_t N, int64_t K) { return g256_fits(M, N, K); }
bool big_dx_eligible(int64_t M, int64_t N, int64_t K) { return g256_fits(M, K, N); }

// [g256: error word, flags, split-K slots] [T when T_out is NULL] [bf16 W0]
size_t big_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  return align256(g256_ws_bytes(M, N)) + align256((size_t)(M * r) * 4) + (size_t)(N * K) * 2;
}

// [g256: error word, flags, split-K slots] [bf16 W0]
size_t big_dx_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return align256(g256_ws_bytes(M, K)) + (size_t)(N * K) * 2;
}

int big_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B, int64_t r,
            float s, void* Y, float* T_out, void* ws, hipStream_t st, const void* Xa,
            float inv_keep) {
  const int64_t N = W.N, K = W.K;
  const void* Z = Xa ? Xa : X;  // the adapter branch's input (dropped under dropout)
  char* w = (char*)ws;
  void* gws = w;
  w += align256(g256_ws_bytes(M, N));
  float* T = T_out ? T_out : (float*)w;
  w += align256((size_t)(M * r) * 4);
  int e = 0;
  const int nz = (int)(g256_flag_bytes(M, N) / 4);
  const void* Q = W.kind == LQ_WEIGHT_DENSE ? W.dense : (const void*)w;
  MultiTab sc{};  // T times 1 / (1 - p) under dropout, in the shrink's stores
  sc.oscale = inv_keep;
  if (W.kind != LQ_WEIGHT_DENSE && shrink_eligible(false, r))
    e = launch_prep(W, w, Z, M, K, A, false, r, T, (int32_t*)gws, nz, st, nullptr, &sc);
  else if (!(e = W.kind == LQ_WEIGHT_DENSE ? 0 : bf16_weight(W, w, st)))
    e = t_only(Z, M, K, A, r, T, st, (int32_t*)gws, nz, inv_keep);
  if (e) return e;
  return launch_g256(false, X, Q, T, B, M, N, K, r, s, Y, gws, st);
}

int big_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B, int64_t r,
           float s, void* dX, float* U, void* ws, hipStream_t st, float uscale) {
  const int64_t N = W.N, K = W.K;
  char* w = (char*)ws;
  void* gws = w;
  w += align256(g256_ws_bytes(M, K));
  int e = 0;
  const int nz = (int)(g256_flag_bytes(M, K) / 4);
  const void* Q = W.kind == LQ_WEIGHT_DENSE ? W.dense : (const void*)w;
  MultiTab sc{};
  sc.oscale = uscale;
  if (W.kind != LQ_WEIGHT_DENSE && shrink_eligible(true, r))
    e = launch_prep(W, w, dY, M, N, B, true, r, U, (int32_t*)gws, nz, st, nullptr, &sc);
  else if (!(e = W.kind == LQ_WEIGHT_DENSE ? 0 : bf16_weight(W, w, st)))
    e = u_only(dY, M, N, B, r, U, st, (int32_t*)gws, nz, uscale);
  if (e) return e;
  return launch_g256(true, dY, Q, U, A, M, K, N, r, s, dX, gws, st);
}

// [row -> adapter, int32 T] [masked T, float32 T x (n_ad r)] [g256 workspace] [bf16 W0]
size_t big_multi_ws_bytes(int64_t T, int64_t N, int64_t K, int64_t rc) {
  return align256((size_t)T * 4) + align256((size_t)(T * rc) * 4) +
         align256(g256_ws_bytes(T, N)) + (size_t)(N * K) * 2;
}

// Multi-adapter forward at large T: T_m = X A_cat^T (A_cat = the adapters' A
// stacked by rows, rc x K) masked to each row's adapter columns and scaled by
// its scale, then the large-tile product whose expand reads the concatenated
// B through the column table.
int big_fwd_multi(const void* X, int64_t T, const lq_weight& W, const void* A_cat,
                  const void* B_cat, const MultiTab& mt, const int32_t* seg_off,
                  const int32_t* seg_ad, int32_t n_seg, void* Y, void* ws, hipStream_t st) {
  const int64_t N = W.N, K = W.K, rc = mt.rc;
  char* w = (char*)ws;
  int32_t* row_ad = (int32_t*)w;
  w += align256((size_t)T * 4);
  float* Tm = (float*)w;
  w += align256((size_t)(T * rc) * 4);
  void* gws = w;
  w += align256(g256_ws_bytes(T, N));
  int e = launch_rowmap(seg_off, seg_ad, n_seg, T, row_ad, st);
  if (e) return e;
  const int nz = (int)(g256_flag_bytes(T, N) / 4);
  const void* Q = W.kind == LQ_WEIGHT_DENSE ? W.dense : (const void*)w;
  if (W.kind != LQ_WEIGHT_DENSE)
    e = launch_prep(W, w, X, T, K, A_cat, false, rc, Tm, (int32_t*)gws, nz, st, row_ad, &mt);
  else
    e = launch_shrink(X, T, K, A_cat, false, rc, Tm, (int32_t*)gws, nz, st, row_ad, &mt);
  if (e) return e;
  return launch_g256(false, X, Q, Tm, B_cat, T, N, K, rc, 1.0f, Y, gws, st, &mt);
}

}  // namespace dispatch
}  // namespace lq

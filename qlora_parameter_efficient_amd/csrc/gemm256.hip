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
// its float32 accumulators to a per-tile slot (device-scope release) and a
// ready flag; the second acquires them, adds them to its own and finishes the
// tile.  The second only ever waits for a workgroup that is already past its
// main loop, so the wait cannot deadlock; it is also bounded, and a wait that
// gives up is counted on the device (lq_debug_wait_giveups), the tile then
// being incomplete.  The kernel that forms T or U clears the flags before each
// launch.
//
// Epilogue.  The expand adds (s V) E as extra MFMAs on the finished
// accumulators (V = T or U rounded to bf16 after scaling by s, E = B or A),
// then the tile is staged in LDS as bf16 and written with 16-byte stores that
// cover whole output lines.
#include <atomic>
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

struct G256Params {
  const uint16_t* P;  // activations, M x KR (X or dY)
  const uint16_t* Q;  // bf16 weight: forward NI x KR, dX KR x NI
  const float* V;     // M x r: T (forward) or U (dX)
  const uint16_t* E;  // forward: B (NI x r); dX: A (r x NI)
  uint16_t* Y;        // M x NI
  float* part;        // split-K slots, Shape<JM>::Slot floats per tile
  int32_t* flags;     // split-K (arrivals, ready) per tile, zero between calls
  int64_t M, NI, KR;
  int32_t r;
  float s;
  int32_t ti, tj, splits, ksteps;
  int32_t tpx;  // split K: tiles per XCD
  int32_t spin;  // split K: bound of the partner wait, in polls
  int32_t multi;  // multi-adapter forward: E is the concatenated B, read through col_*
  int32_t col_base[kMaxRankCols];
  int32_t col_stride[kMaxRankCols];
};

// split-K waits that gave up since the host last read the count (one
// counter per device)
__device__ unsigned long long g_wait_giveups;

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

// 4 bytes per lane from global memory (base + off) straight into LDS at
// m0 + 4 * lane (same rules as dma16).
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
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
  // this split's reduction steps [ka, kb)
  const int ka = split * p.ksteps;
  const int kb = (ka + p.ksteps) < KT ? (ka + p.ksteps) : KT;

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
    const bool more = kt + NST - 1 < kb;
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
  if (ka < kb) {
    issue(ka, 0);
    if (NST > 2 && ka + 1 < kb) {
      issue(ka + 1, 1);
      wait_dma_but<S::DMA>();
    } else {
      wait_dma();
    }
    __syncthreads();
    int kt = ka;
    if (NST == 2) {
      for (; kt + 1 < kb; kt += 2) {
        step(kt, I0{});
        step(kt + 1, I1{});
      }
      if (kt < kb) step(kt, I0{});
    } else {
      for (; kt + 2 < kb; kt += 3) {
        step(kt, I0{});
        step(kt + 1, I1{});
        step(kt + 2, I2{});
      }
      if (kt < kb) step(kt, I0{});
      if (kt + 1 < kb) step(kt + 1, I1{});
    }
  }

  // ---- split K: the second workgroup of a tile to arrive completes it.
  // Only device-scope atomics touch the flags.  The first to arrive publishes
  // its float32 accumulators to the tile's slot.  When its partner is known
  // to run on this XCD (each workgroup publishes its XCD at its start), the
  // two share one L2: plain stores, a wait until every store has reached that
  // L2 (vmcnt 0 in every wave), a barrier, then ready = 1 -- a device-scope
  // release would also write back every dirty line of the XCD's L2, which
  // measured far slower.  Otherwise every thread releases at device scope
  // before the barrier and ready = 2.  The second workgroup polls ready
  // (relaxed loads, bounded) and then acquires at device scope in either
  // case, which orders its reads of the slot after the flag and drops stale
  // L1 lines; a barrier then hands the slot to all its threads.  The first to
  // arrive is already past its main loop, so the wait is short and cannot
  // deadlock.  A wait that still gives up (or that the host forced to give
  // up) is counted on the device (lq_debug_wait_giveups) and the slot is left
  // unread: the tile then holds this workgroup's half of the reduction only,
  // and the nonzero count tells the caller so.  The kernel that forms T / U
  // clears the flags before every launch.
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
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) __hip_atomic_store(fl + 1, mode, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (tid == 0) {
      bool ok = p.spin >= 0;  // a negative bound: give up at once (test aid)
      int it = 0;
      while (ok && __hip_atomic_load(fl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
        if (++it > p.spin) ok = false;
        __builtin_amdgcn_s_sleep(2);
      }
      if (ok)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      else
        __hip_atomic_fetch_add(&g_wait_giveups, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_ready = ok;
    }
    __syncthreads();
    if (s_ready) {
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

// ---------------------------------------------------------------------------
// Forward with the NF4 weight dequantised inside the K loop and the rank-r
// shrink in the same loop (no bf16 copy of W0 anywhere, no separate launch
// for T): Y = X deq(W0)^T + (s T) B^T with T = X A^T formed on the way.
//
// Tile 128 (weight rows n) x 256 (activation rows m), eight waves (two per
// SIMD); wave (wi, wj) owns the 64 x 64 block at (64 wi, 64 wj): 2 x 2
// accumulators of 32 x 32.  Per 64-wide reduction step (one NF4 block per
// weight row):
//   * the activation tile (256 rows x 128 bytes) goes straight into LDS by
//     direct-to-LDS loads, as in g256_kernel, and so does the step's slice of
//     A (r rows x 128 bytes, same swizzle);
//   * the NF4 codes of the weight tile, the blocks' 8-bit constants and c2
//     come by direct-to-LDS loads too, in groups of four steps (a whole
//     128-byte line of codes per row), one group ahead, into two code
//     buffers; during the step before the one that uses them, thread t
//     forms its block's 16 possible bf16 values RNE(fl32(cb[i] a')), a' =
//     fl32(q8 fl32(c2 / 127)), as byte planes in registers, looks its 16
//     weights up with v_perm_b32 (four codes per instruction; no LDS traffic
//     for the table) and stores them as bf16 into the weight tile of the
//     other LDS stage (128-byte rows, the same chunk swizzle as the
//     activations).  The dequantisation is scheduled between the step's
//     MFMAs (sched_group_barrier), so it runs while the matrix cores work.
//     With every global load issued by the kernel itself, the waits are its
//     own: the end of a step waits until only the code group loads issued in
//     it (if any) are outstanding.
//   * the shrink: the two waves that hold the same 64 activation rows split
//     them, wave wi taking the 32 rows of its operand ms = wi, and add A-slice
//     x activation products (one 32 x 32 x 16 MFMA per 32 ranks and substep,
//     ranks past r reading zero or a repeated row of A whose results are never
//     used) to a T accumulator.  Every column tile of a row block forms the
//     same T; the one with tile_i = 0 stores it (T_out).
// Each code is thus dequantised once per 256 activation rows, in registers,
// and fed to bf16 MFMA from LDS.  After the loop T goes through LDS as
// bf16(s T) to the waves that need its rows for the expand, which runs as in
// g256_kernel; the tile is staged in LDS as bf16 and written with 16-byte
// stores.
constexpr int kQI = 128, kQJ = 256;
constexpr int kQWT = kQI * kGK * 2;  // weight tile of one step: 16 KB
constexpr int kQAT = kQJ * kGK * 2;  // activation tile: 32 KB
constexpr int kQStage = kQWT + kQAT;
constexpr int kQThreads = 512;  // 8 waves: two per SIMD
// code buffer: codes (128 rows x 128 bytes), 8-bit constants (one dword per
// row and wave), c2 / absmax [step][row]
constexpr int kQCQ8 = 16384, kQCC2 = 16384 + 2048, kQCB = 16384 + 2048 + 2048;
// slice of A (or of B^T) for one step: up to 64 rank rows x 128 bytes
constexpr int kQAS = 64 * 128;
// second-level steps fl32(c2 / 127) of a 128-row weight tile: 128 K / 64 / 256
// groups (+ 2 for the ends) for K <= 65536
constexpr int kQMaxG = 520;

struct Q256Params {
  const uint16_t* P;  // X, M x K
  WeightArgs W;       // NF4 weight, N x K
  const uint16_t* A;  // A, r x K
  float* T_out;       // T, M x r float32, or NULL
  const uint16_t* E;  // B, N x r
  uint16_t* Y;        // M x N
  int64_t M, N, K;
  int32_t r;
  float s;
  int32_t ti, tj;
  NF4Table tab;
};

__device__ __forceinline__ void write16(uint32_t addr, const u32x4& v) {
  typedef __attribute__((address_space(3))) u32x4* lds_ptr;
  *(lds_ptr)(uintptr_t)addr = v;
}

// RQ: 32-rank blocks of the shrink (1 for r <= 32, 2 for r <= 64).  T16 (r <=
// 16): the shrink runs as one 16 x 16 x 32 MFMA per 16 rows and pair of
// substeps instead of one 32 x 32 x 16 per substep (half the MFMA cycles and
// half the A reads): its activation operand (16 rows x 32 reduction elements,
// four 8-element pieces) is the wave's first activation operands of the two
// substeps with their 16-lane rows regrouped by v_permlane32_swap and
// v_permlane16_swap, and its A operand one 16-byte read per pair.
template <int WK, bool FP8, int RQ, bool T16>
__global__ __launch_bounds__(kQThreads) void q256_fwd_kernel(Q256Params p) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kQStage];
  __shared__ __attribute__((aligned(1024))) char cst[2 * kQCB];
  __shared__ __attribute__((aligned(1024))) char aslc[2 * kQAS];
  __shared__ float steptab[WK == kNF4DQ ? kQMaxG : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave & 1, wj = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;
  float cbq[4];
  quad_levels(p.tab, lane, cbq);
  // tiles in activation-row order, so that an XCD's contiguous range of
  // tiles shares one activation tile (its rows stay in that XCD's L2)
  const int t = xcd_tile(blockIdx.x, p.ti * p.tj);
  const int tile_j = t / p.ti, tile_i = t - tile_j * p.ti;
  const int64_t i0 = (int64_t)tile_i * kQI, j0 = (int64_t)tile_j * kQJ;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KT = (int)(K / kGK);
  const uint32_t sbase = lds_addr(smem);

  // activation DMA: wave w fills rows 32 w .. 32 w + 31, 8 rows per instruction
  uint32_t poff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 32 * wave + 8 * u + (lane >> 3);
    int64_t m = j0 + row;
    m = m < M ? m : M - 1;
    poff[u] = (uint32_t)((m * K + 8 * ((lane & 7) ^ rswz(row))) * 2);
  }
  const char* pbase0 = reinterpret_cast<const char*>(p.P);
  auto issue_act = [&](int kt, int b) {
    const uint32_t at = sbase + b * kQStage + kQWT;
    const char* pb = pbase0 + (int64_t)kt * kGK * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(pb, poff[u], at + (32 * wave + 8 * u) * 128);
  };
  // A slice of a step: wave w brings rank rows 8 w .. 8 w + 7 when 8 w < r
  // (rows past r repeat row r - 1); rows from the next multiple of 8 up to
  // 32 RQ are zero, written once below
  const int r = p.r;
  const uint32_t abase = lds_addr(aslc);
  const bool a_rows = 8 * wave < r;
  uint32_t aoff;
  {
    const int row = 8 * wave + (lane >> 3);
    const int srow = row < r ? row : r - 1;
    aoff = (uint32_t)(((int64_t)srow * K + 8 * ((lane & 7) ^ rswz(row))) * 2);
  }
  const char* abase0 = reinterpret_cast<const char*>(p.A);
  auto issue_a = [&](int kt, int b) {
    if (a_rows) dma16(abase0 + (int64_t)kt * kGK * 2, aoff, abase + b * kQAS + 8 * wave * 128);
  };
  {
    const int rp = (r + 7) & ~7;
    for (int i = tid; i < 2 * (32 * RQ - rp) * 8; i += kQThreads) {
      const int b = i / ((32 * RQ - rp) * 8), rem = i - b * (32 * RQ - rp) * 8;
      write16(abase + b * kQAS + rp * 128 + rem * 16, u32x4{0u, 0u, 0u, 0u});
    }
  }
  // Weight codes and block constants arrive by direct-to-LDS loads as well,
  // in groups of four steps (one 128-byte line of codes per row), into one of
  // two code buffers: the group's codes (128 rows x 128 bytes; chunk c of row
  // x at physical chunk c ^ (x & 7)), the dword of 8-bit constants of each row
  // that holds the group's four blocks (waves 0 and 1; the other waves load
  // copies into unused space, so that every wave issues the same loads), and
  // without a second level each row's float32 absmax for the four steps,
  // [step][row].  (The steps fl32(c2 / 127) of the tile's groups are formed
  // once, into LDS, before the loop.)  Group g + 1 is loaded during step
  // 4 g + 1.  Thread t dequantises row t / 4, weights 16 (t & 3) .. + 15 of
  // each block, from LDS; the quad of threads sharing a row builds its level
  // table together.
  constexpr int NGD = 3;  // group loads per wave
  const uint32_t cbase = lds_addr(cst);
  const int64_t KB = K / 64;
  const int64_t g_lo = (i0 * KB) >> 8;
  if (WK == kNF4DQ) {
    const int ng = (int)((((i0 + kQI) * KB - 1) >> 8) - g_lo + 1);
    for (int i = tid; i < ng; i += kQThreads) steptab[i] = dq_step(p.W.c2[g_lo + i]);
  }
  const int64_t wrow_blk = (i0 + (tid >> 2)) * KB;  // first block of this thread's row
  const int NG = KT / 4;
  const int wx = tid >> 2, wq = tid & 3;
  uint32_t coff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 16 * wave + 8 * u + (lane >> 3);
    coff[u] = (uint32_t)((((i0 + row) * K) >> 1) + 16 * ((lane & 7) ^ (row & 7)));
  }
  const uint32_t qoff = (uint32_t)((i0 + ((64 * wave + lane) & (kQI - 1))) * KB);
  const int ce = 64 * wave + lane;  // the c2 entry this lane brings: step ce / 128, row ce % 128
  const int64_t sblk = (i0 + (ce & 127)) * KB + (ce >> 7);
  uint32_t wdst[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) wdst[d] = (uint32_t)(wx * 128 + (((2 * wq + d) ^ rswz(wx)) << 4));
  auto issue_group = [&](int g, int buf) {
    const uint32_t cb = cbase + buf * kQCB;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      dma16(reinterpret_cast<const char*>(p.W.codes) + (int64_t)g * 128, coff[u],
            cb + (16 * wave + 8 * u) * 128);
    if (WK == kNF4DQ) {
      dma4(p.W.q8 + 4 * g, qoff, cb + kQCQ8 + 256 * wave);
    } else {
      const int64_t blk = sblk + 4 * g;
      dma4(p.W.absmax, (uint32_t)(blk * 4), cb + kQCC2 + 256 * wave);
    }
  };
  // this thread's 16 codes of the step at position pos of the group in code
  // buffer buf (two words), and the raw constants of its block: (c2 or float32
  // absmax bits, the row's word of 8-bit constants); then the block scale a'
  auto codes_at = [&](int buf, int pos) {
    typedef __attribute__((address_space(3))) const u32x2* lp;
    const int ch = (2 * pos + (wq >> 1)) ^ (wx & 7);
    return *(lp)(uintptr_t)(cbase + buf * kQCB + wx * 128 + ch * 16 + 8 * (wq & 1));
  };
  // (float32 absmax bits, or the row's word of 8-bit constants)
  auto raw_at = [&](int buf, int pos) {
    typedef __attribute__((address_space(3))) const uint32_t* lp;
    const uint32_t cb = cbase + buf * kQCB;
    return WK == kNF4DQ ? *(lp)(uintptr_t)(cb + kQCQ8 + 4 * wx)
                        : *(lp)(uintptr_t)(cb + kQCC2 + 4 * (128 * pos + wx));
  };
  // block scale of this thread's row at step kt (position pos of its group)
  auto scale_of = [&](uint32_t v, int pos, int kt) {
    if (WK == kNF4DQ)
      return dq_value<FP8>((v >> (8 * pos)) & 0xFFu) *
             steptab[(int)(((wrow_blk + kt) >> 8) - g_lo)];
    return __uint_as_float(v);
  };

  // operand reads (128-byte-row tiles, as g256_kernel)
  const int sw = rswz(l32);
  uint32_t pcx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) pcx[s] = (uint32_t)(((2 * s + h) ^ sw) << 4);
  // activation operand ms covers rows 64 wj + 32 (ms ^ wi) .. + 31 of the
  // tile, so that operand 0 is always the 32 rows of this wave's shrink
  uint32_t prowm[2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) prowm[ms] = (uint32_t)((64 * wj + 32 * (ms ^ wi) + l32) * 128);
  const uint32_t qrow = (uint32_t)((64 * wi + l32) * 128);
  const uint32_t arow = (uint32_t)(l32 * 128);
  // T16: lane l reads rank l % 16, 8-element piece l / 16 of the substep pair
  uint32_t a16[2];
#pragma unroll
  for (int w = 0; w < 2; ++w)
    a16[w] = (uint32_t)((lane & 15) * 128 + (((4 * w + (lane >> 4)) ^ rswz(lane & 15)) << 4));
  auto load_frags = [&](uint32_t st, uint32_t as, int s, u32x4 (&wf)[2], u32x4 (&xf)[2],
                        u32x4 (&af)[RQ]) {
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) xf[ms] = read16(st + kQWT + prowm[ms] + pcx[s]);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) wf[ns] = read16(st + qrow + ns * 32 * 128 + pcx[s]);
    if (!T16) {
#pragma unroll
      for (int q = 0; q < RQ; ++q) af[q] = read16(as + arow + q * 32 * 128 + pcx[s]);
    }
  };

  f32x16 acc[2][2], tacc[T16 ? 1 : RQ];
  f32x4 t16[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
#pragma unroll
  for (int q = 0; q < (T16 ? 1 : RQ); ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) tacc[q][v] = 0.0f;
  // T16: the 16 x 16 x 32 shrink over a substep pair from the first activation
  // operands x0 (first substep) and x1 (second): 16-lane rows (x0: rows 0-15 h0,
  // rows 16-31 h0, rows 0-15 h1, rows 16-31 h1) regrouped so that operand lo
  // holds rows 0-15 and hi rows 16-31, pieces in reduction order
  auto shrink16 = [&](const u32x4& x0, const u32x4& x1, const u32x4& a) {
    u32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto s32 = __builtin_amdgcn_permlane32_swap(x0[e], x1[e], false, false);
      const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
      lo[e] = s16[0];
      hi[e] = s16[1];
    }
    t16[0] = mfma16(a, lo, t16[0]);
    t16[1] = mfma16(a, hi, t16[1]);
  };

  // prologue: step 0's tiles in stage 0, group 0's codes in code buffer 0
  issue_act(0, 0);
  issue_a(0, 0);
  issue_group(0, 0);
  wait_dma();
  __syncthreads();
  {
    const u32x2 cw = codes_at(0, 0);
    const PermTable pt = perm_table_quad(cbq, scale_of(raw_at(0, 0), 0, 0));
#pragma unroll
    for (int d = 0; d < 2; ++d) write16(sbase + wdst[d], perm_deq8(cw[d], pt));
  }
  __syncthreads();

  // Step kt (J = kt mod 8: stage J & 1, code buffer J >> 2, position J & 3):
  // the activation loads of step kt + 1, in position 1 the loads of the next
  // code group, the MFMAs of step kt with the dequantisation of step kt + 1
  // (level table, then one code word in each of the next two substeps) into
  // the other weight tile scheduled between them; at the end, wait for
  // everything but the code group loads issued in this step.  The MFMAs of a
  // step's last substep run after the barrier, behind the first LDS reads of
  // the next step, whose latency they cover (their operands are already in
  // registers; the first step's are zeros).  Unrolled by eight so that every
  // LDS address is a base plus an immediate.
  u32x4 pw[2], px[2], pa[RQ], px2, pa16;
#pragma unroll
  for (int i = 0; i < 2; ++i) pw[i] = px[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < RQ; ++q) pa[q] = u32x4{0u, 0u, 0u, 0u};
  px2 = pa16 = u32x4{0u, 0u, 0u, 0u};
  auto pending = [&]() {
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) acc[ns][ms] = mfma32(pw[ns], px[ms], acc[ns][ms]);
    if (T16) {
      shrink16(px2, px[0], pa16);  // the second substep pair
    } else {
#pragma unroll
      for (int q = 0; q < RQ; ++q) tacc[q] = mfma32(pa[q], px[0], tacc[q]);
    }
  };
  auto step = [&](int kt, auto jj) {
    constexpr int J = decltype(jj)::value;
    constexpr int B = J & 1, POS = J & 3, BUF = J >> 2;
    constexpr int NPOS = (POS + 1) & 3, NBUF = POS == 3 ? BUF ^ 1 : BUF;  // step kt + 1
    const bool more = kt + 1 < KT;
    if (more) {
      issue_act(kt + 1, B ^ 1);
      issue_a(kt + 1, B ^ 1);
    }
    const bool grp = POS == 1 && (kt >> 2) + 1 < NG;
    if (grp) issue_group((kt >> 2) + 1, BUF ^ 1);
    const uint32_t st = sbase + B * kQStage;
    const uint32_t as = abase + B * kQAS;
    const uint32_t wt = sbase + (B ^ 1) * kQStage;
    // (after the last step the words read here are stale and their
    // dequantised values land in a tile nobody reads: no branch, so that the
    // dequantisation can be scheduled between the MFMAs)
    u32x4 wf[2][2], xf[2][2], af[2][RQ];
    load_frags(st, as, 0, wf[0], xf[0], af[0]);
    u32x4 ta16[2], x16[2];
    if (T16) {
#pragma unroll
      for (int w = 0; w < 2; ++w) ta16[w] = read16(as + a16[w]);
    }
    const u32x2 cw = codes_at(NBUF, NPOS);
    const uint32_t raw = raw_at(NBUF, NPOS);
    __builtin_amdgcn_sched_barrier(0);
    pending();  // the previous step's last substep
    __builtin_amdgcn_sched_barrier(0);
    PermTable pt;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = s & 1;
      if (s < 3) load_frags(st, as, s + 1, wf[c ^ 1], xf[c ^ 1], af[c ^ 1]);
      if (s == 0) pt = perm_table_quad(cbq, scale_of(raw, NPOS, kt + 1));
      if (s < 3) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) acc[ns][ms] = mfma32(wf[c][ns], xf[c][ms], acc[ns][ms]);
        if (T16) {
          if (s == 0 || s == 2) x16[s >> 1] = xf[c][0];
          if (s == 1) shrink16(x16[0], xf[c][0], ta16[0]);
        } else {
#pragma unroll
          for (int q = 0; q < RQ; ++q) tacc[q] = mfma32(af[c][q], xf[c][0], tacc[q]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          pw[i] = wf[c][i];
          px[i] = xf[c][i];
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) pa[q] = af[c][q];
        if (T16) {
          px2 = x16[1];
          pa16 = ta16[1];
        }
      }
      if (s == 1 || s == 2) write16(wt + wdst[s - 1], perm_deq8(cw[s - 1], pt));
      // the next substep's reads first, then each MFMA followed by a share of
      // the dequantisation (and the lane swaps of the 16-row shrink), then the
      // store of the dequantised word
      constexpr int NR = T16 ? 4 : 4 + RQ;  // LDS reads of a substep
      if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
      if (s == 0) {
#pragma unroll
        for (int i = 0; i < (T16 ? 4 : 4 + RQ); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 52 / (T16 ? 4 : 4 + RQ), 0);
        }
      } else if (s == 1 && T16) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 40 / 6, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      } else if (s < 3) {
#pragma unroll
        for (int i = 0; i < (T16 ? 4 : 4 + RQ); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 32 / (T16 ? 4 : 4 + RQ), 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (grp)
      wait_dma_but<NGD>();
    else
      wait_dma();
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  int kt = 0;
  for (; kt + 8 <= KT; kt += 8) {
    step(kt, I0{});
    step(kt + 1, I1{});
    step(kt + 2, I2{});
    step(kt + 3, I3{});
    step(kt + 4, I4{});
    step(kt + 5, I5{});
    step(kt + 6, I6{});
    step(kt + 7, I7{});
  }
  if (kt < KT) {  // KT % 4 == 0: one more group of four
    step(kt, I0{});
    step(kt + 1, I1{});
    step(kt + 2, I2{});
    step(kt + 3, I3{});
  }
  pending();  // the last step's last substep

  // ---- T: lane (l32, h) of wave (wi, wj) holds T[m][32 q + 8 v + 4 h + e]
  // in tacc[q][4 v + e], m = 64 wj + 32 wi + l32 of the tile.  The column
  // tile 0 stores it; every tile passes bf16(s T) (zero past r) through LDS
  // (row m, 128 bytes, after the stages' 64 KB of output staging) to the
  // waves of the expand.
  if (T16) {
    // lane l holds T[m][4 (l / 16) + e] in t16[q][e], m = 64 wj + 32 wi + 16 q
    // + l % 16 (ranks past r: garbage rows of the A slice, never used)
    const int j = 4 * (lane >> 4);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ml = 64 * wj + 32 * wi + 16 * q + (lane & 15);
      const int64_t m16 = j0 + ml;
      if (tile_i == 0 && p.T_out && m16 < M) {
        float* trow = p.T_out + m16 * r;
        if (j + 4 <= r && (r & 3) == 0) {
          *reinterpret_cast<f32x4*>(trow + j) = t16[q];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < r) trow[j + e] = t16[q][e];
        }
      }
      float e4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) e4[e] = j + e < r ? p.s * t16[q][e] : 0.0f;
      typedef __attribute__((address_space(3))) u32x2* lds_ptr;
      *(lds_ptr)(uintptr_t)(sbase + 65536 + (uint32_t)(ml * 128 + 2 * j)) =
          u32x2{pack_bf16x2(e4[0], e4[1]), pack_bf16x2(e4[2], e4[3])};
    }
  }
  const int64_t mt = j0 + 64 * wj + 32 * wi + l32;
  if (!T16 && tile_i == 0 && p.T_out && mt < M) {
    float* trow = p.T_out + mt * r;
#pragma unroll
    for (int q = 0; q < RQ; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 32 * q + 8 * v + 4 * h;
        if (j + 4 <= r && (r & 3) == 0) {
          *reinterpret_cast<f32x4*>(trow + j) =
              f32x4{tacc[q][4 * v], tacc[q][4 * v + 1], tacc[q][4 * v + 2], tacc[q][4 * v + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < r) trow[j + e] = tacc[q][4 * v + e];
        }
      }
  }
  const uint32_t tl = sbase + 65536;
  if (!T16) {
    const uint32_t trow = tl + (uint32_t)((64 * wj + 32 * wi + l32) * 128);
    const float sc = p.s;
#pragma unroll
    for (int q = 0; q < RQ; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 32 * q + 8 * v + 4 * h;
        float e4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) e4[e] = j + e < r ? sc * tacc[q][4 * v + e] : 0.0f;
        typedef __attribute__((address_space(3))) u32x2* lds_ptr;
        *(lds_ptr)(uintptr_t)(trow + 2 * j) =
            u32x2{pack_bf16x2(e4[0], e4[1]), pack_bf16x2(e4[2], e4[3])};
      }
  }
  __syncthreads();

  // ---- expand: acc += B rows x bf16(s T) over rank chunks of 16
  for (int c = 0; c < r; c += 16) {
    const int jr = c + 8 * h;
    u32x4 ef[2], vf[2];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
      const int64_t i = i0 + 64 * wi + 32 * ns + l32;
      ef[ns] = e_operand_row(p.E + i * r, jr, r);
    }
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
      vf[ms] = read16(tl + (uint32_t)((64 * wj + 32 * (ms ^ wi) + l32) * 128 + 2 * jr));
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) acc[ns][ms] = mfma32(ef[ns], vf[ms], acc[ns][ms]);
  }

  // ---- store: bf16 tile in LDS (row j of 256 bytes; chunk c at c ^ (j & 15)),
  // then whole 256-byte output row segments with 16-byte stores
  __syncthreads();
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int j = 64 * wj + 32 * (ms ^ wi) + l32;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 64 * wi + 32 * ns + 8 * q + 4 * h;  // 4 outputs i .. i + 3
        const uint32_t a = sbase + (uint32_t)(j * 256 + (((i >> 3) ^ (j & 15)) << 4) + (i & 7) * 2);
        typedef __attribute__((address_space(3))) u32x2* lds_ptr;
        *(lds_ptr)(uintptr_t)a = u32x2{pack_bf16x2(acc[ns][ms][4 * q], acc[ns][ms][4 * q + 1]),
                                       pack_bf16x2(acc[ns][ms][4 * q + 2], acc[ns][ms][4 * q + 3])};
      }
  }
  __syncthreads();
  const int cl = tid & 15;
#pragma unroll 4
  for (int it = 0; it < 8; ++it) {
    const int j = 32 * it + (tid >> 4);
    const int64_t m = j0 + j;
    const u32x4 v = read16(sbase + (uint32_t)(j * 256 + ((cl ^ (j & 15)) << 4)));
    if (m < M) *reinterpret_cast<u32x4*>(p.Y + m * N + i0 + 8 * cl) = v;
  }
}


// ---------------------------------------------------------------------------
// dX with the NF4 weight dequantised inside the K loop and U = dY B formed in
// the same loop (no bf16 copy of W0 anywhere, no separate launch for U):
// dX = dY deq(W0) + (s U) A.
//
// Tile 128 (outputs k) x 256 (activation rows m), eight waves (two per SIMD);
// wave (wi, wj) owns the 64 x 64 block at (64 wi, 64 wj).  The reduction runs
// over the weight's rows n, 64 per step:
//   * the dY tile (256 rows x 128 bytes) and the step's rows of B (64 x r
//     bf16, contiguous in B) arrive by direct-to-LDS loads;
//   * the weight tile is W0's rows n0 .. n0 + 63 over the tile's 128 columns:
//     64 code bytes per row and two NF4 blocks, which share one 8-bit
//     constant word and one c2 (the blocks are an even-odd pair, so they sit
//     in one dword of constants and one group of 256).  Codes and constants
//     come by direct-to-LDS loads in groups of two steps (128 rows), issued
//     two steps before the step that dequantises them, into two code buffers.
//     Thread t dequantises row t / 8, columns 16 (t & 7) .. + 15 of the next
//     step (one block: the same byte-plane table and v_perm_b32 lookups as
//     the forward), between the current step's MFMAs, and stores them into
//     the other stage's weight tile in storage order (row n of 256 bytes,
//     16-byte chunk c at c ^ 4 (n & 3) ^ (n >> 2 & 1));
//   * the weight operand (one output column, eight consecutive n) is read
//     with the transposing ds_read_b64_tr_b16; with the swizzle above the 32
//     lanes of a read touch 16 distinct 16-byte bank groups, and so do the
//     16 lanes of each quarter of a dequantising store (8 rows x 8 chunks per
//     instruction: the low bit of the swizzle puts rows n and n + 4 on
//     opposite halves of the bank groups);
//   * U: the waves holding the same 64 dY rows split them as in the forward;
//     the B operand (one rank, eight consecutive n) is read from the step's
//     rows of B with the same transposing read (ranks past r read
//     neighbouring rows; those results are never used).
// Needs r % 8 == 0 (the transposing read's 8-byte alignment in rows of 2r
// bytes).  The column tile 0 stores U; the expand adds (s U) A in the
// epilogue as in g256_kernel.
constexpr int kDCodes = 128 * 64;                 // codes of a group: 128 rows x 64 bytes
constexpr int kDCB = kDCodes + 512 + 512;         // + constant words, + c2 (per row)
constexpr int kDBS = 64 * 128 + 256;              // step's rows of B (up to 64 x 64), padded

struct Q256DxParams {
  const uint16_t* P;  // dY, M x N
  WeightArgs W;       // NF4 weight, N x K
  const uint16_t* G;  // B, N x r
  float* U_out;       // U, M x r float32 (column tile 0 stores it)
  const uint16_t* E;  // A, r x K
  uint16_t* Y;        // dX, M x K
  int64_t M, N, K;
  int32_t r;
  float s;
  int32_t ti, tj;
  NF4Table tab;
};

template <int WK, bool FP8, int RQ>
__global__ __launch_bounds__(kQThreads) void q256_dx_kernel(Q256DxParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kQStage];
  __shared__ __attribute__((aligned(1024))) char cst[2 * kDCB];
  __shared__ __attribute__((aligned(1024))) char bslc[2 * kDBS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave & 1, wj = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;
  float cbq[4];
  quad_levels(p.tab, lane, cbq);
  const int t = xcd_tile(blockIdx.x, p.ti * p.tj);
  const int tile_j = t / p.ti, tile_i = t - tile_j * p.ti;
  const int64_t i0 = (int64_t)tile_i * kQI, j0 = (int64_t)tile_j * kQJ;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KT = (int)(N / kGK);  // even
  const int NG = KT / 2;
  const int r = p.r;
  const uint32_t sbase = lds_addr(smem);
  const uint32_t cbase = lds_addr(cst);
  const uint32_t bbase = lds_addr(bslc);

  // dY DMA: wave w fills rows 32 w .. 32 w + 31, 8 rows per instruction
  uint32_t poff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 32 * wave + 8 * u + (lane >> 3);
    int64_t m = j0 + row;
    m = m < M ? m : M - 1;
    poff[u] = (uint32_t)((m * N + 8 * ((lane & 7) ^ rswz(row))) * 2);
  }
  const char* pbase0 = reinterpret_cast<const char*>(p.P);
  auto issue_act = [&](int kt, int b) {
    const uint32_t at = sbase + b * kQStage + kQWT;
    const char* pb = pbase0 + (int64_t)kt * kGK * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16(pb, poff[u], at + (32 * wave + 8 * u) * 128);
  };
  // the step's rows of B: 128 r contiguous bytes, wave w brings the w-th KB
  const bool b_part = 8 * wave < r;
  const char* gbase0 = reinterpret_cast<const char*>(p.G);
  auto issue_b = [&](int kt, int b) {
    if (b_part)
      dma16(gbase0 + (int64_t)kt * kGK * r * 2, (uint32_t)(1024 * wave + 16 * lane),
            bbase + b * kDBS + 1024 * wave);
  };
  // Group g (steps 2 g, 2 g + 1: weight rows 128 g .. + 127): codes, wave w
  // rows 16 w .. + 15 (four lanes per 64-byte row); waves 0 and 1 the dwords
  // of 8-bit constants (float32 absmax of the even block without a second
  // level) of rows 0 .. 63 and 64 .. 127, waves 2 and 3 the rows' c2 (the odd
  // block's absmax).
  const int64_t KB = K / 64;
  const int64_t cb0 = i0 / 64;  // the tile's first block within a row (even)
  const uint32_t coff = (uint32_t)((16 * wave + (lane >> 2)) * (K / 2) + i0 / 2 + 16 * (lane & 3));
  const int crow = 64 * (wave & 1) + lane;  // constants row of waves 0 .. 3
  const bool c_part = wave < 4;
  auto issue_group = [&](int g, int buf) {
    const uint32_t cb = cbase + buf * kDCB;
    dma16(reinterpret_cast<const char*>(p.W.codes) + (int64_t)g * 128 * (K / 2), coff,
          cb + 16 * wave * 64);
    if (c_part) {
      const int64_t blk = (128 * (int64_t)g + crow) * KB + cb0;
      const uint32_t dst = cb + kDCodes + (wave >> 1) * 512 + 256 * (wave & 1);
      if (WK == kNF4DQ) {
        if (wave < 2) dma4(p.W.q8, (uint32_t)(blk & ~(int64_t)3), dst);
        else dma4(p.W.c2, (uint32_t)((blk >> 8) * 4), dst);
      } else {
        dma4(p.W.absmax, (uint32_t)((blk + (wave >> 1)) * 4), dst);
      }
    }
  };
  auto wait_but_group = [&]() {
    if (c_part) wait_dma_but<2>();
    else wait_dma_but<1>();
  };
  // dequantisation: thread t, row t / 8 of the step, columns 16 (t & 7) .. + 15
  const int dx_row = tid >> 3, dx_j = tid & 7;
  auto codes_at = [&](int buf, int pos) {
    typedef __attribute__((address_space(3))) const u32x2* lp;
    return *(lp)(uintptr_t)(cbase + buf * kDCB + (64 * pos + dx_row) * 64 + 8 * dx_j);
  };
  auto raw_at = [&](int buf, int pos) {
    typedef __attribute__((address_space(3))) const uint32_t* lp;
    const uint32_t cb = cbase + buf * kDCB + kDCodes + 4 * (64 * pos + dx_row);
    return u32x2{*(lp)(uintptr_t)cb, *(lp)(uintptr_t)(cb + 512)};
  };
  const int qsh = 8 * ((int)(cb0 & 3) + (dx_j >> 2));  // the block's byte in the dword
  auto scale_of = [&](const u32x2& v) {
    if (WK == kNF4DQ) return dq_value<FP8>((v[0] >> qsh) & 0xFFu) * dq_step(__uint_as_float(v[1]));
    return __uint_as_float((dx_j >> 2) ? v[1] : v[0]);
  };
  uint32_t wdst[2];
#pragma unroll
  for (int d = 0; d < 2; ++d)
    wdst[d] = (uint32_t)(dx_row * 256 +
                         (((2 * dx_j + d) ^ (4 * (dx_row & 3)) ^ ((dx_row >> 2) & 1)) << 4));

  // operand reads: dY as the forward's activations; the weight and B
  // operands transposed (lane group of 16: rows nlo = gc / 4 and nlo + 4,
  // four columns 4 (gc & 3) .. + 3 of its 16-column half)
  const int sw = rswz(l32);
  uint32_t pcx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) pcx[s] = (uint32_t)(((2 * s + h) ^ sw) << 4);
  uint32_t prowm[2];  // dY operand ms: rows 64 wj + 32 (ms ^ wi) .. + 31, as the forward
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) prowm[ms] = (uint32_t)((64 * wj + 32 * (ms ^ wi) + l32) * 128);
  const int gc = l32 & 15, half = l32 >> 4, nlo = gc >> 2;
  // rows 16 s + 8 h + nlo (swizzle bit 0 clear) and those + 4 (bit 0 set)
  uint32_t qtr[2], qtrh[2];
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) {
    const int col = 64 * wi + 32 * ns + 16 * half + 4 * (gc & 3);
    const int pc = (col >> 3) ^ (4 * nlo);
    qtr[ns] = (uint32_t)((8 * h + nlo) * 256 + (pc << 4) + (col & 7) * 2);
    qtrh[ns] = (uint32_t)((8 * h + nlo + 4) * 256 + ((pc ^ 1) << 4) + (col & 7) * 2);
  }
  const uint32_t btr = (uint32_t)((8 * h + nlo) * 2 * r + 2 * (16 * half + 4 * (gc & 3)));
  auto load_frags = [&](uint32_t st, uint32_t bs, int s, u32x4 (&wf)[2], u32x4 (&xf)[2],
                        u32x4 (&bf)[RQ]) {
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) xf[ms] = read16(st + kQWT + prowm[ms] + pcx[s]);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
      const uint32_t a = st + (uint32_t)(16 * s * 256);
      const u32x2 lo = read_tr(a + qtr[ns]), hi = read_tr(a + qtrh[ns]);
      wf[ns] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const uint32_t a = bs + (uint32_t)(16 * s * 2 * r + 64 * q) + btr;
      const u32x2 lo = read_tr(a), hi = read_tr(a + (uint32_t)(8 * r));
      bf[q] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };

  f32x16 acc[2][2], uacc[RQ];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) uacc[q][v] = 0.0f;

  // prologue: step 0's tiles in stage 0, groups 0 and 1 in code buffers 0, 1;
  // step 0 dequantised into stage 0
  issue_act(0, 0);
  issue_b(0, 0);
  issue_group(0, 0);
  if (NG > 1) issue_group(1, 1);
  wait_dma();
  __syncthreads();
  {
    const u32x2 cw = codes_at(0, 0);
    const PermTable pt = perm_table_quad(cbq, scale_of(raw_at(0, 0)));
#pragma unroll
    for (int d = 0; d < 2; ++d) write16(sbase + wdst[d], perm_deq8(cw[d], pt));
  }
  __syncthreads();

  // Step kt (J = kt mod 4: stage and position in the group J & 1, code
  // buffer J >> 1): the dY and B loads of step kt + 1; in position 1 the
  // loads of group kt / 2 + 2 into this step's (now free) code buffer; the
  // MFMAs of step kt with the dequantisation of step kt + 1 between them; at
  // the end, wait for everything but the group loads issued in this step.
  // As in the forward, a step's last substep of MFMAs runs after the barrier.
  u32x4 pw[2], px[2], pb[RQ];
#pragma unroll
  for (int i = 0; i < 2; ++i) pw[i] = px[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < RQ; ++q) pb[q] = u32x4{0u, 0u, 0u, 0u};
  auto pending = [&]() {
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) acc[ns][ms] = mfma32(pw[ns], px[ms], acc[ns][ms]);
#pragma unroll
    for (int q = 0; q < RQ; ++q) uacc[q] = mfma32(pb[q], px[0], uacc[q]);
  };
  auto step = [&](int kt, auto jj) {
    constexpr int J = decltype(jj)::value;
    constexpr int B = J & 1, POS = J & 1, BUF = J >> 1;
    constexpr int NPOS = POS ^ 1, NBUF = POS == 1 ? BUF ^ 1 : BUF;  // step kt + 1
    const bool more = kt + 1 < KT;
    if (more) {
      issue_act(kt + 1, B ^ 1);
      issue_b(kt + 1, B ^ 1);
    }
    const bool grp = POS == 1 && (kt >> 1) + 2 < NG;
    if (grp) issue_group((kt >> 1) + 2, BUF);
    const uint32_t st = sbase + B * kQStage;
    const uint32_t bs = bbase + B * kDBS;
    const uint32_t wt = sbase + (B ^ 1) * kQStage;
    // (after the last step the words read here are stale and their
    // dequantised values land in a tile nobody reads)
    u32x4 wf[2][2], xf[2][2], bf[2][RQ];
    load_frags(st, bs, 0, wf[0], xf[0], bf[0]);
    const u32x2 cw = codes_at(NBUF, NPOS);
    const u32x2 raw = raw_at(NBUF, NPOS);
    __builtin_amdgcn_sched_barrier(0);
    pending();  // the previous step's last substep
    __builtin_amdgcn_sched_barrier(0);
    PermTable pt;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = s & 1;
      if (s < 3) load_frags(st, bs, s + 1, wf[c ^ 1], xf[c ^ 1], bf[c ^ 1]);
      if (s == 0) pt = perm_table_quad(cbq, scale_of(raw));
      if (s < 3) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) acc[ns][ms] = mfma32(wf[c][ns], xf[c][ms], acc[ns][ms]);
#pragma unroll
        for (int q = 0; q < RQ; ++q) uacc[q] = mfma32(bf[c][q], xf[c][0], uacc[q]);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          pw[i] = wf[c][i];
          px[i] = xf[c][i];
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) pb[q] = bf[c][q];
      }
      if (s == 1 || s == 2) write16(wt + wdst[s - 1], perm_deq8(cw[s - 1], pt));
      if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, 6 + 2 * RQ, 0);
      if (s == 0) {
#pragma unroll
        for (int i = 0; i < 4 + RQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 52 / (4 + RQ), 0);
        }
      } else if (s < 3) {
#pragma unroll
        for (int i = 0; i < 4 + RQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 32 / (4 + RQ), 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (grp)
      wait_but_group();
    else
      wait_dma();
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int kt = 0;
  for (; kt + 4 <= KT; kt += 4) {
    step(kt, I0{});
    step(kt + 1, I1{});
    step(kt + 2, I2{});
    step(kt + 3, I3{});
  }
  if (kt < KT) {  // KT even: one more group of two
    step(kt, I0{});
    step(kt + 1, I1{});
  }
  pending();  // the last step's last substep

  // ---- U as T in the forward: column tile 0 stores it, bf16(s U) (zero
  // past r) goes through LDS to the waves of the expand
  const int64_t mt = j0 + 64 * wj + 32 * wi + l32;
  if (tile_i == 0 && p.U_out && mt < M) {
    float* urow = p.U_out + mt * r;
#pragma unroll
    for (int q = 0; q < RQ; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 32 * q + 8 * v + 4 * h;
        if (j < r)  // r % 8 == 0: all four or none
          *reinterpret_cast<f32x4*>(urow + j) =
              f32x4{uacc[q][4 * v], uacc[q][4 * v + 1], uacc[q][4 * v + 2], uacc[q][4 * v + 3]};
      }
  }
  const uint32_t tl = sbase + 65536;
  {
    const uint32_t trow = tl + (uint32_t)((64 * wj + 32 * wi + l32) * 128);
    const float sc = p.s;
#pragma unroll
    for (int q = 0; q < RQ; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 32 * q + 8 * v + 4 * h;
        const bool in = j < r;
        typedef __attribute__((address_space(3))) u32x2* lds_ptr;
        *(lds_ptr)(uintptr_t)(trow + 2 * j) =
            in ? u32x2{pack_bf16x2(sc * uacc[q][4 * v], sc * uacc[q][4 * v + 1]),
                       pack_bf16x2(sc * uacc[q][4 * v + 2], sc * uacc[q][4 * v + 3])}
               : u32x2{0u, 0u};
      }
  }
  __syncthreads();

  // ---- expand: acc += A columns x bf16(s U) over rank chunks of 16
  for (int c = 0; c < r; c += 16) {
    const int jr = c + 8 * h;
    u32x4 ef[2], vf[2];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
      const int64_t i = i0 + 64 * wi + 32 * ns + l32;
      ef[ns] = e_operand_col(p.E, K, i, jr, r);
    }
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
      vf[ms] = read16(tl + (uint32_t)((64 * wj + 32 * (ms ^ wi) + l32) * 128 + 2 * jr));
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) acc[ns][ms] = mfma32(ef[ns], vf[ms], acc[ns][ms]);
  }

  // ---- store: bf16 tile in LDS (row j of 256 bytes; chunk c at c ^ (j & 15)),
  // then whole 256-byte output row segments with 16-byte stores
  __syncthreads();
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int j = 64 * wj + 32 * (ms ^ wi) + l32;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 64 * wi + 32 * ns + 8 * q + 4 * h;  // 4 outputs i .. i + 3
        const uint32_t a = sbase + (uint32_t)(j * 256 + (((i >> 3) ^ (j & 15)) << 4) + (i & 7) * 2);
        typedef __attribute__((address_space(3))) u32x2* lds_ptr;
        *(lds_ptr)(uintptr_t)a = u32x2{pack_bf16x2(acc[ns][ms][4 * q], acc[ns][ms][4 * q + 1]),
                                       pack_bf16x2(acc[ns][ms][4 * q + 2], acc[ns][ms][4 * q + 3])};
      }
  }
  __syncthreads();
  const int cl = tid & 15;
#pragma unroll 4
  for (int it = 0; it < 8; ++it) {
    const int j = 32 * it + (tid >> 4);
    const int64_t m = j0 + j;
    const u32x4 v = read16(sbase + (uint32_t)(j * 256 + ((cl ^ (j & 15)) << 4)));
    if (m < M) *reinterpret_cast<u32x4*>(p.Y + m * K + i0 + 8 * cl) = v;
  }
}

}  // namespace

namespace dispatch {

// The bound of the in-kernel waits between workgroups (polls of s_sleep 2,
// about 8 ms at the default).
static std::atomic<int32_t> g_wait_limit{kDefaultWaitPolls};

void set_wait_limit(int32_t polls) {
  g_wait_limit.store(polls > 0 ? polls : polls == 0 ? kDefaultWaitPolls : -1);
}
int32_t wait_limit() { return g_wait_limit.load(); }

int take_g256_giveups(uint64_t* n) {
  unsigned long long v = 0, z = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_wait_giveups), sizeof(v));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_wait_giveups), &z, sizeof(z));
  *n = v;
  return hip_fail(e, "split-K give-up count");
}

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

// a 256-byte header (unused), then four flag words per tile
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
  p.flags = (int32_t*)(w + 256);
  p.part = (float*)(w + g256_flag_bytes(M, NI));
  p.tpx = (int32_t)cdiv(pl.tiles, 8);
  p.spin = wait_limit();
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

// The NF4 forward with the dequantisation in the K loop: enough 128 x 256
// tiles to fill the chip, whole 128-row weight tiles.
bool q256_fwd_fits(const lq_weight& W, int64_t M) {
  return W.kind == LQ_WEIGHT_NF4 && W.N % kQI == 0 && W.K % 256 == 0 &&
         (W.N / kQI) * cdiv(M, kQJ) >= 192 && (double)M * W.K * 2 < 4294967296.0;
}

template <int RQ, bool T16>
void launch_q256_fmt(const lq_weight& W, const Q256Params& p, unsigned blocks, hipStream_t st) {
  if (W.double_quant == LQ_DQ_FP8)
    hipLaunchKernelGGL((q256_fwd_kernel<kNF4DQ, true, RQ, T16>), dim3(blocks), dim3(kQThreads), 0, st, p);
  else if (W.double_quant)
    hipLaunchKernelGGL((q256_fwd_kernel<kNF4DQ, false, RQ, T16>), dim3(blocks), dim3(kQThreads), 0, st, p);
  else
    hipLaunchKernelGGL((q256_fwd_kernel<kNF4, false, RQ, T16>), dim3(blocks), dim3(kQThreads), 0, st, p);
}

int launch_q256_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, float* T_out,
                    const void* B, int64_t r, float s, void* Y, hipStream_t st) {
  Q256Params p{};
  p.P = (const uint16_t*)X;
  p.W = weight_args(W);
  p.A = (const uint16_t*)A;
  p.T_out = T_out;
  p.E = (const uint16_t*)B;
  p.Y = (uint16_t*)Y;
  p.M = M;
  p.N = W.N;
  p.K = W.K;
  p.r = (int32_t)r;
  p.s = s;
  p.ti = (int32_t)(W.N / kQI);
  p.tj = (int32_t)cdiv(M, kQJ);
  p.tab = nf4_table(W.codebook);
  const unsigned blocks = (unsigned)(p.ti * p.tj);
  timing_begin("q256_fwd", st);
  if (r <= 16)
    launch_q256_fmt<1, true>(W, p, blocks, st);
  else if (r <= 32)
    launch_q256_fmt<1, false>(W, p, blocks, st);
  else
    launch_q256_fmt<2, false>(W, p, blocks, st);
  timing_end(st);
  return hip_fail(hipGetLastError(), "q256 launch");
}

// dX of an NF4 weight with the dequantisation and U in the K loop: whole
// 128-column output tiles, weight rows in groups of 128, whole dwords of
// 8-bit constants per row (K % 256), r % 8 == 0, enough tiles to fill the
// chip.
bool q256_dx_fits(const lq_weight& W, int64_t M, int64_t r) {
  return W.kind == LQ_WEIGHT_NF4 && W.K % 256 == 0 && W.N % 128 == 0 && r % 8 == 0 && r <= 64 &&
         (W.K / kQI) * cdiv(M, kQJ) >= 192 && (double)M * W.N * 2 < 4294967296.0;
}

template <int RQ>
void launch_q256dx_fmt(const lq_weight& W, const Q256DxParams& p, unsigned blocks,
                       hipStream_t st) {
  if (W.double_quant == LQ_DQ_FP8)
    hipLaunchKernelGGL((q256_dx_kernel<kNF4DQ, true, RQ>), dim3(blocks), dim3(kQThreads), 0, st, p);
  else if (W.double_quant)
    hipLaunchKernelGGL((q256_dx_kernel<kNF4DQ, false, RQ>), dim3(blocks), dim3(kQThreads), 0, st, p);
  else
    hipLaunchKernelGGL((q256_dx_kernel<kNF4, false, RQ>), dim3(blocks), dim3(kQThreads), 0, st, p);
}

int launch_q256_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
                   int64_t r, float s, void* dX, float* U_out, hipStream_t st) {
  Q256DxParams p{};
  p.P = (const uint16_t*)dY;
  p.W = weight_args(W);
  p.G = (const uint16_t*)B;
  p.U_out = U_out;
  p.E = (const uint16_t*)A;
  p.Y = (uint16_t*)dX;
  p.M = M;
  p.N = W.N;
  p.K = W.K;
  p.r = (int32_t)r;
  p.s = s;
  p.ti = (int32_t)(W.K / kQI);
  p.tj = (int32_t)cdiv(M, kQJ);
  p.tab = nf4_table(W.codebook);
  const unsigned blocks = (unsigned)(p.ti * p.tj);
  timing_begin("q256_dx", st);
  if (r <= 32)
    launch_q256dx_fmt<1>(W, p, blocks, st);
  else
    launch_q256dx_fmt<2>(W, p, blocks, st);
  timing_end(st);
  return hip_fail(hipGetLastError(), "q256 dx launch");
}

// the NF4 weight dequantised to bf16 into the workspace at q (when the prep
// kernel cannot take the shrink as well)
int bf16_weight(const lq_weight& W, void* q, hipStream_t st) {
  return launch_nf4_dequantize(W.codes, W.q8, W.c2, W.absmax, W.double_quant, W.codebook,
                               W.N * W.K, q, LQ_BF16, st);
}

}  // namespace

bool big_fwd_eligible(int64_t M, int64_t N, int64_t K) { return g256_fits(M, N, K); }
bool big_wide_tiles(int64_t M, int64_t NI) { return g256_plan(M, NI).jm == 4; }
bool big_dx_eligible(int64_t M, int64_t N, int64_t K) { return g256_fits(M, K, N); }

// [g256: header, flags, split-K slots] [T when T_out is NULL] [bf16 W0]
size_t big_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  return align256(g256_ws_bytes(M, N)) + align256((size_t)(M * r) * 4) + (size_t)(N * K) * 2;
}

// [g256: header, flags, split-K slots] [bf16 W0]
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

bool inloop_fwd_eligible(const lq_weight& W, int64_t M) { return q256_fwd_fits(W, M); }
bool inloop_dx_eligible(const lq_weight& W, int64_t M, int64_t r) { return q256_dx_fits(W, M, r); }

int inloop_dx(const void* dY, int64_t M, const lq_weight& W, const void* A, const void* B,
              int64_t r, float s, void* dX, float* U_out, hipStream_t st) {
  return launch_q256_dx(dY, M, W, A, B, r, s, dX, U_out, st);
}

int inloop_fwd(const void* X, int64_t M, const lq_weight& W, const void* A, const void* B,
               int64_t r, float s, void* Y, float* T_out, hipStream_t st) {
  return launch_q256_fwd(X, M, W, A, T_out, B, r, s, Y, st);
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

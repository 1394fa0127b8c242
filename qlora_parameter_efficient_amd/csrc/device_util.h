// Device helpers shared by the bf16 kernels: MFMA wrappers, NF4 dequantisation
// through a byte-indexed LDS table, and small register transposes.
//
// MFMA operand layout used throughout (gfx950 v_mfma_f32_32x32x16_bf16):
// lane l supplies row (l % 32) of the A operand and column (l % 32) of the B
// operand, each as 8 consecutive reduction elements starting at 8 * (l / 32);
// the 16 accumulator values of lane l are C[8*(v/4) + 4*(l/32) + v%4][l % 32].
// Because both operands carry the reduction index the same way, any fixed
// relabelling of the 16 reduction elements that is applied to both operands
// leaves the product unchanged; the kernels use that to read each operand
// in the order that is cheapest for it.
#pragma once

#include "common.h"

namespace lq {

constexpr int kPitch = 72;  // LDS row pitch in bf16 elements: 64 + 8 padding

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Weight formats, fixed at compile time: dense bf16, NF4 with 8-bit double
// quantised constants, NF4 with float32 absmax.
// kNF4DQ covers both 8-bit constant formats (integer or E4M3); which one is
// a uniform kernel argument, read where a block scale is formed.
constexpr int kDense = 0, kNF4DQ = 1, kNF4 = 2;

inline int weight_format(const lq_weight& w) {
  if (w.kind == LQ_WEIGHT_DENSE) return kDense;
  return w.double_quant ? kNF4DQ : kNF4;
}


__device__ __forceinline__ u32x4 sel4(bool ok, const u32x4& v) {
  return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

// NF4 weight descriptor as the kernels see it.
struct WeightArgs {
  const uint16_t* dense;
  const uint8_t* codes;
  const uint8_t* q8;
  const float* c2;
  const float* absmax;
  int64_t N, K;
  int32_t dq;
  int32_t pad;
};

inline WeightArgs weight_args(const lq_weight& w) {
  WeightArgs a;
  a.dense = (const uint16_t*)w.dense;
  a.codes = w.codes;
  a.q8 = w.q8;
  a.c2 = w.c2;
  a.absmax = w.absmax;
  a.N = w.N;
  a.K = w.K;
  a.dq = w.double_quant;
  a.pad = 0;
  return a;
}

// Raw block constants as loaded: the 8-bit constant and its group's c2 (or
// the float32 absmax bits).  Kept raw so that no arithmetic waits on the load
// until the value is needed.
struct ScaleRaw {
  uint32_t q;
  float c2;
  int64_t g;
};

__device__ __forceinline__ ScaleRaw load_scale(const WeightArgs& w, int64_t blk) {
  ScaleRaw s;
  if (w.dq) {
    s.q = w.q8[blk];
    s.g = blk >> 8;
    s.c2 = w.c2[s.g];
  } else {
    s.q = __float_as_uint(w.absmax[blk]);
    s.g = -1;
    s.c2 = 0.0f;
  }
  return s;
}

// Block scale a' = fl32(q * fl32(c2 / 127)) (or the float32 absmax), q the
// integer or E4M3 value of the 8-bit constant, with the
// second-level step cached while consecutive blocks stay in one group.
struct ScaleCache {
  int64_t g;
  float step;
  __device__ __forceinline__ void init() {
    g = -1;
    step = 0.0f;
  }
  __device__ __forceinline__ float finish(const WeightArgs& w, const ScaleRaw& s) {
    if (!w.dq) return __uint_as_float(s.q);
    if (s.g != g) {
      g = s.g;
      step = dq_step(s.c2);
    }
    return dq_q_rt(w.dq, s.q) * step;
  }
  __device__ __forceinline__ float scale(const WeightArgs& w, int64_t blk) {
    return finish(w, load_scale(w, blk));
  }
};

// Second-level steps fl32(c2[g] / 127) for groups g_lo .. g_lo + count - 1,
// computed cooperatively into LDS so that a block scale is one LDS read and
// one multiply: a' = fl32(q8 * tab[g - g_lo]).
__device__ __forceinline__ void build_steps(float* tab, const WeightArgs& w, int64_t g_lo,
                                            int count) {
  for (int i = threadIdx.x; i < count; i += blockDim.x) tab[i] = dq_step(w.c2[g_lo + i]);
}

// The raw 8-bit constant of a block and its group relative to a table base
// (or the float32 absmax bits when there is no second level).
struct ScaleRef {
  uint32_t q;
  int32_t gi;
};

__device__ __forceinline__ ScaleRef load_scale_ref(const WeightArgs& w, int64_t blk, int64_t g_lo) {
  ScaleRef s;
  if (w.dq) {
    s.q = w.q8[blk];
    s.gi = (int32_t)((blk >> 8) - g_lo);
  } else {
    s.q = __float_as_uint(w.absmax[blk]);
    s.gi = 0;
  }
  return s;
}

__device__ __forceinline__ float scale_from(const WeightArgs& w, const ScaleRef& s,
                                            const float* tab) {
  return w.dq ? dq_q_rt(w.dq, s.q) * tab[s.gi] : __uint_as_float(s.q);
}

// lut[b] = (cb[b & 15], cb[b >> 4]): both levels of one code byte.  Built by a
// 256-thread workgroup; the caller synchronises before use.
__device__ __forceinline__ void build_lut(float2* lut, const NF4Table& tab) {
  const int t = threadIdx.x;
  if (t < 256) {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((t & 15) == i) lo = tab.cb[i];
      if ((t >> 4) == i) hi = tab.cb[i];
    }
    lut[t] = make_float2(lo, hi);
  }
}

// Eight codes (one 32-bit word, element e in bits 4e..4e+3) -> eight bf16
// values RNE(fl32(cb[code] * a)) packed in natural element order, in two
// halves so that the table reads can be issued well before the products:
// lut_fetch reads the levels of the four code bytes, lut_finish scales and
// rounds them.
struct LutFetch {
  float2 v[4];
};

__device__ __forceinline__ LutFetch lut_fetch(uint32_t w, const float2* lut) {
  LutFetch f;
#pragma unroll
  for (int p = 0; p < 4; ++p) f.v[p] = lut[(w >> (8 * p)) & 0xFFu];
  return f;
}

__device__ __forceinline__ u32x4 lut_finish(const LutFetch& f, float a) {
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(f.v[p].x * a, f.v[p].y * a);
  return o;
}

__device__ __forceinline__ u32x4 deq8(uint32_t w, float a, const float2* lut) {
  return lut_finish(lut_fetch(w, lut), a);
}

// (lo half of x, lo half of y) and (hi half of x, hi half of y).
__device__ __forceinline__ uint32_t pair_lo(uint32_t x, uint32_t y) {
  return (x & 0xFFFFu) | (y << 16);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t x, uint32_t y) {
  return (x >> 16) | (y & 0xFFFF0000u);
}

// Per-block level table in registers: the 16 bf16 results t_i =
// RNE(fl32(cb[i] a')) of one NF4 block, as byte planes (lo[k] holds the low
// bytes of t_4k .. t_4k+3, hi[k] the high bytes), so that one v_perm_b32
// looks up four codes at once.
struct PermTable {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ PermTable perm_table(const NF4Table& tab, float a) {
  uint32_t pr[8];  // bf16 pairs (t_2k, t_2k+1)
#pragma unroll
  for (int k = 0; k < 8; ++k) pr[k] = pack_bf16x2(tab.cb[2 * k] * a, tab.cb[2 * k + 1] * a);
  PermTable t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bytes 0, 2 of pr[2k] and of pr[2k + 1]; bytes 1, 3 for the high plane
    t.lo[k] = __builtin_amdgcn_perm(pr[2 * k + 1], pr[2 * k], 0x06040200u);
    t.hi[k] = __builtin_amdgcn_perm(pr[2 * k + 1], pr[2 * k], 0x07050301u);
  }
  return t;
}

// The same table built by the four lanes of a quad that share the block: lane
// q of the quad forms t_4q .. t_4q+3 from its four levels cbq = cb[4q ..
// 4q + 3] (same products and rounding, so the same bits), and the eight bf16
// pairs are gathered with quad broadcasts: 4 multiplies, 2 conversions and 8
// moves per lane instead of 16 multiplies and 8 conversions.
__device__ __forceinline__ PermTable perm_table_quad(const float (&cbq)[4], float a) {
  const int p0 = (int)pack_bf16x2(cbq[0] * a, cbq[1] * a);
  const int p1 = (int)pack_bf16x2(cbq[2] * a, cbq[3] * a);
  uint32_t pr[8];  // bf16 pairs (t_2k, t_2k+1)
  pr[0] = (uint32_t)__builtin_amdgcn_mov_dpp(p0, 0x00, 0xF, 0xF, false);
  pr[1] = (uint32_t)__builtin_amdgcn_mov_dpp(p1, 0x00, 0xF, 0xF, false);
  pr[2] = (uint32_t)__builtin_amdgcn_mov_dpp(p0, 0x55, 0xF, 0xF, false);
  pr[3] = (uint32_t)__builtin_amdgcn_mov_dpp(p1, 0x55, 0xF, 0xF, false);
  pr[4] = (uint32_t)__builtin_amdgcn_mov_dpp(p0, 0xAA, 0xF, 0xF, false);
  pr[5] = (uint32_t)__builtin_amdgcn_mov_dpp(p1, 0xAA, 0xF, 0xF, false);
  pr[6] = (uint32_t)__builtin_amdgcn_mov_dpp(p0, 0xFF, 0xF, 0xF, false);
  pr[7] = (uint32_t)__builtin_amdgcn_mov_dpp(p1, 0xFF, 0xF, 0xF, false);
  PermTable t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.lo[k] = __builtin_amdgcn_perm(pr[2 * k + 1], pr[2 * k], 0x06040200u);
    t.hi[k] = __builtin_amdgcn_perm(pr[2 * k + 1], pr[2 * k], 0x07050301u);
  }
  return t;
}

// the four levels cb[4q .. 4q + 3] of quad lane q = lane & 3
__device__ __forceinline__ void quad_levels(const NF4Table& tab, int lane, float (&cbq)[4]) {
  const int q = lane & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    cbq[i] = q == 0 ? tab.cb[i] : q == 1 ? tab.cb[4 + i] : q == 2 ? tab.cb[8 + i] : tab.cb[12 + i];
}

// one byte plane for four codes (one per byte of c, values 0..15): the byte
// of t_code for each
__device__ __forceinline__ uint32_t perm_plane(const uint32_t (&pl)[4], uint32_t c7, uint32_t s2) {
  const uint32_t a = __builtin_amdgcn_perm(pl[1], pl[0], c7);  // codes 0..7
  const uint32_t b = __builtin_amdgcn_perm(pl[3], pl[2], c7);  // codes 8..15
  return __builtin_amdgcn_perm(b, a, s2);                       // by bit 3 of each code
}

// Eight codes (element e in bits 4e .. 4e + 3) -> the eight bf16 values t_code
// in natural element order (bit-identical to deq8 with the same a')
__device__ __forceinline__ u32x4 perm_deq8(uint32_t w, const PermTable& t) {
  const uint32_t ce = w & 0x0F0F0F0Fu, co = (w >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
  const uint32_t ce7 = ce & 0x07070707u, co7 = co & 0x07070707u;
  const uint32_t es2 = ((ce >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t os2 = ((co >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t le = perm_plane(t.lo, ce7, es2), he = perm_plane(t.hi, ce7, es2);
  const uint32_t lo = perm_plane(t.lo, co7, os2), ho = perm_plane(t.hi, co7, os2);
  const uint32_t x01 = __builtin_amdgcn_perm(he, le, 0x05010400u);  // (e0, e2)
  const uint32_t x23 = __builtin_amdgcn_perm(he, le, 0x07030602u);  // (e4, e6)
  const uint32_t y01 = __builtin_amdgcn_perm(ho, lo, 0x05010400u);  // (e1, e3)
  const uint32_t y23 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);  // (e5, e7)
  return u32x4{__builtin_amdgcn_perm(y01, x01, 0x05040100u), __builtin_amdgcn_perm(y01, x01, 0x07060302u),
               __builtin_amdgcn_perm(y23, x23, 0x05040100u), __builtin_amdgcn_perm(y23, x23, 0x07060302u)};
}

// Tile -> workgroup mapping.  Workgroups are dispatched round-robin over the
// eight XCDs (block b runs on XCD b % 8); each XCD is given one contiguous
// range of tile indices so that the tiles sharing its L2 are neighbours.
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  return (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

}  // namespace lq

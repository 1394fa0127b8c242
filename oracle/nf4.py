"""NF4 (4-bit NormalFloat) with blockwise absmax and double quantization.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
------------------
* Levels: quantiles of the standard normal distribution, 2^k = 16 of them,
  normalised to [-1, 1] ("LoRA and QLoRA: Mathematical Foundations ...",
  section "1. 4-bit NormalFloat (NF4) Quantization", the q_i formula).
* Blocks: 64 weights share one absmax constant c = max|W|; the block is divided
  by c and each value is mapped to the nearest level (same section, steps 1-3;
  "Large Language Model Fine-tuning and LoRA", section "Quantizing the frozen
  weights: NF4 and double quantization").
* Double quantization: the per-block constants are quantised to 8 bits in
  second-level blocks of 256 constants with one float32 constant c2 each,
  c1_8bit = round(c1 / c2 * 127) ("... Mathematical Foundations ...", section
  "2. Double Quantization (DQ)"; storage 4 + 8/64 + 32/(64*256) bits/param in
  "Large Language Model Fine-tuning and LoRA").
* Dequantization to bf16 happens right before the matrix multiply (both pages).

Readings where the pages are silent or garbled
----------------------------------------------
1. Codebook end points.  The printed q_i averages Q(i/16) and Q((i+1)/16),
   whose outer terms are Q(0) = -inf and Q(1) = +inf, and a symmetric set of
   16 values has no exact zero.  Reading: the asymmetric construction of the
   QLoRA paper the page cites -- 8 positive levels at equally spaced
   probabilities from 1/2 (exclusive) up to 1 - delta, 7 negative levels at
   equally spaced probabilities from 1/2 (exclusive) up to 1 - delta, mirrored,
   plus an exact 0; all divided by Q(1 - delta) so the ends are exactly -1 and
   +1.  delta is half a bin: the positive side spans a 16-bin grid (outer bin
   centre at 1/32 from the tail) and the negative side a 15-bin grid (1/30);
   delta = (1/32 + 1/30) / 2.  Q is computed in float64 by
   ``statistics.NormalDist.inv_cdf`` and each level is rounded once to float32.
2. "Nearest" with ties: thresholds are the float32 midpoints
   t_i = fl32(fl32(cb[i] + cb[i+1]) * 0.5) and code = #{i : x > t_i}; an exact
   tie goes to the lower code.
3. Normalisation: x = fl32(w / c1), correctly rounded float32 division by the
   exact float32 absmax c1.  c1 = 0 gives code 7 (the exact zero) everywhere.
4. Packing: element 2j goes to the low nibble of byte j, element 2j+1 to the
   high nibble.
5. Second-level format: the page's integer formula, q8 = rint(fl32(fl32(c1/c2)
   * 127)) with ties to even, stored as uint8 in [0, 127]; c2 = max c1 over
   the group (an absmax, like the first level); c2 = 0 gives q8 = 0.
6. Dequantization (the plain inverse): a' = fl32(fl32(q8) * fl32(c2 / 127)),
   w' = fl32(cb[code] * a'); the bf16 value is RNE(w').  Without double
   quantization a' = c1.

Format variants the pages also describe
---------------------------------------
7. FP8 second-level constants ("... Mathematical Foundations ...", section
   "2. Double Quantization (DQ)": the constants go to "8-bit integers or FP8";
   "LoRA and QLoRA fine-tuning under the hood", section 3.2, and "Lesson 26"
   call the 8-bit format FP8).  Reading: the same printed formula with "round"
   taken as rounding to the FP8 grid, q = E4M3(fl32(fl32(c1/c2) * 127)), and
   a' = fl32(e4m3(q) * fl32(c2 / 127)).  E4M3 is the OCP 8-bit format with 4
   exponent bits (bias 7), 3 mantissa bits, subnormals m * 2^-9, largest
   finite value 448 and no infinities; rounding is to the nearest value, ties
   to the even code.  Values here lie in [0, 127], so no saturation occurs.
8. Symmetric codebook without zero ("... Mathematical Foundations ...", the
   q_i formula read literally): q_i = (Q(p_i) + Q(p_{i+1})) / 2 for
   i = 0..15 with p_j = j / 16, the infinite end quantiles Q(0) and Q(1)
   replaced by Q(delta) and Q(1 - delta) with the delta of reading 1, then
   divided by the largest so the ends are -1 and +1.  The set is symmetric
   (q_{15-i} = -q_i) and holds no zero.  Ties and zero blocks follow readings
   2 and 3 (code 7, now the negative level nearest zero, times a' = 0).
"""
from __future__ import annotations

import statistics

import numpy as np

BLOCK = 64
DQ_BLOCK = 256
F32 = np.float32


DELTA = 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
CODEBOOKS = ("nf4", "nf4_symmetric")
DQ_FORMATS = ("int8", "fp8")


def nf4_codebook(variant: str = "nf4") -> np.ndarray:
    """The 16 levels as float32, ascending.

    "nf4": reading 1, index 7 is exactly 0.  "nf4_symmetric": reading 8.
    """
    if variant == "nf4_symmetric":
        return nf4_codebook_symmetric()
    if variant != "nf4":
        raise ValueError(f"unknown codebook {variant!r}")
    q = statistics.NormalDist(0.0, 1.0).inv_cdf
    delta = DELTA
    top = 1.0 - delta
    # equally spaced probabilities above 1/2, excluding 1/2 itself
    pos = [q(0.5 + (top - 0.5) * j / 8.0) for j in range(1, 9)]
    neg = [-q(0.5 + (top - 0.5) * j / 7.0) for j in range(1, 8)]
    levels = sorted(neg + [0.0] + pos)
    scale = q(top)
    return np.array([v / scale for v in levels], dtype=np.float64).astype(F32)


def nf4_codebook_symmetric() -> np.ndarray:
    """Reading 8: averages of neighbouring normal quantiles at j/16, ends at
    delta and 1 - delta, normalised to [-1, 1]; symmetric, no zero."""
    q = statistics.NormalDist(0.0, 1.0).inv_cdf
    p = [DELTA] + [j / 16.0 for j in range(1, 16)] + [1.0 - DELTA]
    Q = [q(v) for v in p]
    levels = [0.5 * (Q[i] + Q[i + 1]) for i in range(16)]
    top = levels[15]
    return np.array([v / top for v in levels], dtype=np.float64).astype(F32)


def e4m3_value(code: int) -> float:
    """Value of a non-negative E4M3 code 0..126 (0x7F is NaN and never used)."""
    if not 0 <= code <= 126:
        raise ValueError("code outside the non-negative finite E4M3 range")
    e, m = code >> 3, code & 7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest non-negative E4M3 code (ties to the even code), by search over
    all 127 finite non-negative values.  Inputs in [0, 448]."""
    vals = np.array([e4m3_value(c) for c in range(127)])
    y = np.asarray(y, dtype=np.float64).ravel()
    out = np.empty(y.size, dtype=np.uint8)
    for i, v in enumerate(y):
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        out[i] = best[0] if best.size == 1 else best[best % 2 == 0][0]
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    vals = np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)
    return vals[np.asarray(codes, dtype=np.int64)].astype(F32)


def nf4_thresholds(cb: np.ndarray | None = None) -> np.ndarray:
    """The 15 float32 decision points between neighbouring levels."""
    cb = nf4_codebook() if cb is None else cb
    return ((cb[:-1] + cb[1:]).astype(F32) * F32(0.5)).astype(F32)


def nearest_code(x: np.ndarray, thr: np.ndarray) -> np.ndarray:
    """code = number of thresholds strictly below x (ties go to the lower code)."""
    return np.searchsorted(thr, np.asarray(x, dtype=F32), side="left").astype(np.uint8)


def block_absmax(w: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """c1 per block of ``block`` consecutive elements (last block may be partial)."""
    w = np.asarray(w, dtype=F32).ravel()
    n = w.size
    nb = -(-n // block)
    c1 = np.zeros(nb, dtype=F32)
    full = n // block
    if full:
        c1[:full] = np.abs(w[: full * block].reshape(full, block)).max(axis=1)
    if nb > full:
        c1[full] = np.abs(w[full * block:]).max()
    return c1


def quantize_codes(w: np.ndarray, c1: np.ndarray, block: int = BLOCK,
                   codebook: str = "nf4") -> np.ndarray:
    """Per-element NF4 codes given each block's exact absmax."""
    w = np.asarray(w, dtype=F32).ravel()
    thr = nf4_thresholds(nf4_codebook(codebook))
    scale = np.repeat(c1, block)[: w.size]
    codes = np.full(w.size, 7, dtype=np.uint8)
    nz = scale != 0
    x = (w[nz] / scale[nz]).astype(F32)      # float32, correctly rounded
    codes[nz] = nearest_code(x, thr)
    return codes


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: element 2j low nibble, 2j+1 high nibble."""
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    if codes.size % 2:
        codes = np.concatenate([codes, np.zeros(1, np.uint8)])
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out[:n]


def double_quantize(c1: np.ndarray, group: int = DQ_BLOCK, fmt: str = "int8"):
    """Second level: c2 = max c1 per group, y = fl32(fl32(c1/c2)*127), and
    q8 = rint(y) ("int8", reading 5) or the E4M3 code nearest y ("fp8",
    reading 7)."""
    if fmt not in DQ_FORMATS:
        raise ValueError(f"unknown second-level format {fmt!r}")
    c1 = np.asarray(c1, dtype=F32)
    ng = -(-c1.size // group)
    c2 = np.zeros(ng, dtype=F32)
    for g in range(ng):
        c2[g] = c1[g * group:(g + 1) * group].max()
    c2e = np.repeat(c2, group)[: c1.size]
    q8 = np.zeros(c1.size, dtype=np.uint8)
    nz = c2e != 0
    ratio = (c1[nz] / c2e[nz]).astype(F32)
    y = (ratio * F32(127.0)).astype(F32)
    q8[nz] = np.rint(y).astype(np.uint8) if fmt == "int8" else e4m3_encode(y)
    return q8, c2


class NF4Tensor:
    """Quantised tensor: packed codes, first-level constants, optional DQ."""

    def __init__(self, n, packed, c1, q8=None, c2=None, dq_format="int8", codebook="nf4"):
        self.n = n
        self.packed = packed
        self.c1 = c1          # exact float32 absmax per block
        self.q8 = q8          # uint8 per block (double quantization)
        self.c2 = c2          # float32 per group of 256 blocks
        self.double_quant = q8 is not None
        self.dq_format = dq_format if self.double_quant else None
        self.codebook = codebook

    def nbytes(self) -> int:
        b = self.packed.size
        if self.double_quant:
            return b + self.q8.size + 4 * self.c2.size
        return b + 4 * self.c1.size


def nf4_quantize(w: np.ndarray, double_quant: bool = True, dq_format: str = "int8",
                 codebook: str = "nf4") -> NF4Tensor:
    """Quantise a float32 (or bf16-valued float32) tensor in flattened order."""
    w = np.asarray(w, dtype=F32).ravel()
    c1 = block_absmax(w)
    codes = quantize_codes(w, c1, codebook=codebook)
    packed = pack_codes(codes)
    if double_quant:
        q8, c2 = double_quantize(c1, fmt=dq_format)
        return NF4Tensor(w.size, packed, c1, q8, c2, dq_format, codebook)
    return NF4Tensor(w.size, packed, c1, codebook=codebook)


def block_scale(q: NF4Tensor) -> np.ndarray:
    """Reconstructed per-block scale a' (float32)."""
    if not q.double_quant:
        return q.c1.astype(F32)
    step = (q.c2 / F32(127.0)).astype(F32)                    # fl32(c2/127)
    step_e = np.repeat(step, DQ_BLOCK)[: q.q8.size]
    qv = q.q8.astype(F32) if q.dq_format == "int8" else e4m3_decode(q.q8)
    return (qv * step_e).astype(F32)                          # fl32(q * step)


def nf4_dequantize_f32(q: NF4Tensor) -> np.ndarray:
    """w' = fl32(cb[code] * a') for every element (flattened)."""
    cb = nf4_codebook(q.codebook)
    codes = unpack_codes(q.packed, q.n)
    a = np.repeat(block_scale(q), BLOCK)[: q.n]
    return (cb[codes] * a).astype(F32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs.

    Done on the integer pattern: keep the upper 16 bits and round on the lower
    16, the tie case (exactly 0x8000 below) going to the even upper half.
    """
    u = np.asarray(x, dtype=F32).view(np.uint32)
    upper = u >> np.uint32(16)
    lower = u & np.uint32(0xFFFF)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + up.astype(np.uint32)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32).astype(np.float64)


def nf4_dequantize_bf16(q: NF4Tensor) -> np.ndarray:
    """bf16 bit patterns of RNE(w'), the values fed to the bf16 matrix multiply."""
    return f32_to_bf16_bits(nf4_dequantize_f32(q))


def storage_bits_per_param(n: int, double_quant: bool = True) -> float:
    """Bits per parameter of the stored format, from its byte layout."""
    nb = -(-n // BLOCK)
    codes = -(-n // 2)
    if double_quant:
        return 8.0 * (codes + nb + 4 * (-(-nb // DQ_BLOCK))) / n
    return 8.0 * (codes + 4 * nb) / n


def quantize_loop(w) -> tuple[list, list, list, list]:
    """Scalar pure-Python version for tiny inputs (cross-check of the vector code).

    Returns (codes, c1, q8, c2) as Python lists; every float op is rounded to
    float32 through numpy scalars.
    """
    cb = nf4_codebook()
    thr = [F32(cb[i] + cb[i + 1]) * F32(0.5) for i in range(15)]
    w = [F32(v) for v in np.asarray(w, dtype=F32).ravel()]
    codes, c1s = [], []
    for b0 in range(0, len(w), BLOCK):
        blk = w[b0:b0 + BLOCK]
        c1 = max(abs(v) for v in blk)
        c1s.append(F32(c1))
        for v in blk:
            if c1 == 0:
                codes.append(7)
            else:
                x = F32(v / c1)
                codes.append(sum(1 for t in thr if x > t))
    q8s, c2s = [], []
    for g0 in range(0, len(c1s), DQ_BLOCK):
        grp = c1s[g0:g0 + DQ_BLOCK]
        c2 = max(grp)
        c2s.append(F32(c2))
        for c in grp:
            if c2 == 0:
                q8s.append(0)
            else:
                q8s.append(int(np.rint(F32(F32(c / c2) * F32(127.0)))))
    return codes, c1s, q8s, c2s

"""Pins for the oracle's NF4 codec (CPU only).

Each check ties the oracle to something other than itself: the pages' printed
figures, the defining property of the levels (equal-probability spacing,
checked with the forward normal CDF, not the inverse the oracle uses), an
independent inverse-CDF implementation, brute-force nearest-level search,
exact special cases, and torch's own bfloat16 rounding.
"""
import math
import os

import numpy as np
import pytest

from oracle import nf4

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.txt")


def golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, value = [p.strip() for p in line.split("|")[:2]]
            out[name] = float(value)
    return out


def phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def inv_phi_bisect(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# ---------------------------------------------------------------- codebook

def test_codebook_shape_and_fixed_points():
    cb = nf4.nf4_codebook()
    g = golden()
    assert cb.dtype == np.float32 and cb.size == int(g["nf4_levels"])
    assert np.all(np.diff(cb) > 0)
    assert cb[7].view(np.uint32) == 0          # exact +0.0
    assert cb[0] == F32(-1.0) and cb[15] == F32(1.0)   # normalised to [-1, 1]
    assert (cb < 0).sum() == 7 and (cb > 0).sum() == 8


def test_codebook_equal_probability_spacing_forward_cdf():
    """Levels are normal quantiles at equally spaced probabilities.

    Checked through the forward CDF (erfc) and an independent bisection
    inverse: Phi(level * z_top) must step uniformly from 1/2 to 1 - delta on
    each side.
    """
    cb = nf4.nf4_codebook().astype(np.float64)
    delta = 0.5 * (1 / 32 + 1 / 30)
    z_top = inv_phi_bisect(1 - delta)
    pos = cb[8:]
    neg = -cb[:7][::-1]
    for side, n in ((pos, 8), (neg, 7)):
        probs = np.array([phi(v * z_top) for v in side])
        want = 0.5 + (1 - delta - 0.5) * np.arange(1, n + 1) / n
        np.testing.assert_allclose(probs, want, rtol=0, atol=2e-7)


def test_codebook_matches_independent_inverse_cdf():
    """Same construction through scipy's ndtri gives the same float32 bits."""
    sp = pytest.importorskip("scipy.special")
    delta = 0.5 * (1 / 32 + 1 / 30)
    top = 1 - delta
    pos = [sp.ndtri(0.5 + (top - 0.5) * j / 8) for j in range(1, 9)]
    neg = [-sp.ndtri(0.5 + (top - 0.5) * j / 7) for j in range(1, 8)]
    vals = np.array(sorted(neg + [0.0] + pos)) / sp.ndtri(top)
    assert np.array_equal(vals.astype(F32).view(np.uint32), nf4.nf4_codebook().view(np.uint32))


def test_thresholds_are_float32_midpoints():
    cb = nf4.nf4_codebook()
    t = nf4.nf4_thresholds()
    assert t.size == 15 and np.all(t > cb[:-1]) and np.all(t < cb[1:])
    for i in range(15):
        assert t[i] == F32(F32(cb[i] + cb[i + 1]) * F32(0.5))


# ------------------------------------------------------- code assignment

def test_nearest_code_brute_force():
    """Threshold rule == argmin |x - level| (float64) away from exact midpoints."""
    rng = np.random.default_rng(0)
    cb = nf4.nf4_codebook().astype(np.float64)
    x = rng.uniform(-1, 1, 200000).astype(F32)
    code = nf4.nearest_code(x, nf4.nf4_thresholds())
    d = np.abs(x.astype(np.float64)[:, None] - cb[None, :])
    best = d.argmin(axis=1)
    srt = np.sort(d, axis=1)
    clear = (srt[:, 1] - srt[:, 0]) > 1e-6
    assert np.array_equal(code[clear], best[clear])


def test_tie_goes_to_lower_code():
    t = nf4.nf4_thresholds()
    thr = t
    for i in range(15):
        assert nf4.nearest_code(np.array([t[i]]), thr)[0] == i
        up = np.nextafter(t[i], F32(np.inf))
        assert nf4.nearest_code(np.array([up]), thr)[0] == i + 1


def test_exact_levels_and_absmax_codes():
    cb = nf4.nf4_codebook()
    # one block whose absmax is exactly 1, holding every level
    blk = np.concatenate([cb, cb[::-1], np.zeros(32, F32)]).astype(F32)
    q = nf4.nf4_quantize(blk)
    codes = nf4.unpack_codes(q.packed, 64)
    assert np.array_equal(codes[:16], np.arange(16))
    assert np.array_equal(codes[16:32], np.arange(16)[::-1])
    assert np.all(codes[32:] == 7)
    assert q.c1[0] == F32(1.0)
    # scaled by a power of two the division stays exact
    q2 = nf4.nf4_quantize(blk * F32(0.125))
    assert np.array_equal(q2.packed, q.packed) and q2.c1[0] == F32(0.125)
    # negative absmax element -> code 0, positive -> 15, -0.0 -> 7
    w = np.array([0.5, -2.0, -0.0, 2.0 - 2 ** -20] + [0.0] * 60, F32)
    c = nf4.unpack_codes(nf4.nf4_quantize(w).packed, 64)
    assert c[1] == 0 and c[2] == 7 and c[3] == 15


def test_all_zero_block_and_group():
    w = np.zeros(64 * 300, F32)
    w[64 * 260 + 3] = 0.75          # one non-zero block, in the second group
    q = nf4.nf4_quantize(w)
    codes = nf4.unpack_codes(q.packed, w.size)
    assert np.all(codes[: 64 * 256] == 7)
    assert np.all(q.c1[:256] == 0) and q.c2[0] == 0 and np.all(q.q8[:256] == 0)
    assert q.c2[1] == F32(0.75) and q.q8[260] == 127
    assert np.all(nf4.nf4_dequantize_f32(q)[: 64 * 256] == 0)


def test_packing_order():
    codes = np.arange(16, dtype=np.uint8)
    packed = nf4.pack_codes(codes)
    assert list(packed) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(nf4.unpack_codes(packed, 16), codes)
    odd = nf4.pack_codes(np.array([5, 6, 7], np.uint8))
    assert list(odd) == [0x65, 0x07]


# --------------------------------------------------- double quantization

def test_dq_formula_and_half_even():
    g = golden()
    c1 = np.array([1.0, 0.5, 0.25, 0.0], F32)
    q8, c2 = nf4.double_quantize(c1)
    assert c2[0] == F32(1.0)
    assert list(q8) == [int(g["dq_int_scale"]), 64, 32, 0]   # 63.5 -> 64, 31.75 -> 32
    # float32 ratios whose product with 127 is exactly k + 1/2 round to even
    for k in (0, 2, 4, 10, 62):
        c = F32((k + 0.5) / 127)
        hit = None
        for d in range(-64, 65):
            cand = c
            for _ in range(abs(d)):
                cand = np.nextafter(cand, F32(np.inf) if d > 0 else F32(-np.inf))
            if F32(F32(cand / F32(1.0)) * F32(127.0)) == F32(k + 0.5):
                hit = cand
                break
        assert hit is not None
        q8, _ = nf4.double_quantize(np.array([1.0, hit], F32))
        assert q8[1] == (k if k % 2 == 0 else k + 1)


def test_dq_groups_partial_tail():
    rng = np.random.default_rng(3)
    c1 = np.abs(rng.standard_normal(256 * 3 + 17)).astype(F32)
    q8, c2 = nf4.double_quantize(c1)
    assert c2.size == 4 and q8.size == c1.size
    for gi in range(4):
        grp = c1[gi * 256:(gi + 1) * 256]
        assert c2[gi] == grp.max()
        assert q8[gi * 256 + int(grp.argmax())] == 127
    assert q8.max() <= 127


def test_scalar_loop_matches_vector_code():
    rng = np.random.default_rng(11)
    for n in (64, 130, 64 * 256 + 64 * 3 + 5):
        w = (rng.standard_normal(n) * 0.02).astype(F32)
        if n > 1000:
            w[64:128] = 0
        codes, c1, q8, c2 = nf4.quantize_loop(w)
        q = nf4.nf4_quantize(w)
        assert np.array_equal(nf4.unpack_codes(q.packed, n), np.array(codes, np.uint8))
        assert np.array_equal(q.c1, np.array(c1, F32))
        assert np.array_equal(q.q8, np.array(q8, np.uint8))
        assert np.array_equal(q.c2, np.array(c2, F32))


# ------------------------------------------------------- dequantization

def test_dequant_error_bound():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(64 * 512) * 0.02).astype(F32)
    q = nf4.nf4_quantize(w)
    deq = nf4.nf4_dequantize_f32(q).astype(np.float64)
    cb = nf4.nf4_codebook().astype(np.float64)
    max_gap = np.diff(cb).max()
    a = np.repeat(nf4.block_scale(q).astype(np.float64), 64)
    c1 = np.repeat(q.c1.astype(np.float64), 64)
    bound = c1 * max_gap / 2 + np.abs(c1 - a) + 1e-6 * c1
    assert np.all(np.abs(w - deq) <= bound)
    # the 8-bit constant reconstructs c1 to within half a step of c2 / 127
    c2e = np.repeat(q.c2.astype(np.float64), 256)[: q.c1.size]
    assert np.all(np.abs(nf4.block_scale(q) - q.c1) <= c2e / 127 * 0.5 * (1 + 1e-5))


def test_requantize_idempotent():
    for seed in (1, 2, 3):
        rng = np.random.default_rng(seed)
        w = (rng.standard_normal(64 * 256 * 3) * 0.02).astype(F32)
        q = nf4.nf4_quantize(w)
        q2 = nf4.nf4_quantize(nf4.nf4_dequantize_f32(q))
        assert np.array_equal(q2.packed, q.packed)
        assert np.array_equal(q2.q8, q.q8)
        np.testing.assert_allclose(q2.c2, q.c2, rtol=1e-6)


def test_single_level_scale_is_absmax():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(64 * 8) * 0.02).astype(F32)
    q = nf4.nf4_quantize(w, double_quant=False)
    assert np.array_equal(nf4.block_scale(q), q.c1)
    deq = nf4.nf4_dequantize_f32(q)
    cb = nf4.nf4_codebook()
    codes = nf4.unpack_codes(q.packed, w.size)
    assert np.array_equal(deq, (cb[codes] * np.repeat(q.c1, 64)).astype(F32))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = rng.standard_normal(100000).astype(F32) * F32(0.03)
    # exact ties in both directions
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(F32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1.0, 65504.0], F32)])
    ours = nf4.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------- storage rate

def test_storage_rates_match_pages():
    g = golden()
    n = 4096 * 4096
    dq = nf4.storage_bits_per_param(n, True)
    single = nf4.storage_bits_per_param(n, False)
    assert single == g["nf4_bits_single_level"]
    assert dq == 4 + 8 / 64 + 32 / (64 * 256) == 4.126953125
    assert round(dq, 3) == g["nf4_bits_double_quant"]
    assert round(single - dq, 3) == g["nf4_dq_saving_bits"]
    assert round(dq - 4, 3) == g["nf4_dq_overhead_bits"]
    assert single - 4 == g["nf4_single_overhead_bits"]
    q = nf4.nf4_quantize(np.ones(64 * 256 * 4, F32))
    assert q.nbytes() * 8 / (64 * 256 * 4) == dq
    assert round(7e9 * dq / 8 / 1e9, 2) == g["qlora_7b_base_gb"]
    # 4096^2 weight: 8,388,608 code bytes + 262,144 q8 + 4,096 c2
    assert -(-n // 2) + n // 64 + 4 * (n // 64 // 256) == 8654848


# ------------------------------------------------ format variants (E4M3, symmetric)

def test_e4m3_values_fixed_by_the_format():
    # OCP E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9, max finite 448
    assert nf4.e4m3_value(0x00) == 0.0
    assert nf4.e4m3_value(0x01) == 2.0 ** -9
    assert nf4.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert nf4.e4m3_value(0x08) == 2.0 ** -6
    assert nf4.e4m3_value(0x38) == 1.0
    assert nf4.e4m3_value(0x7E) == 448.0
    vals = [nf4.e4m3_value(c) for c in range(127)]
    assert all(a < b for a, b in zip(vals, vals[1:]))          # codes are ordered
    with pytest.raises(ValueError):
        nf4.e4m3_value(0x7F)


def test_e4m3_matches_torch_float8():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    codes = torch.arange(127, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(nf4.e4m3_decode(np.arange(127)), tv)
    rng = np.random.default_rng(4)
    y = np.concatenate([rng.uniform(0, 127, 4000), rng.uniform(0, 0.05, 2000),
                        (tv[:-1].astype(np.float64) + tv[1:]) / 2]).astype(F32)   # ties
    y = y[y <= 127]
    ours = nf4.e4m3_encode(y)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_fp8_double_quant_scale_bound():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal(64 * 600) * 0.02).astype(F32)
    q = nf4.nf4_quantize(w, double_quant=True, dq_format="fp8")
    assert q.dq_format == "fp8" and q.q8.max() <= 126
    a = nf4.block_scale(q).astype(np.float64)
    c2 = np.repeat(q.c2, nf4.DQ_BLOCK)[: q.c1.size].astype(np.float64)
    # the group maximum is 127 before rounding -> 128 = code 0x70
    for g in range(q.c2.size):
        grp = q.c1[g * 256:(g + 1) * 256]
        assert q.q8[g * 256 + int(np.argmax(grp))] == 0x70
    # E4M3 keeps 3 mantissa bits: relative error at most 2^-4 in the normal
    # range (y >= 2^-6), absolute 2^-10 * c2/127 below it; plus float32 steps
    y = q.c1.astype(np.float64) / c2 * 127
    bound = np.where(y >= 2 ** -6, 2.0 ** -4 * q.c1, 2.0 ** -10 * c2 / 127) + 1e-6 * q.c1
    assert np.all(np.abs(a - q.c1) <= bound)
    # same bytes as the integer format
    assert q.nbytes() == nf4.nf4_quantize(w).nbytes()


def test_fp8_and_int8_agree_where_the_integer_is_representable():
    # integers 0..16 are exact in E4M3, so small ratios give the same code value
    c1 = np.array([127, 16, 9, 3, 0.5, 0], dtype=F32)
    qi, c2i = nf4.double_quantize(c1, fmt="int8")
    qf, c2f = nf4.double_quantize(c1, fmt="fp8")
    assert np.array_equal(c2i, c2f)
    dec = nf4.e4m3_decode(qf)
    assert list(dec[1:]) == [16.0, 9.0, 3.0, 0.5, 0.0]
    assert list(qi[1:]) == [16, 9, 3, 0, 0]     # 0.5 rounds half to even -> 0
    assert dec[0] == 128.0 and qi[0] == 127


def test_symmetric_codebook_properties():
    cb = nf4.nf4_codebook("nf4_symmetric")
    assert cb.dtype == F32 and cb.size == 16
    assert cb[0] == -1.0 and cb[15] == 1.0
    assert np.all(np.diff(cb) > 0) and not np.any(cb == 0)
    assert np.array_equal(cb[::-1], -cb)                       # exact mirror
    t = nf4.nf4_thresholds(cb)
    assert t[7] == 0.0


def test_symmetric_codebook_matches_independent_inverse_cdf():
    sp = pytest.importorskip("scipy.special")
    delta = 0.5 * (1 / 32 + 1 / 30)
    p = [delta] + [j / 16 for j in range(1, 16)] + [1 - delta]
    Q = [float(sp.ndtri(v)) for v in p]
    lv = np.array([(Q[i] + Q[i + 1]) / 2 for i in range(16)])
    want = (lv / lv[15]).astype(F32)
    got = nf4.nf4_codebook("nf4_symmetric")
    assert np.max(np.abs(got.view(np.int32) - want.view(np.int32))) <= 1   # float32 steps


def test_symmetric_codes_brute_force_nearest():
    rng = np.random.default_rng(8)
    w = rng.standard_normal(64 * 50).astype(F32)
    q = nf4.nf4_quantize(w, double_quant=False, codebook="nf4_symmetric")
    codes = nf4.unpack_codes(q.packed, q.n)
    cb = nf4.nf4_codebook("nf4_symmetric").astype(np.float64)
    x = (w / np.repeat(q.c1, 64)).astype(F32).astype(np.float64)
    d = np.abs(x[:, None] - cb[None, :])
    srt = np.sort(d, axis=1)
    clear = (srt[:, 1] - srt[:, 0]) > 1e-6
    assert np.array_equal(codes[clear], d.argmin(axis=1)[clear])
    # each block's absmax element lands on an end level
    blk = np.abs(w).reshape(-1, 64).argmax(axis=1) + 64 * np.arange(50)
    assert set(codes[blk].tolist()) <= {0, 15}
    deq = nf4.nf4_dequantize_f32(q)
    assert np.all(np.abs(deq - w) <= np.repeat(q.c1, 64) * 0.5 * np.diff(cb).max() + 1e-7)

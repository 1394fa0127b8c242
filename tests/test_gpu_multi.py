"""Segmented multi-adapter forward on one shared base against the oracle's
loop of single-adapter forwards; the adapter term Y - Y_base is checked on
its own so a wrong routing cannot hide under the shared base term."""
import numpy as np
import pytest
import torch

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import BF16_TOL, DEV, announce, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu


def adapter_term_check(Yg, Ybg, Yo, dYo, absterm, K):
    """The adapter term Y - Y_base on its own, element by element.

    Y and Y_base (B = 0) come from the same base accumulation, each rounded
    once to bf16, so Y - Y_base differs from the exact term dYo by at most half
    a bf16 ulp of each output, plus the bf16 rounding of the expand operand
    s T (2^-9 relative per rank term, so 2^-9 sum_j |s T_j B_nj|, taken twice
    for margin) and the float32 accumulation of T (K 2^-24 per unit of
    sum_k |X A|, times |B| and s: ``absterm[1]``).  ``absterm[0]`` is
    sum_j |s T_j B_nj|.  A wrong adapter misses by the whole term."""
    base_o = Yo - dYo
    bound = (0.5 * bf16_ulp(np.maximum(np.abs(Yo), np.abs(Yg)))
             + 0.5 * bf16_ulp(np.maximum(np.abs(base_o), np.abs(Ybg)))
             + 2.0 ** -8 * absterm[0] + K * 2.0 ** -24 * absterm[1])
    err = np.abs((Yg - Ybg) - dYo)
    worst = float((err / bound).max())
    assert worst <= 1.0, f"adapter term exceeds its rounding bound by {worst:.2f}x"
    assert rel_err(Yg - Ybg, dYo) <= 0.05


def adapter_terms(Xo, As, Bs, scales, rows_of):
    """Exact adapter term s_a (X A_a^T) B_a^T of every row and the two
    magnitude sums adapter_term_check needs, from each row's own adapter."""
    T, N = Xo.shape[0], Bs[0].shape[0]
    dY = np.zeros((T, N))
    a0 = np.zeros((T, N))
    a1 = np.zeros((T, N))
    for a, pick in rows_of.items():
        xa = Xo[pick]
        sa = scales[a]
        Ta = xa @ As[a].T
        dY[pick] = sa * (Ta @ Bs[a].T)
        a0[pick] = sa * (np.abs(Ta) @ np.abs(Bs[a]).T)
        a1[pick] = sa * ((np.abs(xa) @ np.abs(As[a]).T) @ np.abs(Bs[a]).T)
    return dY, (a0, a1)


def rows_by_adapter(offsets, ids):
    seg_of = np.repeat(np.arange(len(ids)), np.diff(offsets))
    row_ad = np.asarray(ids)[seg_of]
    return {int(a): np.nonzero(row_ad == a)[0] for a in np.unique(row_ad)}


def run_multi(X_t, W0_t, A_t, B_t, offsets, ids, s, label="", fused=False, nf4=False):
    announce(f"multi {label} T={X_t.shape[0]} n_seg={len(ids)} n_ad={A_t.shape[0]} r={A_t.shape[1]}")
    T = X_t.shape[0]
    assert lq.lq_check_segments(offsets, ids, T, A_t.shape[0]) == 0
    X, W0, A, B = to_dev(X_t), to_dev(W0_t), to_dev(A_t), to_dev(B_t)
    if nf4:  # shared NF4 base: the oracle multiplies by its own bf16 dequantisation
        W0 = lq.lq_nf4_quantize(W0)
        q = onf4.nf4_quantize(W0_t.value)
        W0_t = wl.Tensor(onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(q))
                         .reshape(W0_t.value.shape).astype(np.float32), "f32")
    off = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    ad = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    Y = lq.lq_lora_fwd_multi(X, W0, A, B, s, off, ad, fused=fused)
    Yb = lq.lq_lora_fwd_multi(X, W0, A, torch.zeros_like(B), s, off, ad, fused=fused)
    torch.cuda.synchronize()
    Xo, Wo, Ao, Bo = X_t.f64(), W0_t.f64(), A_t.f64(), B_t.f64()
    Yo = olora.lora_forward_multi(Xo, Wo, Ao, Bo, s, offsets, ids)
    Yg = f64(Y)
    e = rel_err(Yg, Yo)
    assert e <= BF16_TOL, f"Y rel err {e:.3e}"
    n_ad = Ao.shape[0]
    dYo, absterm = adapter_terms(Xo, list(Ao), list(Bo), [s] * n_ad, rows_by_adapter(offsets, ids))
    adapter_term_check(Yg, f64(Yb), Yo, dYo, absterm, Xo.shape[1])
    return Y


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def small_multi(counts, ids, n_ad, r, K=256, N=256, seed=3):
    rng = np.random.default_rng(seed)
    T = int(np.sum(counts))
    X = wl.Tensor(rng.standard_normal((T, K), dtype=np.float32), "bf16")
    W0 = wl.Tensor(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02), "bf16")
    A = wl.Tensor(rng.standard_normal((n_ad, r, K), dtype=np.float32) * np.float32(0.1), "bf16")
    B = wl.Tensor(rng.standard_normal((n_ad, N, r), dtype=np.float32) * np.float32(0.1), "bf16")
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return X, W0, A, B, off, np.asarray(ids, np.int32)


@pytest.mark.parametrize("n_ad,r", [(3, 5), (4, 16), (2, 8), (1, 64)])
def test_small_segments(n_ad, r):
    counts = [0, 1, 37, 129, 0, 300, 2, 64, 65]
    rng = np.random.default_rng(n_ad * 100 + r)
    ids = rng.integers(0, n_ad, len(counts))
    X, W0, A, B, off, ids = small_multi(counts, ids, n_ad, r)
    run_multi(X, W0, A, B, off, ids, 2.0, label="small")
    run_multi(X, W0, A, B, off, ids, 2.0, label="small-fused", fused=True)


def test_single_adapter_equals_single_forward():
    counts = [100, 200, 33]
    X, W0, A, B, off, ids = small_multi(counts, [1, 1, 1], 2, 16, seed=9)
    Y = run_multi(X, W0, A, B, off, ids, 2.0, label="one-adapter")
    Y1 = lq.lq_lora_fwd(to_dev(X), to_dev(W0), to_dev(A)[1].contiguous(), to_dev(B)[1].contiguous(), 2.0)
    torch.cuda.synchronize()
    assert rel_err(f64(Y), f64(Y1)) <= 1e-2


def test_config5_full():
    """4 adapters (r = 16, alpha = 32), 256 requests of 1..512 tokens, 4096^2 base."""
    c = wl.config5()
    run_multi(c["X"], c["W0"], c["A"], c["B"], c["offsets"], c["adapter"], c["alpha"] / c["r"],
              label="config5")


@pytest.mark.parametrize("n_ad,r", [(3, 8), (4, 5), (2, 32)])
def test_large_segments(n_ad, r):
    """T >= 2048 with N = 256: the large-tile path with several row tiles
    (masked T from the shrink kernel, expand over the stacked B), including an
    odd rank."""
    counts = [0, 700, 1, 513, 0, 900, 129, 64]
    T = sum(counts)
    assert (lq.lq_workspace_size(lq.LQ_OP_FWD_MULTI, T, 256, 256, r, n_ad)
            > lq.lq_workspace_size(lq.LQ_OP_FWD_MULTI_FUSED, T, 256, 256, r, n_ad))
    rng = np.random.default_rng(n_ad * 10 + r)
    ids = rng.integers(0, n_ad, len(counts))
    X, W0, A, B, off, ids = small_multi(counts, ids, n_ad, r, seed=r)
    run_multi(X, W0, A, B, off, ids, 2.0, label="large")
    run_multi(X, W0, A, B, off, ids, 2.0, label="large-fused", fused=True)


@pytest.mark.parametrize("counts", [[0, 37, 129, 300, 2], [0, 700, 1, 513, 0, 900, 129, 64]],
                         ids=["fused", "large"])
def test_nf4_shared_base(counts):
    """Segmented forward over one NF4 + DQ base: the prep kernel's bf16 copy
    and masked T with the default workspace, the fused kernel with the smallest."""
    rng = np.random.default_rng(len(counts))
    ids = rng.integers(0, 3, len(counts))
    X, W0, A, B, off, ids = small_multi(counts, ids, 3, 16, seed=7)
    run_multi(X, W0, A, B, off, ids, 2.0, label="nf4 base", nf4=True)
    run_multi(X, W0, A, B, off, ids, 2.0, label="nf4 base fused", nf4=True, fused=True)


def run_multi_ranks(counts, ids, ranks, scales, N=256, K=256, seed=13, nf4=False, fused=False,
                    label=""):
    """Adapters of different ranks and scales against the oracle's per-segment
    forward, plus the adapter term on its own (as in run_multi)."""
    rng = np.random.default_rng(seed)
    T = int(np.sum(counts))
    X = wl.Tensor(rng.standard_normal((T, K), dtype=np.float32), "bf16")
    W0 = wl.Tensor(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02), "bf16")
    As = [wl.Tensor(rng.standard_normal((r, K), dtype=np.float32) * np.float32(0.1), "bf16")
          for r in ranks]
    Bs = [wl.Tensor(rng.standard_normal((N, r), dtype=np.float32) * np.float32(0.1), "bf16")
          for r in ranks]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ids = np.asarray(ids, np.int32)
    roff = np.concatenate([[0], np.cumsum(ranks)]).astype(np.int32)
    announce(f"multi ranks {label} T={T} ranks={list(ranks)} nf4={nf4} fused={fused}")
    A_cat = torch.cat([to_dev(a) for a in As], 0).contiguous()
    B_cat = torch.cat([to_dev(b).reshape(-1) for b in Bs]).contiguous()
    Xd = to_dev(X)
    Wd = to_dev(W0)
    Wo = W0.f64()
    if nf4:
        Wd = lq.lq_nf4_quantize(Wd)
        q = onf4.nf4_quantize(W0.value)
        Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(q)).reshape(N, K)
    so = torch.from_numpy(off).to(DEV)
    sa = torch.from_numpy(ids).to(DEV)
    Y = lq.lq_lora_fwd_multi_ranks(Xd, Wd, A_cat, B_cat, roff, scales, so, sa, fused=fused)
    Yb = lq.lq_lora_fwd_multi_ranks(Xd, Wd, A_cat, torch.zeros_like(B_cat), roff, scales, so, sa,
                                     fused=fused)
    torch.cuda.synchronize()
    Ao_l, Bo_l = [a.f64() for a in As], [b.f64() for b in Bs]
    Yo = olora.lora_forward_multi(X.f64(), Wo, Ao_l, Bo_l, list(scales), off, ids)
    Yg = f64(Y)
    assert rel_err(Yg, Yo) <= BF16_TOL
    dYo, absterm = adapter_terms(X.f64(), Ao_l, Bo_l, list(scales), rows_by_adapter(off, ids))
    adapter_term_check(Yg, f64(Yb), Yo, dYo, absterm, K)


@pytest.mark.parametrize("nf4", [False, True], ids=["bf16", "nf4"])
@pytest.mark.parametrize("fused", [False, True], ids=["large", "fused"])
def test_mixed_ranks(fused, nf4):
    """Ranks 4, 16, 1, 8 (R = 29) with their own scales; T = 2307 takes the
    large-tile path unless the fused-size workspace is given."""
    counts = [0, 700, 1, 513, 0, 900, 129, 64]
    ids = [2, 0, 3, 1, 1, 2, 0, 3]
    run_multi_ranks(counts, ids, [4, 16, 1, 8], [8.0, 2.0, 32.0, 4.0], nf4=nf4, fused=fused,
                    label="mixed")


def test_mixed_ranks_equal_ranks_match_uniform_call():
    """Equal ranks through lq_lora_fwd_multi_ranks give exactly the result of
    lq_lora_fwd_multi (the same kernels and the same table)."""
    counts = [0, 700, 1, 513, 0, 900, 129, 64]
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 3, len(counts))
    X, W0, A, B, off, ids = small_multi(counts, ids, 3, 8)
    Xd, Wd, Ad, Bd = to_dev(X), to_dev(W0), to_dev(A), to_dev(B)
    so = torch.from_numpy(off).to(DEV)
    sa = torch.from_numpy(ids).to(DEV)
    Y1 = lq.lq_lora_fwd_multi(Xd, Wd, Ad, Bd, 2.0, so, sa)
    Y2 = lq.lq_lora_fwd_multi_ranks(Xd, Wd, Ad.reshape(24, 256).contiguous(),
                                    Bd.reshape(-1).contiguous(), [0, 8, 16, 24], [2.0] * 3, so, sa)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)

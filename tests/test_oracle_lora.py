"""Pins for the oracle's LoRA forward / backward / merge / multi-adapter (CPU only).

Gradients are checked by central finite differences (Y is linear in X, A and
B separately, so the difference quotient is exact up to rounding); the
forward by B = 0 and A = 0 reductions to a plain matrix product, the merge
identity, and a scalar-loop version; parameter and FLOP counts by the
figures the pages print.
"""
import os

import numpy as np

from oracle import lora

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


def tiny(seed=0, M=3, N=5, K=7, r=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K)), rng.standard_normal((N, K)),
            rng.standard_normal((r, K)), rng.standard_normal((N, r)),
            rng.standard_normal((M, N)))


def loss(X, W0, A, B, G, s):
    return float(np.sum(G * lora.lora_forward(X, W0, A, B, s)[0]))


def fd_grad(f, P, h=1e-3):
    g = np.zeros_like(P)
    for idx in np.ndindex(P.shape):
        Pp = P.copy(); Pp[idx] += h
        Pm = P.copy(); Pm[idx] -= h
        g[idx] = (f(Pp) - f(Pm)) / (2 * h)
    return g


def test_backward_matches_finite_differences():
    for seed, s in ((0, 2.0), (1, 0.37), (2, 1.0)):
        X, W0, A, B, G = tiny(seed)
        dX, dA, dB = lora.lora_backward(G, X, W0, A, B, s)
        np.testing.assert_allclose(dX, fd_grad(lambda P: loss(P, W0, A, B, G, s), X), atol=1e-9)
        np.testing.assert_allclose(dA, fd_grad(lambda P: loss(X, W0, P, B, G, s), A), atol=1e-9)
        np.testing.assert_allclose(dB, fd_grad(lambda P: loss(X, W0, A, P, G, s), B), atol=1e-9)


def test_backward_per_sample_column_form():
    """Row-batched gradients equal the per-sample column-vector formulas summed."""
    X, W0, A, B, G = tiny(4, M=4, N=6, K=5, r=3)
    s = 1.5
    dA = np.zeros_like(A)
    dB = np.zeros_like(B)
    dX = np.zeros_like(X)
    for m in range(X.shape[0]):
        x = X[m][:, None]
        g = G[m][None, :]                 # dL/dy as a 1 x d_out row
        dB += s * g.T @ (A @ x).T
        dA += s * B.T @ g.T @ x.T
        dX[m] = ((W0 + s * B @ A).T @ g.T)[:, 0]
    got = lora.lora_backward(G, X, W0, A, B, s)
    for a, b in zip(got, (dX, dA, dB)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_zero_b_is_base_model():
    X, W0, A, B, G = tiny(5, M=6, N=9, K=8, r=3)
    B = np.zeros_like(B)
    Y, Y_base, _ = lora.lora_forward(X, W0, A, B, 2.0)
    assert np.array_equal(Y, Y_base)
    assert np.array_equal(Y, X @ W0.T)
    dX, dA, dB = lora.lora_backward(G, X, W0, A, B, 2.0)
    assert np.array_equal(dA, np.zeros_like(A))          # only B learns at step 0
    assert np.array_equal(dX, G @ W0)
    assert np.any(dB != 0)


def test_zero_a_reduces_to_matmul():
    X, W0, A, B, _ = tiny(6)
    Y = lora.lora_forward(X, W0, np.zeros_like(A), B, 3.0)[0]
    assert np.array_equal(Y, np.matmul(X, W0.T))


def test_merge_identity():
    X, W0, A, B, _ = tiny(7, M=5, N=8, K=12, r=4)
    s = 2.0
    Wm = lora.lora_merge(W0, A, B, s)
    Y = lora.lora_forward(X, W0, A, B, s)[0]
    np.testing.assert_allclose(X @ Wm.T, Y, rtol=1e-12, atol=1e-12)
    assert Wm.shape == W0.shape


def test_scalar_loop_forward():
    X, W0, A, B, _ = tiny(8, M=3, N=4, K=6, r=2)
    Y = lora.lora_forward(X, W0, A, B, 0.75)[0]
    np.testing.assert_allclose(np.array(lora.forward_loop(X, W0, A, B, 0.75)), Y, rtol=1e-12)


def test_multi_is_loop_of_single():
    rng = np.random.default_rng(9)
    K, N, r, n_ad = 16, 12, 3, 3
    W0 = rng.standard_normal((N, K))
    As = rng.standard_normal((n_ad, r, K))
    Bs = rng.standard_normal((n_ad, N, r))
    counts = np.array([3, 0, 5, 1, 4])
    ids = np.array([2, 0, 1, 2, 0])
    off = np.concatenate([[0], np.cumsum(counts)])
    X = rng.standard_normal((off[-1], K))
    Y = lora.lora_forward_multi(X, W0, As, Bs, 2.0, off, ids)
    for i in range(len(ids)):
        lo, hi = off[i], off[i + 1]
        want = X[lo:hi] @ W0.T + 2.0 * (X[lo:hi] @ As[ids[i]].T) @ Bs[ids[i]].T
        np.testing.assert_allclose(Y[lo:hi], want, rtol=1e-12, atol=1e-12)
    # one adapter everywhere == the single-adapter forward on all rows
    Y1 = lora.lora_forward_multi(X, W0, As, Bs, 2.0, off, np.ones_like(ids))
    np.testing.assert_allclose(Y1, lora.lora_forward(X, W0, As[1], Bs[1], 2.0)[0], rtol=1e-12)


def test_multi_mixed_ranks_equals_zero_padded_uniform():
    """Adapters of different ranks, each with its own scale: padding every
    adapter to the largest rank with zero rows of A (and zero columns of B)
    and folding its scale into B gives the same output through the uniform
    path with scale 1 (zero rank directions add nothing)."""
    rng = np.random.default_rng(21)
    K, N = 10, 7
    ranks, scales = [1, 4, 2], [3.0, 0.5, 1.25]
    W0 = rng.standard_normal((N, K))
    As = [rng.standard_normal((r, K)) for r in ranks]
    Bs = [rng.standard_normal((N, r)) for r in ranks]
    counts = np.array([2, 3, 0, 4, 1])
    ids = np.array([1, 0, 2, 2, 1])
    off = np.concatenate([[0], np.cumsum(counts)])
    X = rng.standard_normal((off[-1], K))
    Y = lora.lora_forward_multi(X, W0, As, Bs, scales, off, ids)
    R = max(ranks)
    Ap = np.zeros((3, R, K))
    Bp = np.zeros((3, N, R))
    for a, r in enumerate(ranks):
        Ap[a, :r] = As[a]
        Bp[a, :, :r] = scales[a] * Bs[a]
    np.testing.assert_allclose(Y, lora.lora_forward_multi(X, W0, Ap, Bp, 1.0, off, ids),
                               rtol=1e-12, atol=1e-12)
    # equal ranks and one scale given per adapter reduce to the scalar form
    Yu = lora.lora_forward_multi(X, W0, Ap, Bp, [2.0] * 3, off, ids)
    np.testing.assert_allclose(Yu, lora.lora_forward_multi(X, W0, Ap, Bp, 2.0, off, ids),
                               rtol=0, atol=0)


def test_parameter_counts_match_pages():
    g = golden()
    d, ffn = 4096, 11008
    assert lora.lora_num_params(d, d, 8) == g["lora_params_4096sq_r8"]
    assert lora.lora_num_params(d, d, 16) == g["lora_params_4096sq_r16"]
    assert d * d // lora.lora_num_params(d, d, 16) == g["reduction_4096sq_r16"]
    assert d * d == g["full_params_4096sq"]
    base = lora.trainable_params(32, [(d, d), (d, d)], 8)
    exp = lora.trainable_params(32, [(d, d)] * 3 + [(d, ffn)], 16)
    assert base == g["calc_baseline"] == g["lora_params_qv_r8_32layers"]
    assert exp == g["calc_expanded"]
    assert exp / base == g["calc_ratio"]
    assert lora.lora_num_params(d, ffn, 16) == g["calc_down_per_layer_r16"]
    assert lora.trainable_params(32, [(d, d)], 8) == g["lora_params_v_r8_32layers"]


def test_merge_flops_match_pages():
    g = golden()
    d, ffn = 4096, 11008
    assert lora.merge_flops(d, d, 8) == g["merge_flops_4096sq_r8"]
    assert round(32 * 2 * lora.merge_flops(d, d, 8) / 1e9, 2) == g["merge_gflops_qv_r8_32"]
    tot = 32 * (3 * lora.merge_flops(d, d, 16) + lora.merge_flops(d, ffn, 16))
    assert round(tot / 1e9, 2) == g["merge_gflops_qvo_down_r16"]


# ------------------------------------------------------------ LoRA-input dropout

def test_dropout_mask_bit_order():
    # byte 0b00000101 keeps elements 0 and 2; the second byte's bit 7 is element 15
    keep = lora.unpack_keep(np.array([0b00000101, 0b10000000], np.uint8), 2, 8)
    assert keep[0].tolist() == [True, False, True, False, False, False, False, False]
    assert keep[1].tolist() == [False] * 7 + [True]
    rng = np.random.default_rng(1)
    k = rng.random((3, 16)) < 0.7
    assert np.array_equal(lora.unpack_keep(np.packbits(k.ravel(), bitorder="little"), 3, 16), k)


def test_dropout_all_kept_p0_is_plain_lora():
    X, W0, A, B, G = tiny(4)
    keep = np.ones(X.shape, bool)
    Y, T = lora.lora_forward_dropout(X, W0, A, B, 1.5, keep, 0.0)
    Y0, _, T0 = lora.lora_forward(X, W0, A, B, 1.5)
    assert np.array_equal(Y, Y0) and np.array_equal(T, T0)
    for a, b in zip(lora.lora_backward_dropout(G, X, W0, A, B, 1.5, keep, 0.0),
                    lora.lora_backward(G, X, W0, A, B, 1.5)):
        assert np.array_equal(a, b)


def test_dropout_all_dropped_is_base_and_no_adapter_grads():
    X, W0, A, B, G = tiny(5)
    keep = np.zeros(X.shape, bool)
    Y, T = lora.lora_forward_dropout(X, W0, A, B, 2.0, keep, 0.3)
    assert not T.any()
    assert np.array_equal(Y, X @ W0.T)
    dX, dA, dB = lora.lora_backward_dropout(G, X, W0, A, B, 2.0, keep, 0.3)
    assert np.array_equal(dX, G @ W0) and not dA.any() and not dB.any()


def test_dropout_expectation_over_all_masks_is_plain_lora():
    # brute force over every mask of one row of K = 6: the keep-probability
    # weighted mean of the adapter term is exactly the undropped one
    rng = np.random.default_rng(2)
    K, N, r, p, s = 6, 4, 2, 0.3, 2.0
    X = rng.standard_normal((1, K))
    W0 = rng.standard_normal((N, K))
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    mean = np.zeros((1, N))
    for bits in range(2 ** K):
        keep = np.array([[(bits >> k) & 1 for k in range(K)]], bool)
        w = (1 - p) ** keep.sum() * p ** (K - keep.sum())
        mean += w * lora.lora_forward_dropout(X, W0, A, B, s, keep, p)[0]
    want = lora.lora_forward(X, W0, A, B, s)[0]
    np.testing.assert_allclose(mean, want, rtol=1e-12, atol=1e-12)


def test_dropout_gradients_match_finite_differences():
    X, W0, A, B, G = tiny(6, M=3, N=4, K=5, r=2)
    rng = np.random.default_rng(7)
    keep = rng.random(X.shape) < 0.6
    p, s = 0.4, 1.25

    def f(X_, A_, B_):
        return float(np.sum(G * lora.lora_forward_dropout(X_, W0, A_, B_, s, keep, p)[0]))
    dX, dA, dB = lora.lora_backward_dropout(G, X, W0, A, B, s, keep, p)
    np.testing.assert_allclose(dX, fd_grad(lambda P: f(P, A, B), X), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dA, fd_grad(lambda P: f(X, P, B), A), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dB, fd_grad(lambda P: f(X, A, P), B), rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------------ DoRA

def test_dora_magnitude_at_row_norms_is_plain_lora():
    # with m equal to the row norms of W0 + s B A the direction is rescaled
    # back to itself: Y is the plain LoRA output
    X, W0, A, B, G = tiny(8)
    s = 1.7
    W = W0 + s * (B @ A)
    m = np.sqrt((W * W).sum(axis=1))
    Y, Z, c = lora.dora_forward(X, W0, A, B, s, m)
    np.testing.assert_allclose(Y, lora.lora_forward(X, W0, A, B, s)[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c, m, rtol=1e-15)


def test_dora_output_depends_only_on_direction():
    # scaling W0 and B together scales every row of W0 + s B A: Y is unchanged
    X, W0, A, B, G = tiny(9)
    m = np.random.default_rng(9).uniform(0.5, 2.0, W0.shape[0])
    Y1 = lora.dora_forward(X, W0, A, B, 0.8, m)[0]
    Y2 = lora.dora_forward(X, 3.5 * W0, A, 3.5 * B, 0.8, m)[0]
    np.testing.assert_allclose(Y1, Y2, rtol=1e-12, atol=1e-12)
    # and row n of Y scales with m_n alone
    m2 = m.copy()
    m2[2] *= 4.0
    Y3 = lora.dora_forward(X, W0, A, B, 0.8, m2)[0]
    np.testing.assert_allclose(Y3[:, 2], 4.0 * Y1[:, 2], rtol=1e-12)
    np.testing.assert_allclose(np.delete(Y3, 2, axis=1), np.delete(Y1, 2, axis=1), rtol=1e-15)


def test_dora_gradients_match_finite_differences():
    X, W0, A, B, G = tiny(10, M=3, N=4, K=5, r=2)
    s = 1.3
    m = np.random.default_rng(10).uniform(0.5, 2.0, 4)

    def f(X_, A_, B_, m_):
        return float(np.sum(G * lora.dora_forward(X_, W0, A_, B_, s, m_)[0]))
    dX, dA, dB, dm = lora.dora_backward(G, X, W0, A, B, s, m)
    np.testing.assert_allclose(dX, fd_grad(lambda P: f(P, A, B, m), X), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dA, fd_grad(lambda P: f(X, P, B, m), A), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dB, fd_grad(lambda P: f(X, A, P, m), B), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dm, fd_grad(lambda P: f(X, A, B, P), m), rtol=1e-6, atol=1e-8)

"""Parity at the size limits the boundary accepts.

* K = 65536 and N = 65536, the largest reduction and output widths (the
  kernels address weights and activations with 32-bit offsets), on the decode
  path (M = 16) and past it (M = 300): whole tensors against the oracle.
* M K just below 2^31 elements, the largest activation tensor: X of 262143 x
  8192 (4.3 GB in bf16) drawn on the device; the oracle checks sampled rows of
  Y, T and dX, and the whole of dA and dB as the sum of its backward over row
  chunks streamed to the host."""
import numpy as np
import pytest
import torch

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import BF16_TOL, DEV, announce, f64, rel_err, to_dev
from .test_gpu_lora_bf16 import check_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("M,N,K", [(16, 256, 65536), (300, 256, 65536), (16, 65536, 256),
                                   (300, 65536, 256)],
                         ids=["decode-k64k", "k64k", "decode-n64k", "n64k"])
def test_widest(M, N, K, kind):
    c = wl.small_case(M, N, K, 16, seed=M + N // 256 + K // 256)
    check_layer(c, kind, bwd=M > 16, merge=False, label="limits")


def bf16_rows(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


@pytest.mark.parametrize("kind", ["dense", "nf4"])
def test_largest_activation(kind):
    M, N, K, r = 262143, 64, 8192, 16
    assert M * K < 2 ** 31 <= (M + 1) * K
    announce(f"limits largest activation {kind} M={M} K={K}")
    c = wl.small_case(4, N, K, r, seed=91)          # W0, A, B from the host generator
    X = wl.device_normal((M, K), 1.0, seed=92, device=DEV)
    dY = wl.device_normal((M, N), 1.0, seed=93, device=DEV)
    s = c["alpha"] / r
    A, B = to_dev(c["A"]), to_dev(c["B"])
    W0v = c["W0"].value
    if kind == "nf4":
        Wd = lq.lq_nf4_quantize(to_dev(c["W0"]))
        Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(onf4.nf4_quantize(W0v))).reshape(N, K)
    else:
        Wd, Wo = to_dev(c["W0"]), W0v.astype(np.float64)
    Ao, Bo = c["A"].f64(), c["B"].f64()
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    Y = lq.lq_lora_fwd(X, Wd, A, B, s, T_out=T)
    dX, dA, dB = lq.lq_lora_bwd(dY, X, Wd, A, B, s, T_saved=T)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4097, M // 2, M - 17, M - 2, M - 1])
    ri = torch.as_tensor(rows, device=DEV)
    Xs, dYs = bf16_rows(X[ri]), bf16_rows(dY[ri])
    Yo, _, To = olora.lora_forward(Xs, Wo, Ao, Bo, s)
    dXo = olora.lora_backward(dYs, Xs, Wo, Ao, Bo, s)[0]
    for name, got, want in (("Y", Y[ri], Yo), ("T", T[ri], To), ("dX", dX[ri], dXo)):
        e = rel_err(f64(got), want)
        assert e <= BF16_TOL, f"{name} sampled rows rel err {e:.3e}"
    # dA and dB sum over all rows: the oracle's backward on row chunks (X and dY
    # streamed to the host), its dA and dB added over the chunks; dA compared on
    # every column, dB whole
    dAo = np.zeros((r, K))
    dBo = np.zeros((N, r))
    for m0 in range(0, M, 16384):
        sl = slice(m0, min(m0 + 16384, M))
        _, dA_c, dB_c = olora.lora_backward(bf16_rows(dY[sl]), bf16_rows(X[sl]), Wo, Ao, Bo, s)
        dAo += dA_c
        dBo += dB_c
    for name, got, want in (("dA", dA, dAo), ("dB", dB, dBo)):
        e = rel_err(f64(got), want)
        assert e <= BF16_TOL, f"{name} rel err {e:.3e}"

"""LoRA-input dropout on the GPU (lq_lora_fwd_dropout / lq_lora_bwd_dropout)
against the oracle: the fused path, the large-tile path and decode-sized M, a
dense or NF4 base, p from the pages' configuration (0.05) and a heavy 0.5,
all outputs within the bf16 bar (2e-2 relative to max |oracle|).  Special
masks: every element dropped gives the base output and exactly zero adapter
gradients; every element kept with p = 0 gives the plain layer."""
import numpy as np
import pytest
import torch

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import BF16_TOL, DEV, announce, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu


def base_for(c, kind):
    W0v = c["W0"].value
    if kind == "nf4":
        Wd = lq.lq_nf4_quantize(to_dev(c["W0"]))
        q = onf4.nf4_quantize(W0v)
        return Wd, onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(q)).reshape(W0v.shape)
    return to_dev(c["W0"]), W0v.astype(np.float64)


def keep_of(bits, M, K):
    # the layout the oracle's unpack_keep defines (its pins check it against
    # numpy's little-endian bit order)
    return np.unpackbits(bits, bitorder="little")[: M * K].reshape(M, K).astype(bool)


def run(c, kind, p, bits, fused, label, rows=None):
    M, K = c["X"].value.shape
    N, r = c["W0"].value.shape[0], c["r"]
    s = c["alpha"] / r
    announce(f"dropout {label} {kind} M={M} N={N} K={K} r={r} p={p} fused={fused}")
    X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
    Wd, Wo = base_for(c, kind)
    keep_d = torch.from_numpy(bits).to(DEV)
    keep = keep_of(bits, M, K)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    Y = lq.lq_lora_fwd_dropout(X, Wd, A, B, s, keep_d, p, T_out=T, fused=fused)
    dX, dA, dB = lq.lq_lora_bwd_dropout(dY, X, Wd, A, B, s, keep_d, p, T_saved=T, fused=fused)
    dX2, dA2, dB2 = lq.lq_lora_bwd_dropout(dY, X, Wd, A, B, s, keep_d, p, fused=fused)  # T again
    torch.cuda.synchronize()
    Xo, Ao, Bo, dYo = c["X"].f64(), c["A"].f64(), c["B"].f64(), c["dY"].f64()
    sel = np.arange(M) if rows is None else rows
    Yo, To = olora.lora_forward_dropout(Xo[sel], Wo, Ao, Bo, s, keep[sel], p)
    dXo, dAo, dBo = olora.lora_backward_dropout(dYo, Xo, Wo, Ao, Bo, s, keep, p)
    for name, got, want in (("Y", f64(Y)[sel], Yo), ("T", f64(T)[sel], To),
                            ("dX", f64(dX)[sel], dXo[sel]), ("dA", f64(dA), dAo),
                            ("dB", f64(dB), dBo), ("dX (T recomputed)", f64(dX2)[sel], dXo[sel]),
                            ("dA (T recomputed)", f64(dA2), dAo),
                            ("dB (T recomputed)", f64(dB2), dBo)):
        e = rel_err(got, want)
        assert e <= BF16_TOL, f"{name} rel err {e:.3e}"
    return dict(X=X, A=A, B=B, dY=dY, Wd=Wd, keep=keep_d, s=s, Y=Y, dX=dX, dA=dA, dB=dB)


SHAPES = [
    (300, 384, 512, 16, True),     # fused, ragged M
    (130, 192, 192, 5, True),      # odd rank, partial tiles
    (700, 256, 320, 64, True),     # rank 64
    (16, 256, 512, 8, True),       # decode-sized M
    (3, 128, 256, 4, True),
    (2100, 256, 256, 16, False),   # large-tile forward and dX
    (2304, 512, 768, 64, False),
]


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}r{r}{'' if f else '-large'}"
                                               for m, n, k, r, f in SHAPES])
@pytest.mark.parametrize("p", [0.05, 0.5])
def test_dropout_layer(shape, kind, p):
    M, N, K, r, fused = shape
    c = wl.small_case(M, N, K, r, seed=M + N + K + r + 11)
    bits = wl.dropout_keep_bits(M, K, p, seed=M + K)
    # the default workspace (the large-tile path where the shapes allow it) and
    # the fused kernels with the smaller workspace, same inputs
    run(c, kind, p, bits, False, "small")
    run(c, kind, p, bits, True, "small-fused")


def test_all_dropped_is_base_output_and_zero_adapter_grads():
    M, N, K, r = 300, 256, 256, 16
    c = wl.small_case(M, N, K, r, seed=3)
    bits = np.zeros((M * K + 7) // 8, np.uint8)
    o = run(c, "dense", 0.3, bits, True, "all-dropped")
    assert not o["dA"].any() and not o["dB"].any()
    assert rel_err(f64(o["Y"]), c["X"].f64() @ c["W0"].value.astype(np.float64).T) <= BF16_TOL


def test_all_kept_p0_matches_plain_layer():
    M, N, K, r = 300, 384, 512, 16
    c = wl.small_case(M, N, K, r, seed=4)
    bits = np.full((M * K + 7) // 8, 0xFF, np.uint8)
    o = run(c, "nf4", 0.0, bits, True, "all-kept")
    Y = lq.lq_lora_fwd(o["X"], o["Wd"], o["A"], o["B"], o["s"])
    dX, dA, dB = lq.lq_lora_bwd(o["dY"], o["X"], o["Wd"], o["A"], o["B"], o["s"])
    torch.cuda.synchronize()
    for name, a, b in (("Y", o["Y"], Y), ("dX", o["dX"], dX), ("dA", o["dA"], dA),
                       ("dB", o["dB"], dB)):
        e = rel_err(f64(a), f64(b))
        assert e <= BF16_TOL, f"{name}: dropout path vs plain path rel diff {e:.3e}"


def test_config3_full_size_p005():
    # the benchmark workload with the pages' lora_dropout = 0.05, both paths,
    # every output in full
    c = wl.config3()
    M, K = c["X"].value.shape
    bits = wl.dropout_keep_bits(M, K, 0.05, seed=99)
    run(c, "nf4", 0.05, bits, False, "config3")
    run(c, "nf4", 0.05, bits, True, "config3-fused")

"""The one-launch decode over several layers that read the same activations
(lq_lora_fwd_decode_layers): each layer's Y and T against the oracle, and
against the single-layer decode call on the same inputs (which differs only in
how T's partial sums are split, so Y may differ in the last bit of a few
elements); layer lists with different output widths (the key / value widths of
grouped-query attention, the MLP's gate and up), ranks 16 and 64, the
single-level constant format and a dense bf16 weight, the largest layer count,
and a captured graph of grouped and single-layer calls on one stream (which
share the stream's call tags) replayed between eager calls."""
import numpy as np
import pytest
import torch

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import BF16_TOL, DEV, F32_TOL, announce, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu


def make_layers(Ns, K, r, seed, fmt="nf4"):
    """Layer g: weight N_g x K (sigma 0.02), A ~ N(0, 1/r), B ~ N(0, 0.01^2),
    alpha = 2 r; returns device tensors and the oracle's dequantised weight."""
    out = []
    for g, N in enumerate(Ns):
        c = wl.small_case(1, N, K, r, seed=seed + 7 * g)
        if fmt == "dense":
            Wd = to_dev(c["W0"])
            W = Wd
            Wo = c["W0"].f64()
        else:
            dq = fmt == "nf4"
            W = lq.lq_nf4_quantize(to_dev(c["W0"]), double_quant=dq)
            q = onf4.nf4_quantize(c["W0"].value, double_quant=dq)
            Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(q)).reshape(N, K)
        out.append({"c": c, "W": W, "Wo": Wo, "A": to_dev(c["A"]), "B": to_dev(c["B"]),
                    "s": c["alpha"] / c["r"]})
    return out


def x_rows(M, K, seed):
    rng = np.random.default_rng(seed)
    return wl.Tensor(rng.standard_normal((M, K), dtype=np.float32), "bf16")


def run_group(layers, X, M, r):
    Ts = [torch.empty((M, r), dtype=torch.float32, device=DEV) for _ in layers]
    Ys = lq.lq_lora_fwd_decode_layers(X, [L["W"] for L in layers], [L["A"] for L in layers],
                                      [L["B"] for L in layers], [L["s"] for L in layers],
                                      T_outs=Ts)
    return Ys, Ts


def check(layers, Xh, Ys, Ts, single=True):
    Xd = to_dev(Xh)
    for g, (L, Y, T) in enumerate(zip(layers, Ys, Ts)):
        c = L["c"]
        Yo, _, To = olora.lora_forward(Xh.f64(), L["Wo"], c["A"].f64(), c["B"].f64(), L["s"])
        ey, et = rel_err(f64(Y), Yo), rel_err(f64(T), To)
        assert ey <= BF16_TOL, f"layer {g}: Y rel err {ey:.3e}"
        assert et <= F32_TOL, f"layer {g}: T rel err {et:.3e}"
        if not single:
            continue
        # the single-layer call: same kernel body, T split differently
        T1 = torch.empty_like(T)
        Y1 = lq.lq_lora_fwd(Xd, L["W"], L["A"], L["B"], L["s"], T_out=T1)
        torch.cuda.synchronize()
        assert rel_err(f64(T), f64(T1)) <= 1e-6, f"layer {g}: T differs from the single call"
        # Y = bf16(base + s T B^T) with the same base: the two differ by at
        # most what T's difference moves through s |B|, plus each side's
        # rounding (half an ulp, at most 2^-9 |y|)
        a, b = f64(Y), f64(Y1)
        d = np.abs(a - b)
        moved = L["s"] * (np.abs(f64(T) - f64(T1)) @ np.abs(c["B"].f64()).T)
        bound = 1.01 * moved + 2.0 ** -8 * (np.abs(a) + np.abs(b)) + 1e-12
        assert np.all(d <= bound), f"layer {g}: Y differs beyond T's difference"
        assert np.count_nonzero(d) <= max(8, a.size // 100), f"layer {g}: {np.count_nonzero(d)} differ"


@pytest.mark.parametrize("M", [1, 4, 16])
def test_qkv_shapes(M):
    """Three 4096 x 4096 NF4 layers (query, key, value of a Llama-2-7B block)."""
    K, r = 4096, 16
    layers = make_layers([4096, 4096, 4096], K, r, seed=101)
    Xh = x_rows(M, K, seed=5 + M)
    announce(f"decode layers qkv M={M}")
    Ys, Ts = run_group(layers, to_dev(Xh), M, r)
    torch.cuda.synchronize()
    check(layers, Xh, Ys, Ts)


@pytest.mark.parametrize("Ns,M,r,K", [((4096, 1024, 1024), 4, 64, 4096),
                                      ((11008, 11008), 16, 16, 4096),
                                      ((256,) * 8, 3, 8, 4096),
                                      ((1024, 512), 16, 64, 4096),
                                      ((1024, 4096), 2, 16, 11008)],
                         ids=["gqa-r64", "gate-up", "eight-layers", "m16-r64", "down-k11008"])
def test_mixed_widths(Ns, M, r, K):
    """m16-r64: M r = 1024 elements of T and 16 r = 1024 of B, two per thread;
    down-k11008: no activation staging, several rounds of loads per block."""
    layers = make_layers(list(Ns), K, r, seed=211)
    Xh = x_rows(M, K, seed=17)
    announce(f"decode layers {Ns} M={M} r={r}")
    Ys, Ts = run_group(layers, to_dev(Xh), M, r)
    torch.cuda.synchronize()
    check(layers, Xh, Ys, Ts)


@pytest.mark.parametrize("fmt", ["single", "dense"])
def test_formats(fmt):
    K, r, M = 2048, 16, 2
    layers = make_layers([1024, 512], K, r, seed=307, fmt=fmt)
    Xh = x_rows(M, K, seed=23)
    announce(f"decode layers format {fmt}")
    Ys, Ts = run_group(layers, to_dev(Xh), M, r)
    torch.cuda.synchronize()
    check(layers, Xh, Ys, Ts)


def test_graph_with_single_layer_calls():
    """Grouped and single-layer decode calls share the stream's slot: a graph
    of both, replayed with eager calls between, gives the eager bits."""
    K, r = 4096, 16
    layers = make_layers([4096, 1024], K, r, seed=401)
    Xs = [to_dev(x_rows(m, K, seed=40 + m)) for m in (1, 16)]
    Yg = [[torch.empty((x.shape[0], L["W"].N), dtype=torch.bfloat16, device=DEV)
           for L in layers] for x in Xs]
    Y1 = [torch.empty((x.shape[0], 4096), dtype=torch.bfloat16, device=DEV) for x in Xs]

    def run():
        for x, yg, y1 in zip(Xs, Yg, Y1):
            lq.lq_lora_fwd_decode_layers(x, [L["W"] for L in layers], [L["A"] for L in layers],
                                         [L["B"] for L in layers], [L["s"] for L in layers],
                                         Ys=yg)
            lq.lq_lora_fwd(x, layers[0]["W"], layers[0]["A"], layers[0]["B"], layers[0]["s"],
                           Y=y1)

    announce("decode layers graph replay")
    run()
    torch.cuda.synchronize()
    outs = [t for yg in Yg for t in yg] + Y1
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"replay {i}: output {k} differs from the eager call"
        run()
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("v", [(True, "int8", "nf4"), (False, "int8", "nf4"), (True, "fp8", "nf4"),
                               (True, "int8", "nf4_symmetric")],
                         ids=["default", "single", "fp8", "sym"])
@pytest.mark.parametrize("M,K", [(4, 4096), (16, 4096), (3, 8192)], ids=["m4", "m16", "k8192"])
def test_grouped_dequant_is_exact(v, M, K):
    """With B = 0 and one-hot activation rows, Y[g] = onehot(k) W'_g^T is
    column k of layer g's dequantised weight (bf16) bit for bit: the grouped
    kernel's register level tables give the codec's values."""
    from .test_gpu_formats import one_hot_rows, quant_both
    from .gpu_helpers import bits
    r, Ns = 16, (512, 256, 768)
    rng = np.random.default_rng(M + K + len(v[1]))
    qs, Wps = [], []
    for N in Ns:
        W = wl.Tensor((rng.standard_normal((N, K)) * 0.02).astype(np.float32), "bf16")
        q, o = quant_both(W.value, to_dev(W), v)
        qs.append(q)
        Wps.append(onf4.nf4_dequantize_bf16(o).reshape(N, K))
    A = torch.zeros((r, K), dtype=torch.bfloat16, device=DEV)
    Bs = [torch.zeros((N, r), dtype=torch.bfloat16, device=DEV) for N in Ns]
    ks = rng.integers(0, K, M)
    announce(f"decode layers exact dequant M={M} K={K} {v}")
    Ys = lq.lq_lora_fwd_decode_layers(one_hot_rows(M, K, ks), qs, [A] * 3, Bs, [2.0] * 3)
    torch.cuda.synchronize()
    for g, (Y, Wp) in enumerate(zip(Ys, Wps)):
        assert np.array_equal(bits(Y), Wp[:, ks].T), f"layer {g}: dequant differs"


@pytest.mark.parametrize("Ns,K", [((65536, 256), 256), ((256, 128), 65536)],
                         ids=["n64k", "k64k"])
def test_limits(Ns, K):
    """The widest output and reduction the boundary accepts: N = 65536 (about
    16 blocks per workgroup, a layer switch inside one range) and K = 65536
    (16 rounds of loads per block, activations read from global memory);
    whole tensors against the oracle."""
    M, r = 16, 16
    layers = make_layers(list(Ns), K, r, seed=601)
    Xh = x_rows(M, K, seed=67)
    announce(f"decode layers limits {Ns} K={K}")
    Ys, Ts = run_group(layers, to_dev(Xh), M, r)
    torch.cuda.synchronize()
    check(layers, Xh, Ys, Ts)

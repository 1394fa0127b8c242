"""bf16 path (MFMA kernels) against the float64 oracle, 2e-2 relative max error.

Every comparison covers the whole output tensor (Y, T, dX, dA, dB and the
merged weight), with the reference from the oracle's own forward, backward
and merge.  Small cases span several tiles with ragged edges (M not a
multiple of the 128/256-row tiles, N with a partial 128-column tile and a
partial 64-row reduction step, odd ranks).  The workload sizes (configs 2, 3
and 4) run through both the default workspace and the smaller fused-kernel
workspace, with the dense and the NF4 base where the workload names both."""
import functools

import numpy as np
import pytest
import torch

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import BF16_TOL, announce, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu


def base_for(c, kind):
    """(device W0 argument, oracle float64 W0 the GEMM multiplies by)."""
    W0v = c["W0"].value
    if kind == "nf4":
        Wd = lq.lq_nf4_quantize(to_dev(c["W0"]))
        q = onf4.nf4_quantize(W0v)
        Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(q)).reshape(W0v.shape)
        return Wd, Wo
    return to_dev(c["W0"]), W0v.astype(np.float64)


def oracle_ref(c, Wo, bwd=True):
    """The oracle's forward (Y, T) and backward (dX, dA, dB) on the whole batch."""
    s = c["alpha"] / c["r"]
    Xo, Ao, Bo = c["X"].f64(), c["A"].f64(), c["B"].f64()
    Yo, _, To = olora.lora_forward(Xo, Wo, Ao, Bo, s)
    ref = dict(Y=Yo, T=To)
    if bwd:
        ref["dX"], ref["dA"], ref["dB"] = olora.lora_backward(c["dY"].f64(), Xo, Wo, Ao, Bo, s)
    return ref


def check_gpu(c, Wd, ref, label="", fused=False, no_ws=False):
    """The GPU layer on the same inputs against ``ref`` over whole tensors.
    ``fused``: the LQ_OP_*_FUSED workspaces (for an NF4 forward at large M,
    the product that dequantises in its K loop); ``no_ws``: a forward with no
    workspace (the fused forward kernel)."""
    s = c["alpha"] / c["r"]
    X, A, B = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"])
    M, r = X.shape[0], A.shape[0]
    announce(f"bf16 fwd {label} fused={fused} no_ws={no_ws} M={M} N={ref['Y'].shape[1]} "
             f"K={X.shape[1]} r={r}")
    T = torch.empty((M, r), dtype=torch.float32, device=X.device)
    Y = lq.lq_lora_fwd(X, Wd, A, B, s, T_out=T, fused=fused, no_ws=no_ws)
    torch.cuda.synchronize()
    for name, got, want in (("Y", Y, ref["Y"]), ("T", T, ref["T"])):
        e = rel_err(f64(got), want)
        assert e <= BF16_TOL, f"{name} rel err {e:.3e}"
    del Y
    if "dX" not in ref:
        return
    announce(f"bf16 bwd {label} fused={fused} M={M}")
    dY = to_dev(c["dY"])
    dX, dA, dB = lq.lq_lora_bwd(dY, X, Wd, A, B, s, T_saved=T if M > 16 else None, fused=fused)
    torch.cuda.synchronize()
    for name, got in (("dX", dX), ("dA", dA), ("dB", dB)):
        e = rel_err(f64(got), ref[name])
        assert e <= BF16_TOL, f"{name} rel err {e:.3e}"
    # dX alone (dA = dB = NULL) runs the same kernel: bit-identical dX
    dX2, dA2, dB2 = lq.lq_lora_bwd(dY, X, Wd, A, B, s, need_grads=False, fused=fused)
    torch.cuda.synchronize()
    assert dA2 is None and dB2 is None
    assert torch.equal(dX2, dX), "dX-only call differs from the full backward"


def check_layer(c, kind, bwd=True, merge=True, label="", fused=False):
    Wd, Wo = base_for(c, kind)
    check_gpu(c, Wd, oracle_ref(c, Wo, bwd=bwd), label=f"{label} {kind}", fused=fused)
    if merge:
        announce(f"bf16 merge {label} {kind}")
        s = c["alpha"] / c["r"]
        Wm = lq.lq_lora_merge(Wd, to_dev(c["A"]), to_dev(c["B"]), s, dtype=torch.bfloat16)
        torch.cuda.synchronize()
        e = rel_err(f64(Wm), olora.lora_merge(Wo, c["A"].f64(), c["B"].f64(), s))
        assert e <= BF16_TOL, f"merge rel err {e:.3e}"


def check_both_paths(c, kind, label):
    """Default and fused-kernel workspaces on one oracle reference; for an NF4
    base also the forward with no workspace (the fused kernel where the
    smaller workspace selects the K-loop dequantising product)."""
    Wd, Wo = base_for(c, kind)
    ref = oracle_ref(c, Wo)
    for fused in (False, True):
        check_gpu(c, Wd, ref, label=f"{label} {kind}", fused=fused)
    if kind == "nf4" and c["X"].value.shape[0] > 96:  # (decode chunks need their workspace)
        check_gpu(c, Wd, dict(Y=ref["Y"], T=ref["T"]), label=f"{label} {kind}", no_ws=True)


SMALL = [
    (300, 384, 512, 16),     # ragged M, three 128-column tiles
    (2100, 256, 256, 16),    # 256-row tiles, ragged
    (700, 256, 320, 64),     # rank 64 (two 32-row shrink blocks)
    (130, 192, 192, 5),      # odd rank, partial column tile, partial k tile
    (17, 128, 128, 8),       # forward on the decode kernels (one 16-row chunk and one row)
    (97, 256, 512, 16),      # smallest forward past the decode chunks
]


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("shape", SMALL, ids=[f"{m}x{n}x{k}r{r}" for m, n, k, r in SMALL])
def test_small(shape, kind):
    # the default workspace (the large-tile path where N or K is a multiple of
    # 256) and the fused kernels with the smallest workspace
    M, N, K, r = shape
    c = wl.small_case(M, N, K, r, seed=M + N + K + r)
    check_layer(c, kind, label="small")
    check_layer(c, kind, merge=False, label="small-fused", fused=True)


# Shapes that take the large-tile path (256 x 256 tiles, bf16 weight copy in
# the workspace) with the default workspace; with the smaller LQ_OP_*_FUSED
# workspace the fused kernels, or for an NF4 forward with enough 128 x 256
# tiles the product that dequantises in its K loop.
LARGE = [
    (2100, 256, 256, 16),    # split K (9 tiles), ragged last row tile
    (2304, 512, 768, 5),     # split K, odd rank, three 256-wide dX tiles
    (2048, 5376, 256, 64),   # 256 x 128 forward tiles, no split; rank 64
    (4096, 3072, 256, 16),   # 256 x 256 forward tiles
    (2100, 3072, 768, 16),   # NF4, small workspace: 128 x 256 tiles dequantised in the K
                             # loop, ragged M, three four-step code groups
    (2048, 3072, 256, 64),   # NF4 in the K loop at rank 64 (four expand chunks of 16)
    (2100, 3072, 320, 16),   # reduction not a multiple of 256: fused kernels instead
]


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("shape", LARGE, ids=[f"{m}x{n}x{k}r{r}" for m, n, k, r in LARGE])
def test_large_tile_path(shape, kind):
    M, N, K, r = shape
    assert (lq.lq_workspace_size(lq.LQ_OP_FWD, M, N, K, r)
            > lq.lq_workspace_size(lq.LQ_OP_FWD_FUSED, M, N, K, r))
    if K % 256 == 0:  # dX on the large-tile path: output width K in 256-wide tiles
        assert (lq.lq_workspace_size(lq.LQ_OP_BWD, M, N, K, r)
                > lq.lq_workspace_size(lq.LQ_OP_BWD_FUSED, M, N, K, r))
    c = wl.small_case(M, N, K, r, seed=M + N + K + r + 7)
    check_both_paths(c, kind, label="large")


# NF4 shapes with enough 128 x 256 tiles for the products that dequantise in
# their K loop and form T (forward) and U (dX) in the same loop, whatever the
# workspace: ragged M, rank 64 and 40 (two 32-rank blocks), rank 8, and an odd
# rank (forward in the K loop; dX on the other paths, which need r % 8 == 0).
KLOOP = [
    (2100, 2816, 2816, 16),
    (2000, 3072, 3072, 64),
    (2100, 2816, 2816, 40),
    (2100, 2816, 2816, 8),
    (2100, 2816, 2816, 5),
    (1024, 128, 6144, 16),   # dX in the K loop with one code group (N = 128, two steps)
    (1000, 256, 6144, 64),   # dX with two code groups, rank 64, ragged M
    (1536, 24576, 256, 24),  # forward in the K loop with one code group (K = 256), rank 24
]


@pytest.mark.parametrize("shape", KLOOP, ids=[f"{m}x{n}x{k}r{r}" for m, n, k, r in KLOOP])
def test_kloop_nf4(shape):
    M, N, K, r = shape
    c = wl.small_case(M, N, K, r, seed=M + N + K + r + 13)
    check_both_paths(c, "nf4", label="kloop")


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("M", [1, 4, 16, 33, 96])  # 33, 96: 16-row decode chunks
def test_decode_small(M, kind):
    c = wl.small_case(M, 256, 512, 16, seed=100 + M)
    check_layer(c, kind, label="decode", bwd=True, merge=False)
    c = wl.small_case(M, 192, 192, 5, seed=200 + M)
    check_layer(c, kind, label="decode-odd", bwd=False, merge=False)


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("M", [24, 48, 96])
def test_mid_rows_wide_output(M, kind):
    """Outputs wider than 4096: past 32 rows (NF4) or 16 (bf16) the default
    workspace takes the large-tile path instead of the decode chunks; the
    smaller workspace keeps the chunks."""
    c = wl.small_case(M, 4352, 256, 16, seed=400 + M)
    check_both_paths(c, kind, label="mid-wide")


@pytest.mark.parametrize("M", [1, 31, 33, 64])
def test_small_rows_nf4_dx(M):
    """dX for at most 64 rows with an NF4 weight and the default workspace:
    the weight-streaming kernel (128-column x 512-row pieces of the codes,
    float32 partial sums of dY W' and of U per row range, added in order by a
    second launch).  The config-3 weight at 4096^2 (8 row ranges, 32 column
    slabs, one rank column per slab); 1088 x 256 at rank 64 (a last row range
    of 64 rows, two column slabs holding 32 rank columns each); 320 x 768 with
    single-level constants (one ragged row range)."""
    c = wl.config3(M=M)
    check_layer(c, "nf4", merge=False, label="small-rows-dx config3")
    c = wl.small_case(M, 1088, 256, 64, seed=600 + M)
    check_layer(c, "nf4", merge=False, label="small-rows-dx r64")
    c = wl.small_case(M, 320, 768, 8, seed=500 + M)
    Wd = lq.lq_nf4_quantize(to_dev(c["W0"]), double_quant=False)
    W0v = c["W0"].value
    Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(
        onf4.nf4_quantize(W0v, double_quant=False))).reshape(W0v.shape)
    check_gpu(c, Wd, oracle_ref(c, Wo), label="small-rows-dx single-level")


@pytest.mark.parametrize("M", [17, 32, 33, 64])
def test_small_rows_nf4_fwd(M):
    """Forward of 17 to 64 rows with an NF4 weight and the default workspace:
    the weight-streaming kernel (128-row x 512-column pieces, each code read
    and dequantised once, partial sums per column range added in order by a
    second launch that applies the expand and writes T).  The config-3 weight
    at 4096^2 (8 column ranges); 1024 x 1536 at rank 40 (two 32-rank blocks of
    T partial sums, three column ranges); 384 x 1024 at rank 5 with
    single-level constants."""
    c = wl.config3(M=M)
    check_layer(c, "nf4", bwd=False, merge=False, label="small-rows-fwd config3")
    c = wl.small_case(M, 1024, 1536, 40, seed=700 + M)
    check_layer(c, "nf4", bwd=False, merge=False, label="small-rows-fwd r40")
    c = wl.small_case(M, 384, 1024, 5, seed=800 + M)
    Wd = lq.lq_nf4_quantize(to_dev(c["W0"]), double_quant=False)
    W0v = c["W0"].value
    Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(
        onf4.nf4_quantize(W0v, double_quant=False))).reshape(W0v.shape)
    check_gpu(c, Wd, oracle_ref(c, Wo, bwd=False), label="small-rows-fwd single-level r5")


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("M", [1, 16, 96])
def test_decode_rank64(M, kind):
    """Ranks past 32 on the decode kernels (the widest T partial layout)."""
    c = wl.small_case(M, 256, 512, 64, seed=300 + M)
    check_layer(c, kind, label="decode-r64", bwd=False, merge=False)


@pytest.mark.parametrize("kind", ["dense", "nf4"])
@pytest.mark.parametrize("M", [3, 300])
def test_zero_b_is_base_output(M, kind):
    """B = 0: the adapter branch adds exact zeros -- same bits as with A = 0."""
    announce(f"bf16 B=0 {kind} M={M}")
    c = wl.small_case(M, 256, 256, 16, seed=5, zero_b=True)
    X, A, B = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"])
    Wd, Wo = base_for(c, kind)
    Y = lq.lq_lora_fwd(X, Wd, A, B, 2.0)
    Y0 = lq.lq_lora_fwd(X, Wd, torch.zeros_like(A), B, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))
    assert rel_err(f64(Y), c["X"].f64() @ Wo.T) <= BF16_TOL
    dY = to_dev(c["dY"])
    _, dA, dB = lq.lq_lora_bwd(dY, X, Wd, A, B, 2.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA).item() == 0


@pytest.mark.parametrize("kind", ["nf4", "dense"])
def test_config3_qlora_full(kind):
    """QLoRA linear 4096^2, r = 16, alpha = 32, M = 2048: the NF4 + DQ base of
    the workload and, for the fused kernels' dense form, the same weight in
    bf16; whole tensors through both workspaces and the merge."""
    c = wl.config3()
    check_both_paths(c, kind, label="config3")
    if kind == "nf4":
        check_layer(c, kind, bwd=False, label="config3-merge")


@pytest.mark.parametrize("M", [1, 4, 16, 48])
def test_config3_decode(M):
    c = wl.config3(M=32)
    c["X"] = wl.decode_inputs(M)
    check_layer(c, "nf4", bwd=False, merge=False, label=f"config3-decode")


@pytest.mark.parametrize("proj", ["q", "v"])
def test_config2_lora_bf16(proj):
    """LoRA on q_proj / v_proj shapes, dense bf16 base, r = 8, M = 4096."""
    c2 = wl.config2(projections=(proj,))
    p = c2["proj"][proj]
    c = dict(W0=p["W0"], A=p["A"], B=p["B"], dY=p["dY"], X=c2["X"], r=8, alpha=16.0)
    check_both_paths(c, "dense", label=f"config2-{proj}")


@functools.lru_cache(maxsize=1)
def _config4():
    return wl.config4(only=("q", "gate", "down"))


@pytest.mark.parametrize("kind", ["nf4", "dense"])
@pytest.mark.parametrize("proj", ["q", "gate", "down"])
def test_config4_block(proj, kind):
    """One Llama-2-7B-shaped block, r = 64, alpha = 128, M = 8192: the three
    distinct shapes (4096 x 4096, 11008 x 4096, 4096 x 11008), with the
    workload's NF4 + DQ base and the same weight in bf16."""
    c4 = _config4()
    p = c4["proj"][proj]
    X = c4["X_down"] if proj == "down" else c4["X"]
    c = dict(W0=p["W0"], A=p["A"], B=p["B"], dY=p["dY"], X=X, r=64, alpha=128.0)
    check_both_paths(c, kind, label=f"config4-{proj}")


@pytest.mark.parametrize("shape", [(2100, 256, 256, 16), (2048, 5376, 256, 64)],
                         ids=["splitK", "nosplit"])
def test_graph_replay_matches_eager(shape):
    """Forward + backward captured in one HIP graph: every replay (with eager
    calls and synchronisation between replays) equals the eager result
    bitwise, including the split-K flags that the shrink kernel clears."""
    M, N, K, r = shape
    c = wl.small_case(M, N, K, r, seed=11)
    s = c["alpha"] / c["r"]
    X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
    Wd, _ = base_for(c, "nf4")
    dev = X.device
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    T = torch.empty((M, r), dtype=torch.float32, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    wsf = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD, M, N, K, r), dtype=torch.uint8, device=dev)
    wsb = torch.empty(lq.lq_workspace_size(lq.LQ_OP_BWD, M, N, K, r), dtype=torch.uint8, device=dev)

    def run():
        lq.lq_lora_fwd(X, Wd, A, B, s, T_out=T, Y=Y, ws=wsf)
        lq.lq_lora_bwd(dY, X, Wd, A, B, s, T_saved=T, dA=dA, dB=dB, ws=wsb, dX=dX)

    announce(f"graph replay M={M} N={N} K={K} r={r}")
    lq.lq_debug_wait_giveups()  # count from zero
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (Y, T, dX, dA, dB)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        for t in (Y, T, dX, dA, dB):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("Y", "T", "dX", "dA", "dB"), (Y, T, dX, dA, dB), ref):
            assert torch.equal(got, want), f"replay {i}: {name} differs from the eager result"
        run()  # eager work between replays
        torch.cuda.synchronize()
    assert lq.lq_debug_wait_giveups() == 0  # no split-K wait gave up


def test_timing_aid_counts_large_tile_launches():
    """lq_timing_enable brackets the product launches with events on their
    stream: two forward calls on the large-tile path give two g256_fwd
    records with positive durations, and reading forgets them."""
    M, N, K, r = 2100, 256, 256, 16
    c = wl.small_case(M, N, K, r, seed=5)
    X, A, B = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"])
    Wd, _ = base_for(c, "nf4")
    lq.lq_timing_enable(True)
    try:
        lq.lq_timing_read("g256_fwd")
        for _ in range(2):
            lq.lq_lora_fwd(X, Wd, A, B, 2.0)
        torch.cuda.synchronize()
        ms, n = lq.lq_timing_read("g256_fwd")
        assert n == 2 and ms > 0.0
        assert lq.lq_timing_read("g256_fwd") == (0.0, 0)
    finally:
        lq.lq_timing_enable(False)

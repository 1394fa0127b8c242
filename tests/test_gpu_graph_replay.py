"""HIP graph capture of the plain forward + backward (decode, fused and
large-tile paths, dense or NF4 base), dropout, DoRA and AdamW entry points: every replay
(with eager calls and synchronisation between replays) gives the eager
result bit for bit.  None of these calls records a memset; the flags and
partial sums they use are written by kernels."""
import numpy as np
import pytest
import torch

from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import DEV, announce, to_dev

pytestmark = pytest.mark.gpu


def capture(run):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    return g


def check_replays(run, outs, names, label):
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = capture(run)
    for i in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, ref):
            assert torch.equal(got, want), f"{label} replay {i}: {name} differs from eager"
        run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [8, 300, 2100], ids=["decode", "fused", "large"])
@pytest.mark.parametrize("kind", ["dense", "nf4"])
def test_plain_step_replays(M, kind):
    N, K, r = 256, 512, 16
    announce(f"graph plain {kind} M={M}")
    c = wl.small_case(M, N, K, r, seed=30)
    s = c["alpha"] / r
    X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
    Wd = lq.lq_nf4_quantize(to_dev(c["W0"])) if kind == "nf4" else to_dev(c["W0"])
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dA = torch.empty((r, K), dtype=torch.float32, device=DEV)
    dB = torch.empty((N, r), dtype=torch.float32, device=DEV)
    wsf = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD, M, N, K, r), dtype=torch.uint8,
                      device=DEV)
    wsb = torch.empty(lq.lq_workspace_size(lq.LQ_OP_BWD, M, N, K, r), dtype=torch.uint8,
                      device=DEV)

    def run():
        lq.lq_lora_fwd(X, Wd, A, B, s, T_out=T, Y=Y, ws=wsf)
        lq.lq_lora_bwd(dY, X, Wd, A, B, s, T_saved=T, dA=dA, dB=dB, ws=wsb, dX=dX)
    check_replays(run, (Y, T, dX, dA, dB), ("Y", "T", "dX", "dA", "dB"), "plain")


@pytest.mark.parametrize("M", [300, 2100], ids=["fused", "large"])
def test_dropout_step_replays(M):
    N, K, r = 256, 256, 16
    announce(f"graph dropout M={M}")
    c = wl.small_case(M, N, K, r, seed=31)
    s = c["alpha"] / r
    X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
    Wd = lq.lq_nf4_quantize(to_dev(c["W0"]))
    keep = torch.from_numpy(wl.dropout_keep_bits(M, K, 0.1, seed=5)).to(DEV)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dA = torch.empty((r, K), dtype=torch.float32, device=DEV)
    dB = torch.empty((N, r), dtype=torch.float32, device=DEV)
    wsf = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD_DROPOUT, M, N, K, r), dtype=torch.uint8,
                      device=DEV)
    wsb = torch.empty(lq.lq_workspace_size(lq.LQ_OP_BWD_DROPOUT, M, N, K, r), dtype=torch.uint8,
                      device=DEV)

    def run():
        lq.lq_lora_fwd_dropout(X, Wd, A, B, s, keep, 0.1, T_out=T, Y=Y, ws=wsf)
        lq.lq_lora_bwd_dropout(dY, X, Wd, A, B, s, keep, 0.1, T_saved=T, dA=dA, dB=dB, ws=wsb,
                               dX=dX)
    check_replays(run, (Y, T, dX, dA, dB), ("Y", "T", "dX", "dA", "dB"), "dropout")


@pytest.mark.parametrize("M", [300, 2100], ids=["fused", "large"])
def test_dora_step_replays(M):
    N, K, r = 256, 256, 16
    announce(f"graph dora M={M}")
    c = wl.small_case(M, N, K, r, seed=32)
    s = c["alpha"] / r
    X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
    Wd = lq.lq_nf4_quantize(to_dev(c["W0"]))
    m = torch.from_numpy(wl.dora_magnitude(N, K)).to(DEV)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    Z = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    sv = torch.empty(lq.lq_dora_saved_floats(N, r), dtype=torch.float32, device=DEV)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dA = torch.empty((r, K), dtype=torch.float32, device=DEV)
    dB = torch.empty((N, r), dtype=torch.float32, device=DEV)
    dm = torch.empty(N, dtype=torch.float32, device=DEV)
    wsf = torch.empty(lq.lq_workspace_size(lq.LQ_OP_DORA_FWD, M, N, K, r), dtype=torch.uint8,
                      device=DEV)
    wsb = torch.empty(lq.lq_workspace_size(lq.LQ_OP_DORA_BWD, M, N, K, r), dtype=torch.uint8,
                      device=DEV)

    def run():
        lq.lq_dora_fwd(X, Wd, A, B, s, m, Z_out=Z, T_out=T, saved_out=sv, Y=Y, ws=wsf)
        lq.lq_dora_bwd(dY, X, Wd, A, B, s, m, Z, T_saved=T, saved=sv, dA=dA, dB=dB, dmag=dm,
                       ws=wsb, dX=dX)
    check_replays(run, (Y, Z, T, sv, dX, dA, dB, dm), ("Y", "Z", "T", "saved", "dX", "dA", "dB",
                                                       "dm"), "dora")


def test_adamw_step_replays():
    # the step updates its state in place: a graph replayed k times equals k
    # eager calls on a copy of the same state
    sizes = [16 * 512, 512 * 16, 1000, 3]
    announce("graph adamw")
    masters, grads = wl.adamw_case(sizes, 1, seed=33)

    def state():
        return [(torch.from_numpy(p).to(DEV), torch.zeros(n, device=DEV),
                 torch.zeros(n, device=DEV), torch.from_numpy(g).to(DEV),
                 torch.empty(n, dtype=torch.bfloat16, device=DEV))
                for n, p, g in zip(sizes, masters, grads[0])]
    eager, graphed = state(), state()
    g = capture(lambda: lq.lq_adamw_step(graphed, 3, lr=1e-3, weight_decay=0.01))
    # the capture's warm-up call ran once eagerly on the graphed state: match it
    lq.lq_adamw_step(eager, 3, lr=1e-3, weight_decay=0.01)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        lq.lq_adamw_step(eager, 3, lr=1e-3, weight_decay=0.01)
        torch.cuda.synchronize()
        for a, b in zip(eager, graphed):
            for k, name in enumerate(("master", "m", "v", "grad", "weight")):
                assert torch.equal(a[k], b[k]), f"adamw replay {i}: {name} differs"

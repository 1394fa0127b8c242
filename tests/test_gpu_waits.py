"""The bounded waits between workgroups of one launch, with give-ups forced
from the host (lq_debug_set_wait_limit(-1): every such wait gives up at once,
and every kernel still runs to its end).

* Decode (M <= 16): every workgroup gives up on the published partial sums of
  T and computes T itself; the output still meets the usual bar against the
  oracle, and the device counts one give-up per workgroup.
* Split K (the large-tile path with few tiles): the waiting workgroup of each
  tile gives up and leaves its partner's partial sums unread; the count is
  reported and the output differs from the normal one.
* Grouped decode (several layers in one launch): one give-up per workgroup
  and layer it touches, outputs still within the bar.
* With the default bound nothing gives up, and the outputs are those of the
  normal path again (the flags are cleared by each call)."""
import numpy as np
import pytest
import torch

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq
from qlora_parameter_efficient_amd import workloads as wl

from .gpu_helpers import BF16_TOL, DEV, announce, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def forced_giveups():
    lq.lq_debug_wait_giveups()  # start from zero
    lq.lq_debug_set_wait_limit(-1)
    try:
        yield
    finally:
        lq.lq_debug_set_wait_limit(0)


def nf4_case(c):
    W0v = c["W0"].value
    Wd = lq.lq_nf4_quantize(to_dev(c["W0"]))
    Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(onf4.nf4_quantize(W0v)))
    return Wd, Wo.reshape(W0v.shape)


@pytest.mark.parametrize("M", [1, 16])
def test_decode_giveups_fall_back_to_direct_t(M, forced_giveups):
    c = wl.config3(M=32)
    c["X"] = wl.decode_inputs(M)
    Wd, Wo = nf4_case(c)
    s = c["alpha"] / c["r"]
    X, A, B = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"])
    N = Wo.shape[0]
    announce(f"waits decode forced give-up M={M}")
    T = torch.empty((M, c["r"]), dtype=torch.float32, device=DEV)
    calls = 3
    for _ in range(calls):
        Y = lq.lq_lora_fwd(X, Wd, A, B, s, T_out=T)
    n = lq.lq_debug_wait_giveups()
    assert n == calls * (N // 16), f"{n} give-ups, expected one per workgroup per call"
    Yo, _, To = olora.lora_forward(c["X"].f64(), Wo, c["A"].f64(), c["B"].f64(), s)
    assert rel_err(f64(Y), Yo) <= BF16_TOL
    assert rel_err(f64(T), To) <= BF16_TOL
    lq.lq_debug_set_wait_limit(0)
    Y2 = lq.lq_lora_fwd(X, Wd, A, B, s, T_out=T)
    assert lq.lq_debug_wait_giveups() == 0
    assert rel_err(f64(Y2), Yo) <= BF16_TOL


def test_split_k_giveups_are_reported(forced_giveups):
    # 2100 x 256 x 256: nine 256 x 256 output tiles, each reduction split in two
    M, N, K, r = 2100, 256, 256, 16
    c = wl.small_case(M, N, K, r, seed=77)
    s = c["alpha"] / c["r"]
    Wd, Wo = nf4_case(c)
    X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
    announce("waits split-K forced give-up")
    Y = lq.lq_lora_fwd(X, Wd, A, B, s)
    dX, _, _ = lq.lq_lora_bwd(dY, X, Wd, A, B, s, need_grads=False)
    n = lq.lq_debug_wait_giveups()
    assert n > 0, "forced give-ups were not counted"
    lq.lq_debug_set_wait_limit(0)
    announce("waits split-K default bound")
    Y2 = lq.lq_lora_fwd(X, Wd, A, B, s)
    dX2, _, _ = lq.lq_lora_bwd(dY, X, Wd, A, B, s, need_grads=False)
    assert lq.lq_debug_wait_giveups() == 0
    Xo, Ao, Bo = c["X"].f64(), c["A"].f64(), c["B"].f64()
    Yo = olora.lora_forward(Xo, Wo, Ao, Bo, s)[0]
    dXo = olora.lora_backward(c["dY"].f64(), Xo, Wo, Ao, Bo, s)[0]
    assert rel_err(f64(Y2), Yo) <= BF16_TOL
    assert rel_err(f64(dX2), dXo) <= BF16_TOL
    # the forced run left each tile with half of its reduction
    assert not torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    assert not torch.equal(dX.view(torch.int16), dX2.view(torch.int16))


def test_no_giveups_in_normal_operation():
    lq.lq_debug_set_wait_limit(0)
    lq.lq_debug_wait_giveups()
    announce("waits normal operation")
    for (M, N, K, r) in ((2100, 256, 256, 16), (4, 4096, 4096, 16), (2304, 512, 768, 5)):
        c = wl.small_case(M, N, K, r, seed=M + 5)
        Wd, _ = nf4_case(c)
        X, A, B, dY = to_dev(c["X"]), to_dev(c["A"]), to_dev(c["B"]), to_dev(c["dY"])
        for _ in range(3):
            lq.lq_lora_fwd(X, Wd, A, B, 2.0)
            lq.lq_lora_bwd(dY, X, Wd, A, B, 2.0, need_grads=False)
    assert lq.lq_debug_wait_giveups() == 0


@pytest.mark.parametrize("M", [1, 16])
def test_grouped_decode_giveups_fall_back_to_direct_t(M, forced_giveups):
    """lq_lora_fwd_decode_layers: a workgroup reads a layer's T once, at its
    first block of that layer, so with every wait giving up it computes T
    itself once per layer it touches (its blocks are a contiguous range over
    the layers' blocks, one workgroup per compute unit)."""
    from .test_gpu_decode_layers import make_layers, run_group, x_rows
    K, r, Ns = 4096, 16, [4096, 4096, 4096]
    layers = make_layers(Ns, K, r, seed=503)
    Xh = x_rows(M, K, seed=61)
    nb = sum(n // 16 for n in Ns)
    grid = min(nb, torch.cuda.get_device_properties(0).multi_processor_count)
    starts = np.cumsum([0] + [n // 16 for n in Ns])
    layer_of = lambda b: int(np.searchsorted(starts, b, side="right") - 1)
    per_call = sum(len({layer_of(b) for b in range(w * nb // grid, (w + 1) * nb // grid)})
                   for w in range(grid))
    announce(f"waits grouped decode forced give-up M={M}")
    calls = 2
    for _ in range(calls):
        Ys, Ts = run_group(layers, to_dev(Xh), M, r)
    n = lq.lq_debug_wait_giveups()
    assert n == calls * per_call, f"{n} give-ups, expected {calls * per_call}"
    for g, (L, Y, T) in enumerate(zip(layers, Ys, Ts)):
        c = L["c"]
        Yo, _, To = olora.lora_forward(Xh.f64(), L["Wo"], c["A"].f64(), c["B"].f64(), L["s"])
        assert rel_err(f64(Y), Yo) <= BF16_TOL, f"layer {g}"
        assert rel_err(f64(T), To) <= BF16_TOL, f"layer {g}"
    lq.lq_debug_set_wait_limit(0)
    run_group(layers, to_dev(Xh), M, r)
    torch.cuda.synchronize()
    assert lq.lq_debug_wait_giveups() == 0

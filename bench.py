#!/usr/bin/env python3
"""Benchmark of the QLoRA adapted linear layer on one MI355X.

Default run (python bench.py [--steps K] [--warmup W]):

* step = one forward + backward of the QLoRA linear at 4096 x 4096, NF4 base
  with double quantisation, r = 16, alpha = 32, M = 2048 tokens, bf16 compute.
  Forward: one launch, the product that dequantises NF4 inside its K loop,
  forms T = X A^T in the same loop and adds the expand (no bf16 copy of W0
  anywhere).  Backward: the same for dX (U = dY B in the K loop, expand
  (s U) A), then the dA / dB reductions.  value = algorithmic fwd+bwd FLOPs /
  wall time per step, the step launched eagerly; the GPU-event time of the
  same timed region and the step replayed from a HIP graph are reported
  beside it.  The step first runs untimed for CLOCK_WARMUP_S seconds so that
  the clocks have settled, and the shader clock is sampled from sysfs during
  the timed region.
* roofline: the dominant kernel -- the K-loop product of the forward or of
  dX, whichever is slower (each does 2 M N K + 2 M K r + 2 M N r FLOPs: the
  product, the rank-r shrink and the expand) -- timed with HIP events that
  the library records
  around its launches on the launch stream (lq_timing_enable), algorithmic
  FLOPs per launch / average duration, against the bf16 dense MFMA peak, and
  against that peak scaled to the sampled clock; traffic (HBM bytes per
  launch) from rocprofv3 FETCH_SIZE / WRITE_SIZE counters scaled by the same
  counters on a plain copy, when they were taken on the current kernel
  source.  Beside it: the forward and dX calls, the forward through the
  older fused kernel (the weight dense bf16, as its only K-loop form here),
  and roofline["decode"]: NF4 decode at M = 1, weight-stream bytes
  per graph-replayed call over 40 cold weight copies, against the HBM peak.
* cpu_baseline: the CPU oracle (float64 NumPy) on the same step.
* secondary lines in the same JSON object: NF4 decode (M = 1, 4, 16) GB/s on
  the weight stream with cold weights, merge, quantise, multi-adapter, the
  forwards of 32 and 64 rows (the weight streamed once), the step with LoRA-input
  dropout and as DoRA, the AdamW step, the plain bf16
  GEMMs of the product kernel's shape through torch (context), and forward +
  backward of config 2 (q and v, bf16, M = 4096, r = 8) and of config 4 (the
  seven projections of a block, NF4, M = 8192, r = 64).

Profiling helpers (for rocprofv3): --mode fwd | fwd_fused | dx | step
| decode | decode1 (M = 1 only) | decode_layers | copy | quant run only that part, a few iterations (after CLOCK_WARMUP_S seconds of
the same work for the first five), and print one line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s (4096²,r=16,M=2048); NF4 decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CUs x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
M, N, K, R = 2048, 4096, 4096, 16
PROD_FLOP = 2 * M * N * K + 2 * M * K * R + 2 * M * N * R       # product + shrink + expand
STEP_FLOP = 2 * (2 * M * N * K) + 6 * M * R * (N + K)             # fwd + bwd, algorithmic
NF4_STREAM_BYTES = N * K // 2 + N * K // 64 + 4 * (N * K // 64 // 256)   # 8,654,848
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "qlora_parameter_efficient_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(KERNEL_SRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PROD_SOURCES = ["gemm256.hip", "device_util.h", "common.h"]
DEC_SOURCES = ["decode.hip", "device_util.h", "common.h", "dispatch.h"]


def traffic_for(kernel, sources):
    """HBM bytes per launch from stored counter runs, if taken on this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_sha") != src_hash(sources):
        return None
    return e.get("bytes_per_launch")


def cuda_time(fn, iters, torch, warm=3):
    """Average GPU time (ms) of fn() over iters back-to-back calls (HIP events),
    after `warm` untimed calls (the first launch of a kernel in a process also
    loads its code)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


CLOCK_WARMUP_S = 0.5
PEAK_SCLK_MHZ = 2400.0         # the clock the peak figures assume


class SclkSampler:
    """Samples the shader clock the driver reports (the starred level of
    pp_dpm_sclk in sysfs, which carries the current frequency) every few
    milliseconds from a background thread while the block runs; ``mhz`` is
    the median of the samples, or None where the file is unreadable."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def read(self):
        import re
        for f in self.files:
            try:
                with open(f) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                return float(m.group(1))
            except OSError:
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self.read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()
        return False

    @property
    def mhz(self):
        return statistics.median(self.samples) if self.samples else None


def spin_sync(ev, torch):
    """Wait for event ``ev`` by polling it, then synchronise the device (the
    poll keeps the host from sleeping in the driver's blocking wait)."""
    while not ev.query():
        pass
    torch.cuda.synchronize()


def setup(torch):
    import numpy as np

    from qlora_parameter_efficient_amd import lq
    from qlora_parameter_efficient_amd import workloads as wl

    dev = "cuda:0"
    c = wl.config3()

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)

    S = dict(c=c, lq=lq, dev=dev, s=c["alpha"] / c["r"])
    S["W0d"] = to_dev(c["W0"])
    S["W"] = lq.lq_nf4_quantize(S["W0d"])
    for k in ("X", "A", "B", "dY"):
        S[k] = to_dev(c[k])
    S["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    S["T"] = torch.empty((M, R), dtype=torch.float32, device=dev)
    S["dX"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    S["dA"] = torch.empty((R, K), dtype=torch.float32, device=dev)
    S["dB"] = torch.empty((N, R), dtype=torch.float32, device=dev)
    S["ws"] = torch.empty(lq.lq_workspace_size(lq.LQ_OP_BWD, M, N, K, R), dtype=torch.uint8,
                          device=dev)
    S["wsf"] = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD, M, N, K, R), dtype=torch.uint8,
                           device=dev)
    torch.cuda.synchronize()
    return S


def fwd(S):
    lq = S["lq"]
    lq.lq_lora_fwd(S["X"], S["W"], S["A"], S["B"], S["s"], T_out=S["T"], Y=S["Y"], ws=S["wsf"])


def fwd_fused(S):
    """The forward of the same layer with the weight dense bf16 and no
    workspace: the older fused kernel (T in the same K loop, bf16 operands
    from LDS), for comparison with the K-loop NF4 product."""
    lq = S["lq"]
    lq.lq_lora_fwd(S["X"], S["W0d"], S["A"], S["B"], S["s"], T_out=S["T"], Y=S["Y"], no_ws=True)


def bwd(S):
    lq = S["lq"]
    lq.lq_lora_bwd(S["dY"], S["X"], S["W"], S["A"], S["B"], S["s"], T_saved=S["T"], dA=S["dA"],
                   dB=S["dB"], ws=S["ws"], dX=S["dX"])


def dx_only(S):
    lq = S["lq"]
    lq.lq_lora_bwd(S["dY"], S["X"], S["W"], S["A"], S["B"], S["s"], ws=S["ws"], dX=S["dX"],
                   need_grads=False)


def step(S):
    fwd(S)
    bwd(S)


def step_graph(S, torch):
    """One step captured in a HIP graph (all buffers preallocated in S)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(S)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(S)
    torch.cuda.synchronize()
    return g


def cpu_baseline(S):
    """The oracle on the same fwd+bwd step, on the host cores."""
    import numpy as np

    from oracle import lora as olora
    from oracle import nf4 as onf4
    affinity = len(os.sched_getaffinity(0))
    threads, blas = affinity, "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} "
                             f"({i.get('threading_layer', '?')})" for i in info)
    except Exception:  # noqa: BLE001
        pass
    c = S["c"]
    q = onf4.nf4_quantize(c["W0"].value)
    Wo = onf4.bf16_bits_to_f64(onf4.nf4_dequantize_bf16(q)).reshape(N, K)
    X, A, B, dY = c["X"].f64(), c["A"].f64(), c["B"].f64(), c["dY"].f64()
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        olora.lora_forward(X, Wo, A, B, S["s"])
        olora.lora_backward(dY, X, Wo, A, B, S["s"])
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(STEP_FLOP / t / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "affinity_cores": affinity, "blas": blas, "kind": "oracle",
            "sample": "full step: float64 NumPy forward + backward of the 4096^2, r=16, M=2048 "
                      f"layer on the NF4-dequantised weight, median of 3 ({t:.2f} s each)"}


def decode_bench(S, torch, iters=200, copies=40, replays=20, ms=(1, 4, 16)):
    """NF4 decode (M = 1, 4, 16) with cold weights: a sequence of calls over
    `copies` distinct NF4 copies (copies x 8.65 MB > the 256 MB Infinity
    Cache).  Graph: the sequence captured once in a HIP graph and replayed
    (launch and host overhead amortised); eager: back-to-back calls from
    Python.  GB/s counts the 4-bit weight stream only."""
    import numpy as np

    from qlora_parameter_efficient_amd import workloads as wl
    lq = S["lq"]
    W = S["W"]
    Ws = [lq.NF4Weight(W.codes.clone(), N, K, W.q8.clone(), W.c2.clone()) for _ in range(copies)]
    out = {}
    for m in ms:
        Xm = torch.from_numpy(wl.decode_inputs(m).bits.view(np.int16).copy()).view(
            torch.bfloat16).to(S["dev"])
        Ym = torch.empty((m, N), dtype=torch.bfloat16, device=S["dev"])
        Tm = torch.empty((m, R), dtype=torch.float32, device=S["dev"])
        wsm = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD, m, N, K, R), dtype=torch.uint8,
                          device=S["dev"])
        it = iter(range(10 ** 9))

        def call(w):
            lq.lq_lora_fwd(Xm, w, S["A"], S["B"], S["s"], T_out=Tm, ws=wsm, Y=Ym)

        def call_cold():
            call(Ws[next(it) % copies])

        for _ in range(20):
            call_cold()
        t_eager = cuda_time(call_cold, iters, torch)
        t_warm = cuda_time(lambda: call(W), iters, torch)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(Ws[0])
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            for w in Ws:
                call(w)
        g.replay()
        t_graph = cuda_time(g.replay, replays, torch) / copies
        out[f"M{m}"] = {"us_per_call_graph_cold": round(t_graph * 1e3, 2),
                        "weight_stream_GBs_graph_cold": round(NF4_STREAM_BYTES / (t_graph * 1e-3) / 1e9, 1),
                        "us_per_call_eager_cold": round(t_eager * 1e3, 2),
                        "us_per_call_eager_warm": round(t_warm * 1e3, 2)}
        del g
    del Ws
    return out


def decode_layers_bench(S, torch, n_layers=3, groups=14, replays=20):
    """One-launch decode of n_layers 4096^2 NF4 layers that read the same X
    (the query, key and value projections of a block), M = 1, 4, 16, with
    cold weights: `groups` calls over groups x n_layers distinct weight copies
    (> the 256 MB Infinity Cache), captured in a HIP graph and replayed.  GB/s
    counts the 4-bit weight streams of the call's layers."""
    import numpy as np

    from qlora_parameter_efficient_amd import workloads as wl
    lq = S["lq"]
    W = S["W"]
    Ws = [[lq.NF4Weight(W.codes.clone(), N, K, W.q8.clone(), W.c2.clone())
           for _ in range(n_layers)] for _ in range(groups)]
    As, Bs = [S["A"]] * n_layers, [S["B"]] * n_layers
    sc = [S["s"]] * n_layers
    out = {"layers": n_layers, "N": N, "K": K, "r": R}
    for m in (1, 4, 16):
        Xm = torch.from_numpy(wl.decode_inputs(m).bits.view(np.int16).copy()).view(
            torch.bfloat16).to(S["dev"])
        Ys = [torch.empty((m, N), dtype=torch.bfloat16, device=S["dev"]) for _ in range(n_layers)]

        def call(ws):
            lq.lq_lora_fwd_decode_layers(Xm, ws, As, Bs, sc, Ys=Ys)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(Ws[0])
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for ws in Ws:
                call(ws)
        g.replay()
        t = cuda_time(g.replay, replays, torch) / groups
        out[f"M{m}"] = {"us_per_call_graph_cold": round(t * 1e3, 2),
                        "us_per_layer": round(t * 1e3 / n_layers, 2),
                        "weight_stream_GBs_graph_cold":
                            round(n_layers * NF4_STREAM_BYTES / (t * 1e-3) / 1e9, 1)}
        del g
    del Ws
    return out


def graph_time(fn, torch, calls=20, replays=10):
    """GPU time (ms) per fn() call: `calls` calls captured in one HIP graph,
    replayed `replays` times (host and launch overhead amortised)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    t = cuda_time(g.replay, replays, torch) / calls
    del g
    return t


def secondary(S, torch, dec=None):
    import numpy as np
    lq = S["lq"]
    res = {}
    res["decode_nf4"] = dec if dec is not None else decode_bench(S, torch)
    res["decode_nf4_three_layers_one_launch"] = decode_layers_bench(S, torch)
    # forwards of 32 and 64 rows (the weight-streaming kernel), graph-launched, warm weights
    from qlora_parameter_efficient_amd import workloads as wlc
    chunks = {}
    for m in (32, 64):
        Xm = torch.from_numpy(wlc.decode_inputs(m).bits.view(np.int16).copy()).view(
            torch.bfloat16).to(S["dev"])
        Ym = torch.empty((m, N), dtype=torch.bfloat16, device=S["dev"])
        wsm = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD, m, N, K, R), dtype=torch.uint8,
                          device=S["dev"])
        t = graph_time(lambda: lq.lq_lora_fwd(Xm, S["W"], S["A"], S["B"], S["s"], ws=wsm, Y=Ym),
                       torch)
        chunks[f"M{m}"] = {"us_per_call_graph": round(t * 1e3, 2)}
    res["forward_nf4_small_rows"] = chunks
    # one-time ops, HBM-bound: GPU time per call from graph-captured sequences
    Wm = torch.empty((N, K), dtype=torch.bfloat16, device=S["dev"])
    t = graph_time(lambda: lq.lq_lora_merge(S["W"], S["A"], S["B"], S["s"],
                                            dtype=torch.bfloat16, out=Wm), torch)
    del Wm
    mbytes = NF4_STREAM_BYTES + 2 * N * K + 2 * R * (N + K)
    res["merge_nf4_to_bf16"] = {"us": round(t * 1e3, 2), "GBs": round(mbytes / (t * 1e-3) / 1e9, 1)}
    t = graph_time(lambda: lq.lq_nf4_quantize(S["W0d"]), torch)
    qbytes = 2 * N * K + NF4_STREAM_BYTES
    res["nf4_quantize_bf16"] = {"us": round(t * 1e3, 2), "GBs": round(qbytes / (t * 1e-3) / 1e9, 1)}
    t = graph_time(lambda: lq.lq_nf4_dequantize(S["W"], dtype=torch.bfloat16), torch)
    res["nf4_dequantize_bf16"] = {"us": round(t * 1e3, 2),
                                  "GBs": round(qbytes / (t * 1e-3) / 1e9, 1)}
    # context for the product kernel: the plain bf16 GEMMs of the same shape through torch
    # (hipBLASLt), without the expand, on the dequantised weight
    Wb = lq.lq_nf4_dequantize(S["W"], dtype=torch.bfloat16).view(N, K)
    Yb = torch.empty((M, N), dtype=torch.bfloat16, device=S["dev"])
    dXb = torch.empty((M, K), dtype=torch.bfloat16, device=S["dev"])
    gf = lambda: torch.matmul(S["X"], Wb.t(), out=Yb)  # noqa: E731
    gd = lambda: torch.matmul(S["dY"], Wb, out=dXb)  # noqa: E731
    for _ in range(10):  # library handle, workspace and kernel selection
        gf()
        gd()
    t_f = cuda_time(gf, 50, torch)
    t_d = cuda_time(gd, 50, torch)
    res["torch_bf16_gemm_same_shape"] = {
        "fwd_us": round(t_f * 1e3, 2), "dx_us": round(t_d * 1e3, 2),
        "TFLOPs_fwd": round(2 * M * N * K / (t_f * 1e-3) / 1e12, 1),
        "TFLOPs_dx": round(2 * M * N * K / (t_d * 1e-3) / 1e12, 1)}
    del Wb, Yb, dXb
    # multi-adapter serving workload: 4 adapters r=16 over 256 requests, 4096^2 bf16 base
    from qlora_parameter_efficient_amd import workloads as wl
    c5 = wl.config5()
    T5 = int(c5["offsets"][-1])

    def td(t_):
        return torch.from_numpy(t_.bits.view(np.int16).copy()).view(torch.bfloat16).to(S["dev"])

    X5, W5, A5, B5 = td(c5["X"]), td(c5["W0"]), td(c5["A"]), td(c5["B"])
    off = torch.from_numpy(c5["offsets"]).to(S["dev"])
    ad = torch.from_numpy(c5["adapter"]).to(S["dev"])
    Y5 = torch.empty((T5, N), dtype=torch.bfloat16, device=S["dev"])
    ws5 = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD_MULTI, T5, N, K, 16, 4), dtype=torch.uint8,
                      device=S["dev"])
    f = lambda: lq.lq_lora_fwd_multi(X5, W5, A5, B5, 2.0, off, ad, ws=ws5, Y=Y5)  # noqa: E731
    f()
    t = cuda_time(f, 5, torch)
    flop = 2 * T5 * N * K + 2 * T5 * 16 * (N + K)
    res["multi_adapter_config5"] = {"tokens": T5, "ms": round(t, 3),
                                    "TFLOPs": round(flop / (t * 1e-3) / 1e12, 1)}
    del X5, Y5, ws5
    # the config-3 step with the pages' lora_dropout = 0.05 (seeded keep mask)
    keep = torch.from_numpy(wl.dropout_keep_bits(M, K, 0.05, seed=99)).to(S["dev"])
    wsdf = torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD_DROPOUT, M, N, K, R), dtype=torch.uint8,
                       device=S["dev"])
    wsdb = torch.empty(lq.lq_workspace_size(lq.LQ_OP_BWD_DROPOUT, M, N, K, R), dtype=torch.uint8,
                       device=S["dev"])

    def drop_step():
        lq.lq_lora_fwd_dropout(S["X"], S["W"], S["A"], S["B"], S["s"], keep, 0.05, T_out=S["T"],
                               Y=S["Y"], ws=wsdf)
        lq.lq_lora_bwd_dropout(S["dY"], S["X"], S["W"], S["A"], S["B"], S["s"], keep, 0.05,
                               T_saved=S["T"], dA=S["dA"], dB=S["dB"], ws=wsdb, dX=S["dX"])
    drop_step()
    t = cuda_time(drop_step, 20, torch)
    res["dropout_step_config3_p005"] = {"ms": round(t, 4),
                                        "TFLOPs": round(STEP_FLOP / (t * 1e-3) / 1e12, 1)}
    del wsdf, wsdb
    # the config-3 step as DoRA (magnitude per output row, exact backward)
    mag = torch.from_numpy(wl.dora_magnitude(N, K, seed=N + K)).to(S["dev"])
    Zd = torch.empty((M, N), dtype=torch.bfloat16, device=S["dev"])
    dmag = torch.empty(N, dtype=torch.float32, device=S["dev"])
    sv = torch.empty(lq.lq_dora_saved_floats(N, R), dtype=torch.float32, device=S["dev"])
    wsof = torch.empty(lq.lq_workspace_size(lq.LQ_OP_DORA_FWD, M, N, K, R), dtype=torch.uint8,
                       device=S["dev"])
    wsob = torch.empty(lq.lq_workspace_size(lq.LQ_OP_DORA_BWD, M, N, K, R), dtype=torch.uint8,
                       device=S["dev"])

    def dora_step():
        lq.lq_dora_fwd(S["X"], S["W"], S["A"], S["B"], S["s"], mag, Z_out=Zd, T_out=S["T"],
                       saved_out=sv, Y=S["Y"], ws=wsof)
        lq.lq_dora_bwd(S["dY"], S["X"], S["W"], S["A"], S["B"], S["s"], mag, Zd, T_saved=S["T"],
                       saved=sv, dA=S["dA"], dB=S["dB"], dmag=dmag, ws=wsob, dX=S["dX"])
    dora_step()
    t = cuda_time(dora_step, 20, torch)
    res["dora_step_config3"] = {"ms": round(t, 4),
                                "TFLOPs": round(STEP_FLOP / (t * 1e-3) / 1e12, 1)}
    del wsof, wsob, Zd
    # configs 2 and 4 as steps: forward + backward of every linear, inputs drawn on the GPU
    # from a seeded generator with the workloads' shapes and standard deviations
    gen = torch.Generator(device=S["dev"]).manual_seed(2024)

    def normal(shape, sigma):
        return (torch.randn(shape, generator=gen, device=S["dev"]) * sigma).to(torch.bfloat16)

    def linear_step(Mx, Nx, Kx, rx, alpha, nf4):
        W0 = normal((Nx, Kx), 0.02)
        Wl = lq.lq_nf4_quantize(W0) if nf4 else W0
        Al, Bl = normal((rx, Kx), 1.0 / rx ** 0.5), normal((Nx, rx), 0.01)
        Xl, dYl = normal((Mx, Kx), 1.0), normal((Mx, Nx), 1.0)
        bufs = dict(Y=torch.empty((Mx, Nx), dtype=torch.bfloat16, device=S["dev"]),
                    T=torch.empty((Mx, rx), device=S["dev"]),
                    dX=torch.empty((Mx, Kx), dtype=torch.bfloat16, device=S["dev"]),
                    dA=torch.empty((rx, Kx), device=S["dev"]),
                    dB=torch.empty((Nx, rx), device=S["dev"]),
                    wf=torch.empty(lq.lq_workspace_size(lq.LQ_OP_FWD, Mx, Nx, Kx, rx),
                                   dtype=torch.uint8, device=S["dev"]),
                    wb=torch.empty(lq.lq_workspace_size(lq.LQ_OP_BWD, Mx, Nx, Kx, rx),
                                   dtype=torch.uint8, device=S["dev"]))
        sl = alpha / rx

        def run():
            lq.lq_lora_fwd(Xl, Wl, Al, Bl, sl, T_out=bufs["T"], Y=bufs["Y"], ws=bufs["wf"])
            lq.lq_lora_bwd(dYl, Xl, Wl, Al, Bl, sl, T_saved=bufs["T"], dA=bufs["dA"],
                           dB=bufs["dB"], ws=bufs["wb"], dX=bufs["dX"])
        flop = 2 * (2 * Mx * Nx * Kx) + 6 * Mx * rx * (Nx + Kx)
        return run, flop, (W0, Wl, Al, Bl, Xl, dYl, bufs)

    for name, layers, Mx, rx, alpha, nf4 in (
            ("config2_qv_bf16_M4096_r8", [(4096, 4096)] * 2, 4096, 8, 16.0, False),
            ("config4_block_nf4_M8192_r64",
             [(n, k) for _, n, k in wl.LLAMA_BLOCK], 8192, 64, 128.0, True)):
        runs, keep, flop = [], [], 0
        for Nx, Kx in layers:
            run, f, k = linear_step(Mx, Nx, Kx, rx, alpha, nf4)
            runs.append(run)
            keep.append(k)
            flop += f
        step_all = lambda: [f() for f in runs]  # noqa: E731
        step_all()
        t = cuda_time(step_all, 5, torch)
        res[name] = {"linears": len(layers), "ms": round(t, 3),
                     "TFLOPs": round(flop / (t * 1e-3) / 1e12, 1)}
        del runs, keep
    torch.cuda.empty_cache()
    # AdamW step on the adapters: float32 master, m, v and gradient, bf16 working
    # copy (16 bytes read and 14 written per parameter)
    for name, sizes in (("adamw_config4_block_r64", wl.config4_adapter_sizes()),
                        ("adamw_config3_r16", [R * K, N * R])):
        masters, grads = wl.adamw_case(sizes, 1, seed=19)
        ps = []
        for m0, g0 in zip(masters, grads[0]):
            n = m0.size
            ps.append((torch.from_numpy(m0).to(S["dev"]), torch.zeros(n, device=S["dev"]),
                       torch.zeros(n, device=S["dev"]), torch.from_numpy(g0).to(S["dev"]),
                       torch.empty(n, dtype=torch.bfloat16, device=S["dev"])))
        f = lambda: lq.lq_adamw_step(ps, 1, lr=1e-4, weight_decay=0.01)  # noqa: E731
        t = graph_time(f, torch)
        nparam = sum(sizes)
        res[name] = {"tensors": len(sizes), "params": nparam, "us": round(t * 1e3, 2),
                     "GBs": round(30 * nparam / (t * 1e-3) / 1e9, 1)}
        del ps
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", default="full",
                    choices=["full", "step", "fwd", "fwd_fused", "dx", "decode", "decode1",
                             "decode_layers", "copy", "quant"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-secondary", action="store_true")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the layer would shard by tokens, with one all-reduce of dA and dB)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if a.mode == "copy":
        # a plain elementwise kernel of known traffic (reads 1 GiB, writes
        # 1 GiB), for scaling the HBM byte counters
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "kernel": "neg (elementwise float32)",
                          "bytes_read": nbytes, "bytes_written": nbytes, "launches": a.steps}))
        return 0

    S = setup(torch)

    def settle(fn):
        """Run fn untimed for CLOCK_WARMUP_S seconds so that a profiled run sees the
        clocks of steady work (see the timed region below)."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < CLOCK_WARMUP_S:
            for _ in range(20):
                fn(S)
            torch.cuda.synchronize()

    if a.mode in ("fwd", "dx", "step", "fwd_fused"):
        settle({"fwd": fwd, "dx": dx_only, "step": step, "fwd_fused": fwd_fused}[a.mode])
    if a.mode == "fwd":
        for _ in range(a.steps):
            fwd(S)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "fwd", "launches": a.steps}))
        return 0
    if a.mode == "fwd_fused":
        for _ in range(a.steps):
            fwd_fused(S)
        torch.cuda.synchronize()
        print(json.dumps({"mode": a.mode, "launches": a.steps}))
        return 0
    if a.mode == "dx":
        for _ in range(a.steps):
            dx_only(S)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "dx", "launches": a.steps}))
        return 0
    if a.mode == "step":
        for _ in range(a.steps):
            step(S)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "step", "steps": a.steps}))
        return 0
    if a.mode == "quant":
        for _ in range(a.steps):
            S["lq"].lq_nf4_quantize(S["W0d"])
        torch.cuda.synchronize()
        print(json.dumps({"mode": "quant", "launches": a.steps}))
        return 0
    if a.mode == "decode":
        print(json.dumps({"mode": "decode", "decode_nf4": decode_bench(S, torch, iters=a.steps)}))
        return 0
    if a.mode == "decode1":
        print(json.dumps({"mode": "decode1", "decode_nf4": decode_bench(S, torch, iters=a.steps,
                                                                         replays=2, ms=(1,))}))
        return 0
    if a.mode == "decode_layers":
        print(json.dumps({"mode": "decode_layers", "decode_layers": decode_layers_bench(S, torch)}))
        return 0

    # The GPU's clocks settle only after some milliseconds of sustained work:
    # with five warm-up steps (about 1 ms) the first timed steps run up to 10%
    # slower than the steady state.  So the step first runs, untimed, for
    # CLOCK_WARMUP_S seconds, then the W warm-up steps, then the K timed steps.
    t0 = time.perf_counter()
    n_clock = 0
    while time.perf_counter() - t0 < CLOCK_WARMUP_S:
        for _ in range(50):
            step(S)
        torch.cuda.synchronize()
        n_clock += 50
    for _ in range(a.warmup):
        step(S)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # nothing else runs in this process during the timed region (the clock
    # sampler's thread contends for the interpreter lock with the launches, so
    # the clock is sampled over a second, untimed run of the same steps below)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(a.steps):
        step(S)
    ev1.record()
    spin_sync(ev1, torch)
    wall = time.perf_counter() - t0
    with SclkSampler() as clk:
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < max(wall, 0.02):
            for _ in range(a.steps):
                step(S)
            torch.cuda.synchronize()
    ms_per_step = wall * 1e3 / a.steps
    ev_ms_per_step = ev0.elapsed_time(ev1) / a.steps
    value = STEP_FLOP / (wall / a.steps) / 1e12
    # the same step captured in a HIP graph and replayed, for reference
    g = step_graph(S, torch)
    for _ in range(a.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        g.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) * 1e3 / a.steps
    del g

    # dominant kernel: the K-loop product of the forward or of dX (the same
    # algorithmic FLOPs); event pairs recorded by the library around each
    # launch, on the stream it is launched on
    lq = S["lq"]
    t_fwd_call = cuda_time(lambda: fwd(S), 50, torch)
    t_dx_call = cuda_time(lambda: dx_only(S), 50, torch)
    t_fused_call = cuda_time(lambda: fwd_fused(S), 20, torch)
    t_step_ev = cuda_time(lambda: step(S), 20, torch)
    lq.lq_timing_enable(True)
    for k in ("q256_fwd", "q256_dx"):
        lq.lq_timing_read(k)
    with SclkSampler() as kclk:
        for _ in range(50):
            fwd(S)
            dx_only(S)
        torch.cuda.synchronize()
    ms_f, n_f = lq.lq_timing_read("q256_fwd")
    ms_d, n_d = lq.lq_timing_read("q256_dx")
    lq.lq_timing_enable(False)
    t_fwd, t_dx = ms_f / max(n_f, 1), ms_d / max(n_d, 1)
    if t_dx > t_fwd:
        name, t_dom = ("q256_dx_kernel (dY deq(W0) with NF4 dequantised in the K loop, U = dY B "
                       "in the same loop, expand; 128x256 tiles)"), t_dx
        traffic = traffic_for("q256_dx", PROD_SOURCES)
    else:
        name, t_dom = ("q256_fwd_kernel (X deq(W0)^T with NF4 dequantised in the K loop, T = X A^T "
                       "in the same loop, expand; 128x256 tiles)"), t_fwd
        traffic = traffic_for("q256_fwd", PROD_SOURCES)
    achieved = PROD_FLOP / (t_dom * 1e-3) / 1e12
    roof = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "flop_per_launch": PROD_FLOP, "us_per_launch": round(t_dom * 1e3, 2),
            "sclk_mhz": kclk.mhz,
            "frac_at_sclk": (round(achieved / (PEAK_BF16_TFLOPS * kclk.mhz / PEAK_SCLK_MHZ), 4)
                             if kclk.mhz else None),
            "launches_timed": min(n_f, n_d),
            "us_fwd_kernel": round(t_fwd * 1e3, 2), "us_dx_kernel": round(t_dx * 1e3, 2),
            "us_fwd_call": round(t_fwd_call * 1e3, 2), "us_dx_call": round(t_dx_call * 1e3, 2),
            "us_fwd_fused_dense_call": round(t_fused_call * 1e3, 2)}
    # NF4 decode at M = 1: weight-stream bytes per call over the graph-replayed
    # call time with cold weights, against the HBM peak
    dec = decode_bench(S, torch)
    d1 = dec["M1"]
    roof["decode"] = {"kernel": "dq_kernel (NF4 decode, T formed in the same launch), M=1",
                      "bound": "hbm", "achieved": d1["weight_stream_GBs_graph_cold"],
                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(d1["weight_stream_GBs_graph_cold"] / PEAK_HBM_GBS, 4),
                      "bytes_per_call": NF4_STREAM_BYTES,
                      "us_per_call": d1["us_per_call_graph_cold"],
                      "traffic": traffic_for("dq_m1", DEC_SOURCES)}
    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "QLoRA linear fwd+bwd: W0 4096x4096 NF4 (block 64, 8-bit double "
                                  "quant block 256), r=16, alpha=32, X 2048x4096 bf16, dY 2048x4096",
                      "M": M, "N": N, "K": K, "r": R, "step_flop": STEP_FLOP},
           "gpu_event_ms_per_step": round(ev_ms_per_step, 4),
           "gpu_event_ms_per_step_steady": round(t_step_ev, 4),
           "clock_warmup_steps": n_clock,
           "graph_ms_per_step": round(ms_graph, 4),
           "sclk_mhz_same_steps": clk.mhz, "sclk_samples": len(clk.samples),
           "roofline": roof}
    if not a.no_cpu:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(S)
    if not a.no_secondary:
        log("secondary measurements ...")
        out["secondary"] = secondary(S, torch, dec)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

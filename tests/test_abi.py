"""C-ABI checks that need no GPU: the library loads, exports every function
include/lq.h declares, its host-side entry points agree with the pages and the
oracle, and argument errors are reported before anything would launch."""
import ctypes
import os

import numpy as np
import pytest

from oracle import lora as olora
from oracle import nf4 as onf4
from qlora_parameter_efficient_amd import lq

pytestmark = pytest.mark.skipif(not os.path.exists(lq.LIB_PATH),
                                reason="liblq.so not built (run __graft_entry__.build())")


def test_exports_every_declared_symbol():
    declared = lq.declared_symbols()
    assert len(declared) == 24
    L = lq.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(lq._SIGS)


@pytest.mark.parametrize("cb", ["nf4", "nf4_symmetric"])
def test_library_codebook_equals_oracle_bitwise(cb):
    ours = np.array(lq.lq_nf4_codebook(cb), dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), onf4.nf4_codebook(cb).view(np.uint32))
    assert lq.lib().lq_nf4_codebook(2, ctypes.cast((ctypes.c_float * 16)(), ctypes.c_void_p)) == -1


def test_num_params_matches_oracle():
    for N, K, r in ((4096, 4096, 16), (4096, 4096, 8), (11008, 4096, 64), (4096, 11008, 16)):
        assert lq.lq_lora_num_params(N, K, r) == olora.lora_num_params(N, K, r)
    assert lq.lq_lora_num_params(4096, 4096, 16) == 131072


def test_check_segments():
    off = np.array([0, 3, 3, 10], np.int32)
    ad = np.array([1, 0, 3], np.int32)
    assert lq.lq_check_segments(off, ad, 10, 4) == 0
    assert lq.lq_check_segments(off, ad, 11, 4) == -1               # wrong end
    assert lq.lq_check_segments(off, np.array([1, 0, 4], np.int32), 10, 4) == -1   # id range
    assert lq.lq_check_segments(np.array([0, 5, 3, 10], np.int32), ad, 10, 4) == -1  # decrease
    assert lq.lq_check_segments(np.array([1, 3, 3, 10], np.int32), ad, 10, 4) == -1  # start
    assert "adapter id" in lq.lq_last_error() or "offsets" in lq.lq_last_error()


def test_workspace_sizes():
    # up to 16 rows: the one-launch decode kernel needs no workspace (its
    # handoff of T lives in the library's per-stream slot)
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 16, 256, 256, 8) == 0
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 4, 4096, 4096, 16) == 0
    assert lq.lq_workspace_size(lq.LQ_OP_FWD_FUSED, 5, 256, 256, 8) == 0
    # 17 to 96 rows: the chunk kernels, 8 partial sums of T per row (16-row
    # chunks, rows padded to a multiple of 16)
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 33, 256, 256, 8) == 8 * 48 * 8 * 4
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 90, 256, 256, 8) == 8 * 96 * 8 * 4
    # wider than 4096 outputs: past 32 rows the LQ_OP_FWD size also holds the large-tile
    # path's part (bf16 weight copy), which then runs; the fused size stays the chunks'
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 32, 4352, 256, 16) == 8 * 32 * 16 * 4
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 48, 4352, 256, 16) > 4352 * 256 * 2
    assert lq.lq_workspace_size(lq.LQ_OP_FWD_FUSED, 48, 4352, 256, 16) == 8 * 48 * 16 * 4
    assert lq.lq_workspace_size(lq.LQ_OP_FWD_FUSED, 97, 256, 256, 8) == 97 * 8 * 4
    # beyond: the default size also holds the large-tile path's bf16 copy of W0
    assert lq.lq_workspace_size(lq.LQ_OP_FWD, 97, 256, 256, 8) >= 97 * 8 * 4 + 256 * 256 * 2
    assert lq.lq_workspace_size(lq.LQ_OP_BWD, 2048, 4096, 4096, 16) >= 2 * 2048 * 16 * 4
    assert lq.lq_workspace_size(lq.LQ_OP_FWD_MULTI, 1000, 4096, 4096, 16, 4) >= 1000 * 4


def _weight(kind=0, N=256, K=256, dtype=lq.LQ_BF16, ptr=0x1000):
    w = lq.LqWeightStruct()
    w.kind, w.dtype, w.N, w.K = kind, dtype, N, K
    if kind == 0:
        w.dense = ptr
    else:
        w.codes, w.q8, w.c2 = ptr, ptr, ptr
        w.double_quant = 1
    return w


def _fwd(w, X=0x1000, M=64, A=0x1000, B=0x1000, r=8, dt=lq.LQ_BF16, Y=0x1000, ws=None, wsb=0):
    return lq.lib().lq_lora_fwd(X, M, ctypes.byref(w), A, B, r, 2.0, dt, Y, None, ws, wsb, None)


def test_argument_errors_launch_nothing():
    L = lq.lib()
    # null weight pointers / descriptors
    assert _fwd(_weight(ptr=0)) == -1
    assert L.lq_lora_fwd(0x1000, 64, None, 0x1000, 0x1000, 8, 2.0, 1, 0x1000, None, None, 0, None) == -1
    # rank outside [1, 64]
    assert _fwd(_weight(), r=0) == -2 and _fwd(_weight(), r=65) == -2
    # bf16 shape rules: K % 64, N % 32
    assert _fwd(_weight(K=200)) == -2
    assert _fwd(_weight(N=100)) == -2
    assert _fwd(_weight(N=96)) == -2                # N % 64
    # dtype mismatch between descriptor and call
    assert _fwd(_weight(dtype=lq.LQ_F32)) == -1
    # missing workspace when T_out is NULL (M > 0)
    assert _fwd(_weight(), M=40) == -3              # 16-row decode chunks keep partial sums of T in ws
    assert "workspace" in lq.lq_last_error()
    # M = 0 is a no-op
    assert _fwd(_weight(), M=0) == 0
    # bad quantise arguments
    assert L.lq_nf4_quantize(None, 1, 10, 1, 0, 0x1000, 0x1000, 0x1000, None, None) == -1
    assert L.lq_nf4_quantize(0x1000, 1, 0, 1, 0, 0x1000, 0x1000, 0x1000, None, None) == -1
    assert L.lq_nf4_quantize(0x1000, 1, 10, 1, 0, 0x1000, None, 0x1000, None, None) == -1
    assert L.lq_nf4_quantize(0x1000, 7, 10, 1, 0, 0x1000, 0x1000, 0x1000, None, None) == -1
    assert L.lq_nf4_quantize(0x1000, 1, 10, 3, 0, 0x1000, 0x1000, 0x1000, None, None) == -1
    assert L.lq_nf4_quantize(0x1000, 1, 10, 2, 5, 0x1000, 0x1000, 0x1000, None, None) == -1
    assert L.lq_nf4_dequantize(0x1000, None, None, None, 0, 0, 10, 0x1000, 1, None) == -1
    assert L.lq_nf4_dequantize(0x1000, 0x1000, 0x1000, None, 2, 7, 10, 0x1000, 1, None) == -1
    # backward workspace
    w = _weight()
    assert L.lq_lora_bwd(0x1000, 0x1000, 64, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0, 1, None,
                         0x1000, 0x1000, 0x1000, 0, None, 0, None) == -3
    # dA and dB go together; nothing requested is an error
    assert L.lq_lora_bwd(0x1000, 0x1000, 64, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0, 1, None,
                         0x1000, 0x1000, None, 0, 0x1000, 1 << 30, None) == -1
    assert L.lq_lora_bwd(0x1000, 0x1000, 64, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0, 1, None,
                         None, None, None, 0, 0x1000, 1 << 30, None) == -1
    # multi-adapter: rank * adapters over 64, float32, no segments
    assert L.lq_lora_fwd_multi(0x1000, 10, ctypes.byref(w), 0x1000, 0x1000, 5, 16, 2.0, 0x1000,
                               0x1000, 1, 1, 0x1000, 0x1000, 1 << 20, None) == -2
    wf = _weight(dtype=lq.LQ_F32)
    assert L.lq_lora_fwd_multi(0x1000, 10, ctypes.byref(wf), 0x1000, 0x1000, 4, 16, 2.0, 0x1000,
                               0x1000, 1, 0, 0x1000, 0x1000, 1 << 20, None) == -2
    assert L.lq_lora_fwd_multi(0x1000, 10, ctypes.byref(w), 0x1000, 0x1000, 4, 16, 2.0, 0x1000,
                               0x1000, 0, 1, 0x1000, 0x1000, 1 << 20, None) == -1
    # multi-adapter with per-adapter ranks: offsets must start at 0, rise, total <= 64
    sc = (ctypes.c_float * 3)(2.0, 2.0, 2.0)

    def ranks(*offs):
        ro = (ctypes.c_int32 * len(offs))(*offs)
        return L.lq_lora_fwd_multi_ranks(0x1000, 10, ctypes.byref(w), 0x1000, 0x1000, 3, ro, sc,
                                         0x1000, 0x1000, 1, 1, 0x1000, 0x1000, 1 << 20, None)
    assert ranks(1, 2, 3, 4) == -1
    assert ranks(0, 4, 4, 8) == -1
    assert ranks(0, 30, 50, 70) == -2
    assert L.lq_lora_fwd_multi_ranks(0x1000, 10, ctypes.byref(w), 0x1000, 0x1000, 3, None, sc,
                                     0x1000, 0x1000, 1, 1, 0x1000, 0x1000, 1 << 20, None) == -1
    # merge
    assert L.lq_lora_merge(ctypes.byref(w), None, 0x1000, 8, 2.0, 1, 0x1000, None) == -1
    # unknown codebook or constant format in the descriptor
    w2 = _weight()
    w2.codebook = 2
    assert _fwd(w2) == -1
    w3 = _weight(kind=1)
    w3.double_quant = 3
    assert _fwd(w3) == -1


def test_adamw_argument_errors_launch_nothing():
    L = lq.lib()

    def step(entries, gdt=lq.LQ_F32, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, t=1, gs=1.0):
        arr = (lq.LqAdamwTensor * max(1, len(entries)))(*entries)
        return L.lq_adamw_step(arr, len(entries), gdt, lr, b1, b2, eps, wd, t, gs, None)

    ok = lq.LqAdamwTensor(0x1000, 0x2000, 0x3000, 0x4000, None, 100)
    assert step([]) == 0                                  # nothing to do
    assert L.lq_adamw_step(None, 1, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, None) == -1
    assert step([ok], t=0) == -1                          # steps count from 1
    assert step([ok], gdt=7) == -1
    assert step([ok], b1=1.0) == -1 and step([ok], b2=-0.1) == -1
    assert step([ok], lr=float("nan")) == -1 and step([ok], eps=-1.0) == -1
    assert step([ok], wd=-0.5) == -1 and step([ok], gs=float("inf")) == -1
    assert step([ok, lq.LqAdamwTensor(0x1000, None, 0x3000, 0x4000, None, 5)]) == -1
    assert "tensor 1" in lq.lq_last_error()
    assert step([lq.LqAdamwTensor(0x1000, 0x2000, 0x3000, 0x4000, None, -1)]) == -1


def test_dropout_argument_errors_launch_nothing():
    L = lq.lib()
    w = _weight()
    big = 1 << 30

    def fwd(keep=0x1000, p=0.05, dt=lq.LQ_BF16, ws=0x1000, wsb=big, M=64):
        return L.lq_lora_fwd_dropout(0x1000, M, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0, keep, p,
                                     dt, 0x1000, None, ws, wsb, None)

    def bwd(keep=0x1000, p=0.05, dA=0x1000, dB=0x1000, dX=0x1000, wsb=big):
        return L.lq_lora_bwd_dropout(0x1000, 0x1000, 64, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0,
                                     keep, p, lq.LQ_BF16, None, dX, dA, dB, 0, 0x1000, wsb, None)
    assert fwd(keep=None) == -1
    assert fwd(p=1.0) == -1 and fwd(p=-0.1) == -1 and fwd(p=float("nan")) == -1
    assert fwd(dt=lq.LQ_F32) == -2                       # bf16 only
    assert fwd(wsb=100) == -3 and fwd(ws=None) == -3
    assert fwd(M=0, keep=None) == 0                      # no-op
    assert (lq.lq_workspace_size(lq.LQ_OP_FWD_DROPOUT, 2048, 4096, 4096, 16)
            > lq.lq_workspace_size(lq.LQ_OP_FWD_DROPOUT_FUSED, 2048, 4096, 4096, 16)
            >= 2048 * 4096 * 2)
    assert (lq.lq_workspace_size(lq.LQ_OP_BWD_DROPOUT, 2048, 4096, 4096, 16)
            > lq.lq_workspace_size(lq.LQ_OP_BWD_DROPOUT_FUSED, 2048, 4096, 4096, 16))
    assert bwd(keep=None) == -1 and bwd(p=1.5) == -1
    assert bwd(dA=None) == -1                            # dA and dB go together
    assert bwd(dA=None, dB=None, dX=None) == -1
    assert bwd(wsb=100) == -3


def test_dora_argument_errors_launch_nothing():
    L = lq.lib()
    w = _weight(kind=1)
    big = 1 << 34

    def fwd(mag=0x1000, dt=lq.LQ_BF16, wsb=big, M=64):
        return L.lq_dora_fwd(0x1000, M, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0, mag, dt, 0x1000,
                             None, None, None, 0x1000, wsb, None)

    def bwd(dmag=0x1000, Z=0x1000, wsb=big):
        return L.lq_dora_bwd(0x1000, 0x1000, 64, ctypes.byref(w), 0x1000, 0x1000, 8, 2.0, 0x1000,
                             lq.LQ_BF16, Z, None, None, 0x1000, 0x1000, 0x1000, dmag, 0, 0x1000,
                             wsb, None)
    assert fwd(mag=None) == -1
    assert fwd(dt=lq.LQ_F32) == -2
    assert fwd(wsb=1000) == -3
    assert fwd(M=0, mag=None) == 0
    assert bwd(dmag=None) == -1 and bwd(Z=None) == -1
    assert bwd(wsb=1000) == -3
    assert lq.lq_dora_saved_floats(4096, 16) == 4096 + 4096 * 16 + 256
    for op in (lq.LQ_OP_DORA_FWD, lq.LQ_OP_DORA_BWD):
        assert (lq.lq_workspace_size(op, 2048, 4096, 4096, 16)
                > lq.lq_workspace_size(op + 1, 2048, 4096, 4096, 16) > 4096 * 4096 * 2)


def test_timing_read_without_launches():
    lq.lq_timing_enable(True)
    assert lq.lq_timing_read("g256_fwd") == (0.0, 0)
    lq.lq_timing_enable(False)
    assert lq.lib().lq_timing_read(None, None, None) == -1


def test_noalloc_backward_rejects_past_the_static_size():
    """The backward on the library's static workspace refuses a layer whose
    smallest workspace exceeds LQ_NOALLOC_SCRATCH_BYTES, before any HIP call
    (the pointers here are never dereferenced)."""
    N = K = 8192
    M, r = 65536, 64
    need = lq.lq_workspace_size(lq.LQ_OP_BWD_FUSED, M, N, K, r)
    assert need > lq.LQ_NOALLOC_SCRATCH_BYTES
    w = lq.LqWeightStruct()
    w.kind, w.dtype, w.N, w.K = lq.LQ_WEIGHT_DENSE, lq.LQ_BF16, N, K
    w.dense = 256
    rc = lq.lib().lq_lora_bwd_noalloc(256, 256, M, w, 256, 256, r, 1.0, lq.LQ_BF16, None, 256, 256,
                                      256, 0, None)
    assert rc == -3
    assert "static workspace" in lq.lib().lq_last_error().decode()
    assert lq.lib().lq_lora_bwd_noalloc(256, 256, M, None, 256, 256, r, 1.0, lq.LQ_BF16, None,
                                        256, 256, 256, 0, None) == -1


def test_noalloc_size_matches_header():
    text = open(lq.HEADER).read()
    assert "#define LQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert lq.LQ_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_decode_layers_argument_errors_launch_nothing():
    """lq_lora_fwd_decode_layers rejects bad layer counts, M > 16, layers with
    different K or weight formats and NULL pointers before any launch."""
    L = lq.lib()

    def call(ws, M=4, n=None, r=16, X=0x1000, ptrs=0x1000):
        n = len(ws) if n is None else n
        k = max(len(ws), 1)
        warr = (lq.LqWeightStruct * k)(*ws) if ws else None
        vp = ctypes.c_void_p * k
        arr = vp(*([ptrs] * k))
        sc = (ctypes.c_float * k)(*([2.0] * k))
        return L.lq_lora_fwd_decode_layers(
            X, M, n, None if warr is None else ctypes.cast(warr, ctypes.POINTER(lq.LqWeightStruct)),
            ctypes.cast(arr, ctypes.c_void_p), ctypes.cast(arr, ctypes.c_void_p), r,
            ctypes.cast(sc, ctypes.c_void_p), ctypes.cast(arr, ctypes.c_void_p), None, None)

    nf4 = lambda N=256, K=256: _weight(kind=1, N=N, K=K)
    assert call([nf4()], n=0) == -1
    assert call([nf4()] * 9) == -1
    assert call([nf4()], M=17) == -2
    assert call([nf4()], r=65) == -2
    assert call([nf4(), nf4(K=512)]) == -1
    assert call([nf4(), _weight(kind=0)]) == -1
    single = nf4()
    single.double_quant = 0
    single.absmax = 0x1000
    assert call([nf4(), single]) == -1
    assert call([nf4(), nf4(N=96)]) == -2       # N % 64 != 0
    assert call([nf4(), nf4()], ptrs=0) == -1   # NULL A / B / Y entries
    assert call([nf4()], X=0) == -1
    assert call([nf4(), nf4()], M=0, ptrs=0) == 0  # M = 0: nothing to do

"""Seeded synthetic inputs for the LoRA / QLoRA linear workloads.

This module only draws random numbers and rounds them to the storage type the
workload names.  It contains none of the method's arithmetic (no LoRA product,
no quantisation), so both the HIP path and the CPU oracle may take their inputs
from here.

Recipe (one generator per workload, ``numpy.random.default_rng(1000 + c)``):
normal tensors are ``rng.standard_normal(shape, dtype=float32) * sigma`` drawn in
the listed order; tensors stored as bfloat16 are rounded to nearest-even from
that float32 draw.  Shapes follow the Llama-2-7B projections the pages use
(d_model 4096, MLP width 11008; "LLM fine-tuning and LoRA", memory ledger and
target-module calculator).  No trained weights or datasets are involved.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round_bits",
    "bf16_bits_to_f32",
    "Tensor",
    "config1",
    "config2",
    "config3",
    "config4",
    "config5",
    "decode_inputs",
    "small_case",
    "adamw_case",
    "config4_adapter_sizes",
    "dropout_keep_bits",
    "dora_magnitude",
]


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Used only to store the synthetic draws in the workload's dtype; inputs are
    finite by construction.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exactly equal float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """A synthetic tensor in its storage dtype.

    ``bits`` holds the stored representation (uint16 for bf16, float32 for
    fp32); ``value`` is the exact float32 value of every element.
    """

    def __init__(self, f32: np.ndarray, dtype: str):
        assert dtype in ("bf16", "f32")
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = bf16_round_bits(f32)
            self.value = bf16_bits_to_f32(self.bits)
        else:
            self.bits = np.ascontiguousarray(f32, dtype=np.float32)
            self.value = self.bits
        self.shape = self.value.shape

    def f64(self) -> np.ndarray:
        return self.value.astype(np.float64)


def _normal(rng, shape, sigma, dtype):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return Tensor(x, dtype)


def config1(zero_b: bool = False):
    """Single LoRA linear in fp32: W0 256x256, r=8, alpha=16, M=64."""
    rng = np.random.default_rng(1001)
    W0 = _normal(rng, (256, 256), 0.02, "f32")
    A = _normal(rng, (8, 256), 1.0 / np.sqrt(8.0), "f32")
    B = _normal(rng, (256, 8), 0.02, "f32")
    X = _normal(rng, (64, 256), 1.0, "f32")
    dY = _normal(rng, (64, 256), 1.0, "f32")
    if zero_b:
        B = Tensor(np.zeros((256, 8), np.float32), "f32")
    return dict(W0=W0, A=A, B=B, X=X, dY=dY, r=8, alpha=16.0)


def config2(projections=("q", "v"), M: int = 4096):
    """LoRA on Llama-2-7B q_proj / v_proj shapes in bf16: 4096^2, r=8, alpha=16.

    X is 4 sequences x 1024 tokens; one (W0, A, B, dY) per projection, X shared.
    """
    rng = np.random.default_rng(1002)
    per = {}
    for p in ("q", "v"):
        W0 = _normal(rng, (4096, 4096), 0.02, "bf16")
        A = _normal(rng, (8, 4096), 1.0 / np.sqrt(8.0), "bf16")
        B = _normal(rng, (4096, 8), 0.01, "bf16")
        dY = _normal(rng, (4096, 4096), 1.0, "bf16")
        per[p] = dict(W0=W0, A=A, B=B, dY=dY)
    X = _normal(rng, (4096, 4096), 1.0, "bf16")
    out = {p: per[p] for p in projections}
    if M != 4096:
        X = Tensor(X.value[:M], "bf16")
        for p in out:
            out[p]["dY"] = Tensor(out[p]["dY"].value[:M], "bf16")
    return dict(proj=out, X=X, r=8, alpha=16.0)


def config3(M: int = 2048):
    """QLoRA linear: W0 4096^2 (quantised to NF4 by the caller), r=16, alpha=32."""
    rng = np.random.default_rng(1003)
    W0 = _normal(rng, (4096, 4096), 0.02, "bf16")
    A = _normal(rng, (16, 4096), 0.25, "bf16")
    B = _normal(rng, (4096, 16), 0.01, "bf16")
    X = _normal(rng, (2048, 4096), 1.0, "bf16")
    dY = _normal(rng, (2048, 4096), 1.0, "bf16")
    if M != 2048:
        X = Tensor(X.value[:M], "bf16")
        dY = Tensor(dY.value[:M], "bf16")
    return dict(W0=W0, A=A, B=B, X=X, dY=dY, r=16, alpha=32.0)


def decode_inputs(M: int):
    """Decode-sized activations for the config-3 weight (M = 1, 4, 16 in the bench)."""
    rng = np.random.default_rng(2003 + M)
    return _normal(rng, (M, 4096), 1.0, "bf16")


LLAMA_BLOCK = (
    ("q", 4096, 4096),
    ("k", 4096, 4096),
    ("v", 4096, 4096),
    ("o", 4096, 4096),
    ("gate", 11008, 4096),
    ("up", 11008, 4096),
    ("down", 4096, 11008),
)


def config4(M: int = 8192, only=None):
    """All seven projections of one Llama-2-7B block, NF4 base, r=64, alpha=128.

    Returns a generator-free dict of lazily drawn tensors: every projection
    draws (W0, A, B, dY) in block order, then X (M x 4096) and X_down (M x 11008).
    ``only`` restricts which projections are materialised (the draw order is
    kept, skipped tensors are still drawn so the stream stays identical).
    """
    rng = np.random.default_rng(1004)
    r = 64
    per = {}
    for name, N, K in LLAMA_BLOCK:
        keep = only is None or name in only
        W0 = _normal(rng, (N, K), 0.02, "bf16")
        A = _normal(rng, (r, K), 1.0 / 8.0, "bf16")
        B = _normal(rng, (N, r), 0.01, "bf16")
        dY = _normal(rng, (8192, N), 1.0, "bf16")
        if keep:
            if M != 8192:
                dY = Tensor(dY.value[:M], "bf16")
            per[name] = dict(W0=W0, A=A, B=B, dY=dY, N=N, K=K)
        del W0, A, B, dY
    X = _normal(rng, (8192, 4096), 1.0, "bf16")
    X_down = _normal(rng, (8192, 11008), 1.0, "bf16")
    if M != 8192:
        X = Tensor(X.value[:M], "bf16")
        X_down = Tensor(X_down.value[:M], "bf16")
    return dict(proj=per, X=X, X_down=X_down, r=r, alpha=128.0)


def config5(n_requests: int = 256, max_tokens: int = 512, n_adapters: int = 4, K: int = 4096,
            N: int = 4096, seed: int = 1005):
    """Multi-adapter serving on one shared bf16 base: 4 adapters, r=16, alpha=32.

    256 requests with token counts uniform in [1, 512] and adapter ids uniform
    in {0..3}; tokens concatenated into one X with per-segment offsets.
    """
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, max_tokens + 1, n_requests)
    ids = rng.integers(0, n_adapters, n_requests)
    r = 16
    A = []
    B = []
    for _ in range(n_adapters):
        A.append(_normal(rng, (r, K), 0.02, "bf16"))
        B.append(_normal(rng, (N, r), 0.02, "bf16"))
    W0 = _normal(rng, (N, K), 0.02, "bf16")
    T = int(counts.sum())
    X = _normal(rng, (T, K), 1.0, "bf16")
    offsets = np.zeros(n_requests + 1, np.int32)
    offsets[1:] = np.cumsum(counts).astype(np.int32)
    A_stack = Tensor(np.stack([a.value for a in A]), "bf16")
    B_stack = Tensor(np.stack([b.value for b in B]), "bf16")
    return dict(W0=W0, A=A_stack, B=B_stack, X=X, offsets=offsets,
                adapter=ids.astype(np.int32), r=r, alpha=32.0)


def small_case(M, N, K, r, dtype="bf16", seed=7, sw=0.02, sa=None, sb=0.01, zero_b=False):
    """A small seeded case with the same value distributions as the workloads."""
    rng = np.random.default_rng(seed)
    sa = (1.0 / np.sqrt(r)) if sa is None else sa
    W0 = _normal(rng, (N, K), sw, dtype)
    A = _normal(rng, (r, K), sa, dtype)
    B = _normal(rng, (N, r), sb, dtype)
    X = _normal(rng, (M, K), 1.0, dtype)
    dY = _normal(rng, (M, N), 1.0, dtype)
    if zero_b:
        B = Tensor(np.zeros((N, r), np.float32), dtype)
    return dict(W0=W0, A=A, B=B, X=X, dY=dY, r=r, alpha=2.0 * r)


def device_normal(shape, sigma, seed, device):
    """A bf16 tensor ~ N(0, sigma^2) drawn on the device from a seeded torch
    generator: for inputs too large to draw and move from the host (the
    largest activation tensor the boundary accepts)."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device) * sigma).to(torch.bfloat16)


def config4_adapter_sizes(r: int = 64):
    """Element counts of the trainable A (r x K) and B (N x r) of config 4's
    seven projections, in block order: 14 tensors, 4,997,120 parameters."""
    out = []
    for _, N, K in LLAMA_BLOCK:
        out += [r * K, N * r]
    return out


def adamw_case(sizes, steps: int, seed: int = 11, zero_frac: float = 0.01):
    """Seeded state and gradients for AdamW steps on tensors of the given sizes.

    Per tensor i: a float32 master ~ N(0, 0.02^2) (the B and A scales of the
    workloads), then for every step a float32 gradient ~ N(0, sigma_i^2) with
    sigma_i cycling through 1e-3, 1e-2, 1e-1, 1 (so eps matters for some), of
    which a fraction ``zero_frac`` of entries is set exactly to 0.  Moments
    start at zero.  Returns (masters, grads) with grads[t][i] for step t + 1.
    """
    rng = np.random.default_rng(seed)
    sig = (1e-3, 1e-2, 1e-1, 1.0)
    masters = [rng.standard_normal(n, dtype=np.float32) * np.float32(0.02) for n in sizes]
    grads = []
    for _ in range(steps):
        gs = []
        for i, n in enumerate(sizes):
            g = rng.standard_normal(n, dtype=np.float32) * np.float32(sig[i % 4])
            g[rng.random(n) < zero_frac] = 0.0
            gs.append(g)
        grads.append(gs)
    return masters, grads


def dropout_keep_bits(M: int, K: int, p: float, seed: int = 23) -> np.ndarray:
    """A seeded dropout keep-mask for an M x K input, packed one bit per element
    (bit j of byte i is element 8 i + j of the row-major array; 1 = kept).
    Each element is kept independently with probability 1 - p."""
    rng = np.random.default_rng(seed)
    keep = rng.random(M * K) >= p
    return np.packbits(keep, bitorder="little")


def dora_magnitude(N: int, K: int, sigma_w: float = 0.02, seed: int = 29) -> np.ndarray:
    """A seeded DoRA magnitude vector (float32, one entry per output row):
    uniform in [0.5, 1.5] times sigma_w sqrt(K), the typical row norm of a
    weight drawn with standard deviation sigma_w."""
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.5, 1.5, N) * sigma_w * np.sqrt(K)).astype(np.float32)

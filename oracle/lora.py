"""LoRA adapted linear layer: forward, backward, merge, multi-adapter forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation (batched row form of the pages' column-vector formulas): X is M x K,
the frozen W0 is N x K (d_out x d_in), A is r x K, B is N x r, s = alpha / r,
Y is M x N.  Every product is float64 from the exact input values.

* Forward h = W0 x + (alpha/r) B A x ("LoRA and QLoRA: Mathematical
  Foundations ...", section "Initialization and the Scaling Factor" context and
  the forward-pass equation before it; the same formula in "LoRA and QLoRA
  fine-tuning under the hood", section 1.2, and "Lesson 26", section "The
  Decomposition").  Rows: Y = X W0^T + s (X A^T) B^T.
* Backward ("... Mathematical Foundations ...", section "Gradient Dynamics and
  Backpropagation Mechanics"): dL/dB = s (dL/dy)^T (A x)^T,
  dL/dA = s B^T (dL/dy)^T x^T, dL/dx = (W0 + s B A)^T (dL/dy)^T, summed over
  the rows of the batch; W0 gets no gradient.  The "LLMs part 08" page prints
  the adapter gradients without s; the chain rule on its own forward formula
  gives the factor, so s is included (finite differences pin it).
* Merge W_final = W0 + s B A ("... Mathematical Foundations ...", section
  "1. Static Weight Merging").
* Multi-adapter: each request i gets X_i W0^T + s (X_i A_{id_i}^T) B_{id_i}^T,
  the base term shared ("Large Language Model Fine-tuning and LoRA", section
  "Serving many adapters at once"; "... Mathematical Foundations ...", section
  "2. Multi-Tenant Dynamic Multiplexing").
* Trainable parameters per matrix r (d_in + d_out) ("Large Language Model
  Fine-tuning and LoRA", section "Choosing what to adapt: targets and rank").
* LoRA-input dropout ("Lesson 26", section "Putting It Together": the adapter
  configuration with lora_dropout = 0.05; the pages give the setting, not its
  definition).
  Reading: inverted dropout on the adapter branch's input only,
  D(X) = X * keep / (1 - p) with keep a 0/1 mask drawn by the caller, so
  Y = X W0^T + s (D(X) A^T) B^T and, by the chain rule, dX = dY W0 +
  s ((dY B) A) * keep / (1 - p), dA = s (dY B)^T D(X), dB = s dY^T (D(X) A^T).
  The mask arrives packed one bit per element of X in row-major order, bit j
  of byte i standing for element 8 i + j (1 = kept).
* DoRA ("Large Language Model Fine-tuning and LoRA", section "Choosing what to
  adapt": a trained magnitude vector of size d_out times a direction that gets
  the low-rank update on top of the frozen base direction; "... Mathematical
  Foundations ...", section "Advanced Variants: DoRA and LoRA+": W = m (V +
  dW) / ||V + dW||, written there with m in R^{1 x d_in} and a Frobenius
  norm).  The pages conflict on the size of m and on the norm.  Reading: m
  has one entry per output row (d_out, as the first page states) and the norm
  is the vector norm of each output row of V + dW, V = W0 and dW = s B A --
  the per-vector norm of the cited paper in the d_out x d_in layout used here;
  a whole-matrix Frobenius norm would make the normalisation one scalar and m
  no magnitude per vector.  So W' = diag(m / c) (W0 + s B A) with
  c_n = ||W0[n] + s B[n] A||_2 and Y = X W'^T.  Gradients are the exact chain
  rule through the norm (the pages do not detach it).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def lora_forward(X, W0, A, B, s):
    """Returns (Y, Y_base, T) with T = X A^T and Y_base = X W0^T."""
    X, W0, A, B = map(_f64, (X, W0, A, B))
    T = X @ A.T
    Y_base = X @ W0.T
    Y = Y_base + s * (T @ B.T)
    return Y, Y_base, T


def lora_backward(dY, X, W0, A, B, s):
    """Returns (dX, dA, dB) for the loss gradient dY = dL/dY (M x N)."""
    dY, X, W0, A, B = map(_f64, (dY, X, W0, A, B))
    U = dY @ B                      # (dL/dy) B, per row
    T = X @ A.T                     # A x, per row
    dX = dY @ W0 + s * (U @ A)
    dA = s * (U.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB


def lora_merge(W0, A, B, s):
    """W_final = W0 + s B A in float64."""
    W0, A, B = map(_f64, (W0, A, B))
    return W0 + s * (B @ A)


def lora_forward_multi(X, W0, A_stack, B_stack, s, offsets, adapter):
    """Segment i = rows offsets[i]:offsets[i+1] of X uses adapter adapter[i].

    A_stack[a] (r_a x K) and B_stack[a] (N x r_a) may differ in rank from one
    adapter to the next (the serving page's batches hold "adapters of
    different ranks"); ``s`` is one scale for all adapters or a sequence with
    adapter a's own alpha_a / r_a.
    """
    X, W0 = _f64(X), _f64(W0)
    Y = np.zeros((X.shape[0], W0.shape[0]), dtype=np.float64)
    for i in range(len(adapter)):
        lo, hi = int(offsets[i]), int(offsets[i + 1])
        if hi == lo:
            continue
        a = int(adapter[i])
        sa = s[a] if np.ndim(s) else s
        Y[lo:hi] = lora_forward(X[lo:hi], W0, A_stack[a], B_stack[a], sa)[0]
    return Y


def lora_num_params(N, K, r):
    """Trainable parameters LoRA adds to one N x K matrix at rank r."""
    return r * (K + N)


def trainable_params(layers, shapes, rank):
    """Sum of r (d_in + d_out) over the targeted matrices, times the layer count.

    ``shapes`` is a list of (d_out, d_in) for the targeted matrices of one layer.
    """
    return layers * sum(lora_num_params(d_out, d_in, rank) for d_out, d_in in shapes)


def merge_flops(N, K, r):
    """FLOPs of B @ A for one matrix, multiply-add counted as two."""
    return 2 * N * r * K


def forward_loop(X, W0, A, B, s):
    """Scalar pure-Python forward for tiny shapes (column-vector form per row)."""
    M, K = len(X), len(X[0])
    N, r = len(W0), len(A)
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        ax = [sum(float(A[j][k]) * float(X[m][k]) for k in range(K)) for j in range(r)]
        for n in range(N):
            base = sum(float(W0[n][k]) * float(X[m][k]) for k in range(K))
            bax = sum(float(B[n][j]) * ax[j] for j in range(r))
            Y[m][n] = base + s * bax
    return Y


def unpack_keep(bits, M, K):
    """Boolean M x K keep mask from its packed bits (bit j of byte i is element
    8 i + j of the row-major M x K array)."""
    b = np.asarray(bits, dtype=np.uint8).ravel()
    flat = np.zeros(M * K, dtype=bool)
    for e in range(M * K):
        flat[e] = (int(b[e // 8]) >> (e % 8)) & 1
    return flat.reshape(M, K)


def lora_forward_dropout(X, W0, A, B, s, keep, p):
    """Returns (Y, T) with T = D(X) A^T, D(X) = X * keep / (1 - p)."""
    X, W0, A, B = map(_f64, (X, W0, A, B))
    Xd = X * np.asarray(keep, dtype=np.float64) / (1.0 - p)
    T = Xd @ A.T
    Y = X @ W0.T + s * (T @ B.T)
    return Y, T


def lora_backward_dropout(dY, X, W0, A, B, s, keep, p):
    """Returns (dX, dA, dB) of the dropout forward for the loss gradient dY."""
    dY, X, W0, A, B = map(_f64, (dY, X, W0, A, B))
    kf = np.asarray(keep, dtype=np.float64) / (1.0 - p)
    Xd = X * kf
    U = dY @ B
    dX = dY @ W0 + s * ((U @ A) * kf)
    dA = s * (U.T @ Xd)
    dB = s * (dY.T @ (Xd @ A.T))
    return dX, dA, dB


def dora_forward(X, W0, A, B, s, m):
    """Returns (Y, Z, c): Z = X (W0 + s B A)^T, c the row norms, Y = Z * (m / c)."""
    X, W0, A, B, m = map(_f64, (X, W0, A, B, m))
    W = W0 + s * (B @ A)
    c = np.sqrt(np.sum(W * W, axis=1))
    Z = X @ W.T
    return Z * (m / c)[None, :], Z, c


def dora_backward(dY, X, W0, A, B, s, m):
    """Returns (dX, dA, dB, dm) of dora_forward for the loss gradient dY."""
    dY, X, W0, A, B, m = map(_f64, (dY, X, W0, A, B, m))
    W = W0 + s * (B @ A)
    c = np.sqrt(np.sum(W * W, axis=1))
    g = m / c
    Z = X @ W.T
    Gp = dY * g[None, :]               # gradient reaching Z
    h = np.sum(dY * Z, axis=0)         # gradient reaching g, per output row
    dm = h / c
    kappa = -h * m / c ** 3            # gradient reaching c, times 1 / c
    dW = Gp.T @ X + kappa[:, None] * W
    dX = Gp @ W
    dA = s * (B.T @ dW)
    dB = s * (dW @ A.T)
    return dX, dA, dB, dm

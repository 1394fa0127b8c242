"""AdamW update of the LoRA factors A and B, with float32 master weights and moments.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Large Language Model Fine-tuning and LoRA", section "The
real memory ledger: full fine-tuning vs LoRA vs QLoRA"; "Low-Rank Adaptation
(LoRA) and QLoRA: Mathematical Foundations ...", section "The Memory
Bottleneck of Full Fine-Tuning"): every trainable parameter carries a 16-bit
working weight, a 16-bit gradient, a float32 master weight and float32 first
and second moments m and v of AdamW, 16 bytes in all; the frozen base has
none of them.  The pages name AdamW but print no update rule.

Reading: the update is the decoupled-weight-decay Adam of Loshchilov and
Hutter ("Decoupled Weight Decay Regularization", ICLR 2019) in its common
form, for step t = 1, 2, ...:

    theta <- theta (1 - lr lambda)                (decay, decoupled from g)
    m     <- beta1 m + (1 - beta1) g
    v     <- beta2 v + (1 - beta2) g^2
    m_hat =  m / (1 - beta1^t),  v_hat = v / (1 - beta2^t)
    theta <- theta - lr m_hat / (sqrt(v_hat) + eps)

with g = grad_scale * gradient (grad_scale = 1/n folds the mean over n
accumulated micro-batches into the step).  The working weight is the
round-to-nearest-even 16-bit copy of the new master.

Precision: each step is computed in float64 from the stored float32 state
and the new state is rounded to float32, because the pages fix float32 as
the storage of master, m and v.
"""
from __future__ import annotations

import numpy as np

from . import nf4


def adamw_step(master, m, v, grad, t, lr, beta1, beta2, eps, weight_decay,
               grad_scale=1.0):
    """One AdamW step.  Returns the new (master, m, v) as float32 arrays.

    master, m, v: float32 arrays of one shape; grad: same shape, any float
    dtype (a bf16 gradient is passed as its exact float32 widening); t >= 1.
    """
    if t < 1:
        raise ValueError("step count t starts at 1")
    p = np.asarray(master, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64) * float(grad_scale)

    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p.astype(np.float32), m.astype(np.float32), v.astype(np.float32)


def working_copy_bf16_bits(master):
    """bf16 bit patterns (uint16) of the working copy: RNE of the float32 master."""
    return nf4.f32_to_bf16_bits(np.asarray(master, dtype=np.float32))

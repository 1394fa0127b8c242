"""Pins for the oracle's AdamW step on the adapter factors (CPU only).

The oracle's update is checked against things it does not compute itself:
PyTorch's own AdamW (an independent implementation of the same published
rule) run in float64, and closed forms -- a constant gradient moves every
weight by exactly lr g / (|g| + eps) per step once the moments are
bias-corrected, a zero gradient with decay scales the weight by
(1 - lr lambda)^t, and the first step's moments are (1 - beta1) g and
(1 - beta2) g^2.
"""
import numpy as np
import pytest
import torch

from oracle import optim

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def run_oracle(p0, grads, hp, grad_scale=1.0):
    p = p0.astype(np.float32)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for t, g in enumerate(grads, start=1):
        p, m, v = optim.adamw_step(p, m, v, g, t, grad_scale=grad_scale, **hp)
    return p, m, v


@pytest.mark.parametrize("wd", [0.0, 0.01, 0.1])
def test_matches_torch_adamw_float64(wd):
    rng = np.random.default_rng(3)
    hp = dict(HP, weight_decay=wd)
    p0 = rng.standard_normal(257).astype(np.float32) * 0.02
    grads = [rng.standard_normal(257).astype(np.float32) for _ in range(6)]
    p, m, v = run_oracle(p0, grads, hp)

    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]),
                            eps=hp["eps"], weight_decay=wd)
    for g in grads:
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        # the oracle stores float32 state between steps; do the same here
        with torch.no_grad():
            tp.copy_(tp.to(torch.float32).to(torch.float64))
        st = opt.state[tp]
        st["exp_avg"].copy_(st["exp_avg"].to(torch.float32).to(torch.float64))
        st["exp_avg_sq"].copy_(st["exp_avg_sq"].to(torch.float32).to(torch.float64))
    st = opt.state[tp]
    # Both compute in float64 and store float32; their float64 operation
    # orders differ (PyTorch forms m by interpolation), which can move a
    # stored value by one float32 step of its operands, and such a step is
    # carried into later steps.  A wrong term would differ by the size of
    # the values themselves.
    for mine, theirs in ((p, tp.detach().numpy()), (m, st["exp_avg"].numpy()),
                         (v, st["exp_avg_sq"].numpy())):
        theirs = theirs.astype(np.float32)
        tol = 4 * np.spacing(np.abs(theirs).max())
        assert np.abs(mine.astype(np.float64) - theirs).max() <= tol
    assert np.mean(p == tp.detach().numpy().astype(np.float32)) > 0.95


def test_constant_gradient_closed_form():
    # With g fixed, m_t = (1 - beta1^t) g and v_t = (1 - beta2^t) g^2, so the
    # bias-corrected ratio is g / |g| and each step moves theta by
    # lr g / (|g| + eps) (no decay).
    rng = np.random.default_rng(5)
    hp = dict(HP, weight_decay=0.0)
    p0 = rng.standard_normal(64).astype(np.float32)
    g = rng.standard_normal(64).astype(np.float32)
    t = 7
    p, _, _ = run_oracle(p0, [g] * t, hp)
    g64 = g.astype(np.float64)
    want = p0.astype(np.float64) - t * hp["lr"] * g64 / (np.abs(g64) + hp["eps"])
    # float32 storage rounds once per step
    np.testing.assert_allclose(p, want, rtol=0, atol=t * 2.0 ** -23 * 4 + 1e-9)


def test_zero_gradient_is_pure_decay():
    hp = dict(HP, weight_decay=0.1, lr=0.01)
    p0 = np.linspace(-1, 1, 33).astype(np.float32)
    t = 5
    p, m, v = run_oracle(p0, [np.zeros(33, np.float32)] * t, hp)
    want = p0.astype(np.float64) * (1 - hp["lr"] * hp["weight_decay"]) ** t
    np.testing.assert_allclose(p, want, rtol=4e-7 * t, atol=0)
    assert not m.any() and not v.any()


def test_first_step_moments_and_grad_scale():
    rng = np.random.default_rng(9)
    g = rng.standard_normal(50).astype(np.float32)
    p0 = np.zeros(50, np.float32)
    _, m, v = run_oracle(p0, [g], HP, grad_scale=0.25)
    gs = 0.25 * g.astype(np.float64)
    np.testing.assert_allclose(m, (1 - HP["beta1"]) * gs, rtol=1e-7)
    np.testing.assert_allclose(v, (1 - HP["beta2"]) * gs * gs, rtol=1e-7)


def test_step_count_starts_at_one():
    z = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        optim.adamw_step(z, z, z, z, 0, **HP)


def test_working_copy_is_nearest_bf16():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    bits = optim.working_copy_bf16_bits(x)
    # ties to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 -> 1;
    # 1 + 3*2^-8 halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6 (even)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82
    assert bits[3] == 0xC020
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert abs(back[4] - x[4]) <= 2.0 ** -8 * abs(x[4])  # half a bf16 step

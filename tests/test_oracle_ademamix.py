"""Pins of the oracle's AdEMAMix step.  The rule is the one the bitsandbytes
PR 'Fix decoupled weight decay ordering in the CUDA Adam/AdEMAMix kernels'
cites (Pagliardini et al.): m1 and v bias-corrected, the slow EMA m2 not,
u = (m1_hat + alpha*m2) / (sqrt(v_hat) + eps), decay-first.  The PR's
'Why the current tests do not catch it' gives its step-1 form: the AdamW form
plus alpha*(1-b3)*g in the numerator."""
import numpy as np
import pytest

import synth
from tests.common import ULP1, f64, run_oracle

N = 4099
HP = dict(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8)


def test_step1_closed_form():
    p0 = synth.params(N)
    g = synth.grads(N, 1)
    g[:3] = [0.0, 1e-12, -2.0]
    p, _ = run_oracle("ademamix", "f32", N, 1, HP, grad_fn=lambda t: g, p=p0.copy())
    lr, wd, a, b3 = (f64(np.float32(HP[k])) for k in ("lr", "weight_decay", "alpha", "beta3"))
    om3 = f64(np.float32(1) - np.float32(HP["beta3"]))
    ref = f64(p0) * (1 - lr * wd) - lr * (1 + a * om3) * f64(g) / (np.abs(f64(g)) + 1e-8)
    tol = 8 * ULP1 * (np.abs(f64(p0)) + lr * (1 + a * om3))
    assert np.all(np.abs(f64(p) - ref) <= tol)


def test_constant_gradient_closed_form():
    """Same g every step: m1_hat = g, v_hat = g^2 and m2_t = (1-b3^t) g, so
    step t moves p by lr (1 + alpha (1 - b3^t)) g/(|g|+eps).  A small b3 makes
    the slow EMA's recursion visible within a few steps."""
    T = 25
    hp = dict(HP, beta3=0.8, alpha=2.0, lr=1e-2)
    p0 = synth.params(N)
    g = synth.grads(N, 1)
    p, _ = run_oracle("ademamix", "f32", N, T, hp, grad_fn=lambda t: g, p=p0.copy())
    lr, wd, a, b3 = (f64(np.float32(hp[k])) for k in ("lr", "weight_decay", "alpha", "beta3"))
    d = 1 - lr * wd
    u = f64(g) / (np.abs(f64(g)) + 1e-8)
    ref = f64(p0)
    for t in range(1, T + 1):
        ref = ref * d - lr * (1 + a * (1 - b3 ** t)) * u
    tol = sum(lr * (1 + a) * (2 * t + 12) * ULP1 for t in range(1, T + 1)) + T * 4 * ULP1 * np.abs(f64(p0))
    assert np.all(np.abs(f64(p) - ref) <= tol)


def test_zero_betas_every_step_is_sign_step():
    """b1 = b2 = 0 and alpha = 0: m1' = g and v' = g^2 each step and
    c1 = c2 = 1, so every step is p d - lr g / (|g| + eps) with fresh g."""
    T = 6
    hp = dict(HP, beta1=0.0, beta2=0.0, alpha=0.0)
    p0 = synth.params(N)
    p, _ = run_oracle("ademamix", "f32", N, T, hp, p=p0.copy())
    ref = f64(p0)
    lr, wd = f64(np.float32(hp["lr"])), f64(np.float32(hp["weight_decay"]))
    for t in range(1, T + 1):
        g = f64(synth.grads(N, t))
        ref = ref * (1 - lr * wd) - lr * g / (np.abs(g) + 1e-8)
    assert np.all(np.abs(f64(p) - ref) <= T * 8 * ULP1 * (np.abs(ref) + lr))


@pytest.mark.parametrize("beta3", [0.9999, 0.5])
def test_alpha_zero_is_adamw(beta3):
    """With alpha = 0 the slow EMA does not reach the update: p, m and v are
    bit-identical to AdamW for any b3."""
    T, n = 8, 65537
    hp = dict(HP, alpha=0.0, beta3=beta3)
    pa, sa = run_oracle("ademamix", "f32", n, T, hp)
    pb, sb = run_oracle("adamw", "f32", n, T, {k: v for k, v in hp.items() if k not in ("alpha", "beta3")})
    assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))
    assert np.array_equal(sa["s1"].view(np.uint32), sb["s1"].view(np.uint32))
    assert np.array_equal(sa["s2"].view(np.uint32), sb["s2"].view(np.uint32))

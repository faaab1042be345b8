"""Pins of the oracle's update-norm pre-pass (the precondition pass of the
issue 'Investigate SM103 bias-correction broadcast in 32-bit optimizers',
Problem; accumulation in fp64 as in the NeMo PR 'perf(training): fused
multi-tensor gradient-norm reduction', Numerics) and of the scale
min(1, max_unorm * ||p|| / ||u||)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.common import f64, run_oracle


def test_param_norm_is_exact_sum():
    """sum p^2 against the exact rational sum, rounded once."""
    n = 5000
    p = synth.params(n)
    p[:4] = [3e4, -1e-20, 7.0, -3e4]          # cancellation-prone magnitudes
    g = synth.grads(n, 1)
    st = oracle.state_zeros("f32", n)
    _, p2 = oracle.unorm("adamw", "f32", oracle.make_hp(), p, g, **st)
    exact = sum(Fraction(float(x)) ** 2 for x in p)
    assert p2 == float(exact)


def test_update_norm_of_sign_steps_is_count():
    """b1 = b2 = 0, eps = 0: u = g/|g| = +-1 exactly, so sum u^2 = n."""
    n = 3001
    g = np.where(synth.grads(n, 1) >= 0, 1.0, -1.0).astype(np.float32) * np.float32(2.0 ** -5)
    st = oracle.state_zeros("f32", n)
    u2, _ = oracle.unorm("adamw", "f32", oracle.make_hp(beta1=0.0, beta2=0.0, eps=0.0),
                         synth.params(n), g, **st)
    assert u2 == float(n)


def test_step1_scale_closed_form():
    """At step 1 u = g/(|g|+eps), so the scale is max_unorm*||p||/||u||."""
    n, mu = 1 << 16, 1.0
    p = synth.params(n)
    g = synth.grads(n, 1)
    st = oracle.state_zeros("f32", n)
    hp = oracle.make_hp(max_unorm=mu)
    u2, p2 = oracle.unorm("adamw", "f32", hp, p, g, **st)
    u = f64(g) / (np.abs(f64(g)) + 1e-8)
    ref = mu * np.sqrt((f64(p) ** 2).sum()) / np.sqrt((u ** 2).sum())
    s = oracle.unorm_scale(mu, u2, p2)
    assert ref < 1 and abs(s - ref) <= 1e-6 * ref
    assert abs(s - 0.02) < 0.001          # ||p|| ~ 0.02 sqrt(n), ||u|| ~ sqrt(n)


def test_scale_special_cases():
    assert oracle.unorm_scale(0.0, 4.0, 1.0) == 1.0        # off
    assert oracle.unorm_scale(-1.0, 4.0, 1.0) == 1.0       # off
    assert oracle.unorm_scale(1e30, 4.0, 1.0) == 1.0       # bound never reached
    assert oracle.unorm_scale(1.0, 0.0, 1.0) == 1.0        # ||u|| = 0
    assert oracle.unorm_scale(1.0, 4.0, 0.0) == 0.0        # ||p|| = 0, ||u|| > 0
    assert oracle.unorm_scale(0.5, 4.0, 1.0) == np.float32(0.25)


@pytest.mark.parametrize("mu", [0.0, 1e30])
def test_inactive_bound_is_plain_step(mu):
    """A scale of 1 reproduces the plain step bit for bit."""
    n, T = 4099, 5
    hp = dict(lr=1e-3, weight_decay=0.1, max_unorm=mu)

    def scale(h, p, g, st):
        return oracle.unorm_scale(h.max_unorm, *oracle.unorm("adamw", "f32", h, p, g, **st))
    pa, sa = run_oracle("adamw", "f32", n, T, hp, scale_fn=scale)
    pb, sb = run_oracle("adamw", "f32", n, T, dict(lr=1e-3, weight_decay=0.1))
    assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))


def test_active_bound_scales_only_the_update():
    """Scale s multiplies lr*u only; the decay keeps 1 - lr*wd.  Step 1:
    p1 = p0 d - lr s g/(|g|+eps)."""
    n = 4099
    p0 = synth.params(n)
    g = synth.grads(n, 1)
    st = oracle.state_zeros("f32", n)
    hp = oracle.make_hp(lr=1e-3, weight_decay=0.1, max_unorm=1.0)
    s = oracle.unorm_scale(1.0, *oracle.unorm("adamw", "f32", hp, p0, g, **st))
    p = p0.copy()
    oracle.step("adamw", "f32", hp, p, g, scale=s, **st)
    lam = f64(np.float32(np.float32(1e-3) * np.float32(s)))
    ref = f64(p0) * (1 - f64(np.float32(1e-3)) * f64(np.float32(0.1))) - lam * f64(g) / (np.abs(f64(g)) + 1e-8)
    assert np.all(np.abs(f64(p) - ref) <= 8 * 2.0 ** -24 * (np.abs(f64(p0)) + lam))

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


# ---------------------------------------------------------------------------
# The pre-pass over every stored format.  The pre-pass reads the states the
# way the step does ([PR] Verification: the 32-bit and 8-bit kernels start
# from the same values), so over stored states it must equal the fp32 pre-pass
# over those states read back.  The read-back below is written independently
# of the oracle: BF16 words widened by a shift, 8-bit codes as codebook entry
# times block absmax in binary32, FP8 values from torch's float8_e4m3fn and
# the 4-bit grids from their value lists, times 2^(floor(log2 A) - emax)
# ("When Small Updates Disappear", Sec. 2.1; microscaling block scale).

QS, QU = synth.codebook_signed(), synth.codebook_unsigned()
E2M1_VALUES = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
E2M2U_VALUES = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7], dtype=np.float64)


def _e4m3_values():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _block_scaled(codes, amax, n, grid, emax, sign_bit, nibbles):
    """Element values of a block-scaled FP8/FP4 state, in binary32."""
    c = np.asarray(codes, dtype=np.uint8)
    if nibbles:
        c = np.stack([c & 0xF, c >> 4], axis=1).reshape(-1)[:n]
    c = c.astype(np.int64)
    mag = c & (sign_bit - 1) if sign_bit else c
    neg = (c & sign_bit) != 0 if sign_bit else np.zeros(n, bool)
    A = np.repeat(np.asarray(amax, np.float64), 256)[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(A > 0, A, 1.0)))
    val = np.abs(grid[mag]) * np.exp2(e - emax)      # exact in binary64
    val = np.where(A > 0, val, 0.0)
    val = np.where(np.isfinite(A) & ~np.isnan(grid[mag]), val, np.nan)
    out = val.astype(np.float32)                      # one rounding to binary32
    return np.where(neg, -out, out).astype(np.float32)


def _read_back(fmt, st, n):
    """fp32 values of the stored states s1, s2 (and s3), as the step reads them."""
    keys = [k for k in ("s1", "s2", "s3") if k in st]
    out = {}
    for k in keys:
        v_state = k == "s2"
        a = st.get("a" + k[1:])
        if fmt == "f32":
            out[k] = st[k].copy()
        elif fmt.startswith("bf16"):
            out[k] = (st[k].astype(np.uint32) << 16).view(np.float32)
        elif fmt == "q8":
            T = QU if v_state else QS
            out[k] = (T[st[k]] * np.repeat(a, 256)[:n]).astype(np.float32)
        elif fmt.startswith("fp8"):
            out[k] = _block_scaled(st[k], a, n, _e4m3_values(), 8, 0x80, False)
        else:
            grid = E2M2U_VALUES if v_state else E2M1_VALUES
            out[k] = _block_scaled(st[k], a, n, grid, 2, 0 if v_state else 0x8, True)
    return out


@pytest.mark.parametrize("skip_zeros", [False, True], ids=["plain", "skip_zeros"])
@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("fmt", ["bf16_rn", "bf16_sr", "q8", "fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr"])
def test_prepass_over_stored_states_is_fp32_prepass_of_read_back(fmt, opt, skip_zeros):
    """sum u^2 and sum p^2 over stored states == the fp32 pre-pass over the
    same states read back, bit for bit; and the read-back itself is what the
    stored format holds (no element of an fp32 reading is off the format)."""
    n, T = 5 * 256 + 77, 4
    hp = dict(lr=1e-2, weight_decay=0.01, beta1=0.9, beta2=0.99, beta3=0.999, alpha=5.0,
              skip_zeros=skip_zeros)
    zero = np.zeros(n, bool)
    zero[256:512] = True                 # a block whose gradients are all zero
    zero[900::37] = True

    def grads(t):
        g = synth.grads(n, t, std=1e-3)
        g[256:260] = [1e-2, -3e-2, 2e-5, -7e-6]
        if skip_zeros:
            g = np.where(zero, np.float32(-0.0) if t % 2 else np.float32(0.0), g).astype(np.float32)
        return synth.bf16_words(g)

    p, st = run_oracle(opt, fmt, n, T, hp, grad_fn=grads, qs=QS, qu=QU, seed=11)
    g = grads(T + 1)
    h = oracle.make_hp(step=T + 1, seed=11, **hp)
    got = oracle.unorm(opt, fmt, h, p, g, qs=QS, qu=QU, **st)
    f32 = _read_back(fmt, st, n)
    want = oracle.unorm(opt, "f32", h, p, g, **f32)
    assert got == want
    assert np.isfinite(got[0]) and got[0] > 0
    # the read-back is not degenerate: every state holds distinct nonzero values
    for k, v in f32.items():
        assert np.count_nonzero(v) > n // 2 and np.unique(v).size > 8, k

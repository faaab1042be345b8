"""Pins of the oracle's BF16 state storage: nearest rounding against torch's
library cast; stochastic rounding against the exact facts of 'When Small
Updates Disappear' (Sec. 3, 3.1, 3.3, 6.1); the BF16 second moment that cannot
fall under nearest rounding (Sec. 2.2); and the stall-probability model of
Sec. 2.3 and 3.2, whose printed figures the oracle's measured one-step stall
fractions must reproduce."""
import math

import numpy as np
import pytest
import torch
from scipy import integrate, stats

import oracle
import synth
from tests.common import f64, run_oracle


def _torch_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _compare_rne(bits):
    x = bits.view(np.float32)
    got = oracle.bf16_rne_array(x)
    ref = _torch_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # a NaN stays a NaN with its sign
    g = oracle.widen_bf16(got[nan])
    assert np.all(np.isnan(g)) and np.array_equal(np.signbit(g), np.signbit(x[nan]))


def test_rne_matches_torch_cast_all_high_halves():
    """Every high half (all signs, exponents, kept fractions, NaN and inf)
    with the dropped half at the tie and next to it."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000):
        _compare_rne(hi | np.uint32(lo))


def test_rne_matches_torch_cast_random_words():
    rng = np.random.default_rng(11)
    _compare_rne(rng.integers(0, 2**32, 2**22, dtype=np.uint64).astype(np.uint32))


ALL_R = np.arange(65536, dtype=np.uint32)


def test_sr_keeps_representable_values():
    """SR of an exactly representable BF16 value returns that same word for
    each of the 2^16 random integers ("When Small Updates Disappear", Sec. 3:
    no dropped bits, so no carry)."""
    rng = np.random.default_rng(3)
    words = np.concatenate([rng.integers(0, 65536, 300), [0, 0x8000, 0x7F7F, 0xFF7F, 1, 0x8001, 0x3F80]])
    for w in words.astype(np.uint16):
        x = oracle.widen_bf16(np.array([w]))[0]
        out = oracle.bf16_sr_array(np.full(65536, x, dtype=np.float32), ALL_R)
        assert np.all(out == w)


def _finite_samples(count, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 2**32, 4 * count, dtype=np.uint64).astype(np.uint32)
    x = b.view(np.float32)
    keep = np.isfinite(x) & (np.abs(x) < np.float32(3.0e38)) & ((b & 0xFFFF) != 0)
    return x[keep][:count]


def test_sr_unbiased_and_carry_count():
    """Over all 2^16 values of r: the mean of the results is x exactly
    (Sec. 3.1), the number of carries is the dropped integer l (Sec. 6.1), and
    the mean squared error is (x - q-)(q+ - x) (Sec. 3.1)."""
    for x in _finite_samples(120, 5):
        out = oracle.bf16_sr_array(np.full(65536, x, dtype=np.float32), ALL_R)
        vals = f64(oracle.widen_bf16(out))
        assert vals.sum() == 65536.0 * f64(x)
        bits = np.float32(x).view(np.uint32)
        l = int(bits & 0xFFFF)
        kept = np.uint16(bits >> 16)
        assert int(np.count_nonzero(out != kept)) == l
        qm = f64(oracle.widen_bf16(np.array([kept])))[0]
        qp = f64(oracle.widen_bf16(np.array([kept + 1])))[0]
        var = np.mean((vals - f64(x)) ** 2)
        assert math.isclose(var, (f64(x) - qm) * (qp - f64(x)), rel_tol=1e-12) if qm != f64(x) else var == 0


def test_sr_fraction_across_examples(golden):
    """A value 30% (20%) of the way across the gap rounds up 30% (20%) of the
    time; an update of 0.2u stays put under nearest rounding (Sec. 3, 3.3)."""
    for frac, up in golden("rounding_examples.json")["fraction_across_rounds_up"]:
        l = int(round(frac * 65536))
        x = np.array([(0x3F81 << 16) | l], dtype=np.uint32).view(np.float32)[0]
        out = oracle.bf16_sr_array(np.full(65536, x, dtype=np.float32), ALL_R)
        assert abs(np.count_nonzero(out != 0x3F81) / 65536 - up) < 1e-4
        assert oracle.bf16_rne_array(np.array([x]))[0] == (0x3F81 if frac < 0.5 else 0x3F82)


def test_sr_special_values():
    for w in (0x7F800000, 0xFF800000, 0x7FC00001, 0xFFC12345):
        x = np.array([w], dtype=np.uint32).view(np.float32)
        out = oracle.bf16_sr_array(np.repeat(x, 64), np.arange(64, dtype=np.uint32) * 1021)
        ref = oracle.bf16_rne_array(x)[0]
        assert np.all(out == ref)


def _v_bits_never_fall(beta2, steps, grad_std_fn, n=65536):
    st = oracle.state_zeros("bf16_rn", n)
    p = synth.params(n)
    prev = None
    falls = 0
    for t in range(1, steps + 1):
        g = synth.grads(n, t, std=grad_std_fn(t), bf16=True)
        hp = oracle.make_hp(lr=1e-3, weight_decay=0.01, beta2=beta2, step=t)
        oracle.step("adamw", "bf16_rn", hp, p, g, **st)
        v = oracle.widen_bf16(st["s2"])
        if prev is not None:
            falls += int(np.count_nonzero(v < prev))
        prev = v.copy()
    return falls


def test_bf16_second_moment_never_falls_under_rn():
    """beta2 = 0.999 < 1 - 1/512: under nearest rounding no stored v ever
    decreases, even as the gradient scale decays 100x over 200 steps."""
    assert _v_bits_never_fall(0.999, 200, lambda t: synth.decaying_std(t)) == 0


@pytest.mark.parametrize("factor,falls", [(0.9, False), (1.1, True), (5.0, True)])
def test_bf16_monotone_threshold(golden, factor, falls):
    """Sec. 2.2: the argument needs 1 - beta2 < 1/512.  With g = 0 after a
    warm-up, 1 - beta2 = 0.9/512 leaves every v in place; 1.1/512 lets the
    values with a large mantissa fall."""
    thr = golden("rounding_examples.json")["bf16_monotone_threshold"]
    assert thr == 1 / 512
    beta2 = float(np.float32(1 - factor * thr))
    n = 65536
    st = oracle.state_zeros("bf16_rn", n)
    p = synth.params(n)
    v_before = None
    for t in range(1, 4):
        g = synth.grads(n, t, bf16=True) if t == 1 else np.zeros(n, dtype=np.uint16)
        oracle.step("adamw", "bf16_rn", oracle.make_hp(beta2=beta2, step=t), p, g, **st)
        v = oracle.widen_bf16(st["s2"])
        if t >= 2:
            assert (np.count_nonzero(v < v_before) > 0) == falls
        v_before = v.copy()


# ---------------------------------------------------------------------------
# stall model

def _rho(p_bits, beta2):
    return 2.0 ** -p_bits * math.log(2) / (2 * (1 - beta2))


def model_rn(p_bits, beta2):
    """P(|z - 1| < rho), z ~ chi^2_1 (Sec. 2.3)."""
    r = _rho(p_bits, beta2)
    return stats.chi2.cdf(1 + r, 1) - stats.chi2.cdf(max(0.0, 1 - r), 1)


def model_sr(p_bits, beta2):
    """E[(1 - |z - 1| / (2 rho))_+], z ~ chi^2_1 (Sec. 3.2)."""
    r = _rho(p_bits, beta2)
    f = lambda z: max(0.0, 1 - abs(z - 1) / (2 * r)) * stats.chi2.pdf(z, 1)
    lo, hi = max(0.0, 1 - 2 * r), 1 + 2 * r
    pts = [1.0] if lo < 1 < hi else None
    return integrate.quad(f, lo, hi, points=pts, limit=200)[0]


def test_stall_model_reproduces_printed_figures(golden):
    gold = golden("stall_model.json")
    b2, bits, pr = gold["beta2"], gold["fraction_bits"], gold["printed_percent"]
    tol = gold["printed_precision_pp"] + 1e-9
    assert abs(100 * model_rn(bits["bf16"], b2) - pr["bf16_rn"]) <= tol
    assert abs(100 * model_sr(bits["bf16"], b2) - pr["bf16_sr"]) <= tol
    assert abs(100 * model_sr(bits["fp8"], b2) - pr["fp8_sr"]) <= tol
    assert abs(100 * model_sr(bits["fp4"], b2) - pr["fp4_sr"]) <= tol
    assert 100 * model_rn(bits["fp8"], b2) > 99.9 and 100 * model_rn(bits["fp4"], b2) > 99.9


def _one_step_stall(fmt, n=1 << 20, beta2=0.999):
    """One step from a typical state v = RNE(sigma^2), g ~ N(0, sigma), sigma
    log-uniform over [1e-3, 1e-2]; stalled = the stored v word is unchanged."""
    rng = np.random.default_rng(21)
    sigma = (10.0 ** rng.uniform(-3, -2, n)).astype(np.float32)
    g = (rng.standard_normal(n).astype(np.float32) * sigma).astype(np.float32)
    st = oracle.state_zeros(fmt, n)
    st["s2"][:] = oracle.bf16_rne_array(sigma * sigma)
    v0 = st["s2"].copy()
    p = np.zeros(n, dtype=np.float32)
    hp = oracle.make_hp(beta2=beta2, step=1000, seed=synth.SR_SEED)
    oracle.step("adamw", fmt, hp, p, g, **st)
    return np.mean(st["s2"] == v0)


@pytest.mark.parametrize("fmt,model", [("bf16_rn", model_rn), ("bf16_sr", model_sr)])
def test_oracle_stall_fraction_matches_model(fmt, model):
    measured = _one_step_stall(fmt)
    assert abs(measured - model(7, 0.999)) < 0.01


def test_stall_fraction_detects_wrong_rounding():
    """Non-vacuity: nearest and stochastic rounding differ by ~12 pp here."""
    assert _one_step_stall("bf16_rn") - _one_step_stall("bf16_sr") > 0.1


# ---------------------------------------------------------------------------
# the BF16 step is the fp32 step followed by rounding of the stored moments

def _f32_step_from(m_words, v_words, p, g, hp):
    st = {"s1": oracle.widen_bf16(m_words).copy(), "s2": oracle.widen_bf16(v_words).copy()}
    oracle.step("adamw", "f32", hp, p, g, **st)
    return st


def test_bf16_rn_step_is_f32_step_then_library_cast():
    n = 4099
    rng = np.random.default_rng(8)
    m0 = _torch_bf16(rng.standard_normal(n).astype(np.float32) * 1e-3)
    v0 = _torch_bf16(np.abs(rng.standard_normal(n)).astype(np.float32) * 1e-5)
    p0 = synth.params(n)
    g = synth.grads(n, 3, bf16=True)
    hp = oracle.make_hp(lr=1e-3, weight_decay=0.01, step=3)
    ref_p = p0.copy()
    ref = _f32_step_from(m0, v0, ref_p, g, hp)
    p = p0.copy()
    st = {"s1": m0.copy(), "s2": v0.copy()}
    oracle.step("adamw", "bf16_rn", hp, p, g, **st)
    assert np.array_equal(p.view(np.uint32), ref_p.view(np.uint32))
    assert np.array_equal(st["s1"], _torch_bf16(ref["s1"]))
    assert np.array_equal(st["s2"], _torch_bf16(ref["s2"]))


def test_bf16_sr_step_uses_element_words():
    """m takes the low and v the high 16 bits of the element's Philox word;
    rounding adds r to the fp32 word and keeps the high half (Sec. 6.1)."""
    n, k, t, j0 = 4099, 3, 7, 1 << 20
    rng = np.random.default_rng(9)
    m0 = _torch_bf16(rng.standard_normal(n).astype(np.float32) * 1e-3)
    v0 = _torch_bf16(np.abs(rng.standard_normal(n)).astype(np.float32) * 1e-5)
    p0 = synth.params(n)
    g = synth.grads(n, t, bf16=True)
    hp = oracle.make_hp(step=t, seed=synth.SR_SEED, tensor_index=k, index_base=j0)
    ref = _f32_step_from(m0, v0, p0.copy(), g, hp)
    w = oracle.sr_words(synth.SR_SEED, t, k, j0, n)
    exp_m = ((ref["s1"].view(np.uint32).astype(np.uint64) + (w & 0xFFFF)) >> 16).astype(np.uint16)
    exp_v = ((ref["s2"].view(np.uint32).astype(np.uint64) + (w >> 16)) >> 16).astype(np.uint16)
    st = {"s1": m0.copy(), "s2": v0.copy()}
    oracle.step("adamw", "bf16_sr", hp, p0.copy(), g, **st)
    assert np.array_equal(st["s1"], exp_m) and np.array_equal(st["s2"], exp_v)

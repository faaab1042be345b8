"""Pins of the oracle's gradient norms (NeMo Automodel PR 'perf(training):
fused multi-tensor gradient-norm reduction', Numerics and Correctness
properties) against exact rational sums, and of the fused clipping scale."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.common import run_oracle


def _exact_sumsq(x):
    return sum(Fraction(float(v)) ** 2 for v in np.asarray(x, dtype=np.float64))


def _bf16_with_range(n, seed, lo_exp=-10):
    """BF16 words whose magnitudes lie in [2^lo_exp, 1): their squares carry
    16 significant bits above 2^(2*lo_exp - 16), so sums of up to 2^(53-16+2*lo_exp+...)
    of them are exact in binary64."""
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(lo_exp, 0, n) * np.where(rng.random(n) < 0.5, -1, 1)
    return synth.bf16_words(mag.astype(np.float32))


def test_bf16_sum_is_exact(golden):
    """'exact for BF16': binary64 sums of squared BF16 gradients with a
    realistic dynamic range are the exact rational sums."""
    assert golden("grad_norm.json")["bf16_relative_error"] == 0.0
    g = _bf16_with_range(20000, 1)
    s, m = oracle.grad_norm(g)
    gf = oracle.widen_bf16(g)
    assert Fraction(s) == _exact_sumsq(gf)
    assert m == float(np.abs(gf.astype(np.float64)).max())


def test_fp32_sum_within_page_bound(golden):
    bound = golden("grad_norm.json")["fp32_relative_error"]
    g = synth.grads(20000, 1, std=1e-2)
    g[:3] = [3e3, -1e-30, 7.5]
    s, _ = oracle.grad_norm(g)
    ex = _exact_sumsq(g)
    assert abs(Fraction(s) - ex) <= Fraction(bound) * ex


def test_list_total_over_2000_tensors(golden):
    bound = golden("grad_norm.json")["tensors_2000_relative_error"]
    rng = np.random.default_rng(4)
    grads = [synth.grads(int(n), 1, k, std=float(10.0 ** rng.uniform(-4, 0)))
             for k, n in enumerate(rng.integers(1, 300, 2000))]
    (s, m), per = oracle.grad_norm_list(grads)
    ex = sum(_exact_sumsq(g) for g in grads)
    assert abs(Fraction(s) - ex) <= Fraction(bound) * ex
    assert m == max(float(np.abs(g.astype(np.float64)).max()) for g in grads)


def test_nan_poisons_both_norms_and_inf_propagates():
    g = synth.grads(1000, 1)
    g[10] = np.nan
    s, m = oracle.grad_norm(g)
    assert np.isnan(s) and np.isnan(m)
    g = synth.grads(1000, 1)
    g[10] = -np.inf
    s, m = oracle.grad_norm(g)
    assert s == np.inf and m == np.inf
    (s, m), _ = oracle.grad_norm_list([synth.grads(10, 1), g, np.array([np.nan], np.float32)])
    assert np.isnan(m)


def test_empty_and_zero():
    assert oracle.grad_norm(np.zeros(0, np.float32)) == (0.0, 0.0)
    assert oracle.grad_norm(np.zeros(7, np.float32)) == (0.0, 0.0)


@pytest.mark.parametrize("norm,max_norm,expect", [
    (5.0, 1.0, 1.0 / (5.0 + 1e-6)), (0.5, 1.0, 1.0), (0.0, 1.0, 1.0), (np.inf, 1.0, 0.0)])
def test_clip_coefficient(norm, max_norm, expect):
    assert oracle.clip_coef(norm, max_norm) == np.float32(expect)
    assert np.isnan(oracle.clip_coef(np.nan, 1.0))


def test_fused_scale_equals_prescaled_gradient():
    """The step with grad_scale s equals the step on fl(g * s) computed
    outside (fp32 gradients), bit for bit, over several steps."""
    n, T, s = 4099, 4, np.float32(0.37)
    p0 = synth.params(n)
    pa, sa = run_oracle("adamw", "f32", n, T, dict(lr=1e-3, weight_decay=0.1, grad_scale=float(s)),
                        p=p0.copy())
    pb, sb = run_oracle("adamw", "f32", n, T, dict(lr=1e-3, weight_decay=0.1), p=p0.copy(),
                        grad_fn=lambda t: (synth.grads(n, t) * s).astype(np.float32))
    assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))
    assert np.array_equal(sa["s2"].view(np.uint32), sb["s2"].view(np.uint32))


def test_unit_scale_is_identity():
    n = 4099
    pa, _ = run_oracle("ademamix", "q8", n, 3, dict(lr=1e-3, grad_scale=1.0), qs=synth.codebook_signed(),
                       qu=synth.codebook_unsigned())
    pb, _ = run_oracle("ademamix", "q8", n, 3, dict(lr=1e-3), qs=synth.codebook_signed(),
                       qu=synth.codebook_unsigned())
    assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))

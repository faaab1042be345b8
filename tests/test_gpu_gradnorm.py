"""GPU parity of the fused multi-tensor gradient norm and of the clipping
coefficient it feeds into the step (NeMo Automodel PR "perf(training): fused
multi-tensor gradient-norm reduction").

Bars: the inf-norm (a max) is bit-exact; squares of float32 or BF16 values are
exact in binary64, so the only error of a sum of squares is the summation's,
bounded for n non-negative terms in any order by (n - 1) * 2^-53 * sum; on
grid-valued gradients every partial sum is exact and the sums, the norm and
the coefficient must match the oracle bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import Case, compare, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -53
SIZES = [0, 1, 3, 1000, 1024, 1025, 4097, 32768 + 5, 70001, 2 * 32768]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield
    osa.opt_debug_set_launch(32768, 0)


def _gpu_norms(host_grads, max_norm=1.0, norm_type=2, with_coef=True):
    import torch
    import optimizer_step_amd as osa
    dev = [to_dev(g) for g in host_grads]
    out = torch.full((2 + 2 * len(dev),), -1.0, dtype=torch.float64, device="cuda")
    coef = torch.full((1,), -1.0, dtype=torch.float32, device="cuda") if with_coef else None
    osa.opt_grad_norm(dev, out, max_norm, norm_type, coef)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (float(coef.cpu().numpy()[0]) if with_coef else None)


def _random_list(t=1, scale=1e-2):
    return [synth.grads(n, t, k, std=scale, bf16=(k % 2 == 1)) for k, n in enumerate(SIZES)]


def _assert_sum(gpu, orc, n):
    if np.isnan(orc) or np.isinf(orc):
        assert (np.isnan(gpu) and np.isnan(orc)) or gpu == orc, (gpu, orc)
        return
    assert abs(gpu - orc) <= max(n - 1, 0) * U * orc, (gpu, orc, n)


@pytest.mark.parametrize("t", [1, 2])
def test_norms_random_mixed_dtypes(t):
    """Ragged sizes (empty, sub-tile, tile, tile + 1, several chunks), float32
    and BF16 gradients in one list."""
    grads = _random_list(t)
    out, _ = _gpu_norms(grads, with_coef=False)
    (s2, mx), per = oracle.grad_norm_list(grads)
    for k, (ps, pm) in enumerate(per):
        _assert_sum(out[2 + 2 * k], ps, SIZES[k])
        assert out[3 + 2 * k] == pm, (k, out[3 + 2 * k], pm)
    _assert_sum(out[0], s2, sum(SIZES))
    assert out[1] == mx


@pytest.mark.parametrize("norm_type", [2, 0])
@pytest.mark.parametrize("clips", [True, False])
def test_grid_values_bit_exact(norm_type, clips):
    """Grid gradients: every sum exact, so sums, norm and coefficient are
    bit-identical to the oracle; a small max_norm clips, 1e9 gives 1."""
    max_norm = (0.5 if norm_type == 2 else 0.05) if clips else 1e9
    grads = [synth.grid_grads(n, 1, k, bf16=(k % 3 == 0)) for k, n in enumerate(SIZES)]
    out, coef = _gpu_norms(grads, max_norm, norm_type)
    (s2, mx), per = oracle.grad_norm_list(grads)
    for k, (ps, pm) in enumerate(per):
        assert out[2 + 2 * k] == ps and out[3 + 2 * k] == pm, k
    assert out[0] == s2 and out[1] == mx
    want = oracle.clip_coef(np.sqrt(s2) if norm_type == 2 else mx, max_norm)
    assert np.float32(coef).view(np.uint32) == np.float32(want).view(np.uint32), (coef, want)
    if not clips:
        assert coef == 1.0
    else:
        assert coef < 1.0


def test_coefficient_random_within_one_ulp():
    grads = _random_list(3, scale=0.3)
    out, coef = _gpu_norms(grads, 1.0, 2)
    (s2, _), _ = oracle.grad_norm_list(grads)
    want = oracle.clip_coef(np.sqrt(s2), 1.0)
    assert want < 1.0
    d = abs(int(np.float32(coef).view(np.int32)) - int(np.float32(want).view(np.int32)))
    assert d <= 1, (coef, want)


def test_nan_and_inf():
    """A NaN poisons its tensor's sum and max and both totals, and the
    coefficient; an infinity gives an infinite norm and a coefficient of 0."""
    grads = _random_list(1)
    g_nan = [g.copy() for g in grads]
    g_nan[4] = g_nan[4].copy()
    g_nan[4][17] = np.float32(np.nan)
    out, coef = _gpu_norms(g_nan, 1.0, 2)
    assert np.isnan(out[2 + 8]) and np.isnan(out[3 + 8])
    assert np.isnan(out[0]) and np.isnan(out[1]) and np.isnan(coef)
    for k in range(len(SIZES)):
        if k != 4:
            assert not np.isnan(out[2 + 2 * k])

    g_inf = [g.copy() for g in grads]
    w = g_inf[5].copy()                       # BF16 words: -inf
    w[1024] = 0xFF80
    g_inf[5] = w
    for norm_type in (2, 0):
        out, coef = _gpu_norms(g_inf, 1.0, norm_type)
        assert out[2 + 10] == np.inf and out[3 + 10] == np.inf
        assert out[0] == np.inf and out[1] == np.inf
        assert coef == 0.0


def test_empty_list_and_all_empty():
    out, coef = _gpu_norms([], 1.0, 2)
    assert out[0] == 0.0 and out[1] == 0.0 and coef == 1.0
    out, coef = _gpu_norms([np.zeros(0, np.float32), np.zeros(0, np.uint16)], 1.0, 0)
    assert list(out) == [0.0] * 6 and coef == 1.0


def test_deterministic_across_launch_geometry():
    """Tiles of 1024 elements counted from each tensor's start fix the order of
    every addition: chunk size and grid size do not change a bit."""
    import optimizer_step_amd as osa
    grads = _random_list(5)
    ref, c0 = _gpu_norms(grads)
    for chunk, wgs in [(1024, 1), (4096, 2), (65536, 0), (32768, 7)]:
        osa.opt_debug_set_launch(chunk, wgs)
        out, c = _gpu_norms(grads)
        assert np.array_equal(out.view(np.uint64), ref.view(np.uint64)), (chunk, wgs)
        assert c == c0
    osa.opt_debug_set_launch(32768, 0)


BIG = [3 * 2**20 + 7, 0, 5, 2**20, 2 * 2**20 + 1024, 2**20 + 1]


def _big_list(gdt, grid=False):
    out = []
    for k, n in enumerate(BIG):
        if grid:
            out.append(synth.grid_grads(n, 1, k, bf16=(gdt == "bf16")))
        else:
            g = synth.grads(n, 1, k, std=1e-2)
            out.append(synth.bf16_words(g) if gdt == "bf16" else g.astype(np.float16) if gdt == "f16" else g)
    return out


@pytest.mark.parametrize("gdt", ["f32", "bf16", "f16"])
def test_tensors_spanning_several_sum_groups(gdt):
    """Tensors of more than 1024 partials (2^20 elements) are summed over
    several first-level groups, one workgroup each, then in order: sums
    within the summation bound, maxima exact, and no dependence on the launch
    geometry."""
    import optimizer_step_amd as osa
    grads = _big_list(gdt)
    out, _ = _gpu_norms(grads, with_coef=False)
    host = [g.astype(np.float32) if g.dtype == np.float16 else g for g in grads]
    (s2, mx), per = oracle.grad_norm_list(host)
    for k, (ps, pm) in enumerate(per):
        _assert_sum(out[2 + 2 * k], ps, BIG[k])
        assert out[3 + 2 * k] == pm, (k, out[3 + 2 * k], pm)
    _assert_sum(out[0], s2, sum(BIG))
    assert out[1] == mx
    try:
        for chunk, wgs in [(1024, 0), (65536, 3)]:
            osa.opt_debug_set_launch(chunk, wgs)
            again, _ = _gpu_norms(grads, with_coef=False)
            assert np.array_equal(again.view(np.uint64), out.view(np.uint64)), (chunk, wgs)
    finally:
        osa.opt_debug_set_launch(32768, 0)


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
def test_several_sum_groups_grid_values_bit_exact(gdt):
    grads = _big_list(gdt, grid=True)
    out, coef = _gpu_norms(grads, 0.5, 2)
    (s2, mx), per = oracle.grad_norm_list(grads)
    for k, (ps, pm) in enumerate(per):
        assert out[2 + 2 * k] == ps and out[3 + 2 * k] == pm, k
    assert out[0] == s2 and out[1] == mx
    want = oracle.clip_coef(np.sqrt(s2), 0.5)
    assert np.float32(coef).view(np.uint32) == np.float32(want).view(np.uint32), (coef, want)


CLIP_FORMATS = [("adamw", "f32"), ("adamw", "bf16_rn"), ("adamw", "bf16_sr"), ("adamw", "q8"),
                ("ademamix", "f32"), ("ademamix", "bf16_sr"), ("ademamix", "q8")]


@pytest.mark.parametrize("opt,fmt", CLIP_FORMATS)
def test_clip_then_step(opt, fmt):
    """Norm, coefficient and step chained on one stream, the coefficient
    handed to the step through device memory (no host round trip); grid
    gradients make the coefficient exact, so states match to the usual bars."""
    sizes = [1, 1000, 4097, 32768 + 5]
    bf = [False, True, False, True]
    case = Case(opt, fmt, sizes, bf, 3, dict(lr=1e-3, weight_decay=0.1),
                grad_override=lambda t, k, n: synth.grid_grads(n, t, k, bf16=bf[k]), clip=(0.5, 2))
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    assert [np.float32(c).view(np.uint32) for c in case.gpu_coefs] == \
           [np.float32(c).view(np.uint32) for c in case.oracle_coefs]
    assert all(c < 1.0 for c in case.oracle_coefs)
    compare(case, dev, ps, st)


def test_clip_then_step_with_unorm():
    """The update-norm pre-pass sees the clipped gradient too."""
    sizes = [1000, 32768 + 5]
    case = Case("adamw", "f32", sizes, [True, False], 2, dict(lr=1e-3, max_unorm=1.0),
                grad_override=lambda t, k, n: synth.grid_grads(n, t, k, bf16=(k == 0)), clip=(0.05, 0))
    ps, st, norms = case.run_oracle()
    assert all(c < 1.0 for c in case.oracle_coefs)
    dev, gnorms = case.run_gpu()
    assert case.gpu_coefs == case.oracle_coefs
    for t in range(2):
        for k in range(2):
            _, _, u2, p2 = norms[t * 2 + k]
            assert abs(gnorms[t][2 * k] - u2) <= 1e-12 * u2
            # the second step sees p that differs within its bar (the
            # direction is formed with hardware rcp/sqrt): ~1e-7 relative
            assert abs(gnorms[t][2 * k + 1] - p2) <= (1e-12 if t == 0 else 1e-7) * p2
    compare(case, dev, ps, st)


def test_grad_scale_from_host_value():
    """grad_scale is any device float, not only a coefficient from the norm."""
    import torch
    import optimizer_step_amd as osa
    sizes = [3, 4097]
    hp = dict(lr=1e-3, weight_decay=0.01)
    ps, st, _ = Case("adamw", "bf16_sr", sizes, False, 2, dict(hp, grad_scale=0.375)).run_oracle()
    case = Case("adamw", "bf16_sr", sizes, False, 2, hp)
    s = torch.tensor([0.375], dtype=torch.float32, device="cuda")
    dev = case.alloc_gpu()
    tl = osa.TensorList(dev)
    for t in (1, 2):
        for k in range(2):
            dev[k]["g"].copy_(to_dev(case.grad(t, k)))
        osa.opt_step_adamw(tl, "bf16_sr", osa.hparams(step=t, seed=case.seed, grad_scale=s, **hp))
    torch.cuda.synchronize()
    compare(case, dev, ps, st)

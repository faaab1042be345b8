"""GPU parity of the FP8 / FP4 block-scaled optimizer states and of state
resets ("When Small Updates Disappear", Sec. 2.1 and 5) against the oracle.

Bars: codes, stochastic-rounding choices and block absmax bit-exact (the
moments are formed in the same binary32 order on both sides); p within 1e-6
relative (the blockwise kernel forms the direction with the hardware
reciprocal and square root)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import Case, compare, states_bit_identical, to_dev, to_host

pytestmark = pytest.mark.gpu

FP_FMTS = ["fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr"]
SIZES = [1, 255, 257, 1001, 4096, 2 * 32768 + 513]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield
    osa.opt_debug_set_launch(32768, 0)


def _hp(opt):
    hp = dict(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.999, eps=1e-8)
    if opt == "ademamix":
        hp.update(beta3=0.9999, alpha=5.0)
    return hp


@pytest.mark.parametrize("elem", [0, 1, 2])
def test_device_codec_matches_oracle(elem):
    """The kernels' codec, run on the device, against the oracle's grid walk
    (same inputs as the host check of the library), for both roundings."""
    import torch
    import optimizer_step_amd as osa
    from tests.test_abi_cpu import _mini_inputs
    rng = np.random.default_rng(190 + elem)
    for A in [np.float32(v) for v in (1.0, 448.0, 3e-3, 2.5e-12, 1e30, 3e-39, 0.0, np.nan)]:
        x = _mini_inputs(elem, A, rng) if np.isfinite(A) and A > 0 else np.array([0.0, -0.0, 1.0], np.float32)
        if A == 0:
            x = np.array([0.0, -0.0], np.float32)
        for sr in (False, True):
            r = rng.integers(0, 65536, x.size).astype(np.uint32) if sr else None
            xd = to_dev(x)
            rd = None if r is None else torch.from_numpy(r.view(np.int32)).cuda()
            codes = torch.empty(x.size, dtype=torch.uint8, device="cuda")
            dec = torch.empty(x.size, dtype=torch.float32, device="cuda")
            osa.opt_debug_mini(elem, float(A), xd, rd, codes, dec)
            torch.cuda.synchronize()
            c, d = to_host(codes), to_host(dec)
            want = np.array([oracle.mini_encode(elem, v, A, int(r[i]) if sr else -1) for i, v in enumerate(x)])
            assert np.array_equal(c, want), (elem, A, sr)
            wdec = np.array([oracle.mini_decode(elem, int(k), A) for k in want], dtype=np.float32)
            nan = np.isnan(wdec)
            assert np.array_equal(np.isnan(d), nan)
            assert np.array_equal(d[~nan].view(np.uint32), wdec[~nan].view(np.uint32)), (elem, A, sr)


@pytest.mark.parametrize("elem", [0, 1, 2])
def test_step_encoder_matches_oracle(elem):
    """The encoder the blockwise step runs (four values at a time, gfx950's
    scaled conversions for E4M3 stochastic, E2M1, and unsigned E2M2
    stochastic through E5M2) against the oracle's grid walk, for both
    roundings, across block scales: every normal scale the conversions take,
    the ends of their range and past them (where the step rounds in integer
    arithmetic), subnormal absmax included."""
    import torch
    import optimizer_step_amd as osa
    from tests.test_abi_cpu import _mini_inputs
    rng = np.random.default_rng(290 + elem)
    emax, emin = {0: (8, -6), 1: (2, 0), 2: (2, 0)}[elem]
    As = [np.float32(v) for v in (1.0, 1.5, 448.0, 7.0, 3e-3, 2.5e-12, 1e30, 3e-39, 1e-44)]
    # nsc = emax - floor(log2 A) at the conversions' limits (-127 / -113 and 126) and beyond
    for nsc in (-128, -127, -126, -114, -113, -112, 0, 125, 126, 127):
        a = 1.3 * 2.0 ** (emax - nsc)
        if 0 < a < 3.4e38:
            As.append(np.float32(a))
    for A in As:
        x = _mini_inputs(elem, A, rng)
        x = np.concatenate([x, np.zeros((-x.size) % 4, np.float32)])
        for sr in (False, True):
            r = rng.integers(0, 65536, x.size).astype(np.uint32) if sr else None
            codes = torch.empty(x.size, dtype=torch.uint8, device="cuda")
            osa.opt_debug_mini_pack(elem, float(A), to_dev(x), None if r is None else torch.from_numpy(r.view(np.int32)).cuda(),
                                    codes)
            torch.cuda.synchronize()
            got = to_host(codes)
            want = np.array([oracle.mini_encode(elem, v, A, int(r[i]) if sr else -1) for i, v in enumerate(x)])
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (elem, float(A), sr, x[bad[:4]], got[bad[:4]], want[bad[:4]])


@pytest.mark.parametrize("fmt", FP_FMTS)
@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_step_parity(opt, fmt):
    """Ragged sizes (single element, short blocks, an odd FP4 tail, several
    chunks), fp32 and bf16 gradients in one list, 4 steps."""
    case = Case(opt, fmt, SIZES, [False, True, False, True, True, False], 4, _hp(opt))
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)


@pytest.mark.parametrize("fmt", ["fp8_sr", "fp4_rn"])
def test_step_independent_of_launch_geometry(fmt):
    import optimizer_step_amd as osa
    import torch
    case = Case("adamw", fmt, SIZES, True, 2, _hp("adamw"))
    ref, _ = case.run_gpu()
    ref = Case.host(ref)
    try:
        for chunk, wgs in [(1024, 1), (4096, 3), (65536, 0)]:
            osa.opt_debug_set_launch(chunk, wgs)
            dev, _ = case.run_gpu()
            got = Case.host(dev)
            for k in range(len(SIZES)):
                for key in ref[k]:
                    assert np.array_equal(got[k][key].view(np.uint8), ref[k][key].view(np.uint8)), (chunk, k, key)
    finally:
        osa.opt_debug_set_launch(32768, 0)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["f32", "bf16_rn", "bf16_sr", "q8"] + FP_FMTS)
def test_reset_interval(fmt):
    """Moments restart from zero at steps 1, 4, 7 (reset_interval 3): the
    kernels skip the state reads there and restart the bias corrections."""
    case = Case("adamw", fmt, [1001, 32768 + 300], [True, False], 7, dict(_hp("adamw"), reset_interval=3))
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)


@pytest.mark.parametrize("fmt", FP_FMTS)
def test_reset_interval_ademamix_with_update_norm(fmt):
    hp = dict(_hp("ademamix"), reset_interval=2, max_unorm=1.0)
    case = Case("ademamix", fmt, [3000, 257], [False, True], 5, hp)
    ps, st, norms_o = case.run_oracle()
    dev, norms_g = case.run_gpu()
    compare(case, dev, ps, st)
    for (t, k, u2, p2) in norms_o:
        g = norms_g[t - 1]
        # the direction is exact in the pre-pass; p differs by a few ulp of
        # lr*|u| per step after step 1 (hardware rcp/sqrt in the step kernel)
        tol_p = 1e-12 if t == 1 else 1e-7
        assert abs(g[2 * k] - u2) <= 1e-12 * abs(u2), (t, k)
        assert abs(g[2 * k + 1] - p2) <= tol_p * abs(p2), (t, k)


@pytest.mark.parametrize("fmt", FP_FMTS)
def test_update_norm_prepass(fmt):
    case = Case("adamw", fmt, [65537, 0, 3000], [False, False, True], 3, dict(_hp("adamw"), max_unorm=1.0))
    ps, st, norms_o = case.run_oracle()
    dev, norms_g = case.run_gpu()
    compare(case, dev, ps, st)
    for (t, k, u2, p2) in norms_o:
        g = norms_g[t - 1]
        tol_p = 1e-12 if t == 1 else 1e-7
        assert abs(g[2 * k] - u2) <= 1e-12 * abs(u2), (t, k)
        assert abs(g[2 * k + 1] - p2) <= tol_p * abs(p2), (t, k)


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_q8_tiny_moments_in_normal_blocks(opt):
    """Moments below 2^-100 (gradients of 1e-35 and binary32 subnormals) in
    blocks whose absmax is normal: the 8-bit quotient of such a moment may miss
    the correctly rounded one by an ulp, and its code must still be the
    oracle's (the quotient lies far below every codebook midpoint)."""
    def g_of(t, k, n):
        g = synth.grads(n, t, k, std=1e-2)
        rng = np.random.default_rng([11, t, k])
        pick = rng.random(n) < 0.05
        tiny = rng.choice(np.array([1e-35, -1e-35, 3e-38, -2e-40, 1e-44], np.float32), n)
        return np.where(pick, tiny, g).astype(np.float32)
    case = Case(opt, "q8", [4096, 1000], False, 3, _hp(opt), grad_override=g_of)
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


def _linear_signed():
    # entries +-1/255, +-3/255, ...: the middle midpoint is exactly 0
    return np.linspace(-1, 1, 256).astype(np.float32)


def test_q8_huge_absmax_with_tiny_moments():
    """Blocks whose absmax is 1e10..1e13 holding moments of 1e-30..1e-25:
    their quotients m'/A fall below the normal range, where the reused
    reciprocal is not covered, so such blocks take true division.  The
    linear codebook's zero midpoint makes a flushed or misrounded tiny
    quotient change its code."""
    def g_of(t, k, n):
        g = synth.grads(n, t, k, std=1e-2)
        rng = np.random.default_rng([23, t, k])
        for b, big in ((0, 1e11), (1, -3e12), (3, 1e13), (6, 2e10)):
            sl = slice(256 * b, 256 * (b + 1))
            g[sl] = (rng.choice([-1.0, 1.0], 256) * 10.0 ** rng.uniform(-29, -24, 256)).astype(np.float32)
            g[256 * b + 7 * (t + k) % 256] = np.float32(big)
        return g.astype(np.float32)
    case = Case("adamw", "q8", [2048, 1800], False, 3, _hp("adamw"), grad_override=g_of)
    case.qs = _linear_signed()
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)
    assert st[0]["a1"][3] > 2.0 ** 26                  # the fallback's range exercised


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_q8_signed_zero_moments(opt):
    """Exact +-0 gradients at step 1 give moments of +0 and -0 (a fresh
    state decodes to -0 for a negative zero code): both must take the code of
    x <= 0 on the linear codebook, whose midpoint between -1/255 and +1/255 is
    exactly 0, while the smallest positive quotients take the one above."""
    def g_of(t, k, n):
        g = synth.grads(n, t, k, std=1e-2)
        rng = np.random.default_rng([29, t, k])
        z = rng.random(n) < 0.3
        g[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
        return g.astype(np.float32)
    case = Case(opt, "q8", [4096, 777], False, 3, _hp(opt), grad_override=g_of)
    case.qs = _linear_signed()
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


def test_q8_unsigned_codebook_starting_at_negative_zero():
    """An unsigned codebook whose first entry is -0.0: with skip_zeros, a zero
    gradient codes the old v again, and the oracle reads code 0 back as -0.
    The library's table reads it as +0 (its lookup takes v's bits with no
    sign mask); codes, absmax, p and every state word stay the oracle's."""
    def g_of(t, k, n):
        g = synth.grads(n, t, k, std=1e-2)
        rng = np.random.default_rng([31, t, k])
        g[rng.random(n) < 0.4] = np.float32(0.0)
        g[::97] = np.float32(3.0)                      # large values: small v code 0 elsewhere
        return g.astype(np.float32)
    hp = dict(_hp("adamw"), skip_zeros=True)
    case = Case("adamw", "q8", [4096, 777], False, 4, hp, grad_override=g_of)
    qu = synth.codebook_unsigned().copy()
    assert qu[0] == 0.0
    qu[0] = np.float32(-0.0)
    case.qu = qu
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


@pytest.mark.parametrize("fmt", FP_FMTS + ["q8"])
def test_nan_and_tiny_gradients(fmt):
    """A NaN gradient poisons its block's absmax (the block then reads back as
    NaN); gradients spread over 1e-22..1e-12 put moments below 2^-100 in blocks
    whose absmax is normal (the 8-bit quotient must then avoid the reused
    reciprocal); gradients of 1e-20 make v's block absmax subnormal."""
    def g_of(t, k, n):
        if k == 1:
            rng = np.random.default_rng([5, t])
            return (rng.standard_normal(n) * 10.0 ** rng.uniform(-22, -12, n)).astype(np.float32)
        g = synth.grads(n, t, k, std=1e-20 if k == 2 else 1e-2)
        if k == 0 and t == 2:
            g[300] = np.float32(np.nan)
        return g
    case = Case("adamw", fmt, [1024, 2048, 1000], False, 3, _hp("adamw"), grad_override=g_of)
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    assert np.isnan(st[0]["a2"][1])                    # the poisoned block
    assert 0 < st[2]["a2"].min() < 2.0 ** -126          # subnormal absmax exercised

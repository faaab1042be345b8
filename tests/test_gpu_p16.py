"""GPU parity of 16-bit (BF16 / FP16) parameter storage with nearest or
stochastic rounding, FP16 gradients, and the standalone rounding cast
("When Small Updates Disappear", Sec. 6-8; the issue "Investigate SM103
bias-correction broadcast in 32-bit optimizers", Correctness oracle: FP16,
BF16 and FP32 parameter and gradient storage).

Bars: the cast bit-exact; 16-bit parameters and every state bit-exact.  With
16-bit parameters the kernels take the fast direction u (hardware reciprocal
and square root) only where its error bound shows that the parameter rounds
to the word the exact recipe's binary32 value rounds to (one element in
about 2^14 for BF16, 2^11 for FP16 falls back to the exact recipe, which
forms u with correctly rounded division and square root in the oracle's
order), so every stored word is the oracle's.  The bound itself is checked
in test_gpu_direction_bound.py."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import BLOCKED_FMTS, nan_equal_bits, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield


def _special(n, rng):
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-12, 6, n)).astype(np.float32)
    edge = np.array([0.0, -0.0, np.nan, np.inf, -np.inf, 65504, 65519.99, 65520, 65536, 3.4e38,
                     2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 1e-40, -1e-45, 1.0 + 2.0 ** -9], np.float32)
    x[:min(n, edge.size)] = edge[:min(n, edge.size)]
    return x


def _words_equal(a, b, dtype):
    fa = oracle.widen_bf16(a) if dtype == oracle.P_BF16 else a.view(np.float16).astype(np.float32)
    fb = oracle.widen_bf16(b) if dtype == oracle.P_BF16 else b.view(np.float16).astype(np.float32)
    nan = np.isnan(fb)
    return np.array_equal(np.isnan(fa), nan) and np.array_equal(a[~nan], b[~nan])


@pytest.mark.parametrize("n", [0, 1, 3, 4, 1023, (1 << 20) + 3])
@pytest.mark.parametrize("stochastic", [False, True])
@pytest.mark.parametrize("dtype", [oracle.P_BF16, oracle.P_F16])
def test_round_cast(dtype, stochastic, n):
    import torch
    import optimizer_step_amd as osa
    x = _special(n, np.random.default_rng(n + 7))
    out = torch.empty(n, dtype=torch.bfloat16 if dtype == oracle.P_BF16 else torch.float16, device="cuda")
    seed, offset = 0xDEADBEEF12345678, 41
    osa.opt_round_cast(to_dev(x), out, stochastic, seed, offset)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.round_cast(x, dtype, stochastic, seed, offset)
    assert _words_equal(got, want, dtype)
    if stochastic and n > 1000:
        nearest = oracle.round_cast(x, dtype, False)
        assert np.mean(got != nearest) > 0.05


def test_round_cast_nearest_matches_torch():
    import torch
    import optimizer_step_amd as osa
    x = _special(100000, np.random.default_rng(3))
    xd = to_dev(x)
    for dt in (torch.bfloat16, torch.float16):
        out = torch.empty(x.size, dtype=dt, device="cuda")
        osa.opt_round_cast(xd, out)
        ref = xd.to(dt)
        torch.cuda.synchronize()
        a = out.view(torch.int16).cpu().numpy()
        b = ref.view(torch.int16).cpu().numpy()
        nan = np.isnan(ref.float().cpu().numpy())
        assert np.array_equal(a[~nan], b[~nan])


# ---------------------------------------------------------------------------
# steps with 16-bit parameters

GD = {"f32": np.float32, "bf16": "bf16", "f16": np.float16}


def _grad(n, t, k, gd):
    g = synth.grads(n, t, k, std=1e-2)
    if gd == "bf16":
        return synth.bf16_words(g)
    return g.astype(GD[gd])


def _p16(p32, dtype):
    return synth.bf16_words(p32) if dtype == oracle.P_BF16 else p32.astype(np.float16).view(np.uint16)


def _dev_p16(words, dtype):
    import torch
    t = torch.from_numpy(words.view(np.int16).copy()).cuda()
    return t.view(torch.bfloat16 if dtype == oracle.P_BF16 else torch.float16)


def _wide(words, dtype):
    """16-bit parameter words -> float64 values."""
    if dtype == oracle.P_BF16:
        return oracle.widen_bf16(words).astype(np.float64)
    return words.view(np.float16).astype(np.float64)


def _run_p16(opt, fmt, sizes, gds, pdt, p_sr, steps, hp, unorm=False, grad=_grad, seed=synth.SR_SEED):
    """Steps the list on both sides; grad(n, t, k, gd) gives the gradients."""
    import torch
    import optimizer_step_amd as osa
    p0 = [_p16(synth.params(n, k, std=0.5), pdt) for k, n in enumerate(sizes)]
    q8 = fmt == "q8"
    qs, qu = (synth.codebook_signed(), synth.codebook_unsigned()) if q8 else (None, None)
    # oracle
    ps = [p.copy() for p in p0]
    st = [oracle.state_zeros(fmt, n, opt, qs=qs, qu=qu) if q8 else oracle.state_zeros(fmt, n, opt) for n in sizes]
    qkw = dict(qs=qs, qu=qu) if q8 else {}
    norms_o = []
    pmax = [np.abs(_wide(p, pdt)) for p in ps]      # largest |p| along the oracle's steps
    for t in range(1, steps + 1):
        for k, n in enumerate(sizes):
            g = grad(n, t, k, gds[k])
            h = oracle.make_hp(step=t, seed=seed, tensor_index=k, **hp)
            scale = 1.0
            if unorm:
                wide = oracle.widen_bf16(ps[k]) if pdt == oracle.P_BF16 else ps[k].view(np.float16).astype(np.float32)
                u2, p2 = oracle.unorm(opt, fmt, h, wide, g, **st[k], **qkw)
                norms_o.append((t, k, u2, p2))
                scale = oracle.unorm_scale(hp["max_unorm"], u2, p2)
            oracle.step(opt, fmt, h, ps[k], g, scale=scale, p_dtype=pdt, p_sr=p_sr, **st[k], **qkw)
            pmax[k] = np.maximum(pmax[k], np.abs(_wide(ps[k], pdt)))
    # GPU
    dev = []
    for k, n in enumerate(sizes):
        d = {"p": _dev_p16(p0[k], pdt), "g": to_dev(grad(n, 1, k, gds[k]))}
        d.update(osa.state_buffers(fmt, n, opt, qmap_signed=qs, qmap_unsigned=qu))
        dev.append(d)
    tl = osa.TensorList(dev)
    fn = osa.opt_step_adamw if opt == "adamw" else osa.opt_step_ademamix
    norms_g = []
    for t in range(1, steps + 1):
        for k, n in enumerate(sizes):
            dev[k]["g"].copy_(to_dev(grad(n, t, k, gds[k])))
        h = osa.hparams(step=t, seed=seed, p_rounding=1 if p_sr else 0, qmap_signed=qs,
                        qmap_unsigned=qu, **hp)
        un = None
        if unorm:
            un = torch.empty(2 * len(sizes), dtype=torch.float64, device="cuda")
            osa.opt_precondition_unorm(opt, tl, fmt, h, un)
            norms_g.append(un.cpu().numpy().copy())
        fn(tl, fmt, h, un)
    torch.cuda.synchronize()
    return ps, st, dev, norms_o, norms_g, pmax


def _check(ps, st, dev, fmt, opt, pdt, steps, pmax):
    """Every 16-bit parameter word, state word, code and absmax bit-exact
    (NaNs compared as NaNs)."""
    for k in range(len(ps)):
        got = dev[k]["p"].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
        assert _words_equal(got, ps[k], pdt), (k, int(np.sum(got != ps[k])))
        for key in ("s1", "s2", "s3")[:3 if opt == "ademamix" else 2]:
            assert nan_equal_bits(to_host(dev[k][key]), st[k][key]), (k, key)
            if fmt in BLOCKED_FMTS:
                a = "a" + key[1]
                assert nan_equal_bits(to_host(dev[k]["absmax" + key[1]]), st[k][a]), (k, a)


@pytest.mark.parametrize("p_sr", [False, True])
@pytest.mark.parametrize("pdt", [oracle.P_BF16, oracle.P_F16])
@pytest.mark.parametrize("fmt", ["f32", "bf16_sr"])
def test_p16_adamw(fmt, pdt, p_sr):
    sizes = [1, 1001, 4096, 32768 + 77]
    gds = ["f32", "bf16", "f16", "bf16"] if pdt == oracle.P_BF16 else ["f32", "f16", "f16", "f32"]
    ps, st, dev, _, _, pmax = _run_p16("adamw", fmt, sizes, gds, pdt, p_sr, 4, dict(lr=1e-2, weight_decay=0.1))
    _check(ps, st, dev, fmt, "adamw", pdt, 4, pmax)


@pytest.mark.parametrize("p_sr", [False, True])
@pytest.mark.parametrize("pdt", [oracle.P_BF16, oracle.P_F16])
def test_p16_many_elements(pdt, p_sr):
    """2^20 + 5 elements over three steps: a few hundred (BF16) to a few
    thousand (FP16) of them take the exact fallback, every word bit-exact."""
    sizes = [(1 << 20) + 5]
    ps, st, dev, _, _, pmax = _run_p16("adamw", "bf16_sr", sizes, ["bf16"], pdt, p_sr, 3,
                                       dict(lr=1e-3, weight_decay=0.01))
    _check(ps, st, dev, "bf16_sr", "adamw", pdt, 3, pmax)


@pytest.mark.parametrize("fmt", ["bf16_rn", "bf16_sr", "fp8_rn", "fp8_sr"])
def test_p16_chunk_and_grid_do_not_change_results(fmt):
    """16-bit parameters with BF16 or FP8 states under several host chunk
    sizes and grids (one workgroup per tile, and persistent grids walking the
    tiles): every word the same, and the first launch setting bit-exact
    against the oracle.  The tiles of these kernels (two groups of four
    elements per lane, or two blocks per wave) then start and end at other
    places within each tensor."""
    import optimizer_step_amd as osa
    sizes = [300_001, 4097, 1000]
    hp = dict(lr=1e-2, weight_decay=0.1)
    runs = []
    try:
        for chunk, wgs in ((32768, 0), (1024, 1), (65536, 3), (4096, 64)):
            osa.opt_debug_set_launch(chunk, wgs)
            ps, st, dev, _, _, pmax = _run_p16("adamw", fmt, sizes, ["bf16", "f16", "bf16"], oracle.P_BF16, True, 2, hp)
            if not runs:
                _check(ps, st, dev, fmt, "adamw", oracle.P_BF16, 2, pmax)
            runs.append([{k: to_host(v).view(np.uint8).copy() for k, v in d.items() if k != "g"} for d in dev])
    finally:
        osa.opt_debug_set_launch(32768, 0)
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            for key in x:
                assert np.array_equal(x[key], y[key]), key


@pytest.mark.parametrize("eps", [0.0, -1e-3])
@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_p16_eps_edges(opt, eps):
    """eps = 0 keeps the fast direction's bound (tiny v_hat takes the exact
    recipe per element); a negative eps is outside the bound's analysis, so
    every element takes the exact recipe (directions that blow up included).
    Every word bit-exact either way."""
    sizes = [1000, 32768 + 77]
    hp = dict(lr=1e-2, weight_decay=0.1, eps=eps)
    if opt == "ademamix":
        hp.update(beta3=0.999, alpha=5.0)
    ps, st, dev, _, _, pmax = _run_p16(opt, "bf16_sr", sizes, ["bf16", "f16"], oracle.P_BF16, True, 3, hp)
    _check(ps, st, dev, "bf16_sr", opt, oracle.P_BF16, 3, pmax)


@pytest.mark.parametrize("pdt", [oracle.P_BF16, oracle.P_F16])
def test_p16_ademamix_bf16_rn(pdt):
    sizes = [777, 32768 * 2 + 5]
    ps, st, dev, _, _, pmax = _run_p16("ademamix", "bf16_rn", sizes, ["bf16", "f16"], pdt, True, 3,
                                 dict(lr=1e-2, weight_decay=0.1, beta3=0.999, alpha=5.0))
    _check(ps, st, dev, "bf16_rn", "ademamix", pdt, 3, pmax)


def test_p16_with_update_norm():
    sizes = [3000, 65537]
    ps, st, dev, no, ng, pmax = _run_p16("adamw", "f32", sizes, ["bf16", "f32"], oracle.P_BF16, True, 3,
                                   dict(lr=1e-2, max_unorm=0.5), unorm=True)
    _check(ps, st, dev, "f32", "adamw", oracle.P_BF16, 3, pmax)
    for (t, k, u2, p2) in no:
        g = ng[t - 1]
        # p and the states are the oracle's bits at every step, so the sums
        # differ by summation order only
        assert abs(g[2 * k] - u2) <= 1e-12 * u2 and abs(g[2 * k + 1] - p2) <= 1e-12 * p2, (t, k)


def test_one_state_refuses_p16():
    """The one-state optimizers take fp32 parameters only."""
    import torch
    import optimizer_step_amd as osa
    d = {"p": torch.zeros(256, dtype=torch.bfloat16, device="cuda"),
         "g": torch.zeros(256, dtype=torch.bfloat16, device="cuda"),
         "s1": torch.zeros(256, dtype=torch.float32, device="cuda")}
    with pytest.raises(osa.OptError) as e:
        osa.opt_step_1state("momentum", osa.TensorList([d]), "f32", osa.hparams())
    assert e.value.status == osa.OPT_EUNSUPPORTED


def test_grad_norm_f16():
    import torch
    import optimizer_step_amd as osa
    grads = [synth.grads(n, 1, k, std=3.0).astype(np.float16) for k, n in enumerate([5, 4097, 70001])]
    out = torch.empty(8, dtype=torch.float64, device="cuda")
    osa.opt_grad_norm([to_dev(g) for g in grads], out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    (s2, mx), per = oracle.grad_norm_list(grads)
    for k, (ps, pm) in enumerate(per):
        assert abs(o[2 + 2 * k] - ps) <= grads[k].size * 2.0 ** -53 * ps and o[3 + 2 * k] == pm


@pytest.mark.parametrize("p_sr", [False, True])
@pytest.mark.parametrize("pdt", [oracle.P_BF16, oracle.P_F16])
@pytest.mark.parametrize("fmt", ["q8", "fp8_sr", "fp4_rn"])
def test_p16_blockwise_states(fmt, pdt, p_sr):
    """16-bit parameters with the blockwise state formats: p, codes and
    absmax bit-exact."""
    sizes = [1, 1001, 4096, 32768 + 77]
    gds = ["f32", "bf16", "f16", "bf16"]
    ps, st, dev, _, _, pmax = _run_p16("adamw", fmt, sizes, gds, pdt, p_sr, 3, dict(lr=1e-2, weight_decay=0.1))
    _check(ps, st, dev, fmt, "adamw", pdt, 3, pmax)


@pytest.mark.parametrize("fmt", ["q8", "fp8_sr"])
def test_p16_blockwise_ademamix_with_update_norm(fmt):
    sizes = [3000, 65537]
    ps, st, dev, no, ng, pmax = _run_p16("ademamix", fmt, sizes, ["bf16", "f32"], oracle.P_BF16, True, 3,
                                   dict(lr=1e-2, max_unorm=0.5, beta3=0.999, alpha=5.0), unorm=True)
    _check(ps, st, dev, fmt, "ademamix", oracle.P_BF16, 3, pmax)
    for (t, k, u2, p2) in no:
        g = ng[t - 1]
        assert abs(g[2 * k] - u2) <= 1e-12 * u2 and abs(g[2 * k + 1] - p2) <= 1e-12 * p2, (t, k)


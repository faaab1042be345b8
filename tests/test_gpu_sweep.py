"""Seeded sweeps over combinations the focused tests take one at a time.
The two-state sweep draws optimizer x state format x list shape (empty,
one-element, block- and tile-edge sizes, mixed gradient dtypes) x
hyper-parameters x the features around the step (update-norm bound, gradient
clipping, skip_zeros with exact +-0 gradients, state resets, a late first
step) x launch geometry.  Further sweeps draw steps on BF16/FP16 parameters,
the one-state optimizers and the gradient norm; one test steps 3000 ragged
tensors in one call.  Each case is drawn from its own seed and printed
before it runs, so a failure names the case to rerun on its own.

Bars, as in the focused tests: p within 1e-6 relative; fp32 states within
1e-6 relative, BF16-nearest states within one BF16 step per step, every other
state word and block absmax bit-exact; beyond the bars, every stored state
word equals the oracle's (the moments never depend on p).  Clipping runs on
grid gradients, whose norms are exact in any summation order, so its
coefficient must be bit-identical too."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import Case, compare, states_bit_identical

FORMATS = ["f32", "bf16_rn", "bf16_sr", "q8", "fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr"]
SIZE_POOL = [0, 1, 2, 3, 255, 256, 257, 511, 1023, 1024, 1025, 4095, 4096, 4097,
             8191, 32767, 32768, 32769, 65536 + 17, 98304 + 255, 200_003]
GEOMETRY = [(32768, 0), (32768, 0), (1024, 0), (4096, 2), (65536, 0), (16384, 5), (2048, 1)]
N_CASES = 96
MAX_TOTAL = 400_000


@pytest.fixture(scope="module")
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available(), "these tests need the GPU"
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield
    osa.opt_debug_set_launch(32768, 0)
    torch.cuda.synchronize()


def draw(i):
    """Case i of the sweep: a dict of everything that defines it."""
    rng = np.random.default_rng([0x5EED, i])
    opt = ["adamw", "ademamix"][int(rng.integers(2))]
    fmt = FORMATS[i % len(FORMATS)] if i < 2 * len(FORMATS) else FORMATS[int(rng.integers(len(FORMATS)))]
    sizes = []
    for _ in range(int(rng.integers(1, 7))):
        n = int(SIZE_POOL[int(rng.integers(len(SIZE_POOL)))])
        if sum(sizes) + n <= MAX_TOTAL:
            sizes.append(n)
    bf16 = [bool(b) for b in rng.integers(0, 2, len(sizes))]
    hp = dict(lr=float(10.0 ** rng.uniform(-4, -1)),
              weight_decay=float(rng.choice([0.0, 0.01, 0.1, 0.2])),
              beta1=float(rng.uniform(0.8, 0.95)),
              beta2=float(rng.choice([0.95, 0.99, 0.999, 0.9999])),
              eps=float(rng.choice([1e-8, 1e-6])))
    if opt == "ademamix":
        hp.update(beta3=float(rng.choice([0.99, 0.999, 0.9999])), alpha=float(rng.uniform(2.0, 8.0)))
    if rng.random() < 0.3:
        hp["max_unorm"] = float(rng.choice([0.5, 1.0]))
    if rng.random() < 0.3:
        hp["skip_zeros"] = True
    if rng.random() < 0.3:
        hp["reset_interval"] = int(rng.integers(2, 4))
    clip = (float(rng.choice([0.05, 0.5])), int(rng.choice([2, 0]))) if rng.random() < 0.25 else None
    return dict(opt=opt, fmt=fmt, sizes=sizes, bf16=bf16, hp=hp, clip=clip,
                steps=int(rng.integers(2, 5)),
                t0=int(rng.choice([0, 0, 0, 9, 997])),
                zero_frac=float(rng.choice([0.0, 0.05, 0.3])),
                seed=int(rng.integers(1, 2**63)),
                geometry=GEOMETRY[int(rng.integers(len(GEOMETRY)))])


def _grad_fn(c):
    """Gradients of case c: random normal, or grid values when clipping; a
    seeded share of exact zeros of both signs."""
    def g_of(t, k, n):
        bf = c["bf16"][k]
        g = (synth.grid_grads(n, t, k, bf16=bf) if c["clip"] is not None
             else synth.grads(n, t, k, std=1e-2, bf16=bf))
        if c["zero_frac"] > 0 and n:
            rng = np.random.default_rng([c["seed"] & 0xFFFFFFFF, t, k])
            z = rng.random(n) < c["zero_frac"]
            neg = rng.random(n) < 0.5
            if bf:
                g[z & ~neg] = 0x0000
                g[z & neg] = 0x8000
            else:
                g[z & ~neg] = np.float32(0.0)
                g[z & neg] = np.float32(-0.0)
        return g
    return g_of


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i, gpu):
    import torch
    import optimizer_step_amd as osa
    c = draw(i)
    print(f"sweep case {i}: {c}", flush=True)
    case = Case(c["opt"], c["fmt"], c["sizes"], c["bf16"], c["steps"], c["hp"], seed=c["seed"],
                grad_override=_grad_fn(c), clip=c["clip"])
    start = None
    if c["t0"]:
        start = ([p.copy() for p in case.p0],
                 [oracle.state_zeros(c["fmt"], n, c["opt"], case.qs, case.qu) for n in c["sizes"]], c["t0"])
    ps, st, _ = case.run_oracle(start=start)
    try:
        osa.opt_debug_set_launch(*c["geometry"])
        dev, _ = case.run_gpu(t0=c["t0"])
    finally:
        osa.opt_debug_set_launch(32768, 0)
        torch.cuda.synchronize()
    if c["clip"] is not None:
        assert [np.float32(x).view(np.uint32) for x in case.gpu_coefs] == \
               [np.float32(x).view(np.uint32) for x in case.oracle_coefs]
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


def test_sweep_covers_every_format_and_feature():
    """The draws above reach every format, both optimizers, and each feature
    on and off (a host-side check of the sweep itself)."""
    cases = [draw(i) for i in range(N_CASES)]
    assert {c["fmt"] for c in cases} == set(FORMATS)
    assert {c["opt"] for c in cases} == {"adamw", "ademamix"}
    for key in ("max_unorm", "skip_zeros", "reset_interval"):
        on = [key in c["hp"] for c in cases]
        assert any(on) and not all(on), key
    assert any(c["clip"] for c in cases) and not all(c["clip"] for c in cases)
    assert any(c["t0"] for c in cases)
    assert any(0 in c["sizes"] for c in cases)
    assert any(c["geometry"] != (32768, 0) for c in cases)


# ---------------------------------------------------------------------------
# 16-bit parameters and the one-state optimizers

P16_CASES = 48
ONE_STATE_CASES = 48
GRAD_DTYPES = ["f32", "bf16", "f16"]


def _features(rng, hp):
    if rng.random() < 0.3:
        hp["skip_zeros"] = True
    if rng.random() < 0.3:
        hp["reset_interval"] = int(rng.integers(2, 4))
    return float(rng.choice([0.0, 0.05, 0.3]))


def _sizes(rng, cap=MAX_TOTAL):
    sizes = []
    for _ in range(int(rng.integers(1, 6))):
        n = int(SIZE_POOL[int(rng.integers(len(SIZE_POOL)))])
        if sum(sizes) + n <= cap:
            sizes.append(n)
    return sizes


def draw_p16(i):
    """A two-state step on BF16 / FP16 parameters, nearest or stochastic."""
    rng = np.random.default_rng([0x9161, i])
    opt = ["adamw", "ademamix"][int(rng.integers(2))]
    fmt = FORMATS[i % len(FORMATS)]
    sizes = _sizes(rng)
    hp = dict(lr=float(10.0 ** rng.uniform(-4, -1.5)), weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
              beta1=float(rng.uniform(0.8, 0.95)), beta2=float(rng.choice([0.99, 0.999])))
    if opt == "ademamix":
        hp.update(beta3=float(rng.choice([0.999, 0.9999])), alpha=float(rng.uniform(2.0, 8.0)))
    if rng.random() < 0.3:
        hp["max_unorm"] = float(rng.choice([0.5, 1.0]))
    zero_frac = _features(rng, hp)
    return dict(opt=opt, fmt=fmt, sizes=sizes, hp=hp, zero_frac=zero_frac,
                pdt=int(rng.choice([oracle.P_BF16, oracle.P_F16])), p_sr=bool(rng.integers(2)),
                gds=[GRAD_DTYPES[int(j)] for j in rng.integers(0, 3, len(sizes))],
                steps=int(rng.integers(2, 5)), seed=int(rng.integers(1, 2**63)))


def draw_1s(i):
    """A momentum / RMSprop / Adagrad / Lion step."""
    rng = np.random.default_rng([0x1575, i])
    name = ["momentum", "rmsprop", "adagrad", "lion"][i % 4]
    fmt = ["f32", "bf16_rn", "bf16_sr"][(i // 4) % 3]
    sizes = _sizes(rng)
    hp = dict(lr=float(10.0 ** rng.uniform(-4, -1.5)), weight_decay=float(rng.choice([0.0, 0.01, 0.05])),
              beta1=float(rng.uniform(0.8, 0.99)), beta2=float(rng.choice([0.9, 0.99, 0.999])),
              eps=float(rng.choice([1e-8, 1e-6])))
    zero_frac = _features(rng, hp)
    return dict(name=name, fmt=fmt, sizes=sizes, hp=hp, zero_frac=zero_frac,
                gds=[GRAD_DTYPES[int(j)] for j in rng.integers(0, 3, len(sizes))],
                steps=int(rng.integers(2, 5)), seed=int(rng.integers(1, 2**63)))


def _typed_grads(c, std):
    """Gradients of dtype gd (float32, BF16 words or float16) with a seeded
    share of exact zeros of both signs."""
    def g_of(n, t, k, gd):
        g = synth.grads(n, t, k, std=std)
        if c["zero_frac"] > 0 and n:
            rng = np.random.default_rng([c["seed"] & 0xFFFFFFFF, t, k])
            z = rng.random(n) < c["zero_frac"]
            neg = rng.random(n) < 0.5
            g[z & ~neg] = np.float32(0.0)
            g[z & neg] = np.float32(-0.0)
        if gd == "bf16":
            return synth.bf16_words(g)
        return g.astype(np.float16) if gd == "f16" else g
    return g_of


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(P16_CASES))
def test_sweep_p16(i, gpu):
    from tests.test_gpu_p16 import _check, _run_p16
    c = draw_p16(i)
    print(f"p16 sweep case {i}: {c}", flush=True)
    ps, st, dev, _, _, pmax = _run_p16(c["opt"], c["fmt"], c["sizes"], c["gds"], c["pdt"], c["p_sr"], c["steps"],
                                 c["hp"], unorm="max_unorm" in c["hp"], grad=_typed_grads(c, 1e-2),
                                 seed=c["seed"])
    _check(ps, st, dev, c["fmt"], c["opt"], c["pdt"], c["steps"], pmax)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(ONE_STATE_CASES))
def test_sweep_one_state(i, gpu):
    from tests.gpu_common import bf16_ulps, fp32_close, nan_equal_bits, to_host
    from tests.test_gpu_1state import _run_1s
    c = draw_1s(i)
    print(f"one-state sweep case {i}: {c}", flush=True)
    ps, ss, dev = _run_1s(c["name"], c["fmt"], c["gds"], c["steps"], c["hp"], sizes=c["sizes"],
                          grad=_typed_grads(c, 1e-1), seed=c["seed"])
    for k in range(len(c["sizes"])):
        assert nan_equal_bits(to_host(dev[k]["p"]), ps[k]), k
        assert nan_equal_bits(to_host(dev[k]["s1"]), ss[k]), k


def test_sweeps_of_p16_and_one_state_cover_their_space():
    """Host-side check of the two draws: every format, parameter dtype and
    rounding, optimizer, gradient dtype, and each feature on and off."""
    p = [draw_p16(i) for i in range(P16_CASES)]
    assert {c["fmt"] for c in p} == set(FORMATS)
    assert {(c["pdt"], c["p_sr"]) for c in p} == {(d, r) for d in (oracle.P_BF16, oracle.P_F16)
                                                  for r in (False, True)}
    assert {c["opt"] for c in p} == {"adamw", "ademamix"}
    o = [draw_1s(i) for i in range(ONE_STATE_CASES)]
    assert {(c["name"], c["fmt"]) for c in o} == {(n, f) for n in ("momentum", "rmsprop", "adagrad", "lion")
                                                  for f in ("f32", "bf16_rn", "bf16_sr")}
    for cases in (p, o):
        assert {g for c in cases for g in c["gds"]} == set(GRAD_DTYPES)
        for key in ("skip_zeros", "reset_interval"):
            on = [key in c["hp"] for c in cases]
            assert any(on) and not all(on), key
    on = ["max_unorm" in c["hp"] for c in p]
    assert any(on) and not all(on)


# ---------------------------------------------------------------------------
# the gradient norm

GN_CASES = 32
U53 = 2.0 ** -53


def draw_gn(i):
    """A gradient list: 1..40 tensors of pool sizes and mixed dtypes, one
    magnitude per case, maybe one non-finite value, a norm type and maybe a
    clipping coefficient."""
    rng = np.random.default_rng([0x6E0, i])
    ntens = int(rng.integers(1, 41))
    sizes = [int(SIZE_POOL[int(j)]) for j in rng.integers(0, len(SIZE_POOL), ntens)]
    while sum(sizes) > MAX_TOTAL:
        sizes.pop()
    return dict(sizes=sizes, gds=[GRAD_DTYPES[int(j)] for j in rng.integers(0, 3, len(sizes))],
                std=float(10.0 ** rng.choice([-6, -3, -1, 0, 2])),
                norm_type=int(rng.choice([2, 0])),
                max_norm=float(10.0 ** rng.uniform(-2, 3)) if rng.random() < 0.7 else None,
                poison=str(rng.choice(["none", "none", "none", "nan", "inf"])),
                geometry=GEOMETRY[int(rng.integers(len(GEOMETRY)))], t=int(i + 1))


def _gn_inputs(c):
    """Per tensor: the device-side array (float32, BF16 words or float16) and
    the oracle's view of the same values (float32 or BF16 words; float16
    widens exactly)."""
    dev, host = [], []
    for k, (n, gd) in enumerate(zip(c["sizes"], c["gds"])):
        g = synth.grads(n, c["t"], k, std=c["std"])
        if gd == "f16":
            g = np.clip(g, -65504, 65504).astype(np.float16)
        if c["poison"] != "none" and k == len(c["sizes"]) // 2 and n:
            g[n // 2] = np.nan if c["poison"] == "nan" else -np.inf
        g = synth.bf16_words(g) if gd == "bf16" else g
        dev.append(g)
        host.append(g.astype(np.float32) if gd == "f16" else g)
    return dev, host


def _same_or_both_nan(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(GN_CASES))
def test_sweep_grad_norm(i, gpu):
    import torch
    import optimizer_step_amd as osa
    c = draw_gn(i)
    print(f"grad-norm sweep case {i}: {dict(c, sizes=len(c['sizes']), gds=None)} "
          f"sizes={c['sizes']} gds={c['gds']}", flush=True)
    dev_in, host_in = _gn_inputs(c)
    (s2, mx), per = oracle.grad_norm_list(host_in)
    from tests.gpu_common import to_dev
    dev = [to_dev(g) for g in dev_in]
    out = torch.full((2 + 2 * len(dev),), -1.0, dtype=torch.float64, device="cuda")
    coef = torch.full((1,), -1.0, dtype=torch.float32, device="cuda") if c["max_norm"] else None
    try:
        osa.opt_debug_set_launch(*c["geometry"])
        osa.opt_grad_norm(dev, out, c["max_norm"] or 0.0, c["norm_type"], coef)
    finally:
        osa.opt_debug_set_launch(32768, 0)
        torch.cuda.synchronize()
    got = out.cpu().numpy()

    def within(gv, ov, n):       # summation error of n non-negative terms
        if not np.isfinite(ov):
            return _same_or_both_nan(gv, ov)
        return abs(gv - ov) <= max(n - 1, 0) * U53 * ov

    for k, (ps, pm) in enumerate(per):
        assert within(got[2 + 2 * k], ps, c["sizes"][k]), (k, got[2 + 2 * k], ps)
        assert _same_or_both_nan(got[3 + 2 * k], pm), (k, got[3 + 2 * k], pm)
    assert within(got[0], s2, sum(c["sizes"])), (got[0], s2)
    assert _same_or_both_nan(got[1], mx)
    if coef is not None:
        cg = float(coef.cpu().numpy()[0])
        want = oracle.clip_coef(np.sqrt(s2) if c["norm_type"] == 2 else mx, c["max_norm"])
        if np.isnan(want):
            assert np.isnan(cg)
        else:
            d = abs(int(np.float32(cg).view(np.int32)) - int(np.float32(want).view(np.int32)))
            assert d <= (0 if c["norm_type"] == 0 else 1), (cg, want)


def test_grad_norm_sweep_covers_its_space():
    cases = [draw_gn(i) for i in range(GN_CASES)]
    assert {g for c in cases for g in c["gds"]} == set(GRAD_DTYPES)
    assert {c["norm_type"] for c in cases} == {2, 0}
    assert {c["poison"] for c in cases} == {"none", "nan", "inf"}
    assert any(c["max_norm"] is None for c in cases) and any(c["max_norm"] for c in cases)
    assert max(len(c["sizes"]) for c in cases) >= 20


# ---------------------------------------------------------------------------
# thousands of tensors in one call

@pytest.mark.gpu
@pytest.mark.parametrize("opt,fmt", [("adamw", "f32"), ("adamw", "q8"), ("ademamix", "bf16_sr"), ("adamw", "fp4_sr")])
def test_thousands_of_small_tensors(opt, fmt, gpu):
    """3000 ragged tensors (empty to a few thousand elements, mixed gradient
    dtypes) in one call: a chunk table of thousands of entries, per-tensor
    update norms and clipping over the whole list, and skip_zeros."""
    rng = np.random.default_rng(3000)
    sizes = [int(x) for x in rng.choice([0, 1, 3, 17, 255, 256, 257, 1000, 1025, 4097], 3000)]
    bf = [bool(b) for b in rng.integers(0, 2, len(sizes))]
    hp = dict(lr=1e-3, weight_decay=0.1, max_unorm=1.0, skip_zeros=True)
    if opt == "ademamix":
        hp.update(beta3=0.999, alpha=5.0)
    case = Case(opt, fmt, sizes, bf, 2, hp, grad_override=lambda t, k, n: synth.grid_grads(n, t, k, bf16=bf[k]),
                clip=(0.5, 2))
    print(f"{len(sizes)} tensors, {sum(sizes)} elements, {opt} {fmt}", flush=True)
    ps, st, norms_o = case.run_oracle()
    dev, norms_g = case.run_gpu()
    assert [np.float32(x).view(np.uint32) for x in case.gpu_coefs] == \
           [np.float32(x).view(np.uint32) for x in case.oracle_coefs]
    assert all(c < 1.0 for c in case.oracle_coefs)
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)
    # the first step's per-tensor norms see identical inputs on both sides
    for (t, k, u2, p2) in norms_o:
        if t == 1:
            assert abs(norms_g[0][2 * k] - u2) <= 1e-12 * abs(u2), (k, norms_g[0][2 * k], u2)
            assert abs(norms_g[0][2 * k + 1] - p2) <= 1e-12 * abs(p2), (k, norms_g[0][2 * k + 1], p2)

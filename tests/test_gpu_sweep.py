"""A seeded sweep over combinations the focused tests take one at a time:
optimizer x state format x list shape (empty, one-element, block- and
tile-edge sizes, mixed gradient dtypes) x hyper-parameters x the features
around the step (update-norm bound, gradient clipping, skip_zeros with exact
+-0 gradients, state resets, a late first step) x launch geometry.  Each case
is drawn from its own seed and printed before it runs, so a failure names the
case to rerun on its own.

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

"""The library remembers the plan of a call (its tensors' chunk tables and
their slots in the device workspace), keyed by the raw tensor records, the
kind of call, optimizer, format, chunk size and codebook tables.  These
tests step lists in orders that make a remembered plan wrong if any part of
the key or the slot check were missing, and hold every result to the
oracle's bars: lists alike but for their buffers, alternating; more lists
than the workspace has slots and plans, so tables are evicted and replaced
between uses; a codebook change; a chunk-size change."""
import numpy as np
import pytest

import oracle
from tests.gpu_common import Case, compare, states_bit_identical, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield
    osa.opt_debug_set_launch(32768, 0)
    torch.cuda.synchronize()


def _gpu_step(case, dev, tl, t, qs=None, qu=None):
    import optimizer_step_amd as osa
    for k in range(len(case.sizes)):
        dev[k]["g"].copy_(to_dev(case.grad(t, k)))
    hp = osa.hparams(step=t, seed=case.seed, qmap_signed=case.qs if qs is None else qs,
                     qmap_unsigned=case.qu if qu is None else qu, **case.hp)
    fn = osa.opt_step_adamw if case.opt == "adamw" else osa.opt_step_ademamix
    fn(tl, case.fmt, hp)


def _check(case, dev):
    import torch
    torch.cuda.synchronize()
    ps, st, _ = case.run_oracle()
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


@pytest.mark.parametrize("fmt", ["f32", "q8", "fp8_sr"])
def test_alternating_lists_alike_but_for_buffers(fmt):
    """Two lists with the same sizes and dtypes (same chunk tables, other
    pointers) stepped in turn: each must use its own tensor table."""
    import optimizer_step_amd as osa
    sizes = [1000, 40000, 3]
    a = Case("adamw", fmt, sizes, [True, False, True], 4, dict(lr=1e-2, weight_decay=0.1), seed=11)
    b = Case("adamw", fmt, sizes, [True, False, True], 4, dict(lr=1e-3, weight_decay=0.0), seed=12)
    da, db = a.alloc_gpu(), b.alloc_gpu()
    ta, tb = osa.TensorList(da), osa.TensorList(db)
    for t in range(1, 5):
        _gpu_step(a, da, ta, t)
        _gpu_step(b, db, tb, t)
    _check(a, da)
    _check(b, db)


def test_more_lists_than_slots_and_plans():
    """24 lists (each its own chunk table) stepped round-robin three times:
    the workspace holds 16 tables and remembers 8 plans, so by the time a
    list comes round again its table has been replaced by another list's."""
    import optimizer_step_amd as osa
    cases, devs, tls = [], [], []
    for i in range(24):
        sizes = [257 + 1000 * i, 3 + i]
        c = Case("ademamix" if i % 3 == 0 else "adamw", ["f32", "bf16_sr", "q8", "fp4_rn"][i % 4], sizes,
                 [i % 2 == 0, True], 3, dict(lr=1e-3, weight_decay=0.1, beta3=0.999, alpha=5.0), seed=100 + i)
        d = c.alloc_gpu()
        cases.append(c)
        devs.append(d)
        tls.append(osa.TensorList(d))
    for t in range(1, 4):
        for c, d, tl in zip(cases, devs, tls):
            _gpu_step(c, d, tl, t)
    for c, d in zip(cases, devs):
        _check(c, d)


def test_codebook_change_on_the_same_list():
    """The 8-bit tables are part of the plan: a call with other codebooks on
    the same list must quantize with them (both sides switch codebooks at
    step 3)."""
    import torch
    import optimizer_step_amd as osa
    sizes = [5000, 70000]
    case = Case("adamw", "q8", sizes, False, 4, dict(lr=1e-2, weight_decay=0.1))
    qs2 = np.linspace(-1.0, 1.0, 256).astype(np.float32)     # linear, no exact zero
    qu2 = np.linspace(0.0, 1.0, 256).astype(np.float32)
    books = lambda t: (case.qs, case.qu) if t < 3 else (qs2, qu2)
    dev = case.alloc_gpu()
    tl = osa.TensorList(dev)
    for t in range(1, 5):
        _gpu_step(case, dev, tl, t, *books(t))
    torch.cuda.synchronize()
    ps = [p.copy() for p in case.p0]
    st = [oracle.state_zeros("q8", n, "adamw", case.qs, case.qu) for n in sizes]
    for t in range(1, 5):
        qs, qu = books(t)
        for k, n in enumerate(sizes):
            hp = oracle.make_hp(step=t, seed=case.seed, tensor_index=k, **case.hp)
            oracle.step("adamw", "q8", hp, ps[k], case.grad(t, k), qs=qs, qu=qu, **st[k])
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


def test_chunk_size_change_on_the_same_list():
    """The chunk size is part of the plan: the same list stepped under three
    chunk sizes in turn steps as the oracle does."""
    import torch
    import optimizer_step_amd as osa
    sizes = [70001, 4097, 0, 300]
    case = Case("adamw", "bf16_sr", sizes, [True, False, False, True], 3, dict(lr=1e-2, weight_decay=0.1))
    dev = case.alloc_gpu()
    tl = osa.TensorList(dev)
    try:
        for t, chunk in zip(range(1, 4), (32768, 1024, 65536)):
            osa.opt_debug_set_launch(chunk, 0)
            _gpu_step(case, dev, tl, t)
    finally:
        osa.opt_debug_set_launch(32768, 0)
        torch.cuda.synchronize()
    _check(case, dev)


def test_random_schedule_over_two_streams():
    """A seeded schedule of 80 steps over 10 lists (some alike but for their
    buffers), each step on one of two streams under one of three chunk
    sizes, with a pre-pass on the lists that bound the update norm.  The
    caller orders its own data across the streams; the library orders its
    tables.  Every list ends where the oracle's steps take it."""
    import torch
    import optimizer_step_amd as osa
    rng = np.random.default_rng(2024)
    shapes = [[5000, 3], [70000], [257, 4097, 1], [5000, 3], [32768 + 9, 100]]
    cases, devs, tls, ts = [], [], [], []
    for i in range(10):
        sizes = shapes[i % len(shapes)]
        hp = dict(lr=1e-3, weight_decay=0.1, beta3=0.999, alpha=5.0)
        if i % 4 == 1:
            hp["max_unorm"] = 1.0
        c = Case("ademamix" if i % 3 == 0 else "adamw", ["f32", "bf16_sr", "q8", "fp8_rn", "fp4_sr"][i % 5],
                 sizes, [bool(b) for b in rng.integers(0, 2, len(sizes))], 0, hp, seed=500 + i)
        d = c.alloc_gpu()
        cases.append(c)
        devs.append(d)
        tls.append(osa.TensorList(d))
        ts.append(0)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    try:
        for _ in range(80):
            i = int(rng.integers(len(cases)))
            s = streams[int(rng.integers(2))]
            osa.opt_debug_set_launch(int(rng.choice([32768, 1024, 65536])), 0)
            for other in streams:
                if other is not s:
                    s.wait_stream(other)
            c, d, tl = cases[i], devs[i], tls[i]
            ts[i] += 1
            t = ts[i]
            with torch.cuda.stream(s):
                for k in range(len(c.sizes)):
                    d[k]["g"].copy_(to_dev(c.grad(t, k)))
                hp = osa.hparams(step=t, seed=c.seed, qmap_signed=c.qs, qmap_unsigned=c.qu, **c.hp)
                un = None
                if c.hp.get("max_unorm", 0) > 0:
                    un = torch.empty(2 * len(c.sizes), dtype=torch.float64, device="cuda")
                    osa.opt_precondition_unorm(c.opt, tl, c.fmt, hp, un, stream=s)
                fn = osa.opt_step_adamw if c.opt == "adamw" else osa.opt_step_ademamix
                fn(tl, c.fmt, hp, un, stream=s)
                if un is not None:
                    un.record_stream(s)
    finally:
        osa.opt_debug_set_launch(32768, 0)
        torch.cuda.synchronize()
    assert min(ts) >= 3
    for c, d, n in zip(cases, devs, ts):
        c.steps = n
        _check(c, d)

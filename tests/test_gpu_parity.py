"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds: several chunks
and ragged tails, every optimizer x state format x gradient dtype, multi-tensor
lists with empty tensors, NaN/Inf gradients, determinism, chunk-size
invariance, resume, and the device test hooks.

Bars: fp32 values within 1e-6 * max(|x|, rms(x)) per element; BF16 nearest
within one BF16 step per step; stochastic-rounding bits, 8-bit codes and
absmax, and Philox words bit-exact; update norms within 1e-12 relative."""
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import Case, compare, fp32_close, nan_equal_bits, states_bit_identical, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [1, 255, 256, 257, 4095, 4096, 4097, 8191, 8193, 65536, 1_000_003]
FORMATS = ["f32", "bf16_rn", "bf16_sr", "q8"]
HP_ADAMW = dict(lr=0.1, weight_decay=0.1, beta1=0.9, beta2=0.999, eps=1e-8)
HP_ADEMAMIX = dict(lr=1e-2, weight_decay=0.1, beta1=0.9, beta2=0.999, beta3=0.99, alpha=5.0, eps=1e-8)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available(), "these tests need the GPU"
    osa.lib()                      # raises if the HIP library is missing
    print(f"device: {torch.cuda.get_device_name(0)}", flush=True)
    yield
    osa.opt_debug_set_launch(32768, 0)


def _hp(opt):
    return HP_ADAMW if opt == "adamw" else HP_ADEMAMIX


def _run_and_compare(case, label):
    print(f"case {label}", flush=True)
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    # beyond the bars: the stored states are bit-identical to the oracle's
    states_bit_identical(case, dev, st)
    return dev, ps, st


def test_small_flat_fp32_ten_steps():
    """One fp32 tensor of 2^16+1 elements, lr = wd = 0.1, 10 steps."""
    w = synth.WORKLOADS["adamw_f32_small"]
    case = Case("adamw", "f32", w["sizes"], False, w["steps"], w["hp"], g_std=w["g_std"])
    _run_and_compare(case, "adamw f32 n=65537 x10")


def test_step1_closed_form_on_gpu():
    """The GPU's first step against p0 (1 - lr wd) - lr g/(|g|+eps) in binary64."""
    n = 65537
    case = Case("adamw", "f32", [n], False, 1, HP_ADAMW)
    dev, _ = case.run_gpu()
    p = to_host(dev[0]["p"]).astype(np.float64)
    p0 = case.p0[0].astype(np.float64)
    g = case.grad(1, 0).astype(np.float64)
    lr, wd = np.float64(np.float32(0.1)), np.float64(np.float32(0.1))
    ref = p0 * (1 - lr * wd) - lr * g / (np.abs(g) + np.float64(np.float32(1e-8)))
    assert np.all(np.abs(p - ref) <= 8 * 2.0 ** -24 * (np.abs(p0) + lr))


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("grad_bf16", [False, True])
def test_size_matrix(opt, fmt, grad_bf16):
    """Every size of the matrix as one multi-tensor call, 3 steps."""
    case = Case(opt, fmt, SIZES, grad_bf16, 3, _hp(opt))
    _run_and_compare(case, f"{opt} {fmt} bf16grad={grad_bf16} sizes={SIZES}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_mixed_buckets_and_empty_tensors(fmt):
    """fp32 and bf16 gradients in one call (two launches), with empty tensors;
    the tensor position keys stochastic rounding."""
    sizes = [1000, 0, 4097, 3, 70000, 0, 513]
    bf = [False, True, True, False, True, False, False]
    case = Case("adamw", fmt, sizes, bf, 4, HP_ADAMW)
    _run_and_compare(case, f"mixed buckets {fmt}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_nonfinite_and_zero_gradients(fmt):
    """NaN, +-Inf and zero gradients propagate as in the oracle (NaN payloads
    are compared by position only); a NaN poisons its 8-bit block."""
    def grads(t, k, n):
        g = synth.grads(n, t, k)
        if t == 2:
            g[5] = np.nan
            g[300] = np.inf
            g[301] = -np.inf
            g[600:900] = 0.0
        return g
    case = Case("adamw", fmt, [4097, 1500], False, 3, HP_ADAMW, grad_override=grads)
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)


@pytest.mark.parametrize("fmt", FORMATS)
def test_late_step_and_zero_decay(fmt):
    """Step counts far from 1 (bias corrections near 1) and wd = 0."""
    hp = dict(HP_ADAMW, weight_decay=0.0, lr=1e-3)
    case = Case("adamw", fmt, [70001], True, 2, hp)
    ps, st, _ = case.run_oracle()
    dev, _ = case.run_gpu()
    compare(case, dev, ps, st)
    case2 = Case("adamw", fmt, [5000], False, 3, hp)
    start_t = 997
    ps, st, _ = case2.run_oracle(start=([p.copy() for p in case2.p0],
                                        [oracle.state_zeros(fmt, 5000, "adamw", case2.qs, case2.qu)], start_t))
    dev, _ = case2.run_gpu(t0=start_t)
    compare(case2, dev, ps, st)


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_update_norm_prepass(opt, fmt):
    """max_unorm = 1: the pre-pass norms within 1e-12 relative of the oracle's
    compensated sums, and the clipped steps within the bars."""
    hp = dict(_hp(opt), max_unorm=1.0, lr=1e-3)
    case = Case(opt, fmt, [65537, 0, 3000], [False, False, True], 4, hp)
    ps, st, norms_o = case.run_oracle()
    dev, norms_g = case.run_gpu()
    compare(case, dev, ps, st)
    for (t, k, u2, p2) in norms_o:
        g = norms_g[t - 1]
        # Step 1 sees identical inputs on both sides: 1e-12.  Later steps see
        # an fp32 p that differs from the oracle's within the fp32 bar (the
        # direction u of an fp32 p uses the hardware reciprocal and square
        # root), which shifts sum p^2 by at most ~2*max|dp|/rms(p) ~ 1e-7
        # relative.  The moments, and so sum u^2, are exact.  The pre-pass
        # itself is held to 1e-12 at every step on the oracle's own inputs
        # (test_update_norm_prepass_on_oracle_inputs).
        tol_p = 1e-12 if t == 1 else 1e-7
        assert abs(g[2 * k] - u2) <= 1e-12 * abs(u2), (t, k, g[2 * k], u2)
        assert abs(g[2 * k + 1] - p2) <= tol_p * abs(p2), (t, k, g[2 * k + 1], p2)
    # clipping is active: the scale at step 1 is well below 1
    s = oracle.unorm_scale(1.0, norms_o[0][2], norms_o[0][3])
    assert s < 0.1


def _prepass_on_oracle_inputs(case):
    """At every step t, the pre-pass over the oracle's own p and stored states
    (uploaded to the device) against the oracle's sums over the same inputs:
    both sums within 1e-12 relative (the oracle sums with compensation, the
    kernels in a fixed fp64 order).  Then the oracle takes the step."""
    import torch
    import optimizer_step_amd as osa
    ps = [p.copy() for p in case.p0]
    st = [oracle.state_zeros(case.fmt, n, case.opt, case.qs, case.qu) for n in case.sizes]
    checked = 0
    for t in range(1, case.steps + 1):
        grads = [case.grad(t, k) for k in range(len(case.sizes))]
        dev = [{"p": to_dev(ps[k].copy()), "g": to_dev(grads[k]),
                **{key.replace("a", "absmax"): to_dev(v.copy()) for key, v in st[k].items()}}
               for k in range(len(case.sizes))]
        h = osa.hparams(step=t, seed=case.seed, qmap_signed=case.qs, qmap_unsigned=case.qu, **case.hp)
        un = torch.empty(2 * len(case.sizes), dtype=torch.float64, device="cuda")
        osa.opt_precondition_unorm(case.opt, dev, case.fmt, h, un)
        got = un.cpu().numpy()
        for k in range(len(case.sizes)):
            hp = oracle.make_hp(step=t, seed=case.seed, tensor_index=k, **case.hp)
            u2, p2 = oracle.unorm(case.opt, case.fmt, hp, ps[k], grads[k], qs=case.qs, qu=case.qu, **st[k])
            assert abs(got[2 * k] - u2) <= 1e-12 * abs(u2), (t, k, got[2 * k], u2)
            assert abs(got[2 * k + 1] - p2) <= 1e-12 * abs(p2), (t, k, got[2 * k + 1], p2)
            checked += int(u2 > 0)
            scale = oracle.unorm_scale(case.hp["max_unorm"], u2, p2)
            oracle.step(case.opt, case.fmt, hp, ps[k], grads[k], qs=case.qs, qu=case.qu, scale=scale, **st[k])
    assert checked >= case.steps


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_update_norm_prepass_on_oracle_inputs(opt, fmt):
    hp = dict(_hp(opt), max_unorm=1.0, lr=1e-3)
    _prepass_on_oracle_inputs(Case(opt, fmt, [65537, 0, 3000], [False, False, True], 4, hp))


@pytest.mark.parametrize("fmt", ["f32", "q8", "fp4_sr"])
def test_update_norm_prepass_on_oracle_inputs_skip_zeros(fmt):
    """skip_zeros: an element with a zero gradient counts no update."""
    def grads(t, k, n):
        g = synth.grads(n, t, k)
        g[::7] = 0.0
        g[100:400] = -0.0
        return g
    hp = dict(_hp("adamw"), max_unorm=1.0, lr=1e-3, skip_zeros=True)
    _prepass_on_oracle_inputs(Case("adamw", fmt, [4097, 1500], False, 3, hp, grad_override=grads))


@pytest.mark.parametrize("fmt", ["f32", "bf16_sr", "fp8_rn"])
def test_update_norm_spans_sum_groups(fmt):
    """Tensors of more than 1024 partials (2^20 elements) have their norms
    summed over several first-level groups, one workgroup each, then in
    order; an empty and a small tensor sit between them in the list."""
    hp = dict(_hp("adamw"), max_unorm=1.0, lr=1e-3)
    sizes = [2 * 2**20 + 3001, 0, 1000, 2**20, 3 * 2**20]
    case = Case("adamw", fmt, sizes, [False, False, True, True, False], 2, hp)
    ps, st, norms_o = case.run_oracle()
    dev, norms_g = case.run_gpu()
    compare(case, dev, ps, st)
    for (t, k, u2, p2) in norms_o:
        g = norms_g[t - 1]
        tol_p = 1e-12 if t == 1 else 1e-7   # as in test_update_norm_prepass
        assert abs(g[2 * k] - u2) <= 1e-12 * abs(u2), (t, k, g[2 * k], u2)
        assert abs(g[2 * k + 1] - p2) <= tol_p * abs(p2), (t, k, g[2 * k + 1], p2)
    _prepass_on_oracle_inputs(case)


def test_update_norm_is_deterministic():
    """Ten pre-pass runs over a multi-chunk tensor give identical bits."""
    import torch
    import optimizer_step_amd as osa
    n = 3 * 2**20 + 5
    dev = [{"p": to_dev(synth.params(n)), "g": to_dev(synth.grads(n, 1)),
            **osa.state_buffers("f32", n)}]
    dev[0]["s1"].copy_(to_dev(synth.grads(n, 7)))
    dev[0]["s2"].copy_(to_dev(np.abs(synth.grads(n, 8, std=1e-2)) ** 2))
    hp = osa.hparams(step=5, max_unorm=1.0)
    outs = []
    for _ in range(10):
        u = torch.empty(2, dtype=torch.float64, device="cuda")
        osa.opt_precondition_unorm("adamw", dev, "f32", hp, u)
        outs.append(u.cpu().numpy().view(np.uint64).copy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("fmt", FORMATS)
def test_repeat_runs_are_bit_identical(fmt):
    case = Case("ademamix", fmt, [100_003, 777], True, 3, HP_ADEMAMIX)
    a = Case.host(case.run_gpu()[0])
    b = Case.host(case.run_gpu()[0])
    for x, y in zip(a, b):
        for key in x:
            assert nan_equal_bits(x[key], y[key]), key


@pytest.mark.parametrize("fmt", FORMATS)
def test_chunk_size_and_grid_do_not_change_results(fmt):
    import optimizer_step_amd as osa
    case = Case("adamw", fmt, [300_001, 4097], [False, True], 3, dict(HP_ADAMW, max_unorm=1.0))
    try:
        results = []
        for chunk, wgs in ((32768, 0), (1024, 1), (65536, 3), (4096, 64), (32768, 8)):
            osa.opt_debug_set_launch(chunk, wgs)
            results.append(Case.host(case.run_gpu()[0]))
    finally:
        osa.opt_debug_set_launch(32768, 0)
    for r in results[1:]:
        for x, y in zip(results[0], r):
            for key in x:
                assert nan_equal_bits(x[key], y[key]), key


@pytest.mark.parametrize("fmt", FORMATS)
def test_resume_from_copied_state(fmt):
    """6 steps equal 3 steps, a copy of every buffer out and back in, and 3
    more steps: the state lives only in the caller's buffers."""
    case = Case("ademamix", fmt, [50_001], True, 6, HP_ADEMAMIX)
    full = Case.host(case.run_gpu(6)[0])
    dev, _ = case.run_gpu(3)
    snap = Case.host(dev)
    dev2 = case.alloc_gpu(start=([s["p"] for s in snap], [{k: v for k, v in s.items() if k != "p"} for s in snap]))
    part = Case.host(case.run_gpu(3, dev=dev2, t0=3)[0])
    for x, y in zip(full, part):
        for key in x:
            assert nan_equal_bits(x[key], y[key]), key


def test_streams_other_than_the_default():
    import torch
    case = Case("adamw", "bf16_sr", [20_000], True, 2, HP_ADAMW)
    ps, st, _ = case.run_oracle()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dev, _ = case.run_gpu(stream=s)
    compare(case, dev, ps, st)


def test_steps_alternating_between_two_streams():
    """The same tensor list stepped on two streams in turn, each ordered after
    the other as a caller would: every call after the first finds the list's
    tables already uploaded from the other stream (and the pre-pass partials
    last written there), and the results are the oracle's."""
    import torch
    import optimizer_step_amd as osa
    hp = dict(HP_ADAMW, max_unorm=1.0)
    case = Case("adamw", "q8", [5000, 70_000], True, 4, hp)
    ps, st, _ = case.run_oracle()
    dev = case.alloc_gpu()
    tl = osa.TensorList(dev)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for t in range(1, case.steps + 1):
        s, other = streams[t % 2], streams[(t + 1) % 2]
        s.wait_stream(other)
        with torch.cuda.stream(s):
            for k in range(len(case.sizes)):
                dev[k]["g"].copy_(to_dev(case.grad(t, k)))
            h = osa.hparams(step=t, seed=case.seed, qmap_signed=case.qs, qmap_unsigned=case.qu, **hp)
            unorm = torch.empty(2 * len(case.sizes), dtype=torch.float64, device="cuda")
            osa.opt_precondition_unorm("adamw", tl, "q8", h, unorm, stream=s)
            osa.opt_step_adamw(tl, "q8", h, unorm, stream=s)
            unorm.record_stream(s)
    torch.cuda.synchronize()
    compare(case, dev, ps, st)
    states_bit_identical(case, dev, st)


def test_refused_call_leaves_everything_unchanged():
    """An argument the library refuses (here a codebook too dense for its
    lookup table) returns an error before anything is enqueued: p and the
    states keep their bits, and the next valid call steps as usual."""
    import torch
    import optimizer_step_amd as osa
    case = Case("adamw", "q8", [3000], True, 1, HP_ADAMW)
    dev = case.alloc_gpu()
    dev[0]["g"].copy_(to_dev(case.grad(1, 0)))
    before = {k: v.clone() for k, v in dev[0].items()}
    dense = np.linspace(-1, 1, 256).astype(np.float32)
    dense[200] = np.nextafter(dense[201], np.float32(-1))
    dense[199] = np.nextafter(dense[200], np.float32(-1))
    with pytest.raises(osa.OptError) as e:
        osa.opt_step_adamw(osa.TensorList(dev), "q8",
                           osa.hparams(step=1, qmap_signed=dense, qmap_unsigned=case.qu, **HP_ADAMW))
    assert e.value.status == osa.OPT_EUNSUPPORTED
    torch.cuda.synchronize()
    for k, v in dev[0].items():
        assert torch.equal(v.view(torch.uint8) if v.dtype != torch.uint8 else v,
                           before[k].view(torch.uint8) if v.dtype != torch.uint8 else before[k]), k
    ps, st, _ = case.run_oracle()
    dev2, _ = case.run_gpu(dev=dev)
    compare(case, dev2, ps, st)


def test_binding_refuses_short_or_strided_buffers():
    """The library sees pointers only, so the binding refuses buffers it
    would read out of bounds: a strided view, a state shorter than the
    format needs, a short absmax array, a short update-norm buffer."""
    import torch
    import optimizer_step_amd as osa
    n = 1000
    f = lambda k, dt=torch.float32: torch.zeros(k, dtype=dt, device="cuda")
    ok = {"p": f(n), "g": f(n), "s1": f(n), "s2": f(n)}
    osa.opt_step_adamw([ok], "f32", osa.hparams())
    bad = [dict(ok, p=f(2 * n)[::2]), dict(ok, s2=f(n - 1)), dict(ok, g=f(n + 4))]
    for d in bad:
        with pytest.raises(ValueError):
            osa.opt_step_adamw([d], "f32", osa.hparams())
    fp4 = {"p": f(n), "g": f(n), "s1": f(n // 2, torch.uint8), "s2": f(n // 2 - 1, torch.uint8),
           "absmax1": f(4), "absmax2": f(4)}
    with pytest.raises(ValueError):
        osa.opt_step_adamw([fp4], "fp4_rn", osa.hparams())
    fp4["s2"] = f(n // 2, torch.uint8)
    fp4["absmax2"] = f(3)
    with pytest.raises(ValueError):
        osa.opt_step_adamw([fp4], "fp4_rn", osa.hparams())
    with pytest.raises(ValueError):
        osa.opt_precondition_unorm("adamw", [ok], "f32", osa.hparams(max_unorm=1.0), f(1, torch.float64))
    torch.cuda.synchronize()


def test_two_host_threads_two_streams():
    """Two host threads step two different tensor lists at the same time, each
    on a stream of its own (8-bit states with the pre-pass on one, BF16-SR on
    the other): the calls serialize inside the library, each list keeps its
    own tables, and both results are the oracle's."""
    import threading
    import torch
    import optimizer_step_amd as osa
    cases = [Case("adamw", "q8", [5000, 70_000], True, 4, dict(HP_ADAMW, max_unorm=1.0)),
             Case("ademamix", "bf16_sr", [33_333, 1024], False, 4, HP_ADEMAMIX)]
    want = [c.run_oracle() for c in cases]
    devs = [c.alloc_gpu() for c in cases]
    torch.cuda.synchronize()
    errors = []

    def worker(c, dev):
        try:
            s = torch.cuda.Stream()
            tl = osa.TensorList(dev)
            fn = osa.opt_step_adamw if c.opt == "adamw" else osa.opt_step_ademamix
            with torch.cuda.stream(s):
                for t in range(1, c.steps + 1):
                    for k in range(len(c.sizes)):
                        dev[k]["g"].copy_(to_dev(c.grad(t, k)))
                    h = osa.hparams(step=t, seed=c.seed, qmap_signed=c.qs, qmap_unsigned=c.qu, **c.hp)
                    unorm = None
                    if c.hp.get("max_unorm", 0.0) > 0:
                        unorm = torch.empty(2 * len(c.sizes), dtype=torch.float64, device="cuda")
                        osa.opt_precondition_unorm(c.opt, tl, c.fmt, h, unorm, stream=s)
                    fn(tl, c.fmt, h, unorm, stream=s)
                s.synchronize()
        except Exception as e:     # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(c, d)) for c, d in zip(cases, devs)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads) and not errors, errors
    for c, dev, (ps, st, _) in zip(cases, devs, want):
        compare(c, dev, ps, st)
        states_bit_identical(c, dev, st)


# ---------------------------------------------------------------------------
# test hooks: the device functions the kernels use

def test_philox_words_match_oracle():
    import torch
    import optimizer_step_amd as osa
    for j0, n, k, t in ((0, 1 << 22, 0, 1), ((1 << 34) - (1 << 20), 1 << 21, 7, 123456), (12345, 1001, 3, 2**31 + 5)):
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        osa.opt_debug_philox(synth.SR_SEED, t, k, j0, out)
        got = out.cpu().numpy().view(np.uint32)
        ref = oracle.sr_words(synth.SR_SEED, t, k, j0, n)
        assert np.array_equal(got, ref)


def test_bf16_rounding_matches_oracle():
    import torch
    import optimizer_step_amd as osa
    rng = np.random.default_rng(17)
    hi = (np.arange(65536, dtype=np.uint32) << 16)
    words = np.concatenate([hi | np.uint32(lo) for lo in (0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF)] +
                           [rng.integers(0, 2**32, 1 << 21, dtype=np.uint64).astype(np.uint32)])
    x = words.view(np.float32)
    r = rng.integers(0, 2**32, x.size, dtype=np.uint64).astype(np.uint32)
    xd = to_dev(x)
    rd = torch.from_numpy(r.view(np.int32)).cuda()
    out = torch.empty(x.size, dtype=torch.int16, device="cuda")
    osa.opt_debug_round_bf16(xd, None, out)
    rne = out.cpu().numpy().view(np.uint16)
    assert nan_equal_bits(rne, oracle.bf16_rne_array(x))
    osa.opt_debug_round_bf16(xd, rd, out)
    sr = out.cpu().numpy().view(np.uint16)
    assert nan_equal_bits(sr, oracle.bf16_sr_array(x, r & 0xFFFF))


@pytest.mark.parametrize("signed", [True, False])
def test_quantizer_matches_oracle(signed):
    import torch
    import optimizer_step_amd as osa
    T = synth.codebook_signed() if signed else synth.codebook_unsigned()
    mids = ((T[:-1].astype(np.float64) + T[1:].astype(np.float64)) / 2).astype(np.float32)
    rng = np.random.default_rng(4)
    x = np.concatenate([T, mids, np.nextafter(mids, np.float32(2)), np.nextafter(mids, np.float32(-2)),
                        np.array([0.0, -0.0, 1.0, -1.0, np.nan, 1e-30], dtype=np.float32),
                        rng.uniform(-1, 1, 1 << 20).astype(np.float32),
                        (rng.uniform(-1, 1, 1 << 20) ** 9).astype(np.float32)]).astype(np.float32)
    if not signed:
        x = np.abs(x)
    out = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    osa.opt_debug_quantize(T, signed, to_dev(x), out)
    assert np.array_equal(out.cpu().numpy(), oracle.quantize_array(T, x))


@pytest.mark.parametrize("signed", [True, False], ids=["signed", "unsigned"])
def test_device_lookup_on_every_value_in_unit_interval(signed):
    """The step's 8-bit lookup on the device, on every binary32 word in
    [-1, 1] (inputs generated on the device, 2^28 words a launch).  Expected:
    the count of thresholds tau_i <= x, tau_i the smallest binary32 above the
    binary64 midpoint (T_i + T_{i+1})/2 -- the nearest entry, ties to the
    lower index; an unsigned table gives 0 to every x <= 0."""
    import torch
    import optimizer_step_amd as osa
    T = synth.codebook_signed() if signed else synth.codebook_unsigned()
    t = (T[:-1].astype(np.float64) + T[1:].astype(np.float64)) / 2
    tau = t.astype(np.float32)
    tau[tau.astype(np.float64) <= t] = np.nextafter(tau[tau.astype(np.float64) <= t], np.float32(np.inf))
    tau_d = torch.from_numpy(tau).cuda()
    one, chunk = 0x3F800000, 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    checked = 0
    for neg in (False, True):
        for lo in range(0, one + 1, chunk):
            hi = min(lo + chunk, one + 1)
            w = torch.arange(lo, hi, dtype=torch.int64, device="cuda")
            if neg:
                w = w - 2**31                        # the same magnitudes with the sign bit set (int32 view)
            x = w.to(torch.int32).view(torch.float32)
            o = out[:hi - lo]
            osa.opt_debug_quantize(T, signed, x, o)
            want = torch.searchsorted(tau_d, x, right=True).to(torch.uint8)
            if not signed and neg:
                want.zero_()
            bad = int((o != want).sum())
            assert bad == 0, (signed, neg, lo, bad)
            checked += hi - lo
            del w, x, want
    assert checked == 2 * (one + 1)
    torch.cuda.synchronize()

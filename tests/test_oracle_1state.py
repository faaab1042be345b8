"""Pins of the oracle's skip_zeros path and of the one-state optimizers
(bitsandbytes PR "Fix decoupled weight decay ordering in the CUDA
Adam/AdEMAMix kernels": intro -- coupled L2 for momentum, RMSprop and
Adagrad, decoupled decay for Lion -- and "Not covered" -- skip_zeros skips
the decay with the update).

Momentum, RMSprop and Adagrad are pinned to torch.optim's SGD, RMSprop and
Adagrad run in float64 (a library routine; tolerance for the fp32 recipe);
Lion to its first-step closed form, to the exact size of every parameter move
(lr times a sign, up to the rounding of p), to its signSGD special case, and to a float64 run of its
EMA; skip_zeros to the plain step on the other elements."""
import numpy as np
import pytest

import oracle
import synth


def _torch_run(name, p0, grads, lr, b1, eps, wd):
    import torch
    p = torch.tensor(p0.astype(np.float64), requires_grad=True)
    if name == "momentum":
        opt = torch.optim.SGD([p], lr=lr, momentum=b1, weight_decay=wd, foreach=False)
    elif name == "rmsprop":
        opt = torch.optim.RMSprop([p], lr=lr, alpha=b1, eps=eps, weight_decay=wd, foreach=False)
    else:
        opt = torch.optim.Adagrad([p], lr=lr, eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        p.grad = torch.tensor(g.astype(np.float64))
        opt.step()
    return p.detach().numpy()


@pytest.mark.parametrize("wd", [0.0, 0.05])
@pytest.mark.parametrize("name", ["momentum", "rmsprop", "adagrad"])
def test_coupled_l2_family_matches_torch_optim(name, wd):
    n, T = 4000, 12
    lr, b1, eps = 1e-2, 0.9, 1e-8
    p0 = synth.params(n, std=0.5)
    grads = [synth.grads(n, t, std=1e-1) for t in range(1, T + 1)]
    p = p0.copy()
    s = np.zeros(n, np.float32)
    for t, g in enumerate(grads, 1):
        oracle.step_1state(name, "f32", oracle.make_hp(lr=lr, beta1=b1, eps=eps, weight_decay=wd, step=t), p, g, s)
    ref = _torch_run(name, p0, grads, lr, b1, eps, wd)
    # the fp32 recipe drifts from the float64 run by a few ulp per step
    assert np.max(np.abs(p - ref)) <= 1e-5 * np.max(np.abs(ref))
    assert np.max(np.abs(p - p0)) > 1e-3                          # the steps moved p


def test_lion_first_step_closed_form():
    n = 3001
    p0 = synth.params(n)
    g = synth.grads(n, 1)
    g[:5] = 0.0
    lr, wd, b2 = np.float32(1e-3), np.float32(0.1), np.float32(0.99)
    p = p0.copy()
    m = np.zeros(n, np.float32)
    oracle.step_1state("lion", "f32", oracle.make_hp(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.99), p, g, m)
    d = np.float32(1) - lr * wd
    want = (p0 * d - lr * np.sign(g)).astype(np.float32)
    assert np.array_equal(p.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(m, ((np.float32(1) - b2) * g).astype(np.float32))


def test_lion_moves_by_lr_and_reduces_to_sign_sgd():
    n, T = 2000, 8
    p = synth.params(n)
    m = np.zeros(n, np.float32)
    hp = dict(lr=2.0 ** -10, weight_decay=0.0, beta1=0.9, beta2=0.99)
    for t in range(1, T + 1):
        before = p.copy()
        g = synth.grads(n, t)
        oracle.step_1state("lion", "f32", oracle.make_hp(step=t, **hp), p, g, m)
        # with wd = 0 every move is lr (or 0) up to the rounding of p - lr*sign
        moved = np.abs(p.astype(np.float64) - before.astype(np.float64))
        half_ulp = 0.5 * np.spacing(np.abs(p)).astype(np.float64)
        assert np.all((np.abs(moved - 2.0 ** -10) <= half_ulp) | (moved == 0))
        assert np.mean(moved == 0) < 0.01
    # b1 = b2 = 0: signSGD with decoupled decay
    p = synth.params(n)
    p0 = p.copy()
    m = np.zeros(n, np.float32)
    g = synth.grads(n, 3)
    oracle.step_1state("lion", "f32", oracle.make_hp(lr=1e-3, weight_decay=0.2, beta1=0.0, beta2=0.0), p, g, m)
    want = (p0 * (np.float32(1) - np.float32(1e-3) * np.float32(0.2)) - np.float32(1e-3) * np.sign(g)).astype(np.float32)
    assert np.array_equal(p, want) and np.array_equal(m, g)


def test_lion_momentum_is_an_ema():
    n, T = 1000, 20
    b2 = 0.99
    m = np.zeros(n, np.float32)
    p = synth.params(n)
    ref = np.zeros(n)
    for t in range(1, T + 1):
        g = synth.grads(n, t)
        oracle.step_1state("lion", "f32", oracle.make_hp(lr=1e-4, beta1=0.9, beta2=b2, step=t), p, g, m)
        ref = np.float64(np.float32(b2)) * ref + np.float64(np.float32(1) - np.float32(b2)) * g
    assert np.max(np.abs(m - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_momentum_first_step_and_reset():
    """The buffer starts as the gradient on its first step, and again after a
    reset."""
    n = 500
    g1, g2 = synth.grads(n, 1), synth.grads(n, 2)
    p = synth.params(n)
    m = np.zeros(n, np.float32)
    oracle.step_1state("momentum", "f32", oracle.make_hp(lr=1e-2, beta1=0.9, step=1, reset_interval=1), p, g1, m)
    assert np.array_equal(m, g1)
    oracle.step_1state("momentum", "f32", oracle.make_hp(lr=1e-2, beta1=0.9, step=2, reset_interval=1), p, g2, m)
    assert np.array_equal(m, g2)                                    # every step restarts
    oracle.step_1state("momentum", "f32", oracle.make_hp(lr=1e-2, beta1=0.9, step=3), p, g1, m)
    assert np.array_equal(m, (np.float32(0.9) * g2 + g1).astype(np.float32))


@pytest.mark.parametrize("name", ["momentum", "rmsprop", "adagrad", "lion"])
def test_one_state_bf16_is_f32_then_rounding(name):
    n = 3000
    p0 = synth.params(n)
    s0 = synth.bf16_words(np.abs(synth.grads(n, 9)) * 0.1)
    g = synth.grads(n, 4)
    hp = oracle.make_hp(lr=1e-2, beta1=0.9, beta2=0.99, weight_decay=0.01, step=4, seed=3)
    pa, sa = p0.copy(), oracle.widen_bf16(s0).copy()
    oracle.step_1state(name, "f32", hp, pa, g, sa)
    pb, sb = p0.copy(), s0.copy()
    oracle.step_1state(name, "bf16_rn", hp, pb, g, sb)
    assert np.array_equal(pa, pb) and np.array_equal(sb, oracle.bf16_rne_array(sa))
    pc, sc = p0.copy(), s0.copy()
    oracle.step_1state(name, "bf16_sr", hp, pc, g, sc)
    r = oracle.sr_words(3, 4, 0, 0, n) & 0xFFFF
    assert np.array_equal(pa, pc) and np.array_equal(sc, oracle.bf16_sr_array(sa, r))


# ---------------------------------------------------------------------------
# skip_zeros

@pytest.mark.parametrize("fmt", ["f32", "bf16_sr", "q8", "fp8_rn"])
@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_skip_zeros_two_state(opt, fmt):
    """Elements whose gradient is exactly zero keep p (no decay either) and
    their stored moments; fp32 states elsewhere match the plain step."""
    n = 1000
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    hp = dict(lr=1e-2, weight_decay=0.1)
    p_a = synth.params(n)
    st_a = oracle.state_zeros(fmt, n, opt, qs, qu)
    p_b = p_a.copy()
    st_b = oracle.state_zeros(fmt, n, opt, qs, qu)
    for t in range(1, 5):
        g = synth.grads(n, t)
        zero = np.zeros(n, bool)
        zero[t::7] = True
        g[zero] = 0.0
        before = p_a.copy()
        st_before = {k: v.copy() for k, v in st_a.items()}
        oracle.step(opt, fmt, oracle.make_hp(step=t, skip_zeros=True, **hp), p_a, g, qs=qs, qu=qu, **st_a)
        oracle.step(opt, fmt, oracle.make_hp(step=t, **hp), p_b, g, qs=qs, qu=qu, **st_b)
        assert np.array_equal(p_a[zero], before[zero])
        if t > 1:
            assert not np.array_equal(p_b[zero], before[zero])        # without the skip they decay
        if fmt in ("f32", "bf16_sr"):
            for k in st_a:
                assert np.array_equal(st_a[k][zero], st_before[k][zero])
        if fmt == "f32" and t == 1:
            assert np.array_equal(p_a[~zero], p_b[~zero])


def test_skip_zeros_one_state_and_unorm():
    n = 800
    g = synth.grads(n, 2)
    g[::3] = 0.0
    for name in ("momentum", "rmsprop", "adagrad", "lion"):
        p = synth.params(n)
        s = np.abs(synth.grads(n, 5)).astype(np.float32)
        p0, s0 = p.copy(), s.copy()
        oracle.step_1state(name, "f32", oracle.make_hp(lr=1e-2, weight_decay=0.1, step=2, skip_zeros=True), p, g, s)
        assert np.array_equal(p[::3], p0[::3]) and np.array_equal(s[::3], s0[::3])
        assert not np.array_equal(p[1::3], p0[1::3])
    # the update-norm pre-pass counts no update for a skipped element
    p = synth.params(n)
    st = oracle.state_zeros("f32", n)
    u_skip, _ = oracle.unorm("adamw", "f32", oracle.make_hp(skip_zeros=True), p, g, **st)
    gz = g.copy()
    keep = np.ones(n, bool)
    keep[::3] = False
    u_part, _ = oracle.unorm("adamw", "f32", oracle.make_hp(), p[keep].copy(), gz[keep].copy(),
                             **oracle.state_zeros("f32", int(keep.sum())))
    assert abs(u_skip - u_part) <= 1e-12 * u_part

"""The resident-workgroup cap of the element-wise and one-state step kernels
(a launch-time LDS reservation) changes where and when tiles run, never what
they compute: every cap gives the same bits as the uncapped launch, and the
capped launches still meet the oracle's bars."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import Case, compare, nan_equal_bits, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [1, 257, 4099, 2 * 32768 + 513, 5 * 1024]
CAPS = [0, 2, 3, 4, 5, 8]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield
    osa.opt_debug_set_wg_cap(-1)
    torch.cuda.synchronize()


def _hp():
    return dict(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.999, eps=1e-8)


def _bits(host):
    return [{k: v.view(np.uint8).copy() for k, v in d.items()} for d in host]


@pytest.mark.parametrize("fmt,clip,grad_bf16", [("f32", None, True), ("f32", (1.0, 2), True), ("bf16_sr", None, True),
                                               ("f32", None, False)])
def test_two_state_step_independent_of_cap(fmt, clip, grad_bf16):
    import optimizer_step_amd as osa
    case = Case("adamw", fmt, SIZES, grad_bf16, 2, _hp(), clip=clip)
    try:
        osa.opt_debug_set_wg_cap(0)
        ref = _bits(Case.host(case.run_gpu()[0]))
        for cap in CAPS[1:] + [-1]:
            osa.opt_debug_set_wg_cap(cap)
            dev, _ = case.run_gpu()
            got = _bits(Case.host(dev))
            for k in range(len(SIZES)):
                for key in ref[k]:
                    assert np.array_equal(got[k][key], ref[k][key]), (cap, k, key)
        osa.opt_debug_set_wg_cap(3)
        dev, _ = case.run_gpu()
        ps, st, _ = case.run_oracle()
        compare(case, dev, ps, st)
    finally:
        osa.opt_debug_set_wg_cap(-1)


@pytest.mark.parametrize("grad_bf16", [True, False])
@pytest.mark.parametrize("name", ["momentum", "lion"])
def test_one_state_step_independent_of_cap(name, grad_bf16):
    import torch
    import optimizer_step_amd as osa
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.05)
    ps = [synth.params(n, k, std=0.5) for k, n in enumerate(SIZES)]
    gs = [[(synth.bf16_words if grad_bf16 else np.asarray)(synth.grads(n, t, k, std=1e-1)) for k, n in enumerate(SIZES)]
          for t in (1, 2)]
    ss = [np.zeros(n, np.float32) for n in SIZES]
    for t in (1, 2):
        for k in range(len(SIZES)):
            oracle.step_1state(name, "f32", oracle.make_hp(step=t, seed=synth.SR_SEED, tensor_index=k, **hp),
                               ps[k], gs[t - 1][k], ss[k])
    try:
        for cap in [0, 5, 3, -1]:
            osa.opt_debug_set_wg_cap(cap)
            dev = [{"p": to_dev(synth.params(n, k, std=0.5)), "g": to_dev(gs[0][k]),
                    "s1": torch.zeros(n, dtype=torch.float32, device="cuda")} for k, n in enumerate(SIZES)]
            tl = osa.TensorList(dev)
            for t in (1, 2):
                for k in range(len(SIZES)):
                    dev[k]["g"].copy_(to_dev(gs[t - 1][k]))
                osa.opt_step_1state(name, tl, "f32", osa.hparams(step=t, seed=synth.SR_SEED, **hp))
            torch.cuda.synchronize()
            for k in range(len(SIZES)):
                assert nan_equal_bits(to_host(dev[k]["p"]), ps[k]), (cap, k)
                assert nan_equal_bits(to_host(dev[k]["s1"]), ss[k]), (cap, k)
    finally:
        osa.opt_debug_set_wg_cap(-1)


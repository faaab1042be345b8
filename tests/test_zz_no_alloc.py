"""The allocation-free AdamW step (opt_step_adamw_noalloc) against the
ordinary one (opt_step_adamw): the same kernels over the same inputs, so every
output word must be identical.  Two calls in a row, the second over a smaller
list, each compared on identical copies of the inputs; then a list whose
tables exceed the fixed array is refused with nothing changed."""
import numpy as np
import pytest

import synth
from tests.gpu_common import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield


def _list(fmt, sizes, gd, seed, t_steps=2):
    """Fresh states, p ~ N(0, 0.02); returns the tensor dicts and a grad maker."""
    import torch
    import optimizer_step_amd as osa
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    out = []
    for k, n in enumerate(sizes):
        d = {"p": to_dev(synth.params(n, k + seed)),
             "g": torch.zeros(n, dtype=torch.bfloat16 if gd[k] else torch.float32, device="cuda")}
        d.update(osa.state_buffers(fmt, n, "adamw", qmap_signed=qs, qmap_unsigned=qu))
        out.append(d)
    return out, qs, qu


def _clone(lst):
    return [{k: v.clone() for k, v in d.items()} for d in lst]


def _same(a, b):
    import torch
    for da, db in zip(a, b):
        for key in da:
            if not torch.equal(da[key].view(torch.uint8), db[key].view(torch.uint8)):
                return key
    return None


@pytest.mark.parametrize("fmt", ["f32", "bf16_sr", "q8", "fp8_sr"])
def test_no_alloc_step_matches_the_step(fmt):
    import torch
    import optimizer_step_amd as osa
    calls = [([70001, 4096, 3, 300000], [True, False, True, True]),     # mixed gradient storage: 2 launches
             ([1025, 256], [False, True])]                           # the second call: a smaller list
    for c, (sizes, gd) in enumerate(calls):
        ref, qs, qu = _list(fmt, sizes, gd, seed=10 * c)
        mine = _clone(ref)
        for t in (1, 2, 3):
            for k, n in enumerate(sizes):
                g = synth.grads(n, t, k + 10 * c, std=1e-2)
                g = to_dev(synth.bf16_words(g)) if gd[k] else to_dev(g)
                ref[k]["g"].copy_(g)
                mine[k]["g"].copy_(g)
            h = osa.hparams(step=t, lr=1e-2, weight_decay=0.1, seed=synth.SR_SEED + c, qmap_signed=qs,
                            qmap_unsigned=qu)
            osa.opt_step_adamw(osa.TensorList(ref), fmt, h)
            osa.opt_step_adamw_noalloc(osa.TensorList(mine), fmt, h)
        torch.cuda.synchronize()
        diff = _same(ref, mine)
        assert diff is None, (fmt, c, diff)


def test_no_alloc_step_refuses_tables_beyond_its_array():
    """20,000 four-element tensors need 2.2 MB of tensor records: refused with
    OPT_EUNSUPPORTED before anything is enqueued, outputs unchanged; the
    ordinary step takes the same list."""
    import torch
    import optimizer_step_amd as osa
    n, k = 20000, 4
    P = to_dev(synth.params(n * k))
    G = to_dev(synth.grads(n * k, 1))
    M = torch.zeros(n * k, dtype=torch.float32, device="cuda")
    V = torch.zeros(n * k, dtype=torch.float32, device="cuda")
    lst = [{"p": P[i * k:(i + 1) * k], "g": G[i * k:(i + 1) * k], "s1": M[i * k:(i + 1) * k],
            "s2": V[i * k:(i + 1) * k]} for i in range(n)]
    before = P.clone()
    with pytest.raises(osa.OptError) as e:
        osa.opt_step_adamw_noalloc(osa.TensorList(lst), "f32", osa.hparams(step=1))
    assert e.value.status == osa.OPT_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(P, before) and int(torch.count_nonzero(M)) == 0
    osa.opt_step_adamw(osa.TensorList(lst), "f32", osa.hparams(step=1))
    torch.cuda.synchronize()
    assert not torch.equal(P, before)

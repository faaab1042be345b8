"""Pins across state formats: one step from a fresh optimizer moves p the same
way whatever the storage (the bitsandbytes PR 'Fix decoupled weight decay
ordering in the CUDA Adam/AdEMAMix kernels', Verification: AdamW-32bit and
AdamW-8bit show identical numbers), because the zero state reads back exactly
and the update uses the unrounded fp32 moments."""
import numpy as np
import pytest

import synth
from tests.common import run_oracle

QS, QU = synth.codebook_signed(), synth.codebook_unsigned()


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("grad_bf16", [False, True])
def test_step1_identical_across_formats(opt, grad_bf16):
    n = 4099
    g = synth.grads(n, 1, bf16=grad_bf16)
    p0 = synth.params(n)
    hp = dict(lr=0.1, weight_decay=0.1)
    ps = []
    for fmt in ("f32", "bf16_rn", "bf16_sr", "q8"):
        p, _ = run_oracle(opt, fmt, n, 1, hp, grad_fn=lambda t: g, p=p0.copy(), qs=QS, qu=QU,
                          seed=synth.SR_SEED)
        ps.append(p.view(np.uint32))
    for p in ps[1:]:
        assert np.array_equal(p, ps[0])


def test_later_steps_differ_across_formats():
    """Non-vacuity: from step 2 on, rounded or quantized states change p."""
    n = 4099
    p0 = synth.params(n)
    pf, _ = run_oracle("adamw", "f32", n, 3, dict(lr=0.1), p=p0.copy())
    pb, _ = run_oracle("adamw", "bf16_rn", n, 3, dict(lr=0.1), p=p0.copy())
    pq, _ = run_oracle("adamw", "q8", n, 3, dict(lr=0.1), p=p0.copy(), qs=QS, qu=QU)
    assert not np.array_equal(pf, pb) and not np.array_equal(pf, pq)

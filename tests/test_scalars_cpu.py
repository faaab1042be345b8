"""The per-call scalars the library forms on the host (1 - beta, the bias
corrections c = 1 - beta^t' and their reciprocals, 1 - lr*wd, lr) against the
oracle's, bit for bit, over many betas, steps and reset intervals.  The
library raises beta to the power by binary exponentiation in binary64, the
oracle with libm pow; both round 1 - beta^t' once to binary32 (the issue
"Investigate SM103 bias-correction broadcast in 32-bit optimizers", Problem:
one value per call)."""
import os

import numpy as np
import pytest

import oracle

BETAS = [0.0, 0.5, 0.75, 0.8, 0.9, 0.95, 0.98, 0.99, 0.995, 0.997, 0.999, 0.9995, 0.9999, 0.99999]


@pytest.fixture(scope="module")
def L():
    import optimizer_step_amd as osa
    if not os.path.exists(osa.LIB_PATH):
        from optimizer_step_amd import build
        build.build()
    return osa


def _steps():
    return list(range(1, 3001)) + [4096, 10 ** 4, 65535, 10 ** 5, 123457, 10 ** 6, 10 ** 7, 2 ** 31 + 5]


@pytest.mark.parametrize("beta", BETAS)
def test_host_scalars_match_oracle(L, beta):
    b2 = BETAS[(BETAS.index(beta) + 5) % len(BETAS)]
    for t in _steps():
        for R in (0, 7, 1000):
            hp = dict(lr=3e-4, weight_decay=0.1, beta1=beta, beta2=b2, beta3=0.9999, alpha=5.0, eps=1e-8,
                      reset_interval=R)
            got = L.opt_debug_scalars(L.hparams(step=t, **hp))
            want = oracle.scalars(oracle.make_hp(step=t, **hp))
            # om1, om2, om3, c1, c2 | d, lam
            assert np.array_equal(got[:5].view(np.uint32), want[:5].view(np.uint32)), (beta, b2, t, R, got, want)
            assert np.array_equal(got[7:9].view(np.uint32), want[5:7].view(np.uint32)), (beta, t, R)
            c = got[3:5]
            assert np.array_equal(got[5:7], np.float32(1.0) / c), (beta, t, R)   # RN(1/c)
            assert got[9] == 1.0

"""The fast direction's error bound (moments_fast), on which the 16-bit
parameter path's exactness rests: wherever the bound is finite, the fast
direction (hardware reciprocal and square root) lies within half of it of the
exact recipe's (correctly rounded division and square root).  Half, because
the bound carries a factor two of margin over the analysis; the check is of
the analysis itself.  Inputs span the binary32 range: log-uniform magnitudes
with random signs, exact zeros, moments at the edges of the bound's domain,
and AdEMAMix numerators that nearly cancel."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

N = 1 << 21


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    yield


def _logu(rng, n, lo, hi, signed=True):
    x = np.exp2(rng.uniform(lo, hi, n))
    if signed:
        x *= rng.choice([-1.0, 1.0], n)
    return x


def _inputs(seed, opt, beta1, step, alpha):
    rng = np.random.default_rng(seed)
    g = _logu(rng, N, -60, 20)
    m = _logu(rng, N, -110, 40)
    v = _logu(rng, N, -120, 80, signed=False)
    # exact zeros, and moments near the thresholds of the bound's domain
    g[rng.random(N) < 0.02] = 0.0
    m[rng.random(N) < 0.02] = 0.0
    v[rng.random(N) < 0.02] = 0.0
    k = rng.random(N) < 0.05
    m[k] = _logu(rng, k.sum(), -104, -96)
    k = rng.random(N) < 0.05
    v[k] = _logu(rng, k.sum(), -100, -90, signed=False)
    m2 = _logu(rng, N, -80, 40)
    if opt == "ademamix":
        # alpha*m2 close to -mh (g tiny against m there): numerators that cancel
        c1 = 1.0 - beta1 ** step
        k = rng.random(N) < 0.3
        rel = _logu(rng, k.sum(), -30, -1)
        m2[k] = -(beta1 * m[k] / c1) / (alpha * 0.9999) * (1.0 + rel)
        g[k] = m[k] * 2.0 ** -40
    f = lambda a: np.clip(a, -3e38, 3e38).astype(np.float32)
    return f(g), f(m), np.abs(f(v)), f(m2)


CONFIGS = [
    ("adamw", 0.9, 0.999, 0.0, 1, 1e-8),
    ("adamw", 0.9, 0.999, 0.0, 1000, 1e-8),
    ("adamw", 0.9, 0.999, 0.0, 7, 0.0),
    ("adamw", 0.5, 0.95, 0.0, 3, 1e-3),
    ("adamw", 0.0, 0.0, 0.0, 1, 1e-8),
    ("adamw", 0.9, 0.99999, 0.0, 1, 1e-8),
    ("ademamix", 0.9, 0.999, 5.0, 1, 1e-8),
    ("ademamix", 0.9, 0.999, 5.0, 500, 1e-8),
    ("ademamix", 0.8, 0.99, 0.5, 2, 0.0),
]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"{c[0]}-b{c[1]}-{c[2]}-a{c[3]}-t{c[4]}-e{c[5]}")
def test_fast_direction_within_half_its_bound(cfg):
    import torch
    import optimizer_step_amd as osa
    opt, b1, b2, alpha, step, eps = cfg
    hp = osa.hparams(step=step, lr=1e-3, beta1=b1, beta2=b2, beta3=0.9999, alpha=alpha, eps=eps)
    g, m, v, m2 = _inputs(CONFIGS.index(cfg) + 1, opt, b1, step, alpha)
    dev = [torch.from_numpy(a).cuda() for a in (g, m, v, m2)]
    out = torch.empty(3 * N, dtype=torch.float32, device="cuda")
    osa.opt_debug_direction(opt, hp, dev[0], dev[1], dev[2], dev[3] if opt == "ademamix" else None, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    uf, bu, ue = o[:N], o[N:2 * N], o[2 * N:]
    fin = np.isfinite(bu)
    # the bound covers most inputs, and (where finite) both directions are finite
    assert fin.mean() > 0.5, fin.mean()
    assert np.all(np.isfinite(uf[fin])) and np.all(np.isfinite(ue[fin]))
    err = np.abs(uf[fin] - ue[fin])
    ratio = err / bu[fin]
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= 0.5, (ratio[worst], uf[fin][worst], ue[fin][worst], bu[fin][worst])
    # AdamW's errors are a few ulp of u (AdEMAMix's cancelling numerators
    # have large relative errors by construction: the bound is absolute there)
    if opt == "adamw":
        big = np.abs(ue[fin]) > 2.0 ** -100
        rel = err[big] / np.abs(ue[fin][big])
        assert np.quantile(rel, 0.999) < 2.0 ** -19

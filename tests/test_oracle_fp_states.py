"""Pins of the oracle's FP8 / FP4 block-scaled states and of state resets
("When Small Updates Disappear": Sec. 2.1 grids, Sec. 2.3 and 3.2 stall
probabilities, Sec. 3 and 6.1 stochastic rounding, Sec. 5 resets).

The element grids are pinned to a library routine (torch's float8_e4m3fn cast)
and to the closed-form value lists of the 4-bit formats; nearest rounding to a
brute-force argmin; stochastic rounding to an exhaustive count over all 2^16
random integers; the whole step to the fp32-state step it must reduce to; the
stall fractions to the page's printed figures."""
import numpy as np
import pytest

import oracle
import synth
from oracle import E2M1, E2M2U, E4M3

EMAX = {E4M3: 8, E2M1: 2, E2M2U: 2}
MAXCODE = {E4M3: 0x7E, E2M1: 0x7, E2M2U: 0xF}
FRAC_BITS = {E4M3: 3, E2M1: 1, E2M2U: 2}


def _values(f):
    return np.array([oracle.mini_value(f, c) for c in range(MAXCODE[f] + 1)])


# ---------------------------------------------------------------------------
# grids

def test_e4m3_values_match_torch():
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    A = np.float32(256.0)                      # floor(log2 A) = emax: scale 1
    for c in range(256):
        got = oracle.mini_decode(E4M3, c, A)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert np.float32(got).view(np.uint32) == np.float32(ref[c]).view(np.uint32), c


def test_four_bit_value_lists():
    """OCP E2M1 and the unsigned E2M2 grid of the page (two exponent bits,
    bias 1, two fraction bits, no sign)."""
    assert list(_values(E2M1)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(_values(E2M2U)) == [0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7]


def test_grid_coarseness_matches_page():
    """Sec. 2.1: at the same scale the FP8 grid is 16 times and the E2M2 grid
    32 times coarser than BF16's (7 fraction bits)."""
    bf16_ulp_at_1 = 2.0 ** -7
    for f, factor in ((E4M3, 16), (E2M2U, 32)):
        V = _values(f)
        i = int(np.where(V == 1.0)[0][0])
        assert V[i + 1] - V[i] == factor * bf16_ulp_at_1
        # and everywhere in the normal range the spacing is value * 2^-p / m
        for j in range(i, len(V) - 1):
            e = np.floor(np.log2(V[j]))
            assert V[j + 1] - V[j] == 2.0 ** (e - FRAC_BITS[f])


def test_e4m3_nearest_matches_torch_cast():
    import torch
    rng = np.random.default_rng(31)
    V = _values(E4M3)
    mids = (V[:-1] + V[1:]) / 2
    y = np.concatenate([V, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 448, 20000), 2.0 ** rng.uniform(-14, 8.8, 20000)])
    y = y[y <= 448].astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.mini_round(E4M3, float(v)) for v in y])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("f", [E4M3, E2M1, E2M2U])
def test_nearest_is_brute_force_argmin(f):
    """Nearest value, ties to the even code, values past the top take it."""
    V = _values(f)
    rng = np.random.default_rng(32 + f)
    mids = (V[:-1] + V[1:]) / 2
    top = V[-1]
    ys = np.concatenate([V, mids, rng.uniform(0, top * 1.2, 3000), [top * 1.1, top * 2]])
    for y in ys:
        d = np.abs(V - y)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        assert oracle.mini_round(f, float(y)) == want, (f, y)


@pytest.mark.parametrize("f", [E4M3, E2M1, E2M2U])
def test_stochastic_rounding_exhaustive_count(f):
    """Over all 2^16 random integers the value goes up exactly
    floor(frac * 2^16) times (Sec. 3: probability = position across the gap),
    and up for exactly the largest r; representable values never move."""
    V = _values(f)
    rng = np.random.default_rng(40 + f)
    r = np.arange(65536, dtype=np.int32)
    gaps = range(len(V) - 1) if len(V) < 20 else sorted(set(range(0, 10)) | set(range(10, len(V) - 1, 9)) | {len(V) - 2})
    for c in gaps:
        lo, hi = V[c], V[c + 1]
        for frac in list(rng.uniform(0, 1, 3)) + [0.0, 0.5, 2.0 ** -17, 1 - 2.0 ** -16]:
            y = float(np.float32(lo + frac * (hi - lo)))
            fr = (y - lo) / (hi - lo)
            codes = oracle.mini_round_array(f, np.full(65536, y), r)
            assert set(np.unique(codes)) <= {c, c + 1}
            ups = codes == c + 1
            assert int(ups.sum()) == int(np.floor(fr * 65536))
            assert not ups[:65536 - int(np.floor(fr * 65536))].any()
    assert oracle.mini_round(f, V[-1] * 1.01, 65535) == len(V) - 1


# ---------------------------------------------------------------------------
# block scale

@pytest.mark.parametrize("f", [E4M3, E2M1, E2M2U])
def test_block_scale_is_power_of_two_from_absmax(f):
    rng = np.random.default_rng(50 + f)
    for _ in range(200):
        A = np.float32(10.0 ** rng.uniform(-30, 10))
        s = oracle.mini_scale_exp(f, A)
        y = float(A) * 2.0 ** -s
        assert 2.0 ** EMAX[f] <= y < 2.0 ** (EMAX[f] + 1)
        # values already on the scaled grid survive a round trip exactly
        for mag in range(MAXCODE[f] + 1):
            x = np.float32(oracle.mini_value(f, mag) * 2.0 ** s)
            if x == 0 or not np.isfinite(x) or abs(x) < 2.0 ** -126:
                continue
            c = oracle.mini_encode(f, x, A)
            assert oracle.mini_decode(f, c, A) == x


def test_block_special_cases():
    assert oracle.mini_encode(E4M3, -0.0, 0.0) == 0x80 and np.signbit(oracle.mini_decode(E4M3, 0x80, 0.0))
    assert oracle.mini_decode(E4M3, 0x05, 0.0) == 0.0
    assert np.isnan(oracle.mini_decode(E2M1, 3, np.float32(np.inf)))
    assert np.isnan(oracle.mini_decode(E2M2U, 3, np.float32(np.nan)))
    assert oracle.mini_encode(E4M3, 1.0, np.float32(np.nan)) == 0
    assert np.isnan(oracle.mini_decode(E4M3, 0xFF, 1.0))
    # negative values keep their sign in the signed formats only
    assert oracle.mini_encode(E2M1, -1.0, 6.0) & 0x8
    assert oracle.mini_encode(E2M2U, 1.0, 7.0) < 16


# ---------------------------------------------------------------------------
# the step

FP_FMTS = ["fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr"]


def _run(fmt, opt, n, steps, hp, g_fn=None, start=None):
    p = synth.params(n).copy()
    st = oracle.state_zeros(fmt, n, opt)
    for t in range(1, steps + 1):
        g = g_fn(t) if g_fn else synth.grads(n, t, bf16=True)
        oracle.step(opt, fmt, oracle.make_hp(step=t, seed=synth.SR_SEED, **hp), p, g, **st)
    return p, st


@pytest.mark.parametrize("fmt", FP_FMTS)
@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_first_step_equals_fp32_step(fmt, opt):
    """From zero states the step reads exact zeros and updates p from the
    unrounded moments, so p after step 1 is the fp32-state p, bit for bit;
    the stored codes decode to the rounding of the fp32 moments."""
    n = 1000
    hp = dict(lr=1e-3, weight_decay=0.1)
    p, st = _run(fmt, opt, n, 1, hp)
    pf, sf = _run("f32", opt, n, 1, hp)
    assert np.array_equal(p.view(np.uint32), pf.view(np.uint32))
    fp4 = fmt.startswith("fp4")
    fm, fv = (E2M1, E2M2U) if fp4 else (E4M3, E4M3)
    for key, f, a in (("s1", fm, "a1"), ("s2", fv, "a2")):
        codes = oracle.unpack_fp4(st[key], n) if fp4 else st[key]
        x = sf[key]
        for b in range(0, n, 256):
            A = st[a][b // 256]
            assert A == np.abs(x[b:b + 256]).max()
            dec = np.array([oracle.mini_decode(f, c, A) for c in codes[b:b + 256]])
            if fmt.endswith("rn"):
                want = np.array([oracle.mini_decode(f, oracle.mini_encode(f, v, A), A) for v in x[b:b + 256]])
                assert np.array_equal(dec, want)
            # either way the stored value is one of the two grid neighbours
            s = oracle.mini_scale_exp(f, A)
            V = np.array([oracle.mini_value(f, c) for c in range(MAXCODE[f] + 1)]) * 2.0 ** s
            for d, v in zip(dec, x[b:b + 256]):
                lo = V[V <= abs(v)].max()
                hi = V[V >= abs(v)].min() if abs(v) <= V.max() else V.max()
                assert lo <= abs(d) <= hi


def test_fp4_odd_length_pads_high_nibble_with_zero():
    n = 257
    _, st = _run("fp4_sr", "adamw", n, 3, dict(lr=1e-3))
    assert st["s1"].size == 129 and st["s1"][-1] >> 4 == 0 and st["s2"][-1] >> 4 == 0


@pytest.mark.parametrize("fmt", ["fp8_sr", "fp4_sr"])
def test_sr_state_is_unbiased_over_streams(fmt):
    """Across many random streams (seeds) the mean stored v is the unrounded v
    to within sampling error (Sec. 3.1: each rounding is unbiased)."""
    n = 256
    rng = np.random.default_rng(60)
    g = (rng.uniform(0.3, 1.0, n) * 1e-2).astype(np.float32)
    om2 = np.float32(1) - np.float32(0.999)
    v1 = (om2 * (g * g)).astype(np.float32)           # v' from a zero state
    f = E2M2U if fmt.startswith("fp4") else E4M3
    A = v1.max()
    V = np.array([oracle.mini_value(f, c) for c in range(MAXCODE[f] + 1)]) * 2.0 ** oracle.mini_scale_exp(f, A)
    u = np.array([V[V > x].min() - V[V <= x].max() if x < V.max() else 0.0 for x in v1.astype(np.float64)])
    seeds = 400
    acc = np.zeros(n)
    for sd in range(seeds):
        st = oracle.state_zeros(fmt, n)
        p = np.zeros(n, np.float32)
        oracle.step("adamw", fmt, oracle.make_hp(step=1, seed=sd), p, g, **st)
        assert st["a2"][0] == A
        codes = oracle.unpack_fp4(st["s2"], n) if fmt.startswith("fp4") else st["s2"]
        acc += [oracle.mini_decode(f, c, A) for c in codes]
    mean = acc / seeds
    # one rounding has standard deviation <= u/2; 6 sigma of the mean, plus
    # the 2^-16 cut of the fraction
    assert np.all(np.abs(mean - v1) <= 6 * u / 2 / np.sqrt(seeds) + u * 2.0 ** -16)
    assert np.abs(mean - v1).max() > 0                # not vacuous: values moved


# ---------------------------------------------------------------------------
# stalling (Sec. 2.3 and 3.2)

def _model_rn(p, b2):
    from scipy import stats
    rho = 2.0 ** -p * np.log(2) / (2 * (1 - b2))
    return stats.chi2.cdf(1 + rho, 1) - stats.chi2.cdf(max(0.0, 1 - rho), 1)


def _model_sr(p, b2):
    from scipy import integrate, stats
    rho = 2.0 ** -p * np.log(2) / (2 * (1 - b2))
    f = lambda z: max(0.0, 1 - abs(z - 1) / (2 * rho)) * stats.chi2.pdf(z, 1)
    return integrate.quad(f, 0, 1 + 2 * rho, points=[1], limit=200)[0]


def _one_step_stall(fmt, nblocks=1024, beta2=0.999):
    """Blocks whose v sits in the format's normal range under its block scale
    (sigma^2 log-uniform over one binade below an anchor element that fixes
    the scale), g ~ N(0, sigma); stalled = the stored v code is unchanged."""
    fp4 = fmt.startswith("fp4")
    f = E2M2U if fp4 else E4M3
    n = nblocks * 256
    rng = np.random.default_rng(70)
    A0 = np.float32(1.5)                                         # anchor: mid-binade
    s = oracle.mini_scale_exp(f, A0)
    sig2 = (2.0 ** rng.uniform(np.log2(0.3), np.log2(0.6), n)).astype(np.float32)
    sig2[::256] = A0
    st = oracle.state_zeros(fmt, n)
    codes = np.array([oracle.mini_encode(f, v, A0) for v in sig2], dtype=np.uint8)
    st["s2"][:] = (codes[0::2] | (codes[1::2] << 4)) if fp4 else codes
    st["a2"][:] = A0
    g = (rng.standard_normal(n) * np.sqrt(sig2)).astype(np.float32)
    g[::256] = 0.0
    p = np.zeros(n, np.float32)
    before = oracle.unpack_fp4(st["s2"], n) if fp4 else st["s2"].copy()
    oracle.step("adamw", fmt, oracle.make_hp(beta2=beta2, step=1000, seed=synth.SR_SEED), p, g, **st)
    after = oracle.unpack_fp4(st["s2"], n) if fp4 else st["s2"]
    mask = np.ones(n, bool)
    mask[::256] = False
    scales = np.array([oracle.mini_scale_exp(f, a) for a in st["a2"]])
    assert np.all(scales == s)                                  # the grid stayed put
    return float(np.mean(after[mask] == before[mask]))


@pytest.mark.parametrize("fmt,bits,printed", [("fp8_sr", 3, 98.9), ("fp4_sr", 2, 99.4),
                                              ("fp8_rn", 3, None), ("fp4_rn", 2, None)])
def test_stall_fraction_matches_page(golden, fmt, bits, printed):
    gold = golden("stall_model.json")
    measured = 100 * _one_step_stall(fmt)
    if printed is not None:
        assert gold["printed_percent"][fmt] == printed
        assert abs(100 * _model_sr(bits, 0.999) - printed) < 0.05
        assert abs(measured - printed) < 1.0, measured
    else:                                # "almost 100%"
        assert 100 * _model_rn(bits, 0.999) > 99.9
        assert measured > 99.0, measured


# ---------------------------------------------------------------------------
# resets (Sec. 5)

@pytest.mark.parametrize("fmt", ["f32", "bf16_rn", "fp8_rn", "q8"])
def test_reset_restarts_from_zero(fmt):
    """With reset_interval R, step R+1 from any state equals step 1 from zero
    states with bias correction restarted (deterministic formats)."""
    n, R = 700, 4
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    hp = dict(lr=1e-3, weight_decay=0.1, reset_interval=R)
    p = synth.params(n).copy()
    st = oracle.state_zeros(fmt, n, "adamw", qs, qu)
    for t in range(1, R + 1):
        oracle.step("adamw", fmt, oracle.make_hp(step=t, **hp), p, synth.grads(n, t), qs=qs, qu=qu, **st)
    p_fresh = p.copy()
    st_fresh = oracle.state_zeros(fmt, n, "adamw", qs, qu)
    g = synth.grads(n, R + 1)
    oracle.step("adamw", fmt, oracle.make_hp(step=R + 1, **hp), p, g, qs=qs, qu=qu, **st)
    oracle.step("adamw", fmt, oracle.make_hp(step=1, lr=1e-3, weight_decay=0.1), p_fresh, g,
                qs=qs, qu=qu, **st_fresh)
    assert np.array_equal(p.view(np.uint32), p_fresh.view(np.uint32))
    for k in st:
        assert np.array_equal(st[k], st_fresh[k]), k
    # and it is not vacuous: without the reset step R+1 differs
    p2 = synth.params(n).copy()
    st2 = oracle.state_zeros(fmt, n, "adamw", qs, qu)
    for t in range(1, R + 2):
        oracle.step("adamw", fmt, oracle.make_hp(step=t, lr=1e-3, weight_decay=0.1), p2,
                    synth.grads(n, t), qs=qs, qu=qu, **st2)
    assert not np.array_equal(p2, p)


def test_reset_between_resets_counts_from_one():
    """Between resets the bias correction uses the steps since the reset."""
    hp = oracle.make_hp(step=7, beta1=0.9, beta2=0.99, reset_interval=5)
    sc = oracle.scalars(hp)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.99))
    assert sc[3] == np.float32(1 - b1 ** 2) and sc[4] == np.float32(1 - b2 ** 2)


@pytest.mark.parametrize("fp", ["fp8", "fp4"])
def test_stall_fraction_separates_rounding_modes(fp):
    """Non-vacuity: stochastic rounding moves measurably more often than
    nearest rounding here (about 1.1 pp for FP8, 0.6 pp for FP4)."""
    assert _one_step_stall(fp + "_rn") - _one_step_stall(fp + "_sr") > 0.003

"""The 8-bit code lookup, host-compiled from the kernels' own source, on
every binary32 value in [-1, 1] for both synthetic codebooks (the nearest
codebook entry of the bitsandbytes PR "Fix decoupled weight decay ordering in
the CUDA Adam/AdEMAMix kernels", blockwise 8-bit kernel; ties to the lower
index).  The expected code is written from the definition: the count of
midpoints (T_i + T_{i+1})/2, formed in binary64, that x lies strictly above.
For a run of consecutive words the values are sorted, so the count is the
number of thresholds at or before each position: one searchsorted of the 255
thresholds into the run and a cumulative sum, no per-element search."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth

CHUNK = 1 << 24
ONE = 0x3F800000


@pytest.fixture(scope="module")
def L():
    import optimizer_step_amd as osa
    if not os.path.exists(osa.LIB_PATH):
        from optimizer_step_amd import build
        build.build()
    return osa


def _thresholds(T):
    """tau_i: the smallest binary32 above the binary64 midpoint t_i, so that
    x > t_i exactly when x >= tau_i."""
    t = (T[:-1].astype(np.float64) + T[1:].astype(np.float64)) / 2
    tau = t.astype(np.float32)
    up = tau.astype(np.float64) <= t
    tau[up] = np.nextafter(tau[up], np.float32(np.inf))
    return tau


def _expected(x_sorted, tau):
    """Codes of an ascending float32 run: count of tau_i <= x."""
    pos = np.searchsorted(x_sorted, tau, side="left")      # first x >= tau_i
    step = np.bincount(pos, minlength=x_sorted.size + 1)[:x_sorted.size]
    return np.cumsum(step).astype(np.uint8)


def _check_run(L, T, signed, lo, hi, negative):
    """Words lo .. hi-1 of magnitude (sign bit added if negative)."""
    tau = _thresholds(T)
    words = np.arange(lo, hi, dtype=np.uint32)
    if negative:
        words = (words | np.uint32(0x80000000))[::-1]       # ascending values
    x = words.view(np.float32)
    got = L.opt_debug_quantize_host(T, signed, x)
    if signed or not negative:
        want = _expected(x, tau)
    else:
        want = np.zeros(x.size, np.uint8)                    # every midpoint of an unsigned table is > 0
    bad = np.flatnonzero(got != want)
    return (int(bad.size), None if bad.size == 0 else (float(x[bad[0]]), int(got[bad[0]]), int(want[bad[0]])))


@pytest.mark.parametrize("signed", [True, False], ids=["signed", "unsigned"])
def test_lookup_on_every_value_in_unit_interval(L, signed):
    T = synth.codebook_signed() if signed else synth.codebook_unsigned()
    runs = [(a, min(a + CHUNK, ONE + 1), neg) for neg in (False, True) for a in range(0, ONE + 1, CHUNK)]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        results = list(pool.map(lambda r: _check_run(L, T, signed, *r), runs))
    bad = [(r, res) for r, res in zip(runs, results) if res[0]]
    assert not bad, bad[:3]
    covered = sum(b - a for a, b, _ in runs)
    assert covered == 2 * (ONE + 1)                          # +-0 .. +-1, every word


def test_expected_codes_match_brute_force_on_a_sample():
    """The cumulative-count expectation against argmin over the table in
    binary64 (ties to the lower index) on a run that crosses many midpoints."""
    T = synth.codebook_signed()
    words = np.arange(0x33000000, ONE + 1, 2039, dtype=np.uint32)
    x = words.view(np.float32)
    want = _expected(x, _thresholds(T))
    d = np.abs(T.astype(np.float64)[None, :] - x.astype(np.float64)[:, None])
    assert np.array_equal(want, np.argmin(d, axis=1).astype(np.uint8))
    assert np.unique(want).size > 100

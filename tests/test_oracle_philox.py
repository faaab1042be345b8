"""Pins of the oracle's Philox4x32-10 (Salmon et al., SC'11) against rocRAND's
public philox4x32_10 engine (a library implementation compiled here from its
header), and of the per-element counter layout the stochastic rounding uses
('When Small Updates Disappear', Sec. 7.3: the random number is tied to the
element, not to the program)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

HELPER = os.path.join(os.path.dirname(__file__), "helpers", "philox_rocrand.cpp")


@pytest.fixture(scope="module")
def rocrand_words():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "philox_rocrand")
    subprocess.run([hipcc, "-O1", "-I/opt/rocm/include", HELPER, "-o", exe], check=True,
                   capture_output=True)

    def run(rows):
        text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in line.split()] for line in out.strip().split("\n")],
                        dtype=np.uint32)
    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand(rocrand_words):
    rng = np.random.default_rng(1234)
    rows = []
    for _ in range(3000):
        key = rng.integers(0, 2**32, 2)
        ctr = rng.integers(0, 2**32, 4)
        ctr[1] %= 2**30          # the helper positions rocRAND by offset = 4*(c0 | c1<<32)
        rows.append([*key, *ctr])
    rows += [[0, 0, 0, 0, 0, 0], [2**32 - 1, 2**32 - 1, 2**32 - 1, 0, 2**32 - 1, 2**32 - 1]]
    ref = rocrand_words(rows)
    got = np.array([oracle.philox(r[2:], r[:2]) for r in rows])
    assert np.array_equal(got, ref)


def test_element_words_follow_counter_layout(rocrand_words):
    """Element j of tensor k at step t draws word j mod 4 of the block with
    counter (j>>2, j>>34, t, k); the slow-EMA stream sets bit 31 of word 3."""
    seed, t, k = 0x9E3779B97F4A7C15, 17, 5
    for j0, stream in ((0, 0), ((1 << 34) - 6, 0), (12345, 1)):
        n = 12
        got = oracle.sr_words(seed, t, k, j0, n, stream)
        rows = []
        for j in range(j0, j0 + n):
            q = j >> 2
            rows.append([seed & 0xFFFFFFFF, seed >> 32, q & 0xFFFFFFFF, q >> 32, t,
                         k | (0x80000000 if stream else 0)])
        ref = rocrand_words(rows)
        assert np.array_equal(got, ref[np.arange(n), (np.arange(j0, j0 + n) & 3)])


def test_halves_uniform_chi2():
    """The 16-bit halves used as r are uniform over 2^16 bins (chi-square
    within 5 sigma), and the two halves are not identical streams."""
    n = 1 << 22
    w = oracle.sr_words(42, 3, 0, 0, n)
    for half in (w & 0xFFFF, w >> 16):
        counts = np.bincount(half.astype(np.int64), minlength=65536)
        e = n / 65536
        chi2 = ((counts - e) ** 2 / e).sum()
        assert abs(chi2 - 65535) < 5 * np.sqrt(2 * 65535)
    assert np.mean((w & 0xFFFF) == (w >> 16)) < 1e-3

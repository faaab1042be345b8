"""The tolerance helpers the GPU parity tests use, checked on the CPU against
what the formats fix: the spacing of representable 16-bit values and the
BF16 step count."""
import numpy as np

import oracle
from tests.gpu_common import bf16_ulps
from tests.test_gpu_p16 import _step16


def _spacing_from_words(widen, words):
    """Distance from each positive finite word's value to the next word's."""
    return widen(words + 1).astype(np.float64) - widen(words).astype(np.float64)


def test_fp16_step_is_the_gap_to_the_next_value():
    w = np.arange(0x0000, 0x7BFF, dtype=np.uint16)          # +0 .. the word below 65504
    x = w.view(np.float16).astype(np.float64)
    gap = _spacing_from_words(lambda u: u.view(np.float16).astype(np.float64), w)
    assert np.array_equal(_step16(x, oracle.P_F16), gap)


def test_bf16_step_is_the_gap_to_the_next_value():
    w = np.arange(0x0000, 0x7F7F, dtype=np.uint16)          # +0 .. the word below the largest finite
    x = oracle.widen_bf16(w).astype(np.float64)
    gap = _spacing_from_words(oracle.widen_bf16, w)
    assert np.array_equal(_step16(x, oracle.P_BF16), gap)


def test_bf16_step_count_is_the_word_distance():
    """bf16_ulps counts representable values between two words, across 0."""
    a = np.array([0x3F80, 0x3F80, 0x0001, 0x8001, 0xBF80], dtype=np.uint16)
    b = np.array([0x3F80, 0x3F83, 0x8001, 0x0001, 0xBF81], dtype=np.uint16)
    assert list(bf16_ulps(a, b)) == [0, 3, 2, 2, 1]

"""The tolerance helper the GPU parity tests use for BF16 states, checked on
the CPU against what the format fixes: the count of representable BF16
values between two words."""
import numpy as np

from tests.gpu_common import bf16_ulps


def test_bf16_step_count_is_the_word_distance():
    """bf16_ulps counts representable values between two words, across 0."""
    a = np.array([0x3F80, 0x3F80, 0x0001, 0x8001, 0xBF80], dtype=np.uint16)
    b = np.array([0x3F80, 0x3F83, 0x8001, 0x0001, 0xBF81], dtype=np.uint16)
    assert list(bf16_ulps(a, b)) == [0, 3, 2, 2, 1]

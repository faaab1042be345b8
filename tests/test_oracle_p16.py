"""Pins of the oracle's 16-bit parameter storage and of the standalone
rounding cast ("When Small Updates Disappear", Sec. 6, 6.1, 7.3 and 8.1; the
issue "Investigate SM103 bias-correction broadcast in 32-bit optimizers",
Correctness oracle: FP16, BF16 and FP32 parameter storage).

FP16 nearest rounding is pinned to numpy's float16 cast, BF16 nearest to
torch's bfloat16 cast (library routines); stochastic rounding to exhaustive
counts over all 2^16 random integers; the 16-bit parameter step to the fp32
step followed by the library cast; the cast's random stream to a direct
Philox call with the stated counter layout."""
import numpy as np
import pytest

import oracle
import synth


def _torch_bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _all_f16_values():
    w = np.arange(0, 0x7C00, dtype=np.uint16)
    return w.view(np.float16).astype(np.float32)


def test_f16_nearest_matches_numpy():
    V = _all_f16_values().astype(np.float64)
    mids = ((V[:-1] + V[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(11)
    x = np.concatenate([V.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)),
                        (rng.standard_normal(50000) * 10.0 ** rng.uniform(-10, 5.5, 50000)).astype(np.float32),
                        np.array([65504, 65519.99, 65520, 65535, 65536, 1e9, 2.0 ** -25, 2.0 ** -26,
                                  3 * 2.0 ** -26, np.inf], np.float32)])
    x = np.concatenate([x, -x])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.f16_array(x)
    assert np.array_equal(got, ref)


def test_f16_nan_and_widening():
    assert oracle.f16_rne(np.float32(np.nan)) & 0x7FFF == 0x7E00
    w = np.arange(65536, dtype=np.uint16)
    ref = w.view(np.float16).astype(np.float32)
    got = oracle.widen_f16(w)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("lo_code", [0x0001, 0x03FF, 0x0400, 0x3C00, 0x5A3D, 0x7BFE, 0x7BFF])
def test_f16_sr_exhaustive_count(lo_code):
    """Up exactly floor(frac * 2^16) times over all r, for the largest r; the
    gap above 65504 leads to infinity (the carry of Sec. 6.1 into the
    exponent)."""
    lo = float(np.uint16(lo_code).view(np.float16))
    hi = 65536.0 if lo_code == 0x7BFF else float(np.uint16(lo_code + 1).view(np.float16))
    rng = np.random.default_rng(lo_code)
    r = np.arange(65536, dtype=np.uint32)
    for frac in list(rng.uniform(0, 1, 3)) + [0.0, 0.5, 2.0 ** -20]:
        x = np.float32(lo + frac * (hi - lo))
        if not (lo <= x < hi):
            continue
        fr = (float(x) - lo) / (hi - lo)
        out = oracle.f16_array(np.full(65536, x, np.float32), r)
        assert set(np.unique(out)) <= {lo_code, lo_code + 1}
        ups = out == lo_code + 1
        assert int(ups.sum()) == int(np.floor(fr * 65536))
        assert not ups[:65536 - int(np.floor(fr * 65536))].any()
    assert oracle.f16_sr(np.float32(-lo), 65535) & 0x8000


def test_bf16_nearest_is_torch_cast():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    assert np.array_equal(oracle.bf16_rne_array(x), _torch_bf16(x))


# ---------------------------------------------------------------------------
# 16-bit parameters in the step

@pytest.mark.parametrize("fmt", ["f32", "bf16_sr"])
@pytest.mark.parametrize("p_dtype", [oracle.P_BF16, oracle.P_F16])
def test_p16_nearest_step_is_f32_step_then_library_cast(fmt, p_dtype):
    n = 3000
    p32 = synth.params(n)
    p16 = _torch_bf16(p32) if p_dtype == oracle.P_BF16 else p32.astype(np.float16).view(np.uint16)
    wide = oracle.widen_bf16(p16) if p_dtype == oracle.P_BF16 else p16.view(np.float16).astype(np.float32)
    g = synth.grads(n, 2, bf16=True)
    hp = oracle.make_hp(lr=1e-2, weight_decay=0.1, step=2, seed=5)
    st_a = oracle.state_zeros(fmt, n)
    st_b = oracle.state_zeros(fmt, n)
    ref = wide.copy()
    oracle.step("adamw", fmt, hp, ref, g, **st_a)
    got = p16.copy()
    oracle.step("adamw", fmt, hp, got, g, p_dtype=p_dtype, **st_b)
    want = _torch_bf16(ref) if p_dtype == oracle.P_BF16 else ref.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    for k in st_a:
        assert np.array_equal(st_a[k], st_b[k])
    assert not np.array_equal(got, p16)                 # the step moved p


@pytest.mark.parametrize("p_dtype", [oracle.P_BF16, oracle.P_F16])
def test_p16_stochastic_step_uses_second_stream_high_half(p_dtype):
    n, k, t, j0 = 2049, 3, 9, 1 << 33
    p32 = synth.params(n)
    p16 = _torch_bf16(p32) if p_dtype == oracle.P_BF16 else p32.astype(np.float16).view(np.uint16)
    wide = oracle.widen_bf16(p16) if p_dtype == oracle.P_BF16 else p16.view(np.float16).astype(np.float32)
    g = synth.grads(n, t, k)
    hp = oracle.make_hp(lr=1e-2, step=t, seed=77, tensor_index=k, index_base=j0)
    ref = wide.copy()
    oracle.step("adamw", "f32", hp, ref, g, **oracle.state_zeros("f32", n))
    got = p16.copy()
    oracle.step("adamw", "f32", hp, got, g, p_dtype=p_dtype, p_sr=True, **oracle.state_zeros("f32", n))
    r = oracle.sr_words(77, t, k, j0, n, stream=1) >> 16
    want = oracle.bf16_sr_array(ref, r) if p_dtype == oracle.P_BF16 else oracle.f16_array(ref, r)
    assert np.array_equal(got, want)
    nearest = _torch_bf16(ref) if p_dtype == oracle.P_BF16 else ref.astype(np.float16).view(np.uint16)
    assert 0.05 < np.mean(got != nearest) < 0.8           # SR differs from nearest often


# ---------------------------------------------------------------------------
# the standalone cast

def test_cast_nearest_is_library_cast():
    x = (np.random.default_rng(13).standard_normal(5000) * 100).astype(np.float32)
    assert np.array_equal(oracle.round_cast(x, oracle.P_BF16), _torch_bf16(x))
    assert np.array_equal(oracle.round_cast(x, oracle.P_F16), x.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("dtype", [oracle.P_BF16, oracle.P_F16])
def test_cast_random_stream_layout(dtype):
    """Element j takes the low 16 bits of word j%4 of Philox keyed by the seed
    with counter (j>>2 low, j>>34, offset low, offset high)."""
    n, seed, offset = 1031, 0x1234_5678_9ABC_DEF0, 0x0000_0007_0000_0003
    x = (np.random.default_rng(14).standard_normal(n)).astype(np.float32)
    got = oracle.round_cast(x, dtype, True, seed, offset)
    r = np.empty(n, np.uint32)
    for j in range(n):
        q = j >> 2
        w = oracle.philox([q & 0xFFFFFFFF, q >> 32, offset & 0xFFFFFFFF, offset >> 32],
                          [seed & 0xFFFFFFFF, seed >> 32])
        r[j] = w[j & 3] & 0xFFFF
    want = oracle.bf16_sr_array(x, r) if dtype == oracle.P_BF16 else oracle.f16_array(x, r)
    assert np.array_equal(got, want)


def test_cast_unbiased_over_offsets():
    """Sec. 3.1: the mean over many casts (fresh offsets) is the input."""
    x = np.float32(1.0) + np.float32(2.0 ** -9) * np.arange(1, 65, dtype=np.float32)   # 1/4 ulp steps
    acc = np.zeros(x.size)
    casts = 2000
    for off in range(casts):
        acc += oracle.widen_bf16(oracle.round_cast(x, oracle.P_BF16, True, 9, off))
    u = 2.0 ** -7
    assert np.all(np.abs(acc / casts - x) < 5 * 0.5 * u / np.sqrt(casts))
    assert not np.array_equal(oracle.round_cast(x, oracle.P_BF16, True, 9, 1),
                              oracle.round_cast(x, oracle.P_BF16, True, 9, 2))

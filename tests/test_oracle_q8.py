"""Pins of the oracle's 8-bit blockwise state format.  The pages name the
format (the blockwise 8-bit kernel of the bitsandbytes PR; a 256-entry signed
dynamic-exponent codebook for m, an unsigned one for v, blocksize 256, an fp32
absmax per block) and one fact about it: a fresh state is zero and quantizes
exactly ('Why the current tests do not catch it').  The quantizer is pinned by
brute-force nearest-entry search, the whole step by a decomposition into
dequantize / fp32 step / brute-force requantize."""
import numpy as np
import pytest

import oracle
import synth
from tests.common import run_oracle

QS, QU = synth.codebook_signed(), synth.codebook_unsigned()


def brute_force(T, x):
    """argmin_i |T_i - x| in binary64; np.argmin returns the lowest index on a
    tie.  NaN -> 0 (reading: NaN is above no midpoint)."""
    x = np.asarray(x, dtype=np.float32)
    d = np.abs(T.astype(np.float64)[None, :] - x.astype(np.float64)[:, None])
    out = np.argmin(d, axis=1).astype(np.uint8)
    out[np.isnan(x)] = 0
    return out


def _probe_points(T):
    mids = (T[:-1].astype(np.float64) + T[1:].astype(np.float64)) / 2
    m32 = mids.astype(np.float32)
    pts = [T, m32, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf)),
           np.nextafter(np.nextafter(m32, np.float32(np.inf)), np.float32(np.inf)),
           np.array([0.0, -0.0, 1.0, -1.0, np.nan, 1e-30, -1e-30, 5e-8, -5e-8], dtype=np.float32),
           np.random.default_rng(2).uniform(-1, 1, 20000).astype(np.float32),
           (np.random.default_rng(3).uniform(-1, 1, 20000) ** 7).astype(np.float32)]
    return np.concatenate(pts).astype(np.float32)


@pytest.mark.parametrize("T", [QS, QU], ids=["signed", "unsigned"])
def test_quantize_is_nearest_entry(T):
    x = _probe_points(T)
    assert np.array_equal(oracle.quantize_array(T, x), brute_force(T, x))


@pytest.mark.parametrize("T", [QS, QU], ids=["signed", "unsigned"])
def test_quantize_entries_map_to_their_index_and_is_monotone(T):
    assert np.array_equal(oracle.quantize_array(T, T), np.arange(256, dtype=np.uint8))
    x = np.sort(np.random.default_rng(4).uniform(-1, 1, 100000).astype(np.float32))
    c = oracle.quantize_array(T, x).astype(np.int64)
    assert np.all(np.diff(c) >= 0)


def test_codebook_landmarks():
    assert oracle.quantize(QS, -1.0) == 0 and oracle.quantize(QS, 0.0) == 127
    assert oracle.quantize(QS, 1.0) == 255
    assert oracle.quantize(QU, 0.0) == 0 and oracle.quantize(QU, 1.0) == 255


def _fp32_moments_step1(g, hp):
    """m' = fl(fl(1-b1) g) and v' = fl(fl(1-b2) fl(g g)) at step 1 from zero."""
    g = np.asarray(g, dtype=np.float32)
    om1 = np.float32(1) - np.float32(hp["beta1"])
    om2 = np.float32(1) - np.float32(hp["beta2"])
    return (om1 * g).astype(np.float32), (om2 * (g * g)).astype(np.float32)


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_step1_from_zero_state(opt):
    """The zero state reads back as exactly 0, so after step 1 p equals the
    fp32-state step bit for bit, absmax is max|m'| per block and the codes are
    the nearest entries of m'/absmax."""
    n = 4099
    hp = dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999)
    g = synth.grads(n, 1, std=1e-3, bf16=True, mask_scale=(0.1, 100.0))
    gf = oracle.widen_bf16(g)
    p0 = synth.params(n)
    pq, sq = run_oracle(opt, "q8", n, 1, hp, grad_fn=lambda t: g, p=p0.copy(), qs=QS, qu=QU)
    pf, _ = run_oracle(opt, "f32", n, 1, hp, grad_fn=lambda t: g, p=p0.copy())
    assert np.array_equal(pq.view(np.uint32), pf.view(np.uint32))
    m, v = _fp32_moments_step1(gf, hp)
    for arr, T, codes, amax in ((m, QS, sq["s1"], sq["a1"]), (v, QU, sq["s2"], sq["a2"])):
        for b in range((n + 255) // 256):
            blk = arr[b * 256:(b + 1) * 256]
            A = np.abs(blk).max()
            assert amax[b] == A
            x = (blk / A).astype(np.float32) if A != 0 else np.zeros_like(blk)
            assert np.array_equal(codes[b * 256:(b + 1) * 256], brute_force(T, x))


def _dequant(T, codes, amax):
    a = np.repeat(amax, 256)[: codes.size]
    return (T[codes] * a).astype(np.float32)


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
def test_step_is_dequantize_f32_step_requantize(opt):
    """Any step = read T[code]*absmax, take the fp32 step on those values,
    re-quantize the fp32 moments by brute force with per-block absmax."""
    n, T = 3 * 256 + 77, 6
    hp = dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, beta3=0.99, alpha=5.0)
    p, st = run_oracle(opt, "q8", n, T - 1, hp, qs=QS, qu=QU)
    g = synth.grads(n, T, bf16=True)
    h = oracle.make_hp(step=T, **hp)
    names = [("s1", "a1", QS), ("s2", "a2", QU)] + ([("s3", "a3", QS)] if opt == "ademamix" else [])
    f32 = {s: _dequant(Tb, st[s], st[a]) for s, a, Tb in names}
    pf = p.copy()
    oracle.step(opt, "f32", h, pf, g, **f32)
    oracle.step(opt, "q8", h, p, g, qs=QS, qu=QU, **st)
    assert np.array_equal(p.view(np.uint32), pf.view(np.uint32))
    for s, a, Tb in names:
        for b in range((n + 255) // 256):
            blk = f32[s][b * 256:(b + 1) * 256]
            A = np.abs(blk).max()
            assert st[a][b] == A
            x = (blk / A).astype(np.float32) if A != 0 else np.zeros_like(blk)
            assert np.array_equal(st[s][b * 256:(b + 1) * 256], brute_force(Tb, x))


def test_absmax_element_takes_an_end_code():
    """The element at the block absmax quantizes x = +-1 to code 0 or 255."""
    n = 64 * 256
    _, st = run_oracle("adamw", "q8", n, 4, dict(lr=1e-3), qs=QS, qu=QU)
    for b in range(64):
        cm = st["s1"][b * 256:(b + 1) * 256]
        cv = st["s2"][b * 256:(b + 1) * 256]
        assert np.any((cm == 0) | (cm == 255)) and np.any(cv == 255)


def test_nan_poisons_only_its_block():
    """A NaN gradient makes its block's absmax NaN (a max must not skip NaNs)
    and every code of that block 0; other blocks are untouched."""
    n = 4 * 256
    g = synth.grads(n, 1, bf16=True)
    gn = g.copy()
    gn[300] = 0x7FC0   # NaN in block 1
    p1, s1 = run_oracle("adamw", "q8", n, 1, dict(lr=1e-3), grad_fn=lambda t: g, qs=QS, qu=QU)
    p2, s2 = run_oracle("adamw", "q8", n, 1, dict(lr=1e-3), grad_fn=lambda t: gn, qs=QS, qu=QU)
    assert np.isnan(s2["a1"][1]) and np.isnan(s2["a2"][1])
    assert np.all(s2["s1"][256:512] == 0) and np.all(s2["s2"][256:512] == 0)
    for b in (0, 2, 3):
        sl = slice(b * 256, (b + 1) * 256)
        assert np.array_equal(s1["s1"][sl], s2["s1"][sl]) and s1["a1"][b] == s2["a1"][b]
    keep = np.ones(n, bool)
    keep[300] = False
    assert np.array_equal(p1[keep].view(np.uint32), p2[keep].view(np.uint32))


def test_zero_block_stays_zero_code():
    n = 2 * 256
    g = synth.grads(n, 1, bf16=True)
    g[:256] = 0
    _, st = run_oracle("adamw", "q8", n, 1, dict(lr=1e-3), grad_fn=lambda t: g, qs=QS, qu=QU)
    assert st["a1"][0] == 0 and np.all(st["s1"][:256] == 127) and np.all(st["s2"][:256] == 0)

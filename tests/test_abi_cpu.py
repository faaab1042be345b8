"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every function include/opt_step.h declares, rejects bad arguments before any
device work, plans chunks from sizes only, and its host-compiled helpers (the
8-bit lookup tables and the reused-reciprocal division the kernels use) agree
with the oracle and with correctly rounded arithmetic."""
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
QS, QU = synth.codebook_signed(), synth.codebook_unsigned()


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0      # counts without initialising the device
    except Exception:
        return False


# Calls that pass the argument checks go on to launch work on the made-up
# device addresses these tests use, so such tests run only with no GPU.
no_device = pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses would reach a kernel")


@pytest.fixture(scope="module")
def L():
    import optimizer_step_amd as osa
    if not os.path.exists(osa.LIB_PATH):
        from optimizer_step_amd import build
        build.build()
    return osa


def _declared():
    text = open(os.path.join(ROOT, "include", "opt_step.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(opt_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert "opt_step_adamw" in names and "opt_precondition_unorm" in names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def _tensor(L, numel=16, p=4096, g=4096, s1=8192, s2=12288, s3=0, gd=0):
    return [L.OptTensor(p, g, s1, s2, s3 or None, None, None, None, numel, 0, gd)]


def _call(L, fn, tensors, fmt=0, hp=None, unorm=None):
    arr = (L.OptTensor * len(tensors))(*tensors)
    hp = hp or L.hparams()
    return getattr(L.lib(), fn)(arr, len(tensors), fmt, hp, unorm, None)


@pytest.mark.parametrize("case,status", [
    (dict(hp=dict(step=0)), -1),
    (dict(hp=dict(beta1=1.0)), -1),
    (dict(hp=dict(beta2=-0.1)), -1),
    (dict(fmt=9), -1),
    (dict(tensor=dict(p=0)), -1),
    (dict(tensor=dict(numel=-1)), -1),
    (dict(tensor=dict(p=4100)), -3),
    (dict(tensor=dict(s2=12296)), -3),
    (dict(tensor=dict(gd=7)), -1),
    (dict(fmt=3), -1),                          # 8-bit without codebooks
    (dict(hp=dict(max_unorm=1.0)), -1),         # bound without norms
])
def test_bad_arguments_are_rejected_before_device_work(L, case, status):
    hp = L.hparams(**case.get("hp", {}))
    rc = _call(L, "opt_step_adamw", _tensor(L, **case.get("tensor", {})), case.get("fmt", 0), hp)
    assert rc == status
    assert L.opt_last_error() != ""


@pytest.mark.parametrize("case,status", [
    (dict(hp=dict(step=0)), -1),
    (dict(tensor=dict(p=4100)), -3),
    (dict(hp=dict(max_unorm=1.0)), -1),
])
def test_no_alloc_step_checks_its_arguments(L, case, status):
    hp = L.hparams(**case.get("hp", {}))
    assert _call(L, "opt_step_adamw_noalloc", _tensor(L, **case.get("tensor", {})), 0, hp) == status


def test_no_alloc_step_refuses_tables_beyond_its_array(L):
    """20,000 tensor records (2.2 MB of tables) exceed the fixed 2 MiB array:
    OPT_EUNSUPPORTED, decided on the host before any device work."""
    recs = [L.OptTensor(4096 * (i + 1), 4096, 8192, 12288, None, None, None, None, 4, 0, 0) for i in range(20000)]
    assert _call(L, "opt_step_adamw_noalloc", recs) == -2
    assert "2097152" in L.opt_last_error()


def test_ademamix_needs_slow_ema(L):
    assert _call(L, "opt_step_ademamix", _tensor(L)) == -1


def test_bad_codebooks_are_rejected(L):
    bad = QS.copy()
    bad[10] = bad[9]
    for q in (bad, QS * 2):
        hp = L.hparams(qmap_signed=q, qmap_unsigned=QU)
        assert _call(L, "opt_step_adamw", _tensor(L), 3, hp) == -1
    hp = L.hparams(qmap_signed=QS, qmap_unsigned=QS)       # negative entries in the v table
    assert _call(L, "opt_step_adamw", _tensor(L), 3, hp) == -1


def test_empty_call_is_a_no_op(L):
    assert L.lib().opt_step_adamw(None, 0, 0, L.hparams(), None, None) == 0


def test_plan_depends_on_sizes_only(L):
    chunk, nc = L.opt_debug_plan([0, 1, 1023, 1024, 65537, 6 * 2**20])
    assert chunk % 1024 == 0
    assert list(nc) == [0, 1, 1, 1, -(-65537 // chunk), -(-6 * 2**20 // chunk)]


def _probe(T):
    mids = ((T[:-1].astype(np.float64) + T[1:].astype(np.float64)) / 2).astype(np.float32)
    rng = np.random.default_rng(7)
    pts = [T, mids, np.nextafter(mids, np.float32(2)), np.nextafter(mids, np.float32(-2)),
           np.array([0.0, -0.0, 1.0, -1.0, 1e-30, -1e-30, 3e-8, -3e-8, np.nan], dtype=np.float32),
           rng.uniform(-1, 1, 200000).astype(np.float32),
           (rng.uniform(-1, 1, 200000) ** 9).astype(np.float32)]
    x = np.concatenate(pts).astype(np.float32)
    return x


@pytest.mark.parametrize("signed", [True, False])
def test_host_lookup_matches_oracle(L, signed):
    T = QS if signed else QU
    x = _probe(T)
    if not signed:
        x = np.abs(x)
    got = L.opt_debug_quantize_host(T, signed, x)
    ref = oracle.quantize_array(T, x)
    assert np.array_equal(got, ref)


def test_host_lookup_other_codebooks(L):
    """Other strictly increasing tables in [-1, 1]: uniform (with a midpoint
    of exactly 0), and random gaps."""
    rng = np.random.default_rng(3)
    gaps = np.concatenate([[0.0], rng.uniform(0.5, 1.5, 255)])
    rand = (-1 + 2 * np.cumsum(gaps) / gaps.sum()).astype(np.float32)
    for T in (np.linspace(-1, 1, 256).astype(np.float32), rand):
        assert np.all(np.diff(T.astype(np.float64)) > 0)
        x = _probe(T)
        assert np.array_equal(L.opt_debug_quantize_host(T, True, x), oracle.quantize_array(T, x))


def test_codebook_too_dense_for_the_table_is_unsupported(L):
    """Two midpoints closer than the finest bucket cannot share one
    comparison: such a codebook is refused, not approximated."""
    T = np.linspace(-1, 1, 256).astype(np.float32)
    T[200] = np.nextafter(T[201], np.float32(-1))
    T[199] = np.nextafter(T[200], np.float32(-1))
    with pytest.raises(L.OptError) as e:
        L.opt_debug_quantize_host(T, True, np.zeros(1, np.float32))
    assert e.value.status == -2


def test_reused_reciprocal_division_is_correctly_rounded(L):
    """a / b by two residual corrections of a * RN(1/b) equals the correctly
    rounded quotient (numpy float32 division), over random operands, divisors
    with all-ones significands, and dividends next to the divisor."""
    rng = np.random.default_rng(5)
    n = 2_000_000
    b = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(-30, 10, n)).astype(np.float32)
    a = (b * rng.uniform(-1, 1, n)).astype(np.float32)
    ones = (np.float32(2) - np.float32(2.0 ** -23)) * (2.0 ** rng.integers(-24, 1, n // 4)).astype(np.float32)
    b = np.concatenate([b, ones.astype(np.float32), b[:n // 4]])
    a = np.concatenate([a, (ones * rng.uniform(-1, 1, n // 4)).astype(np.float32),
                        np.nextafter(b[:n // 4], np.float32(0))])
    b = b.astype(np.float32)
    a = a.astype(np.float32)
    got = L.opt_debug_div_by(a, b)
    ref = (a / b).astype(np.float32)
    normal = np.abs(ref) >= np.float32(2.0 ** -126)
    assert np.array_equal(got[normal].view(np.uint32), ref[normal].view(np.uint32))


def _gn(L, grads, out=8192, max_norm=1.0, norm_type=2, coef=None, n=None):
    arr = (L.OptGrad * max(1, len(grads)))(*[L.OptGrad(*g) for g in grads])
    return L.lib().opt_grad_norm(arr, len(grads) if n is None else n, out, max_norm, norm_type, coef, None)


@pytest.mark.parametrize("case,status", [
    (dict(n=-1), -1),
    (dict(out=None), -1),
    (dict(out=8196), -3),
    (dict(grads=[(4096, 16, 5, 0)]), -1),            # unknown dtype
    (dict(grads=[(None, 16, 0, 0)]), -1),            # NULL data with elements
    (dict(grads=[(4100, 16, 0, 0)]), -3),            # misaligned data
    (dict(grads=[(4096, -1, 0, 0)]), -1),
    (dict(coef=4096, norm_type=1), -1),              # only 2 and 0 (inf)
    (dict(coef=4096, max_norm=0.0), -1),
    (dict(coef=4096, max_norm=float("inf")), -1),
    (dict(coef=4098), -3),
])
def test_grad_norm_bad_arguments(L, case, status):
    grads = case.pop("grads", [(4096, 16, 0, 0)])
    assert _gn(L, grads, **case) == status
    assert L.opt_last_error() != ""


def test_step_rejects_misaligned_grad_scale(L):
    hp = L.hparams()
    hp.grad_scale = 4098
    assert _call(L, "opt_step_adamw", _tensor(L), 0, hp) == -3


def _mini_inputs(elem, A, rng):
    """Values on, between and next to the scaled grid of a block with absmax A,
    random values below A, signed zeros and tiny values; never NaN or
    infinite (in a step, such an element makes the absmax NaN or infinite)."""
    s = oracle.mini_scale_exp(elem, A) if A > 0 else 0
    top = {0: 0x7E, 1: 7, 2: 15}[elem]
    V = np.array([oracle.mini_value(elem, c) for c in range(top + 1)]) * 2.0 ** s
    mids = (V[:-1] + V[1:]) / 2
    x = np.concatenate([V, mids, rng.uniform(0, 1, 4000) * A, (rng.uniform(0, 1, 2000) ** 8) * A,
                        [0.0, A, A * 0.999, 1e-45, 2.0 ** -140]]).astype(np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))])
    if elem != 2:
        x = np.concatenate([x, -x])
    return x[np.isfinite(x)]


@pytest.mark.parametrize("elem", [0, 1, 2])
def test_host_mini_codec_matches_oracle(L, elem):
    """The library's FP8/FP4 codec (the kernels' source, compiled for the host)
    against the oracle's grid walk: codes and read-back values bit for bit,
    for nearest and stochastic rounding, across block scales (subnormal,
    zero, NaN and infinite absmax included)."""
    rng = np.random.default_rng(90 + elem)
    As = [np.float32(x) for x in (1.0, 1.5, 448.0, 7.0, 3e-3, 2.5e-12, 1e30, 3e-39, 1e-44)]
    # block scales around the switch between the codec's two paths: the
    # scaling exponent nsc = emax - floor(log2 A) at Emin + 125, 126 and 127
    emax, emin = {0: (8, -6), 1: (2, 0), 2: (2, 0)}[elem]
    As += [np.float32(1.3 * 2.0 ** (emax - (emin + d))) for d in (125, 126, 127)]
    for A in As + [np.float32(0.0), np.float32(np.nan), np.float32(np.inf)]:
        x = _mini_inputs(elem, A, rng) if np.isfinite(A) and A > 0 else np.array([0.0, -0.0, 1.0], np.float32)
        if A == 0:
            x = np.array([0.0, -0.0] * 4, np.float32)
        for sr in (False, True):
            r = rng.integers(0, 65536, x.size).astype(np.uint32) if sr else None
            if sr:
                r[:min(8, r.size)] = [0, 1, 32767, 32768, 65534, 65535, 0, 65535][:r.size]
            codes, dec = L.opt_debug_mini_host(elem, A, x, r)
            want = np.array([oracle.mini_encode(elem, v, A, int(r[i]) if sr else -1) for i, v in enumerate(x)])
            assert np.array_equal(codes, want), (elem, A, sr, x[codes != want][:5])
            wdec = np.array([oracle.mini_decode(elem, int(c), A) for c in want], dtype=np.float32)
            nan = np.isnan(wdec)
            assert np.array_equal(np.isnan(dec), nan)
            assert np.array_equal(dec[~nan].view(np.uint32), wdec[~nan].view(np.uint32)), (elem, A)


def test_host_mini_codec_rejects_bad_arguments(L):
    x = np.zeros(4, np.float32)
    for elem, A in ((3, 1.0), (-1, 1.0), (0, -1.0)):
        with pytest.raises(L.OptError):
            L.opt_debug_mini_host(elem, A, x)


@pytest.mark.parametrize("fmt", [4, 5, 6, 7])
def test_fp_formats_need_absmax(L, fmt):
    assert _call(L, "opt_step_adamw", _tensor(L), fmt) == -1


def test_negative_reset_interval_is_rejected(L):
    assert _call(L, "opt_step_adamw", _tensor(L), 0, L.hparams(reset_interval=-1)) == -1


@pytest.mark.parametrize("args,status", [
    (dict(n=-1), -1),
    (dict(dtype=0), -1),
    (dict(stochastic=2), -1),
    (dict(x=None), -1),
    (dict(x=4100), -3),
    (dict(out=4098), -3),
])
def test_round_cast_bad_arguments(L, args, status):
    a = dict(x=4096, out=8192, n=16, dtype=1, stochastic=1)
    a.update(args)
    assert L.lib().opt_round_cast(a["x"], a["out"], a["n"], a["dtype"], a["stochastic"], 0, 0, None) == status


@no_device
def test_p16_rules(L):
    hp = L.hparams(p_rounding=2)
    assert _call(L, "opt_step_adamw", _tensor(L), 0, hp) == -1
    t = [L.OptTensor(4096, 4096, 8192, 12288, None, 16384, 16384, None, 16, 1, 1)]   # BF16 p, FP8 states
    assert _call(L, "opt_step_adamw", t, 4) not in (-1, -2)                           # accepted (needs a GPU)
    t = [L.OptTensor(4096, 4096, 8192, 12288, None, None, None, None, 16, 3, 0)]      # unknown p dtype
    assert _call(L, "opt_step_adamw", t, 0) == -1


def test_one_state_argument_checks(L):
    lib = L.lib()
    arr = (L.OptTensor * 1)(*_tensor(L))
    assert lib.opt_step_1state(9, arr, 1, 0, L.hparams(), None) == -1          # unknown optimizer
    assert lib.opt_step_1state(5, arr, 1, 3, L.hparams(), None) == -2          # blockwise states
    assert lib.opt_step_1state(5, arr, 1, 0, L.hparams(max_unorm=1.0), None) == -2
    assert lib.opt_step_1state(2, arr, 1, 0, L.hparams(skip_zeros=True, beta1=1.5), None) == -1
    bad = (L.OptTensor * 1)(L.OptTensor(4096, 4096, 0, 0, None, None, None, None, 16, 0, 0))
    assert lib.opt_step_1state(2, bad, 1, 0, L.hparams(), None) == -1         # no s1
    assert lib.opt_step_1state(2, None, 0, 0, L.hparams(), None) == 0


def test_binding_refuses_host_tensors(L):
    """The binding checks what the library cannot see: tensors that are not
    on the GPU are refused before any call."""
    import torch
    t = L.TensorList([{"p": torch.zeros(16), "g": torch.zeros(16), "s1": torch.zeros(16), "s2": torch.zeros(16)}])
    with pytest.raises(ValueError):
        t.check(L.STATE_F32, 2)
    with pytest.raises(ValueError):
        L.GradList([torch.zeros(16)])


def test_binding_refuses_bad_grad_scale_and_codebooks(L):
    """grad_scale is read by the kernels, so a host tensor (or another dtype)
    is refused; the codebooks are read on the host, so they must be float32
    host arrays of exactly 256 entries."""
    import torch
    with pytest.raises(ValueError):
        L.hparams(grad_scale=torch.ones(1))                       # host memory
    qs = np.asarray(QS, dtype=np.float32)
    for bad in (qs.astype(np.float64), qs[:255].copy(), np.concatenate([qs, qs[:1]]), qs[::-1],
                torch.from_numpy(qs.astype(np.float64)), list(qs)):
        with pytest.raises(ValueError):
            L.hparams(qmap_signed=bad, qmap_unsigned=QU)
    # float32 arrays of 256 in host memory, numpy or torch, are taken as they are
    h = L.hparams(qmap_signed=qs, qmap_unsigned=torch.from_numpy(np.asarray(QU, dtype=np.float32)))
    assert h.qmap_signed == qs.ctypes.data


@no_device
def test_size_limits(L):
    """numel above 2^46, or index_base + numel above 2^60, is refused before
    any work (the host's chunk arithmetic and the stream indices stay in
    range); sizes at the limits pass the checks and go on to need a GPU."""
    hp = L.hparams()
    for numel, base, bad in ((1 << 46, 0, False), ((1 << 46) + 4, 0, True),
                             (4096, (1 << 60) - 4096, False), (4096, (1 << 60) - 4092, True)):
        t = L.OptTensor(4096, 4096, 8192, 12288, None, None, None, None, numel, 0, 0)
        t.index_base = base
        rc = _call(L, "opt_step_adamw", [t], 0, hp)
        assert (rc == -1) == bad, (numel, base, rc, L.opt_last_error())
    g = L.OptGrad(4096, (1 << 46) + 1, 0, 0)
    arr = (L.OptGrad * 1)(g)
    assert L.lib().opt_grad_norm(arr, 1, 8192, 0.0, 2, None, None) == -1
    assert L.lib().opt_round_cast(4096, 8192, (1 << 46) + 1, 1, 0, 0, 0, None) == -1


@no_device
def test_index_base_and_stream_tensor_checks(L):
    """index_base must be >= 0 and a multiple of 4 (256 for the blockwise
    formats); sr_tensor_set must be 0 or 1, and sr_tensor >= 0 when set.
    Arguments that pass the checks go on to need a GPU (any other status)."""
    hp = L.hparams()
    for fmt, base, bad in ((0, 4, False), (0, 2, True), (0, -4, True), (2, 1 << 40, False),
                           (5, 128, True), (5, 512, False), (4, 256, False), (6, 100, True)):
        blk = fmt >= 3
        t = L.OptTensor(4096, 4096, 8192, 12288, None, 16384 if blk else None, 20480 if blk else None, None,
                        16, 0, 0)
        t.index_base = base
        rc = _call(L, "opt_step_adamw", [t], fmt, hp)
        assert (rc == -1) == bad, (fmt, base, rc, L.opt_last_error())
    for set_, k, bad in ((2, 0, True), (1, -1, True), (1, 0, False), (1, 7, False), (0, -5, False)):
        t = L.OptTensor(4096, 4096, 8192, 12288, None, None, None, None, 16, 0, 0)
        t.sr_tensor, t.sr_tensor_set = k, set_
        rc = _call(L, "opt_step_adamw", [t], 0, hp)
        assert (rc == -1) == bad, (set_, k, rc, L.opt_last_error())


def test_wg_cap_values(L):
    lib = L.lib()
    for bad in (-2, 1, 33, 1 << 20):
        assert lib.opt_debug_set_wg_cap(bad) == -1, bad
    for ok in (0, 2, 3, 32, -1):
        assert lib.opt_debug_set_wg_cap(ok) == 0, ok


@pytest.mark.parametrize("opt,hp,arrays,status", [
    (2, {}, (4096, 4096, 4096, 0, 4096), -1),                       # a one-state optimizer
    (0, dict(beta1=1.0), (4096, 4096, 4096, 0, 4096), -1),           # beta outside [0, 1)
    (0, dict(step=0), (4096, 4096, 4096, 0, 4096), -1),              # step < 1
    (0, {}, (0, 4096, 4096, 0, 4096), -1),                           # NULL g
    (1, {}, (4096, 4096, 4096, 0, 4096), -1),                        # AdEMAMix without m2
])
def test_debug_direction_checks_its_arguments(L, opt, hp, arrays, status):
    import ctypes
    h = L.hparams(**hp)
    g, m, v, m2, out = (a or None for a in arrays)
    assert L.lib().opt_debug_direction(opt, ctypes.byref(h), g, m, v, m2, out, 16, None) == status
    assert L.lib().opt_debug_direction(0, None, 4096, 4096, 4096, None, 4096, 16, None) == -1


@pytest.mark.parametrize("elem,n,A,status", [(3, 4, 1.0, -1), (0, 6, 1.0, -1), (0, -4, 1.0, -1), (1, 4, -1.0, -1)])
def test_mini_pack_checks_its_arguments(L, elem, n, A, status):
    assert L.lib().opt_debug_mini_pack(elem, A, 4096, None, 8192, n, None) == status

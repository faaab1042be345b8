"""CPU oracle for the fused element-wise two-state optimizer step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``optimizer_step_amd``) never imports it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, strict IEEE binary32 with no FMA
contraction); this module only marshals numpy arrays into it.  Inputs are numpy
arrays on the host:

* ``p``: float32 parameters, updated in place;
* ``g``: float32 gradients, or uint16 BF16 words (widened exactly, bits << 16);
* states: float32 (fp32 storage), uint16 (BF16 words) or uint8 (8-bit codes,
  FP8 codes, or two FP4 codes per byte), updated in place; 8-bit, FP8 and FP4
  storage also take float32 absmax arrays of ceil(n/256) entries per state,
  and 8-bit storage the two 256-entry codebooks.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ADAMW, ADEMAMIX = 0, 1
MOMENTUM, RMSPROP, ADAGRAD, LION = 2, 3, 4, 5
ONE_STATE = {"momentum": MOMENTUM, "rmsprop": RMSPROP, "adagrad": ADAGRAD, "lion": LION}
F32, BF16_RN, BF16_SR, Q8 = 0, 1, 2, 3
FP8_RN, FP8_SR, FP4_RN, FP4_SR = 4, 5, 6, 7
FORMATS = {"f32": F32, "bf16_rn": BF16_RN, "bf16_sr": BF16_SR, "q8": Q8,
           "fp8_rn": FP8_RN, "fp8_sr": FP8_SR, "fp4_rn": FP4_RN, "fp4_sr": FP4_SR}
BLOCKED = (Q8, FP8_RN, FP8_SR, FP4_RN, FP4_SR)
E4M3, E2M1, E2M2U = 0, 1, 2          # element formats of the FP8/FP4 states
OPTIMIZERS = {"adamw": ADAMW, "ademamix": ADEMAMIX}
BLOCK = 256


class HP(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("beta3", ctypes.c_float), ("alpha", ctypes.c_float), ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float), ("max_unorm", ctypes.c_float),
        ("step", ctypes.c_int64), ("seed", ctypes.c_uint64), ("index_base", ctypes.c_int64),
        ("tensor_index", ctypes.c_int32), ("decay_after", ctypes.c_int32),
        ("grad_scale", ctypes.c_float), ("reset_interval", ctypes.c_int64),
        ("skip_zeros", ctypes.c_int32), ("pad_", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Load liboracle.so, compiling it with gcc first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32
        L.orc_step.argtypes = [i32, i32, ctypes.POINTER(HP), f32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_step.restype = i32
        L.orc_unorm.argtypes = [i32, i32, ctypes.POINTER(HP), i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_unorm.restype = i32
        L.orc_unorm_scale.argtypes = [f32, ctypes.c_double, ctypes.c_double]
        L.orc_unorm_scale.restype = f32
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_philox4x32_10.restype = None
        L.orc_sr_word.argtypes = [ctypes.c_uint64, i64, i32, i64, i32]
        L.orc_sr_word.restype = ctypes.c_uint32
        L.orc_bf16_rne.argtypes = [f32]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_sr.argtypes = [f32, ctypes.c_uint32]
        L.orc_bf16_sr.restype = ctypes.c_uint16
        L.orc_quantize.argtypes = [vp, f32]
        L.orc_quantize.restype = i32
        L.orc_scalars.argtypes = [ctypes.POINTER(HP), f32, vp]
        L.orc_scalars.restype = None
        L.orc_bf16_rne_array.argtypes = [vp, vp, i64]
        L.orc_bf16_sr_array.argtypes = [vp, vp, vp, i64]
        L.orc_quantize_array.argtypes = [vp, vp, vp, i64]
        L.orc_sr_words.argtypes = [ctypes.c_uint64, i64, i32, i64, i64, i32, vp]
        for fn in (L.orc_bf16_rne_array, L.orc_bf16_sr_array, L.orc_quantize_array, L.orc_sr_words):
            fn.restype = None
        L.orc_grad_norm.argtypes = [vp, i64, vp]
        L.orc_grad_norm.restype = None
        L.orc_clip_coef.argtypes = [ctypes.c_double, f32]
        L.orc_clip_coef.restype = f32
        L.orc_mini_value.argtypes = [i32, i32]
        L.orc_mini_value.restype = ctypes.c_double
        L.orc_mini_round.argtypes = [i32, ctypes.c_double, i32]
        L.orc_mini_round.restype = i32
        L.orc_mini_encode.argtypes = [i32, f32, f32, i32]
        L.orc_mini_encode.restype = i32
        L.orc_mini_decode.argtypes = [i32, i32, f32]
        L.orc_mini_decode.restype = f32
        L.orc_mini_scale_exp.argtypes = [i32, f32]
        L.orc_mini_scale_exp.restype = i32
        L.orc_mini_round_array.argtypes = [i32, vp, vp, vp, i64]
        L.orc_mini_round_array.restype = None
        L.orc_f16_rne.argtypes = [f32]
        L.orc_f16_rne.restype = ctypes.c_uint16
        L.orc_f16_sr.argtypes = [f32, ctypes.c_uint32]
        L.orc_f16_sr.restype = ctypes.c_uint16
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = f32
        L.orc_f16_array.argtypes = [vp, vp, vp, i64]
        L.orc_f16_array.restype = None
        L.orc_step_p16.argtypes = [i32, i32, ctypes.POINTER(HP), f32, i64, vp, i32, i32, vp, vp, vp, vp,
                                   vp, vp, vp, vp, vp, vp]
        L.orc_step_p16.restype = i32
        L.orc_round_cast.argtypes = [vp, vp, i64, i32, i32, ctypes.c_uint64, ctypes.c_uint64]
        L.orc_round_cast.restype = None
        L.orc_step_1state.argtypes = [i32, i32, ctypes.POINTER(HP), i64, vp, vp, vp]
        L.orc_step_1state.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _need(a, dtype, n, name):
    if a is None:
        raise ValueError(f"{name} is required")
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"] or a.size != n:
        raise ValueError(f"{name}: need contiguous {np.dtype(dtype).name}[{n}], got {a.dtype}[{a.size}]")


def widen_bf16(words):
    """BF16 words (uint16) -> float32, exactly (the word is the high half)."""
    return (np.ascontiguousarray(words, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_hp(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
            weight_decay=0.0, max_unorm=0.0, step=1, seed=0, index_base=0,
            tensor_index=0, decay_after=False, grad_scale=1.0, reset_interval=0, skip_zeros=False):
    return HP(lr, beta1, beta2, beta3, alpha, eps, weight_decay, max_unorm,
              int(step), int(seed) & (2**64 - 1), int(index_base), int(tensor_index),
              1 if decay_after else 0, grad_scale, int(reset_interval), 1 if skip_zeros else 0, 0)


def _grad_f32(g):
    """BF16 words (uint16) or float16 or float32 -> float32, exactly."""
    if g.dtype == np.uint16:
        return widen_bf16(g)
    return np.ascontiguousarray(g, dtype=np.float32)


def _state_dtype(fmt):
    return {F32: np.float32, BF16_RN: np.uint16, BF16_SR: np.uint16}.get(fmt, np.uint8)


def state_len(fmt, n):
    """Entries of one state array for n elements (FP4: two codes per byte)."""
    return (n + 1) // 2 if fmt in (FP4_RN, FP4_SR) else n


def _check(opt, fmt, p, g, s1, s2, s3, a1, a2, a3, qs, qu):
    n = p.size
    _need(p, np.float32, n, "p")
    _need(g, np.float32, n, "g")
    sd = _state_dtype(fmt)
    ns = state_len(fmt, n)
    _need(s1, sd, ns, "s1")
    _need(s2, sd, ns, "s2")
    if opt == ADEMAMIX:
        _need(s3, sd, ns, "s3")
    if fmt in BLOCKED:
        nb = (n + BLOCK - 1) // BLOCK
        _need(a1, np.float32, nb, "a1")
        _need(a2, np.float32, nb, "a2")
        if opt == ADEMAMIX:
            _need(a3, np.float32, nb, "a3")
    if fmt == Q8:
        _need(qs, np.float32, 256, "qs")
        _need(qu, np.float32, 256, "qu")


P_F32, P_BF16, P_F16 = 0, 1, 2


def step(opt, fmt, hp, p, g, s1, s2, s3=None, a1=None, a2=None, a3=None,
         qs=None, qu=None, scale=1.0, p_dtype=None, p_sr=False):
    """One optimizer step over one tensor, in place on p and the states.  p is
    float32, or 16-bit words with p_dtype P_BF16 / P_F16 (stored back rounded
    to nearest-even, or stochastically if p_sr)."""
    opt = OPTIMIZERS.get(opt, opt)
    fmt = FORMATS.get(fmt, fmt)
    g = _grad_f32(g)
    if p_dtype in (P_BF16, P_F16):
        if p.dtype != np.uint16 or not p.flags["C_CONTIGUOUS"]:
            raise ValueError("16-bit parameters are uint16 words")
        work = np.zeros(p.size, dtype=np.float32)
        _check(opt, fmt, work, g, s1, s2, s3, a1, a2, a3, qs, qu)
        rc = lib().orc_step_p16(opt, fmt, ctypes.byref(hp), scale, p.size, _ptr(p), p_dtype, 1 if p_sr else 0,
                                _ptr(g), _ptr(s1), _ptr(s2), _ptr(s3), _ptr(a1), _ptr(a2), _ptr(a3),
                                _ptr(qs), _ptr(qu), _ptr(work))
        if rc != 0:
            raise ValueError("orc_step_p16 rejected its arguments")
        return
    _check(opt, fmt, p, g, s1, s2, s3, a1, a2, a3, qs, qu)
    rc = lib().orc_step(opt, fmt, ctypes.byref(hp), scale, p.size, _ptr(p), _ptr(g),
                        _ptr(s1), _ptr(s2), _ptr(s3), _ptr(a1), _ptr(a2), _ptr(a3),
                        _ptr(qs), _ptr(qu))
    if rc != 0:
        raise ValueError("orc_step rejected its arguments")


def unorm(opt, fmt, hp, p, g, s1, s2, s3=None, a1=None, a2=None, a3=None, qs=None, qu=None):
    """(sum u^2, sum p^2) in binary64 for one tensor, before the step."""
    opt = OPTIMIZERS.get(opt, opt)
    fmt = FORMATS.get(fmt, fmt)
    g = _grad_f32(g)
    _check(opt, fmt, p, g, s1, s2, s3, a1, a2, a3, qs, qu)
    out = np.zeros(2, dtype=np.float64)
    rc = lib().orc_unorm(opt, fmt, ctypes.byref(hp), p.size, _ptr(p), _ptr(g),
                         _ptr(s1), _ptr(s2), _ptr(s3), _ptr(a1), _ptr(a2), _ptr(a3),
                         _ptr(qs), _ptr(qu), _ptr(out))
    if rc != 0:
        raise ValueError("orc_unorm rejected its arguments")
    return float(out[0]), float(out[1])


def unorm_scale(max_unorm, u2, p2):
    return float(lib().orc_unorm_scale(max_unorm, u2, p2))


def scalars(hp, scale=1.0):
    """(1-b1, 1-b2, 1-b3, c1, c2, d, lambda) as the oracle forms them."""
    out = np.zeros(7, dtype=np.float32)
    lib().orc_scalars(ctypes.byref(hp), scale, _ptr(out))
    return out


def philox(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed, t, k, j, stream=0):
    return int(lib().orc_sr_word(seed & (2**64 - 1), t, k, j, stream))


def bf16_rne(x):
    return int(lib().orc_bf16_rne(float(np.float32(x))))


def bf16_sr(x, r):
    return int(lib().orc_bf16_sr(float(np.float32(x)), int(r)))


def bf16_rne_array(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_sr_array(x, r):
    x = np.ascontiguousarray(x, dtype=np.float32)
    r = np.ascontiguousarray(np.broadcast_to(np.asarray(r, dtype=np.uint32), x.shape))
    out = np.empty(x.size, dtype=np.uint16)
    lib().orc_bf16_sr_array(_ptr(x), _ptr(r), _ptr(out), x.size)
    return out


def quantize_array(T, x):
    T = np.ascontiguousarray(T, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint8)
    lib().orc_quantize_array(_ptr(T), _ptr(x), _ptr(out), x.size)
    return out


def sr_words(seed, t, k, j0, n, stream=0):
    out = np.empty(n, dtype=np.uint32)
    lib().orc_sr_words(seed & (2**64 - 1), t, k, j0, n, stream, _ptr(out))
    return out


def quantize(T, x):
    T = np.ascontiguousarray(T, dtype=np.float32)
    return int(lib().orc_quantize(_ptr(T), float(np.float32(x))))


def state_zeros(fmt, n, opt="adamw", qs=None, qu=None):
    """Fresh (zero) optimizer state for n elements in format fmt.

    For 8-bit storage the zero state is the code of 0 in each codebook with an
    absmax of 0, so it reads back as exactly 0 (the pages: a fresh state "is
    still zero and therefore quantizes exactly").
    """
    fmt = FORMATS.get(fmt, fmt)
    opt = OPTIMIZERS.get(opt, opt)
    nst = 3 if opt == ADEMAMIX else 2
    st = {}
    if fmt == Q8:
        nb = (n + BLOCK - 1) // BLOCK
        cs = quantize(qs, 0.0)
        cu = quantize(qu, 0.0)
        st["s1"] = np.full(n, cs, dtype=np.uint8)
        st["s2"] = np.full(n, cu, dtype=np.uint8)
        st["a1"] = np.zeros(nb, dtype=np.float32)
        st["a2"] = np.zeros(nb, dtype=np.float32)
        if nst == 3:
            st["s3"] = np.full(n, cs, dtype=np.uint8)
            st["a3"] = np.zeros(nb, dtype=np.float32)
    elif fmt in BLOCKED:
        # code 0 is +0 in every FP8/FP4 element format; absmax 0 reads back 0
        nb = (n + BLOCK - 1) // BLOCK
        for i in range(1, nst + 1):
            st[f"s{i}"] = np.zeros(state_len(fmt, n), dtype=np.uint8)
            st[f"a{i}"] = np.zeros(nb, dtype=np.float32)
    else:
        dt = _state_dtype(fmt)
        for i in range(1, nst + 1):
            st[f"s{i}"] = np.zeros(n, dtype=dt)
    return st


# --------------------------------------------------------------------------
# FP8 / FP4 element codecs (format ids E4M3, E2M1, E2M2U)

def mini_value(f, mag):
    return float(lib().orc_mini_value(f, int(mag)))


def mini_round(f, y, r=-1):
    """Magnitude code of y >= 0 (already divided by the block scale); r < 0 is
    nearest rounding, else stochastic with the 16-bit integer r."""
    return int(lib().orc_mini_round(f, float(y), int(r)))


def mini_round_array(f, y, r=None):
    y = np.ascontiguousarray(y, dtype=np.float64)
    rr = None if r is None else np.ascontiguousarray(np.broadcast_to(np.asarray(r, dtype=np.int32), y.shape))
    out = np.empty(y.size, dtype=np.int32)
    lib().orc_mini_round_array(f, _ptr(y), _ptr(rr), _ptr(out), y.size)
    return out


def mini_encode(f, x, A, r=-1):
    return int(lib().orc_mini_encode(f, float(np.float32(x)), float(np.float32(A)), int(r)))


def mini_decode(f, code, A):
    return float(np.float32(lib().orc_mini_decode(f, int(code), float(np.float32(A)))))


def mini_scale_exp(f, A):
    return int(lib().orc_mini_scale_exp(f, float(np.float32(A))))


def unpack_fp4(codes, n):
    """FP4 state bytes -> one code per element (element 2i in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(2 * c.size, dtype=np.uint8)
    out[0::2] = c & 0xF
    out[1::2] = c >> 4
    return out[:n]


def grad_norm(g):
    """(sum g^2, max |g|) of one gradient tensor, binary64; g is float32 or
    BF16 words (widened exactly)."""
    g = _grad_f32(g)
    out = np.zeros(2, dtype=np.float64)
    lib().orc_grad_norm(_ptr(g), g.size, _ptr(out))
    return float(out[0]), float(out[1])


def grad_norm_list(grads):
    """Norms of a list: per-tensor (sum g^2, max|g|), then the list totals
    (sums of the per-tensor sums in list order, compensated; max of maxes,
    NaN if any is NaN)."""
    per = [grad_norm(g) for g in grads]
    s, c = 0.0, 0.0
    for x, _ in per:        # Neumaier over the per-tensor sums, in list order
        t = s + x
        c += ((s - t) + x) if abs(s) >= abs(x) else ((x - t) + s)
        s = t
    maxes = [m for _, m in per]
    mx = float("nan") if any(m != m for m in maxes) else max(maxes, default=0.0)
    total = s + c if np.isfinite(s) else s
    return (total, mx), per


def clip_coef(norm, max_norm):
    return float(lib().orc_clip_coef(float(norm), float(max_norm)))


# --------------------------------------------------------------------------
# FP16 rounding and the standalone cast

def f16_rne(x):
    return int(lib().orc_f16_rne(float(np.float32(x))))


def f16_sr(x, r):
    return int(lib().orc_f16_sr(float(np.float32(x)), int(r)))


def f16_array(x, r=None):
    """FP16 words of float32 values: nearest-even, or stochastic with r."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rr = None if r is None else np.ascontiguousarray(np.broadcast_to(np.asarray(r, dtype=np.uint32), x.shape))
    out = np.empty(x.size, dtype=np.uint16)
    lib().orc_f16_array(_ptr(x), _ptr(rr), _ptr(out), x.size)
    return out


def widen_f16(words):
    w = np.ascontiguousarray(words, dtype=np.uint16)
    return np.array([lib().orc_f16_to_f32(int(h)) for h in w], dtype=np.float32)


def round_cast(x, dtype, stochastic=False, seed=0, offset=0):
    """fp32 -> BF16 (dtype P_BF16) or FP16 (P_F16) words, as one pass."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().orc_round_cast(_ptr(x), _ptr(out), x.size, dtype, 1 if stochastic else 0,
                         int(seed) & (2**64 - 1), int(offset) & (2**64 - 1))
    return out


# --------------------------------------------------------------------------
# one-state optimizers

def step_1state(opt, fmt, hp, p, g, s1):
    """One momentum / RMSprop / Adagrad / Lion step over one tensor, in place
    on p (float32) and s1 (float32, or BF16 words for the BF16 formats)."""
    opt = ONE_STATE.get(opt, opt)
    fmt = FORMATS.get(fmt, fmt)
    g = _grad_f32(g)
    n = p.size
    _need(p, np.float32, n, "p")
    _need(g, np.float32, n, "g")
    _need(s1, np.float32 if fmt == F32 else np.uint16, n, "s1")
    if lib().orc_step_1state(opt, fmt, ctypes.byref(hp), n, _ptr(p), _ptr(g), _ptr(s1)) != 0:
        raise ValueError("orc_step_1state rejected its arguments")

"""Python binding of the MI355X fused optimizer-step library (libopt_step.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/opt_step.h``; PyTorch supplies
device memory and streams.  Function names match the C entry points.  If the
library has not been built, every call raises (there is no other code path).

Tensors are passed as a list of dicts with torch CUDA tensors under the keys
``p``, ``g``, ``s1``, ``s2`` and, as the format and optimizer need, ``s3``,
``absmax1``, ``absmax2``, ``absmax3`` (see ``opt_tensor`` in the header).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libopt_step.so")

OPT_OK, OPT_EINVAL, OPT_EUNSUPPORTED, OPT_EALIGN, OPT_EHIP = 0, -1, -2, -3, -4
OPT_F32, OPT_BF16, OPT_F16 = 0, 1, 2
STATE_F32, STATE_BF16_RN, STATE_BF16_SR, STATE_Q8 = 0, 1, 2, 3
STATE_FP8_RN, STATE_FP8_SR, STATE_FP4_RN, STATE_FP4_SR = 4, 5, 6, 7
ADAMW, ADEMAMIX = 0, 1
MOMENTUM, RMSPROP, ADAGRAD, LION = 2, 3, 4, 5
ONE_STATE = {"momentum": MOMENTUM, "rmsprop": RMSPROP, "adagrad": ADAGRAD, "lion": LION}
FORMATS = {"f32": STATE_F32, "bf16_rn": STATE_BF16_RN, "bf16_sr": STATE_BF16_SR, "q8": STATE_Q8,
           "fp8_rn": STATE_FP8_RN, "fp8_sr": STATE_FP8_SR, "fp4_rn": STATE_FP4_RN, "fp4_sr": STATE_FP4_SR}
BLOCKED = (STATE_Q8, STATE_FP8_RN, STATE_FP8_SR, STATE_FP4_RN, STATE_FP4_SR)
ELEM_E4M3, ELEM_E2M1, ELEM_E2M2U = 0, 1, 2
OPTIMIZERS = {"adamw": ADAMW, "ademamix": ADEMAMIX}
BLOCK = 256


class OptError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status


class OptTensor(ctypes.Structure):
    _fields_ = [
        ("p", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("s1", ctypes.c_void_p), ("s2", ctypes.c_void_p), ("s3", ctypes.c_void_p),
        ("absmax1", ctypes.c_void_p), ("absmax2", ctypes.c_void_p), ("absmax3", ctypes.c_void_p),
        ("numel", ctypes.c_int64), ("p_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32),
        ("index_base", ctypes.c_int64), ("sr_tensor", ctypes.c_int32), ("sr_tensor_set", ctypes.c_int32),
    ]


class OptHparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
        ("beta3", ctypes.c_float), ("alpha", ctypes.c_float), ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float), ("max_unorm", ctypes.c_float),
        ("step", ctypes.c_int64), ("seed", ctypes.c_uint64),
        ("qmap_signed", ctypes.c_void_p), ("qmap_unsigned", ctypes.c_void_p),
        ("grad_scale", ctypes.c_void_p), ("p_rounding", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("reset_interval", ctypes.c_int64), ("skip_zeros", ctypes.c_int32), ("reserved2", ctypes.c_int32),
    ]


class OptGrad(ctypes.Structure):
    _fields_ = [("g", ctypes.c_void_p), ("numel", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with optimizer_step_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        T = ctypes.POINTER(OptTensor)
        H = ctypes.POINTER(OptHparams)
        sig = {
            "opt_step_adamw": ([T, i64, i32, H, vp, vp], i32),
            "opt_step_ademamix": ([T, i64, i32, H, vp, vp], i32),
            "opt_step_adamw_noalloc": ([T, i64, i32, H, vp, vp], i32),
            "opt_precondition_unorm": ([i32, T, i64, i32, H, vp, vp], i32),
            "opt_last_error": ([], ctypes.c_char_p),
            "opt_shutdown": ([], i32),
            "opt_debug_philox": ([ctypes.c_uint64, i64, i32, i64, i64, vp, vp], i32),
            "opt_debug_round_bf16": ([vp, vp, vp, i64, vp], i32),
            "opt_debug_direction": ([i32, vp, vp, vp, vp, vp, vp, i64, vp], i32),
            "opt_debug_quantize": ([vp, i32, vp, vp, i64, vp], i32),
            "opt_debug_plan": ([vp, i64, vp], i64),
            "opt_debug_quantize_host": ([vp, i32, vp, vp, i64], i32),
            "opt_debug_div_by": ([vp, vp, vp, i64], i32),
            "opt_debug_set_launch": ([i64, i32], i32),
            "opt_debug_set_wg_cap": ([i32], i32),
            "opt_debug_scalars": ([H, vp], i32),
            "opt_debug_stream": ([vp, i32, vp, i32, i64, vp], i32),
            "opt_grad_norm": ([ctypes.POINTER(OptGrad), i64, vp, ctypes.c_float, i32, vp, vp], i32),
            "opt_debug_mini": ([i32, ctypes.c_float, vp, vp, vp, vp, i64, vp], i32),
            "opt_debug_mini_pack": ([i32, ctypes.c_float, vp, vp, vp, i64, vp], i32),
            "opt_round_cast": ([vp, vp, i64, i32, i32, ctypes.c_uint64, ctypes.c_uint64, vp], i32),
            "opt_step_1state": ([i32, T, i64, i32, H, vp], i32),
            "opt_debug_mini_host": ([i32, ctypes.c_float, vp, vp, vp, vp, i64], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status):
    if status != OPT_OK:
        raise OptError(status, lib().opt_last_error().decode())
    return status


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return OPT_F32
    if t.dtype == torch.bfloat16:
        return OPT_BF16
    if t.dtype == torch.float16:
        return OPT_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _current_device(tensors):
    """The current CUDA device index if any tensor given is a CUDA tensor
    (else None: the per-tensor checks then refuse the host tensors)."""
    for d in tensors:
        for t in d.values():
            if getattr(t, "is_cuda", False):
                import torch
                return torch.cuda.current_device()
    return None


def _host_qmap(q, name):
    """Address of a 256-entry float32 codebook in host memory (numpy array or
    CPU torch tensor), which the library reads on the host."""
    if hasattr(q, "data_ptr"):
        import torch
        if q.is_cuda or q.dtype != torch.float32 or not q.is_contiguous() or q.numel() != 256:
            raise ValueError(f"{name} must be a contiguous CPU float32 tensor of 256 entries")
        return q.data_ptr()
    import numpy as np
    if not isinstance(q, np.ndarray) or q.dtype != np.float32 or not q.flags["C_CONTIGUOUS"] or q.size != 256:
        raise ValueError(f"{name} must be a C-contiguous float32 numpy array of 256 entries")
    return q.ctypes.data


class TensorList:
    """The C array of opt_tensor for a list of tensor dicts; build it once and
    pass it to every step when the buffers do not change.  A dict may carry
    "index_base" (the slice's first element within its whole tensor) and
    "sr_tensor" (the tensor number of its stochastic-rounding stream).  All
    tensors must sit on the current CUDA device, whose stream runs the step."""

    def __init__(self, tensors):
        self.keep = list(tensors)
        self.arr = (OptTensor * max(1, len(self.keep)))()
        for i, d in enumerate(self.keep):
            p = d["p"]
            self.arr[i] = OptTensor(
                _ptr(p), _ptr(d["g"]), _ptr(d.get("s1")), _ptr(d.get("s2")), _ptr(d.get("s3")),
                _ptr(d.get("absmax1")), _ptr(d.get("absmax2")), _ptr(d.get("absmax3")),
                p.numel(), _dtype_code(p), _dtype_code(d["g"]), int(d.get("index_base", 0)),
                int(d.get("sr_tensor", 0)), 1 if d.get("sr_tensor") is not None else 0)
        self.n = len(self.keep)
        self._checked = set()

    def check(self, state_fmt, nstates):
        """Raise ValueError unless every tensor given is a contiguous CUDA
        tensor, g has p's element count, and each of the first nstates states
        (and, for the blockwise formats, its absmax array) holds at least the
        bytes the format needs: the library sees only pointers, so a short or
        strided buffer would be read out of bounds.  Checked once per format."""
        dev = _current_device(self.keep)
        key = (state_fmt, nstates, dev)
        if key in self._checked:
            return
        per = {STATE_F32: 8, STATE_BF16_RN: 4, STATE_BF16_SR: 4}.get(state_fmt, 2)   # half-bytes per element
        if state_fmt in (STATE_FP4_RN, STATE_FP4_SR):
            per = 1
        for i, d in enumerate(self.keep):
            n = d["p"].numel()
            for name, t in d.items():
                if hasattr(t, "is_cuda") and (not t.is_cuda or not t.is_contiguous()):
                    raise ValueError(f"tensor {i}: {name} must be a contiguous CUDA tensor")
                if hasattr(t, "is_cuda") and t.device.index != dev:
                    raise ValueError(f"tensor {i}: {name} is on {t.device}, not on the current device cuda:{dev}")
            if d["g"].numel() != n:
                raise ValueError(f"tensor {i}: g has {d['g'].numel()} elements, p has {n}")
            for j in range(1, nstates + 1):
                s = d.get(f"s{j}")
                if s is not None and 2 * s.numel() * s.element_size() < per * n:
                    raise ValueError(f"tensor {i}: s{j} is shorter than {n} elements of this state format")
                a = d.get(f"absmax{j}")
                if state_fmt in BLOCKED and a is not None and a.numel() * a.element_size() < 4 * ((n + BLOCK - 1) // BLOCK):
                    raise ValueError(f"tensor {i}: absmax{j} holds fewer than ceil({n}/256) floats")
        self._checked.add(key)


def _as_list(tensors):
    return tensors if isinstance(tensors, TensorList) else TensorList(tensors)


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
            weight_decay=0.0, max_unorm=0.0, step=1, seed=0, qmap_signed=None, qmap_unsigned=None,
            grad_scale=None, reset_interval=0, p_rounding=0, skip_zeros=False):
    """An OptHparams record.  qmap_* are host float32 arrays (numpy or CPU
    torch tensors) of 256 entries; they are referenced, not copied, so keep
    them alive for the call.  grad_scale is a CUDA float tensor of one element
    (for instance the clipping coefficient opt_grad_norm wrote), or None.
    reset_interval R > 0 restarts the moments from zero every R steps;
    p_rounding 1 stores BF16/FP16 parameters with stochastic rounding;
    skip_zeros leaves elements whose gradient is exactly 0 untouched."""
    if grad_scale is not None:
        import torch
        _device_buffer(grad_scale, 4, 1, "grad_scale")
        if grad_scale.dtype != torch.float32:
            raise ValueError("grad_scale must be a CUDA float32 tensor")
    h = OptHparams(lr, beta1, beta2, beta3, alpha, eps, weight_decay, max_unorm,
                   int(step), int(seed) & (2**64 - 1), None, None, _ptr(grad_scale), int(p_rounding), 0,
                   int(reset_interval), 1 if skip_zeros else 0, 0)
    for field, q in (("qmap_signed", qmap_signed), ("qmap_unsigned", qmap_unsigned)):
        if q is not None:
            setattr(h, field, _host_qmap(q, field))
    h._keep = (qmap_signed, qmap_unsigned, grad_scale)
    return h


class GradList:
    """The C array of opt_grad for a list of gradient tensors, each checked
    once (a contiguous CUDA tensor on the current device); pass it to
    opt_grad_norm in place of the list while the buffers do not change."""

    def __init__(self, grads):
        import torch
        self.keep = list(grads)
        self.arr = (OptGrad * max(1, len(self.keep)))()
        dev = torch.cuda.current_device() if any(getattr(g, "is_cuda", False) for g in self.keep) else None
        for i, g in enumerate(self.keep):
            if not g.is_cuda or not g.is_contiguous():
                raise ValueError(f"gradient {i} must be a contiguous CUDA tensor")
            if g.device.index != dev:
                raise ValueError(f"gradient {i} is on {g.device}, not on the current device")
            self.arr[i] = OptGrad(_ptr(g), g.numel(), _dtype_code(g), 0)
        self.n = len(self.keep)


def opt_grad_norm(grads, out, max_norm=0.0, norm_type=2, coef_out=None, stream=None):
    """Norms of a list of CUDA gradient tensors (or a GradList) into out (CUDA
    float64 tensor of 2 + 2n): totals then per-tensor {sum g^2, max |g|};
    optionally the clipping coefficient into coef_out (CUDA float32 tensor of
    1)."""
    gl = grads if isinstance(grads, GradList) else GradList(grads)
    _device_buffer(out, 8, 2 + 2 * gl.n, "out")
    _device_buffer(coef_out, 4, 1, "coef_out")
    return _check(lib().opt_grad_norm(gl.arr, gl.n, _ptr(out), float(max_norm), int(norm_type),
                                      _ptr(coef_out), _stream(stream)))


def _device_buffer(t, itemsize, count, what):
    """Raise ValueError unless t (if given) is a contiguous CUDA tensor of
    `itemsize`-byte elements holding at least `count` of them."""
    if t is not None and (not t.is_cuda or not t.is_contiguous() or t.element_size() != itemsize
                          or t.numel() < count):
        raise ValueError(f"{what} must be a contiguous CUDA tensor of >= {count} {itemsize}-byte elements")
    _same_device(t, what)


def _same_device(t, what):
    if t is not None:
        import torch
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{what} is on {t.device}, not on the current device")


def _norm_buffer(t, n):
    """The per-tensor {sum u^2, sum p^2} buffer: CUDA float64, 2n entries."""
    if t is not None and (not t.is_cuda or not t.is_contiguous() or t.element_size() != 8 or t.numel() < 2 * n):
        raise ValueError(f"the update-norm buffer must be a contiguous CUDA float64 tensor of >= {2 * n} entries")
    _same_device(t, "the update-norm buffer")
    return _ptr(t)


def opt_step_adamw(tensors, state_fmt, hp, unorm=None, stream=None):
    tl = _as_list(tensors)
    fmt = FORMATS.get(state_fmt, state_fmt)
    tl.check(fmt, 2)
    return _check(lib().opt_step_adamw(tl.arr, tl.n, fmt, ctypes.byref(hp), _norm_buffer(unorm, tl.n),
                                       _stream(stream)))


def opt_step_adamw_noalloc(tensors, state_fmt, hp, unorm=None, stream=None):
    """opt_step_adamw that allocates no device memory (the library's fixed
    2 MiB table array instead of its workspace); calls that overlap on one
    GPU race."""
    tl = _as_list(tensors)
    fmt = FORMATS.get(state_fmt, state_fmt)
    tl.check(fmt, 2)
    return _check(lib().opt_step_adamw_noalloc(tl.arr, tl.n, fmt, ctypes.byref(hp), _norm_buffer(unorm, tl.n),
                                               _stream(stream)))


def opt_step_ademamix(tensors, state_fmt, hp, unorm=None, stream=None):
    tl = _as_list(tensors)
    fmt = FORMATS.get(state_fmt, state_fmt)
    tl.check(fmt, 3)
    return _check(lib().opt_step_ademamix(tl.arr, tl.n, fmt, ctypes.byref(hp), _norm_buffer(unorm, tl.n),
                                          _stream(stream)))


def opt_step_1state(optimizer, tensors, state_fmt, hp, stream=None):
    """One momentum / RMSprop / Adagrad / Lion step; tensors need p, g, s1."""
    tl = _as_list(tensors)
    fmt = FORMATS.get(state_fmt, state_fmt)
    tl.check(fmt, 1)
    return _check(lib().opt_step_1state(ONE_STATE.get(optimizer, optimizer), tl.arr, tl.n, fmt, ctypes.byref(hp),
                                        _stream(stream)))


def opt_precondition_unorm(optimizer, tensors, state_fmt, hp, unorm_out, stream=None):
    tl = _as_list(tensors)
    fmt = FORMATS.get(state_fmt, state_fmt)
    opt = OPTIMIZERS.get(optimizer, optimizer)
    tl.check(fmt, 3 if opt == ADEMAMIX else 2)
    return _check(lib().opt_precondition_unorm(opt, tl.arr, tl.n, fmt, ctypes.byref(hp),
                                               _norm_buffer(unorm_out, tl.n), _stream(stream)))


def opt_last_error():
    return lib().opt_last_error().decode()


def opt_shutdown():
    return _check(lib().opt_shutdown())


def opt_debug_philox(seed, t, k, j0, out, stream=None):
    return _check(lib().opt_debug_philox(int(seed) & (2**64 - 1), t, k, j0, out.numel(), _ptr(out),
                                         _stream(stream)))


def opt_debug_direction(optimizer, hp, g, m, v, m2, out, stream=None):
    """out (device float[3n]): the fast direction, its error bound and the
    exact recipe's direction of each element (m2 unused for AdamW)."""
    code = ADEMAMIX if optimizer == "ademamix" else ADAMW
    return _check(lib().opt_debug_direction(code, ctypes.byref(hp), _ptr(g), _ptr(m), _ptr(v),
                                            _ptr(m2) if m2 is not None else None, _ptr(out), g.numel(),
                                            _stream(stream)))


def opt_debug_round_bf16(x, r, out, stream=None):
    return _check(lib().opt_debug_round_bf16(_ptr(x), _ptr(r), _ptr(out), x.numel(), _stream(stream)))


def opt_debug_quantize(qmap, is_signed, x, out, stream=None):
    return _check(lib().opt_debug_quantize(qmap.ctypes.data, int(is_signed), _ptr(x), _ptr(out),
                                           x.numel(), _stream(stream)))


def opt_debug_plan(numels):
    import numpy as np
    a = np.ascontiguousarray(numels, dtype=np.int64)
    out = np.zeros(a.size, dtype=np.int64)
    chunk = lib().opt_debug_plan(a.ctypes.data, a.size, out.ctypes.data)
    if chunk < 0:
        _check(int(chunk))
    return int(chunk), out


def opt_debug_quantize_host(qmap, is_signed, x):
    import numpy as np
    q = np.ascontiguousarray(qmap, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.size, dtype=np.uint8)
    _check(lib().opt_debug_quantize_host(q.ctypes.data, int(is_signed), x.ctypes.data, out.ctypes.data,
                                         x.size))
    return out


def opt_debug_div_by(a, b):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    out = np.zeros(a.size, dtype=np.float32)
    _check(lib().opt_debug_div_by(a.ctypes.data, b.ctypes.data, out.ctypes.data, a.size))
    return out


def opt_debug_stream(srcs, dsts, stream=None):
    n = dsts[0].numel()
    S = (ctypes.c_void_p * max(1, len(srcs)))(*[t.data_ptr() for t in srcs])
    D = (ctypes.c_void_p * len(dsts))(*[t.data_ptr() for t in dsts])
    return _check(lib().opt_debug_stream(S, len(srcs), D, len(dsts), n, _stream(stream)))


def opt_round_cast(x, out, stochastic=False, seed=0, offset=0, stream=None):
    """x (CUDA float32) -> out (CUDA bfloat16 or float16), nearest-even or
    stochastic."""
    _device_buffer(x, 4, x.numel(), "x")
    _device_buffer(out, 2, x.numel(), "out")
    return _check(lib().opt_round_cast(_ptr(x), _ptr(out), x.numel(), _dtype_code(out), 1 if stochastic else 0,
                                       int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), _stream(stream)))


def opt_debug_mini(elem, A, x, r, codes, decoded, stream=None):
    return _check(lib().opt_debug_mini(int(elem), float(A), _ptr(x), _ptr(r), _ptr(codes), _ptr(decoded),
                                       x.numel(), _stream(stream)))


def opt_debug_mini_pack(elem, A, x, r, codes, stream=None):
    """The blockwise step's encoder (hardware conversions included) on the
    device, four values at a time; x.numel() a multiple of 4."""
    return _check(lib().opt_debug_mini_pack(int(elem), float(A), _ptr(x), _ptr(r) if r is not None else None,
                                            _ptr(codes), x.numel(), _stream(stream)))


def opt_debug_mini_host(elem, A, x, r=None):
    import numpy as np
    x = np.ascontiguousarray(x, dtype=np.float32)
    rr = None if r is None else np.ascontiguousarray(np.broadcast_to(np.asarray(r, dtype=np.uint32), x.shape))
    codes = np.zeros(x.size, dtype=np.uint8)
    dec = np.zeros(x.size, dtype=np.float32)
    _check(lib().opt_debug_mini_host(int(elem), float(A), x.ctypes.data, None if rr is None else rr.ctypes.data,
                                     codes.ctypes.data, dec.ctypes.data, x.size))
    return codes, dec


def opt_debug_set_launch(chunk, wgs_per_cu):
    return _check(lib().opt_debug_set_launch(int(chunk), int(wgs_per_cu)))


def opt_debug_scalars(hp):
    """The per-call scalars the host forms for hp (numpy float32[10])."""
    import numpy as np
    out = np.zeros(10, dtype=np.float32)
    _check(lib().opt_debug_scalars(ctypes.byref(hp), out.ctypes.data))
    return out


def opt_debug_set_wg_cap(cap):
    return _check(lib().opt_debug_set_wg_cap(int(cap)))


def state_buffers(fmt, numel, optimizer="adamw", device="cuda", qmap_signed=None, qmap_unsigned=None):
    """Fresh (zero) optimizer state on the device for one tensor, as a dict of
    s1, s2[, s3][, absmax1, absmax2[, absmax3]].  8-bit codes start at the
    code of 0 in each codebook (the index of its 0 entry) with absmax 0; FP8
    and FP4 codes at 0 (FP4: two per byte) with absmax 0."""
    import torch
    import numpy as np
    fmt = FORMATS.get(fmt, fmt)
    o = OPTIMIZERS.get(optimizer, ONE_STATE.get(optimizer, optimizer))
    nst = 3 if o == ADEMAMIX else (2 if o == ADAMW else 1)
    out = {}
    if fmt == STATE_Q8:
        nb = (numel + BLOCK - 1) // BLOCK
        zs = int(np.argmin(np.abs(np.asarray(qmap_signed, dtype=np.float64))))
        zu = int(np.argmin(np.abs(np.asarray(qmap_unsigned, dtype=np.float64))))
        for i in range(1, nst + 1):
            out[f"s{i}"] = torch.full((numel,), zu if i == 2 else zs, dtype=torch.uint8, device=device)
            out[f"absmax{i}"] = torch.zeros(nb, dtype=torch.float32, device=device)
    elif fmt in BLOCKED:
        nb = (numel + BLOCK - 1) // BLOCK
        nbytes = (numel + 1) // 2 if fmt in (STATE_FP4_RN, STATE_FP4_SR) else numel
        for i in range(1, nst + 1):
            out[f"s{i}"] = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            out[f"absmax{i}"] = torch.zeros(nb, dtype=torch.float32, device=device)
    else:
        dt = torch.float32 if fmt == STATE_F32 else torch.bfloat16
        for i in range(1, nst + 1):
            out[f"s{i}"] = torch.zeros(numel, dtype=dt, device=device)
    return out

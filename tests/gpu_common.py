"""Helpers for the GPU parity tests: run the HIP path through the binding and
the oracle on the same seeded inputs, and compare to the stated bars."""
import numpy as np

import oracle
import synth

FP32_REL = 1e-6   # |gpu - oracle| <= 1e-6 * max(|oracle|, rms(oracle)), per element


def torch():
    import torch as t
    return t


def to_dev(a):
    """numpy -> CUDA tensor; uint16 arrays become bfloat16 tensors (same bits)."""
    T = torch()
    if a.dtype == np.uint16:
        return T.from_numpy(a.view(np.int16).copy()).cuda().view(T.bfloat16)
    return T.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    T = torch()
    if t.dtype == T.bfloat16:
        return t.view(T.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def fp32_close(gpu, orc, rel=FP32_REL):
    """The fp32 bar; NaNs must sit at the same places."""
    g = gpu.astype(np.float64)
    o = orc.astype(np.float64)
    nan = np.isnan(o)
    if not np.array_equal(np.isnan(g), nan):
        return False
    ok = ~nan
    if not ok.any():
        return True
    fin = ok & np.isfinite(o)
    if not np.array_equal(g[ok & ~np.isfinite(o)], o[ok & ~np.isfinite(o)]):
        return False
    if not fin.any():
        return True
    scale = np.maximum(np.abs(o[fin]), np.sqrt(np.mean(o[fin] ** 2)))
    return bool(np.all(np.abs(g[fin] - o[fin]) <= rel * scale))


def bf16_ulps(gpu_words, orc_words):
    """Distance in BF16 steps (same-sign words; NaNs compared by position)."""
    g = oracle.widen_bf16(gpu_words).astype(np.float64)
    o = oracle.widen_bf16(orc_words).astype(np.float64)
    nan = np.isnan(o)
    assert np.array_equal(np.isnan(g), nan)
    gi = gpu_words.astype(np.int64)
    oi = orc_words.astype(np.int64)
    gi = np.where(gi & 0x8000, -(gi & 0x7FFF), gi)
    oi = np.where(oi & 0x8000, -(oi & 0x7FFF), oi)
    d = np.abs(gi - oi)
    d[nan] = 0
    return d


def nan_equal_bits(a, b):
    """Bit equality, treating any two NaNs as equal (payloads differ by CPU)."""
    if a.dtype == np.float32:
        na, nb = np.isnan(a), np.isnan(b)
        return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))
    if a.dtype == np.uint16:
        fa, fb = oracle.widen_bf16(a), oracle.widen_bf16(b)
        na, nb = np.isnan(fa), np.isnan(fb)
        return np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb])
    return np.array_equal(a, b)


class Case:
    """One optimizer run: a list of tensors (host inputs) and how to step it."""

    def __init__(self, opt, fmt, sizes, grad_bf16, steps, hp, seed=synth.SR_SEED,
                 g_std=1e-2, mask_scale=None, grad_override=None, clip=None):
        """clip=(max_norm, norm_type): before each step, the gradient norms of
        the list give a clipping coefficient that the step applies to g."""
        self.opt, self.fmt, self.sizes, self.steps, self.hp = opt, fmt, list(sizes), steps, dict(hp)
        self.clip = clip
        self.grad_bf16 = grad_bf16 if isinstance(grad_bf16, (list, tuple)) else [grad_bf16] * len(self.sizes)
        self.seed = seed
        self.g_std = g_std
        self.mask_scale = mask_scale
        self.grad_override = grad_override
        self.qs = synth.codebook_signed()
        self.qu = synth.codebook_unsigned()
        self.p0 = [synth.params(n, k) for k, n in enumerate(self.sizes)]

    def grad(self, t, k):
        if self.grad_override is not None:
            g = self.grad_override(t, k, self.sizes[k])
            if g is not None:
                return g
        std = synth.decaying_std(t, self.steps) if self.g_std == "decay" else self.g_std
        return synth.grads(self.sizes[k], t, k, std=std, bf16=self.grad_bf16[k],
                           mask_scale=self.mask_scale)

    # -- oracle ------------------------------------------------------------
    def run_oracle(self, steps=None, start=None):
        steps = self.steps if steps is None else steps
        ps = [p.copy() for p in self.p0] if start is None else [p.copy() for p in start[0]]
        st = ([oracle.state_zeros(self.fmt, n, self.opt, self.qs, self.qu) for n in self.sizes]
              if start is None else [{k: v.copy() for k, v in s.items()} for s in start[1]])
        t0 = 0 if start is None else start[2]
        norms = []
        self.oracle_coefs = []
        for t in range(t0 + 1, t0 + steps + 1):
            extra = {}
            if self.clip is not None:
                (s2, mx), _ = oracle.grad_norm_list([self.grad(t, k) for k in range(len(self.sizes))])
                coef = oracle.clip_coef(np.sqrt(s2) if self.clip[1] == 2 else mx, self.clip[0])
                self.oracle_coefs.append(coef)
                extra = {"grad_scale": coef}
            for k, n in enumerate(self.sizes):
                g = self.grad(t, k)
                hp = oracle.make_hp(step=t, seed=self.seed, tensor_index=k, **self.hp, **extra)
                scale = 1.0
                if self.hp.get("max_unorm", 0.0) > 0:
                    u2, p2 = oracle.unorm(self.opt, self.fmt, hp, ps[k], g, qs=self.qs, qu=self.qu, **st[k])
                    norms.append((t, k, u2, p2))
                    scale = oracle.unorm_scale(self.hp["max_unorm"], u2, p2)
                oracle.step(self.opt, self.fmt, hp, ps[k], g, qs=self.qs, qu=self.qu, scale=scale, **st[k])
        return ps, st, norms

    # -- GPU ---------------------------------------------------------------
    def alloc_gpu(self, start=None):
        import optimizer_step_amd as osa
        T = torch()
        dev = []
        for k, n in enumerate(self.sizes):
            p = self.p0[k] if start is None else start[0][k]
            d = {"p": to_dev(p.copy()),
                 "g": T.zeros(n, dtype=T.bfloat16 if self.grad_bf16[k] else T.float32, device="cuda")}
            if start is None:
                d.update(osa.state_buffers(self.fmt, n, self.opt, qmap_signed=self.qs, qmap_unsigned=self.qu))
            else:
                d.update({key: to_dev(v.copy()) for key, v in start[1][k].items()})
            dev.append(d)
        return dev

    def run_gpu(self, steps=None, dev=None, t0=0, stream=None):
        import optimizer_step_amd as osa
        T = torch()
        steps = self.steps if steps is None else steps
        if dev is None:
            dev = self.alloc_gpu()
        tl = osa.TensorList(dev)
        fn = osa.opt_step_adamw if self.opt == "adamw" else osa.opt_step_ademamix
        norms = []
        self.gpu_coefs = []
        for t in range(t0 + 1, t0 + steps + 1):
            for k in range(len(self.sizes)):
                g = self.grad(t, k)
                dev[k]["g"].copy_(to_dev(g))
            coef = None
            if self.clip is not None:
                gn = T.empty(2 + 2 * len(self.sizes), dtype=T.float64, device="cuda")
                coef = T.empty(1, dtype=T.float32, device="cuda")
                osa.opt_grad_norm([d["g"] for d in dev], gn, self.clip[0], self.clip[1], coef, stream=stream)
                self.gpu_coefs.append((gn, coef))    # alive until the synchronize below
            hp = osa.hparams(step=t, seed=self.seed, qmap_signed=self.qs, qmap_unsigned=self.qu,
                             grad_scale=coef, **self.hp)
            unorm = None
            if self.hp.get("max_unorm", 0.0) > 0:
                unorm = T.empty(2 * len(self.sizes), dtype=T.float64, device="cuda")
                osa.opt_precondition_unorm(self.opt, tl, self.fmt, hp, unorm, stream=stream)
                norms.append(unorm.cpu().numpy().copy())
            fn(tl, self.fmt, hp, unorm, stream=stream)
        T.cuda.synchronize()
        self.gpu_coefs = [float(c.cpu().numpy()[0]) for _, c in self.gpu_coefs]
        return dev, norms

    @staticmethod
    def host(dev):
        return [{k: to_host(v) for k, v in d.items() if k != "g"} for d in dev]


STATE_KEYS = {"adamw": ("s1", "s2"), "ademamix": ("s1", "s2", "s3")}
BLOCKED_FMTS = ("q8", "fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr")


def compare(case, dev, ps, st, steps=None):
    """Assert the bars: fp32 p within 1e-6 relative (the direction of an fp32
    parameter uses the hardware reciprocal and square root); every stored
    state word bit-exact -- fp32 and BF16 moments (both sides form them in the
    same binary32 order and round them by the same rules), stochastic-rounding
    bits, codes and absmax.  Returns the fraction of p words that are
    bit-identical (a diagnostic; the bar is the tolerance)."""
    got = Case.host(dev)
    same = total = 0
    for k in range(len(case.sizes)):
        gp, op = got[k]["p"], ps[k]
        assert fp32_close(gp, op), f"tensor {k}: p outside 1e-6 relative"
        na = np.isnan(op)
        same += int(np.sum(gp[~na].view(np.uint32) == op[~na].view(np.uint32))) + int(na.sum())
        total += op.size
        for key in STATE_KEYS[case.opt]:
            g, o = got[k][key], st[k][key]
            if case.fmt in ("f32", "bf16_rn", "bf16_sr"):
                assert nan_equal_bits(g, o), f"tensor {k} {key}: state words differ"
            else:
                assert np.array_equal(g, o), f"tensor {k} {key}: codes differ"
        if case.fmt in BLOCKED_FMTS:
            for key in ("absmax1", "absmax2", "absmax3")[:len(STATE_KEYS[case.opt])]:
                a = key.replace("absmax", "a")
                assert nan_equal_bits(got[k][key], st[k][a]), f"tensor {k} {key}: absmax differs"
    return same / max(total, 1)


def states_bit_identical(case, dev, st):
    """Every stored state word equals the oracle's.  The moments never depend
    on p, and both sides form them in the same binary32 order and round them
    on store by the same rules, so with identical inputs this holds for every
    format (only the direction u, which feeds p alone, may differ by a few
    ulp)."""
    got = Case.host(dev)
    for k in range(len(case.sizes)):
        for key in STATE_KEYS[case.opt]:
            assert nan_equal_bits(got[k][key], st[k][key]), f"tensor {k} {key}: state words differ"

"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the optimizer's arithmetic: it only draws parameters
and gradients with the distributions the workloads call for, builds the two
256-entry codebooks that the 8-bit state format takes as inputs, and describes
the workloads (shapes, hyper-parameters, step counts).  Both the CPU oracle and
the HIP path receive exactly what it produces.

Host draws use numpy's PCG64 (``numpy.random.default_rng``); large inputs that
only live on the GPU are drawn with a seeded ``torch.Generator`` on the device
and the oracle is given the sampled elements it checks.
"""
import numpy as np

PARAM_SEED = 1
GRAD_SEED = 2
MASK_SEED = 3
SR_SEED = 0x9E3779B97F4A7C15


# --------------------------------------------------------------------------
# codebooks (inputs of the 8-bit state format)

def _dynamic_exponent(signed):
    """A 256-entry dynamic-exponent codebook.

    The pages name the format ("signed dynamic-exponent" for m, an unsigned one
    for v) but print no values.  Reading: a decade exponent E followed by a
    linear fraction, value 10^-E * (0.1 + 0.9*j/2^(B-E)), j = 1..2^(B-E);
    B = 7 for the unsigned table (E = 0..7, 255 values, plus 0) and B = 6 for
    the signed one (E = 0..6, 127 values of each sign, plus 0 and +1e-7).
    Built in binary64, rounded to fp32 and sorted; the code is the index.
    """
    B = 6 if signed else 7
    vals = [0.0]
    for E in range(B + 1):
        for j in range(1, 2 ** (B - E) + 1):
            x = 10.0 ** (-E) * (0.1 + 0.9 * j / 2 ** (B - E))
            vals.append(x)
            if signed:
                vals.append(-x)
    if signed:
        vals.append(1e-7)
    t = np.array(sorted(np.float32(v) for v in vals), dtype=np.float32)
    assert t.size == 256 and np.all(np.diff(t.astype(np.float64)) > 0)
    return t


def codebook_signed():
    """Signed table (for m and AdEMAMix's m2): code 0 = -1, 127 = 0, 255 = +1."""
    return _dynamic_exponent(True)


def codebook_unsigned():
    """Unsigned table (for v): code 0 = 0, 255 = 1."""
    return _dynamic_exponent(False)


# --------------------------------------------------------------------------
# host draws

def _rng(seed, *stream):
    return np.random.default_rng([int(seed), *[int(s) for s in stream]])


def normal(seed, n, std, *stream):
    """n float32 draws from N(0, std) (std is a standard deviation)."""
    return (_rng(seed, *stream).standard_normal(n) * std).astype(np.float32)


def bf16_words(x):
    """float32 -> BF16 words (uint16) with the library cast torch provides."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def params(n, k=0, std=0.02):
    return normal(PARAM_SEED, n, std, k)


def grads(n, t, k=0, std=1e-2, bf16=False, mask_scale=None):
    """Gradient of tensor k at step t.  mask_scale=(frac, factor) multiplies a
    fixed random subset of coordinates (the same subset every step) by factor,
    in fp32 before any rounding to BF16."""
    g = normal(GRAD_SEED, n, std, k, t)
    if mask_scale is not None:
        frac, factor = mask_scale
        mask = _rng(MASK_SEED, k).random(n) < frac
        g = np.where(mask, g * np.float32(factor), g).astype(np.float32)
    return bf16_words(g) if bf16 else g


def grid_grads(n, t, k=0, bf16=False):
    """Gradients on a coarse grid, so that every square and every partial sum
    of squares is exact in binary64 whatever the summation order: integers
    |i| <= 255 times 2^-10 for BF16 (8 significant bits), |i| <= 4095 times
    2^-12 for float32; about N(0, 0.04) before clipping to the grid."""
    z = _rng(GRAD_SEED, k, t, 7).standard_normal(n)
    if bf16:
        i = np.clip(np.rint(z * 40.0), -255, 255)
        return bf16_words((i * 2.0**-10).astype(np.float32))
    i = np.clip(np.rint(z * 160.0), -4095, 4095)
    return (i * 2.0**-12).astype(np.float32)


# --------------------------------------------------------------------------
# device draws (large workloads)

def device_normal_(tensor, seed, std, *stream):
    """Fill a CUDA float tensor in place with N(0, std) from a seeded generator."""
    import torch
    gen = torch.Generator(device=tensor.device)
    s = int(seed)
    for x in stream:
        s = (s * 1000003 + int(x) + 1) % (2**63 - 1)
    gen.manual_seed(s)
    if tensor.dtype == torch.float32:
        tensor.normal_(0.0, std, generator=gen)
    else:
        tmp = torch.empty(tensor.shape, dtype=torch.float32, device=tensor.device)
        tmp.normal_(0.0, std, generator=gen)
        tensor.copy_(tmp)
    return tensor


def device_grads(n, device, std, t, k=0, bf16=False, mask_scale=None):
    """Gradient of tensor k at step t on the device: N(0, std) in fp32, a fixed
    random subset scaled in fp32 if mask_scale=(frac, factor), then rounded to
    BF16 by torch's cast if bf16."""
    import torch
    g = torch.empty(n, dtype=torch.float32, device=device)
    device_normal_(g, GRAD_SEED, std, k, t)
    if mask_scale is not None:
        frac, factor = mask_scale
        # elementwise select (the same fp32 product as indexing in place);
        # boolean-mask indexing fails past 2^32 elements
        g = torch.where(device_mask(n, device, frac, k), g * factor, g)
    return g.to(torch.bfloat16) if bf16 else g


def device_mask(n, device, frac, k=0):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(MASK_SEED * 1000003 + k)
    return torch.rand(n, generator=gen, device=device) < frac


# --------------------------------------------------------------------------
# workloads

def llama7b_shapes():
    """(name, numel) of the Llama-7B-shaped list: embed [32000x4096], 32 layers
    of q,k,v,o [4096x4096], gate,up,down [4096x11008], attn_norm,mlp_norm [4096],
    then lm_head [32000x4096]; 290 tensors, 6,738,411,520 elements."""
    out = [("embed", 32000 * 4096)]
    for l in range(32):
        for nm in ("q", "k", "v", "o"):
            out.append((f"l{l}.{nm}", 4096 * 4096))
        for nm in ("gate", "up", "down"):
            out.append((f"l{l}.{nm}", 4096 * 11008))
        out.append((f"l{l}.attn_norm", 4096))
        out.append((f"l{l}.mlp_norm", 4096))
    out.append(("lm_head", 32000 * 4096))
    return out


def decaying_std(t, steps=200, start=1e-2, end=1e-4):
    """Log-linear gradient-scale schedule from start (t=1) to end (t=steps)."""
    return start * (end / start) ** ((t - 1) / (steps - 1))


WORKLOADS = {
    # one flat fp32 tensor with a ragged tail (2^16 + 1 elements)
    "adamw_f32_small": dict(opt="adamw", fmt="f32", sizes=[65537], grad_bf16=False,
                            p_std=0.02, g_std=1e-2, steps=10,
                            hp=dict(lr=0.1, weight_decay=0.1, beta1=0.9, beta2=0.999, eps=1e-8)),
    # Llama-7B-shaped list, fp32 master weights, bf16 grads, fp32 m/v
    "adamw_f32_llama7b": dict(opt="adamw", fmt="f32", sizes=[n for _, n in llama7b_shapes()],
                              grad_bf16=True, p_std=0.02, g_std=1e-3, steps=5,
                              hp=dict(lr=3e-4, weight_decay=0.1, beta1=0.9, beta2=0.999, eps=1e-8)),
    # one 2^30-element buffer, 8-bit blockwise m/v, 10% of grads x100
    "adamw_q8_1g": dict(opt="adamw", fmt="q8", sizes=[2**30], grad_bf16=True,
                        p_std=0.02, g_std=1e-3, mask_scale=(0.1, 100.0), steps=5,
                        hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8)),
    # AdEMAMix, fp32 m1/m2/v, 2^28 elements
    "ademamix_f32_268m": dict(opt="ademamix", fmt="f32", sizes=[2**28], grad_bf16=False,
                              p_std=0.02, g_std=1e-2, steps=10,
                              hp=dict(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.999,
                                      beta3=0.9999, alpha=5.0, eps=1e-8)),
    # AdamW with the update-norm bound, 2^28 elements
    "adamw_f32_unorm_268m": dict(opt="adamw", fmt="f32", sizes=[2**28], grad_bf16=False,
                                 p_std=0.02, g_std=1e-2, steps=10,
                                 hp=dict(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.999,
                                         eps=1e-8, max_unorm=1.0)),
    # BF16 m/v, nearest or stochastic rounding, decaying gradient scale, 2^30 elements
    "adamw_bf16_1g": dict(opt="adamw", fmt="bf16_rn", sizes=[2**30], grad_bf16=True,
                          p_std=0.02, g_std="decay", steps=200,
                          hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8)),
    "adamw_bf16_sr_1g": dict(opt="adamw", fmt="bf16_sr", sizes=[2**30], grad_bf16=True,
                             p_std=0.02, g_std="decay", steps=200,
                             hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8)),
    # FP8 / FP4 block-scaled m/v, nearest or stochastic rounding, 2^30 elements
    **{f"adamw_{f}_1g": dict(opt="adamw", fmt=f, sizes=[2**30], grad_bf16=True, p_std=0.02, g_std=1e-3,
                             mask_scale=(0.1, 100.0), steps=5,
                             hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8))
       for f in ("fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr")},
    # one-state optimizers, bf16 gradients, fp32 state, 2^30 elements
    **{f"{o}_f32_1g": dict(opt=o, fmt="f32", sizes=[2**30], grad_bf16=True, p_std=0.02, g_std=1e-3, steps=5,
                          hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.99, eps=1e-8))
       for o in ("momentum", "lion")},
    # BF16 parameters (a mixed-precision model without fp32 master weights):
    # stored with stochastic rounding next to BF16-SR states, or to nearest
    # next to fp32 states; the direction is then formed exactly
    "adamw_bf16p_bf16_sr_1g": dict(opt="adamw", fmt="bf16_sr", sizes=[2**30], grad_bf16=True, p_dtype="bf16",
                                   p_sr=True, p_std=0.02, g_std=1e-3, steps=5,
                                   hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8)),
    "adamw_bf16p_f32_1g": dict(opt="adamw", fmt="f32", sizes=[2**30], grad_bf16=True, p_dtype="bf16",
                               p_std=0.02, g_std=1e-3, steps=5,
                               hp=dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8)),
    # the standalone FP32 -> BF16 stochastic-rounding cast of 2^30 values
    "cast_bf16_sr_1g": dict(opt="cast", fmt="bf16_sr", sizes=[2**30], grad_bf16=False, p_std=1.0, g_std=1e-3,
                            steps=5, hp=dict()),
    # gradient 2-norm of the Llama-7B-shaped bf16 gradient list alone
    "gradnorm_bf16_llama7b": dict(opt="adamw", fmt="f32", sizes=[n for _, n in llama7b_shapes()],
                                  grad_bf16=True, p_std=0.02, g_std=1e-3, steps=5, norm_only=True,
                                  clip=(1.0, 2), hp=dict()),
    # the headline step preceded by the fused gradient norm, the clipping
    # coefficient handed to the step in device memory
    "adamw_f32_clip_llama7b": dict(opt="adamw", fmt="f32", sizes=[n for _, n in llama7b_shapes()],
                                   grad_bf16=True, p_std=0.02, g_std=1e-3, steps=5, clip=(1.0, 2),
                                   hp=dict(lr=3e-4, weight_decay=0.1, beta1=0.9, beta2=0.999, eps=1e-8)),
}


def bytes_per_element(opt, fmt, grad_bf16, p_bytes=4):
    """Algorithmic HBM bytes one step must move per element: read p, g and the
    states, write p and the states (8-bit: codes plus one fp32 absmax per 256
    elements per state, read and written; FP8 the same with E4M3 codes; FP4
    half a byte per element per state plus the absmax)."""
    nst = 3 if opt == "ademamix" else (2 if opt == "adamw" else 1)
    g = 2 if grad_bf16 else 4
    if fmt == "f32":
        s = 4
    elif fmt.startswith("bf16"):
        s = 2
    elif fmt.startswith("fp4"):
        s = 0.5 + 4 / 256
    else:
        s = 1 + 4 / 256
    return p_bytes * 2 + g + nst * s * 2


def total_elements(sizes):
    return int(sum(sizes))


def human(n):
    for u in ("", "K", "M", "G"):
        if abs(n) < 1000:
            return f"{n:.3g}{u}"
        n /= 1000
    return f"{n:.3g}T"


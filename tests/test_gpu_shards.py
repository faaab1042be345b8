"""A tensor stepped as slices (one rank's shard each, as a ZeRO-style sharded
optimizer holds them) gives the same bits as the whole tensor: each slice
carries its first element's index within the tensor (index_base) and the
tensor's stochastic-rounding number (sr_tensor), so every element draws the
same Philox word, and slices start on 256-element boundaries, so the blockwise
formats' blocks and absmax are the tensor's own.

Checked on every state format with stochastic or blockwise rounding, AdamW and
AdEMAMix, a 16-bit parameter stored stochastically, and a one-state optimizer,
over three steps; the whole tensor sits at a different list position than its
slices, so the stream key must come from sr_tensor.  The whole-tensor run is
itself checked against the oracle elsewhere (the parity tests)."""
import numpy as np
import pytest

import synth
from tests.gpu_common import to_dev

pytestmark = pytest.mark.gpu

N = 300_001
CUTS = [0, 65536 + 3 * 256, 200_192, N]      # slice boundaries, multiples of 256
# element-wise formats: slices on multiples of 4 (fp32 arrays) or 8 (16-bit
# arrays: every pointer must be 16-byte aligned) that are not multiples of 256
CUTS4 = [0, 1028, 70_004, 200_196, N]
CUTS8 = [0, 1032, 70_008, 200_200, N]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)
    yield


def _fresh(opt, fmt, n, p16=None):
    import torch
    import optimizer_step_amd as osa
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    p = to_dev(synth.params(n, 3, std=0.5 if p16 else 0.02))
    if p16 == "bf16":
        p = p.to(torch.bfloat16)
    elif p16 == "f16":
        p = p.to(torch.float16)
    st = osa.state_buffers(fmt, n, opt, qmap_signed=qs, qmap_unsigned=qu)
    return p, st, qs, qu


def _slice(d, a, b, fmt):
    out = {}
    for key, buf in d.items():
        if key.startswith("absmax"):
            out[key] = buf[a // 256:(b + 255) // 256]
        elif fmt.startswith("fp4") and key.startswith("s"):
            out[key] = buf[a // 2:(b + 1) // 2]
        else:
            out[key] = buf[a:b]
    return out


def _grads(t, zeros, cuts=CUTS, f32=False):
    g = synth.grads(N, t, 5, std=1e-2)
    if zeros:
        # exact zeros of both signs on both sides of every cut (v = 0 at step
        # 1); before each element's direction was chosen on its own, such an
        # element sent its whole wave to the exact recipe, and the waves of a
        # slice that starts off a 256-element boundary group other elements
        for c in cuts[1:-1]:
            g[c - 9:c + 7:3] = 0.0
            g[c - 2:c + 2:2] = -0.0
        g[::997] = 0.0
    return to_dev(g) if f32 else to_dev(synth.bf16_words(g))


def _run(opt, fmt, p16=None, steps=3, cuts=CUTS, zeros=False):
    import torch
    import optimizer_step_amd as osa
    one_state = opt in osa.ONE_STATE
    step = (lambda tl, h: osa.opt_step_1state(opt, tl, fmt, h)) if one_state else \
           (lambda tl, h: (osa.opt_step_adamw if opt == "adamw" else osa.opt_step_ademamix)(tl, fmt, h))
    other_p, other_st, qs, qu = _fresh(opt, fmt, 1000)
    other_g = to_dev(synth.grads(1000, 1, 9))
    # whole tensor at list position 1
    p_w, st_w, _, _ = _fresh(opt, fmt, N, p16)
    p_s, st_s = p_w.clone(), {k: v.clone() for k, v in st_w.items()}
    other = {"p": other_p, "g": other_g, **other_st}
    results = []
    for sharded, p, st in ((False, p_w, st_w), (True, p_s, st_s)):
        for t in range(1, steps + 1):
            g = _grads(t, zeros, cuts, f32=fmt == "f32" and cuts is CUTS4)
            if sharded:
                tl = [other]
                for a, b in zip(cuts[:-1], cuts[1:]):
                    tl.append({"p": p[a:b], "g": g[a:b], **_slice(st, a, b, fmt), "index_base": a, "sr_tensor": 1})
            else:
                tl = [other, {"p": p, "g": g, **st}]
            h = osa.hparams(step=t, lr=1e-3, weight_decay=0.01, seed=synth.SR_SEED, qmap_signed=qs,
                            qmap_unsigned=qu, p_rounding=1 if p16 else 0)
            step(osa.TensorList(tl), h)
        torch.cuda.synchronize()
        results.append({"p": p.view(torch.uint8).cpu().numpy(),
                        **{k: v.view(torch.uint8).cpu().numpy() for k, v in st.items()}})
    whole, shards = results
    for key in whole:
        assert np.array_equal(whole[key], shards[key]), (opt, fmt, p16, key)


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("fmt", ["f32", "bf16_sr", "q8", "fp8_sr", "fp4_sr", "fp4_rn"])
def test_slices_step_as_the_whole_tensor(opt, fmt):
    _run(opt, fmt)


@pytest.mark.parametrize("opt", ["adamw", "ademamix"])
@pytest.mark.parametrize("fmt", ["f32", "bf16_rn", "bf16_sr"])
def test_unaligned_slices_with_zero_gradients(opt, fmt):
    """Element-wise formats accept slices on any 16-byte-aligned element (a
    multiple of 4 for fp32 arrays, here with fp32 gradients; of 8 with BF16
    words); elements whose gradient is exactly zero sit on both sides of each
    cut, and every element's result depends on its own inputs only."""
    _run(opt, fmt, cuts=CUTS4 if fmt == "f32" else CUTS8, zeros=True)


@pytest.mark.parametrize("p16", ["bf16", "f16"])
def test_slices_with_stochastic_16bit_parameters(p16):
    _run("adamw", "bf16_sr", p16=p16)


@pytest.mark.parametrize("opt", ["momentum", "lion"])
def test_slices_one_state(opt):
    _run(opt, "bf16_sr")


def test_shifted_base_changes_the_stream():
    """Negative control: the same slices without their index base draw other
    words, so the stochastic-rounding bits differ."""
    import torch
    import optimizer_step_amd as osa
    p, st, qs, qu = _fresh("adamw", "bf16_sr", N)
    p2, st2 = p.clone(), {k: v.clone() for k, v in st.items()}
    g = _grads(1, False)
    a, b = CUTS[1], CUTS[2]
    h = osa.hparams(step=1, seed=synth.SR_SEED)
    osa.opt_step_adamw(osa.TensorList([{"p": p[a:b], "g": g[a:b], **_slice(st, a, b, "bf16_sr"),
                                        "index_base": a, "sr_tensor": 0}]), "bf16_sr", h)
    osa.opt_step_adamw(osa.TensorList([{"p": p2[a:b], "g": g[a:b], **_slice(st2, a, b, "bf16_sr"),
                                        "sr_tensor": 0}]), "bf16_sr", h)
    torch.cuda.synchronize()
    assert not torch.equal(st["s2"][a:b], st2["s2"][a:b])

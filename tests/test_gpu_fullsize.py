"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Every output the oracle can compute one element (or one
8-bit block) at a time is checked on a seeded sample that always includes the
first and last elements of every tensor; the update-norm workload, whose
scale couples all elements, is replayed in full by the oracle.  Inputs are
drawn on the device from seeded generators and the oracle is handed exactly
the sampled input values (never a value the HIP path produced)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import FP32_REL, bf16_ulps, fp32_close, nan_equal_bits, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import optimizer_step_amd as osa
    assert torch.cuda.is_available()
    osa.lib()
    osa.opt_debug_set_launch(32768, 0)      # the benchmark's geometry
    yield
    torch.cuda.empty_cache()


def _sample_idx(n, count, seed):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(min(4, n)), np.arange(max(0, n - 5), n),
                          rng.integers(0, n, count)])
    return np.unique(idx)


def _flat_states(fmt, total, opt, qs, qu):
    import optimizer_step_amd as osa
    return osa.state_buffers(fmt, total, opt, qmap_signed=qs, qmap_unsigned=qu)


def _views(P, G, states, sizes, fmt):
    tensors, off = [], 0
    for n in sizes:
        d = {"p": P[off:off + n], "g": G[off:off + n]}
        for key, buf in states.items():
            d[key] = buf[off // 256:(off + n + 255) // 256] if key.startswith("absmax") else buf[off:off + n]
        tensors.append(d)
        off += n
    return tensors


def _gather(t, idx):
    import torch
    return to_host(t[torch.from_numpy(idx).cuda()])


def test_llama7b_list_adamw_fp32_states():
    """290 tensors, 6,738,411,520 elements, bf16 gradients, 5 steps, one launch
    per step; 72 sampled elements per tensor against the oracle."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["adamw_f32_llama7b"]
    sizes, hp, steps = w["sizes"], w["hp"], w["steps"]
    total = sum(sizes)
    offs = np.cumsum([0] + sizes[:-1])
    print(f"llama7b list: {len(sizes)} tensors, {total} elements", flush=True)
    P = torch.empty(total, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = _flat_states("f32", total, "adamw", None, None)
    samples = [_sample_idx(n, 64, 100 + k) + offs[k] for k, n in enumerate(sizes)]
    allidx = np.concatenate(samples)
    p0 = _gather(P, allidx)
    g_hist = []
    G = None
    tl = None
    for t in range(1, steps + 1):
        del G
        G = synth.device_grads(total, "cuda", w["g_std"], t, bf16=True)
        tensors = _views(P, G, st, sizes, "f32")
        tl = osa.TensorList(tensors)
        osa.opt_step_adamw(tl, "f32", osa.hparams(step=t, **hp))
        g_hist.append(_gather(G, allidx))
    torch.cuda.synchronize()
    gp, gm, gv = _gather(P, allidx), _gather(st["s1"], allidx), _gather(st["s2"], allidx)
    # the oracle on each tensor's sample (element-wise, so the sample is exact)
    pos = 0
    for k, idx in enumerate(samples):
        m = idx.size
        p = p0[pos:pos + m].copy()
        s = oracle.state_zeros("f32", m)
        for t in range(1, steps + 1):
            oracle.step("adamw", "f32", oracle.make_hp(step=t, tensor_index=k, **hp), p,
                        g_hist[t - 1][pos:pos + m], **s)
        assert fp32_close(gp[pos:pos + m], p), f"tensor {k}: p"
        assert nan_equal_bits(gm[pos:pos + m], s["s1"]), f"tensor {k}: m"
        assert nan_equal_bits(gv[pos:pos + m], s["s2"]), f"tensor {k}: v"
        pos += m
    del P, G, st, tensors, tl
    torch.cuda.empty_cache()


def test_q8_one_billion_elements():
    """2^30 elements, 8-bit blockwise m and v, 10% of gradients x100, 5 steps;
    64 sampled blocks (first and last included): codes and absmax bit-exact,
    p within the fp32 bar."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["adamw_q8_1g"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = _flat_states("q8", n, "adamw", qs, qu)
    nb = n // 256
    blocks = np.unique(np.concatenate([[0, 1, nb - 1], np.random.default_rng(9).integers(0, nb, 61)]))
    idx = (blocks[:, None] * 256 + np.arange(256)[None, :]).reshape(-1)
    p0 = _gather(P, idx)
    g_hist = []
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", w["g_std"], t, bf16=True, mask_scale=w["mask_scale"])
        tl = osa.TensorList(_views(P, G, st, [n], "q8"))
        osa.opt_step_adamw(tl, "q8", osa.hparams(step=t, qmap_signed=qs, qmap_unsigned=qu, **hp))
        g_hist.append(_gather(G, idx))
        del G
    torch.cuda.synchronize()
    p = p0.copy()
    s = oracle.state_zeros("q8", idx.size, "adamw", qs, qu)
    for t in range(1, steps + 1):
        oracle.step("adamw", "q8", oracle.make_hp(step=t, **hp), p, g_hist[t - 1], qs=qs, qu=qu, **s)
    assert fp32_close(_gather(P, idx), p)
    assert np.array_equal(_gather(st["s1"], idx), s["s1"])
    assert np.array_equal(_gather(st["s2"], idx), s["s2"])
    assert nan_equal_bits(_gather(st["absmax1"], blocks), s["a1"])
    assert nan_equal_bits(_gather(st["absmax2"], blocks), s["a2"])
    del P, st
    torch.cuda.empty_cache()


def test_ademamix_268m():
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["ademamix_f32_268m"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = _flat_states("f32", n, "ademamix", None, None)
    idx = _sample_idx(n, 4096, 12)
    p0 = _gather(P, idx)
    g_hist = []
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", w["g_std"], t)
        osa.opt_step_ademamix(osa.TensorList(_views(P, G, st, [n], "f32")), "f32", osa.hparams(step=t, **hp))
        g_hist.append(_gather(G, idx))
        del G
    torch.cuda.synchronize()
    p = p0.copy()
    s = oracle.state_zeros("f32", idx.size, "ademamix")
    for t in range(1, steps + 1):
        oracle.step("ademamix", "f32", oracle.make_hp(step=t, **hp), p, g_hist[t - 1], **s)
    assert fp32_close(_gather(P, idx), p)
    for key in ("s1", "s2", "s3"):
        assert nan_equal_bits(_gather(st[key], idx), s[key]), key
    del P, st
    torch.cuda.empty_cache()


def test_update_norm_268m_full_replay():
    """AdamW with max_unorm = 1 on 2^28 elements for 10 steps.  The scale ties
    every element to the norms, so the oracle replays the whole tensor.  At
    every step the pre-pass norms are within 1e-12 relative of the oracle's on
    the same inputs (the GPU's state before the step; the two trajectories of
    p part by a few ulp of lr*|u| per step, since the kernel forms the
    direction with the hardware reciprocal and square root); p, m and v end
    within the fp32 bar of the oracle's own trajectory; a repeated pre-pass
    gives identical bits."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["adamw_f32_unorm_268m"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = _flat_states("f32", n, "adamw", None, None)
    p = to_host(P).copy()
    s = oracle.state_zeros("f32", n)
    unorm = torch.empty(2, dtype=torch.float64, device="cuda")
    again = torch.empty(2, dtype=torch.float64, device="cuda")
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", w["g_std"], t)
        tl = osa.TensorList(_views(P, G, st, [n], "f32"))
        h = osa.hparams(step=t, **hp)
        torch.cuda.synchronize()
        p_in = to_host(P).copy()
        s_in = {k: to_host(st[k]).copy() for k in ("s1", "s2")}
        osa.opt_precondition_unorm("adamw", tl, "f32", h, unorm)
        osa.opt_precondition_unorm("adamw", tl, "f32", h, again)
        osa.opt_step_adamw(tl, "f32", h, unorm)
        g = to_host(G)
        hpo = oracle.make_hp(step=t, **hp)
        gu = unorm.cpu().numpy()
        assert np.array_equal(gu.view(np.uint64), again.cpu().numpy().view(np.uint64)), t
        u2_in, p2_in = oracle.unorm("adamw", "f32", hpo, p_in, g, **s_in)
        assert abs(gu[0] - u2_in) <= 1e-12 * u2_in and abs(gu[1] - p2_in) <= 1e-12 * p2_in, (t, gu, u2_in, p2_in)
        del p_in, s_in
        u2, p2 = oracle.unorm("adamw", "f32", hpo, p, g, **s)
        scale = oracle.unorm_scale(hp["max_unorm"], u2, p2)
        if t == 1:
            assert scale < 0.05
        oracle.step("adamw", "f32", hpo, p, g, scale=scale, **s)
        print(f"step {t}: scale {scale:.6f}", flush=True)
        del G
    torch.cuda.synchronize()
    assert fp32_close(to_host(P), p)
    assert nan_equal_bits(to_host(st["s1"]), s["s1"])     # the moments never see p or the scale
    assert nan_equal_bits(to_host(st["s2"]), s["s2"])
    del P, st
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16_rn", "bf16_sr"])
def test_bf16_states_one_billion_200_steps(fmt):
    """2^30 elements, BF16 m/v, gradient scale decaying 1e-2 -> 1e-4 over 200
    steps.  The oracle replays a contiguous run of 2^20 elements (the run
    keeps its element indices, so the stochastic-rounding stream is the
    tensor's) plus 2048 scattered elements: m, v bit-exact and p within the
    fp32 bar.  Per step, the stalled fraction of v (stored word unchanged) is
    taken over the whole tensor and over the run on the GPU, and over the run
    in the oracle; the two run fractions are equal, and the run estimates the
    tensor's.  Under RN with beta2 = 0.999 no stored v ever decreases."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["adamw_bf16_1g"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    R0, RN_ = 3 << 27, 1 << 20                       # the contiguous run
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = _flat_states(fmt, n, "adamw", None, None)
    idx = _sample_idx(n, 2048, 14)
    p0, p0_run = _gather(P, idx), to_host(P[R0:R0 + RN_]).copy()
    g_hist, g_run = [], []
    stalled, stalled_run = [], []
    v_prev = st["s2"].clone()
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", synth.decaying_std(t, steps), t, bf16=True)
        osa.opt_step_adamw(osa.TensorList(_views(P, G, st, [n], fmt)), fmt,
                           osa.hparams(step=t, seed=synth.SR_SEED, **hp))
        g_hist.append(_gather(G, idx))
        g_run.append(to_host(G[R0:R0 + RN_]).copy())
        v_new = st["s2"]
        same = v_new.view(torch.int16) == v_prev.view(torch.int16)
        stalled.append(float(same.float().mean()))
        stalled_run.append(float(same[R0:R0 + RN_].float().mean()))
        if fmt == "bf16_rn" and t > 1:
            assert bool((v_new.float() >= v_prev.float()).all()), f"v fell at step {t}"
        v_prev.copy_(v_new)
        del G
    torch.cuda.synchronize()
    # the oracle on the run, one call per step
    p_run = p0_run.copy()
    s_run = oracle.state_zeros(fmt, RN_)
    so_run = []
    for t in range(1, steps + 1):
        v_before = s_run["s2"].copy()
        oracle.step("adamw", fmt, oracle.make_hp(step=t, seed=synth.SR_SEED, index_base=R0, **hp), p_run,
                    g_run[t - 1], **s_run)
        so_run.append(float(np.mean(s_run["s2"] == v_before)))
    assert fp32_close(to_host(P[R0:R0 + RN_]), p_run)
    assert nan_equal_bits(to_host(st["s1"][R0:R0 + RN_]), s_run["s1"])
    assert nan_equal_bits(to_host(st["s2"][R0:R0 + RN_]), s_run["s2"])
    assert stalled_run == so_run
    # the scattered sample, each element at its own index
    p = p0.copy()
    s = oracle.state_zeros(fmt, idx.size)
    for t in range(1, steps + 1):
        hpo = oracle.make_hp(step=t, seed=synth.SR_SEED, **hp)
        for i, j in enumerate(idx):
            hpo.index_base = int(j)
            sl = slice(i, i + 1)
            sub = {k2: v2[sl] for k2, v2 in s.items()}
            oracle.step("adamw", fmt, hpo, p[sl], g_hist[t - 1][sl], **sub)
    assert fp32_close(_gather(P, idx), p)
    assert nan_equal_bits(_gather(st["s1"], idx), s["s1"]) and nan_equal_bits(_gather(st["s2"], idx), s["s2"])
    print(f"{fmt} stalled v fraction at steps 2,50,100,200: whole tensor "
          f"{stalled[1]:.4f} {stalled[49]:.4f} {stalled[99]:.4f} {stalled[199]:.4f}; "
          f"GPU on the 2^20 run {stalled_run[1]:.4f} {stalled_run[49]:.4f} {stalled_run[99]:.4f} "
          f"{stalled_run[199]:.4f}; oracle on the run {so_run[1]:.4f} {so_run[49]:.4f} {so_run[99]:.4f} "
          f"{so_run[199]:.4f}", flush=True)
    # 2^20 elements estimate the tensor's fraction to well within 0.5 pp
    for t in (1, 49, 99, 199):
        assert abs(stalled[t] - so_run[t]) < 0.005
    del P, st, v_prev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr"])
def test_fp8_fp4_one_billion_elements(fmt):
    """2^30 elements, FP8 / FP4 block-scaled m and v, 10% of gradients x100,
    5 steps; 32 sampled blocks (first and last included), each replayed by the
    oracle at its own element index (the stochastic-rounding stream is tied to
    it): codes and absmax bit-exact, p within the fp32 bar."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS[f"adamw_{fmt}_1g"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    fp4 = fmt.startswith("fp4")
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = osa.state_buffers(fmt, n, "adamw")
    nb = n // 256
    blocks = np.unique(np.concatenate([[0, nb - 1], np.random.default_rng(21).integers(0, nb, 30)]))
    idx = (blocks[:, None] * 256 + np.arange(256)[None, :]).reshape(-1)
    cidx = (blocks[:, None] * 128 + np.arange(128)[None, :]).reshape(-1) if fp4 else idx
    p0 = _gather(P, idx)
    g_hist = []
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", w["g_std"], t, bf16=True, mask_scale=w["mask_scale"])
        views = {"p": P, "g": G, **st}
        osa.opt_step_adamw(osa.TensorList([views]), fmt, osa.hparams(step=t, seed=synth.SR_SEED, **hp))
        g_hist.append(_gather(G, idx))
        del G
    torch.cuda.synchronize()
    gp = _gather(P, idx)
    gm, gv = _gather(st["s1"], cidx), _gather(st["s2"], cidx)
    ga1, ga2 = _gather(st["absmax1"], blocks), _gather(st["absmax2"], blocks)
    cb = 128 if fp4 else 256
    for i, b in enumerate(blocks):
        sl = slice(256 * i, 256 * (i + 1))
        p = p0[sl].copy()
        s = oracle.state_zeros(fmt, 256, "adamw")
        for t in range(1, steps + 1):
            h = oracle.make_hp(step=t, seed=synth.SR_SEED, index_base=int(b) * 256, **hp)
            oracle.step("adamw", fmt, h, p, g_hist[t - 1][sl], **s)
        assert fp32_close(gp[sl], p), (fmt, b)
        assert np.array_equal(gm[cb * i:cb * (i + 1)], s["s1"]), (fmt, b, "m")
        assert np.array_equal(gv[cb * i:cb * (i + 1)], s["s2"]), (fmt, b, "v")
        assert nan_equal_bits(ga1[i:i + 1], s["a1"]) and nan_equal_bits(ga2[i:i + 1], s["a2"]), (fmt, b)
    del P, st
    torch.cuda.empty_cache()


def test_gradient_norm_llama7b_list():
    """The bf16 gradient norm of the 290-tensor list in one call: four whole
    tensors (the two 131M-element matrices, a 16M-element one, a norm vector)
    against the oracle within the summation bound, maxima exact, the total
    equal to the sum of the per-tensor sums within the bound."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["gradnorm_bf16_llama7b"]
    sizes = w["sizes"]
    total = sum(sizes)
    offs = np.cumsum([0] + sizes[:-1])
    G = synth.device_grads(total, "cuda", w["g_std"], 1, bf16=True)
    grads = [G[o:o + n] for o, n in zip(offs, sizes)]
    out = torch.empty(2 + 2 * len(sizes), dtype=torch.float64, device="cuda")
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    osa.opt_grad_norm(grads, out, 1.0, 2, coef)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    U = 2.0 ** -53
    for k in (0, 1, 8, len(sizes) - 1):
        ps, pm = oracle.grad_norm(to_host(grads[k]))
        assert abs(o[2 + 2 * k] - ps) <= (sizes[k] - 1) * U * ps, (k, o[2 + 2 * k], ps)
        assert o[3 + 2 * k] == pm, k
    per = o[2::2]
    assert abs(o[0] - per.sum()) <= len(sizes) * U * o[0]
    assert o[1] == o[3::2].max()
    want = np.float32(oracle.clip_coef(np.sqrt(o[0]), 1.0)).view(np.int32)
    assert abs(int(coef.cpu().numpy().view(np.int32)[0]) - int(want)) <= 1
    del G, grads
    torch.cuda.empty_cache()


@pytest.mark.parametrize("opt", ["momentum", "lion"])
def test_one_state_one_billion_elements(opt):
    """2^30 elements, bf16 gradients, fp32 state, 5 steps; 4096 sampled
    elements (first and last included) against the oracle."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS[f"{opt}_f32_1g"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    S = torch.zeros(n, dtype=torch.float32, device="cuda")
    idx = _sample_idx(n, 4096, 33)
    p0 = _gather(P, idx)
    g_hist = []
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", w["g_std"], t, bf16=True)
        osa.opt_step_1state(opt, osa.TensorList([{"p": P, "g": G, "s1": S}]), "f32", osa.hparams(step=t, **hp))
        g_hist.append(_gather(G, idx))
        del G
    torch.cuda.synchronize()
    p, s1 = p0.copy(), np.zeros(idx.size, np.float32)
    for t in range(1, steps + 1):
        oracle.step_1state(opt, "f32", oracle.make_hp(step=t, **hp), p, g_hist[t - 1], s1)
    assert nan_equal_bits(_gather(P, idx), p)
    assert nan_equal_bits(_gather(S, idx), s1)
    del P, S
    torch.cuda.empty_cache()


def test_round_cast_one_billion_values():
    """The stochastic BF16 cast of 2^30 values in one launch: the first 2^24
    outputs bit-exact against the oracle, and every output one of the two
    BF16 neighbours of its input (the rounding never leaves its gap)."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["cast_bf16_sr_1g"]
    n = w["sizes"][0]
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(x, synth.PARAM_SEED, w["p_std"])
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    osa.opt_round_cast(x, out, True, synth.SR_SEED, 7)
    torch.cuda.synchronize()
    m = 1 << 24
    xh = to_host(x[:m])
    assert np.array_equal(to_host(out[:m]), oracle.round_cast(xh, oracle.P_BF16, True, synth.SR_SEED, 7))
    xb = x.view(torch.int32)
    lo = (xb & ~0xFFFF).view(torch.float32)                # toward zero: the gap's inner end
    wide = out.float()
    inner = wide == lo
    outer = (wide.view(torch.int32) == ((xb & ~0xFFFF) + 0x10000)) & ((xb & 0xFFFF) != 0)
    assert bool((inner | outer).all())
    del x, out, xb, lo, wide
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["f32", "q8"])
def test_one_tensor_past_2_to_32(fmt):
    """One tensor of 2^32 + 1027 elements (a ragged last block), bf16
    gradients, 2 steps: elements and whole 8-bit blocks around 2^31 and 2^32
    and in the tail against the oracle, so that no element offset, block
    index or stream index wraps at 32 bits."""
    import torch
    import optimizer_step_amd as osa
    n = (1 << 32) + 1027
    hp = dict(lr=1e-3, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8)
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    print(f"one tensor of {n} elements, {fmt} states", flush=True)
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, 0.02)
    st = _flat_states(fmt, n, "adamw", qs if fmt == "q8" else None, qu if fmt == "q8" else None)
    nb = (n + 255) // 256
    blocks = np.array([0, (1 << 23) - 1, 1 << 23, (1 << 24) - 1, nb - 2, nb - 1])   # 2^31 and 2^32 edges
    idx = np.concatenate([np.arange(256 * b, min(256 * (b + 1), n)) for b in blocks])
    p0 = _gather(P, idx)
    g_hist = []
    for t in (1, 2):
        G = synth.device_grads(n, "cuda", 1e-3, t, bf16=True)
        tl = osa.TensorList(_views(P, G, st, [n], fmt))
        osa.opt_step_adamw(tl, fmt, osa.hparams(step=t, qmap_signed=qs, qmap_unsigned=qu, **hp))
        g_hist.append(_gather(G, idx))
        del G, tl
    torch.cuda.synchronize()
    gp = _gather(P, idx)
    pos = 0
    for b in blocks:
        m = min(256 * (b + 1), n) - 256 * b
        sl = slice(pos, pos + m)
        p = p0[sl].copy()
        s = oracle.state_zeros(fmt, m, "adamw", qs, qu)
        for t in (1, 2):
            oracle.step("adamw", fmt, oracle.make_hp(step=t, index_base=256 * int(b), **hp), p, g_hist[t - 1][sl],
                        qs=qs, qu=qu, **s)
        assert fp32_close(gp[sl], p), (fmt, b)
        if fmt == "q8":
            assert np.array_equal(_gather(st["s1"], idx[sl]), s["s1"]), (fmt, b)
            assert np.array_equal(_gather(st["s2"], idx[sl]), s["s2"]), (fmt, b)
            assert nan_equal_bits(_gather(st["absmax1"], np.array([b])), s["a1"]), (fmt, b)
            assert nan_equal_bits(_gather(st["absmax2"], np.array([b])), s["a2"]), (fmt, b)
        else:
            assert nan_equal_bits(_gather(st["s1"], idx[sl]), s["s1"]), (fmt, b)
            assert nan_equal_bits(_gather(st["s2"], idx[sl]), s["s2"]), (fmt, b)
        pos += m
    del P, st
    torch.cuda.empty_cache()


def test_gradient_norm_one_tensor_past_2_to_32():
    """One bf16 gradient of 2^32 + 5 elements: 2^-10 everywhere but 1.0 in
    the last five, so the sum of squares is exactly 2^32 * 2^-20 + 5 = 4101
    and the maximum 1.0; a unit index that wrapped at 32 bits would drop or
    repeat the tail."""
    import torch
    import optimizer_step_amd as osa
    n = (1 << 32) + 5
    G = torch.full((n,), 2.0 ** -10, dtype=torch.bfloat16, device="cuda")
    G[1 << 32:] = 1.0
    out = torch.empty(4, dtype=torch.float64, device="cuda")
    osa.opt_grad_norm([G], out)
    o = out.cpu().numpy()
    assert o[0] == 4101.0 and o[2] == 4101.0, o
    assert o[1] == 1.0 and o[3] == 1.0, o
    del G
    torch.cuda.empty_cache()


def test_round_cast_past_2_to_34():
    """The stochastic BF16 cast of 2^34 + 4099 values: the element index
    enters the Philox counter as (j >> 2) low word and j >> 34, so values past
    2^34 use the second word; sampled outputs around 2^32, 2^34 and the tail
    against the oracle's rounding with the words formed from that layout."""
    import torch
    import optimizer_step_amd as osa
    n = (1 << 34) + 4099
    seed, offset = synth.SR_SEED, 0x0000_0005_0000_0009
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(x, synth.PARAM_SEED, 1.0)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    osa.opt_round_cast(x, out, True, seed, offset)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([np.arange(0, 8), (1 << 32) + np.arange(-8, 8), (1 << 34) + np.arange(-8, 8),
                                    np.arange(n - 13, n)]))
    xs, got = _gather(x, idx), _gather(out, idx)
    for j, xj, gj in zip(idx, xs, got):
        q = int(j) >> 2
        w = oracle.philox([q & 0xFFFFFFFF, q >> 32, offset & 0xFFFFFFFF, offset >> 32],
                          [seed & 0xFFFFFFFF, seed >> 32])
        assert int(gj) == oracle.bf16_sr(xj, int(w[int(j) & 3]) & 0xFFFF), j
    del x, out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# whole-buffer checks: the oracle replays every element of the workload from
# the same seeded inputs, in slices that host threads step in parallel (each
# oracle call is one C call that releases the interpreter lock; the blockwise
# formats and the element-wise step make slices independent)

def _pool():
    from concurrent.futures import ThreadPoolExecutor
    return ThreadPoolExecutor(max_workers=max(1, min(16, len(__import__("os").sched_getaffinity(0)))))


def test_q8_one_billion_every_block():
    """2^30 elements, 8-bit blockwise m and v, 10% of gradients x100, 5 steps,
    in the benchmark's launch configuration: all 4,194,304 blocks' codes and
    absmax bit-exact and every p within the fp32 bar, the oracle replaying all
    five steps over 2^24-element slices from the same seeded inputs."""
    import time
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["adamw_q8_1g"]
    n, hp, steps = w["sizes"][0], w["hp"], w["steps"]
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    P = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    p_host = to_host(P).copy()
    st = _flat_states("q8", n, "adamw", qs, qu)
    g_host = []
    for t in range(1, steps + 1):
        G = synth.device_grads(n, "cuda", w["g_std"], t, bf16=True, mask_scale=w["mask_scale"])
        tl = osa.TensorList(_views(P, G, st, [n], "q8"))
        osa.opt_step_adamw(tl, "q8", osa.hparams(step=t, qmap_signed=qs, qmap_unsigned=qu, **hp))
        g_host.append(to_host(G).copy())
        del G, tl
    torch.cuda.synchronize()
    got = {"p": to_host(P), "s1": to_host(st["s1"]), "s2": to_host(st["s2"]),
           "a1": to_host(st["absmax1"]), "a2": to_host(st["absmax2"])}
    del P, st
    torch.cuda.empty_cache()
    S = 1 << 24
    t0 = time.time()

    def check(lo):
        hi = min(n, lo + S)
        p = p_host[lo:hi].copy()
        s = oracle.state_zeros("q8", hi - lo, "adamw", qs, qu)
        for t in range(1, steps + 1):
            oracle.step("adamw", "q8", oracle.make_hp(step=t, index_base=lo, **hp), p, g_host[t - 1][lo:hi],
                        qs=qs, qu=qu, **s)
        b0, b1 = lo // 256, (hi + 255) // 256
        bad = {"s1": int(np.sum(got["s1"][lo:hi] != s["s1"])), "s2": int(np.sum(got["s2"][lo:hi] != s["s2"])),
               "a1": not nan_equal_bits(got["a1"][b0:b1], s["a1"]), "a2": not nan_equal_bits(got["a2"][b0:b1], s["a2"]),
               "p": not fp32_close(got["p"][lo:hi], p)}
        print(f"q8 slice {lo // S}: {bad} ({time.time() - t0:.0f} s)", flush=True)
        return lo, bad

    with _pool() as pool:
        results = list(pool.map(check, range(0, n, S)))
    failed = [(lo, b) for lo, b in results if any(b.values())]
    assert not failed, failed[:4]
    assert len(results) == n // S


def test_llama7b_whole_tensors_of_every_shape():
    """The 290-tensor list stepped 5 times in one launch per step; the oracle
    replays every element of one tensor of each shape (embed, an attention
    projection, an MLP projection, a norm vector, lm_head): p within the fp32
    bar, m and v bit-exact (the moments follow the oracle's binary32 order)."""
    import torch
    import optimizer_step_amd as osa
    w = synth.WORKLOADS["adamw_f32_llama7b"]
    sizes, hp, steps = w["sizes"], w["hp"], w["steps"]
    names = [nm for nm, _ in synth.llama7b_shapes()]
    pick = [names.index(x) for x in ("embed", "l0.q", "l17.gate", "l31.mlp_norm", "lm_head")]
    total = sum(sizes)
    offs = np.cumsum([0] + sizes[:-1])
    P = torch.empty(total, dtype=torch.float32, device="cuda")
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    st = _flat_states("f32", total, "adamw", None, None)
    p0 = {k: to_host(P[offs[k]:offs[k] + sizes[k]]).copy() for k in pick}
    g_hist = {k: [] for k in pick}
    for t in range(1, steps + 1):
        G = synth.device_grads(total, "cuda", w["g_std"], t, bf16=True)
        tl = osa.TensorList(_views(P, G, st, sizes, "f32"))
        osa.opt_step_adamw(tl, "f32", osa.hparams(step=t, **hp))
        for k in pick:
            g_hist[k].append(to_host(G[offs[k]:offs[k] + sizes[k]]).copy())
        del G, tl
    torch.cuda.synchronize()
    got = {k: {key: to_host(buf[offs[k]:offs[k] + sizes[k]]) for key, buf in (("p", P), ("s1", st["s1"]),
                                                                                  ("s2", st["s2"]))} for k in pick}
    del P, st
    torch.cuda.empty_cache()
    S = 1 << 24

    def check(job):
        k, lo = job
        hi = min(sizes[k], lo + S)
        p = p0[k][lo:hi].copy()
        s = oracle.state_zeros("f32", hi - lo)
        for t in range(1, steps + 1):
            oracle.step("adamw", "f32", oracle.make_hp(step=t, tensor_index=k, index_base=lo, **hp), p,
                        g_hist[k][t - 1][lo:hi], **s)
        return (k, lo, fp32_close(got[k]["p"][lo:hi], p), nan_equal_bits(got[k]["s1"][lo:hi], s["s1"]),
                nan_equal_bits(got[k]["s2"][lo:hi], s["s2"]))

    jobs = [(k, lo) for k in pick for lo in range(0, sizes[k], S)]
    with _pool() as pool:
        results = list(pool.map(check, jobs))
    for k in pick:
        print(f"{names[k]} ({sizes[k]} elements): whole tensor checked", flush=True)
    failed = [r for r in results if not all(r[2:])]
    assert not failed, failed[:4]

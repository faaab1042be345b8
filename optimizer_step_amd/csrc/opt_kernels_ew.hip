// opt_kernels_ew.hip -- gfx950 kernel of the element-wise two-state step
// with fp32 or BF16 states (AdamW, AdEMAMix), for fp32, BF16 or FP16
// parameters and gradients.
//
// One workgroup per tile of 1024 consecutive elements of one tensor (the
// tile scheduling of opt_elem.h): 256 threads, or 128 for 16-bit parameters
// with BF16 states (EwShape below).  Inside a tile every lane owns one or two
// groups of 4 consecutive elements, so fp32 arrays move as 128-bit
// accesses and 16-bit ones as 64-bit accesses, every access instruction of a
// wave64 fully coalesced; a full tile issues all its loads before any
// arithmetic (the per-call scalars come formed in the kernel arguments).  The
// moments are formed exactly (fixed binary32 order); the direction u, which
// only feeds p, uses the hardware reciprocal and square root (measured on
// MI355X: +2 % on the 290-tensor AdamW step, +5-6 % with BF16 states), for a
// 16-bit parameter only where its error bound proves the stored word
// (moments16 in opt_elem.h).  HBM-bound: every byte is read or written once
// per step and no intermediate leaves registers.
#include "opt_elem.h"

namespace optstep {

// ---------------------------------------------------------------------------
// fp32 and BF16 states

struct Group {
    float p[4], g[4], m[4], v[4], m2[4];
};

// One tile's arrays: the tensor's arrays advanced to the tile's first element
// (wave-uniform), addressed by a 32-bit element index within the tile.
struct TileRef {
    void *p, *s1, *s2, *s3;
    const void *g;
    int64_t j0;      // element index of the tile's first element within the whole tensor
    uint32_t rk;     // the tensor number of its stochastic-rounding stream
};

template <int OPT, int GD, int SF, int PD>
__device__ __forceinline__ TileRef tile_ref(const DevTensor &T, int64_t e0)
{
    constexpr int pb = PD == kP32 ? 4 : 2, gb = GD == kGradF32 ? 4 : 2, sb = SF == kF32 ? 4 : 2;
    TileRef r;
    r.p = (char *)(void *)T.p + e0 * pb;
    r.g = (const char *)T.g + e0 * gb;
    r.s1 = (char *)T.s1 + e0 * sb;
    r.s2 = (char *)T.s2 + e0 * sb;
    r.s3 = OPT == kAdEMAMix ? (void *)((char *)T.s3 + e0 * sb) : nullptr;
    r.j0 = T.jbase + e0;
    r.rk = T.rk;
    return r;
}

template <int OPT, int GD, int SF, int PD>
__device__ __forceinline__ void ew_load(const TileRef &R, uint32_t i, bool fresh, Group &x)
{
    load_p4_at<PD>(R.p, i, x.p);
    load_grad4_at<GD>(R.g, i, x.g);
#pragma unroll
    for (int k = 0; k < 4; ++k) x.m[k] = x.v[k] = x.m2[k] = 0.0f;
    if (!fresh) {   // a step that restarts the moments from zero reads none
        load_state4_at<SF>(R.s1, i, x.m);
        load_state4_at<SF>(R.s2, i, x.v);
        if (OPT == kAdEMAMix) load_state4_at<SF>(R.s3, i, x.m2);
    }
}

// PLAIN: no gradient scale and no skip_zeros in this call (a uniform choice
// made by the launcher), so neither costs an instruction per element.
template <int OPT, int GD, int SF, int PD, bool PLAIN>
__device__ __forceinline__ void ew_finish(const StepArgs &a, const Scalars &s, const TileRef &R,
                                          uint32_t i, float lam, Group &x)
{
    float mo[4], vo[4], m2o[4];
    // stochastic rounding: the first stream's word rounds m (its low half) and
    // v (its high half), the second stream's m2 (low half) and a 16-bit p
    // (high half); the stores take the 16 bits in the high half of a word
    uint32_t rm[4] = {0, 0, 0, 0}, rv[4] = {0, 0, 0, 0}, rm2[4] = {0, 0, 0, 0}, rp[4] = {0, 0, 0, 0};
    const uint64_t q = (uint64_t)(R.j0 + i) >> 2;
    if (SF == kBF16SR) {
        PhiloxOut w = sr_block(a.seed, a.step, R.rk, q, false);
        rm[0] = w.w0 << 16; rm[1] = w.w1 << 16; rm[2] = w.w2 << 16; rm[3] = w.w3 << 16;
        rv[0] = w.w0; rv[1] = w.w1; rv[2] = w.w2; rv[3] = w.w3;
    }
    const bool psr = PD != kP32 && a.p_sr;
    if ((SF == kBF16SR && OPT == kAdEMAMix) || psr) {
        PhiloxOut w2 = sr_block(a.seed, a.step, R.rk, q, true);
        rm2[0] = w2.w0 << 16; rm2[1] = w2.w1 << 16; rm2[2] = w2.w2 << 16; rm2[3] = w2.w3 << 16;
        rp[0] = w2.w0; rp[1] = w2.w1; rp[2] = w2.w2; rp[3] = w2.w3;
    }
    // fp32 parameters: the direction with the hardware reciprocal and square
    // root (exact recipe for an element with a tiny v_hat); 16-bit
    // parameters: the same where it provably stores the exact recipe's word
    Mom rr[4];
    float pn[4];
    if (PD == kP32) {
        moments4<OPT, !PLAIN>(s, a, x.g, x.m, x.v, x.m2, rr);
#pragma unroll
        for (int i = 0; i < 4; ++i) pn[i] = apply_update(x.p[i], s.d, lam, rr[i].u);
    } else {
        moments16<OPT, PD, !PLAIN>(s, a, x.p, x.g, x.m, x.v, x.m2, lam, psr, rp, rr, pn);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const Mom &r = rr[i];
        mo[i] = r.m; vo[i] = r.v; m2o[i] = r.m2;
        if (!PLAIN && a.skip_zeros && x.g[i] == 0.0f) {   // p (decay included) and the states as they were
            mo[i] = x.m[i]; vo[i] = x.v[i]; m2o[i] = x.m2[i];
        } else {
            x.p[i] = pn[i];
        }
    }
    // the store policy measured fastest for this configuration (opt_elem.h)
    constexpr bool sc1 = OPT == kAdamW && GD != kGradF32 && SF == kF32 && PD == kP32;
    store_p4_at<PD, sc1>(R.p, i, x.p, psr, rp);
    store_state4_at<SF, sc1>(R.s1, i, mo, rm);
    store_state4_at<SF, sc1>(R.s2, i, vo, rv);
    if (OPT == kAdEMAMix) store_state4_at<SF>(R.s3, i, m2o, rm2);
}

template <int OPT, int GD, int SF, int PD>
__device__ __forceinline__ void ew_single(const StepArgs &a, const Scalars &s, const DevTensor &T,
                                          int64_t e, float lam)
{
    float g = load_grad1<GD>(T.g, e);
    float m = 0.0f, v = 0.0f, m2 = 0.0f;
    if (!a.fresh) {
        m = load_state1<SF>(T.s1, e);
        v = load_state1<SF>(T.s2, e);
        if (OPT == kAdEMAMix) m2 = load_state1<SF>(T.s3, e);
    }
    Mom r = moments<OPT>(s, a, g, m, v, m2);
    const float p_old = load_p1<PD>(T.p, e);
    float pn = apply_update(p_old, s.d, lam, r.u);
    if (a.skip_zeros && g == 0.0f) {
        pn = p_old;
        r.m = m; r.v = v; r.m2 = m2;
    }
    uint32_t rm = 0, rv = 0, rm2 = 0, rp = 0;   // random bits in the high half, as in ew_finish
    if (SF == kBF16SR) {
        uint32_t w = philox_word(sr_block(a.seed, a.step, T.rk, (uint64_t)(T.jbase + e) >> 2, false), (int)(e & 3));
        rm = w << 16; rv = w;
    }
    const bool psr = PD != kP32 && a.p_sr;
    if ((SF == kBF16SR && OPT == kAdEMAMix) || psr) {
        uint32_t w2 = philox_word(sr_block(a.seed, a.step, T.rk, (uint64_t)(T.jbase + e) >> 2, true), (int)(e & 3));
        rm2 = w2 << 16; rp = w2;
    }
    store_p1<PD>(T.p, e, pn, psr, rp);
    store_state1<SF>(T.s1, e, r.m, rm);
    store_state1<SF>(T.s2, e, r.v, rv);
    if (OPT == kAdEMAMix) store_state1<SF>(T.s3, e, r.m2, rm2);
}

#ifndef OPT_EW_WAVES_PER_EU
#define OPT_EW_WAVES_PER_EU 0
#endif
#if OPT_EW_WAVES_PER_EU
#define OPT_EW_ATTR __attribute__((amdgpu_waves_per_eu(OPT_EW_WAVES_PER_EU)))
#else
#define OPT_EW_ATTR
#endif

#ifndef OPT_EW_THREADS
#define OPT_EW_THREADS 256
#endif

// Workgroup shape of the element-wise step: threads, and groups of four
// elements per lane, all loaded before any arithmetic.  BF16 or FP16
// parameters with BF16 states take 128 threads with two groups each (the
// same 1024-element tile).  Measured on MI355X, paired, 2^30 elements,
// BF16 p with BF16-SR states 2.59 ms against 3.05 (256 x 2: 2.60, 64 x 2:
// 2.56, 256 x 4: 2.89), with BF16 nearest states 2.36 against 2.82,
// AdEMAMix (2^28) 0.830 against 0.884; BF16 p with fp32 states loses 3-9 %
// with any of these, and fp32 p gains nothing (BF16 nearest states 1 %,
// BF16-SR -2 to -4 %).
template <int SF, int PD>
struct EwShape {
    static constexpr bool kPair = PD != kP32 && SF != kF32;
    static constexpr int kThreads = kPair ? 128 : OPT_EW_THREADS;
    static constexpr int kGroups = kPair ? 2 : kEwGroups;
    static constexpr int64_t kTile = (int64_t)kThreads * kGroups * 4;
};

template <int OPT, int GD, int SF, int PD, bool PLAIN>
__global__ __launch_bounds__((EwShape<SF, PD>::kThreads)) OPT_EW_ATTR void step_ew_kernel(const DevTensor *__restrict__ tens,
                                                                       const int32_t *__restrict__ ctab, StepArgs a)
{
    typedef EwShape<SF, PD> Sh;
    const Scalars s = call_scalars(a);
    const bool fresh = a.fresh != 0;
    for (int64_t w = blockIdx.x; w < a.ntiles; w += gridDim.x) {
        DevTensor T;
        int64_t e0, len;
        if (!locate_tile(tens, ctab, a, w, T, e0, len)) continue;
        const TileRef R = tile_ref<OPT, GD, SF, PD>(T, e0);
        if (len == Sh::kTile) {
            Group x[Sh::kGroups];
            load_prio_hi(SF != kBF16RN);
#pragma unroll
            for (int u = 0; u < Sh::kGroups; ++u)
                ew_load<OPT, GD, SF, PD>(R, 4u * (threadIdx.x + u * Sh::kThreads), fresh, x[u]);
            load_prio_lo(SF != kBF16RN);
            const float lam = a.unorm ? lam_for(a, T.k) : s.lam;
#pragma unroll
            for (int u = 0; u < Sh::kGroups; ++u)
                ew_finish<OPT, GD, SF, PD, PLAIN>(a, s, R, 4u * (threadIdx.x + u * Sh::kThreads), lam, x[u]);
        } else {   // a tensor's last, short tile
            const float lam = a.unorm ? lam_for(a, T.k) : s.lam;
            const uint32_t ngroups = (uint32_t)(len >> 2);
            for (uint32_t i = threadIdx.x; i < ngroups; i += Sh::kThreads) {
                Group x0;
                ew_load<OPT, GD, SF, PD>(R, 4u * i, fresh, x0);
                ew_finish<OPT, GD, SF, PD, PLAIN>(a, s, R, 4u * i, lam, x0);
            }
            const int64_t tail = len & 3;
            if ((int64_t)threadIdx.x < tail) ew_single<OPT, GD, SF, PD>(a, s, T, e0 + 4 * ngroups + threadIdx.x, lam);
        }
    }
}

// Resident workgroups per compute unit of an element-wise step (0: as many
// as registers allow, 8 for most of them).  Measured on MI355X in paired runs
// over one arena.  fp32-state AdamW with BF16 g and fp32 p, caps 0 / 3 / 4 /
// 5 / 6: 290-tensor Llama-7B-shaped list 29.41 / 27.45 / 27.71 / 28.56 /
// 29.41 ms, and with a gradient scale (the kernel that also reads it) 29.0 /
// 28.4 / 27.7 / 29.0 / 29.0 ms; 3 x 2^30 elements 13.83 / 12.73 / 12.89 /
// 13.42 / 13.83 ms; one 2^30 tensor 4.69 / 4.59 / 4.60 / 4.59 / 4.69 ms;
// 2^29 elements 2.32 / 2.40 / 2.31 / 2.28 / 2.32 ms; 2^28 elements 1.17 /
// 1.22 / 1.17 / 1.16 / 1.17 ms.  BF16 parameters (2^30): 3.85 / 4.31 /
// 3.82 / 3.73 / 3.84 ms.  AdEMAMix with fp32 states (2^28), caps 0 / 4 / 5 /
// 6: 1.735 / 1.685 / 1.701 / 1.736 ms; AdamW with BF16 nearest states (2^30),
// caps 0 / 5 / 6 / 7: 3.108 / 3.093 / 3.065 / 3.107 ms.  BF16 stochastic
// states gain nothing from a cap (and lose up to 10 % at 4).  AdamW with fp32
// g and states, caps 0 / 3 / 4 / 5 / 6: 2^28 elements 1.282 / 1.324 / 1.259 /
// 1.225 / 1.256 ms, 2^30 5.416 / 5.274 / 5.266 / 5.242 / 5.330 ms.
template <int OPT, int GD, int SF, int PD, bool PLAIN>
static int ew_wg_cap(const StepArgs &a)
{
    if (OPT == kAdEMAMix) return SF == kF32 ? 4 : 0;
    if (GD == kGradF32) return SF == kF32 && PD == kP32 ? 5 : 0;
    if (SF == kBF16RN) return PD == kP32 ? 6 : 0;
    if (SF != kF32) return 0;
    if (PD != kP32 || a.nchunks * a.chunk < ((int64_t)1 << 30)) return 5;
    return PLAIN ? 3 : 4;
}

template <int OPT, int GD, int PD, bool PLAIN>
static hipError_t launch_ew_p(int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    switch (fmt) {
    case kF32:
        return launch_tiles<EwShape<kF32, PD>::kThreads>(step_ew_kernel<OPT, GD, kF32, PD, PLAIN>, EwShape<kF32, PD>::kTile,
                                        cap_lds(lg, ew_wg_cap<OPT, GD, kF32, PD, PLAIN>(a)), lg, a, st);
    case kBF16RN:
        return launch_tiles<EwShape<kBF16RN, PD>::kThreads>(step_ew_kernel<OPT, GD, kBF16RN, PD, PLAIN>, EwShape<kBF16RN, PD>::kTile,
                                        cap_lds(lg, ew_wg_cap<OPT, GD, kBF16RN, PD, PLAIN>(a)), lg, a, st);
    case kBF16SR:
        return launch_tiles<EwShape<kBF16SR, PD>::kThreads>(step_ew_kernel<OPT, GD, kBF16SR, PD, PLAIN>, EwShape<kBF16SR, PD>::kTile,
                                        cap_lds(lg, ew_wg_cap<OPT, GD, kBF16SR, PD, PLAIN>(a)), lg, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <int OPT, int GD, int PD>
static hipError_t launch_ew_t(int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    return plain_call(a) ? launch_ew_p<OPT, GD, PD, true>(fmt, a, lg, st) : launch_ew_p<OPT, GD, PD, false>(fmt, a, lg, st);
}

template <int OPT, int GD>
static hipError_t launch_ew_g(int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    switch (a.p_dtype) {
    case kP32: return launch_ew_t<OPT, GD, kP32>(fmt, a, lg, st);
    case kPBF16: return launch_ew_t<OPT, GD, kPBF16>(fmt, a, lg, st);
    case kPF16: return launch_ew_t<OPT, GD, kPF16>(fmt, a, lg, st);
    default: return hipErrorInvalidValue;
    }
}

template <int OPT>
static hipError_t launch_ew_o(int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    switch (gd) {
    case kGradF32: return launch_ew_g<OPT, kGradF32>(fmt, a, lg, st);
    case kGradBF16: return launch_ew_g<OPT, kGradBF16>(fmt, a, lg, st);
    case kGradF16: return launch_ew_g<OPT, kGradF16>(fmt, a, lg, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step_ew(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    return opt == kAdamW ? launch_ew_o<kAdamW>(gd, fmt, a, lg, st) : launch_ew_o<kAdEMAMix>(gd, fmt, a, lg, st);
}

}  // namespace optstep

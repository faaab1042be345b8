// opt_elem.h -- helpers shared by the kernels: loads and stores of four
// consecutive elements of p, g and a state in their storage formats (the
// element-wise two-state and one-state steps), and the tile scheduling every
// multi-tensor launch uses.
#pragma once

#include <algorithm>

#include "opt_device.h"

namespace optstep {

#ifndef OPT_EW_GROUPS
#define OPT_EW_GROUPS 1
#endif
// Groups of four elements per lane in a tile of the element-wise steps.  One
// (1024-element tiles) measured fastest on MI355X for the 290-tensor list:
// 5.70-5.90 TB/s against 5.56-5.79 with two and 5.52-5.81 with four per lane,
// and 5.13-5.49 for the persistent grid walking 32 k-element chunks that came
// before.
constexpr int kEwGroups = OPT_EW_GROUPS;

#ifndef OPT_LOAD_PRIO
#define OPT_LOAD_PRIO 1
#endif

// A wave raises its issue priority while it issues a tile's loads and drops
// it before the arithmetic, so that waves holding loads get them to memory
// ahead of waves that are computing or storing.  On MI355X, against the same
// kernels without it, in one process: the 290-tensor AdamW step +0.5-0.8 %
// in every paired run, BF16-SR and FP4-SR states +0.6-2 %, AdEMAMix and the
// update-norm pass +0.1-0.7 %, 8-bit and FP8-RN states unchanged, and BF16
// nearest states -0.2-0.6 % (that instantiation leaves it off).
__device__ __forceinline__ void load_prio_hi(bool on = true)
{
    if (OPT_LOAD_PRIO && on) __builtin_amdgcn_s_setprio(3);
}
__device__ __forceinline__ void load_prio_lo(bool on = true)
{
    if (OPT_LOAD_PRIO && on) __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// element groups of four

// Four 16-bit words (BF16 if BF, else FP16) widened to fp32.
template <bool BF>
__device__ __forceinline__ void widen4(u2 w, float out[4])
{
    if (BF) {
        out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    } else {
        out[0] = f16_lo(w.x); out[1] = f16_hi(w.x); out[2] = f16_lo(w.y); out[3] = f16_hi(w.y);
    }
}

template <int GD>
__device__ __forceinline__ void load_grad4(const void *g, int64_t e, float out[4])
{
    if (GD == kGradF32) {
        f4 x = sld<f4>((const float *)g + e);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        widen4<GD == kGradBF16>(sld<u2>((const uint16_t *)g + e), out);
    }
}

template <int GD>
__device__ __forceinline__ float load_grad1(const void *g, int64_t e)
{
    if (GD == kGradF32) return gld<float>((const float *)g + e);
    const uint32_t h = gld<uint16_t>((const uint16_t *)g + e);
    return GD == kGradBF16 ? bf16_lo(h) : f16_lo(h);
}

// Parameters: fp32, or BF16 / FP16 words widened exactly and stored back
// rounded to nearest-even or, with sr, stochastically.  Every random operand
// of the stores below carries the element's 16 random bits in its HIGH half
// (the low half is ignored), the convention of gfx950's stochastic BF16
// conversion.
template <int PD>
__device__ __forceinline__ void load_p4(const float *p, int64_t e, float out[4])
{
    if (PD == kP32) {
        f4 x = sld<f4>(p + e);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        widen4<PD == kPBF16>(sld<u2>((const uint16_t *)(const void *)p + e), out);
    }
}

template <int PD>
__device__ __forceinline__ float load_p1(const float *p, int64_t e)
{
    if (PD == kP32) return gld<float>(p + e);
    const uint32_t h = gld<uint16_t>((const uint16_t *)(const void *)p + e);
    return PD == kPBF16 ? bf16_lo(h) : f16_lo(h);
}

template <int PD>
__device__ __forceinline__ uint32_t round_p(float x, bool sr, uint32_t rh)
{
    if (PD == kPBF16) return sr ? bf16_sr(x, rh >> 16) : bf16_rne(x);
    return sr ? f16_sr(x, rh >> 16) : f16_rne(x);
}

// ---------------------------------------------------------------------------
// 16-bit parameters.  Their stored word must be the one the exact recipe's
// binary32 parameter rounds to.  With the fast direction u and its bound bu
// (moments_fast), pf = RN(RN(p*d) - step) with step = RN(lam*u), and the
// exact recipe's pe differs from pf by at most |lam|*bu/2 + 2^-23 (|step| +
// |pf|) + 2^-148 to first order (the step's and the parameter's roundings;
// bu already holds a factor two).  B = |lam|*bu + 2^-22 (|step| + |pf|) +
// 2^-126 covers that twice over, and the rounding of pf -+ B besides, for
// |lam| <= 2^20 (the caller's test) and with step, pf and B well inside the
// binary32 range, so that nothing on either path overflows.  Both 16-bit
// roundings are monotone in |x| for a fixed random operand, so when pf - B
// and pf + B have one sign and round to one word, pe rounds to it too.
template <int PD>
__device__ __forceinline__ bool p16_same(float pf, float step, float bu, float lam, bool sr, uint32_t rh)
{
    const float as = __builtin_fabsf(step), ap = __builtin_fabsf(pf);
    const float B = __builtin_fmaf(__builtin_fabsf(lam), bu, __builtin_fmaf(0x1p-22f, as + ap, 0x1p-126f));
    const float lo = pf - B, hi = pf + B;
    if (!(B < 0x1p100f) || !(__builtin_fmaxf(as, ap) < 0x1p126f) || ((fbits(lo) ^ fbits(hi)) >> 31) != 0u)
        return false;
    if (PD == kPBF16) {
        const uint32_t w = sr ? bf16x2_sr_hi(lo, rh, hi, rh) : bf16x2_rne(lo, hi);
        return (w & 0xFFFFu) == (w >> 16);
    }
    // FP16: well inside its range, where its stochastic rounding is plain
    return __builtin_fabsf(lo) < 0x1p15f && __builtin_fabsf(hi) < 0x1p15f &&
           round_p<PD>(lo, sr, rh) == round_p<PD>(hi, sr, rh);
}

// Moments, direction and new binary32 parameter of four elements with a
// 16-bit parameter (rh: their rounding bits, as the store takes them): the
// fast direction where p16_same shows that the stored word is the exact
// recipe's, else (about one element in 2^14 for BF16, 2^11 for FP16, and all
// of them for eps < 0 or |lam| > 2^20, which the bound does not cover) the
// exact recipe.  The wave skips the exact pass when no lane needs it; each
// element's result depends on its own inputs alone.
template <int OPT, int PD, bool GS>
__device__ __forceinline__ void moments16(const Scalars &s, const StepArgs &a, const float p[4], const float g[4],
                                          const float m[4], const float v[4], const float m2[4], float lam, bool sr,
                                          const uint32_t rh[4], Mom r[4], float pn[4])
{
    const bool fast = a.eps >= 0.0f && __builtin_fabsf(lam) <= 0x1p20f;
    bool slow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float bu;
        r[i] = moments_fast<OPT, GS>(s, a, g[i], m[i], v[i], m2[i], &bu);
        pn[i] = apply_update(p[i], s.d, lam, r[i].u);
        slow[i] = !(fast && fast_ok<OPT>(s, r[i]) && p16_same<PD>(pn[i], lam * r[i].u, bu, lam, sr, rh[i]));
    }
    if (__any(slow[0] || slow[1] || slow[2] || slow[3])) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (slow[i]) {
                r[i] = moments<OPT, GS>(s, a, g[i], m[i], v[i], m2[i]);
                pn[i] = apply_update(p[i], s.d, lam, r[i].u);
            }
        }
    }
}

template <int PD>
__device__ __forceinline__ void store_p4(float *p, int64_t e, const float x[4], bool sr, const uint32_t rh[4])
{
    if (PD == kP32) {
        sst<f4>(p + e, f4{x[0], x[1], x[2], x[3]});
    } else if (PD == kPBF16) {
        u2 w = sr ? u2{bf16x2_sr_hi(x[0], rh[0], x[1], rh[1]), bf16x2_sr_hi(x[2], rh[2], x[3], rh[3])}
                  : u2{bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3])};
        sst<u2>((uint16_t *)(void *)p + e, w);
    } else {
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = round_p<PD>(x[i], sr, rh[i]);
        sst<u2>((uint16_t *)(void *)p + e, u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
    }
}

template <int PD>
__device__ __forceinline__ void store_p1(float *p, int64_t e, float x, bool sr, uint32_t rh)
{
    if (PD == kP32) gst<float>(p + e, x);
    else gst<uint16_t>((uint16_t *)(void *)p + e, (uint16_t)round_p<PD>(x, sr, rh));
}

template <int SF>
__device__ __forceinline__ void load_state4(const void *s, int64_t e, float out[4])
{
    if (SF == kF32) {
        f4 x = sld<f4>((const float *)s + e);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        u2 w = sld<u2>((const uint16_t *)s + e);
        out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
        out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    }
}

template <int SF>
__device__ __forceinline__ float load_state1(const void *s, int64_t e)
{
    if (SF == kF32) return gld<float>((const float *)s + e);
    return bf16_lo(gld<uint16_t>((const uint16_t *)s + e));
}

// Store four fp32 moments in format SF; rh[i] hold the 16 random bits of
// stochastic rounding in their high half (ignored by the other formats).
template <int SF>
__device__ __forceinline__ void store_state4(void *s, int64_t e, const float x[4], const uint32_t rh[4])
{
    if (SF == kF32) {
        sst<f4>((float *)s + e, f4{x[0], x[1], x[2], x[3]});
    } else if (SF == kBF16SR) {
        sst<u2>((uint16_t *)s + e, u2{bf16x2_sr_hi(x[0], rh[0], x[1], rh[1]), bf16x2_sr_hi(x[2], rh[2], x[3], rh[3])});
    } else {
        sst<u2>((uint16_t *)s + e, u2{bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3])});
    }
}

template <int SF>
__device__ __forceinline__ void store_state1(void *s, int64_t e, float x, uint32_t rh)
{
    if (SF == kF32) gst<float>((float *)s + e, x);
    else gst<uint16_t>((uint16_t *)s + e, (uint16_t)(SF == kBF16SR ? bf16_sr(x, rh >> 16) : bf16_rne(x)));
}

// ---------------------------------------------------------------------------
// The same group loads and stores addressed as a wave-uniform base pointer
// plus a 32-bit byte offset per lane (base + zero-extended offset: the
// global_* saddr form, one VGPR per address instead of two).  i is the
// element index within the run that starts at the base (i * 4 < 2^32).

template <class V>
__device__ __forceinline__ V sld_at(const void *base, uint32_t off)
{
    return sld<V>((const char *)base + off);
}

// Stores of the element-wise steps: the global store with the non-temporal
// hint, or (SC1) a buffer store with the system-coherence bit and no
// non-temporal hint.  Paired on MI355X in one process over one arena, on two
// boxes: the 290-tensor AdamW step (fp32 p, m, v; BF16 g) 30.01 -> 29.29 ms
// and 30.02 -> 29.31 ms with SC1 on its 16-byte stores; the same policy cost
// 2.7 % on AdEMAMix (fp32 g) and 0.8-1.3 % on BF16-state and BF16-parameter
// steps, so only that configuration takes it.  Other policy bits on the same
// buffer store, paired on that step (290-tensor list / 3 x 2^30 elements):
// SC0|SC1 the same, NT|SC1 and NT|SC0|SC1 0.1-1 % slower, NT and NT|SC0 2-4 %,
// no bits or SC0 alone 5-15 %.  The buffer resource spans
// 2^32 - 1 bytes from the tile's base; every offset here is below a tile's
// bytes.
template <bool SC1, class V>
__device__ __forceinline__ void sst_at(void *base, uint32_t off, V v)
{
    if constexpr (SC1 && sizeof(V) == 16) {
        __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, -1, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, 16 /* sc1 */);
    } else {
        sst<V>((char *)base + off, v);
    }
}

template <int PD>
__device__ __forceinline__ void load_p4_at(const void *p, uint32_t i, float out[4])
{
    if (PD == kP32) {
        f4 x = sld_at<f4>(p, i * 4u);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        widen4<PD == kPBF16>(sld_at<u2>(p, i * 2u), out);
    }
}

template <int GD>
__device__ __forceinline__ void load_grad4_at(const void *g, uint32_t i, float out[4])
{
    if (GD == kGradF32) {
        f4 x = sld_at<f4>(g, i * 4u);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        widen4<GD == kGradBF16>(sld_at<u2>(g, i * 2u), out);
    }
}

template <int SF>
__device__ __forceinline__ void load_state4_at(const void *s, uint32_t i, float out[4])
{
    if (SF == kF32) {
        f4 x = sld_at<f4>(s, i * 4u);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
        u2 w = sld_at<u2>(s, i * 2u);
        out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
        out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    }
}

template <int PD, bool SC1 = false>
__device__ __forceinline__ void store_p4_at(void *p, uint32_t i, const float x[4], bool sr, const uint32_t rh[4])
{
    if (PD == kP32) {
        sst_at<SC1, f4>(p, i * 4u, f4{x[0], x[1], x[2], x[3]});
    } else if (PD == kPBF16) {
        u2 w = sr ? u2{bf16x2_sr_hi(x[0], rh[0], x[1], rh[1]), bf16x2_sr_hi(x[2], rh[2], x[3], rh[3])}
                  : u2{bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3])};
        sst_at<false, u2>(p, i * 2u, w);
    } else {
        uint32_t h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) h[k] = round_p<PD>(x[k], sr, rh[k]);
        sst_at<false, u2>(p, i * 2u, u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
    }
}

template <int SF, bool SC1 = false>
__device__ __forceinline__ void store_state4_at(void *s, uint32_t i, const float x[4], const uint32_t rh[4])
{
    if (SF == kF32) {
        sst_at<SC1, f4>(s, i * 4u, f4{x[0], x[1], x[2], x[3]});
    } else if (SF == kBF16SR) {
        sst_at<false, u2>(s, i * 2u, u2{bf16x2_sr_hi(x[0], rh[0], x[1], rh[1]), bf16x2_sr_hi(x[2], rh[2], x[3], rh[3])});
    } else {
        sst_at<false, u2>(s, i * 2u, u2{bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3])});
    }
}

// ---------------------------------------------------------------------------
// Tile scheduling.  A launch covers its bucket's chunk space in tiles of
// consecutive elements of one tensor; a chunk of the host's table (a power of
// two, as is the kernel's tile) holds chunk/tile of them.  By default the grid
// has one workgroup per tile: the dispatcher hands tiles out in order as
// workgroups retire, so the tiles in flight form one compact window over each
// array and nothing waits on a straggler.  A persistent grid of wgs_per_cu
// workgroups per compute unit walking the same tiles with a grid stride is
// kept as a launch option; results do not depend on the grid.

constexpr int64_t kMaxGrid = (int64_t)1 << 23;   // workgroups per launch (x threads < 2^32)

// Fills the tile fields of a for a kernel whose tile is ktile elements.
__host__ inline void set_tiles(StepArgs &a, int64_t ktile)
{
    a.tile = ktile < a.chunk ? ktile : a.chunk;
    int sh = 0;
    while ((a.tile << sh) < a.chunk) ++sh;
    a.tile_sh = sh;
    a.ntiles = a.nchunks << sh;
}

__host__ inline unsigned tile_grid(const StepArgs &a, const LaunchGeom &lg)
{
    int64_t g = a.ntiles;
    if (lg.wgs_per_cu > 0) g = std::min<int64_t>(g, (int64_t)lg.ncu * lg.wgs_per_cu);
    return (unsigned)std::max<int64_t>(1, std::min(g, kMaxGrid));
}

// Tile w of the launch: its tensor, first element and length.  False for a
// tile past its tensor's end (a tensor's last chunk may be partly empty).
// Uniform over the workgroup.
__device__ __forceinline__ bool locate_tile(const DevTensor *__restrict__ tens, const int32_t *__restrict__ ctab,
                                            const StepArgs &a, int64_t w, DevTensor &T, int64_t &e0, int64_t &len)
{
    const int64_t c = w >> a.tile_sh;
    T = tens[ctab[c]];
    e0 = (c - T.chunk_begin) * a.chunk + (w & (((int64_t)1 << a.tile_sh) - 1)) * a.tile;
    len = min(a.tile, T.numel - e0);
    return len > 0;
}

// A call with no gradient scale, no skip_zeros and no state reset on this
// step: the step kernels have a variant that spends no instruction on any.
__host__ inline bool plain_call(const StepArgs &a) { return a.grad_scale == nullptr && !a.skip_zeros && !a.fresh; }

// Occupancy cap.  A tile kernel is held to `cap` resident workgroups per
// compute unit (cap waves per SIMD for 256 threads) by reserving, at launch,
// LDS it never touches: 1 KiB under a cap-th of the 160 KiB each gfx950
// compute unit holds, which leaves room for the kernels' few bytes of static
// LDS and keeps cap + 1 workgroups from fitting.  Measured on MI355X, some
// element-wise configurations run faster with fewer waves in flight than
// their registers allow (the launchers name them).
constexpr size_t kLdsPerCu = 160 * 1024;

__host__ inline size_t cap_lds(const LaunchGeom &lg, int dflt)
{
    const int cap = lg.wg_cap >= 0 ? lg.wg_cap : dflt;
    return cap >= 2 ? kLdsPerCu / cap - 1024 : 0;
}

// One launch of a tile kernel taking (tens, ctab, a), THREADS per workgroup.
template <int THREADS = kThreads, class K>
static hipError_t launch_tiles(K kernel, int64_t ktile, size_t lds, const LaunchGeom &lg, StepArgs a, hipStream_t st)
{
    set_tiles(a, ktile);
    hipLaunchKernelGGL(kernel, dim3(tile_grid(a, lg)), dim3(THREADS), lds, st, a.tens, a.chunk_tensor, a);
    return hipGetLastError();
}

}  // namespace optstep

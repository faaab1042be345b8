// opt_kernels_1s.hip -- gfx950 kernels of the one-state optimizers: momentum,
// RMSprop and Adagrad with coupled L2, and Lion with decoupled decay
// (bitsandbytes PR "Fix decoupled weight decay ordering in the CUDA
// Adam/AdEMAMix kernels", intro: how the 1-state kernels couple the decay).
//
// Same layout as the two-state element-wise step: one workgroup per tile of
// kEwTile1 elements (the tile scheduling of opt_elem.h); lanes own groups of
// four consecutive elements, kEwGroups groups loaded before any arithmetic.
// Per element, in binary32 with no contraction:
//   g' = g*scale (+ wd*p for the coupled-L2 three when wd != 0)
//   momentum  m' = g' on the state's first step, else b1*m + g';  p' = p - lr*m'
//   RMSprop   v' = b1*v + (1-b1)*g'^2;  p' = p - lr*(g'/(sqrt(v') + eps))
//   Adagrad   v' = v + g'^2;            p' = p - lr*(g'/(sqrt(v') + eps))
//   Lion      c = b1*m + (1-b1)*g';  p' = p*(1 - lr*wd) - lr*sign(c);
//             m' = b2*m + (1-b2)*g'
// The state is fp32 or BF16 (nearest, or stochastic with the low half of the
// element's first-stream Philox word).  HBM-bound: 4+4 (p) + 2|4 (g) + 2x the
// state bytes per element.
#include "opt_elem.h"

namespace optstep {

struct Scalars1 {
    float om1, om2;   // 1 - beta1, 1 - beta2
    float d;          // 1 - lr*wd (Lion)
    float gs;         // gradient scale
    bool first;       // the state's first step (momentum starts from g')
};

__device__ __forceinline__ float sign_f(float c)
{
    return c != c ? c : (c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f));
}

// One element: returns the new state, updates p in place.
template <int OPT>
__device__ __forceinline__ float one_state(const StepArgs &a, const Scalars1 &s, float g, float &p, float st)
{
    const float gs = g * s.gs;
    float gp = gs;
    if (OPT != kLion && a.wd != 0.0f) gp = gs + a.wd * p;
    float sn;
    if (OPT == kMomentum) {
        sn = s.first ? gp : a.beta1 * st + gp;
        p = p - a.lr * sn;
    } else if (OPT == kRMSprop || OPT == kAdagrad) {
        const float gg = gp * gp;
        sn = OPT == kRMSprop ? a.beta1 * st + s.om1 * gg : st + gg;
        const float den = __builtin_sqrtf(sn) + a.eps;
        const float u = gp / den;
        p = p - a.lr * u;
    } else {
        const float c = a.beta1 * st + s.om1 * gs;
        const float decayed = p * s.d;
        p = decayed - a.lr * sign_f(c);
        sn = a.beta2 * st + s.om2 * gs;
    }
    return sn;
}

struct Group1 {
    float p[4], g[4], s[4];
};

constexpr int64_t kEwTile1 = (int64_t)kThreads * kEwGroups * 4;

// The call's scalars (uniform: every lane forms the same values).
__device__ __forceinline__ Scalars1 scalars1(const StepArgs &a)
{
    Scalars1 s;
    s.om1 = 1.0f - a.beta1;
    s.om2 = 1.0f - a.beta2;
    const float lrwd = a.lr * a.wd;
    s.d = 1.0f - lrwd;
    s.gs = a.grad_scale ? *a.grad_scale : 1.0f;
    s.first = a.bc_step == 1;
    return s;
}

template <int OPT, int GD, int SF>
__device__ __forceinline__ void s1_load(const DevTensor &T, int64_t e, bool fresh, Group1 &x)
{
    f4 pv = sld<f4>(T.p + e);
    x.p[0] = pv.x; x.p[1] = pv.y; x.p[2] = pv.z; x.p[3] = pv.w;
    load_grad4<GD>(T.g, e, x.g);
    x.s[0] = x.s[1] = x.s[2] = x.s[3] = 0.0f;
    if (!fresh) load_state4<SF>(T.s1, e, x.s);
}

template <int OPT, int GD, int SF>
__device__ __forceinline__ void s1_finish(const StepArgs &a, const Scalars1 &s, const DevTensor &T, int64_t e,
                                          Group1 &x)
{
    float sn[4];
    uint32_t r[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float p_old = x.p[j];
        sn[j] = one_state<OPT>(a, s, x.g[j], x.p[j], x.s[j]);
        if (a.skip_zeros && x.g[j] == 0.0f) {   // p and the state as they were
            x.p[j] = p_old;
            sn[j] = x.s[j];
        }
    }
    if (SF == kBF16SR) {
        const PhiloxOut w = sr_block(a.seed, a.step, T.rk, (uint64_t)(T.jbase + e) >> 2, false);
        r[0] = w.w0 << 16; r[1] = w.w1 << 16; r[2] = w.w2 << 16; r[3] = w.w3 << 16;   // low halves, moved up
    }
    sst<f4>(T.p + e, f4{x.p[0], x.p[1], x.p[2], x.p[3]});
    store_state4<SF>(T.s1, e, sn, r);
}

template <int OPT, int GD, int SF>
__device__ __forceinline__ void s1_single(const StepArgs &a, const Scalars1 &s, const DevTensor &T, int64_t e,
                                          bool fresh)
{
    float p = gld<float>(T.p + e);
    const float g = load_grad1<GD>(T.g, e);
    const float st = fresh ? 0.0f : load_state1<SF>(T.s1, e);
    const float p_old = p;
    float sn = one_state<OPT>(a, s, g, p, st);
    if (a.skip_zeros && g == 0.0f) {
        p = p_old;
        sn = st;
    }
    uint32_t r = 0;
    if (SF == kBF16SR)
        r = philox_word(sr_block(a.seed, a.step, T.rk, (uint64_t)(T.jbase + e) >> 2, false), (int)(e & 3)) << 16;
    gst<float>(T.p + e, p);
    store_state1<SF>(T.s1, e, sn, r);
}

template <int OPT, int GD, int SF>
__global__ __launch_bounds__(kThreads) void step_1s_kernel(const DevTensor *__restrict__ tens,
                                                           const int32_t *__restrict__ ctab, StepArgs a)
{
    const Scalars1 s = scalars1(a);
    const bool fresh = a.fresh != 0;
    for (int64_t w = blockIdx.x; w < a.ntiles; w += gridDim.x) {
        DevTensor T;
        int64_t e0, len;
        if (!locate_tile(tens, ctab, a, w, T, e0, len)) continue;
        if (len == kEwTile1) {
            Group1 x[kEwGroups];
            load_prio_hi();
#pragma unroll
            for (int u = 0; u < kEwGroups; ++u) s1_load<OPT, GD, SF>(T, e0 + 4 * (threadIdx.x + u * kThreads), fresh, x[u]);
            load_prio_lo();
#pragma unroll
            for (int u = 0; u < kEwGroups; ++u) s1_finish<OPT, GD, SF>(a, s, T, e0 + 4 * (threadIdx.x + u * kThreads), x[u]);
        } else {   // a tensor's last, short tile
            const int64_t ngroups = len >> 2;
            for (int64_t i = threadIdx.x; i < ngroups; i += kThreads) {
                Group1 x0;
                s1_load<OPT, GD, SF>(T, e0 + 4 * i, fresh, x0);
                s1_finish<OPT, GD, SF>(a, s, T, e0 + 4 * i, x0);
            }
            const int64_t tail = len & 3;
            if ((int64_t)threadIdx.x < tail) s1_single<OPT, GD, SF>(a, s, T, e0 + 4 * ngroups + threadIdx.x, fresh);
        }
    }
}

template <int OPT, int GD>
static hipError_t launch_1s_t(int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    switch (fmt) {
    // fp32 state: at most 5 resident workgroups per compute unit (measured on
    // MI355X, 2^30 elements, BF16 g: momentum 3.19 -> 3.09 ms, Lion 3.19 ->
    // 3.08 ms; fp32 g: momentum 3.635 -> 3.493 ms)
    case kF32:
        return launch_tiles(step_1s_kernel<OPT, GD, kF32>, kEwTile1, cap_lds(lg, 5), lg, a, st);
    case kBF16RN: return launch_tiles(step_1s_kernel<OPT, GD, kBF16RN>, kEwTile1, cap_lds(lg, 0), lg, a, st);
    case kBF16SR: return launch_tiles(step_1s_kernel<OPT, GD, kBF16SR>, kEwTile1, cap_lds(lg, 0), lg, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <int OPT>
static hipError_t launch_1s_o(int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    switch (gd) {
    case kGradF32: return launch_1s_t<OPT, kGradF32>(fmt, a, lg, st);
    case kGradBF16: return launch_1s_t<OPT, kGradBF16>(fmt, a, lg, st);
    case kGradF16: return launch_1s_t<OPT, kGradF16>(fmt, a, lg, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step_1state(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st)
{
    switch (opt) {
    case kMomentum: return launch_1s_o<kMomentum>(gd, fmt, a, lg, st);
    case kRMSprop: return launch_1s_o<kRMSprop>(gd, fmt, a, lg, st);
    case kAdagrad: return launch_1s_o<kAdagrad>(gd, fmt, a, lg, st);
    case kLion: return launch_1s_o<kLion>(gd, fmt, a, lg, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace optstep

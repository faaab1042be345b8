// opt_kernels.hip -- gfx950 kernels of the deterministic update-norm
// pre-pass, the fused multi-tensor gradient norm, the standalone rounding
// cast and the test hooks.  (The element-wise two-state step is in
// opt_kernels_ew.hip, the blockwise-state step in opt_kernels_q8.hip, the
// one-state optimizers in opt_kernels_1s.hip.)  Every kernel here is
// HBM-bound or close to it (no dense contraction, so no MFMA): each byte is
// read or written once per call.
#include "opt_blk.h"

namespace optstep {

// ---------------------------------------------------------------------------
// max_unorm pre-pass.  The tensor is cut into tiles of kUTile elements from
// element 0; one wave sums a tile ({sum u^2, sum p^2} in binary64: per lane in
// element order, then a fixed butterfly) and writes one partial per tile, and
// one workgroup per tensor then sums its tiles in a fixed order.  Nothing
// depends on the chunk size, the grid or timing, and there are no atomics, so
// repeated runs give identical bits.

// One stored state value at element e of a tensor.  WHICH: 0 = m, 1 = v, 2 = m2.
template <int SF, int WHICH>
__device__ __forceinline__ float read_state(const uint32_t *lds, const void *s, const float *amax, int64_t e)
{
    if (SF == kF32 || SF == kBF16RN) return load_state1<SF == kF32 ? kF32 : kBF16RN>(s, e);
    uint32_t c;
    if (fp4_fmt(SF)) c = ((uint32_t)gld<uint8_t>((const uint8_t *)s + e / 2) >> (4 * (e & 1))) & 0xFu;
    else c = gld<uint8_t>((const uint8_t *)s + e);
    float out[4];
    blk_decode4<SF, WHICH>(lds, c, gld<float>(amax + e / kQBlock), out);
    return out[0];
}

// Four consecutive state values starting at e (a multiple of 4, so one block
// holds all four).
template <int SF, int WHICH>
__device__ __forceinline__ void read_state4(const uint32_t *lds, const void *s, const float *amax, int64_t e,
                                            float out[4])
{
    if (SF == kF32 || SF == kBF16RN) {
        load_state4<SF == kF32 ? kF32 : kBF16RN>(s, e, out);
        return;
    }
    const uint32_t c = fp4_fmt(SF) ? (uint32_t)sld<uint16_t>((const uint8_t *)s + e / 2)
                                   : sld<uint32_t>((const uint8_t *)s + e);
    blk_decode4<SF, WHICH>(lds, c, gld<float>(amax + e / kQBlock), out);
}

template <int OPT, int GD, int SF>
__global__ __launch_bounds__(kThreads) void unorm_partials_kernel(const DevTensor *__restrict__ tens,
                                                                  const int32_t *__restrict__ ctab,
                                                                  const uint32_t *__restrict__ qwords,
                                                                  StepArgs a)
{
    extern __shared__ uint32_t lds[];
    if (SF == kQ8)
        for (uint32_t i = threadIdx.x; i < 512; i += kThreads) lds[i] = qwords[i];
    __syncthreads();
    const Scalars s = call_scalars(a);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t w = blockIdx.x; w < a.ntiles; w += gridDim.x) {
        DevTensor T;
        int64_t e0, len;
        if (!locate_tile(tens, ctab, a, w, T, e0, len)) continue;
        const int64_t slot0 = w * a.tile / kUTile;   // the tile's first partial in the chunk space
        const int64_t ntile = (len + kUTile - 1) / kUTile;
        for (int64_t tt = wave; tt < ntile; tt += kWaves) {
            double su = 0.0, sp = 0.0;
            const bool full = (tt + 1) * kUTile <= len;
            if (full) {
                // the whole tile is in range: 4 groups of 4 per lane, loads first
                float p[4][4], g[4][4], m[4][4], v[4][4], m2[4][4];
                load_prio_hi();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t e = e0 + tt * kUTile + q * 256 + lane * 4;
                    if (a.p_dtype == kP32) load_p4<kP32>(T.p, e, p[q]);
                    else if (a.p_dtype == kPBF16) load_p4<kPBF16>(T.p, e, p[q]);
                    else load_p4<kPF16>(T.p, e, p[q]);
                    load_grad4<GD>(T.g, e, g[q]);
                    m[q][0] = m[q][1] = m[q][2] = m[q][3] = 0.0f;
                    v[q][0] = v[q][1] = v[q][2] = v[q][3] = 0.0f;
                    m2[q][0] = m2[q][1] = m2[q][2] = m2[q][3] = 0.0f;
                    if (!a.fresh) {   // a step that restarts the moments reads none
                        read_state4<SF, 0>(lds, T.s1, T.a1, e, m[q]);
                        read_state4<SF, 1>(lds, T.s2, T.a2, e, v[q]);
                        if (OPT == kAdEMAMix) read_state4<SF, 2>(lds, T.s3, T.a3, e, m2[q]);
                    }
                }
                load_prio_lo();
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        Mom r = moments<OPT>(s, a, g[q][j], m[q][j], v[q][j], m2[q][j]);
                        if (a.skip_zeros && g[q][j] == 0.0f) r.u = 0.0f;   // no update there
                        su += (double)r.u * (double)r.u;
                        sp += (double)p[q][j] * (double)p[q][j];
                    }
            } else {
                for (int q = 0; q < kUTile / 256; ++q) {
                    const int64_t i0 = tt * kUTile + q * 256 + lane * 4;   // within the chunk
                    const int n = (int)max((int64_t)0, min((int64_t)4, len - i0));
                    for (int j = 0; j < n; ++j) {
                        const int64_t e = e0 + i0 + j;
                        float g = load_grad1<GD>(T.g, e);
                        float m = 0.0f, v = 0.0f, m2 = 0.0f;
                        if (!a.fresh) {
                            m = read_state<SF, 0>(lds, T.s1, T.a1, e);
                            v = read_state<SF, 1>(lds, T.s2, T.a2, e);
                            if (OPT == kAdEMAMix) m2 = read_state<SF, 2>(lds, T.s3, T.a3, e);
                        }
                        Mom r = moments<OPT>(s, a, g, m, v, m2);
                        if (a.skip_zeros && g == 0.0f) r.u = 0.0f;
                        const float p = a.p_dtype == kP32 ? load_p1<kP32>(T.p, e)
                                      : a.p_dtype == kPBF16 ? load_p1<kPBF16>(T.p, e) : load_p1<kPF16>(T.p, e);
                        su += (double)r.u * (double)r.u;
                        sp += (double)p * (double)p;
                    }
                }
            }
            su = wave_sum(su);
            sp = wave_sum(sp);
            if (lane == 0) {
                const int64_t slot = slot0 + tt;
                gst<double>(a.partials + 2 * slot, su);
                gst<double>(a.partials + 2 * slot + 1, sp);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void unorm_reduce_kernel(const DevTensor *__restrict__ tens,
                                                              const double *groups, double *out)
{
    __shared__ double red[kWaves][2];
    const DevTensor T = tens[blockIdx.x];
    const int64_t ng = norm_groups(T.numel);
    double su = 0.0, sp = 0.0;
    for (int64_t i = threadIdx.x; i < ng; i += kThreads) {
        su += gld<double>(groups + 2 * (T.rg_begin + i));
        sp += gld<double>(groups + 2 * (T.rg_begin + i) + 1);
    }
    su = wave_sum(su);
    sp = wave_sum(sp);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { red[wave][0] = su; red[wave][1] = sp; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double U = red[0][0], P = red[0][1];
        for (int w = 1; w < kWaves; ++w) { U += red[w][0]; P += red[w][1]; }
        gst<double>(out + 2 * (int64_t)T.k, U);
        gst<double>(out + 2 * (int64_t)T.k + 1, P);
    }
}

// ---------------------------------------------------------------------------
// Gradient norms (the NeMo PR's fused multi-tensor reduction): per tile of
// kUTile elements one wave forms {sum g^2 in binary64, max |g| as bits}, then
// one workgroup per tensor sums its tiles, then one workgroup totals the list
// in tensor order.  Fixed orders, no atomics.  The tile partials reuse the
// update-norm partials buffer; slot 2t+1 carries the max as a double.

// One full tile's contribution from this lane: its 16 elements in order.
// The 16 gradients one lane holds of a full 1024-element partial unit, as
// raw 16-byte loads: elements q*256 + 4*lane + j (fp32, q < 4) or q*512 +
// 8*lane + j (16-bit, q < 2), summed by the lane in that order.
template <int GD>
struct GnRaw {
    u4 w[GD == kGradF32 ? 4 : 2];
};

template <int GD>
__device__ __forceinline__ void gnorm_load_unit(const void *g, int64_t e, int lane, GnRaw<GD> &r)
{
    if (GD == kGradF32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) r.w[q] = sld<u4>((const float *)g + e + q * 256 + lane * 4);
    } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) r.w[q] = sld<u4>((const uint16_t *)g + e + q * 512 + lane * 8);
    }
}

typedef uint16_t h2 __attribute__((ext_vector_type(2)));

// sq += x*x in binary64 for the unit's 16 values and mx = max |x| as an fp32
// bit pattern.  x*x is exact in binary64 for any fp32 or 16-bit x (at most 48
// significant bits, no overflow or underflow), so the fused multiply-add
// rounds exactly as the separate product and sum.  16-bit magnitudes are
// compared as packed 16-bit integers (their bit order is their numeric order,
// NaN above infinity), then widened exactly.
template <int GD>
__device__ __forceinline__ void gnorm_acc(const GnRaw<GD> &r, double &sq, uint32_t &mx)
{
    if (GD == kGradF32) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double x = (double)bitsf(r.w[q][j]);
                sq = __builtin_fma(x, x, sq);
                mx = max(mx, r.w[q][j] & 0x7FFFFFFFu);
            }
    } else {
        h2 m = {0, 0};
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t wd = r.w[q][j];
                const double lo = (double)(GD == kGradBF16 ? bf16_lo(wd) : f16_lo(wd));
                const double hi = (double)(GD == kGradBF16 ? bf16_hi(wd) : f16_hi(wd));
                sq = __builtin_fma(lo, lo, sq);
                sq = __builtin_fma(hi, hi, sq);
                m = __builtin_elementwise_max(m, __builtin_bit_cast(h2, wd & 0x7FFF7FFFu));
            }
        const uint32_t h = max((uint32_t)m.x, (uint32_t)m.y);
        mx = max(mx, GD == kGradBF16 ? h << 16 : fbits(f16_lo(h)));
    }
}
__device__ __forceinline__ void gnorm_store(const StepArgs &a, int64_t slot, int lane, double sq, uint32_t mx)
{
    sq = wave_sum(sq);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        gst<double>(a.partials + 2 * slot, sq);
        gst<double>(a.partials + 2 * slot + 1, (double)bitsf(mx));
    }
}

#ifndef OPT_GN_UNITS
#define OPT_GN_UNITS 2
#endif
#ifndef OPT_GN_WAVES
#define OPT_GN_WAVES 8
#endif
// One workgroup per tile of kGnTile gradient elements: kGnUnits partial units
// of 1024 elements per wave (16 KB of bf16 per workgroup), held to OPT_GN_WAVES
// waves per SIMD (56-64 registers, no spills).  A read-only stream wants bytes
// in flight: on the 290-tensor bf16 list this reads at 6.34-6.45 TB/s,
// against 6.19-6.25 with four units and no cap (92 registers, 5 waves).
constexpr int kGnUnits = OPT_GN_UNITS;
constexpr int64_t kGnTile = (int64_t)kWaves * kGnUnits * kUTile;
#define OPT_GN_ATTR __attribute__((amdgpu_waves_per_eu(OPT_GN_WAVES)))
template <int GD>
__global__ __launch_bounds__(kThreads) OPT_GN_ATTR void gnorm_partials_kernel(const DevTensor *__restrict__ tens,
                                                                  const int32_t *__restrict__ ctab,
                                                                  StepArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t w = blockIdx.x; w < a.ntiles; w += gridDim.x) {
        DevTensor T;
        int64_t e0, len;
        if (!locate_tile(tens, ctab, a, w, T, e0, len)) continue;
        const int64_t slot0 = w * a.tile / kUTile;   // the tile's first partial in the chunk space
        if (len == kGnTile) {
            // a full tile: every load of the wave's kGnUnits units before the sums
            GnRaw<GD> g[kGnUnits];
            load_prio_hi();
#pragma unroll
            for (int u = 0; u < kGnUnits; ++u) gnorm_load_unit<GD>(T.g, e0 + (wave + u * kWaves) * kUTile, lane, g[u]);
            load_prio_lo();
#pragma unroll
            for (int u = 0; u < kGnUnits; ++u) {
                double sq = 0.0;
                uint32_t mx = 0;
                gnorm_acc<GD>(g[u], sq, mx);
                gnorm_store(a, slot0 + wave + u * kWaves, lane, sq, mx);
            }
            continue;
        }
        const int64_t ntile = (len + kUTile - 1) / kUTile;
        const int64_t nfull = len / kUTile;
        for (int64_t tt = wave; tt < ntile; tt += kWaves) {
            double sq = 0.0;
            uint32_t mx = 0;
            if (tt < nfull) {
                GnRaw<GD> g;
                gnorm_load_unit<GD>(T.g, e0 + tt * kUTile, lane, g);
                gnorm_acc<GD>(g, sq, mx);
            } else {   // the tensor's short last unit: elements q*256 + 4*lane + j, one at a time
                for (int q = 0; q < kUTile / 256; ++q) {
                    const int64_t i0 = tt * kUTile + q * 256 + lane * 4;
                    const int n = (int)max((int64_t)0, min((int64_t)4, len - i0));
                    for (int j = 0; j < n; ++j) {
                        const float gv = load_grad1<GD>(T.g, e0 + i0 + j);
                        const double x = (double)gv;
                        sq += x * x;
                        mx = max(mx, fbits(gv) & 0x7FFFFFFFu);
                    }
                }
            }
            gnorm_store(a, slot0 + tt, lane, sq, mx);
        }
    }
}

// Max of doubles in which any NaN wins.
__device__ __forceinline__ double nanmax(double x, double y)
{
    return (x != x || y != y) ? __builtin_nan("") : fmax(x, y);
}

__device__ __forceinline__ double wave_nanmax(double x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = nanmax(x, __shfl_xor(x, off, 64));
    return x;
}

// ---------------------------------------------------------------------------
// Per-tensor sums of the norm partials, in two fixed-order levels so that no
// tensor's sum rests on one workgroup: group j of a tensor holds its partials
// [j*kRGroup, (j+1)*kRGroup) counted from its first; one workgroup sums a
// group (each lane four consecutive partials in order, then the wave
// butterfly, then the waves in order), and one workgroup per tensor then sums
// its groups (strided lanes, butterfly, waves in order).  Which partials meet
// in which order depends on the tensor's length alone.

// MAX: the second value of a pair is combined by a NaN-poisoning max (the
// gradient norm's max |g|), else summed (the update norm's sum of p^2).
template <bool MAX>
__global__ __launch_bounds__(kThreads) void norm_group_kernel(const DevTensor *__restrict__ tens, int ntens,
                                                            int64_t chunk, int64_t ngroups,
                                                            const double *partials, double *groups)
{
    static_assert(kRGroup == 4 * kThreads, "four partials per lane");
    __shared__ double red[kWaves][2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t gid = blockIdx.x; gid < ngroups; gid += gridDim.x) {
        // the tensor holding group gid: the last whose first group is <= gid
        int lo = 0, hi = ntens - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tens[mid].rg_begin <= gid) lo = mid;
            else hi = mid - 1;
        }
        const DevTensor T = tens[lo];
        const int64_t first = T.chunk_begin * (chunk / kUTile);
        const int64_t nt = (T.numel + kUTile - 1) / kUTile;
        const int64_t i0 = (gid - T.rg_begin) * kRGroup + 4 * threadIdx.x;
        const int64_t i1 = min(nt, i0 + 4);
        double a = 0.0, b = 0.0;
        for (int64_t i = i0; i < i1; ++i) {
            a += gld<double>(partials + 2 * (first + i));
            const double y = gld<double>(partials + 2 * (first + i) + 1);
            b = MAX ? nanmax(b, y) : b + y;
        }
        a = wave_sum(a);
        b = MAX ? wave_nanmax(b) : wave_sum(b);
        if (lane == 0) { red[wave][0] = a; red[wave][1] = b; }
        __syncthreads();
        if (threadIdx.x == 0) {
            double A = red[0][0], B = red[0][1];
            for (int w = 1; w < kWaves; ++w) { A += red[w][0]; B = MAX ? nanmax(B, red[w][1]) : B + red[w][1]; }
            gst<double>(groups + 2 * gid, A);
            gst<double>(groups + 2 * gid + 1, B);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void gnorm_reduce_kernel(const DevTensor *__restrict__ tens,
                                                              const double *groups, double *out)
{
    __shared__ double red[kWaves][2];
    const DevTensor T = tens[blockIdx.x];
    const int64_t ng = norm_groups(T.numel);
    double sq = 0.0, mx = 0.0;
    for (int64_t i = threadIdx.x; i < ng; i += kThreads) {
        sq += gld<double>(groups + 2 * (T.rg_begin + i));
        mx = nanmax(mx, gld<double>(groups + 2 * (T.rg_begin + i) + 1));
    }
    sq = wave_sum(sq);
    mx = wave_nanmax(mx);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { red[wave][0] = sq; red[wave][1] = mx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double S = red[0][0], M = red[0][1];
        for (int w = 1; w < kWaves; ++w) { S += red[w][0]; M = nanmax(M, red[w][1]); }
        gst<double>(out + 2 + 2 * (int64_t)T.k, S);
        gst<double>(out + 3 + 2 * (int64_t)T.k, M);
    }
}

// List totals in tensor order (lane-strided, fixed butterfly, waves in
// order) and, if asked, the clipping coefficient.
__global__ __launch_bounds__(kThreads) void gnorm_total_kernel(int64_t n, double *out, float max_norm,
                                                             int norm_type, float *coef)
{
    __shared__ double red[kWaves][2];
    double sq = 0.0, mx = 0.0;
    for (int64_t k = threadIdx.x; k < n; k += kThreads) {
        sq += gld<double>(out + 2 + 2 * k);
        mx = nanmax(mx, gld<double>(out + 3 + 2 * k));
    }
    sq = wave_sum(sq);
    mx = wave_nanmax(mx);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { red[wave][0] = sq; red[wave][1] = mx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double S = red[0][0], M = red[0][1];
        for (int w = 1; w < kWaves; ++w) { S += red[w][0]; M = nanmax(M, red[w][1]); }
        gst<double>(out, S);
        gst<double>(out + 1, M);
        if (coef) {
            const double norm = norm_type == 2 ? sqrt(S) : M;
            const double cf = (double)max_norm / (norm + 1e-6);
            gst<float>(coef, cf != cf ? __builtin_nanf("") : (float)(cf < 1.0 ? cf : 1.0));
        }
    }
}

// ---------------------------------------------------------------------------
// test hooks

__global__ void debug_philox_kernel(uint64_t seed, int64_t t, int32_t k, int64_t j0, int64_t n,
                                    uint32_t *out)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        uint64_t j = (uint64_t)(j0 + i);
        out[i] = philox_word(sr_block(seed, t, k, j >> 2, false), (int)(j & 3));
    }
}

// The BF16 roundings the step kernels store with (gfx950's pair conversions,
// the element's 16 random bits in the high half of the operand).
__global__ void debug_round_kernel(const float *x, const uint32_t *r, uint16_t *out, int64_t n)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t rh = r ? (r[i] & 0xFFFFu) << 16 : 0u;
        out[i] = (uint16_t)((r ? bf16x2_sr_hi(x[i], rh, x[i], rh) : bf16x2_rne(x[i], x[i])) & 0xFFFFu);
    }
}

// For each element: the fast direction, its error bound (infinite where the
// step takes the exact recipe regardless), and the exact recipe's direction.
template <int OPT>
__global__ void debug_direction_kernel(StepArgs a, const float *g, const float *m, const float *v, const float *m2,
                                       float *out, int64_t n)
{
    const Scalars s = call_scalars(a);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float mm2 = OPT == kAdEMAMix ? m2[i] : 0.0f;
        float bu;
        const Mom f = moments_fast<OPT, false>(s, a, g[i], m[i], v[i], mm2, &bu);
        const Mom e = moments<OPT, false>(s, a, g[i], m[i], v[i], mm2);
        out[i] = f.u;
        out[n + i] = a.eps >= 0.0f && fast_ok<OPT>(s, f) ? bu : __builtin_inff();
        out[2 * n + i] = e.u;
    }
}

// codes[i] of x[i] against one codebook's table in LDS.  Inputs in the step's
// fast-path domain (|x| <= 1, normal or zero; for the unsigned table x >= +0)
// take the step's own lookup (q8_code_hi_lds); other inputs the general one.
__global__ void debug_quantize_kernel(QTabs q, int is_signed, const float *x, uint8_t *out, int64_t n)
{
    extern __shared__ uint32_t lds[];
    for (uint32_t i = threadIdx.x; i < q.nwords; i += blockDim.x) lds[i] = q.words[i];
    __syncthreads();
    const QTabParams P = is_signed ? q.s : q.u;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float v = x[i];
        const uint32_t b = fbits(v), a = b & 0x7FFFFFFFu;
        const bool step_domain = a <= 0x3F800000u && (a == 0u || a >= 0x00800000u) && (is_signed || (b >> 31) == 0u);
        uint32_t c;
        if (v != v) c = 0u;
        else if (step_domain) c = (is_signed ? q8_code_hi_lds<true>(v, lds, P) : q8_code_hi_lds<false>(v, lds, P)) >> 24;
        else c = q8_lookup(v, lds, P, is_signed != 0);
        out[i] = (uint8_t)c;
    }
}

// codes[i] = the FP8/FP4 code of x[i] in a block of absmax A (nearest, or
// stochastic with r[i]); decoded[i] = what that code reads back as.
template <class F>
__device__ __forceinline__ void debug_mini_one(float A, float x, const uint32_t *r, int64_t i, uint8_t *codes,
                                               float *decoded)
{
    uint32_t c = 0;
    if (finite_f(A)) {
        const int nsc = mini_enc_shift<F>(A);
        c = r ? mini_encode<F, true>(x, nsc, r[i] & 0xFFFFu) : mini_encode<F, false>(x, nsc, 0u);
    }
    codes[i] = (uint8_t)c;
    decoded[i] = finite_f(A) ? mini_decode<F>(c, mini_dec_shift<F>(A)) : bitsf(0x7FC00000u);
}

__global__ void debug_mini_kernel(int elem, float A, const float *x, const uint32_t *r, uint8_t *codes,
                                  float *decoded, int64_t n)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        if (elem == 0) debug_mini_one<E4M3>(A, x[i], r, i, codes, decoded);
        else if (elem == 1) debug_mini_one<E2M1>(A, x[i], r, i, codes, decoded);
        else debug_mini_one<E2M2U>(A, x[i], r, i, codes, decoded);
    }
}

// codes[i] of x[i] as the step's blockwise encoder forms them: four values of
// a block at a time through mini_pack4 (gfx950's scaled conversions wherever
// the step uses them), one byte per element on output.
template <class F, bool SR>
__device__ __forceinline__ void debug_pack_group(float A, const float *x, const uint32_t *r, uint8_t *codes,
                                                 int64_t g)
{
    float v[4];
    uint32_t rr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[k] = x[4 * g + k];
        rr[k] = SR ? (r[4 * g + k] & 0xFFFFu) : 0u;
    }
    const uint32_t w = mini_pack4<F, SR>(v, A, rr);
    constexpr int W = F::kSign == 0x80u ? 8 : 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) codes[4 * g + k] = (uint8_t)((w >> (W * k)) & ((1u << W) - 1u));
}

__global__ void debug_mini_pack_kernel(int elem, float A, const float *x, const uint32_t *r, uint8_t *codes,
                                       int64_t ngroups)
{
    for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < ngroups;
         g += (int64_t)gridDim.x * blockDim.x) {
        if (elem == 0) r ? debug_pack_group<E4M3, true>(A, x, r, codes, g) : debug_pack_group<E4M3, false>(A, x, r, codes, g);
        else if (elem == 1) r ? debug_pack_group<E2M1, true>(A, x, r, codes, g) : debug_pack_group<E2M1, false>(A, x, r, codes, g);
        else r ? debug_pack_group<E2M2U, true>(A, x, r, codes, g) : debug_pack_group<E2M2U, false>(A, x, r, codes, g);
    }
}

// The standalone rounding cast: n fp32 values to BF16 (BF) or FP16 words,
// nearest-even or stochastic.  Element j's random integer is the low half of
// word j%4 of Philox4x32-10 keyed by the seed, counter (j>>2, j>>34, offset):
// tied to the element, so the grid does not change the result.  Each lane
// takes groups of 4 elements: 128-bit loads, 64-bit stores.
template <bool BF, bool SR>
__device__ __forceinline__ void cast_group(const float v[4], uint16_t *out, int64_t q, int cnt, uint64_t seed,
                                           uint64_t offset)
{
    uint32_t r[4] = {0, 0, 0, 0};
    if (SR) {
        const PhiloxOut w = philox4x32_10((uint32_t)q, (uint32_t)((uint64_t)q >> 32), (uint32_t)offset,
                                          (uint32_t)(offset >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
        r[0] = w.w0 & 0xFFFFu; r[1] = w.w1 & 0xFFFFu; r[2] = w.w2 & 0xFFFFu; r[3] = w.w3 & 0xFFFFu;
    }
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        h[i] = BF ? (SR ? bf16_sr(v[i], r[i]) : bf16_rne(v[i])) : (SR ? f16_sr(v[i], r[i]) : f16_rne(v[i]));
    if (cnt == 4) {
        sst<u2>(out + 4 * q, u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
    } else {
        for (int i = 0; i < cnt; ++i) gst<uint16_t>(out + 4 * q + i, (uint16_t)h[i]);
    }
}

// The standalone rounding cast: n fp32 values to BF16 (BF) or FP16 words,
// nearest-even or stochastic.  Element j's random integer is the low half of
// word j%4 of Philox4x32-10 keyed by the seed, counter (j>>2, j>>34, offset):
// tied to the element, so the grid does not change the result.  Lanes take
// groups of 4 elements (128-bit loads, 64-bit stores), four groups loaded
// before any rounding.
// One workgroup per tile of kCastTile values (kCastGroups groups of four per
// lane), dispatched in order as workgroups retire.
constexpr int kCastGroups = 2;
constexpr int64_t kCastTile = 256 * kCastGroups * 4;

template <bool BF, bool SR>
__global__ __launch_bounds__(256) void round_cast_kernel(const float *__restrict__ x, uint16_t *__restrict__ out,
                                                         int64_t n, uint64_t seed, uint64_t offset)
{
    const int64_t ntiles = (n + kCastTile - 1) / kCastTile;
    for (int64_t w = blockIdx.x; w < ntiles; w += gridDim.x) {
        const int64_t q0 = w * (kCastTile / 4);   // the tile's first group of four
        if ((w + 1) * kCastTile <= n) {
            float v[kCastGroups][4];
            load_prio_hi();
#pragma unroll
            for (int u = 0; u < kCastGroups; ++u) {
                const f4 t = sld<f4>(x + 4 * (q0 + threadIdx.x + u * 256));
                v[u][0] = t.x; v[u][1] = t.y; v[u][2] = t.z; v[u][3] = t.w;
            }
            load_prio_lo();
#pragma unroll
            for (int u = 0; u < kCastGroups; ++u) cast_group<BF, SR>(v[u], out, q0 + threadIdx.x + u * 256, 4, seed, offset);
        } else {   // the short last tile
            for (int64_t q = q0 + threadIdx.x; 4 * q < n; q += 256) {
                const int cnt = (int)min((int64_t)4, n - 4 * q);
                float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (cnt == 4) {
                    const f4 t = sld<f4>(x + 4 * q);
                    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
                } else {
                    for (int i = 0; i < cnt; ++i) v[i] = gld<float>(x + 4 * q + i);
                }
                cast_group<BF, SR>(v, out, q, cnt, seed, offset);
            }
        }
    }
}


// Calibration stream: dst[j][i] = sum_k src[k][i] over fp32 arrays, 4 per
// lane per access, grid-stride.  With nsrc reads and ndst writes it moves the
// same mix of bytes as a step without the arithmetic.
struct StreamArgs {
    const float *src[6];
    float *dst[6];
    int nsrc, ndst;
    int64_t n;   // elements, multiple of 4
};

#ifndef OPT_STREAM_UNROLL
#define OPT_STREAM_UNROLL 4
#endif

__global__ __launch_bounds__(kThreads) void debug_stream_kernel(StreamArgs a)
{
    constexpr int U = OPT_STREAM_UNROLL;
    constexpr int64_t kTileG = (int64_t)kThreads * U;   // groups of four per tile
    const int64_t ng = a.n >> 2;
    const int64_t ntiles = (ng + kTileG - 1) / kTileG;
    for (int64_t w = blockIdx.x; w < ntiles; w += gridDim.x) {
        const int64_t i0 = w * kTileG + threadIdx.x;
        if ((w + 1) * kTileG <= ng) {
            f4 acc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 6; ++k)
                if (k < a.nsrc) {
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[u] += sld<f4>(a.src[k] + 4 * (i0 + u * kThreads));
                }
#pragma unroll
            for (int k = 0; k < 6; ++k)
                if (k < a.ndst) {
#pragma unroll
                    for (int u = 0; u < U; ++u) sst<f4>(a.dst[k] + 4 * (i0 + u * kThreads), acc[u]);
                }
        } else {
            for (int64_t i = i0; i < ng; i += kThreads) {
                f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < 6; ++k)
                    if (k < a.nsrc) acc += sld<f4>(a.src[k] + 4 * i);
#pragma unroll
                for (int k = 0; k < 6; ++k)
                    if (k < a.ndst) sst<f4>(a.dst[k] + 4 * i, acc);
            }
        }
    }
}

hipError_t launch_debug_stream(const float *const *src, int nsrc, float *const *dst, int ndst, int64_t n,
                               const LaunchGeom &lg, hipStream_t st)
{
    StreamArgs a{};
    for (int k = 0; k < nsrc; ++k) a.src[k] = src[k];
    for (int k = 0; k < ndst; ++k) a.dst[k] = dst[k];
    a.nsrc = nsrc;
    a.ndst = ndst;
    a.n = n;
    const int64_t tile_g = (int64_t)kThreads * OPT_STREAM_UNROLL;
    int64_t want = (n / 4 + tile_g - 1) / tile_g;
    if (lg.wgs_per_cu > 0) want = min(want, (int64_t)lg.ncu * lg.wgs_per_cu);
    const unsigned grid = (unsigned)max((int64_t)1, min(want, kMaxGrid));
    // no cap unless one is set (opt_debug_set_wg_cap), to read a capped stream's rate
    hipLaunchKernelGGL(debug_stream_kernel, dim3(grid), dim3(kThreads), cap_lds(lg, 0), st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers (called by opt_api.cpp)

// The update-norm pre-pass over tiles of one 1024-element partial per wave.
constexpr int64_t kUnTile = (int64_t)kWaves * kUTile;

template <class K>
static hipError_t launch_unorm_tiles(K kernel, size_t lds, const LaunchGeom &lg, StepArgs a, hipStream_t st)
{
    set_tiles(a, kUnTile);
    hipLaunchKernelGGL(kernel, dim3(tile_grid(a, lg)), dim3(kThreads), lds, st, a.tens, a.chunk_tensor, a.q.words, a);
    return hipGetLastError();
}

template <int OPT, int GD>
static hipError_t launch_unorm_t(int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    switch (fmt) {
    case kF32: return launch_unorm_tiles(unorm_partials_kernel<OPT, GD, kF32>, 0, lg, a, st);
    case kBF16RN:
    case kBF16SR: return launch_unorm_tiles(unorm_partials_kernel<OPT, GD, kBF16RN>, 0, lg, a, st);
    case kQ8: return launch_unorm_tiles(unorm_partials_kernel<OPT, GD, kQ8>, lds, lg, a, st);
    case kFP8RN:
    case kFP8SR: return launch_unorm_tiles(unorm_partials_kernel<OPT, GD, kFP8RN>, 0, lg, a, st);
    case kFP4RN:
    case kFP4SR: return launch_unorm_tiles(unorm_partials_kernel<OPT, GD, kFP4RN>, 0, lg, a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_unorm(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds,
                        int ntens, double *out, hipStream_t st)
{
    hipError_t e = hipSuccess;
    if (a.nchunks > 0) {
        if (opt == kAdamW) e = gd == kGradF32    ? launch_unorm_t<kAdamW, kGradF32>(fmt, a, lg, lds, st)
                               : gd == kGradBF16 ? launch_unorm_t<kAdamW, kGradBF16>(fmt, a, lg, lds, st)
                                                 : launch_unorm_t<kAdamW, kGradF16>(fmt, a, lg, lds, st);
        else e = gd == kGradF32    ? launch_unorm_t<kAdEMAMix, kGradF32>(fmt, a, lg, lds, st)
                 : gd == kGradBF16 ? launch_unorm_t<kAdEMAMix, kGradBF16>(fmt, a, lg, lds, st)
                                   : launch_unorm_t<kAdEMAMix, kGradF16>(fmt, a, lg, lds, st);
    }
    if (e != hipSuccess) return e;
    if (a.ngroups > 0) {
        hipLaunchKernelGGL(norm_group_kernel<false>, dim3((unsigned)min(a.ngroups, kMaxGrid)), dim3(kThreads), 0, st,
                           a.tens, ntens, a.chunk, a.ngroups, (const double *)a.partials, a.groups);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(unorm_reduce_kernel, dim3(ntens), dim3(kThreads), 0, st, a.tens, (const double *)a.groups, out);
    return hipGetLastError();
}

hipError_t launch_gnorm(int gd, const StepArgs &a, const LaunchGeom &lg, int ntens, double *out, hipStream_t st)
{
    hipError_t e = hipSuccess;
    if (a.nchunks > 0)
        e = gd == kGradF32    ? launch_tiles(gnorm_partials_kernel<kGradF32>, kGnTile, 0, lg, a, st)
            : gd == kGradBF16 ? launch_tiles(gnorm_partials_kernel<kGradBF16>, kGnTile, 0, lg, a, st)
                              : launch_tiles(gnorm_partials_kernel<kGradF16>, kGnTile, 0, lg, a, st);
    if (e != hipSuccess) return e;
    if (a.ngroups > 0) {
        hipLaunchKernelGGL(norm_group_kernel<true>, dim3((unsigned)min(a.ngroups, kMaxGrid)), dim3(kThreads), 0, st,
                           a.tens, ntens, a.chunk, a.ngroups, (const double *)a.partials, a.groups);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gnorm_reduce_kernel, dim3(ntens), dim3(kThreads), 0, st, a.tens, (const double *)a.groups, out);
    return hipGetLastError();
}

hipError_t launch_gnorm_total(int64_t n, double *out, float max_norm, int norm_type, float *coef, hipStream_t st)
{
    hipLaunchKernelGGL(gnorm_total_kernel, dim3(1), dim3(kThreads), 0, st, n, out, max_norm, norm_type, coef);
    return hipGetLastError();
}

hipError_t launch_debug_philox(uint64_t seed, int64_t t, int32_t k, int64_t j0, int64_t n,
                               uint32_t *out, hipStream_t st)
{
    int64_t blocks = min((int64_t)4096, (n + 255) / 256);
    hipLaunchKernelGGL(debug_philox_kernel, dim3((unsigned)max((int64_t)1, blocks)), dim3(256), 0, st,
                       seed, t, k, j0, n, out);
    return hipGetLastError();
}

hipError_t launch_debug_round(const float *x, const uint32_t *r, uint16_t *out, int64_t n, hipStream_t st)
{
    int64_t blocks = min((int64_t)4096, (n + 255) / 256);
    hipLaunchKernelGGL(debug_round_kernel, dim3((unsigned)max((int64_t)1, blocks)), dim3(256), 0, st,
                       x, r, out, n);
    return hipGetLastError();
}

hipError_t launch_debug_direction(int opt, const StepArgs &a, const float *g, const float *m, const float *v,
                                  const float *m2, float *out, int64_t n, hipStream_t st)
{
    int64_t blocks = min((int64_t)4096, (n + 255) / 256);
    if (opt == kAdEMAMix)
        hipLaunchKernelGGL(debug_direction_kernel<kAdEMAMix>, dim3((unsigned)max((int64_t)1, blocks)), dim3(256), 0,
                           st, a, g, m, v, m2, out, n);
    else
        hipLaunchKernelGGL(debug_direction_kernel<kAdamW>, dim3((unsigned)max((int64_t)1, blocks)), dim3(256), 0, st,
                           a, g, m, v, m2, out, n);
    return hipGetLastError();
}

hipError_t launch_round_cast(const float *x, uint16_t *out, int64_t n, int bf16, int sr, uint64_t seed,
                             uint64_t offset, const LaunchGeom &lg, hipStream_t st)
{
    int64_t want = (n + kCastTile - 1) / kCastTile;
    if (lg.wgs_per_cu > 0) want = min(want, (int64_t)lg.ncu * lg.wgs_per_cu);
    const unsigned grid = (unsigned)max((int64_t)1, min(want, kMaxGrid));
    if (bf16) {
        if (sr) hipLaunchKernelGGL((round_cast_kernel<true, true>), dim3(grid), dim3(256), 0, st, x, out, n, seed, offset);
        else hipLaunchKernelGGL((round_cast_kernel<true, false>), dim3(grid), dim3(256), 0, st, x, out, n, seed, offset);
    } else {
        if (sr) hipLaunchKernelGGL((round_cast_kernel<false, true>), dim3(grid), dim3(256), 0, st, x, out, n, seed, offset);
        else hipLaunchKernelGGL((round_cast_kernel<false, false>), dim3(grid), dim3(256), 0, st, x, out, n, seed, offset);
    }
    return hipGetLastError();
}

hipError_t launch_debug_mini(int elem, float A, const float *x, const uint32_t *r, uint8_t *codes, float *decoded,
                             int64_t n, hipStream_t st)
{
    int64_t blocks = min((int64_t)1024, (n + 255) / 256);
    hipLaunchKernelGGL(debug_mini_kernel, dim3((unsigned)max((int64_t)1, blocks)), dim3(256), 0, st, elem, A, x, r,
                       codes, decoded, n);
    return hipGetLastError();
}

hipError_t launch_debug_mini_pack(int elem, float A, const float *x, const uint32_t *r, uint8_t *codes, int64_t n,
                                  hipStream_t st)
{
    const int64_t ng = n / 4;
    int64_t blocks = min((int64_t)1024, (ng + 255) / 256);
    hipLaunchKernelGGL(debug_mini_pack_kernel, dim3((unsigned)max((int64_t)1, blocks)), dim3(256), 0, st, elem, A, x,
                       r, codes, ng);
    return hipGetLastError();
}

hipError_t launch_debug_quantize(const QTabs &q, int is_signed, const float *x, uint8_t *out, int64_t n,
                                 hipStream_t st)
{
    int64_t blocks = min((int64_t)1024, (n + 255) / 256);
    hipLaunchKernelGGL(debug_quantize_kernel, dim3((unsigned)max((int64_t)1, blocks)), dim3(256),
                       (size_t)q.nwords * 4, st, q, is_signed, x, out, n);
    return hipGetLastError();
}

}  // namespace optstep

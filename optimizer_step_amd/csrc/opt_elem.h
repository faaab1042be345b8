// opt_elem.h -- element-group helpers shared by the element-wise kernels
// (two-state and one-state steps): loads and stores of four consecutive
// elements of p, g and a state in their storage formats, and the persistent
// launch shape.
#pragma once

#include <algorithm>

#include "opt_device.h"

namespace optstep {

#ifndef OPT_EW_GROUPS
#define OPT_EW_GROUPS 4
#endif
constexpr int kEwGroups = OPT_EW_GROUPS;   // groups of four in flight per lane

#ifndef OPT_XCD_REMAP
#define OPT_XCD_REMAP 0
#endif

// The chunk a workgroup starts at.  Workgroups are dealt to the 8 XCDs in
// turn; with the remap, the workgroups of one XCD take a contiguous run of
// each round's chunks instead of every 8th chunk.
__device__ __forceinline__ int64_t first_chunk()
{
#if OPT_XCD_REMAP
    const unsigned g = gridDim.x, b = blockIdx.x;
    if (g % 8 == 0) return (int64_t)(b % 8) * (g / 8) + b / 8;
#endif
    return blockIdx.x;
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
// rounded to nearest-even or, with sr, stochastically by the 16-bit r.
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
__device__ __forceinline__ uint32_t round_p(float x, bool sr, uint32_t r)
{
    if (PD == kPBF16) return sr ? bf16_sr(x, r) : bf16_rne(x);
    return sr ? f16_sr(x, r) : f16_rne(x);
}

template <int PD>
__device__ __forceinline__ void store_p4(float *p, int64_t e, const float x[4], bool sr, const uint32_t r[4])
{
    if (PD == kP32) {
        sst<f4>(p + e, f4{x[0], x[1], x[2], x[3]});
    } else {
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = round_p<PD>(x[i], sr, r[i]);
        sst<u2>((uint16_t *)(void *)p + e, u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
    }
}

template <int PD>
__device__ __forceinline__ void store_p1(float *p, int64_t e, float x, bool sr, uint32_t r)
{
    if (PD == kP32) gst<float>(p + e, x);
    else gst<uint16_t>((uint16_t *)(void *)p + e, (uint16_t)round_p<PD>(x, sr, r));
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

// Store four fp32 moments in format SF; r[i] are the 16-bit random integers of
// stochastic rounding (ignored otherwise).
template <int SF>
__device__ __forceinline__ void store_state4(void *s, int64_t e, const float x[4], const uint32_t r[4])
{
    if (SF == kF32) {
        sst<f4>((float *)s + e, f4{x[0], x[1], x[2], x[3]});
    } else {
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = SF == kBF16SR ? bf16_sr(x[i], r[i]) : bf16_rne(x[i]);
        sst<u2>((uint16_t *)s + e, u2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
    }
}

template <int SF>
__device__ __forceinline__ void store_state1(void *s, int64_t e, float x, uint32_t r)
{
    if (SF == kF32) gst<float>((float *)s + e, x);
    else gst<uint16_t>((uint16_t *)s + e, (uint16_t)(SF == kBF16SR ? bf16_sr(x, r) : bf16_rne(x)));
}

// ---------------------------------------------------------------------------
// persistent launches: as many workgroups as fit on the chip at once (the
// kernel's occupancy, or a fixed count per compute unit), never more than
// there are chunks; each walks the chunks with a grid stride.

template <class K>
static int grid_size(K kernel, size_t lds, const LaunchGeom &lg, int64_t nchunks, int threads)
{
    int per_cu = lg.wgs_per_cu;
    if (per_cu <= 0) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, lds) != hipSuccess || occ < 1)
            occ = 1;
        per_cu = occ;
    }
    return (int)std::max<int64_t>(1, std::min<int64_t>(nchunks, (int64_t)lg.ncu * per_cu));
}

template <class K, class... Args>
static hipError_t launch_persistent(K kernel, size_t lds, const LaunchGeom &lg, int64_t nchunks, hipStream_t st,
                                    Args... args)
{
    const int grid = grid_size(kernel, lds, lg, nchunks, kThreads);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, st, args...);
    return hipGetLastError();
}

}  // namespace optstep

// opt_kernels_q8.hip -- gfx950 kernel of the blockwise-state step (8-bit
// codebook, FP8 and FP4 states) for AdamW and AdEMAMix, fp32, BF16 or FP16
// parameters and gradients, and the step's launcher (the element-wise formats
// go to opt_kernels_ew.hip).  Each byte is read or written once per step;
// what bounds each format (its traffic pattern, or the codec's and the
// random generator's VALU work) decides its workgroup shape below.
#include "opt_blk.h"

namespace optstep {

// Workgroup shape and tile of the blockwise kernel, per state format.  A
// wave takes one 256-element block at a time; a tile's blocks go to the
// workgroup's waves in turn.  Measured on MI355X, AdamW over 2^30 elements,
// paired runs in one process:
//  * 8-bit: 512 threads over 32 K-element tiles (one LDS copy of the
//    lookup tables per workgroup, up to 60 KB): 16 K tiles 2.84, 8 K 2.91,
//    4 K 3.14, 2 K 4.06 ms against 2.80.  Smaller one-shot shapes lose
//    even with the table cut to 5 KB (a timing copy whose codes were not
//    the format's): 128 threads over 1 K 3.03, 256 over 2 K 2.76, 512 over
//    4 K 2.74 ms against 2.77.
//  * FP8 and FP4 nearest: 128 threads over 1 K-element tiles, each wave
//    loading its second block while it finishes its first: FP8 2.47 and
//    FP4 2.08 ms against 2.67 and 2.25 with 512 threads over 8 K tiles;
//    256 threads over 2 K tiles 2.51 / 2.13, 64 over 512 2.53 / 2.17.
//  * FP8 stochastic: 128 threads over 2 K-element tiles, four blocks per
//    wave in turn: 2.60-2.66 ms against 2.75 with 512 threads over 8 K;
//    256 over 4 K 2.66, 128 over 1 K 2.73, the prefetching shape 3.04.
//  * FP4 stochastic: 512 threads over 8 K-element tiles; the shapes above
//    land within 2 % either side of it or lose up to 17 %.
//  AdEMAMix over 2^28 elements moves within 1 % with any of these shapes.
template <int SF>
struct Q8Shape {
    static constexpr bool kPrefetch = SF == kFP8RN || SF == kFP4RN;   // a wave loads its next block before finishing this one
    static constexpr bool kSmall = kPrefetch || SF == kFP8SR;
    static constexpr int kThreads = kSmall ? 128 : 512;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int64_t kTile = SF == kQ8 ? 32768 : !kSmall ? 8192 : kPrefetch ? 1024 : 2048;
    static_assert(kTile % (kWaves * kQBlock) == 0, "blockwise tile");
};

// Waves per SIMD the AdamW instantiations are held to (their registers fit
// 7 without spilling; AdEMAMix's third state does not, and is left free).
constexpr int kQ8WavesAdamW = 7;

// The tiles of one workgroup: one 256-element block per wave at a time.
template <int OPT, int GD, int SF, int PD, bool PLAIN>
__device__ __forceinline__ void q8_tiles(const DevTensor *__restrict__ tens, const int32_t *__restrict__ ctab,
                                         const StepArgs &a, const Scalars &s, const uint32_t *lds,
                                         const float *mtab, int lane, int wave)
{
    for (int64_t w = blockIdx.x; w < a.ntiles; w += gridDim.x) {
        DevTensor T;
        int64_t e0, len;
        if (!locate_tile(tens, ctab, a, w, T, e0, len)) continue;
        const float lam = a.unorm ? lam_for(a, T.k) : s.lam;
        const uint32_t nblk = (uint32_t)((len + kQBlock - 1) / kQBlock);
        const uint32_t nfull = (uint32_t)(len / kQBlock);
        const QChunk C = q8_chunk<GD, SF, PD>(T, e0);
        uint32_t b = wave;
        if (Q8Shape<SF>::kPrefetch) {
            // the wave's next block is loaded while it finishes this one
            QIn xa;
            if (b < nfull) {
                load_prio_hi();
                q8_load<OPT, GD, SF, PD, true>(a, C, b, 4, lane, xa);
                load_prio_lo();
            }
            while (b < nfull) {
                const uint32_t bn = b + Q8Shape<SF>::kWaves;
                const bool more = bn < nfull;
                QIn xb;
                if (more) {
                    load_prio_hi();
                    q8_load<OPT, GD, SF, PD, true>(a, C, bn, 4, lane, xb);
                    load_prio_lo();
                }
                q8_finish<OPT, SF, PD, true, PLAIN>(a, s, C, lds, mtab, b, 4, lane, lam, xa);
                b = bn;
                if (more) xa = xb;
            }
        } else {
            for (; b < nfull; b += Q8Shape<SF>::kWaves) {
                QIn x0;
                load_prio_hi();
                q8_load<OPT, GD, SF, PD, true>(a, C, b, 4, lane, x0);
                load_prio_lo();
                q8_finish<OPT, SF, PD, true, PLAIN>(a, s, C, lds, mtab, b, 4, lane, lam, x0);
            }
        }
        if (b < nblk) {   // the tensor's short last block
            const int nm = q8_mine(T, e0 + (int64_t)b * kQBlock, lane);
            QIn x0;
            q8_load<OPT, GD, SF, PD, false>(a, C, b, nm, lane, x0);
            q8_finish<OPT, SF, PD, false, PLAIN>(a, s, C, lds, mtab, b, nm, lane, lam, x0);
        }
    }
}

// Blockwise states (8-bit codebook, FP8, FP4): one workgroup per tile (the
// tile scheduling of opt_elem.h).
template <int OPT, int GD, int SF, int PD, bool PLAIN>
__global__ __launch_bounds__(Q8Shape<SF>::kThreads)
__attribute__((amdgpu_waves_per_eu(OPT == kAdamW ? kQ8WavesAdamW : 1))) void step_q8_kernel(const DevTensor *__restrict__ tens,
                                                             const int32_t *__restrict__ ctab,
                                                             const uint32_t *__restrict__ qwords,
                                                             StepArgs a)
{
    extern __shared__ uint32_t lds[];
    __shared__ float mtab_s[mini_fmt(SF) ? kMiniTab : 1];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (SF == kQ8)
        for (uint32_t i = threadIdx.x; i < a.q.nwords; i += Q8Shape<SF>::kThreads) lds[i] = qwords[i];
    if (mini_fmt(SF)) fill_mini_tab<SF>(mtab_s, threadIdx.x, Q8Shape<SF>::kThreads);
    const float *mtab = mini_fmt(SF) ? mtab_s : nullptr;
    __syncthreads();
    const Scalars s = call_scalars(a);
    q8_tiles<OPT, GD, SF, PD, PLAIN>(tens, ctab, a, s, lds, mtab, lane, wave);
}

// ---------------------------------------------------------------------------
// launchers (called by opt_api.cpp)

// The blockwise step of state format SF over its tiles (opt_elem.h).
template <int SF, class K>
static hipError_t launch_q8_tiles(K kernel, size_t lds, const LaunchGeom &lg, StepArgs a, hipStream_t st)
{
    set_tiles(a, Q8Shape<SF>::kTile);
    hipLaunchKernelGGL(kernel, dim3(tile_grid(a, lg)), dim3(Q8Shape<SF>::kThreads), lds, st, a.tens,
                       a.chunk_tensor, a.q.words, a);
    return hipGetLastError();
}

hipError_t launch_step_ew(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st);

template <int OPT, int GD, int PD, bool PLAIN>
static hipError_t launch_q8_pl(int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    switch (fmt) {
    case kQ8: return launch_q8_tiles<kQ8>(step_q8_kernel<OPT, GD, kQ8, PD, PLAIN>, lds, lg, a, st);
    case kFP8RN: return launch_q8_tiles<kFP8RN>(step_q8_kernel<OPT, GD, kFP8RN, PD, PLAIN>, 0, lg, a, st);
    case kFP8SR: return launch_q8_tiles<kFP8SR>(step_q8_kernel<OPT, GD, kFP8SR, PD, PLAIN>, 0, lg, a, st);
    case kFP4RN: return launch_q8_tiles<kFP4RN>(step_q8_kernel<OPT, GD, kFP4RN, PD, PLAIN>, 0, lg, a, st);
    case kFP4SR: return launch_q8_tiles<kFP4SR>(step_q8_kernel<OPT, GD, kFP4SR, PD, PLAIN>, 0, lg, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <int OPT, int GD, int PD>
static hipError_t launch_q8_pd(int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    return plain_call(a) ? launch_q8_pl<OPT, GD, PD, true>(fmt, a, lg, lds, st)
                         : launch_q8_pl<OPT, GD, PD, false>(fmt, a, lg, lds, st);
}

// This translation unit holds the kernels for one parameter storage,
// OPT_Q8_PD (0 fp32, 1 BF16, 2 FP16); the library compiles it once for each,
// and the fp32 unit also holds the step's dispatcher.
#ifndef OPT_Q8_PD
#define OPT_Q8_PD 0
#endif
#define OPT_Q8_FN_(pd) launch_step_q8_p##pd
#define OPT_Q8_FN(pd) OPT_Q8_FN_(pd)

hipError_t OPT_Q8_FN(OPT_Q8_PD)(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds,
                                 hipStream_t st)
{
    constexpr int PD = OPT_Q8_PD;
    if (opt == kAdamW) {
        switch (gd) {
        case kGradF32: return launch_q8_pd<kAdamW, kGradF32, PD>(fmt, a, lg, lds, st);
        case kGradBF16: return launch_q8_pd<kAdamW, kGradBF16, PD>(fmt, a, lg, lds, st);
        case kGradF16: return launch_q8_pd<kAdamW, kGradF16, PD>(fmt, a, lg, lds, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (gd) {
    case kGradF32: return launch_q8_pd<kAdEMAMix, kGradF32, PD>(fmt, a, lg, lds, st);
    case kGradBF16: return launch_q8_pd<kAdEMAMix, kGradBF16, PD>(fmt, a, lg, lds, st);
    case kGradF16: return launch_q8_pd<kAdEMAMix, kGradF16, PD>(fmt, a, lg, lds, st);
    default: return hipErrorInvalidValue;
    }
}

#if OPT_Q8_PD == 0
hipError_t launch_step_q8_p1(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds,
                             hipStream_t st);
hipError_t launch_step_q8_p2(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds,
                             hipStream_t st);

hipError_t launch_step(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    if (!blocked(fmt)) return launch_step_ew(opt, gd, fmt, a, lg, st);
    switch (a.p_dtype) {
    case kP32: return launch_step_q8_p0(opt, gd, fmt, a, lg, lds, st);
    case kPBF16: return launch_step_q8_p1(opt, gd, fmt, a, lg, lds, st);
    case kPF16: return launch_step_q8_p2(opt, gd, fmt, a, lg, lds, st);
    default: return hipErrorInvalidValue;
    }
}
#endif

}  // namespace optstep

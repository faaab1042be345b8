// opt_kernels_q8.hip -- gfx950 kernel of the blockwise-state step (8-bit
// codebook, FP8 and FP4 states) for AdamW and AdEMAMix, fp32, BF16 or FP16
// parameters and gradients, and the step's launcher (the element-wise formats
// go to opt_kernels_ew.hip).  HBM-bound, with the codecs' VALU work close
// behind: each byte is read or written once per step.
#include "opt_blk.h"

namespace optstep {

#ifndef OPT_Q8_THREADS
#define OPT_Q8_THREADS 512
#endif
// Workgroup size of the blockwise kernel (one LDS copy of the 8-bit tables
// per workgroup).
constexpr int kQ8Threads = OPT_Q8_THREADS;
constexpr int kQ8Waves = kQ8Threads / 64;

#ifndef OPT_Q8_TILE
#define OPT_Q8_TILE 32768
#endif
// Elements per tile of the blockwise step (a power of two, a multiple of the
// 8 x 256 elements one pass of the workgroup's waves covers).
constexpr int64_t kQ8Tile = OPT_Q8_TILE;
static_assert(kQ8Tile % (kQ8Waves * kQBlock) == 0, "blockwise tile");

#ifndef OPT_MINI_TILE
#define OPT_MINI_TILE 8192
#endif
// Elements per tile of the FP8/FP4 formats, which load no lookup table: four
// passes of the workgroup's waves.  Measured on MI355X, FP8 nearest: 8 K and
// 4 K tiles 2.70 ms, 16 K 2.83 ms, 32 K 2.80 ms, 2 K 3.09 ms per 2^30
// elements; the 8-bit format, whose tables every workgroup copies into LDS,
// keeps 32 K (16 K 2.84, 8 K 2.91, 4 K 3.14, 2 K 4.06 ms against 2.80).
constexpr int64_t kMiniTile = OPT_MINI_TILE;
static_assert(kMiniTile % (kQ8Waves * kQBlock) == 0, "blockwise tile");

#ifndef OPT_Q8_PREFETCH
#define OPT_Q8_PREFETCH (-1)
#endif
// Whether a wave loads its next block before finishing the current one
// (OPT_Q8_PREFETCH: -1 per format, 0 never, 1 always).
constexpr bool q8_prefetch(int sf) { return sf == kFP8RN || sf == kFP4RN; }

#ifndef OPT_Q8_WAVES
#define OPT_Q8_WAVES 7
#endif
// Waves per SIMD the AdamW instantiations are held to (their registers fit
// 7 without spilling; AdEMAMix's third state does not, and is left free).
constexpr int kQ8WavesAdamW = OPT_Q8_WAVES;

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
        if (OPT_Q8_PREFETCH < 0 ? q8_prefetch(SF) : OPT_Q8_PREFETCH != 0) {
            // the wave's next block is loaded while it finishes this one
            QIn xa;
            if (b < nfull) {
                load_prio_hi();
                q8_load<OPT, GD, SF, PD, true>(a, C, b, 4, lane, xa);
                load_prio_lo();
            }
            while (b < nfull) {
                const uint32_t bn = b + kQ8Waves;
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
            for (; b < nfull; b += kQ8Waves) {
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
__global__ __launch_bounds__(kQ8Threads)
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
        for (uint32_t i = threadIdx.x; i < a.q.nwords; i += kQ8Threads) lds[i] = qwords[i];
    if (mini_fmt(SF)) fill_mini_tab<SF>(mtab_s, threadIdx.x, kQ8Threads);
    const float *mtab = mini_fmt(SF) ? mtab_s : nullptr;
    __syncthreads();
    const Scalars s = call_scalars(a);
    q8_tiles<OPT, GD, SF, PD, PLAIN>(tens, ctab, a, s, lds, mtab, lane, wave);
}

// ---------------------------------------------------------------------------
// launchers (called by opt_api.cpp)

// The blockwise step over tiles of `tile` elements (opt_elem.h).
template <class K>
static hipError_t launch_q8_tiles(K kernel, size_t lds, const LaunchGeom &lg, StepArgs a, hipStream_t st,
                                  int64_t tile = kQ8Tile)
{
    set_tiles(a, tile);
    hipLaunchKernelGGL(kernel, dim3(tile_grid(a, lg)), dim3(kQ8Threads), lds, st, a.tens, a.chunk_tensor,
                       a.q.words, a);
    return hipGetLastError();
}

hipError_t launch_step_ew(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st);

template <int OPT, int GD, int PD, bool PLAIN>
static hipError_t launch_q8_pl(int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    switch (fmt) {
    case kQ8: return launch_q8_tiles(step_q8_kernel<OPT, GD, kQ8, PD, PLAIN>, lds, lg, a, st);
    case kFP8RN: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP8RN, PD, PLAIN>, 0, lg, a, st, kMiniTile);
    case kFP8SR: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP8SR, PD, PLAIN>, 0, lg, a, st, kMiniTile);
    case kFP4RN: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP4RN, PD, PLAIN>, 0, lg, a, st, kMiniTile);
    case kFP4SR: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP4SR, PD, PLAIN>, 0, lg, a, st, kMiniTile);
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

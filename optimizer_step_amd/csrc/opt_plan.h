// opt_plan.h -- records shared by the host planner (opt_api.cpp) and the
// kernels (opt_kernels.hip).  Plain data only.
#pragma once

#include <stdint.h>

namespace optstep {

constexpr int kThreads = 256;      // threads per workgroup (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kQBlock = 256;       // elements per 8-bit absmax block
constexpr int kUTile = 1024;       // elements per norm partial (update norm, gradient norm)
constexpr int kRGroup = 1024;      // partials per first-level group of the per-tensor norm sums

enum Opt : int { kAdamW = 0, kAdEMAMix = 1, kMomentum = 2, kRMSprop = 3, kAdagrad = 4, kLion = 5 };
enum Fmt : int { kF32 = 0, kBF16RN = 1, kBF16SR = 2, kQ8 = 3, kFP8RN = 4, kFP8SR = 5, kFP4RN = 6, kFP4SR = 7 };

// Formats stored as blocks of 256 codes with one fp32 absmax per block.
constexpr bool blocked(int f) { return f >= kQ8; }
constexpr bool fp4_fmt(int f) { return f == kFP4RN || f == kFP4SR; }
constexpr bool mini_fmt(int f) { return f >= kFP8RN; }
constexpr bool sr_fmt(int f) { return f == kBF16SR || f == kFP8SR || f == kFP4SR; }
enum GradT : int { kGradF32 = 0, kGradBF16 = 1, kGradF16 = 2 };   // gradient storage
enum ParamT : int { kP32 = 0, kPBF16 = 1, kPF16 = 2 };             // parameter storage

// One tensor of a dtype bucket, as the kernels see it (device memory).
struct alignas(16) DevTensor {
    float *p;              // fp32, or 16-bit words for BF16/FP16 parameters
    const void *g;
    void *s1, *s2, *s3;
    float *a1, *a2, *a3;
    int64_t numel;
    int64_t chunk_begin;   // first chunk of this tensor in the bucket's chunk space
    int32_t k;             // position in the caller's list (norm output slot)
    uint32_t rk;           // tensor number of the stochastic-rounding counter
    int64_t rg_begin;      // first norm-sum group of this tensor in the bucket (groups of kRGroup partials)
    int64_t jbase;         // element index of element 0 within the whole tensor (stochastic rounding)
    int64_t pad_;
};
static_assert(sizeof(DevTensor) == 112, "DevTensor layout");

// Norm-sum groups of a tensor of numel elements: kRGroup partials of kUTile
// elements each, the last group possibly short.
constexpr int64_t norm_groups(int64_t numel) { return ((numel + kUTile - 1) / kUTile + kRGroup - 1) / kRGroup; }

// 8-bit codebook lookup-table parameters (see build_search in opt_api.cpp).
// For |x| <= 1 the magnitude bits a = bits(max(|x|, lo_f)) give the bucket
// b = (a - lo) >> shift and the in-bucket key k = (a - lo) & mask (shift is
// at most 17, so k < 2^17).  An unsigned table holds one entry per bucket; a
// signed table two, interleaved: entry 2b for x > 0, 2b + 1 for x <= 0.  An
// entry E carries the code in its top byte after one 32-bit add:
// code = (E + k) >> 24 for x > 0 and (E + ~k) >> 24 for x <= 0, i.e. the
// bucket's base code plus one when k is past the bucket's threshold.
struct QTabParams {
    uint32_t lo;       // bit pattern of the smallest magnitude kept apart
    uint32_t shift;    // log2 of the bucket width in ulps
    uint32_t nb;       // buckets per sign
    uint32_t offset;   // first entry of this table in the packed search area (words)
};

// Packed 8-bit tables in device memory and LDS (32-bit words):
//   [0, 256)          signed codebook values (m, m2)
//   [256, 512)        unsigned codebook values (v)
//   [512, ...)        search entries: signed table (2*nb) then unsigned (nb)
struct QTabs {
    const uint32_t *words;   // device
    uint32_t nwords;
    QTabParams s, u;
};

// Launch geometry: compute units, workgroups per compute unit (0: one
// workgroup per tile; k > 0: a persistent grid of k per compute unit), and
// the cap on workgroups resident per compute unit of the element-wise tile
// kernels (-1: each kernel's own choice; 0: none; k: at most k).
struct LaunchGeom {
    int ncu;
    int wgs_per_cu;
    int wg_cap = -1;
};

// Per-call scalars of the two-state steps, formed once by the host
// (make_scalars) in the order the element recipe expects; the gradient scale
// is read from device memory by the kernels.
struct Scalars {
    float om1, om2, om3;   // 1 - beta
    float c1, c2;          // 1 - beta^t, formed in binary64 and rounded once
    float rc1, rc2;        // RN(1/c1), RN(1/c2)
    float d;               // 1 - lr*wd
    float lam;             // lr (the update-norm scale is applied per tensor)
    float gs;              // gradient scale (a clipping coefficient), 1 if none
};

// Kernel arguments (passed by value).
struct StepArgs {
    const DevTensor *tens;
    const int32_t *chunk_tensor;   // bucket-local tensor of each chunk
    int64_t nchunks;
    int64_t chunk;                 // elements per chunk (multiple of 1024)
    const double *unorm;           // caller's {sum u^2, sum p^2} per tensor k, or null
    double *partials;              // norm passes: {sum u^2, sum p^2} or {sum g^2, max |g|} per kUTile elements
    double *groups;                // norm passes: the same pairs summed over groups of kRGroup partials
    int64_t ngroups;               // groups in the bucket
    QTabs q;
    float lr, beta1, beta2, beta3, alpha, eps, wd, max_unorm;
    int64_t step;                  // t: keys the stochastic-rounding stream
    int64_t bc_step;               // steps since the moments last started from zero
    int32_t fresh;                 // 1: this step starts the moments from zero (a reset)
    uint64_t seed;
    const float *grad_scale;       // device float or null (1)
    int32_t p_dtype;               // ParamT of the bucket's parameters
    int32_t p_sr;                  // 1: 16-bit parameters are stored with stochastic rounding
    int32_t skip_zeros;            // 1: elements whose gradient is exactly 0 keep p and their states
    Scalars sc;                    // make_scalars of these arguments (gs = 1)
    // tile space of the launch (set by the launcher from the kernel's tile):
    // chunk c holds tiles [c << tile_sh, (c + 1) << tile_sh) of tile elements each
    int64_t tile;
    int64_t ntiles;
    int32_t tile_sh;
};

}  // namespace optstep

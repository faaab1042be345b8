// opt_kernels.hip -- gfx950 kernels of the blockwise-state step (8-bit
// codebook, FP8 and FP4 states), the deterministic update-norm pre-pass, the
// fused multi-tensor gradient norm, the standalone rounding cast and the test
// hooks.  (The element-wise two-state step is in opt_kernels_ew.hip, the
// one-state optimizers in opt_kernels_1s.hip.)
//
// The blockwise formats hand one 256-element block to one wave (64 lanes x 4
// consecutive elements), which makes the block absmax a wave reduction; codes
// move as 32-bit (8-bit formats) or 16-bit (FP4) accesses per lane, fully
// coalesced.  Every kernel here is HBM-bound or close to it (no dense
// contraction, so no MFMA): each byte is read or written once per call.
#include "opt_elem.h"

namespace optstep {

// ---------------------------------------------------------------------------
// 8-bit blockwise states

// Codes of this lane's four fp32 moments against their block absmax A (a
// wave-uniform value).  When A and 1/A are normal and no moment of the wave is
// a nonzero value below 2^-100, div_by gives the correctly rounded x = m'/A
// (|x| <= 1); otherwise x = 0 for A = 0, else the correctly rounded m'/A, and
// a NaN quotient (A NaN or infinite) gets code 0.
template <bool SIGNED>
__device__ __forceinline__ uint32_t quant4(const float x[4], float A, const uint32_t *lds, const QTabParams &P)
{
    uint32_t out = 0;
    bool tiny = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) tiny |= (fbits(x[i]) & 0x7FFFFFFFu) - 1u < 0x0D7FFFFFu;   // 0 < |x| < 2^-100
    if (div_by_ok(A) && !__any(tiny)) {
        const float y = 1.0f / A;
#pragma unroll
        for (int i = 0; i < 4; ++i) out |= q8_code(div_by(x[i], A, y), lds, P, SIGNED) << (8 * i);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float q = A == 0.0f ? 0.0f : x[i] / A;
            out |= (q != q ? 0u : q8_lookup(q, lds, P, SIGNED)) << (8 * i);
        }
    }
    return out;
}

// The block absmax from this lane's four values: max |x| as unsigned bit
// patterns across the wave, so NaN poisons it.  Values of lanes past the end
// of a short block are passed as 0.
__device__ __forceinline__ float block_absmax(const float x[4])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, fbits(x[i]) & 0x7FFFFFFFu);
    return bitsf(wave_max_u32(m));
}

// One chunk's arrays, offset to the chunk's first element (absmax to its
// first block): wave-uniform base pointers, indexed with 32-bit offsets.
struct QChunk {
    float *p;
    const uint8_t *g;      // bytes
    uint8_t *s1, *s2, *s3; // bytes (FP4: two elements per byte)
    float *a1, *a2, *a3;
    int64_t e0;            // the chunk's first element within its whole tensor (index_base included)
    int32_t k;             // the tensor number of its stochastic-rounding stream
};

template <int GD, int SF>
__device__ __forceinline__ QChunk q8_chunk(const DevTensor &T, int64_t e0)
{
    const int64_t sb = fp4_fmt(SF) ? e0 / 2 : e0;
    QChunk c;
    c.p = T.p + e0;
    c.g = (const uint8_t *)T.g + e0 * (GD == kGradF32 ? 4 : 2);   // bytes per gradient
    c.s1 = (uint8_t *)T.s1 + sb;
    c.s2 = (uint8_t *)T.s2 + sb;
    c.s3 = (uint8_t *)T.s3 + sb;
    c.a1 = T.a1 + e0 / kQBlock;
    c.a2 = T.a2 + e0 / kQBlock;
    c.a3 = T.a3 + e0 / kQBlock;
    c.e0 = T.jbase + e0;
    c.k = (int32_t)T.rk;
    return c;
}

// One lane's four elements of a 256-element block, as loaded.  Codes are
// packed in element order: 8 bits each, or 4 bits each for FP4.
struct QIn {
    float p[4], g[4];
    uint32_t cm, cv, cm2;
    float A1, A2, A3;
};

// Four codes of one state at element e (a multiple of 4) of the chunk.
template <int SF, bool FULL>
__device__ __forceinline__ uint32_t load_codes(const uint8_t *s, uint32_t e, int nmine)
{
    if (fp4_fmt(SF)) {
        if (FULL || nmine == 4) return sld<uint16_t>(s + e / 2);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; i += 2)
            if (i < nmine) c |= (uint32_t)gld<uint8_t>(s + e / 2 + i / 2) << (4 * i);
        return nmine & 1 ? c & ~(0xFu << (4 * nmine)) : c;
    }
    if (FULL || nmine == 4) return sld<uint32_t>(s + e);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < nmine) c |= (uint32_t)gld<uint8_t>(s + e + i) << (8 * i);
    return c;
}

template <int SF, bool FULL>
__device__ __forceinline__ void store_codes(uint8_t *s, uint32_t e, int nmine, uint32_t c)
{
    if (fp4_fmt(SF)) {
        if (FULL || nmine == 4) { sst<uint16_t>(s + e / 2, (uint16_t)c); return; }
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            if (i < nmine) {
                // past an odd tensor's last element the high nibble is 0
                const uint32_t hi = i + 1 < nmine ? (c >> (4 * i + 4)) & 0xFu : 0u;
                gst<uint8_t>(s + e / 2 + i / 2, (uint8_t)(((c >> (4 * i)) & 0xFu) | (hi << 4)));
            }
        }
        return;
    }
    if (FULL || nmine == 4) { sst<uint32_t>(s + e, c); return; }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < nmine) gst<uint8_t>(s + e + i, (uint8_t)(c >> (8 * i)));
}

// Block b of the chunk (elements 256*b ..); lanes own 4 elements each.  A
// step that starts the moments from zero reads no state.
template <int OPT, int GD, int SF, bool FULL>
__device__ __forceinline__ void q8_load(const StepArgs &a, const QChunk &C, uint32_t b, int nmine, int lane,
                                        QIn &x)
{
    if (FULL) nmine = 4;
    const uint32_t e = b * kQBlock + lane * 4;
    if (nmine == 4) {
        f4 pv = sld<f4>(C.p + e);
        x.p[0] = pv.x; x.p[1] = pv.y; x.p[2] = pv.z; x.p[3] = pv.w;
        if (GD == kGradF32) {
            f4 gv = sld<f4>(C.g + 4 * e);
            x.g[0] = gv.x; x.g[1] = gv.y; x.g[2] = gv.z; x.g[3] = gv.w;
        } else {
            widen4<GD == kGradBF16>(sld<u2>(C.g + 2 * e), x.g);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x.p[i] = 0.0f;
            x.g[i] = 0.0f;
            if (i < nmine) {
                x.p[i] = gld<float>(C.p + e + i);
                x.g[i] = GD == kGradF32    ? gld<float>(C.g + 4 * (e + i))
                         : GD == kGradBF16 ? bf16_lo(gld<uint16_t>(C.g + 2 * (e + i)))
                                           : f16_lo(gld<uint16_t>(C.g + 2 * (e + i)));
            }
        }
    }
    x.cm = x.cv = x.cm2 = 0;
    x.A1 = x.A2 = x.A3 = 0.0f;
    if (!a.fresh) {
        x.cm = load_codes<SF, FULL>(C.s1, e, nmine);
        x.cv = load_codes<SF, FULL>(C.s2, e, nmine);
        if (OPT == kAdEMAMix) x.cm2 = load_codes<SF, FULL>(C.s3, e, nmine);
        x.A1 = gld<float>(C.a1 + b);
        x.A2 = gld<float>(C.a2 + b);
        if (OPT == kAdEMAMix) x.A3 = gld<float>(C.a3 + b);
    }
}

// Four stored values of one state.  WHICH: 0 = m, 1 = v, 2 = m2.
// Grid values of every FP8/FP4 code (scale 1), one copy per workgroup in LDS:
// E4M3 codes 0..255, or E2M1 codes 0..15 then unsigned E2M2 codes 0..15.
constexpr int kMiniTab = 256;

template <int SF>
__device__ __forceinline__ void fill_mini_tab(float *tab, int tid, int nthreads)
{
    for (int i = tid; i < (fp4_fmt(SF) ? 32 : 256); i += nthreads)
        tab[i] = fp4_fmt(SF) ? (i < 16 ? mini_decode<E2M1>((uint32_t)i, 0) : mini_decode<E2M2U>((uint32_t)(i - 16), 0))
                             : mini_decode<E4M3>((uint32_t)i, 0);
}

// Four stored values of one state.  WHICH: 0 = m, 1 = v, 2 = m2.  FP8/FP4
// codes read their grid value from `mtab` (fill_mini_tab) when it is given,
// else decode it arithmetically; either way value(code) * 2^(floor(log2 A) -
// emax) rounded to binary32.
template <int SF, int WHICH>
__device__ __forceinline__ void blk_decode4(const uint32_t *lds, uint32_t c, float A, float out[4],
                                            const float *mtab = nullptr)
{
    if (SF == kQ8) {
        const float *tab = (const float *)lds + (WHICH == 1 ? 256 : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = tab[(c >> (8 * i)) & 0xFFu] * A;
    } else if (fp4_fmt(SF) && WHICH == 1) {
        const int sc = mini_dec_shift<E2M2U>(A);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = mtab ? ldexpf(mtab[16 + ((c >> (4 * i)) & 0xFu)], sc) : mini_decode<E2M2U>((c >> (4 * i)) & 0xFu, sc);
    } else if (fp4_fmt(SF)) {
        const int sc = mini_dec_shift<E2M1>(A);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = mtab ? ldexpf(mtab[(c >> (4 * i)) & 0xFu], sc) : mini_decode<E2M1>((c >> (4 * i)) & 0xFu, sc);
    } else {
        const int sc = mini_dec_shift<E4M3>(A);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = mtab ? ldexpf(mtab[(c >> (8 * i)) & 0xFFu], sc) : mini_decode<E4M3>((c >> (8 * i)) & 0xFFu, sc);
    }
    if (mini_fmt(SF) && !finite_f(A)) {          // a poisoned block reads as NaN
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = bitsf(0x7FC00000u);
    }
}

template <class F, bool SR>
__device__ __forceinline__ uint32_t mini_pack4(const float x[4], float A, const uint32_t r[4])
{
    if (!finite_f(A)) return 0u;
    const int nsc = mini_enc_shift<F>(A);
    constexpr int W = (F::kSign == 0x80u) ? 8 : 4;
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) out |= mini_encode<F, SR>(x[i], nsc, r[i]) << (W * i);
    return out;
}

template <int SF, int WHICH>
__device__ __forceinline__ uint32_t blk_encode4(const uint32_t *lds, const StepArgs &a, const float x[4], float A,
                                                const uint32_t r[4])
{
    constexpr bool SR = sr_fmt(SF);
    if (SF == kQ8) return WHICH == 1 ? quant4<false>(x, A, lds, a.q.u) : quant4<true>(x, A, lds, a.q.s);
    if (fp4_fmt(SF)) return WHICH == 1 ? mini_pack4<E2M2U, SR>(x, A, r) : mini_pack4<E2M1, SR>(x, A, r);
    return mini_pack4<E4M3, SR>(x, A, r);
}

// FULL: every lane holds four elements (all blocks but a tensor's short last one).
template <int OPT, int SF, bool FULL>
__device__ __forceinline__ void q8_finish(const StepArgs &a, const Scalars &s, const QChunk &C,
                                          const uint32_t *lds, const float *mtab, uint32_t b, int nmine,
                                          int lane, float lam, const QIn &x)
{
    if (FULL) nmine = 4;
    const uint32_t e = b * kQBlock + lane * 4;
    float m_in[4], v_in[4], m2_in[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    blk_decode4<SF, 0>(lds, x.cm, x.A1, m_in, mtab);
    blk_decode4<SF, 1>(lds, x.cv, x.A2, v_in, mtab);
    if (OPT == kAdEMAMix) blk_decode4<SF, 2>(lds, x.cm2, x.A3, m2_in, mtab);
    if (a.fresh) {
#pragma unroll
        for (int i = 0; i < 4; ++i) m_in[i] = v_in[i] = m2_in[i] = 0.0f;
    }
    // The stored moments are exact binary32; only the direction u (for p)
    // takes the fast path, unless some v_hat in the wave is tiny or NaN.
    float p[4], mo[4], vo[4], m2o[4];
    float vmin = 1.0f;
    Mom r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = moments_fast<OPT>(s, a, x.g[i], m_in[i], v_in[i], m2_in[i]);
        vmin = fminf(vmin, r[i].v * s.rc2);
    }
    if (__any(!(vmin >= 0x1p-96f))) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = moments<OPT>(s, a, x.g[i], m_in[i], v_in[i], m2_in[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool valid = i < nmine;
        const bool skip = a.skip_zeros && x.g[i] == 0.0f;   // keep p; code the old moments again
        p[i] = skip ? x.p[i] : apply_update(x.p[i], s.d, lam, r[i].u);
        mo[i] = valid ? (skip ? m_in[i] : r[i].m) : 0.0f;
        vo[i] = valid ? (skip ? v_in[i] : r[i].v) : 0.0f;
        m2o[i] = valid ? (skip ? m2_in[i] : r[i].m2) : 0.0f;
    }
    // stochastic rounding: the element's Philox word, low half for m, high
    // half for v, low half of the second stream's word for m2
    uint32_t rm[4] = {0, 0, 0, 0}, rv[4] = {0, 0, 0, 0}, rm2[4] = {0, 0, 0, 0};
    if (sr_fmt(SF)) {
        const uint64_t q = (uint64_t)(C.e0 + e) >> 2;
        PhiloxOut w = sr_block(a.seed, a.step, C.k, q, false);
        rm[0] = w.w0 & 0xFFFFu; rm[1] = w.w1 & 0xFFFFu; rm[2] = w.w2 & 0xFFFFu; rm[3] = w.w3 & 0xFFFFu;
        rv[0] = w.w0 >> 16; rv[1] = w.w1 >> 16; rv[2] = w.w2 >> 16; rv[3] = w.w3 >> 16;
        if (OPT == kAdEMAMix) {
            PhiloxOut w2 = sr_block(a.seed, a.step, C.k, q, true);
            rm2[0] = w2.w0 & 0xFFFFu; rm2[1] = w2.w1 & 0xFFFFu; rm2[2] = w2.w2 & 0xFFFFu; rm2[3] = w2.w3 & 0xFFFFu;
        }
    }
    const float Am = block_absmax(mo), Av = block_absmax(vo);
    const uint32_t om = blk_encode4<SF, 0>(lds, a, mo, Am, rm);
    const uint32_t ov = blk_encode4<SF, 1>(lds, a, vo, Av, rv);
    uint32_t om2 = 0;
    float Am2 = 0.0f;
    if (OPT == kAdEMAMix) {
        Am2 = block_absmax(m2o);
        om2 = blk_encode4<SF, 2>(lds, a, m2o, Am2, rm2);
    }
    if (nmine == 4) {
        sst<f4>(C.p + e, f4{p[0], p[1], p[2], p[3]});
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < nmine) gst<float>(C.p + e + i, p[i]);
    }
    store_codes<SF, FULL>(C.s1, e, nmine, om);
    store_codes<SF, FULL>(C.s2, e, nmine, ov);
    if (OPT == kAdEMAMix) store_codes<SF, FULL>(C.s3, e, nmine, om2);
    if (lane == 0) {
        gst<float>(C.a1 + b, Am);
        gst<float>(C.a2 + b, Av);
        if (OPT == kAdEMAMix) gst<float>(C.a3 + b, Am2);
    }
}

// Lanes of this wave that hold elements of the block starting at eb.
__device__ __forceinline__ int q8_mine(const DevTensor &T, int64_t eb, int lane)
{
    const int nvalid = (int)min((int64_t)kQBlock, T.numel - eb);
    return max(0, min(4, nvalid - lane * 4));
}

#ifndef OPT_Q8_THREADS
#define OPT_Q8_THREADS 512
#endif
#ifndef OPT_Q8_BLOCKS
#define OPT_Q8_BLOCKS 1
#endif
// Workgroup size of the blockwise kernel (one LDS copy of the 8-bit tables
// per workgroup) and full blocks in flight per wave.
constexpr int kQ8Threads = OPT_Q8_THREADS;
constexpr int kQ8Waves = kQ8Threads / 64;
constexpr int kQ8Blocks = OPT_Q8_BLOCKS;

#ifndef OPT_Q8_TILE
#define OPT_Q8_TILE 32768
#endif
// Elements per tile of the blockwise step (a power of two, a multiple of the
// 8 x 256 elements one pass of the workgroup's waves covers).
constexpr int64_t kQ8Tile = OPT_Q8_TILE;
static_assert(kQ8Tile % (kQ8Waves * kQBlock) == 0, "blockwise tile");

// Blockwise states (8-bit codebook, FP8, FP4): one workgroup per tile (the
// tile scheduling of opt_elem.h), one 256-element block per wave at a time,
// kQ8Blocks blocks in flight per wave.
// Waves per SIMD the AdamW instantiations are held to (their registers fit
// 7 without spilling; AdEMAMix's third state does not, and is left free).
constexpr int kQ8WavesAdamW = 7;

template <int OPT, int GD, int SF>
__global__ __launch_bounds__(kQ8Threads)
__attribute__((amdgpu_waves_per_eu(OPT == kAdamW ? kQ8WavesAdamW : 1))) void step_q8_kernel(const DevTensor *__restrict__ tens,
                                                             const int32_t *__restrict__ ctab,
                                                             const uint32_t *__restrict__ qwords,
                                                             StepArgs a)
{
    extern __shared__ uint32_t lds[];
    __shared__ Scalars sh;
    __shared__ float mtab_s[mini_fmt(SF) ? kMiniTab : 1];
    if (SF == kQ8)
        for (uint32_t i = threadIdx.x; i < a.q.nwords; i += kQ8Threads) lds[i] = qwords[i];
    if (mini_fmt(SF)) fill_mini_tab<SF>(mtab_s, threadIdx.x, kQ8Threads);
    const float *mtab = mini_fmt(SF) ? mtab_s : nullptr;
    if (threadIdx.x == 0) sh = make_scalars(a);
    __syncthreads();
    const Scalars s = sh;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    for (int64_t w = blockIdx.x; w < a.ntiles; w += gridDim.x) {
        DevTensor T;
        int64_t e0, len;
        if (!locate_tile(tens, ctab, a, w, T, e0, len)) continue;
        const float lam = a.unorm ? lam_for(a, T.k) : s.lam;
        const uint32_t nblk = (uint32_t)((len + kQBlock - 1) / kQBlock);
        const uint32_t nfull = (uint32_t)(len / kQBlock);
        const QChunk C = q8_chunk<GD, SF>(T, e0);
        uint32_t b = wave;
        // kQ8Blocks full blocks per iteration: all their loads before any math
        for (; b + (kQ8Blocks - 1) * kQ8Waves < nfull; b += kQ8Blocks * kQ8Waves) {
            QIn x[kQ8Blocks];
#pragma unroll
            for (int u = 0; u < kQ8Blocks; ++u) q8_load<OPT, GD, SF, true>(a, C, b + u * kQ8Waves, 4, lane, x[u]);
#pragma unroll
            for (int u = 0; u < kQ8Blocks; ++u)
                q8_finish<OPT, SF, true>(a, s, C, lds, mtab, b + u * kQ8Waves, 4, lane, lam, x[u]);
        }
        for (; b < nfull; b += kQ8Waves) {
            QIn x0;
            q8_load<OPT, GD, SF, true>(a, C, b, 4, lane, x0);
            q8_finish<OPT, SF, true>(a, s, C, lds, mtab, b, 4, lane, lam, x0);
        }
        if (b < nblk) {   // the tensor's short last block
            const int nm = q8_mine(T, e0 + (int64_t)b * kQBlock, lane);
            QIn x0;
            q8_load<OPT, GD, SF, false>(a, C, b, nm, lane, x0);
            q8_finish<OPT, SF, false>(a, s, C, lds, mtab, b, nm, lane, lam, x0);
        }
    }
}

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
    __shared__ Scalars sh;
    if (SF == kQ8)
        for (uint32_t i = threadIdx.x; i < 512; i += kThreads) lds[i] = qwords[i];
    if (threadIdx.x == 0) sh = make_scalars(a);
    __syncthreads();
    const Scalars s = sh;
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
#define OPT_GN_UNITS 4
#endif
// One workgroup per tile of kGnTile gradient elements: kGnUnits partial units
// of 1024 elements per wave.
constexpr int kGnUnits = OPT_GN_UNITS;
constexpr int64_t kGnTile = (int64_t)kWaves * kGnUnits * kUTile;

template <int GD>
__global__ __launch_bounds__(kThreads) void gnorm_partials_kernel(const DevTensor *__restrict__ tens,
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
#pragma unroll
            for (int u = 0; u < kGnUnits; ++u) gnorm_load_unit<GD>(T.g, e0 + (wave + u * kWaves) * kUTile, lane, g[u]);
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

__global__ void debug_round_kernel(const float *x, const uint32_t *r, uint16_t *out, int64_t n)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = (uint16_t)(r ? bf16_sr(x[i], r[i] & 0xFFFFu) : bf16_rne(x[i]));
}

__global__ void debug_quantize_kernel(QTabs q, int is_signed, const float *x, uint8_t *out, int64_t n)
{
    extern __shared__ uint32_t lds[];
    for (uint32_t i = threadIdx.x; i < q.nwords; i += blockDim.x) lds[i] = q.words[i];
    __syncthreads();
    const QTabParams P = is_signed ? q.s : q.u;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = x[i];
        out[i] = (uint8_t)(v != v ? 0u : q8_lookup(v, lds, P, is_signed != 0));
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
#pragma unroll
            for (int u = 0; u < kCastGroups; ++u) {
                const f4 t = sld<f4>(x + 4 * (q0 + threadIdx.x + u * 256));
                v[u][0] = t.x; v[u][1] = t.y; v[u][2] = t.z; v[u][3] = t.w;
            }
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
    hipLaunchKernelGGL(debug_stream_kernel, dim3(grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers (called by opt_api.cpp)

// The blockwise step over tiles of kQ8Tile elements (opt_elem.h).
template <class K>
static hipError_t launch_q8_tiles(K kernel, size_t lds, const LaunchGeom &lg, StepArgs a, hipStream_t st)
{
    set_tiles(a, kQ8Tile);
    hipLaunchKernelGGL(kernel, dim3(tile_grid(a, lg)), dim3(kQ8Threads), lds, st, a.tens, a.chunk_tensor,
                       a.q.words, a);
    return hipGetLastError();
}

hipError_t launch_step_ew(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st);

template <int OPT, int GD>
static hipError_t launch_step_t(int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    if (!blocked(fmt)) return launch_step_ew(OPT, GD, fmt, a, lg, st);
    if (a.p_dtype != kP32) return hipErrorInvalidValue;
    switch (fmt) {
    case kQ8: return launch_q8_tiles(step_q8_kernel<OPT, GD, kQ8>, lds, lg, a, st);
    case kFP8RN: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP8RN>, 0, lg, a, st);
    case kFP8SR: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP8SR>, 0, lg, a, st);
    case kFP4RN: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP4RN>, 0, lg, a, st);
    case kFP4SR: return launch_q8_tiles(step_q8_kernel<OPT, GD, kFP4SR>, 0, lg, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <int OPT>
static hipError_t launch_step_o(int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    switch (gd) {
    case kGradF32: return launch_step_t<OPT, kGradF32>(fmt, a, lg, lds, st);
    case kGradBF16: return launch_step_t<OPT, kGradBF16>(fmt, a, lg, lds, st);
    case kGradF16: return launch_step_t<OPT, kGradF16>(fmt, a, lg, lds, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, hipStream_t st)
{
    return opt == kAdamW ? launch_step_o<kAdamW>(gd, fmt, a, lg, lds, st)
                         : launch_step_o<kAdEMAMix>(gd, fmt, a, lg, lds, st);
}

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

hipError_t launch_debug_quantize(const QTabs &q, int is_signed, const float *x, uint8_t *out, int64_t n,
                                 hipStream_t st)
{
    int64_t blocks = min((int64_t)1024, (n + 255) / 256);
    hipLaunchKernelGGL(debug_quantize_kernel, dim3((unsigned)max((int64_t)1, blocks)), dim3(256),
                       (size_t)q.nwords * 4, st, q, is_signed, x, out, n);
    return hipGetLastError();
}

}  // namespace optstep

// opt_blk.h -- device building blocks of the blockwise state formats (8-bit
// codebook, FP8 and FP4): codes, block absmax, loading and finishing one
// 256-element block per wave.  Used by the blockwise step (opt_kernels_q8.hip)
// and the update-norm pre-pass (opt_kernels.hip).
//
// The blockwise formats hand one 256-element block to one wave (64 lanes x 4
// consecutive elements), which makes the block absmax a wave reduction; codes
// move as 32-bit (8-bit formats) or 16-bit (FP4) accesses per lane, fully
// coalesced.
#pragma once

#include "opt_elem.h"

namespace optstep {

// ---------------------------------------------------------------------------
// 8-bit blockwise states

// The top bytes of four words, packed low to high (two byte permutes and an
// or): the codes q8_code_hi leaves there.
__device__ __forceinline__ uint32_t pack_top_bytes(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3)
{
    // selector bytes 0-3 pick from the second operand, 4-7 from the first,
    // 0x0C gives a zero byte
    return __builtin_amdgcn_perm(h1, h0, 0x0C0C0703u) | __builtin_amdgcn_perm(h3, h2, 0x07030C0Cu);
}

// q8_code_hi for the step's fast path, x normal or 0 with |x| <= 1 (for the
// unsigned table x >= +0, as every v is), the table in LDS: the same entry
// and sum with byte-offset addressing.  s is all ones iff x <= +0 as a signed
// integer (a saturating b - 1 keeps -0 negative), and picks the odd entry
// through its bit 2 (the table starts 8-byte aligned).
template <bool SIGNED>
__device__ __forceinline__ uint32_t q8_code_hi_lds(float x, const uint32_t *tab, const QTabParams &P)
{
    const uint32_t b = fbits(x);
    const uint32_t a = SIGNED ? b & 0x7FFFFFFFu : b;
    const uint32_t d = a > P.lo ? a - P.lo : 0u;
    const uint32_t k = d & ((1u << P.shift) - 1u);
    const uint32_t j = d >> P.shift;
    typedef __attribute__((address_space(3))) const uint32_t lds_word;
    const uint32_t base = (uint32_t)(uintptr_t)(lds_word *)(tab + P.offset);   // LDS byte address
    if (!SIGNED) return *(lds_word *)(uintptr_t)(base + (j << 2)) + k;
    const uint32_t s = (uint32_t)(__builtin_elementwise_sub_sat((int32_t)b, 1) >> 31);
    const uint32_t e = *(lds_word *)(uintptr_t)((j << 3) + ((s & 4u) | base));
    return e + (k ^ s);
}

// Codes of this lane's four fp32 moments against their block absmax A (a
// wave-uniform value).  When div_by_ok(A) and no moment of the wave is a
// nonzero value below 2^-100, div_by gives the correctly rounded x = m'/A
// (|x| <= 1, normal or 0); otherwise x = 0 for A = 0, else the correctly
// rounded m'/A, and a NaN quotient (A NaN or infinite) gets code 0.
template <bool SIGNED>
__device__ __forceinline__ uint32_t quant4(const float x[4], float A, const uint32_t *lds, const QTabParams &P)
{
    uint32_t out = 0;
    // 0 < |x| < 2^-100 for some x: |x| - 1 (as unsigned, 0 wraps to the top)
    // below the bits of 2^-100 - 1
    uint32_t t = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) t = min(t, (SIGNED ? fbits(x[i]) & 0x7FFFFFFFu : fbits(x[i])) - 1u);
    if (div_by_ok(A) && !__any(t < 0x0D7FFFFFu)) {
        const float y = recip_rn(A);
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = q8_code_hi_lds<SIGNED>(div_by(x[i], A, y), lds, P);
        out = pack_top_bytes(h[0], h[1], h[2], h[3]);
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
// of a short block are passed as 0.  NONNEG: the values are +0 or positive
// (v) or NaN, so their bit patterns need no sign mask (a NaN with its sign
// bit set still exceeds every number, and the absmax reads as NaN either
// way).
template <bool NONNEG = false>
__device__ __forceinline__ float block_absmax(const float x[4])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, NONNEG ? fbits(x[i]) : fbits(x[i]) & 0x7FFFFFFFu);
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

template <int GD, int SF, int PD>
__device__ __forceinline__ QChunk q8_chunk(const DevTensor &T, int64_t e0)
{
    const int64_t sb = fp4_fmt(SF) ? e0 / 2 : e0;
    QChunk c;
    c.p = (float *)(void *)((uint8_t *)(void *)T.p + e0 * (PD == kP32 ? 4 : 2));   // fp32, or 16-bit words
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
template <int OPT, int GD, int SF, int PD, bool FULL>
__device__ __forceinline__ void q8_load(const StepArgs &a, const QChunk &C, uint32_t b, int nmine, int lane,
                                        QIn &x)
{
    if (FULL) nmine = 4;
    const uint32_t e = b * kQBlock + lane * 4;
    if (nmine == 4) {
        load_p4<PD>(C.p, e, x.p);
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
                x.p[i] = load_p1<PD>(C.p, e + i);
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

typedef short s2_t __attribute__((ext_vector_type(2)));

// Codes of four values of one block by gfx950's scaled conversions, for
// E4M3, E2M1 and (through E5M2) unsigned E2M2 when the conversion's scale is
// a normal binary32 value (the caller's uniform test).  Each value is first clamped to the grid's largest
// finite value times the scale (past it the conversion gives NaN; our rule
// takes the largest value, and clamping first gives the same code).  The
// nearest conversions are IEEE; the stochastic ones add their random
// operand's top bits to the dropped bits, so the element's 16 random bits go
// in the high half, which makes them round up exactly when the top 16 dropped
// bits plus r carry.  The packed FP4 stochastic conversion draws its second
// element's bits elsewhere, so each element gets a conversion of its own.
// Checked on MI355X against mini_encode: 33.5 M hashed values and 33.5 M edge
// cases (zeros of both signs, binary32 subnormals, values at the clamp, every
// normal scale), no difference in any of the four conversions.
template <class F, bool SR>
__device__ __forceinline__ uint32_t mini_pack4_hw(const float x[4], int nsc, const uint32_t r[4])
{
    const float scale = ldexpf(1.0f, -nsc);
    const float lim = (F::kSign == 0x80u ? 448.0f : F::kSign == 0u ? 7.0f : 6.0f) * scale;
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(x[i], -lim, lim);
    if (F::kSign == 0u) {
        // Unsigned E2M2 through E5M2: a grid value y (0 .. 7, step 1/4 below
        // 1) times 2^-14 is the E5M2 value with the same exponent and fraction
        // fields (E5M2's subnormals have step 2^-16), so the E5M2 code's low
        // nibble is the E2M2 code; the scale 2^(14 - nsc) must be normal, which
        // the caller's nsc >= -113 keeps.  Checked on MI355X against
        // mini_encode: 67 M hashed and edge inputs over every admissible
        // scale, nearest and stochastic, no difference.
        const float sc = ldexpf(1.0f, 14 - nsc);
        uint32_t w;
        if (!SR) {
            s2_t p = {};
            p = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(p, c[0], c[1], sc, false);
            p = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(p, c[2], c[3], sc, true);
            w = __builtin_bit_cast(uint32_t, p);
        } else {
            w = 0;
            w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, c[0], r[0] << 16, sc, 0);
            w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, c[1], r[1] << 16, sc, 1);
            w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, c[2], r[2] << 16, sc, 2);
            w = __builtin_amdgcn_cvt_scalef32_sr_bf8_f32(w, c[3], r[3] << 16, sc, 3);
        }
        return (w & 0xFu) | ((w >> 4) & 0xF0u) | ((w >> 8) & 0xF00u) | ((w >> 12) & 0xF000u);
    }
    if (F::kSign == 0x80u) {                     // E4M3, a byte each
        if (!SR) {
            s2_t w = {};
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c[0], c[1], scale, false);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c[2], c[3], scale, true);
            return __builtin_bit_cast(uint32_t, w);
        }
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, c[0], r[0] << 16, scale, 0);
        w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, c[1], r[1] << 16, scale, 1);
        w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, c[2], r[2] << 16, scale, 2);
        w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, c[3], r[3] << 16, scale, 3);
        return w;
    }
    if (!SR) {                                   // E2M1, two nibbles a byte
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[0], c[1], scale, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[2], c[3], scale, 1);
        return w & 0xFFFFu;
    }
    typedef float f2v __attribute__((ext_vector_type(2)));
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (f2v){c[i], c[i]}, r[i] << 16, scale, 0);
        out |= (b & 0xFu) << (4 * i);
    }
    return out;
}

template <class F, bool SR>
__device__ __forceinline__ uint32_t mini_pack4(const float x[4], float A, const uint32_t r[4])
{
    if (!finite_f(A)) return 0u;
    const int nsc = mini_enc_shift<F>(A);
    // E4M3 and E2M1 both ways, unsigned E2M2 stochastic (through E5M2).
    // Paired on MI355X, 2^30 elements: FP8-SR 2.89 -> 2.72 ms, FP4-SR 2.65 ->
    // 2.51 (E2M1) -> 2.39 (E2M2 too), FP4-RN 2.32 -> 2.29, and, since the
    // nearest kernels run VALU-bound in their 1 K-element tiles, FP8-RN 2.49
    // -> 2.39.  Nearest E2M2 keeps its few integer instructions (the
    // conversion costs FP4-RN 1.4 %).  Decoding by the matching conversions
    // instead of the LDS grid table measured 0 to -7 %.
    constexpr bool hw = F::kSign == 0x80u || F::kMB == 1 || (F::kSign == 0u && SR);
    if (hw && nsc >= (F::kSign == 0u ? -113 : -127) && nsc <= 126) return mini_pack4_hw<F, SR>(x, nsc, r);
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

// FULL: every lane holds four elements (all blocks but a tensor's short last
// one).  PLAIN: no gradient scale and no skip_zeros in this call.
template <int OPT, int SF, int PD, bool FULL, bool PLAIN = false>
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
    if (!PLAIN && a.fresh) {
#pragma unroll
        for (int i = 0; i < 4; ++i) m_in[i] = v_in[i] = m2_in[i] = 0.0f;
    }
    // stochastic rounding: the element's Philox word, low half for m, high
    // half for v; the second stream's word, low half for m2 and high half
    // for a 16-bit parameter stored stochastically (rm, rv, rm2: the 16 bits
    // as an integer; rp: the whole word, as the parameter store takes them)
    uint32_t rm[4] = {0, 0, 0, 0}, rv[4] = {0, 0, 0, 0}, rm2[4] = {0, 0, 0, 0}, rp[4] = {0, 0, 0, 0};
    const bool psr = PD != kP32 && a.p_sr;
    const uint64_t q = (uint64_t)(C.e0 + e) >> 2;
    if (sr_fmt(SF)) {
        PhiloxOut w = sr_block(a.seed, a.step, C.k, q, false);
        rm[0] = w.w0 & 0xFFFFu; rm[1] = w.w1 & 0xFFFFu; rm[2] = w.w2 & 0xFFFFu; rm[3] = w.w3 & 0xFFFFu;
        rv[0] = w.w0 >> 16; rv[1] = w.w1 >> 16; rv[2] = w.w2 >> 16; rv[3] = w.w3 >> 16;
    }
    if ((sr_fmt(SF) && OPT == kAdEMAMix) || psr) {
        PhiloxOut w2 = sr_block(a.seed, a.step, C.k, q, true);
        rm2[0] = w2.w0 & 0xFFFFu; rm2[1] = w2.w1 & 0xFFFFu; rm2[2] = w2.w2 & 0xFFFFu; rm2[3] = w2.w3 & 0xFFFFu;
        rp[0] = w2.w0; rp[1] = w2.w1; rp[2] = w2.w2; rp[3] = w2.w3;
    }
    // The stored moments are exact binary32; only the direction u takes the
    // fast path, per element: for an fp32 p (moments4), and for a 16-bit p
    // where it provably stores the exact recipe's word (moments16).
    float p[4], mo[4], vo[4], m2o[4];
    Mom r[4];
    if (PD == kP32) {
        moments4<OPT, !PLAIN>(s, a, x.g, m_in, v_in, m2_in, r);
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = apply_update(x.p[i], s.d, lam, r[i].u);
    } else {
        moments16<OPT, PD, !PLAIN>(s, a, x.p, x.g, m_in, v_in, m2_in, lam, psr, rp, r, p);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mo[i] = r[i].m;
        vo[i] = r[i].v;
        m2o[i] = r[i].m2;
    }
    if (!PLAIN && a.skip_zeros) {   // a zero gradient keeps p and codes the old moments again
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (x.g[i] == 0.0f) {
                p[i] = x.p[i];
                mo[i] = m_in[i];
                vo[i] = v_in[i];
                m2o[i] = m2_in[i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nmine) mo[i] = vo[i] = m2o[i] = 0.0f;   // past the end of a short block
    }
    const float Am = block_absmax(mo), Av = block_absmax<true>(vo);
    const uint32_t om = blk_encode4<SF, 0>(lds, a, mo, Am, rm);
    const uint32_t ov = blk_encode4<SF, 1>(lds, a, vo, Av, rv);
    uint32_t om2 = 0;
    float Am2 = 0.0f;
    if (OPT == kAdEMAMix) {
        Am2 = block_absmax(m2o);
        om2 = blk_encode4<SF, 2>(lds, a, m2o, Am2, rm2);
    }
    if (nmine == 4) {
        store_p4<PD>(C.p, e, p, psr, rp);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < nmine) store_p1<PD>(C.p, e + i, p[i], psr, rp[i]);
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

}  // namespace optstep

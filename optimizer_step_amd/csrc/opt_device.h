// opt_device.h -- device building blocks of the optimizer-step kernels.
//
// Functions marked __host__ __device__ are also compiled into the host side
// of the library so that the CPU tests exercise the very same source.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "opt_plan.h"

namespace optstep {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Accesses through the global address space, so the compiler emits global_*
// (not flat_*) instructions for pointers it reads out of the tensor table.
#define OPT_GLOBAL __attribute__((address_space(1)))

template <class V>
__device__ __forceinline__ V gld(const void *p) { return *(const OPT_GLOBAL V *)p; }

template <class V>
__device__ __forceinline__ void gst(void *p, V v) { *(OPT_GLOBAL V *)p = v; }

// Streaming accesses of the per-element arrays (p, g, states): each byte is
// touched once per step, so they carry the non-temporal hint (measured on
// MI355X: +2-4% step bandwidth over plain accesses).  Buffer loads with the
// same hint, alone or with SC0/SC1, ran within 1 % of these on the headline
// step; with SC1 and no hint they lost 8-13 %.
#ifndef OPT_NT_LOAD
#define OPT_NT_LOAD 1
#endif
#ifndef OPT_NT_STORE
#define OPT_NT_STORE 1
#endif

template <class V>
__device__ __forceinline__ V sld(const void *p)
{
#if OPT_NT_LOAD
    return __builtin_nontemporal_load((const OPT_GLOBAL V *)p);
#else
    return *(const OPT_GLOBAL V *)p;
#endif
}

template <class V>
__device__ __forceinline__ void sst(void *p, V v)
{
#if OPT_NT_STORE
    __builtin_nontemporal_store(v, (OPT_GLOBAL V *)p);
#else
    *(OPT_GLOBAL V *)p = v;
#endif
}

__host__ __device__ inline uint32_t fbits(float x)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __float_as_uint(x);
#else
    uint32_t u; memcpy(&u, &x, 4); return u;
#endif
}

__host__ __device__ inline float bitsf(uint32_t u)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __uint_as_float(u);
#else
    float x; memcpy(&x, &u, 4); return x;
#endif
}

// ---------------------------------------------------------------------------
// BF16 words.  A BF16 word is the high half of a binary32 word.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return bitsf(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bitsf(w & 0xFFFF0000u); }

// Round to nearest even ("When Small Updates Disappear", Sec. 6: the built-in
// cast): add 0x7FFF plus the last kept bit, keep the high half.  NaN keeps its
// sign and becomes quiet.
__host__ __device__ inline uint32_t bf16_rne(float x)
{
    uint32_t b = fbits(x);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x0040u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Stochastic rounding (same page, Sec. 6.1): add a 16-bit random integer to
// the word and keep the high half; the carry reaches the kept bits with
// probability (dropped bits)/2^16.  Infinities and NaNs round to nearest.
__host__ __device__ inline uint32_t bf16_sr(float x, uint32_t r16)
{
    uint32_t b = fbits(x);
    if ((b & 0x7F800000u) == 0x7F800000u) return bf16_rne(x);
    return (b + r16) >> 16;
}

// The same two roundings for a pair of values, by gfx950's conversion
// instructions (x0 in the low half of the result).  Nearest-even is the IEEE
// conversion; it equals bf16_rne on every non-NaN binary32 word (all 2^32
// checked on MI355X), and NaNs stay NaNs.  The stochastic conversion adds the
// HIGH 16 bits of its random operand to the dropped bits: it equals
// bf16_sr(x, r >> 16) (checked on 2^28 hashed words and random operands);
// callers pass the element's 16 random bits in the high half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_rne(float x0, float x1)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){x0, x1}, bf16x2_t));
}

__device__ __forceinline__ uint32_t bf16x2_sr_hi(float x0, uint32_t rh0, float x1, uint32_t rh1)
{
    bf16x2_t o = {};
    o = __builtin_amdgcn_cvt_sr_bf16_f32(o, x0, rh0, false);
    o = __builtin_amdgcn_cvt_sr_bf16_f32(o, x1, rh1, true);
    return __builtin_bit_cast(uint32_t, o);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies and a key-dependent exchange, the key bumped by the
// Weyl constants between rounds.

struct PhiloxOut { uint32_t w0, w1, w2, w3; };

// a ^ b ^ c; one three-input bitwise instruction on gfx950 (truth table 0x96)
__host__ __device__ inline uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
    return a ^ b ^ c;
#endif
}

__host__ __device__ inline PhiloxOut philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                   uint32_t c3, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
    }
    return PhiloxOut{c0, c1, c2, c3};
}

// The block that serves elements 4q..4q+3 of tensor k at step t.
__host__ __device__ inline PhiloxOut sr_block(uint64_t seed, int64_t t, int32_t k, uint64_t q,
                                              bool slow_ema)
{
    return philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), (uint32_t)(uint64_t)t,
                         (uint32_t)k | (slow_ema ? 0x80000000u : 0u),
                         (uint32_t)seed, (uint32_t)(seed >> 32));
}

__host__ __device__ inline uint32_t philox_word(const PhiloxOut &o, int i)
{
    return i == 0 ? o.w0 : i == 1 ? o.w1 : i == 2 ? o.w2 : o.w3;
}

// ---------------------------------------------------------------------------
// Division by a divisor b that is the same for many dividends, given
// y = RN(1/b).  q0 = a*y is within 1.5 ulp of a/b; one residual correction
// (r = a - b*q exactly by fma, q += r*y) makes it faithful, and a second
// correction then yields the correctly rounded quotient (Markstein's theorem:
// y within half an ulp of 1/b and q faithful => RN(q + r*y) = RN(a/b)).
// Requires b and 1/b normal, a/b not below the normal range, and |a| >= 2^-100
// or a = 0: the residual is exact only while ulp(b)*ulp(q) >= 2^-149, which
// holds for e(a) >= -102 since e(a) is e(b) + e(q) within one.  Callers check
// b and the dividends as described where they use it.
__host__ __device__ inline float div_by(float a, float b, float y)
{
    float q = a * y;
    float r = fmaf(-b, q, a);
    q = fmaf(r, y, q);
    r = fmaf(-b, q, a);
    return fmaf(r, y, q);
}

// b for which div_by is exact for every dividend a with |a| >= 2^-100 or
// a = 0 and |a| <= |b|: 2^-124 <= |b| <= 2^26 keeps b and 1/b normal and the
// quotient at or above 2^-126.  An integer test of the bits, so a wave-uniform
// b is checked on the scalar unit.
__host__ __device__ inline bool div_by_ok(float b)
{
    return (fbits(b) & 0x7FFFFFFFu) - 0x01800000u <= 0x4C800000u - 0x01800000u;
}

// RN(1/b) for b with 2^-126 <= |b| <= 2^126 (the range div_by_ok admits).
// The hardware reciprocal in binary64 refined by two Newton steps is 1/b to
// within 2^-52 relative, and 1/b is never that close to a binary32 rounding
// boundary: a midpoint m of 25 significant bits has |1 - b*m| >= 2^-49 unless
// b*m = 1, which needs b and m powers of two (m is then no midpoint), so the
// one rounding to binary32 gives the correctly rounded reciprocal.  Seven
// instructions, against about a dozen for the IEEE division sequence.
__device__ __forceinline__ float recip_rn(float b)
{
    const double d = (double)b;
    double r = __builtin_amdgcn_rcp(d);
    double e = __builtin_fma(-d, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-d, r, 1.0);
    r = __builtin_fma(r, e, r);
    return (float)r;
}

// Dividends for which div_by is correctly rounded (with a divisor that passes
// div_by_ok): zero, or a finite magnitude of at least 2^-100.  Others (tiny,
// infinite, NaN) take the plain division.
__host__ __device__ inline bool div_by_arg(float a)
{
    const uint32_t m = fbits(a) & 0x7FFFFFFFu;
    return m == 0u || m - 0x0D800000u < 0x7F800000u - 0x0D800000u;
}

// ---------------------------------------------------------------------------
// 8-bit code of x against a codebook's lookup table (layout in opt_plan.h),
// for x with |x| <= 1 that is not NaN (and, for an unsigned table, x >= 0 or
// -0), returned in the top byte of the word (the low bits are noise).  The
// magnitude max(|x|, lo) picks a bucket that holds at most one threshold, so
// the code is the bucket's entry plus the in-bucket key.  +0 reads the x <= 0
// side: a midpoint of exactly 0 sits between +0 and the smallest positive
// float, and that side holds code(0) for m -> 0.  On the x <= 0 side the key
// enters complemented (s = all ones), which the entries expect.
__host__ __device__ inline uint32_t q8_code_hi(float x, const uint32_t *tab, const QTabParams &P,
                                               bool is_signed)
{
    const uint32_t b = fbits(x);
    const uint32_t a = b & 0x7FFFFFFFu;
    const uint32_t d = a > P.lo ? a - P.lo : 0u;       // all |x| < lo share one code
    const uint32_t k = d & ((1u << P.shift) - 1u);
    const uint32_t j = d >> P.shift;
    if (!is_signed) return tab[P.offset + j] + k;
    const uint32_t s = (int32_t)b <= 0 ? ~0u : 0u;
    return tab[P.offset + 2u * j + (s & 1u)] + (k ^ s);
}

__host__ __device__ inline uint32_t q8_code(float x, const uint32_t *tab, const QTabParams &P,
                                            bool is_signed)
{
    return q8_code_hi(x, tab, P, is_signed) >> 24;
}

// The same for any x that is not NaN (callers map NaN to code 0): magnitudes
// above 1 read as 1, which keeps the nearest-entry code (entries lie in
// [-1, 1]), and an unsigned table gives code 0 to every x <= 0 (all its
// midpoints are above 0).
__host__ __device__ inline uint32_t q8_lookup(float x, const uint32_t *tab, const QTabParams &P,
                                              bool is_signed)
{
    const uint32_t b = fbits(x);
    if (!is_signed && (b >> 31)) return 0u;
    if ((b & 0x7FFFFFFFu) > 0x3F800000u) x = bitsf((b & 0x80000000u) | 0x3F800000u);
    return q8_code(x, tab, P, is_signed);
}

// ---------------------------------------------------------------------------
// FP8 and FP4 state elements ("When Small Updates Disappear", Sec. 2.1: grids
// with three and two fraction bits; Sec. 5: such states with nearest or
// stochastic rounding).  FP8 is OCP E4M3 (no infinities, magnitude 0x7F is
// NaN); FP4 stores m and m2 as OCP E2M1 and v, which is never negative, as
// unsigned E2M2.  A 256-element block keeps its absmax A; its elements are
// coded as x / X with X = 2^(floor(log2 A) - EMAX), EMAX the exponent of the
// format's top binade, so the block maximum lands in the top binade and the
// grid keeps its relative spacing.  Codes come straight from the binary32
// bits of x / X: exponent and top fraction bits give the code below, and the
// dropped bits decide nearest-even or stochastic rounding (up iff the top 16
// dropped bits plus the element's 16-bit random integer carry, the rule of
// Sec. 6.1); values past the largest finite one take it.

template <int MB, int BIAS, uint32_t MAXC, uint32_t SIGN, int NANC>
struct MiniFmt {
    static constexpr int kMB = MB;                      // fraction bits
    static constexpr int kBias = BIAS;
    static constexpr int kEmin = 1 - BIAS;              // exponent of the smallest normal
    static constexpr int kEmax = (int)(MAXC >> MB) - BIAS;
    static constexpr uint32_t kMaxC = MAXC;             // largest finite magnitude code
    static constexpr uint32_t kSign = SIGN;             // sign bit of a code, 0 if unsigned
    static constexpr int kNan = NANC;                   // NaN magnitude code, -1 if none
};
using E4M3 = MiniFmt<3, 7, 0x7Eu, 0x80u, 0x7F>;
using E2M1 = MiniFmt<1, 1, 0x7u, 0x8u, -1>;
using E2M2U = MiniFmt<2, 1, 0xFu, 0u, -1>;

// floor(log2 A) for finite A > 0 (binary32 subnormals included).
__host__ __device__ inline int floor_log2(float A)
{
    const uint32_t u = fbits(A) & 0x7FFFFFFFu;
    const int ef = (int)(u >> 23);
    return ef ? ef - 127 : -118 - __builtin_clz(u);
}

__host__ __device__ inline bool finite_f(float A) { return (fbits(A) & 0x7F800000u) != 0x7F800000u; }

// Exponent shift that takes a block's values to its grid (x * 2^nsc), from
// the block absmax: 0 if A is 0 (all elements are zeros).
template <class F>
__host__ __device__ inline int mini_enc_shift(float A)
{
    return A > 0.0f ? F::kEmax - floor_log2(A) : 0;
}

// Exponent that takes grid values back (v * 2^sc); a zero absmax reads every
// element as a zero of its sign (2^-400 flushes any grid value to zero).
template <class F>
__host__ __device__ inline int mini_dec_shift(float A)
{
    return A > 0.0f ? floor_log2(A) - F::kEmax : -400;
}

// Magnitude code of y >= 0 on F's grid; SR with the 16-bit integer r.  In
// the format's normal range (y >= 2^Emin) the binary32 exponent and top MB
// fraction bits are the code below y, less a constant, and the other
// `drop` = 23 - MB fraction bits decide the rounding (nearest-even: the usual
// add-and-shift; SR: their top 16 bits plus r carry).  Below 2^Emin the grid
// step is 2^(Emin - MB): t = y / step is exact, its integer part is the code
// below and its fraction decides.  A carry moves to the next code, which is
// the next grid value across binades too; codes past the largest finite one
// take it.
template <class F, bool SR>
__host__ __device__ inline uint32_t mini_mag(float y, uint32_t r)
{
    constexpr int drop = 23 - F::kMB;
    constexpr uint32_t K = (uint32_t)(127 + F::kEmin - 1) << F::kMB;   // code = (bits >> drop) - K
    const uint32_t u = fbits(y) & 0x7FFFFFFFu;
    uint32_t cn;
    if (SR) {
        const uint32_t l16 = drop >= 16 ? (u >> (drop >= 16 ? drop - 16 : 0)) & 0xFFFFu
                                        : (u << (drop >= 16 ? 0 : 16 - drop)) & 0xFFFFu;
        cn = (u >> drop) - K + ((l16 + r) >> 16);
    } else {
        cn = ((u + (1u << (drop - 1)) - 1u + ((u >> drop) & 1u)) >> drop) - K;
    }
    const float t = bitsf(fbits(y) & 0x7FFFFFFFu) * (float)(1u << (F::kMB - F::kEmin));   // exact
    uint32_t cs;
    if (SR) {
        const float fl = floorf(t);
        const uint32_t l16 = (uint32_t)((t - fl) * 65536.0f);   // exact: floor(frac * 2^16)
        cs = (uint32_t)fl + ((l16 + r) >> 16);
    } else {
        cs = (uint32_t)rintf(t);                                // ties to even
    }
    const uint32_t code = u < ((uint32_t)(127 + F::kEmin) << 23) ? cs : cn;
    return code < F::kMaxC ? code : F::kMaxC;
}

// Code of x * 2^nsc.  When nsc < Emin + 126 (the block's absmax is not far
// below the binary32 normal range; uniform over a block), every x whose
// binary32 exponent field is 0 lies below the grid's normal range, so the
// grid binade of y = |x| * 2^nsc is E = max(field - 127 + nsc, Emin) and its
// step is 2^(E - MB).  Then q = |x| * 2^(nsc + MB - E) in [0, 2^(MB+1)) is
// exact (a power-of-two scaling; a q below 2^-126 is far below one step and
// codes as 0 either way), the code below y is ((E - Emin) << MB) + floor(q),
// and rounding q to an integer (nearest-even, or up iff the top 16 bits of
// its fraction plus r carry) gives the code; a carry to 2^(MB+1) lands on the
// next binade's first code.  Other blocks take mini_mag on x * 2^nsc.
template <class F, bool SR>
__host__ __device__ inline uint32_t mini_encode(float x, int nsc, uint32_t r)
{
    uint32_t c;
    if (nsc < F::kEmin + 126) {
        // infinities and NaNs as the largest finite binary32, which codes as
        // the largest code like any value past the grid's end
        const uint32_t u = min(fbits(x) & 0x7FFFFFFFu, 0x7F7FFFFFu);
        const int e = (int)(u >> 23) - 127 + nsc;
        const int E = e > F::kEmin ? e : F::kEmin;
        const float q = ldexpf(bitsf(u), nsc + F::kMB - E);
        uint32_t k;
        if (SR) {
            const float fl = floorf(q);
            const uint32_t l16 = (uint32_t)((q - fl) * 65536.0f);   // exact: floor(frac * 2^16)
            k = (uint32_t)fl + ((l16 + r) >> 16);
        } else {
            k = (uint32_t)rintf(q);                                 // ties to even
        }
        c = ((uint32_t)(E - F::kEmin) << F::kMB) + k;
        c = c < F::kMaxC ? c : F::kMaxC;
    } else {
        // exact unless x * 2^nsc falls below the binary32 normal range, where
        // it is far below the grid's smallest step and codes as 0 either way
        c = mini_mag<F, SR>(ldexpf(x, nsc), r);
    }
    if (F::kSign && (fbits(x) >> 31)) c |= F::kSign;
    return c;
}

// IEEE binary16 as a grid for stochastic rounding: past the largest finite
// value (65504) the next value is infinity, as a carry into the exponent gives.
using F16 = MiniFmt<10, 15, 0x7C00u, 0x8000u, -1>;

// FP32 -> FP16 bits with stochastic rounding by the 16-bit integer r (up iff
// the top 16 dropped bits plus r carry); NaN stays NaN with its sign.
__host__ __device__ inline uint32_t f16_sr(float x, uint32_t r)
{
    if (x != x) return ((fbits(x) >> 16) & 0x8000u) | 0x7E00u;
    return mini_encode<F16, true>(x, 0, r);
}

// FP16 words: widening is exact; nearest-even narrowing is the hardware
// conversion (v_cvt_f16_f32 under the default round-to-nearest-even mode).
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ uint32_t f16_rne(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// Grid value of a magnitude code (exact in binary32).
template <class F>
__host__ __device__ inline float mini_val(uint32_t mag)
{
    const uint32_t e = mag >> F::kMB, f = mag & ((1u << F::kMB) - 1u);
    if (e == 0) return ldexpf((float)f, 1 - F::kBias - F::kMB);
    return bitsf(((e + 127u - (uint32_t)F::kBias) << 23) | (f << (23 - F::kMB)));
}

template <class F>
__host__ __device__ inline float mini_decode(uint32_t code, int sc)
{
    const uint32_t mag = F::kSign ? code & (F::kSign - 1u) : code;
    float x = ldexpf(mini_val<F>(mag), sc);
    if (F::kNan >= 0 && mag == (uint32_t)F::kNan) x = bitsf(0x7FC00000u);
    return (F::kSign && (code & F::kSign)) ? -x : x;
}

// ---------------------------------------------------------------------------
// Bias corrections and the other per-call scalars.  They are uniform across
// the launch (the issue "Investigate SM103 bias-correction broadcast in
// 32-bit optimizers", Problem), so the host forms them once per call and the
// kernels receive them in their arguments (StepArgs::sc).

__host__ __device__ inline double powi(double b, int64_t t)
{
    double r = 1.0;
    while (t > 0) {
        if (t & 1) r *= b;
        b *= b;
        t >>= 1;
    }
    return r;
}

// The call's scalars from its hyperparameters; the host forms them once per
// call (StepArgs::sc), with IEEE binary64 and binary32 operations only, so
// they are the same bits on either side.
__host__ __device__ inline Scalars make_scalars(const StepArgs &a)
{
    Scalars s;
    s.om1 = 1.0f - a.beta1;
    s.om2 = 1.0f - a.beta2;
    s.om3 = 1.0f - a.beta3;
    s.c1 = (float)(1.0 - powi((double)a.beta1, a.bc_step));
    s.c2 = (float)(1.0 - powi((double)a.beta2, a.bc_step));
    // 0 <= beta < 1 (checked by the host) keeps c in [2^-24, 1], where div_by
    // by c is correctly rounded for every moment that passes div_by_arg
    s.rc1 = 1.0f / s.c1;
    s.rc2 = 1.0f / s.c2;
    float lrwd = a.lr * a.wd;
    s.d = 1.0f - lrwd;
    s.lam = a.lr;
    s.gs = 1.0f;
    return s;
}

// The scalars a kernel works with: the host's, and the gradient scale from
// device memory (read when the kernel runs).
__device__ __forceinline__ Scalars call_scalars(const StepArgs &a)
{
    Scalars s = a.sc;
    if (a.grad_scale) s.gs = *a.grad_scale;
    return s;
}

// lr times the update-norm scale of tensor k: min(1, max_unorm*||p||/||u||).
__device__ inline float lam_for(const StepArgs &a, int32_t k)
{
    if (!(a.max_unorm > 0.0f) || a.unorm == nullptr) return a.lr;
    double u2 = a.unorm[2 * (int64_t)k], p2 = a.unorm[2 * (int64_t)k + 1];
    double un = sqrt(u2), bound = (double)a.max_unorm * sqrt(p2);
    float s = un > bound ? (float)(bound / un) : 1.0f;
    return a.lr * s;
}

// ---------------------------------------------------------------------------
// The per-element recipe (fixed binary32 order; built with -ffp-contract=off).

struct Mom { float m, v, m2, u; };

template <int OPT, bool GS = true>
__device__ __forceinline__ Mom moments(const Scalars &s, const StepArgs &a, float g, float m,
                                       float v, float m2)
{
    Mom r;
    if (GS) g = g * s.gs;    // clipping fused into the step (GS false: no scale given)
    float gg = g * g;
    r.m = a.beta1 * m + s.om1 * g;
    r.v = a.beta2 * v + s.om2 * gg;
    float mh = div_by(r.m, s.c1, s.rc1);
    float vh = div_by(r.v, s.c2, s.rc2);
    if (!(div_by_arg(r.m) && div_by_arg(r.v))) {   // rare: the plain correctly rounded division
        mh = r.m / s.c1;
        vh = r.v / s.c2;
    }
    float den = __builtin_sqrtf(vh) + a.eps;
    if (OPT == kAdEMAMix) {
        r.m2 = a.beta3 * m2 + s.om3 * g;
        float num = mh + a.alpha * r.m2;
        r.u = num / den;
    } else {
        r.m2 = 0.0f;
        r.u = mh / den;
    }
    return r;
}

// The same moments, with the direction u (which only feeds the parameter
// update, never a stored moment, code or rounding bit) formed with the
// hardware reciprocal and square root (each within 1 ulp) instead of
// correctly rounded division and square root: u is within a few ulp of the
// exact recipe, far inside the fp32 parameter tolerance.  Used for fp32
// parameters, and for a 16-bit parameter where the bound below shows that the
// stored word is the exact recipe's (moments16); an element whose own v_hat
// is below 2^-96 (where the
// hardware square root loses accuracy) takes the exact recipe (fast_ok), so
// every element's result depends on its own inputs alone.  NaN and infinite
// moments give the same u either way.
//
// With bu given, *bu bounds |u - u_exact| when eps >= 0 and fast_ok holds.
// Each step's error against the exact recipe's, relative (units of 2^-24):
// m*RN(1/c1) against RN(m/c1) 3; v_hat likewise 3, its hardware square root
// (1 ulp) against the correctly rounded one 4.5, so sqrt + eps (eps >= 0
// only shrinks relative errors) and its rounding 6.5; the hardware
// reciprocal 2 and the product's rounding 1 against the exact quotient's 1:
// about 14 for AdamW.  AdEMAMix's numerator mh + alpha*m2 may cancel, so its
// error is bounded against |mh| + |alpha*m2| instead (3.1 for mh, 2 for the
// two roundings of the sum, 10.6 for the rest: under 16 in all).  *bu =
// 2^-19 (|mh| + |alpha*m2|) / den + 2^-140 is twice that, plus room for the
// absolute error of a direction that falls below the normal range.  The
// analysis needs mh and 1/den normal (or mh = 0, which only m = 0 gives, and
// then both directions are the same zero) and (|mh| + |alpha*m2|) / den
// below 2^126, so that no direction overflows: elsewhere *bu is infinite.
template <int OPT, bool GS = true>
__device__ __forceinline__ Mom moments_fast(const Scalars &s, const StepArgs &a, float g, float m,
                                            float v, float m2, float *bu = nullptr)
{
    Mom r;
    if (GS) g = g * s.gs;
    float gg = g * g;
    r.m = a.beta1 * m + s.om1 * g;
    r.v = a.beta2 * v + s.om2 * gg;
    const float mh = r.m * s.rc1;
    const float vh = r.v * s.rc2;
    const float rden = __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(vh) + a.eps);
    float t = 0.0f;
    if (OPT == kAdEMAMix) {
        r.m2 = a.beta3 * m2 + s.om3 * g;
        t = a.alpha * r.m2;
        r.u = (mh + t) * rden;
    } else {
        r.m2 = 0.0f;
        r.u = mh * rden;
    }
    if (bu) {
        const float amh = __builtin_fabsf(mh);
        const float mag = (amh + __builtin_fabsf(t)) * rden;
        const bool ok = (amh >= 0x1p-100f || r.m == 0.0f) && rden >= 0x1p-126f && mag < 0x1p126f;
        *bu = ok ? __builtin_fmaf(0x1p-19f, mag, 0x1p-140f) : __builtin_inff();
    }
    return r;
}

// Whether moments_fast's direction is used for this element (else the exact
// recipe): its fast v_hat is at least 2^-96, or NaN.
template <int OPT>
__device__ __forceinline__ bool fast_ok(const Scalars &s, const Mom &r)
{
    return !(r.v * s.rc2 < 0x1p-96f);
}

// The moments and direction of four elements with fp32 parameters: the
// fast direction, with the exact recipe for the elements fast_ok rejects.
// The wave skips the exact pass when no lane needs it; the result of an
// element never depends on other lanes.
template <int OPT, bool GS = true>
__device__ __forceinline__ void moments4(const Scalars &s, const StepArgs &a, const float g[4],
                                         const float m[4], const float v[4], const float m2[4], Mom r[4])
{
    bool slow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = moments_fast<OPT, GS>(s, a, g[i], m[i], v[i], m2[i]);
        slow[i] = !fast_ok<OPT>(s, r[i]);
    }
    if (__any(slow[0] || slow[1] || slow[2] || slow[3])) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (slow[i]) r[i] = moments<OPT, GS>(s, a, g[i], m[i], v[i], m2[i]);
    }
}

// Decay-first: both terms from the previous p (bitsandbytes PR "Fix decoupled
// weight decay ordering in the CUDA Adam/AdEMAMix kernels", intro).
__device__ __forceinline__ float apply_update(float p, float d, float lam, float u)
{
    float decayed = p * d;
    float step = lam * u;
    return decayed - step;
}

// ---------------------------------------------------------------------------
// Wave64 reductions.

// Max over the 64 lanes of unsigned words (for |x| bit patterns this is the
// numeric max, and any NaN pattern beats every number, so a NaN anywhere
// poisons the result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    // each step is one v_max_u32 with a DPP source: quad_perm [1,0,3,2], [2,3,0,1],
    // then row_ror 4 and 8 leave every lane of a 16-lane row with the row max
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true));
    // row_bcast:15 into rows 1 and 3 (row 1 = rows 0-1, row 3 = rows 2-3), then
    // row_bcast:31 into rows 2 and 3: lane 63 ends with the wave max; rows
    // outside a step's row mask see 0, the identity of the max
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// Sum over the 64 lanes in a fixed butterfly order; every lane ends with the
// same bits (each level adds the same two partial sums, commutatively).
__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace optstep

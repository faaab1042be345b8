/*
 * oracle.c -- plain, slow CPU oracle for the fused element-wise two-state
 * optimizer step (AdamW and AdEMAMix with decoupled weight decay; fp32, BF16
 * and 8-bit blockwise optimizer states; the update-norm pre-pass).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant generator with the
 * HIP path; both sides receive the same seeded inputs and nothing else.
 *
 * Arithmetic model.  Every + - * / sqrt below is one IEEE binary32 operation,
 * rounded to nearest-even, with no contraction into fused multiply-add and no
 * flush of subnormals (build: gcc -O2 -ffp-contract=off -fno-fast-math; on
 * x86-64 SSE, FLT_EVAL_METHOD is 0).  The pages state the step in fp32 (the
 * states are fp32 words; "Reading the stored value into FP32 is exact, so new
 * error only enters when the result is written back", When Small Updates
 * Disappear, Sec. 1.1), and the integer results that depend on it (quantized
 * codes, stochastic-rounding bits) must be decided in that same precision.
 * The bias-correction powers beta^t and the update-norm sums are binary64.
 *
 * Sources (page title, then section):
 *  [PR]  bitsandbytes PR "Fix decoupled weight decay ordering in the CUDA
 *        Adam/AdEMAMix kernels": intro (decay-first order, AdEMAMix rule
 *        reference); "Why the current tests do not catch it" (step-1 closed
 *        form, state zero quantizes exactly, 8-bit blockwise kernel).
 *  [SU]  "When Small Updates Disappear": Sec. 1.1 (the two EMAs), Sec. 3
 *        (stochastic rounding), Sec. 6 and 6.1 (the FP32->BF16 bit trick),
 *        Sec. 7.3 (random number tied to the element).
 *  [ISS] bitsandbytes fork issue "Investigate SM103 bias-correction broadcast
 *        in 32-bit optimizers": Problem (bias-correction scalars, max_unorm
 *        precondition kernel, unorm buffer), Result (the non-deterministic
 *        atomic unorm sum).
 *  [GN]  NeMo Automodel PR "perf(training): fused multi-tensor gradient-norm
 *        reduction": Numerics and Correctness properties (fp64 accumulation,
 *        NaN poisoning of a max).
 *
 * Readings where the pages are silent (each is restated at its use):
 *  - eps is added to sqrt(v_hat), as in torch.optim.AdamW, which [PR] intro
 *    says the fixed kernels match;
 *  - AdEMAMix (Pagliardini et al., cited in [PR] intro): m1 and v are
 *    bias-corrected, the slow EMA m2 is not; u = (m1_hat + alpha*m2)/(sqrt(v_hat)+eps);
 *  - 8-bit codes: the nearest codebook entry, ties to the lower index; the
 *    block absmax is the max |value| over a 256-element block, NaN poisons it
 *    ([GN] Correctness properties); a zero absmax gives x = 0;
 *  - stochastic rounding draws r from Philox4x32-10 (Salmon, Moraes, Dror,
 *    Shaw, SC'11) keyed by the seed, with counter (j>>2, j>>34, t, k);
 *    the low 16 bits of word j mod 4 round m, the high 16 bits round v;
 *  - FP8/FP4 states: see the block-scaled section below;
 *  - a state reset ([SU] Sec. 5) restarts the moments from zero and the
 *    bias-correction count from 1; the random stream keeps the absolute t.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* public enums and hyper-parameter record (oracle-private definitions) */

enum { ORC_ADAMW = 0, ORC_ADEMAMIX = 1 };
enum { ORC_F32 = 0, ORC_BF16_RN = 1, ORC_BF16_SR = 2, ORC_Q8 = 3,
       ORC_FP8_RN = 4, ORC_FP8_SR = 5, ORC_FP4_RN = 6, ORC_FP4_SR = 7 };

typedef struct {
    float lr, beta1, beta2, beta3, alpha, eps, weight_decay, max_unorm;
    int64_t step;         /* t, 1-based                                        */
    uint64_t seed;        /* Philox key for stochastic rounding                */
    int64_t index_base;   /* element index j of the first element passed in    */
    int32_t tensor_index; /* k: the tensor's position in the caller's list     */
    int32_t decay_after;  /* 0: decay-first (the method).  1: the decay-after
                             ordering that [PR] removes; a planted mistake that
                             tests use to show their checks are not vacuous.  */
    float grad_scale;     /* gradient clipping fused into the step: the step
                             uses fl(g * grad_scale); 1 leaves g unchanged   */
    int64_t reset_interval; /* R > 0: the moments restart from zero at steps
                             1, R+1, 2R+1, ... ([SU] Sec. 5); 0: never        */
    int32_t skip_zeros;   /* 1: an element whose gradient is exactly zero keeps
                             its parameter and its states ([PR] Not covered:
                             the decay is skipped with the update)           */
    int32_t pad_;
} orc_hp;

/* ------------------------------------------------------------------ */
/* bit views                                                          */

static uint32_t f2u(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float u2f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* A bf16 word is the high half of a binary32 word, so widening is exact. */
float orc_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* ------------------------------------------------------------------ */
/* BF16 rounding                                                      */

/* Round-to-nearest-even FP32 -> BF16, written from the definition: of the two
 * BF16 magnitudes that bracket |x| (the truncation toward zero and the next
 * one up), take the nearer in exact (binary64) arithmetic; on a tie take the
 * one whose last kept bit is 0.  Above the largest finite BF16 the "next one
 * up" is infinity, which IEEE rounding treats as the value 2^128.  A NaN stays
 * a NaN with its sign, made quiet.  ([SU] Sec. 6: the built-in nearest cast.) */
uint16_t orc_bf16_rne(float x)
{
    uint32_t b = f2u(x);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t mag = b & 0x7FFFFFFFu;
    uint16_t lo = (uint16_t)(mag >> 16);           /* |q-| <= |x|            */
    if ((mag & 0xFFFFu) == 0) return sign | lo;     /* exactly representable  */
    uint16_t hi = (uint16_t)(lo + 1);               /* |q+| >  |x|            */
    double a = fabs((double)x);
    double qlo = (double)orc_bf16_to_f32(lo);
    double qhi = (hi == 0x7F80u) ? ldexp(1.0, 128) : (double)orc_bf16_to_f32(hi);
    double dlo = a - qlo, dhi = qhi - a;
    if (dlo < dhi) return sign | lo;
    if (dhi < dlo) return sign | hi;
    return sign | ((lo & 1u) ? hi : lo);
}

/* Stochastic rounding FP32 -> BF16 with a 16-bit random integer r ([SU]
 * Sec. 3 and 6.1): l is the integer held by the 16 dropped bits; adding r to
 * the word carries into the kept bits exactly when l + r >= 2^16, which moves
 * the magnitude up one BF16 step (away from zero) with probability l/2^16.
 * Infinities and NaNs are kept as they are (the page's special-value lines are
 * lost in extraction; reading: use the nearest cast for them).  A finite value
 * just below the largest float may carry into infinity, as the bit trick does. */
uint16_t orc_bf16_sr(float x, uint32_t r)
{
    uint32_t b = f2u(x);
    if (!isfinite(x)) return orc_bf16_rne(x);
    uint32_t l = b & 0xFFFFu;
    uint16_t kept = (uint16_t)(b >> 16);
    return (l + (r & 0xFFFFu) >= 0x10000u) ? (uint16_t)(kept + 1) : kept;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11).  State: four 32-bit counter words and a two-word
 * key.  One round multiplies counter words 0 and 2 by the two Philox
 * multipliers into 64-bit products, then the new counter is
 *   (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));
 * between rounds the key is bumped by the two Weyl constants (the golden
 * ratio and sqrt(3)-1 in 32-bit fixed point).  Ten rounds.                 */

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 32-bit random word for element j of tensor k at step t.  The counter is
 * tied to the element, not to any launch geometry ([SU] Sec. 7.3): one Philox
 * block serves four consecutive elements.  `stream` selects the second call
 * used for AdEMAMix's slow EMA (counter word 3 = k | 2^31).               */
static uint32_t sr_word(uint64_t seed, int64_t t, int32_t k, int64_t j, int stream)
{
    uint32_t ctr[4], key[2], out[4];
    uint64_t q = (uint64_t)j >> 2;
    ctr[0] = (uint32_t)q;
    ctr[1] = (uint32_t)(q >> 32);
    ctr[2] = (uint32_t)(uint64_t)t;
    ctr[3] = (uint32_t)k | (stream ? 0x80000000u : 0u);
    key[0] = (uint32_t)seed;
    key[1] = (uint32_t)(seed >> 32);
    orc_philox4x32_10(ctr, key, out);
    return out[(uint64_t)j & 3u];
}

/* Exported for tests: the word sr_word() draws. */
uint32_t orc_sr_word(uint64_t seed, int64_t t, int32_t k, int64_t j, int32_t stream)
{
    return sr_word(seed, t, k, j, stream);
}

/* ------------------------------------------------------------------ */
/* 8-bit codebook quantization                                        */

/* Code of x against a strictly increasing 256-entry codebook T: the index of
 * the nearest entry, ties to the lower index.  Written as a count of the
 * midpoints x lies strictly above; each midpoint is formed in binary64, where
 * (T[i] + T[i+1]) / 2 is exact for entries of similar size.  NaN lies above
 * no midpoint and gets code 0.  The midpoints never decrease with i (a
 * rounded sum is monotone), so those below x are a prefix of them and the
 * count is found by bisection: the first midpoint not below x.          */
static double q8_mid(const float *T, int i)
{
    return ((double)T[i] + (double)T[i + 1]) / 2.0;
}

int orc_quantize(const float *T, float x)
{
    int lo = 0, hi = 255;            /* the count lies in [lo, hi] */
    while (lo < hi) {
        int m = (lo + hi) / 2;
        if ((double)x > q8_mid(T, m)) lo = m + 1;
        else hi = m;
    }
    return lo;
}

/* ------------------------------------------------------------------ */
/* Per-call scalars ([ISS] Problem: uniform across the whole launch).     */

typedef struct {
    float om1, om2, om3;   /* 1 - beta                           */
    float c1, c2;          /* bias corrections 1 - beta^t        */
    float d;               /* decay factor 1 - lr*wd             */
    float lam;             /* lr, times the update-norm scale    */
} scalars_t;

static int skipped(const orc_hp *hp, float g) { return hp->skip_zeros && g == 0.0f; }

/* Steps since the moments last started from zero (1 on the step that
 * starts them), and whether this step starts them. */
static int64_t cycle_step(const orc_hp *hp)
{
    if (hp->reset_interval > 0) return (hp->step - 1) % hp->reset_interval + 1;
    return hp->step;
}

static int fresh_states(const orc_hp *hp)
{
    return hp->reset_interval > 0 && cycle_step(hp) == 1;
}

static scalars_t make_scalars(const orc_hp *hp, float scale)
{
    scalars_t s;
    int64_t t = cycle_step(hp);
    s.om1 = 1.0f - hp->beta1;
    s.om2 = 1.0f - hp->beta2;
    s.om3 = 1.0f - hp->beta3;
    s.c1 = (float)(1.0 - pow((double)hp->beta1, (double)t));
    s.c2 = (float)(1.0 - pow((double)hp->beta2, (double)t));
    float lrwd = hp->lr * hp->weight_decay;
    s.d = 1.0f - lrwd;
    s.lam = hp->lr * scale;   /* exact when scale is 1 */
    return s;
}

/* Exported for tests. */
void orc_scalars(const orc_hp *hp, float scale, float out[7])
{
    scalars_t s = make_scalars(hp, scale);
    out[0] = s.om1; out[1] = s.om2; out[2] = s.om3;
    out[3] = s.c1; out[4] = s.c2; out[5] = s.d; out[6] = s.lam;
}

/* ------------------------------------------------------------------ */
/* One element.  Inputs are the fp32 values read from storage (exact for
 * fp32 and BF16 storage; T[code]*absmax for 8-bit storage).              */

typedef struct { float m, v, m2, u; } moments_t;

static moments_t moments_and_direction(int opt, const orc_hp *hp, const scalars_t *s,
                                       float g, float m, float v, float m2)
{
    moments_t r;
    /* A clipping coefficient ([GN]) scales the gradient before it enters the
     * step; a scale of 1 is exact. */
    g = g * hp->grad_scale;
    /* EMAs ([SU] Sec. 1.1):  m' = b1 m + (1-b1) g,  v' = b2 v + (1-b2) g^2,
     * AdEMAMix adds the slow EMA m2' = b3 m2 + (1-b3) g.  g^2 is formed in
     * fp32 from the widened gradient. */
    float gg = g * g;
    r.m = hp->beta1 * m + s->om1 * g;
    r.v = hp->beta2 * v + s->om2 * gg;
    r.m2 = 0.0f;
    /* Bias-corrected direction; eps added to sqrt(v_hat) (reading above). */
    float mh = r.m / s->c1;
    float vh = r.v / s->c2;
    float den = sqrtf(vh) + hp->eps;
    if (opt == ORC_ADEMAMIX) {
        r.m2 = hp->beta3 * m2 + s->om3 * g;
        float num = mh + hp->alpha * r.m2;
        r.u = num / den;
    } else {
        r.u = mh / den;
    }
    return r;
}

/* Decoupled weight decay.  Decay-first ([PR] intro): both the decay and the
 * update are taken from the previous p,  p' = p (1 - lr wd) - lr u.
 * Decay-after, the ordering the PR removes:  p' = (p - lr u)(1 - lr wd).  */
static float apply_update(const orc_hp *hp, const scalars_t *s, float p, float u)
{
    float step = s->lam * u;
    if (hp->decay_after) {
        float q = p - step;
        return q * s->d;
    }
    float decayed = p * s->d;
    return decayed - step;
}

/* ------------------------------------------------------------------ */
/* Whole-tensor steps.  Arrays hold n elements; g is the gradient widened to
 * fp32.  `scale` is the update-norm scale s_k (1.0f when max_unorm is off).  */

static int step_f32(int opt, const orc_hp *hp, float scale, int64_t n,
                    float *p, const float *g, float *m, float *v, float *m2)
{
    scalars_t s = make_scalars(hp, scale);
    int fresh = fresh_states(hp);
    for (int64_t j = 0; j < n; ++j) {
        float m_old = fresh ? 0.0f : m[j];
        float v_old = fresh ? 0.0f : v[j];
        float m2_old = (opt == ORC_ADEMAMIX && !fresh) ? m2[j] : 0.0f;
        if (skipped(hp, g[j])) {          /* p and the states as they were */
            m[j] = m_old;
            v[j] = v_old;
            if (opt == ORC_ADEMAMIX) m2[j] = m2_old;
            continue;
        }
        moments_t r = moments_and_direction(opt, hp, &s, g[j], m_old, v_old, m2_old);
        p[j] = apply_update(hp, &s, p[j], r.u);
        m[j] = r.m;
        v[j] = r.v;
        if (opt == ORC_ADEMAMIX) m2[j] = r.m2;
    }
    return 0;
}

static int step_bf16(int opt, int stochastic, const orc_hp *hp, float scale, int64_t n,
                     float *p, const float *g, uint16_t *m, uint16_t *v, uint16_t *m2)
{
    scalars_t s = make_scalars(hp, scale);
    int fresh = fresh_states(hp);
    for (int64_t j = 0; j < n; ++j) {
        float m_old = fresh ? 0.0f : orc_bf16_to_f32(m[j]);
        float v_old = fresh ? 0.0f : orc_bf16_to_f32(v[j]);
        float m2_old = (opt == ORC_ADEMAMIX && !fresh) ? orc_bf16_to_f32(m2[j]) : 0.0f;
        if (skipped(hp, g[j])) {          /* a stored BF16 value rounds to itself */
            m[j] = (uint16_t)(f2u(m_old) >> 16);
            v[j] = (uint16_t)(f2u(v_old) >> 16);
            if (opt == ORC_ADEMAMIX) m2[j] = (uint16_t)(f2u(m2_old) >> 16);
            continue;
        }
        moments_t r = moments_and_direction(opt, hp, &s, g[j], m_old, v_old, m2_old);
        /* The parameter update uses the unrounded fp32 moments; rounding
         * happens only at write-back ([SU] Sec. 1.1). */
        p[j] = apply_update(hp, &s, p[j], r.u);
        if (stochastic) {
            int64_t jj = hp->index_base + j;
            uint32_t w = sr_word(hp->seed, hp->step, hp->tensor_index, jj, 0);
            m[j] = orc_bf16_sr(r.m, w & 0xFFFFu);
            v[j] = orc_bf16_sr(r.v, w >> 16);
            if (opt == ORC_ADEMAMIX) {
                uint32_t w2 = sr_word(hp->seed, hp->step, hp->tensor_index, jj, 1);
                m2[j] = orc_bf16_sr(r.m2, w2 & 0xFFFFu);
            }
        } else {
            m[j] = orc_bf16_rne(r.m);
            v[j] = orc_bf16_rne(r.v);
            if (opt == ORC_ADEMAMIX) m2[j] = orc_bf16_rne(r.m2);
        }
    }
    return 0;
}

/* Largest |x| over a block; any NaN makes it NaN ([GN] Correctness
 * properties: a maximum must not silently skip NaNs). */
static float block_absmax(const float *x, int64_t len)
{
    float a = 0.0f;
    for (int64_t i = 0; i < len; ++i) {
        if (isnan(x[i])) return NAN;
        float ax = fabsf(x[i]);
        if (ax > a) a = ax;
    }
    return a;
}

static void quantize_block(const float *T, const float *x, int64_t len, float amax, uint8_t *codes)
{
    for (int64_t i = 0; i < len; ++i) {
        float q = (amax == 0.0f) ? 0.0f : x[i] / amax;
        codes[i] = (uint8_t)orc_quantize(T, q);
    }
}

#define Q8_BLOCK 256

/* 8-bit blockwise states ([PR] intro: the 2-state branch of the blockwise
 * 8-bit kernel; "Why the current tests do not catch it": a zero state
 * quantizes exactly).  Blocks are 256 consecutive elements from element 0 of
 * the tensor; the last block may be short.  m and m2 use the signed codebook
 * qs, v the unsigned codebook qu; each state has its own absmax per block.
 * A stored state reads back as T[code] * absmax.                          */
static int step_q8(int opt, const orc_hp *hp, float scale, int64_t n,
                   float *p, const float *g, uint8_t *c1, uint8_t *c2, uint8_t *c3,
                   float *a1, float *a2, float *a3, const float *qs, const float *qu)
{
    scalars_t s = make_scalars(hp, scale);
    int fresh = fresh_states(hp);
    float bm[Q8_BLOCK], bv[Q8_BLOCK], bm2[Q8_BLOCK];
    for (int64_t b0 = 0, blk = 0; b0 < n; b0 += Q8_BLOCK, ++blk) {
        int64_t len = (n - b0 < Q8_BLOCK) ? n - b0 : Q8_BLOCK;
        for (int64_t i = 0; i < len; ++i) {
            int64_t j = b0 + i;
            float m_old = fresh ? 0.0f : qs[c1[j]] * a1[blk];
            float v_old = fresh ? 0.0f : qu[c2[j]] * a2[blk];
            float m2_old = (opt == ORC_ADEMAMIX && !fresh) ? qs[c3[j]] * a3[blk] : 0.0f;
            if (skipped(hp, g[j])) {      /* the old values, coded again with the block */
                bm[i] = m_old; bv[i] = v_old; bm2[i] = m2_old;
                continue;
            }
            moments_t r = moments_and_direction(opt, hp, &s, g[j], m_old, v_old, m2_old);
            p[j] = apply_update(hp, &s, p[j], r.u);
            bm[i] = r.m; bv[i] = r.v; bm2[i] = r.m2;
        }
        float am = block_absmax(bm, len);
        float av = block_absmax(bv, len);
        quantize_block(qs, bm, len, am, c1 + b0);
        quantize_block(qu, bv, len, av, c2 + b0);
        a1[blk] = am;
        a2[blk] = av;
        if (opt == ORC_ADEMAMIX) {
            float am2 = block_absmax(bm2, len);
            quantize_block(qs, bm2, len, am2, c3 + b0);
            a3[blk] = am2;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* FP8 and FP4 block-scaled states ([SU] Sec. 2.1: an FP8 grid with three
 * fraction bits, 16 times coarser than BF16 at the same scale, and an
 * unsigned FP4 grid E2M2, 32 times coarser, for a state that is never
 * negative; Sec. 5: both formats, with nearest or stochastic rounding).
 *
 * Readings (the pages give the grids and nothing else):
 *  - FP8 is OCP E4M3 (bias 7, no infinities, magnitude 1111.111 is NaN,
 *    largest finite 448) for m, v and m2.
 *  - FP4 keeps v in unsigned E2M2 (bias 1: 0, 1/4, ..., 7/4, 2, ..., 7) and
 *    the signed m and m2 in OCP E2M1 (bias 1: 0, 1/2, 1, 3/2, 2, 3, 4, 6),
 *    the signed 4-bit format the page contrasts E2M2 with.  Two codes share a
 *    byte, element 2i in the low nibble; the high nibble after an odd
 *    tensor's last element is 0.
 *  - Neither grid can hold gradient-sized moments as they are, so every
 *    256-element block is scaled by a power of two taken from its absmax A,
 *    as in the OCP microscaling rule: X = 2^(floor(log2 A) - emax), emax the
 *    exponent of the format's top binade.  A stored element is the rounding
 *    of x / X on the format's grid, clamped to the largest finite value, and
 *    reads back as value(code) * X rounded to binary32.  A power-of-two X
 *    leaves the grid's relative spacing unchanged, which is what the pages'
 *    stall analysis depends on.  The block keeps A itself (fp32), like the
 *    8-bit format.
 *  - Nearest rounding breaks ties to the even code.  Stochastic rounding
 *    takes the element's 16-bit random integer r (as BF16 stochastic
 *    rounding does) and goes up iff floor(f * 2^16) + r >= 2^16, f in [0, 1)
 *    the position of the value across the gap between its two neighbours:
 *    the carry rule of [SU] Sec. 6.1 with the dropped part cut to 16 bits.
 *  - A = 0 reads back as signed zeros; a block whose A is NaN or infinite
 *    stores codes 0 and reads back as NaN.  An E4M3 NaN code reads as NaN.
 */

typedef struct {
    int mbits, bias, maxcode, nan_code, sign;   /* sign: the sign bit, or 0 */
} mini_t;

static const mini_t MINI_E4M3 = {3, 7, 0x7E, 0x7F, 0x80};
static const mini_t MINI_E2M1 = {1, 1, 0x7, -1, 0x8};
static const mini_t MINI_E2M2U = {2, 1, 0xF, -1, 0};

static const mini_t *mini_fmt(int id)
{
    return id == 0 ? &MINI_E4M3 : id == 1 ? &MINI_E2M1 : &MINI_E2M2U;
}

/* The value of a magnitude code: exponent field e, fraction field f. */
static double mini_value(const mini_t *F, int c)
{
    int e = c >> F->mbits, f = c & ((1 << F->mbits) - 1);
    if (e == 0) return ldexp((double)f, 1 - F->bias - F->mbits);
    return ldexp((double)((1 << F->mbits) + f), e - F->bias - F->mbits);
}

static int mini_emax(const mini_t *F) { return (F->maxcode >> F->mbits) - F->bias; }

/* Magnitude code of y >= 0 on the format's grid.  r < 0: nearest, ties to the
 * even code; else stochastic with the 16-bit integer r.  Values at or above
 * the largest finite value take it.  Found by walking the grid from 0. */
static int mini_round(const mini_t *F, double y, int32_t r)
{
    if (!(y > 0.0)) return 0;
    if (y >= mini_value(F, F->maxcode)) return F->maxcode;
    int c = 0;
    while (mini_value(F, c + 1) <= y) ++c;
    double lo = mini_value(F, c), hi = mini_value(F, c + 1);
    if (r < 0) {
        double dl = y - lo, dh = hi - y;
        if (dl < dh) return c;
        if (dh < dl) return c + 1;
        return (c & 1) ? c + 1 : c;
    }
    /* y - lo is exact (y and lo are within a factor of two, or lo = 0) and
     * hi - lo is a power of two, so the product is exact before the floor. */
    uint32_t l = (uint32_t)floor((y - lo) / (hi - lo) * 65536.0);
    return (l + (uint32_t)r >= 65536u) ? c + 1 : c;
}

/* floor(log2 A) - emax, for finite A > 0. */
static int mini_scale_exp(const mini_t *F, float A)
{
    int E;
    frexp((double)A, &E);          /* A = f 2^E with f in [1/2, 1) */
    return (E - 1) - mini_emax(F);
}

static int mini_encode(const mini_t *F, float x, float A, int32_t r)
{
    if (!isfinite(A)) return 0;
    int s = A > 0.0f ? mini_scale_exp(F, A) : 0;
    int c = mini_round(F, ldexp(fabs((double)x), -s), r);
    if (F->sign && signbit(x)) c |= F->sign;
    return c;
}

static float mini_decode(const mini_t *F, int code, float A)
{
    if (!isfinite(A)) return NAN;
    int neg = F->sign && (code & F->sign);
    int mag = F->sign ? (code & (F->sign - 1)) : code;
    if (mag == F->nan_code) return NAN;
    if (A == 0.0f) return neg ? -0.0f : 0.0f;
    float x = (float)ldexp(mini_value(F, mag), mini_scale_exp(F, A));
    return neg ? -x : x;
}

static int mini_get(int nib, const uint8_t *s, int64_t j)
{
    return nib ? (s[j >> 1] >> (4 * (j & 1))) & 0xF : s[j];
}

static void mini_put(int nib, uint8_t *s, int64_t j, int c)
{
    if (!nib) { s[j] = (uint8_t)c; return; }
    int sh = 4 * (int)(j & 1);
    s[j >> 1] = (uint8_t)((s[j >> 1] & ~(0xF << sh)) | (c << sh));
}

/* The 16-bit random integer of element j for state `which`: 0 = m (low half
 * of the element's word), 1 = v (high half), 2 = m2 (low half of the word of
 * the second stream). */
static int32_t rand16(const orc_hp *hp, int64_t j, int which)
{
    uint32_t w = sr_word(hp->seed, hp->step, hp->tensor_index, hp->index_base + j, which == 2);
    return (int32_t)(which == 1 ? w >> 16 : w & 0xFFFFu);
}

static void mini_store_block(const mini_t *F, int nib, int sr, int which, const orc_hp *hp,
                             const float *x, int64_t len, int64_t b0, uint8_t *codes, float *A_out)
{
    float A = block_absmax(x, len);
    *A_out = A;
    for (int64_t i = 0; i < len; ++i)
        mini_put(nib, codes, b0 + i, mini_encode(F, x[i], A, sr ? rand16(hp, b0 + i, which) : -1));
}

static int step_mini(int opt, int fp4, int sr, const orc_hp *hp, float scale, int64_t n,
                     float *p, const float *g, uint8_t *c1, uint8_t *c2, uint8_t *c3,
                     float *a1, float *a2, float *a3)
{
    const mini_t *Fm = fp4 ? &MINI_E2M1 : &MINI_E4M3;
    const mini_t *Fv = fp4 ? &MINI_E2M2U : &MINI_E4M3;
    scalars_t s = make_scalars(hp, scale);
    int fresh = fresh_states(hp);
    float bm[Q8_BLOCK], bv[Q8_BLOCK], bm2[Q8_BLOCK];
    for (int64_t b0 = 0, blk = 0; b0 < n; b0 += Q8_BLOCK, ++blk) {
        int64_t len = (n - b0 < Q8_BLOCK) ? n - b0 : Q8_BLOCK;
        for (int64_t i = 0; i < len; ++i) {
            int64_t j = b0 + i;
            float m_old = 0.0f, v_old = 0.0f, m2_old = 0.0f;
            if (!fresh) {
                m_old = mini_decode(Fm, mini_get(fp4, c1, j), a1[blk]);
                v_old = mini_decode(Fv, mini_get(fp4, c2, j), a2[blk]);
                if (opt == ORC_ADEMAMIX) m2_old = mini_decode(Fm, mini_get(fp4, c3, j), a3[blk]);
            }
            if (skipped(hp, g[j])) {
                bm[i] = m_old; bv[i] = v_old; bm2[i] = m2_old;
                continue;
            }
            moments_t r = moments_and_direction(opt, hp, &s, g[j], m_old, v_old, m2_old);
            p[j] = apply_update(hp, &s, p[j], r.u);
            bm[i] = r.m; bv[i] = r.v; bm2[i] = r.m2;
        }
        mini_store_block(Fm, fp4, sr, 0, hp, bm, len, b0, c1, &a1[blk]);
        mini_store_block(Fv, fp4, sr, 1, hp, bv, len, b0, c2, &a2[blk]);
        if (opt == ORC_ADEMAMIX) mini_store_block(Fm, fp4, sr, 2, hp, bm2, len, b0, c3, &a3[blk]);
    }
    if (fp4 && (n & 1)) {
        c1[n >> 1] &= 0x0F;
        c2[n >> 1] &= 0x0F;
        if (opt == ORC_ADEMAMIX) c3[n >> 1] &= 0x0F;
    }
    return 0;
}

/* Exported for tests: format id 0 = E4M3, 1 = E2M1, 2 = unsigned E2M2. */
double orc_mini_value(int32_t f, int32_t mag) { return mini_value(mini_fmt(f), mag); }
int32_t orc_mini_round(int32_t f, double y, int32_t r) { return mini_round(mini_fmt(f), y, r); }
int32_t orc_mini_encode(int32_t f, float x, float A, int32_t r) { return mini_encode(mini_fmt(f), x, A, r); }
float orc_mini_decode(int32_t f, int32_t code, float A) { return mini_decode(mini_fmt(f), code, A); }
int32_t orc_mini_scale_exp(int32_t f, float A) { return mini_scale_exp(mini_fmt(f), A); }

void orc_mini_round_array(int32_t f, const double *y, const int32_t *r, int32_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mini_round(mini_fmt(f), y[i], r ? r[i] : -1);
}

/* One optimizer step over one tensor.  s1/s2/s3 are m (m1 for AdEMAMix), v,
 * and m2, in the storage of `fmt`: float*, uint16_t* (BF16 bits) or uint8_t*
 * (codes).  Returns 0, or -1 for an unknown optimizer or format.          */
int orc_step(int opt, int fmt, const orc_hp *hp, float scale, int64_t n,
             float *p, const float *g, void *s1, void *s2, void *s3,
             float *a1, float *a2, float *a3, const float *qs, const float *qu)
{
    if (opt != ORC_ADAMW && opt != ORC_ADEMAMIX) return -1;
    switch (fmt) {
    case ORC_F32:
        return step_f32(opt, hp, scale, n, p, g, (float *)s1, (float *)s2, (float *)s3);
    case ORC_BF16_RN:
        return step_bf16(opt, 0, hp, scale, n, p, g, (uint16_t *)s1, (uint16_t *)s2, (uint16_t *)s3);
    case ORC_BF16_SR:
        return step_bf16(opt, 1, hp, scale, n, p, g, (uint16_t *)s1, (uint16_t *)s2, (uint16_t *)s3);
    case ORC_Q8:
        return step_q8(opt, hp, scale, n, p, g, (uint8_t *)s1, (uint8_t *)s2, (uint8_t *)s3,
                       a1, a2, a3, qs, qu);
    case ORC_FP8_RN: case ORC_FP8_SR: case ORC_FP4_RN: case ORC_FP4_SR:
        return step_mini(opt, fmt >= ORC_FP4_RN, fmt == ORC_FP8_SR || fmt == ORC_FP4_SR, hp, scale, n,
                         p, g, (uint8_t *)s1, (uint8_t *)s2, (uint8_t *)s3, a1, a2, a3);
    }
    return -1;
}

/* ------------------------------------------------------------------ */
/* BF16 and FP16 parameters, and the standalone rounding cast ([SU] Sec. 6
 * and 7: FP32 -> BF16 with stochastic rounding as one pass over the tensor;
 * Sec. 8.1: the rounding inside the step; [ISS] Correctness oracle: FP16,
 * BF16 and FP32 parameter storage).
 *
 * Readings:
 *  - a BF16 or FP16 parameter is widened exactly, stepped in fp32 exactly as
 *    an fp32 parameter, and the new value is stored rounded to nearest-even
 *    or stochastically;
 *  - stochastic rounding of a parameter uses the high 16 bits of the word
 *    that the second Philox stream (counter word 3 = k | 2^31) gives the
 *    element, the half that no state uses;
 *  - FP16 stochastic rounding goes up to the next FP16 value iff
 *    floor(f * 2^16) + r >= 2^16, f the position across the gap (the rule
 *    the FP8/FP4 states use); past the largest finite value the next value
 *    is infinity, as for BF16, where the carry of Sec. 6.1 reaches the
 *    exponent;
 *  - the cast's random integer for element j is the low 16 bits of word
 *    j mod 4 of Philox4x32-10 keyed by the seed with counter
 *    (j>>2 low, j>>34, offset low, offset high): tied to the element, with a
 *    fresh offset for each cast ([SU] Sec. 7.3).
 */

/* Positive FP16 magnitude of code c (0 <= c <= 0x7C00; 0x7C00 stands for the
 * first value past the largest finite one, 2^16, which IEEE rounding treats
 * as infinity). */
static double f16_value(int c)
{
    int e = c >> 10, f = c & 1023;
    if (e == 0) return ldexp((double)f, -24);
    return ldexp((double)(1024 + f), e - 25);
}

/* Largest code c with f16_value(c) <= y, for 0 <= y < 2^16 (bisection). */
static int f16_floor_code(double y)
{
    int lo = 0, hi = 0x7C00;           /* f16_value(lo) <= y < f16_value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (f16_value(mid) <= y) lo = mid;
        else hi = mid;
    }
    return lo;
}

/* FP32 -> FP16 bits; r < 0: nearest-even, else stochastic with the 16-bit r. */
static uint16_t f16_round(float x, int32_t r)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    double y = fabs((double)x);
    if (y >= 65536.0) return (uint16_t)(sign | 0x7C00u);
    int c = f16_floor_code(y);
    double lo = f16_value(c), hi = f16_value(c + 1);
    int up;
    if (r < 0) {
        double dl = y - lo, dh = hi - y;
        up = dl > dh || (dl == dh && (c & 1));
    } else {
        uint32_t l = (uint32_t)floor((y - lo) / (hi - lo) * 65536.0);
        up = l + (uint32_t)r >= 65536u;
    }
    return (uint16_t)(sign | (c + up));
}

uint16_t orc_f16_rne(float x) { return f16_round(x, -1); }
uint16_t orc_f16_sr(float x, uint32_t r) { return f16_round(x, (int32_t)(r & 0xFFFFu)); }

float orc_f16_to_f32(uint16_t h)
{
    int e = (h >> 10) & 31, f = h & 1023;
    float v;
    if (e == 31) v = f ? NAN : INFINITY;
    else v = (float)(e ? ldexp((double)(1024 + f), e - 25) : ldexp((double)f, -24));
    return (h & 0x8000u) ? -v : v;
}

enum { ORC_P_F32 = 0, ORC_P_BF16 = 1, ORC_P_F16 = 2 };

static uint16_t round16(int dtype, float x, int32_t r)
{
    if (dtype == ORC_P_BF16) return r < 0 ? orc_bf16_rne(x) : orc_bf16_sr(x, (uint32_t)r);
    return f16_round(x, r);
}

/* One step over a tensor whose parameters are stored as BF16 or FP16 words:
 * widen, step as fp32, store rounded (p_sr: stochastically). */
int orc_step_p16(int opt, int fmt, const orc_hp *hp, float scale, int64_t n, uint16_t *p16,
                 int32_t p_dtype, int32_t p_sr, const float *g, void *s1, void *s2, void *s3,
                 float *a1, float *a2, float *a3, const float *qs, const float *qu, float *work)
{
    if (p_dtype != ORC_P_BF16 && p_dtype != ORC_P_F16) return -1;
    for (int64_t j = 0; j < n; ++j)
        work[j] = p_dtype == ORC_P_BF16 ? orc_bf16_to_f32(p16[j]) : orc_f16_to_f32(p16[j]);
    int rc = orc_step(opt, fmt, hp, scale, n, work, g, s1, s2, s3, a1, a2, a3, qs, qu);
    if (rc) return rc;
    for (int64_t j = 0; j < n; ++j) {
        int32_t r = -1;
        if (p_sr) r = (int32_t)(sr_word(hp->seed, hp->step, hp->tensor_index, hp->index_base + j, 1) >> 16);
        p16[j] = round16(p_dtype, work[j], r);
    }
    return 0;
}

/* The standalone cast of n fp32 values to BF16 or FP16 words. */
void orc_round_cast(const float *x, uint16_t *out, int64_t n, int32_t dtype, int32_t stochastic,
                    uint64_t seed, uint64_t offset)
{
    for (int64_t j = 0; j < n; ++j) {
        int32_t r = -1;
        if (stochastic) {
            uint32_t ctr[4], key[2], w[4];
            uint64_t q = (uint64_t)j >> 2;
            ctr[0] = (uint32_t)q; ctr[1] = (uint32_t)(q >> 32);
            ctr[2] = (uint32_t)offset; ctr[3] = (uint32_t)(offset >> 32);
            key[0] = (uint32_t)seed; key[1] = (uint32_t)(seed >> 32);
            orc_philox4x32_10(ctr, key, w);
            r = (int32_t)(w[j & 3] & 0xFFFFu);
        }
        out[j] = round16(dtype, x[j], r);
    }
}

void orc_f16_array(const float *x, const uint32_t *r, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f16_round(x[i], r ? (int32_t)(r[i] & 0xFFFFu) : -1);
}

/* ------------------------------------------------------------------ */
/* One-state optimizers ([PR] intro: the 1-state kernels use coupled L2
 * for momentum, RMSprop and Adagrad, and decoupled decay for Lion).
 *
 * Readings (the pages name the family and how each couples the decay):
 *  - coupled L2: when wd != 0 the gradient becomes g' = g + wd*p before it
 *    enters the state, and the update carries no separate decay;
 *  - momentum (heavy ball, as torch.optim.SGD with dampening 0): m' = g' on
 *    the state's first step, else m' = b1*m + g'; p' = p - lr*m';
 *  - RMSprop (as torch.optim.RMSprop, alpha = b1):
 *    v' = b1*v + (1-b1)*g'^2, p' = p - lr*(g'/(sqrt(v') + eps));
 *  - Adagrad (as torch.optim.Adagrad with no lr decay): v' = v + g'^2,
 *    p' = p - lr*(g'/(sqrt(v') + eps));
 *  - Lion (Chen et al., "Symbolic Discovery of Optimization Algorithms"):
 *    c = b1*m + (1-b1)*g, p' = p*(1 - lr*wd) - lr*sign(c) (sign(0) = 0),
 *    m' = b2*m + (1-b2)*g;
 *  - the state is fp32 or BF16 (nearest, or stochastic with the low half of
 *    the element's first-stream word); grad_scale, skip_zeros and resets act
 *    as for the two-state optimizers.
 */
enum { ORC_MOMENTUM = 2, ORC_RMSPROP = 3, ORC_ADAGRAD = 4, ORC_LION = 5 };

static float sign_f(float c)
{
    if (c != c) return c;
    return c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f);
}

int orc_step_1state(int opt, int fmt, const orc_hp *hp, int64_t n, float *p, const float *g, void *s1)
{
    if (opt < ORC_MOMENTUM || opt > ORC_LION) return -1;
    if (fmt != ORC_F32 && fmt != ORC_BF16_RN && fmt != ORC_BF16_SR) return -1;
    int fresh = fresh_states(hp);
    int first = cycle_step(hp) == 1;
    float om1 = 1.0f - hp->beta1, om2 = 1.0f - hp->beta2;
    float lrwd = hp->lr * hp->weight_decay;
    float d = 1.0f - lrwd;
    for (int64_t j = 0; j < n; ++j) {
        float s_old;
        if (fresh) s_old = 0.0f;
        else if (fmt == ORC_F32) s_old = ((float *)s1)[j];
        else s_old = orc_bf16_to_f32(((uint16_t *)s1)[j]);
        float s_new = s_old;
        if (!skipped(hp, g[j])) {
            float gs = g[j] * hp->grad_scale;
            float gp = gs;
            if (opt != ORC_LION && hp->weight_decay != 0.0f) gp = gs + hp->weight_decay * p[j];
            if (opt == ORC_MOMENTUM) {
                s_new = first ? gp : hp->beta1 * s_old + gp;
                p[j] = p[j] - hp->lr * s_new;
            } else if (opt == ORC_RMSPROP || opt == ORC_ADAGRAD) {
                float gg = gp * gp;
                s_new = opt == ORC_RMSPROP ? hp->beta1 * s_old + om1 * gg : s_old + gg;
                float den = sqrtf(s_new) + hp->eps;
                float u = gp / den;
                p[j] = p[j] - hp->lr * u;
            } else {
                float c = hp->beta1 * s_old + om1 * gs;
                float decayed = p[j] * d;
                p[j] = decayed - hp->lr * sign_f(c);
                s_new = hp->beta2 * s_old + om2 * gs;
            }
        }
        if (fmt == ORC_F32) {
            ((float *)s1)[j] = s_new;
        } else if (fmt == ORC_BF16_RN || s_new == s_old) {
            ((uint16_t *)s1)[j] = orc_bf16_rne(s_new);   /* a stored value rounds to itself */
        } else {
            uint32_t w = sr_word(hp->seed, hp->step, hp->tensor_index, hp->index_base + j, 0);
            ((uint16_t *)s1)[j] = orc_bf16_sr(s_new, w & 0xFFFFu);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Update-norm pre-pass ([ISS] Problem: the precondition kernel used when
 * max_unorm > 0 recomputes the would-be update and accumulates its norm).
 * U2 = sum_j u_j^2 and P2 = sum_j p_j^2 for one tensor, with u the direction
 * of the step (no lr, no decay) and p the parameter before the step, summed
 * in element order in binary64 with Neumaier's compensation.             */

typedef struct { double s, c; } nsum_t;

/* The compensated total; once the running sum is infinite or NaN the
 * compensation term is meaningless (inf - inf), and the sum itself is it. */
static double nsum_total(const nsum_t *a)
{
    return isfinite(a->s) ? a->s + a->c : a->s;
}

static void nsum_add(nsum_t *a, double x)
{
    double t = a->s + x;
    if (fabs(a->s) >= fabs(x)) a->c += (a->s - t) + x;
    else a->c += (x - t) + a->s;
    a->s = t;
}

int orc_unorm(int opt, int fmt, const orc_hp *hp, int64_t n, const float *p, const float *g,
              const void *s1, const void *s2, const void *s3,
              const float *a1, const float *a2, const float *a3,
              const float *qs, const float *qu, double out[2])
{
    if (opt != ORC_ADAMW && opt != ORC_ADEMAMIX) return -1;
    if (fmt < ORC_F32 || fmt > ORC_FP4_SR) return -1;
    scalars_t s = make_scalars(hp, 1.0f);
    int fresh = fresh_states(hp);
    int fp4 = fmt >= ORC_FP4_RN;
    const mini_t *Fm = fp4 ? &MINI_E2M1 : &MINI_E4M3;
    const mini_t *Fv = fp4 ? &MINI_E2M2U : &MINI_E4M3;
    nsum_t su = {0.0, 0.0}, sp = {0.0, 0.0};
    for (int64_t j = 0; j < n; ++j) {
        float m, v, m2 = 0.0f;
        if (fresh) {
            m = v = 0.0f;
        } else if (fmt >= ORC_FP8_RN) {
            int64_t blk = j / Q8_BLOCK;
            m = mini_decode(Fm, mini_get(fp4, (const uint8_t *)s1, j), a1[blk]);
            v = mini_decode(Fv, mini_get(fp4, (const uint8_t *)s2, j), a2[blk]);
            if (opt == ORC_ADEMAMIX) m2 = mini_decode(Fm, mini_get(fp4, (const uint8_t *)s3, j), a3[blk]);
        } else if (fmt == ORC_F32) {
            m = ((const float *)s1)[j];
            v = ((const float *)s2)[j];
            if (opt == ORC_ADEMAMIX) m2 = ((const float *)s3)[j];
        } else if (fmt == ORC_Q8) {
            int64_t blk = j / Q8_BLOCK;
            m = qs[((const uint8_t *)s1)[j]] * a1[blk];
            v = qu[((const uint8_t *)s2)[j]] * a2[blk];
            if (opt == ORC_ADEMAMIX) m2 = qs[((const uint8_t *)s3)[j]] * a3[blk];
        } else {
            m = orc_bf16_to_f32(((const uint16_t *)s1)[j]);
            v = orc_bf16_to_f32(((const uint16_t *)s2)[j]);
            if (opt == ORC_ADEMAMIX) m2 = orc_bf16_to_f32(((const uint16_t *)s3)[j]);
        }
        moments_t r = moments_and_direction(opt, hp, &s, g[j], m, v, m2);
        if (skipped(hp, g[j])) r.u = 0.0f;   /* no update for this element */
        nsum_add(&su, (double)r.u * (double)r.u);
        nsum_add(&sp, (double)p[j] * (double)p[j]);
    }
    out[0] = nsum_total(&su);
    out[1] = nsum_total(&sp);
    return 0;
}

/* The update-norm scale: min(1, max_unorm * ||p|| / ||u||), rounded to fp32;
 * 1 when max_unorm <= 0 (the precondition pass runs only when max_unorm > 0,
 * [ISS] Problem) or when ||u|| does not exceed the bound.               */
float orc_unorm_scale(float max_unorm, double u2, double p2)
{
    if (!(max_unorm > 0.0f)) return 1.0f;
    double un = sqrt(u2), bound = (double)max_unorm * sqrt(p2);
    if (un > bound) return (float)(bound / un);
    return 1.0f;
}

/* ------------------------------------------------------------------ */
/* Array forms of the element functions above, for exhaustive tests.    */

void orc_bf16_rne_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

void orc_bf16_sr_array(const float *x, const uint32_t *r, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_sr(x[i], r[i]);
}

void orc_quantize_array(const float *T, const float *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_quantize(T, x[i]);
}

void orc_sr_words(uint64_t seed, int64_t t, int32_t k, int64_t j0, int64_t n, int32_t stream,
                  uint32_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = sr_word(seed, t, k, j0 + i, stream);
}

/* ------------------------------------------------------------------ */
/* Gradient norms for clipping ([GN] What and Numerics: the 2-norm and the
 * inf-norm of a list of gradients, accumulated in binary64, with NaN
 * propagating into both).  For one tensor: out[0] = sum_j g_j^2 (binary64,
 * element order, Neumaier compensation; each g_j^2 is exact in binary64),
 * out[1] = max_j |g_j|, NaN if any g_j is NaN ("tl.maximum follows IEEE
 * maxNum and ignores NaN ... the kernel counts NaNs and poisons the
 * partial").                                                             */
void orc_grad_norm(const float *g, int64_t n, double out[2])
{
    nsum_t s = {0.0, 0.0};
    double mx = 0.0;
    int nan_seen = 0;
    for (int64_t j = 0; j < n; ++j) {
        double x = (double)g[j];
        nsum_add(&s, x * x);
        if (isnan(x)) nan_seen = 1;
        else if (fabs(x) > mx) mx = fabs(x);
    }
    out[0] = nsum_total(&s);
    out[1] = nan_seen ? NAN : mx;
}

/* The clipping coefficient for a total norm: max_norm / (norm + 1e-6),
 * capped at 1, formed in binary64 and rounded to binary32 (reading: the
 * formula of torch.nn.utils.clip_grad_norm_, which the clipping in [GN]
 * reimplements).  A NaN norm gives NaN.                                  */
float orc_clip_coef(double norm, float max_norm)
{
    double c = (double)max_norm / (norm + 1e-6);
    if (isnan(c)) return NAN;
    return (float)(c < 1.0 ? c : 1.0);
}

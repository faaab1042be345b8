/*
 * opt_step.h -- C ABI of the MI355X (gfx950) fused element-wise two-state
 * optimizer step: AdamW and AdEMAMix with decoupled weight decay applied in
 * the decay-first order, optimizer states stored as fp32, BF16 (nearest or
 * stochastic rounding) or 8-bit blockwise codes, and a deterministic
 * update-norm pre-pass for max_unorm.
 *
 * The operation (sources are the four pages this library is built from):
 *  - decay-first AdamW, p' = p*(1 - lr*wd) - lr*u with u = m_hat/(sqrt(v_hat)+eps):
 *    bitsandbytes PR "Fix decoupled weight decay ordering in the CUDA
 *    Adam/AdEMAMix kernels", intro (both terms from the same previous p);
 *  - AdEMAMix (the rule that PR cites): a slow EMA m2 with beta3, mixed into
 *    the numerator with alpha, u = (m1_hat + alpha*m2)/(sqrt(v_hat)+eps);
 *  - the EMAs m' = b1*m + (1-b1)*g, v' = b2*v + (1-b2)*g^2 and BF16 storage
 *    with nearest or stochastic rounding: "When Small Updates Disappear",
 *    Sec. 1.1, 3, 6.1 and 8.1 (the fused step with BF16 moments);
 *  - 8-bit blockwise states, one absmax per 256-element block: the blockwise
 *    8-bit kernel of the bitsandbytes PR;
 *  - FP8 and FP4 states with nearest or stochastic rounding, and periodic
 *    state resets: "When Small Updates Disappear", Sec. 2.1 (an FP8 grid with
 *    three fraction bits, an unsigned E2M2 FP4 grid) and Sec. 5 (both fixes);
 *  - the max_unorm precondition pass and its per-tensor norm buffer: issue
 *    "Investigate SM103 bias-correction broadcast in 32-bit optimizers",
 *    Problem and Result (here without atomics, so bit-reproducible).
 *
 * Arithmetic.  Each element's moments are formed in binary32 in the fixed
 * order m' = fl(fl(b1*m) + fl((1-b1)*g)), v' = fl(fl(b2*v) + fl((1-b2)*fl(g*g))),
 * m2' = fl(fl(b3*m2) + fl((1-b3)*g)), with no fused multiply-add, so BF16 and
 * 8-bit results are bit-reproducible.  The update uses these unrounded fp32
 * moments; rounding or quantization happens only when they are stored.
 * Bias corrections c = 1 - beta^t are formed in binary64 and rounded once.
 * The direction u feeds the parameter alone.  For an fp32 parameter it is
 * formed with the hardware reciprocal and square root (a few ulp from the
 * correctly rounded recipe; the recipe itself for a tiny v_hat).  A 16-bit
 * parameter stores the word the correctly rounded recipe's value rounds to:
 * the kernels use the fast direction only where its error bound proves that
 * word (opt_debug_direction exposes both directions and the bound).
 *
 * Calls and memory.  Every call is asynchronous on `stream` (a hipStream_t
 * passed as void*; NULL is the null stream).  All tensors, states and the
 * unorm buffer are caller-owned device memory; the library touches them
 * only through the work a call enqueues.  It owns a small per-device
 * workspace (tensor tables, codebook search tables, norm partials) that it
 * grows on demand and releases in opt_shutdown, and it remembers the tensor
 * records (pointers and sizes) of recent calls to recognise a repeated call
 * and reuse its device tables.  Calls from several host threads are
 * serialized inside the library.
 *
 * Errors.  Every entry point returns OPT_OK (0) or a negative status, and
 * opt_last_error() then describes the failure.  Invalid arguments are found
 * before anything is enqueued.  A HIP error while enqueuing (OPT_EHIP) may
 * leave the launches of earlier storage buckets of the same call queued.
 */
#ifndef OPT_STEP_H
#define OPT_STEP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define OPT_OK            0
#define OPT_EINVAL       (-1)  /* null pointer, negative size, step < 1, bad enum, bad codebook */
#define OPT_EUNSUPPORTED (-2)  /* a dtype / format / optimizer combination not provided        */
#define OPT_EALIGN       (-3)  /* a device pointer not aligned as required (see opt_tensor)    */
#define OPT_EHIP         (-4)  /* a HIP runtime error; its text is in opt_last_error()         */

/* ---- enumerations -------------------------------------------------------- */
typedef enum { OPT_F32 = 0, OPT_BF16 = 1, OPT_F16 = 2 } opt_dtype;

typedef enum {
    OPT_STATE_F32 = 0,      /* fp32 words                                          */
    OPT_STATE_BF16_RN = 1,  /* BF16 words, round to nearest even on store          */
    OPT_STATE_BF16_SR = 2,  /* BF16 words, stochastic rounding with Philox4x32-10  */
    OPT_STATE_Q8 = 3,       /* 8-bit codes + one fp32 absmax per 256 elements      */
    OPT_STATE_FP8_RN = 4,   /* E4M3 codes + one fp32 absmax per 256 elements,
                               nearest-even                                        */
    OPT_STATE_FP8_SR = 5,   /* the same, stochastic rounding                       */
    OPT_STATE_FP4_RN = 6,   /* 4-bit codes (m, m2: E2M1; v: unsigned E2M2), two
                               per byte, + one fp32 absmax per 256 elements        */
    OPT_STATE_FP4_SR = 7    /* the same, stochastic rounding                       */
} opt_state_fmt;

typedef enum {
    OPT_ADAMW = 0, OPT_ADEMAMIX = 1,                                  /* two states  */
    OPT_MOMENTUM = 2, OPT_RMSPROP = 3, OPT_ADAGRAD = 4, OPT_LION = 5  /* one state   */
} opt_optimizer;

/* ---- one tensor of the multi-tensor list --------------------------------
 * All pointers are device pointers owned by the caller.
 *   p        numel parameters in p_dtype, read and written: OPT_F32, or
 *            OPT_BF16 / OPT_F16 with any state format (the two-state steps;
 *            the one-state optimizers take OPT_F32 only).  A 16-bit value is
 *            widened exactly, stepped in fp32, and stored back rounded to
 *            nearest-even or stochastically (hp->p_rounding).
 *   g        numel gradients in g_dtype (OPT_F32, OPT_BF16 or OPT_F16), read.
 *   s1       first moment m (AdamW) or fast EMA m1 (AdEMAMix), read and written.
 *   s2       second moment v, read and written.
 *   s3       AdEMAMix's slow EMA m2, read and written; NULL for AdamW.
 *            State storage: OPT_STATE_F32 -> float[numel]; BF16 formats ->
 *            uint16_t[numel] BF16 words; OPT_STATE_Q8 and FP8 -> uint8_t[numel]
 *            codes; FP4 -> uint8_t[ceil(numel/2)], element 2i in the low
 *            nibble of byte i (after an odd tensor's last element the high
 *            nibble is written as 0).
 *   absmax1..3  Q8, FP8 and FP4 only: float[ceil(numel/256)] per-block absmax
 *            of s1..s3; NULL otherwise.  Blocks are 256 consecutive elements
 *            from element 0 of the tensor; the last block may be short.
 *            FP8/FP4 code a block's values as x / X, X = 2^(floor(log2 A) -
 *            emax) with A its absmax and emax 8 (E4M3) or 2 (E2M1, E2M2),
 *            clamped to the largest finite value (448, 6, 7); they read back
 *            as value(code) * X.  A block whose A is 0 reads back as zeros,
 *            one whose A is NaN or infinite as NaN.
 *   numel    element count, 0 <= numel <= 2^46 (0 is a no-op); index_base +
 *            numel <= 2^60.
 * Alignment: p, g, s1, s2, s3 must be 16-byte aligned (any PyTorch allocation
 * is); absmax arrays 4-byte aligned.  Buffers of different tensors must not
 * overlap.  The tensor's position k in the list keys its stochastic rounding
 * unless sr_tensor_set says otherwise; element j of the record is element
 * index_base + j of its tensor for that purpose.  A zero-initialised record
 * (index_base 0, sr_tensor_set 0) is a whole tensor keyed by its position.
 * A fresh 8-bit state is every code set to the code of 0 (127 for a signed
 * table whose entry 127 is 0, 0 for an unsigned table) and absmax 0; a fresh
 * FP8 or FP4 state is all-zero bytes and absmax 0.
 */
typedef struct {
    void *p;
    const void *g;
    void *s1, *s2, *s3;
    float *absmax1, *absmax2, *absmax3;
    int64_t numel;
    int32_t p_dtype;
    int32_t g_dtype;
    int64_t index_base;     /* index, within the whole tensor, of this record's element 0 (0 for a
                               whole tensor).  A record that holds a slice of a tensor (one rank's
                               shard) steps exactly as that part of the whole tensor would: the
                               stochastic-rounding counter takes index_base + j as the element
                               index.  >= 0 and a multiple of 4; a multiple of 256 for the 8-bit,
                               FP8 and FP4 formats, so the slice's blocks are the tensor's.      */
    int32_t sr_tensor;      /* the tensor number k of the stochastic-rounding counter when
                               sr_tensor_set is 1 (0 <= sr_tensor < 2^31), so that a slice keeps
                               its tensor's stream whatever its position in this list           */
    int32_t sr_tensor_set;  /* 0: k is the record's position in the list; 1: k is sr_tensor     */
} opt_tensor;

/* ---- hyper-parameters -----------------------------------------------------
 *   lr, weight_decay   decay-first: p' = p*(1 - lr*wd) - lr*s_k*u.
 *   beta1, beta2, eps  AdamW moments, 0 <= beta < 1; eps is added to sqrt(v_hat).
 *   beta3, alpha       AdEMAMix slow EMA (0 <= beta3 <= 1) and its mixing
 *                      weight (both ignored by AdamW).
 *   max_unorm          > 0: scale the update of tensor k by
 *                      s_k = min(1, max_unorm*||p_k|| / ||u_k||), from the norms
 *                      opt_precondition_unorm wrote; <= 0: off (s_k = 1).
 *   step               t >= 1; the bias corrections are 1 - beta1^t, 1 - beta2^t.
 *   seed               Philox key of the stochastic-rounding formats: element j
 *                      of tensor k at step t draws word j%4 of Philox4x32-10 with
 *                      counter (j>>2 low, j>>34, t, k) [k | 2^31 for m2]; the low
 *                      16 bits r round m (and m2), the high 16 bits round v.
 *                      BF16: add r to the fp32 word, keep the high half.  FP8/FP4:
 *                      up to the next grid value iff floor(f * 2^16) + r >= 2^16,
 *                      f the position of x / X across its grid gap.
 *   qmap_signed        OPT_STATE_Q8 only: HOST pointer to 256 floats, strictly
 *                      increasing, finite, within [-1, 1]; codebook of m and m2.
 *   qmap_unsigned      OPT_STATE_Q8 only: HOST pointer to 256 floats as above,
 *                      all >= 0; codebook of v.  The library copies both during
 *                      the call.  A code is the index of the nearest entry to
 *                      x = m'/absmax (ties to the lower index; NaN -> 0).
 */
typedef struct {
    float lr, beta1, beta2, beta3, alpha, eps, weight_decay, max_unorm;
    int64_t step;
    uint64_t seed;
    const float *qmap_signed;
    const float *qmap_unsigned;
    const float *grad_scale;    /* DEVICE pointer to one float, or NULL: the step
                                   uses fl(g * (*grad_scale)) in place of g, read
                                   when the kernel runs (so a clipping coefficient
                                   that opt_grad_norm writes earlier on the same
                                   stream fuses into the step); NULL means 1. */
    int32_t p_rounding;         /* BF16/FP16 parameters: 0 nearest-even, 1
                                   stochastic with the high 16 bits of the
                                   element's word from the second Philox
                                   stream (counter word 3 = k | 2^31); FP16
                                   goes up iff floor(f * 2^16) + r >= 2^16, f
                                   the position across the gap, infinity
                                   past 65504.                               */
    int32_t reserved;           /* 0 */
    int64_t reset_interval;     /* R > 0: the moments restart from zero at
                                   steps 1, R+1, 2R+1, ... (the stored states are
                                   not read on those steps) and the bias
                                   corrections count from there: 1 - beta^t'
                                   with t' = (t-1) mod R + 1; the random stream
                                   keeps the absolute t.  0: never.          */
    int32_t skip_zeros;         /* 1: an element whose gradient is exactly 0
                                   keeps its parameter (no decay either) and
                                   its stored moments (blockwise formats code
                                   the old values again against the block's
                                   new absmax); the update-norm pre-pass
                                   counts no update for it.  bitsandbytes PR
                                   "Fix decoupled weight decay ordering ...",
                                   Not covered.                              */
    int32_t reserved2;          /* 0 */
} opt_hparams;

/* One AdamW step over the n tensors of `tensors` (host array, read during the
 * call only), with decoupled weight decay applied decay-first: per element,
 * in binary32, m' = b1*m + (1-b1)*g, v' = b2*v + (1-b2)*g^2 ("When Small
 * Updates Disappear", Sec. 1.1), u = (m'/c1)/(sqrt(v'/c2) + eps) with
 * c = 1 - beta^t, and p' = p*(1 - lr*wd) - lr*s_k*u, both terms from the old
 * p (bitsandbytes PR "Fix decoupled weight decay ordering in the CUDA
 * Adam/AdEMAMix kernels", intro); s_k is the update-norm scale (1 unless
 * max_unorm > 0).  Tensors are grouped by gradient and parameter storage and
 * each group runs as one kernel launch over a host-built chunk table (NeMo
 * Automodel PR "perf(training): fused multi-tensor gradient-norm
 * reduction", What).  Errors: negative status, nothing enqueued.
 * unorm: device double[2*n] written by opt_precondition_unorm with the same
 * tensors, format and hyper-parameters, on the same stream, before this call;
 * required when hp->max_unorm > 0 and ignored otherwise. */
int opt_step_adamw(const opt_tensor *tensors, int64_t n, int32_t state_fmt,
                   const opt_hparams *hp, const double *unorm, void *stream);

/* opt_step_adamw for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results, with the call's tables (tensor
 * records, chunk table, 8-bit lookup tables) copied into one fixed 2 MiB
 * device array that each GPU the library runs on holds until the process
 * ends, instead of the library's grown workspace.  It calls no hipMalloc,
 * hipFree or other allocating routine.  A list whose tables exceed 2 MiB
 * (about 500,000 chunks of the current chunk size, with the tensor records)
 * returns OPT_EUNSUPPORTED before anything is enqueued.  Every call on a GPU
 * rewrites that GPU's array: calls in order on one stream are safe; calls
 * that overlap on one GPU (other streams or threads) race, and the caller
 * must order them. */
int opt_step_adamw_noalloc(const opt_tensor *tensors, int64_t n, int32_t state_fmt,
                           const opt_hparams *hp, const double *unorm, void *stream);

/* One AdEMAMix step (the rule the bitsandbytes PR "Fix decoupled weight
 * decay ordering in the CUDA Adam/AdEMAMix kernels" intro cites, Pagliardini
 * et al.): as opt_step_adamw plus the slow EMA m2' = b3*m2 + (1-b3)*g, kept in
 * s3, and u = (m1'/c1 + alpha*m2')/(sqrt(v'/c2) + eps) (m2 is not
 * bias-corrected).  Arguments as opt_step_adamw, with s3 (and absmax3 for the
 * blockwise formats) required for every tensor. */
int opt_step_ademamix(const opt_tensor *tensors, int64_t n, int32_t state_fmt,
                      const opt_hparams *hp, const double *unorm, void *stream);

/* One step of a one-state optimizer (bitsandbytes PR "Fix decoupled weight
 * decay ordering in the CUDA Adam/AdEMAMix kernels", intro: the 1-state
 * kernels use coupled L2 for momentum, RMSprop and Adagrad and decoupled
 * decay for Lion).  optimizer: OPT_MOMENTUM, OPT_RMSPROP, OPT_ADAGRAD or
 * OPT_LION.  Each tensor needs p (fp32), g and s1 (the state; s2, s3 and the
 * absmax arrays are ignored); state_fmt OPT_STATE_F32, _BF16_RN or _BF16_SR
 * (others: OPT_EUNSUPPORTED).  Per element, in binary32, g' = g*grad_scale,
 * plus wd*p for the coupled-L2 three when wd != 0:
 *   momentum  m' = g' on the state's first step (t = 1 or a reset), else
 *             b1*m + g';  p' = p - lr*m'
 *   RMSprop   v' = b1*v + (1-b1)*g'^2;  p' = p - lr*(g'/(sqrt(v') + eps))
 *   Adagrad   v' = v + g'^2;            p' = p - lr*(g'/(sqrt(v') + eps))
 *   Lion      c = b1*m + (1-b1)*g';  p' = p*(1 - lr*wd) - lr*sign(c), sign(0) = 0;
 *             m' = b2*m + (1-b2)*g'
 * beta1 in [0, 1]; max_unorm must be <= 0; seed, skip_zeros, grad_scale and
 * reset_interval act as for the two-state steps (SR: the low 16 bits of the
 * element's first-stream word). */
int opt_step_1state(int32_t optimizer, const opt_tensor *tensors, int64_t n, int32_t state_fmt,
                    const opt_hparams *hp, void *stream);

/* The max_unorm pre-pass: for each tensor k, recompute the direction u of the
 * coming step (no lr, no decay) from p, g and the states without writing them,
 * and store unorm_out[2k] = sum u^2 and unorm_out[2k+1] = sum p^2, in binary64.
 * Deterministic: per-chunk partials reduced in a fixed order, no atomics, so
 * repeated calls give the same bits.  unorm_out is device double[2*n]. */
int opt_precondition_unorm(int32_t optimizer, const opt_tensor *tensors, int64_t n,
                           int32_t state_fmt, const opt_hparams *hp, double *unorm_out,
                           void *stream);

/* ---- gradient norms for clipping --------------------------------------
 * NeMo Automodel PR "perf(training): fused multi-tensor gradient-norm
 * reduction": the 2-norm and the inf-norm of a list of gradients in one
 * launch per dtype, accumulated in binary64 after widening in registers,
 * deterministic (fixed tiles and reduction order, no atomics), with NaN
 * poisoning the inf-norm as well as the 2-norm. */
typedef struct {
    const void *g;      /* device, numel gradients in dtype, read      */
    int64_t numel;      /* 0 <= numel <= 2^46                           */
    int32_t dtype;      /* OPT_F32 or OPT_BF16                          */
    int32_t reserved;   /* 0                                            */
} opt_grad;

/* out: device double[2 + 2n].  out[0] = sum of g^2 over every element of
 * every tensor, out[1] = max |g| over all of them (NaN if any g is NaN);
 * out[2 + 2k], out[3 + 2k]: the same for tensor k alone.  If coef_out is not
 * NULL (device float[1]) it receives the clipping coefficient
 * min(1, max_norm / (norm + 1e-6)) with norm = sqrt(out[0]) for norm_type 2
 * or out[1] for norm_type 0 (the inf-norm); pass it as hp->grad_scale of a
 * later step on the same stream.  g must be 16-byte aligned. */
int opt_grad_norm(const opt_grad *grads, int64_t n, double *out, float max_norm, int32_t norm_type,
                  float *coef_out, void *stream);

/* The standalone rounding cast ("When Small Updates Disappear", Sec. 6 and 7:
 * FP32 -> BF16 in one pass, stochastic rounding costing about as much as
 * nearest).  x: device float[n] (16-byte aligned); out: device uint16_t[n]
 * (8-byte aligned) of BF16 (out_dtype OPT_BF16) or FP16 (OPT_F16) words.
 * stochastic 0: nearest-even.  1: element j draws the low 16 bits r of word
 * j%4 of Philox4x32-10 keyed by `seed` with counter (j>>2 low, j>>34, offset
 * low, offset high) -- tied to the element, so any launch shape gives the
 * same words; pass a new offset for each cast.  BF16 adds r to the fp32 word
 * and keeps the high half (Sec. 6.1); FP16 rounds as for parameters. */
int opt_round_cast(const float *x, void *out, int64_t n, int32_t out_dtype, int32_t stochastic, uint64_t seed,
                   uint64_t offset, void *stream);

/* Test hook: the FP8/FP4 element codec of the state formats.  elem 0 = E4M3,
 * 1 = E2M1, 2 = unsigned E2M2.  For i < n: codes[i] = the code of x[i] in a
 * block whose absmax is A (A >= 0 or NaN), nearest-even if r is NULL, else
 * stochastic with the 16-bit integer r[i] & 0xFFFF; decoded[i] = the value
 * that code reads back as.  Device arrays, asynchronous on `stream`. */
int opt_debug_mini(int32_t elem, float A, const float *x, const uint32_t *r, uint8_t *codes, float *decoded,
                   int64_t n, void *stream);

/* The step's encoder for the same formats: codes[i] for groups of four values
 * of one block with absmax A, as the blockwise step forms them (gfx950's
 * scaled conversions for E4M3 stochastic, E2M1, and unsigned E2M2 stochastic
 * through E5M2; integer rounding otherwise).  n a multiple of 4; r as for
 * opt_debug_mini.  Device arrays, asynchronous on `stream`.  OPT_EINVAL for a
 * bad elem, n, A or NULL array. */
int opt_debug_mini_pack(int32_t elem, float A, const float *x, const uint32_t *r, uint8_t *codes, int64_t n,
                        void *stream);

/* The same, computed on the host from the same source (host arrays). */
int opt_debug_mini_host(int32_t elem, float A, const float *x, const uint32_t *r, uint8_t *codes,
                        float *decoded, int64_t n);

/* Text of the last failure on the calling thread ("" if none). */
const char *opt_last_error(void);

/* Wait for the library's outstanding work and free its workspace on every
 * device.  Later calls re-create it. */
int opt_shutdown(void);

/* ---- test hooks (the same device functions the step kernels use) -------- */

/* out[i] = Philox4x32-10 word (j0+i) % 4 of the block with counter
 * ((j0+i)>>2 low, (j0+i)>>34, t, k) and key (seed low, seed high), for
 * i < count.  out is device uint32_t[count]. */
int opt_debug_philox(uint64_t seed, int64_t t, int32_t k, int64_t j0, int64_t count,
                     uint32_t *out, void *stream);

/* out[i] = BF16 word of x[i]: round to nearest even if r is NULL, else
 * stochastic rounding with the 16-bit integer r[i] & 0xFFFF.  Device arrays. */
int opt_debug_round_bf16(const float *x, const uint32_t *r, uint16_t *out, int64_t n,
                         void *stream);

/* The step's two directions for n elements with inputs g, m, v (and m2 for
 * AdEMAMix; NULL for AdamW), the moments formed from them with hp's betas,
 * alpha, eps and bias-correction step (no gradient scale): out[i] = the
 * direction with the hardware reciprocal and square root, out[n+i] = its
 * error bound against the exact recipe (infinite where the step would take
 * the exact recipe for that element anyway), out[2n+i] = the exact recipe's
 * direction (correctly rounded division and square root).  Device arrays;
 * out is float[3n].  OPT_EINVAL for another optimizer, NULL arrays, betas
 * outside [0, 1) or step < 1. */
int opt_debug_direction(int32_t optimizer, const opt_hparams *hp, const float *g, const float *m,
                        const float *v, const float *m2, float *out, int64_t n, void *stream);

/* out[i] = code of x[i] against the host codebook qmap (256 floats, as
 * qmap_signed; pass is_signed = 0 for a table of non-negative entries, which
 * must hold 0 <= x <= 1), using the lookup tables the 8-bit step builds.
 * x and out are device arrays of n entries. */
int opt_debug_quantize(const float *qmap, int32_t is_signed, const float *x, uint8_t *out,
                       int64_t n, void *stream);

/* Host only, no device work: the number of chunks the planner gives each
 * tensor of `numels` (n entries) at the library's chunk size, written to
 * chunks_out[n]; returns the chunk size in elements, or a negative status. */
int64_t opt_debug_plan(const int64_t *numels, int64_t n, int64_t *chunks_out);

/* Host only: the lookup of opt_debug_quantize run on the CPU over host arrays
 * (the same table builder and lookup source).  x[i] must be NaN or in [-1, 1]
 * (OPT_EINVAL otherwise). */
int opt_debug_quantize_host(const float *qmap, int32_t is_signed, const float *x, uint8_t *out,
                            int64_t n);

/* Host only: out[i] = a[i] / b[i] by the kernels' division with a reused
 * reciprocal (two residual corrections of a[i] * RN(1/b[i])), on the CPU.
 * Each b[i] must have 2^-124 <= |b[i]| <= 2^26, the range in which the
 * kernels take this division (OPT_EINVAL otherwise); the quotient is the
 * correctly rounded one when |a[i]| <= |b[i]| and a[i] is 0 or at least
 * 2^-100 in magnitude. */
int opt_debug_div_by(const float *a, const float *b, float *out, int64_t n);

/* Calibration: dst[j][i] = sum_k src[k][i] for i < n over fp32 device arrays
 * (0..6 sources, 1..6 destinations, 16-byte aligned, n a multiple of 4), a
 * plain streaming kernel with the step's access pattern and no arithmetic,
 * used to read the achievable bandwidth and to scale HBM byte counters. */
int opt_debug_stream(const float *const *src, int32_t nsrc, float *const *dst, int32_t ndst, int64_t n,
                     void *stream);

/* Launch geometry for all later calls in this process: elements per chunk of
 * the host's chunk table (a power of two in [1024, 2^24]; default 32768) and
 * workgroups per compute unit: 0 (the default) launches one workgroup per
 * tile (of each kernel's size, at most one chunk), 1..64 a persistent grid of that
 * many per compute unit walking the same tiles with a grid stride.  Results
 * do not depend on either.  OPT_EINVAL for other values. */
int opt_debug_set_launch(int64_t chunk, int32_t wgs_per_cu);

/* The per-call scalars the host forms for a step with hyper-parameters hp
 * (host array out[10]): 1-beta1, 1-beta2, 1-beta3, c1 = 1-beta1^t',
 * c2 = 1-beta2^t' (binary64, rounded once; t' counts from the last state
 * reset), RN(1/c1), RN(1/c2), 1-lr*wd, lr, and the gradient scale 1 (the
 * kernels read a given scale from device memory). */
int opt_debug_scalars(const opt_hparams *hp, float *out);

/* Cap on the workgroups each compute unit holds at once for the element-wise
 * and one-state step kernels, for all later calls in this process: -1 (the
 * default) lets each kernel configuration take its own measured choice, 0
 * sets no cap, 2..32 caps at that many (a launch-time LDS reservation that
 * the kernels do not use).  Results do not depend on it.  OPT_EINVAL for
 * other values. */
int opt_debug_set_wg_cap(int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* OPT_STEP_H */

// opt_api.cpp -- the C ABI declared in include/opt_step.h: argument checks,
// dtype bucketing, the host-built chunk table, the per-device workspace, and
// the 8-bit codebook lookup tables.  Device work is in opt_kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "opt_device.h"
#include "opt_step.h"

namespace optstep {

hipError_t launch_step(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds,
                       hipStream_t st);
hipError_t launch_unorm(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, size_t lds, int ntens,
                        double *out, hipStream_t st);
hipError_t launch_gnorm(int gd, const StepArgs &a, const LaunchGeom &lg, int ntens, double *out, hipStream_t st);
hipError_t launch_step_1state(int opt, int gd, int fmt, const StepArgs &a, const LaunchGeom &lg, hipStream_t st);
hipError_t launch_gnorm_total(int64_t n, double *out, float max_norm, int norm_type, float *coef, hipStream_t st);
hipError_t launch_debug_philox(uint64_t seed, int64_t t, int32_t k, int64_t j0, int64_t n, uint32_t *out,
                               hipStream_t st);
hipError_t launch_debug_round(const float *x, const uint32_t *r, uint16_t *out, int64_t n, hipStream_t st);
hipError_t launch_debug_direction(int opt, const StepArgs &a, const float *g, const float *m, const float *v,
                                  const float *m2, float *out, int64_t n, hipStream_t st);
hipError_t launch_debug_quantize(const QTabs &q, int is_signed, const float *x, uint8_t *out, int64_t n,
                                 hipStream_t st);
hipError_t launch_debug_mini(int elem, float A, const float *x, const uint32_t *r, uint8_t *codes, float *decoded,
                             int64_t n, hipStream_t st);
hipError_t launch_debug_mini_pack(int elem, float A, const float *x, const uint32_t *r, uint8_t *codes, int64_t n,
                                  hipStream_t st);
hipError_t launch_round_cast(const float *x, uint16_t *out, int64_t n, int bf16, int sr, uint64_t seed,
                             uint64_t offset, const LaunchGeom &lg, hipStream_t st);
hipError_t launch_debug_stream(const float *const *src, int nsrc, float *const *dst, int ndst, int64_t n,
                               const LaunchGeom &lg, hipStream_t st);

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(OPT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// launch configuration

int64_t g_chunk = 32768;      // elements per chunk; a power of two >= 1024
int g_wgs_per_cu = 0;         // workgroups per compute unit (0: one per tile, or occupancy)
int g_wg_cap = -1;            // resident workgroups per compute unit (-1: per kernel, 0: no cap)

constexpr int kMaxDevices = 64;
constexpr int kSlots = 16;
constexpr int kPlans = 8;                  // planned calls remembered per device
constexpr int64_t kPlanMaxTensors = 1 << 16;
// Size limits, far beyond any device's memory, that keep the host's chunk
// arithmetic and the element indices of the random streams in range.
constexpr int64_t kMaxNumel = (int64_t)1 << 46;
constexpr int64_t kMaxIndex = (int64_t)1 << 60;
constexpr uint32_t kMaxSearchWords = 15000;   // LDS budget of the search tables

// ---------------------------------------------------------------------------
// 8-bit codebook lookup tables

struct BuiltTable {
    std::vector<uint32_t> entries;
    QTabParams P{};
};

static uint32_t fb(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bf(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

// The code of x is the number of midpoints t_i = (T_i + T_{i+1})/2 (formed in
// binary64) that x lies strictly above, i.e. the count of tau_i <= x with
// tau_i the smallest float above t_i: the nearest entry, ties to the lower
// index.  The table splits [lo, 1] into buckets of 2^shift ulps (one sign at
// a time) holding at most one tau each, so one add finishes the code.
// The comparison is folded into the entry (opt_plan.h): with base taus at or
// below the bucket and the bucket's tau at in-bucket key K, x > 0 takes
// E = ((base + 1) << 24) - K, so E + k carries into the top byte iff k >= K;
// x = -m (m's key k) takes E = ((base + 1) << 24) + K', K' the key of -tau,
// so E + ~k = E - k - 1 keeps base + 1 iff k <= K' - 1.  A bucket with no tau
// uses K = 2^shift and K' = 0 (never and always past).  Sums stay within 2^24
// of the top byte's boundary because k and K are below 2^18, and arithmetic
// is modulo 2^32, which is what the device does.
int build_search(const float *T, bool is_signed, BuiltTable &out)
{
    for (int i = 0; i < 256; ++i) {
        if (!std::isfinite(T[i]) || T[i] < -1.0f || T[i] > 1.0f)
            return fail(OPT_EINVAL, "codebook entry %d (%g) is not a finite value in [-1, 1]", i, T[i]);
        if (i > 0 && !(T[i] > T[i - 1]))
            return fail(OPT_EINVAL, "codebook is not strictly increasing at entry %d", i);
    }
    if (!is_signed && T[0] < 0.0f) return fail(OPT_EINVAL, "unsigned codebook has a negative entry");
    float tau[255];
    float minmag = INFINITY;
    for (int i = 0; i < 255; ++i) {
        double t = ((double)T[i] + (double)T[i + 1]) / 2.0;
        float f = (float)t;
        if ((double)f <= t) f = nextafterf(f, INFINITY);
        tau[i] = f;
        // a midpoint of exactly 0 gives tau = the smallest positive float; the
        // lookup sends +0 to the x < 0 half, so only the others bound lo
        if (t != 0.0) minmag = std::min(minmag, std::fabs(f));
    }
    if (!(minmag > 0x1p-100f)) return fail(OPT_EUNSUPPORTED, "codebook midpoints too close to zero");
    // lo: the largest power of two strictly below every |tau|.
    uint32_t lo = fb(minmag) & 0x7F800000u;
    if (lo == fb(minmag)) lo -= 0x00800000u;
    const uint32_t one = 0x3F800000u;
    for (uint32_t shift = 17; shift >= 10; --shift) {
        const uint32_t nb = ((one - lo) >> shift) + 1;
        const uint32_t sides = is_signed ? 2 : 1;
        if (nb * sides > kMaxSearchWords) break;
        std::vector<uint32_t> ent(nb * sides);
        bool ok = true;
        for (uint32_t b = 0; b < nb && ok; ++b) {
            const uint32_t L = lo + (b << shift), H = L + (1u << shift) - 1u;
            const float xl = bf(L), xh = bf(H);
            // x > 0 with magnitude bits in [L, H]: past the tau at key K
            uint32_t base = 0, nin = 0, K = 1u << shift;
            for (int i = 0; i < 255; ++i) {
                if (tau[i] <= xl) ++base;
                else if (tau[i] <= xh) { ++nin; K = fb(tau[i]) - L; }
            }
            ent[sides * b] = ((base + 1u) << 24) - K;
            ok = nin <= 1;
            if (is_signed && ok) {
                // x = -m, m in [xl, xh]: one more code while m's key <= key(-tau)
                base = 0; nin = 0; K = 0;
                for (int i = 0; i < 255; ++i) {
                    if (tau[i] <= -xh) ++base;
                    else if (tau[i] <= -xl) { ++nin; K = fb(-tau[i]) - L + 1u; }
                }
                ent[2 * b + 1] = ((base + 1u) << 24) + K;
                ok = nin <= 1;
            }
        }
        if (ok) {
            out.entries.swap(ent);
            out.P.lo = lo;
            out.P.shift = shift;
            out.P.nb = nb;
            return OPT_OK;
        }
    }
    return fail(OPT_EUNSUPPORTED, "codebook too dense for the lookup table");
}

// Packs [signed values | unsigned values | signed search | unsigned search].
int build_qwords(const float *qs, const float *qu, std::vector<uint32_t> &words, QTabParams &ps,
                 QTabParams &pu)
{
    BuiltTable S, U;
    int rc;
    if ((rc = build_search(qs, true, S)) != OPT_OK) return rc;
    if ((rc = build_search(qu, false, U)) != OPT_OK) return rc;
    if (S.entries.size() + U.entries.size() > kMaxSearchWords)
        return fail(OPT_EUNSUPPORTED, "codebook lookup tables exceed the LDS budget");
    words.resize(512 + S.entries.size() + U.entries.size());
    memcpy(words.data(), qs, 1024);
    memcpy(words.data() + 256, qu, 1024);
    // The unsigned table's values read back as v, which the kernels keep at
    // +0 or above (its code lookup and block absmax take the bit pattern with
    // no sign mask).  A -0 first entry reads back as +0, which codes, scales
    // and steps exactly as -0 does.
    if (words[256] == 0x80000000u) words[256] = 0u;
    std::copy(S.entries.begin(), S.entries.end(), words.begin() + 512);
    std::copy(U.entries.begin(), U.entries.end(), words.begin() + 512 + S.entries.size());
    ps = S.P;
    ps.offset = 512;
    pu = U.P;
    pu.offset = 512 + (uint32_t)S.entries.size();
    return OPT_OK;
}

struct QCache {
    float qs[256], qu[256];
    std::vector<uint32_t> words;
    QTabParams ps, pu;
    bool valid = false;
    uint64_t gen = 0;               // bumped whenever the tables change
};

// ---------------------------------------------------------------------------
// per-device workspace

struct Slot {
    void *dev = nullptr;
    void *host = nullptr;           // pinned staging copy
    size_t cap = 0;
    std::vector<unsigned char> content;
    hipEvent_t ev = nullptr;        // after the last kernel that read the slot
    hipEvent_t ready = nullptr;     // after the copy that filled it
    hipStream_t upload_stream = nullptr;
    hipStream_t last_stream = nullptr;
    bool multi_stream = false;
    bool used = false;
    uint64_t tick = 0;
    uint64_t gen = 0;               // bumped whenever the contents are replaced
};

// One bucket's launch in a planned call: its tables' slot and offsets.
struct PlanItem {
    int bi = 0;                     // bucket: (gradient dtype, parameter dtype) index
    Slot *slot = nullptr;
    uint64_t gen = 0;               // the slot's generation when the tables went in
    size_t off_ct = 0, off_q = 0;
    int64_t nchunks = 0;
    int ntens = 0;
    size_t partial_doubles = 0;
    int64_t ngroups = 0;
};

// A planned call, keyed by the raw tensor records and everything else the
// tables depend on (kind of call, optimizer, format, chunk size, codebook
// tables); valid while every slot it names still holds its tables.
struct PlanEntry {
    std::vector<unsigned char> key;
    std::vector<PlanItem> items;
    size_t need = 0;                // doubles of norm workspace
    uint64_t tick = 0;
};

struct Workspace {
    bool init = false;
    int ncu = 0;
    Slot slots[kSlots];
    uint64_t tick = 0;
    double *partials = nullptr;
    size_t partials_cap = 0;          // doubles
    hipEvent_t partials_ev = nullptr;
    hipStream_t partials_stream = nullptr;
    bool partials_used = false;
    QCache q;
    PlanEntry plans[kPlans];
};

std::mutex g_mu;
Workspace g_ws[kMaxDevices];

int workspace(Workspace *&out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(OPT_EUNSUPPORTED, "device %d out of range", dev);
    Workspace &w = g_ws[dev];
    if (!w.init) {
        e = hipDeviceGetAttribute(&w.ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        for (Slot &s : w.slots) {
            e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
            if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
            e = hipEventCreateWithFlags(&s.ready, hipEventDisableTiming);
            if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        }
        e = hipEventCreateWithFlags(&w.partials_ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        w.init = true;
    }
    out = &w;
    return OPT_OK;
}

// Wait until neither the copy that filled the slot (which reads its pinned
// staging buffer) nor a queued kernel that reads the slot is pending.
int slot_quiesce(Slot &s)
{
    if (s.upload_stream || !s.content.empty()) {
        hipError_t e = hipEventSynchronize(s.ready);
        if (e != hipSuccess) return hip_fail(e, "waiting for a workspace copy");
    }
    if (!s.used) return OPT_OK;
    hipError_t e = s.multi_stream ? hipDeviceSynchronize() : hipEventSynchronize(s.ev);
    if (e != hipSuccess) return hip_fail(e, "waiting for a workspace slot");
    s.used = false;
    s.multi_stream = false;
    return OPT_OK;
}

// Device copy of `blob`, reusing a slot that already holds the same bytes.
// A slot filled on another stream is reused after that stream's copy: the
// caller's stream waits on the copy's event (no wait on the filling stream).
int upload(Workspace &w, const std::vector<unsigned char> &blob, hipStream_t st, Slot *&out)
{
    ++w.tick;
    for (Slot &s : w.slots) {
        if (s.dev && s.content.size() == blob.size() && memcmp(s.content.data(), blob.data(), blob.size()) == 0) {
            if (s.upload_stream != st) {
                hipError_t e = hipStreamWaitEvent(st, s.ready, 0);
                if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (tables)");
            }
            s.tick = w.tick;
            out = &s;
            return OPT_OK;
        }
    }
    Slot *v = &w.slots[0];
    for (Slot &s : w.slots) if (s.tick < v->tick) v = &s;
    int rc = slot_quiesce(*v);
    if (rc != OPT_OK) return rc;
    hipError_t e;
    // The slot holds nothing valid until the copy below is queued, so a
    // failure from here on can never let a later call reuse it.
    v->content.clear();
    v->upload_stream = nullptr;
    ++v->gen;
    if (v->cap < blob.size()) {
        if (v->dev) { (void)hipFree(v->dev); v->dev = nullptr; }
        if (v->host) { (void)hipHostFree(v->host); v->host = nullptr; }
        v->cap = 0;
        size_t cap = std::max<size_t>(blob.size(), 64 * 1024);
        if ((e = hipMalloc(&v->dev, cap)) != hipSuccess) return hip_fail(e, "hipMalloc (workspace)");
        if ((e = hipHostMalloc(&v->host, cap, hipHostMallocDefault)) != hipSuccess)
            return hip_fail(e, "hipHostMalloc (workspace)");
        v->cap = cap;
    }
    memcpy(v->host, blob.data(), blob.size());
    v->content = blob;
    if ((e = hipMemcpyAsync(v->dev, v->host, blob.size(), hipMemcpyHostToDevice, st)) != hipSuccess) {
        v->content.clear();
        return hip_fail(e, "hipMemcpyAsync (tables)");
    }
    if ((e = hipEventRecord(v->ready, st)) != hipSuccess) {
        // with no event to wait on later, let the queued copy finish reading
        // the staging buffer before a later fill may overwrite it
        v->content.clear();
        (void)hipStreamSynchronize(st);
        return hip_fail(e, "hipEventRecord (tables)");
    }
    v->upload_stream = st;
    v->tick = w.tick;
    out = v;
    return OPT_OK;
}

int slot_mark_used(Slot &s, hipStream_t st)
{
    if (s.used && s.last_stream != st) s.multi_stream = true;
    s.used = true;
    s.last_stream = st;
    hipError_t e = hipEventRecord(s.ev, st);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    return OPT_OK;
}

int partials_reserve(Workspace &w, size_t ndoubles, hipStream_t st)
{
    hipError_t e;
    if (w.partials_cap < ndoubles) {
        if (w.partials_used) {
            if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
            w.partials_used = false;
        }
        if (w.partials) (void)hipFree(w.partials);
        w.partials = nullptr;
        w.partials_cap = 0;
        size_t cap = std::max<size_t>(ndoubles, 1 << 16);
        if ((e = hipMalloc((void **)&w.partials, cap * sizeof(double))) != hipSuccess)
            return hip_fail(e, "hipMalloc (norm partials)");
        w.partials_cap = cap;
    } else if (w.partials_used && w.partials_stream != st) {
        // the previous pre-pass ran on another stream: order after it
        if ((e = hipStreamWaitEvent(st, w.partials_ev, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }
    return OPT_OK;
}

// ---------------------------------------------------------------------------
// argument checks and planning

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_hparams(const opt_hparams *hp, int fmt)
{
    if (!hp) return fail(OPT_EINVAL, "hp is NULL");
    if (hp->step < 1) return fail(OPT_EINVAL, "step must be >= 1 (got %lld)", (long long)hp->step);
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(OPT_EINVAL, "beta1 and beta2 must lie in [0, 1)");
    if (!(hp->beta3 >= 0.0f && hp->beta3 <= 1.0f)) return fail(OPT_EINVAL, "beta3 must lie in [0, 1]");
    if (fmt == kQ8 && (!hp->qmap_signed || !hp->qmap_unsigned))
        return fail(OPT_EINVAL, "8-bit states need qmap_signed and qmap_unsigned");
    if (hp->grad_scale && !aligned(hp->grad_scale, 4)) return fail(OPT_EALIGN, "grad_scale must be 4-byte aligned");
    if (hp->reset_interval < 0) return fail(OPT_EINVAL, "reset_interval must be >= 0");
    if (hp->p_rounding != 0 && hp->p_rounding != 1) return fail(OPT_EINVAL, "p_rounding must be 0 or 1");
    if (hp->skip_zeros != 0 && hp->skip_zeros != 1) return fail(OPT_EINVAL, "skip_zeros must be 0 or 1");
    return OPT_OK;
}

// index_base and the stochastic-rounding tensor number of one record.
int check_slice(const opt_tensor &x, int64_t k, int64_t align)
{
    if (x.numel > kMaxNumel) return fail(OPT_EINVAL, "tensor %lld: numel above 2^46", (long long)k);
    if (x.index_base > kMaxIndex - x.numel)
        return fail(OPT_EINVAL, "tensor %lld: index_base + numel above 2^60", (long long)k);
    if (x.index_base < 0 || x.index_base % align != 0)
        return fail(OPT_EINVAL, "tensor %lld: index_base must be >= 0 and a multiple of %lld", (long long)k,
                    (long long)align);
    if (x.sr_tensor_set != 0 && x.sr_tensor_set != 1) return fail(OPT_EINVAL, "tensor %lld: sr_tensor_set must be 0 or 1", (long long)k);
    if (x.sr_tensor_set && x.sr_tensor < 0) return fail(OPT_EINVAL, "tensor %lld: sr_tensor must be >= 0", (long long)k);
    return OPT_OK;
}

int check_tensors(const opt_tensor *t, int64_t n, int opt, int fmt)
{
    int rc;
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (n > 0 && !t) return fail(OPT_EINVAL, "tensors is NULL");
    if (n > INT32_MAX) return fail(OPT_EINVAL, "too many tensors");
    if (fmt < kF32 || fmt > kFP4SR) return fail(OPT_EINVAL, "unknown state format %d", fmt);
    for (int64_t k = 0; k < n; ++k) {
        const opt_tensor &x = t[k];
        if (x.numel < 0) return fail(OPT_EINVAL, "tensor %lld: numel < 0", (long long)k);
        if (x.p_dtype != OPT_F32 && x.p_dtype != OPT_BF16 && x.p_dtype != OPT_F16)
            return fail(OPT_EINVAL, "tensor %lld: unknown p_dtype %d", (long long)k, x.p_dtype);
        if (x.g_dtype != OPT_F32 && x.g_dtype != OPT_BF16 && x.g_dtype != OPT_F16)
            return fail(OPT_EINVAL, "tensor %lld: unknown g_dtype %d", (long long)k, x.g_dtype);
        if ((rc = check_slice(x, k, blocked(fmt) ? kQBlock : 4)) != OPT_OK) return rc;
        if (x.numel == 0) continue;
        const bool q8 = blocked(fmt), m2 = opt == kAdEMAMix;
        if (!x.p || !x.g || !x.s1 || !x.s2 || (m2 && !x.s3))
            return fail(OPT_EINVAL, "tensor %lld: missing p, g or a state", (long long)k);
        if (q8 && (!x.absmax1 || !x.absmax2 || (m2 && !x.absmax3)))
            return fail(OPT_EINVAL, "tensor %lld: missing an absmax array", (long long)k);
        if (!aligned(x.p, 16) || !aligned(x.g, 16) || !aligned(x.s1, 16) || !aligned(x.s2, 16) ||
            (m2 && !aligned(x.s3, 16)))
            return fail(OPT_EALIGN, "tensor %lld: p, g and states must be 16-byte aligned", (long long)k);
        if (q8 && (!aligned(x.absmax1, 4) || !aligned(x.absmax2, 4) || (m2 && !aligned(x.absmax3, 4))))
            return fail(OPT_EALIGN, "tensor %lld: absmax arrays must be 4-byte aligned", (long long)k);
    }
    return OPT_OK;
}

struct Bucket {
    std::vector<DevTensor> tens;
    std::vector<int32_t> chunk_tensor;
    int64_t ngroups = 0;   // norm-sum groups of kRGroup partials, over the bucket's tensors

    // doubles of workspace the norm passes use: a pair per partial, then a pair per group
    size_t partial_doubles(int64_t chunk) const { return chunk_tensor.size() * (size_t)(chunk / kUTile) * 2; }
    size_t norm_doubles(int64_t chunk) const { return partial_doubles(chunk) + 2 * (size_t)ngroups; }
};

// The tensors whose (gradient, parameter) storage is (gd, pd); opt_dtype,
// GradT and ParamT share their numbering.
void plan_bucket(const opt_tensor *t, int64_t n, int gd, int pd, int64_t chunk, Bucket &b)
{
    int64_t next = 0;
    for (int64_t k = 0; k < n; ++k) {
        const opt_tensor &x = t[k];
        // empty tensors ride in the first bucket with no chunks, so the norm
        // pre-passes still write zeros for them
        const bool mine = x.numel == 0 ? (gd == kGradF32 && pd == kP32) : (x.g_dtype == gd && x.p_dtype == pd);
        if (!mine) continue;
        DevTensor d{};
        d.p = (float *)x.p;
        d.g = x.g;
        d.s1 = x.s1; d.s2 = x.s2; d.s3 = x.s3;
        d.a1 = x.absmax1; d.a2 = x.absmax2; d.a3 = x.absmax3;
        d.numel = x.numel;
        d.chunk_begin = next;
        d.k = (int32_t)k;
        d.rk = x.sr_tensor_set ? (uint32_t)x.sr_tensor : (uint32_t)k;
        d.jbase = x.index_base;
        d.rg_begin = b.ngroups;
        b.ngroups += norm_groups(x.numel);
        const int64_t nc = (x.numel + chunk - 1) / chunk;
        const int32_t idx = (int32_t)b.tens.size();
        b.tens.push_back(d);
        b.chunk_tensor.insert(b.chunk_tensor.end(), (size_t)nc, idx);
        next += nc;
    }
}

size_t round16(size_t x) { return (x + 15) & ~(size_t)15; }

// Blob = DevTensor[] | int32 chunk_tensor[] | uint32 q-words[]; returns the
// byte offsets of the second and third parts.
void make_blob(const Bucket &b, const std::vector<uint32_t> *qw, std::vector<unsigned char> &blob,
               size_t &off_ct, size_t &off_q)
{
    const size_t n0 = b.tens.size() * sizeof(DevTensor);
    off_ct = round16(n0);
    off_q = round16(off_ct + b.chunk_tensor.size() * 4);
    const size_t total = off_q + (qw ? qw->size() * 4 : 0);
    blob.assign(total, 0);
    memcpy(blob.data(), b.tens.data(), n0);
    memcpy(blob.data() + off_ct, b.chunk_tensor.data(), b.chunk_tensor.size() * 4);
    if (qw) memcpy(blob.data() + off_q, qw->data(), qw->size() * 4);
}

int qtables(Workspace &w, const opt_hparams *hp)
{
    QCache &q = w.q;
    if (q.valid && !memcmp(q.qs, hp->qmap_signed, 1024) && !memcmp(q.qu, hp->qmap_unsigned, 1024))
        return OPT_OK;
    q.valid = false;
    int rc = build_qwords(hp->qmap_signed, hp->qmap_unsigned, q.words, q.ps, q.pu);
    if (rc != OPT_OK) return rc;
    memcpy(q.qs, hp->qmap_signed, 1024);
    memcpy(q.qu, hp->qmap_unsigned, 1024);
    q.valid = true;
    ++q.gen;
    return OPT_OK;
}

StepArgs base_args(const opt_hparams *hp, int64_t chunk)
{
    StepArgs a{};
    a.chunk = chunk;
    a.lr = hp->lr; a.beta1 = hp->beta1; a.beta2 = hp->beta2; a.beta3 = hp->beta3;
    a.alpha = hp->alpha; a.eps = hp->eps; a.wd = hp->weight_decay; a.max_unorm = hp->max_unorm;
    a.step = hp->step;
    // a reset every R steps restarts the moments at steps 1, R+1, 2R+1, ...
    const int64_t R = hp->reset_interval;
    a.bc_step = R > 0 ? (hp->step - 1) % R + 1 : hp->step;
    a.fresh = R > 0 && a.bc_step == 1;
    a.seed = hp->seed;
    a.grad_scale = hp->grad_scale;
    a.p_sr = hp->p_rounding;
    a.skip_zeros = hp->skip_zeros;
    a.sc = make_scalars(a);
    return a;
}

LaunchGeom geom(const Workspace &w) { return LaunchGeom{w.ncu, g_wgs_per_cu, g_wg_cap}; }

// The device tables of a call's buckets (bucket bi = 3 * gradient dtype +
// parameter dtype).  A call whose tensor records, kind, optimizer, format,
// chunk size and codebook tables equal those of a remembered call, and whose
// tables are all still in their slots, reuses that plan; otherwise the
// buckets are planned and their tables uploaded (or found) now.  Buckets
// whose tensors are all empty are kept only if keep_chunkless (the norm
// passes write zeros for them).
int plan_call(Workspace &w, int kind, int opt, int fmt, bool keep_chunkless, const opt_tensor *t, int64_t n,
              const std::vector<uint32_t> *qw, hipStream_t st, std::vector<PlanItem> &items, size_t &need)
{
    const int64_t chunk = g_chunk;
    const bool cache = n <= kPlanMaxTensors;
    std::vector<unsigned char> key;
    if (cache) {
        const int64_t head[6] = {kind, opt, fmt, keep_chunkless ? 1 : 0, chunk, qw ? (int64_t)w.q.gen : -1};
        key.resize(sizeof head + (size_t)n * sizeof(opt_tensor));
        memcpy(key.data(), head, sizeof head);
        if (n) memcpy(key.data() + sizeof head, t, (size_t)n * sizeof(opt_tensor));
        for (PlanEntry &e : w.plans) {
            if (e.key.size() != key.size() || memcmp(e.key.data(), key.data(), key.size()) != 0) continue;
            bool live = true;
            for (const PlanItem &it : e.items) live = live && it.slot->gen == it.gen;
            if (!live) {            // a table was evicted since: plan afresh
                e = PlanEntry();
                break;
            }
            for (const PlanItem &it : e.items) {
                Slot &s = *it.slot;
                if (s.upload_stream != st) {    // as in upload(): order after the copy
                    hipError_t er = hipStreamWaitEvent(st, s.ready, 0);
                    if (er != hipSuccess) return hip_fail(er, "hipStreamWaitEvent (tables)");
                }
                s.tick = ++w.tick;
            }
            e.tick = ++w.tick;
            items = e.items;
            need = e.need;
            return OPT_OK;
        }
    }
    items.clear();
    need = 0;
    for (int bi = 0; bi < 9; ++bi) {
        Bucket bk;
        plan_bucket(t, n, bi / 3, bi % 3, chunk, bk);
        if (bk.tens.empty() || (!keep_chunkless && bk.chunk_tensor.empty())) continue;
        std::vector<unsigned char> blob;
        PlanItem it;
        it.bi = bi;
        make_blob(bk, qw, blob, it.off_ct, it.off_q);
        Slot *s;
        int rc = upload(w, blob, st, s);
        if (rc != OPT_OK) return rc;
        it.slot = s;
        it.gen = s->gen;
        it.nchunks = (int64_t)bk.chunk_tensor.size();
        it.ntens = (int)bk.tens.size();
        it.partial_doubles = bk.partial_doubles(chunk);
        it.ngroups = bk.ngroups;
        need = std::max(need, bk.norm_doubles(chunk));
        items.push_back(it);
    }
    if (cache) {
        PlanEntry *v = &w.plans[0];
        for (PlanEntry &e : w.plans) if (e.tick < v->tick) v = &e;
        v->key = std::move(key);
        v->items = items;
        v->need = need;
        v->tick = ++w.tick;
    }
    return OPT_OK;
}

// The shared body of the step and the pre-pass.
int run(int opt, const opt_tensor *t, int64_t n, int fmt, const opt_hparams *hp, const double *unorm,
        double *unorm_out, void *stream)
{
    int rc;
    if ((rc = check_hparams(hp, fmt)) != OPT_OK) return rc;
    if ((rc = check_tensors(t, n, opt, fmt)) != OPT_OK) return rc;
    const bool pre = unorm_out != nullptr;
    if (!pre && hp->max_unorm > 0.0f && !unorm)
        return fail(OPT_EINVAL, "max_unorm > 0 needs the norms from opt_precondition_unorm");
    if (pre && !aligned(unorm_out, 8)) return fail(OPT_EALIGN, "unorm_out must be 8-byte aligned");
    if (n == 0) return OPT_OK;

    std::lock_guard<std::mutex> lock(g_mu);
    Workspace *w;
    if ((rc = workspace(w)) != OPT_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const bool q8 = fmt == kQ8;
    if (q8 && (rc = qtables(*w, hp)) != OPT_OK) return rc;
    const int64_t chunk = g_chunk;

    std::vector<PlanItem> items;
    size_t need = 0;
    if ((rc = plan_call(*w, 0, opt, fmt, pre, t, n, q8 ? &w->q.words : nullptr, st, items, need)) != OPT_OK)
        return rc;
    if (pre && (rc = partials_reserve(*w, need, st)) != OPT_OK) return rc;

    for (const PlanItem &it : items) {
        const int gd = it.bi / 3;
        Slot *s = it.slot;
        StepArgs a = base_args(hp, chunk);
        a.p_dtype = it.bi % 3;
        a.tens = (const DevTensor *)s->dev;
        a.chunk_tensor = (const int32_t *)((unsigned char *)s->dev + it.off_ct);
        a.nchunks = it.nchunks;
        a.unorm = (!pre && hp->max_unorm > 0.0f) ? unorm : nullptr;
        size_t lds = 0;
        if (q8) {
            a.q.words = (const uint32_t *)((unsigned char *)s->dev + it.off_q);
            a.q.nwords = (uint32_t)w->q.words.size();
            a.q.s = w->q.ps;
            a.q.u = w->q.pu;
            lds = (size_t)a.q.nwords * 4;
        }
        hipError_t e;
        if (pre) {
            a.partials = w->partials;
            a.groups = w->partials + it.partial_doubles;
            a.ngroups = it.ngroups;
            e = launch_unorm(opt, gd, fmt, a, geom(*w), q8 ? 2048 : 0, it.ntens, unorm_out, st);
            if (e == hipSuccess) {
                w->partials_used = true;
                w->partials_stream = st;
                e = hipEventRecord(w->partials_ev, st);
            }
        } else {
            e = launch_step(opt, gd, fmt, a, geom(*w), lds, st);
        }
        if (e != hipSuccess) return hip_fail(e, pre ? "norm pre-pass launch" : "step launch");
        if ((rc = slot_mark_used(*s, st)) != OPT_OK) return rc;
    }
    return OPT_OK;
}

// ---------------------------------------------------------------------------
// The allocation-free AdamW step.  Its tables (DevTensor records, chunk
// table, 8-bit lookup tables) go into a fixed device array instead of the
// grown workspace: one copy per device of kScratchBytes, which the device
// holds until the process ends.  On the host only its address, taken once per
// device with hipGetSymbolAddress, is ever used (the array's own name in host
// code is not a device address).

constexpr size_t kScratchBytes = (size_t)2 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchDev {
    bool init = false;
    unsigned char *ptr = nullptr;   // device address of `scratch` on this device
    int ncu = 0;
    hipEvent_t copied = nullptr;    // after the last call's table copy
    bool pending = false;
    std::vector<unsigned char> host;   // host image of the tables (pageable)
};
ScratchDev g_scratch[kMaxDevices];

// The current device's scratch record, set up on its first use (with g_mu held).
int scratch_dev(ScratchDev *&out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(OPT_EUNSUPPORTED, "device %d out of range", dev);
    ScratchDev &d = g_scratch[dev];
    if (!d.init) {
        if ((e = hipGetSymbolAddress((void **)&d.ptr, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress (scratch)");
        if ((e = hipDeviceGetAttribute(&d.ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return hip_fail(e, "hipDeviceGetAttribute");
        if ((e = hipEventCreateWithFlags(&d.copied, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e, "hipEventCreate");
        d.init = true;
    }
    out = &d;
    return OPT_OK;
}

int run_noalloc(int opt, const opt_tensor *t, int64_t n, int fmt, const opt_hparams *hp, const double *unorm,
                void *stream)
{
    int rc;
    if ((rc = check_hparams(hp, fmt)) != OPT_OK) return rc;
    if ((rc = check_tensors(t, n, opt, fmt)) != OPT_OK) return rc;
    if (hp->max_unorm > 0.0f && !unorm)
        return fail(OPT_EINVAL, "max_unorm > 0 needs the norms from opt_precondition_unorm");
    if (n == 0) return OPT_OK;
    std::lock_guard<std::mutex> lock(g_mu);
    const bool q8 = fmt == kQ8;
    std::vector<uint32_t> qw;
    QTabParams ps{}, pu{};
    if (q8 && (rc = build_qwords(hp->qmap_signed, hp->qmap_unsigned, qw, ps, pu)) != OPT_OK) return rc;
    const int64_t chunk = g_chunk;
    // every bucket's tables, one after another, each on a 256-byte boundary
    struct Item { int bi; size_t off, off_ct, off_q; int64_t nchunks; };
    std::vector<Item> items;
    std::vector<unsigned char> image;
    for (int bi = 0; bi < 9; ++bi) {
        Bucket bk;
        plan_bucket(t, n, bi / 3, bi % 3, chunk, bk);
        if (bk.chunk_tensor.empty()) continue;
        std::vector<unsigned char> blob;
        Item it{bi, (image.size() + 255) & ~(size_t)255, 0, 0, (int64_t)bk.chunk_tensor.size()};
        make_blob(bk, q8 ? &qw : nullptr, blob, it.off_ct, it.off_q);
        if (it.off + blob.size() > kScratchBytes)
            return fail(OPT_EUNSUPPORTED, "the tensor list needs more than the %zu bytes of tables the "
                        "allocation-free step holds (%zu tensors, %lld chunks so far)", kScratchBytes,
                        (size_t)n, (long long)it.nchunks);
        image.resize(it.off + blob.size(), 0);
        memcpy(image.data() + it.off, blob.data(), blob.size());
        items.push_back(it);
    }
    if (items.empty()) return OPT_OK;

    ScratchDev *d;
    if ((rc = scratch_dev(d)) != OPT_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    // the host image of the previous call must have been read before it is
    // overwritten (a pageable source is staged when the copy is queued; the
    // wait covers the case where it is read later)
    if (d->pending && (e = hipEventSynchronize(d->copied)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    d->pending = false;
    d->host.swap(image);
    if ((e = hipMemcpyAsync(d->ptr, d->host.data(), d->host.size(), hipMemcpyHostToDevice, st)) != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync (tables into scratch)");
    if ((e = hipEventRecord(d->copied, st)) != hipSuccess) {
        (void)hipStreamSynchronize(st);
        return hip_fail(e, "hipEventRecord");
    }
    d->pending = true;
    for (const Item &it : items) {
        StepArgs a = base_args(hp, chunk);
        a.p_dtype = it.bi % 3;
        a.tens = (const DevTensor *)(d->ptr + it.off);
        a.chunk_tensor = (const int32_t *)(d->ptr + it.off + it.off_ct);
        a.nchunks = it.nchunks;
        a.unorm = hp->max_unorm > 0.0f ? unorm : nullptr;
        size_t lds = 0;
        if (q8) {
            a.q.words = (const uint32_t *)(d->ptr + it.off + it.off_q);
            a.q.nwords = (uint32_t)qw.size();
            a.q.s = ps;
            a.q.u = pu;
            lds = (size_t)a.q.nwords * 4;
        }
        e = launch_step(opt, it.bi / 3, fmt, a, LaunchGeom{d->ncu, g_wgs_per_cu, g_wg_cap}, lds, st);
        if (e != hipSuccess) return hip_fail(e, "step launch");
    }
    return OPT_OK;
}

template <class F>
void mini_host_one(float A, float x, const uint32_t *r, int64_t i, uint8_t *codes, float *decoded)
{
    uint32_t c = 0;
    if (finite_f(A)) {
        const int nsc = mini_enc_shift<F>(A);
        c = r ? mini_encode<F, true>(x, nsc, r[i] & 0xFFFFu) : mini_encode<F, false>(x, nsc, 0u);
    }
    codes[i] = (uint8_t)c;
    decoded[i] = finite_f(A) ? mini_decode<F>(c, mini_dec_shift<F>(A)) : bitsf(0x7FC00000u);
}

int check_mini(int32_t elem, float A, const float *x, uint8_t *codes, float *decoded, int64_t n)
{
    if (elem < 0 || elem > 2) return fail(OPT_EINVAL, "elem must be 0 (E4M3), 1 (E2M1) or 2 (unsigned E2M2)");
    if (n < 0 || (n > 0 && (!x || !codes || !decoded))) return fail(OPT_EINVAL, "bad arguments");
    if (A == A && A < 0.0f) return fail(OPT_EINVAL, "A must not be negative");
    return OPT_OK;
}

}  // namespace
}  // namespace optstep

using namespace optstep;

extern "C" {

int opt_step_adamw(const opt_tensor *tensors, int64_t n, int32_t state_fmt, const opt_hparams *hp,
                   const double *unorm, void *stream)
{
    return run(kAdamW, tensors, n, state_fmt, hp, unorm, nullptr, stream);
}

int opt_step_ademamix(const opt_tensor *tensors, int64_t n, int32_t state_fmt, const opt_hparams *hp,
                      const double *unorm, void *stream)
{
    return run(kAdEMAMix, tensors, n, state_fmt, hp, unorm, nullptr, stream);
}

int opt_step_adamw_noalloc(const opt_tensor *tensors, int64_t n, int32_t state_fmt, const opt_hparams *hp,
                           const double *unorm, void *stream)
{
    return run_noalloc(kAdamW, tensors, n, state_fmt, hp, unorm, stream);
}

int opt_precondition_unorm(int32_t optimizer, const opt_tensor *tensors, int64_t n, int32_t state_fmt,
                           const opt_hparams *hp, double *unorm_out, void *stream)
{
    if (optimizer != kAdamW && optimizer != kAdEMAMix) return fail(OPT_EINVAL, "unknown optimizer %d", optimizer);
    if (!unorm_out) return fail(OPT_EINVAL, "unorm_out is NULL");
    return run(optimizer, tensors, n, state_fmt, hp, nullptr, unorm_out, stream);
}

int opt_grad_norm(const opt_grad *grads, int64_t n, double *out, float max_norm, int32_t norm_type,
                  float *coef_out, void *stream)
{
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (n > 0 && !grads) return fail(OPT_EINVAL, "grads is NULL");
    if (n > INT32_MAX) return fail(OPT_EINVAL, "too many tensors");
    if (!out) return fail(OPT_EINVAL, "out is NULL");
    if (!aligned(out, 8)) return fail(OPT_EALIGN, "out must be 8-byte aligned");
    if (coef_out) {
        if (norm_type != 2 && norm_type != 0) return fail(OPT_EINVAL, "norm_type must be 2 or 0 (inf)");
        if (!(max_norm > 0.0f) || !std::isfinite(max_norm)) return fail(OPT_EINVAL, "max_norm must be finite and > 0");
        if (!aligned(coef_out, 4)) return fail(OPT_EALIGN, "coef_out must be 4-byte aligned");
    }
    std::vector<opt_tensor> t((size_t)n);
    for (int64_t k = 0; k < n; ++k) {
        const opt_grad &x = grads[k];
        if (x.numel < 0) return fail(OPT_EINVAL, "tensor %lld: numel < 0", (long long)k);
        if (x.numel > kMaxNumel) return fail(OPT_EINVAL, "tensor %lld: numel above 2^46", (long long)k);
        if (x.dtype != OPT_F32 && x.dtype != OPT_BF16 && x.dtype != OPT_F16)
            return fail(OPT_EINVAL, "tensor %lld: unknown dtype %d", (long long)k, x.dtype);
        if (x.numel > 0 && !x.g) return fail(OPT_EINVAL, "tensor %lld: g is NULL", (long long)k);
        if (x.numel > 0 && !aligned(x.g, 16)) return fail(OPT_EALIGN, "tensor %lld: g must be 16-byte aligned", (long long)k);
        t[k] = opt_tensor{};
        t[k].g = x.g;
        t[k].numel = x.numel;
        t[k].p_dtype = OPT_F32;
        t[k].g_dtype = x.dtype;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace *w;
    int rc;
    if ((rc = workspace(w)) != OPT_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t chunk = g_chunk;
    std::vector<PlanItem> items;
    size_t need = 0;
    if ((rc = plan_call(*w, 1, 0, 0, true, t.data(), n, nullptr, st, items, need)) != OPT_OK) return rc;
    if ((rc = partials_reserve(*w, need, st)) != OPT_OK) return rc;
    hipError_t e;
    for (const PlanItem &it : items) {
        Slot *s = it.slot;
        StepArgs a{};
        a.tens = (const DevTensor *)s->dev;
        a.chunk_tensor = (const int32_t *)((unsigned char *)s->dev + it.off_ct);
        a.nchunks = it.nchunks;
        a.chunk = chunk;
        a.partials = w->partials;
        a.groups = w->partials + it.partial_doubles;
        a.ngroups = it.ngroups;
        e = launch_gnorm(it.bi / 3, a, geom(*w), it.ntens, out, st);
        if (e != hipSuccess) return hip_fail(e, "gradient norm launch");
        if ((rc = slot_mark_used(*s, st)) != OPT_OK) return rc;
    }
    e = launch_gnorm_total(n, out, max_norm, norm_type, coef_out, st);
    if (e != hipSuccess) return hip_fail(e, "gradient norm total launch");
    w->partials_used = true;
    w->partials_stream = st;
    if ((e = hipEventRecord(w->partials_ev, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return OPT_OK;
}

int opt_step_1state(int32_t optimizer, const opt_tensor *t, int64_t n, int32_t state_fmt, const opt_hparams *hp,
                    void *stream)
{
    int rc;
    if (optimizer < OPT_MOMENTUM || optimizer > OPT_LION) return fail(OPT_EINVAL, "unknown one-state optimizer %d", optimizer);
    if (state_fmt < kF32 || state_fmt > kFP4SR) return fail(OPT_EINVAL, "unknown state format %d", state_fmt);
    if (blocked(state_fmt))
        return fail(OPT_EUNSUPPORTED, "the one-state optimizers take fp32 or BF16 states");
    if ((rc = check_hparams(hp, state_fmt)) != OPT_OK) return rc;
    if (hp->max_unorm > 0.0f) return fail(OPT_EUNSUPPORTED, "max_unorm is provided for the two-state optimizers only");
    if (!(hp->beta1 >= 0.0f && hp->beta1 <= 1.0f)) return fail(OPT_EINVAL, "beta1 must lie in [0, 1]");
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (n > 0 && !t) return fail(OPT_EINVAL, "tensors is NULL");
    if (n > INT32_MAX) return fail(OPT_EINVAL, "too many tensors");
    for (int64_t k = 0; k < n; ++k) {
        const opt_tensor &x = t[k];
        if (x.numel < 0) return fail(OPT_EINVAL, "tensor %lld: numel < 0", (long long)k);
        if (x.g_dtype != OPT_F32 && x.g_dtype != OPT_BF16 && x.g_dtype != OPT_F16)
            return fail(OPT_EINVAL, "tensor %lld: unknown g_dtype %d", (long long)k, x.g_dtype);
        if (x.p_dtype != OPT_F32)
            return fail(OPT_EUNSUPPORTED, "tensor %lld: the one-state optimizers take fp32 parameters", (long long)k);
        if ((rc = check_slice(x, k, 4)) != OPT_OK) return rc;
        if (x.numel == 0) continue;
        if (!x.p || !x.g || !x.s1) return fail(OPT_EINVAL, "tensor %lld: missing p, g or s1", (long long)k);
        if (!aligned(x.p, 16) || !aligned(x.g, 16) || !aligned(x.s1, 16))
            return fail(OPT_EALIGN, "tensor %lld: p, g and s1 must be 16-byte aligned", (long long)k);
    }
    if (n == 0) return OPT_OK;
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace *w;
    if ((rc = workspace(w)) != OPT_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t chunk = g_chunk;
    std::vector<PlanItem> items;
    size_t need = 0;
    if ((rc = plan_call(*w, 2, optimizer, state_fmt, false, t, n, nullptr, st, items, need)) != OPT_OK) return rc;
    for (const PlanItem &it : items) {
        Slot *s = it.slot;
        StepArgs a = base_args(hp, chunk);
        a.tens = (const DevTensor *)s->dev;
        a.chunk_tensor = (const int32_t *)((unsigned char *)s->dev + it.off_ct);
        a.nchunks = it.nchunks;
        hipError_t e = launch_step_1state(optimizer, it.bi / 3, state_fmt, a, geom(*w), st);
        if (e != hipSuccess) return hip_fail(e, "one-state step launch");
        if ((rc = slot_mark_used(*s, st)) != OPT_OK) return rc;
    }
    return OPT_OK;
}

int opt_round_cast(const float *x, void *out, int64_t n, int32_t out_dtype, int32_t stochastic, uint64_t seed,
                   uint64_t offset, void *stream)
{
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (n > kMaxNumel) return fail(OPT_EINVAL, "n above 2^46");
    if (out_dtype != OPT_BF16 && out_dtype != OPT_F16) return fail(OPT_EINVAL, "out_dtype must be OPT_BF16 or OPT_F16");
    if (stochastic != 0 && stochastic != 1) return fail(OPT_EINVAL, "stochastic must be 0 or 1");
    if (n == 0) return OPT_OK;
    if (!x || !out) return fail(OPT_EINVAL, "x or out is NULL");
    if (!aligned(x, 16) || !aligned(out, 8)) return fail(OPT_EALIGN, "x must be 16-byte and out 8-byte aligned");
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace *w;
    int rc;
    if ((rc = workspace(w)) != OPT_OK) return rc;
    hipError_t e = launch_round_cast(x, (uint16_t *)out, n, out_dtype == OPT_BF16, stochastic, seed, offset, geom(*w),
                                     (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "round cast launch");
}

const char *opt_last_error(void) { return g_err.c_str(); }

int opt_shutdown(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (int d = 0; d < kMaxDevices; ++d) {
        Workspace &w = g_ws[d];
        if (!w.init) continue;
        (void)hipSetDevice(d);
        (void)hipDeviceSynchronize();
        for (Slot &s : w.slots) {
            if (s.dev) (void)hipFree(s.dev);
            if (s.host) (void)hipHostFree(s.host);
            if (s.ev) (void)hipEventDestroy(s.ev);
            if (s.ready) (void)hipEventDestroy(s.ready);
            s = Slot();
        }
        if (w.partials) (void)hipFree(w.partials);
        if (w.partials_ev) (void)hipEventDestroy(w.partials_ev);
        w = Workspace();
    }
    (void)hipSetDevice(cur);
    return OPT_OK;
}

int opt_debug_philox(uint64_t seed, int64_t t, int32_t k, int64_t j0, int64_t count, uint32_t *out,
                     void *stream)
{
    if (count < 0 || j0 < 0) return fail(OPT_EINVAL, "negative count or start");
    if (count == 0) return OPT_OK;
    if (!out) return fail(OPT_EINVAL, "out is NULL");
    hipError_t e = launch_debug_philox(seed, t, k, j0, count, out, (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "debug philox launch");
}

int opt_debug_round_bf16(const float *x, const uint32_t *r, uint16_t *out, int64_t n, void *stream)
{
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (n == 0) return OPT_OK;
    if (!x || !out) return fail(OPT_EINVAL, "x or out is NULL");
    hipError_t e = launch_debug_round(x, r, out, n, (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "debug round launch");
}

int opt_debug_direction(int32_t optimizer, const opt_hparams *hp, const float *g, const float *m, const float *v,
                        const float *m2, float *out, int64_t n, void *stream)
{
    if (optimizer != OPT_ADAMW && optimizer != OPT_ADEMAMIX) return fail(OPT_EINVAL, "optimizer must be AdamW or AdEMAMix");
    if (!hp) return fail(OPT_EINVAL, "hp is NULL");
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (n == 0) return OPT_OK;
    if (!g || !m || !v || !out || (optimizer == OPT_ADEMAMIX && !m2)) return fail(OPT_EINVAL, "NULL array");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f) || hp->step < 1)
        return fail(OPT_EINVAL, "betas must be in [0, 1) and step >= 1");
    StepArgs a{};
    a.lr = hp->lr;
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.beta3 = hp->beta3;
    a.alpha = hp->alpha;
    a.eps = hp->eps;
    a.wd = hp->weight_decay;
    a.bc_step = hp->step;
    a.grad_scale = nullptr;
    a.sc = make_scalars(a);
    hipError_t e = launch_debug_direction(optimizer == OPT_ADEMAMIX ? kAdEMAMix : kAdamW, a, g, m, v, m2, out, n,
                                          (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "debug direction launch");
}

int opt_debug_quantize(const float *qmap, int32_t is_signed, const float *x, uint8_t *out, int64_t n,
                       void *stream)
{
    if (n < 0) return fail(OPT_EINVAL, "n < 0");
    if (!qmap) return fail(OPT_EINVAL, "qmap is NULL");
    BuiltTable B;
    int rc = build_search(qmap, is_signed != 0, B);
    if (rc != OPT_OK) return rc;
    if (n == 0) return OPT_OK;
    if (!x || !out) return fail(OPT_EINVAL, "x or out is NULL");
    std::vector<uint32_t> words(512 + B.entries.size());
    memcpy(words.data() + (is_signed ? 0 : 256), qmap, 1024);
    std::copy(B.entries.begin(), B.entries.end(), words.begin() + 512);
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace *w;
    if ((rc = workspace(w)) != OPT_OK) return rc;
    std::vector<unsigned char> blob(words.size() * 4);
    memcpy(blob.data(), words.data(), blob.size());
    Slot *s;
    hipStream_t st = (hipStream_t)stream;
    if ((rc = upload(*w, blob, st, s)) != OPT_OK) return rc;
    QTabs q{};
    q.words = (const uint32_t *)s->dev;
    q.nwords = (uint32_t)words.size();
    QTabParams P = B.P;
    P.offset = 512;
    if (is_signed) q.s = P; else q.u = P;
    hipError_t e = launch_debug_quantize(q, is_signed, x, out, n, st);
    if (e != hipSuccess) return hip_fail(e, "debug quantize launch");
    return slot_mark_used(*s, st);
}

int opt_debug_quantize_host(const float *qmap, int32_t is_signed, const float *x, uint8_t *out, int64_t n)
{
    if (n < 0 || !qmap || (n > 0 && (!x || !out))) return fail(OPT_EINVAL, "bad arguments");
    BuiltTable B;
    int rc = build_search(qmap, is_signed != 0, B);
    if (rc != OPT_OK) return rc;
    QTabParams P = B.P;
    P.offset = 0;
    for (int64_t i = 0; i < n; ++i) {
        float v = x[i];
        if (v != v) { out[i] = 0; continue; }
        if (!(std::fabs(v) <= 1.0f)) return fail(OPT_EINVAL, "x[%lld] is outside [-1, 1]", (long long)i);
        out[i] = (uint8_t)q8_lookup(v, B.entries.data(), P, is_signed != 0);
    }
    return OPT_OK;
}


int opt_debug_mini_host(int32_t elem, float A, const float *x, const uint32_t *r, uint8_t *codes, float *decoded,
                        int64_t n)
{
    int rc = check_mini(elem, A, x, codes, decoded, n);
    if (rc != OPT_OK) return rc;
    for (int64_t i = 0; i < n; ++i) {
        if (elem == 0) mini_host_one<E4M3>(A, x[i], r, i, codes, decoded);
        else if (elem == 1) mini_host_one<E2M1>(A, x[i], r, i, codes, decoded);
        else mini_host_one<E2M2U>(A, x[i], r, i, codes, decoded);
    }
    return OPT_OK;
}

int opt_debug_mini(int32_t elem, float A, const float *x, const uint32_t *r, uint8_t *codes, float *decoded,
                   int64_t n, void *stream)
{
    int rc = check_mini(elem, A, x, codes, decoded, n);
    if (rc != OPT_OK || n == 0) return rc;
    hipError_t e = launch_debug_mini(elem, A, x, r, codes, decoded, n, (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "debug mini launch");
}

int opt_debug_mini_pack(int32_t elem, float A, const float *x, const uint32_t *r, uint8_t *codes, int64_t n,
                        void *stream)
{
    if (elem < 0 || elem > 2) return fail(OPT_EINVAL, "elem must be 0 (E4M3), 1 (E2M1) or 2 (unsigned E2M2)");
    if (n < 0 || n % 4 != 0) return fail(OPT_EINVAL, "n must be a non-negative multiple of 4");
    if (n > 0 && (!x || !codes)) return fail(OPT_EINVAL, "x or codes is NULL");
    if (A == A && A < 0.0f) return fail(OPT_EINVAL, "A must not be negative");
    if (n == 0) return OPT_OK;
    hipError_t e = launch_debug_mini_pack(elem, A, x, r, codes, n, (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "debug mini pack launch");
}

int opt_debug_div_by(const float *a, const float *b, float *out, int64_t n)
{
    if (n < 0 || (n > 0 && (!a || !b || !out))) return fail(OPT_EINVAL, "bad arguments");
    for (int64_t i = 0; i < n; ++i) {
        if (!div_by_ok(b[i])) return fail(OPT_EINVAL, "divisor %lld outside the fast range", (long long)i);
        out[i] = div_by(a[i], b[i], 1.0f / b[i]);
    }
    return OPT_OK;
}

int64_t opt_debug_plan(const int64_t *numels, int64_t n, int64_t *chunks_out)
{
    if (n < 0 || (n > 0 && (!numels || !chunks_out))) return fail(OPT_EINVAL, "bad arguments");
    for (int64_t k = 0; k < n; ++k) {
        if (numels[k] < 0) return fail(OPT_EINVAL, "numel < 0");
        chunks_out[k] = (numels[k] + g_chunk - 1) / g_chunk;
    }
    return g_chunk;
}

int opt_debug_stream(const float *const *src, int32_t nsrc, float *const *dst, int32_t ndst, int64_t n,
                     void *stream)
{
    if (nsrc < 0 || nsrc > 6 || ndst < 1 || ndst > 6 || n < 0 || n % 4 != 0)
        return fail(OPT_EINVAL, "need 0..6 sources, 1..6 destinations and n a multiple of 4");
    if ((nsrc > 0 && !src) || !dst) return fail(OPT_EINVAL, "NULL array list");
    for (int k = 0; k < nsrc; ++k)
        if (!src[k] || !aligned(src[k], 16)) return fail(OPT_EALIGN, "source %d not 16-byte aligned", k);
    for (int k = 0; k < ndst; ++k)
        if (!dst[k] || !aligned(dst[k], 16)) return fail(OPT_EALIGN, "destination %d not 16-byte aligned", k);
    if (n == 0) return OPT_OK;
    Workspace *w;
    int rc;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if ((rc = workspace(w)) != OPT_OK) return rc;
    }
    hipError_t e = launch_debug_stream(src, nsrc, dst, ndst, n, geom(*w), (hipStream_t)stream);
    return e == hipSuccess ? OPT_OK : hip_fail(e, "debug stream launch");
}

int opt_debug_set_launch(int64_t chunk, int32_t wgs_per_cu)
{
    if (chunk < 1024 || chunk > (1 << 24) || (chunk & (chunk - 1)) != 0)
        return fail(OPT_EINVAL, "chunk must be a power of two in [1024, 2^24]");
    if (wgs_per_cu < 0 || wgs_per_cu > 64) return fail(OPT_EINVAL, "wgs_per_cu must be in [0, 64]");
    std::lock_guard<std::mutex> lock(g_mu);
    g_chunk = chunk;
    g_wgs_per_cu = wgs_per_cu;
    return OPT_OK;
}

int opt_debug_scalars(const opt_hparams *hp, float *out)
{
    if (!hp || !out) return fail(OPT_EINVAL, "hp or out is NULL");
    const StepArgs a = base_args(hp, 32768);
    const Scalars &c = a.sc;
    const float v[10] = {c.om1, c.om2, c.om3, c.c1, c.c2, c.rc1, c.rc2, c.d, c.lam, c.gs};
    memcpy(out, v, sizeof v);
    return OPT_OK;
}

int opt_debug_set_wg_cap(int32_t cap)
{
    if (cap != -1 && (cap < 0 || cap == 1 || cap > 32)) return fail(OPT_EINVAL, "cap must be -1, 0 or in [2, 32]");
    std::lock_guard<std::mutex> lock(g_mu);
    g_wg_cap = cap;
    return OPT_OK;
}

}  // extern "C"

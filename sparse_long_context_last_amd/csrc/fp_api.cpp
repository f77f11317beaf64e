// Host side of the C ABI declared in include/fp_prefill.h: argument
// validation (before any HIP call), plan ownership, stream-ordered workspace
// and kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "fp_launch.h"
#include "fp_prefill.h"

using namespace fp;

struct fp_plan {
    int B, Hq, Hkv, N, d, bs, nb;
    fp_dtype dtype;
    float gamma, tau;
    int min_budget, max_budget, qa_selection;
    int device;
    hipStream_t stream;
    PlanDev dev;
    std::vector<void*> allocs;
};

namespace {

thread_local char g_err[512] = "";

fp_status fail(fp_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

fp_status hip_fail(hipError_t e, const char* what) {
    return fail(e == hipErrorOutOfMemory ? FP_ERR_OOM : FP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FP_HIP(call, what)                                  \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return hip_fail(e_, what);    \
    } while (0)

// ---------------------------------------------------------------- validation
fp_status check_shape(fp_dtype dtype, int B, int Hq, int Hkv, int N, int d, int block) {
    if (dtype != FP_BF16 && dtype != FP_FP32) return fail(FP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0) return fail(FP_ERR_INVALID_ARG, "negative size");
    if (d != kHeadDim) return fail(FP_ERR_UNSUPPORTED, "head dim %d (supported: %d)", d, kHeadDim);
    if (block != 64 && block != 128) return fail(FP_ERR_UNSUPPORTED, "block %d (supported: 64, 128)", block);
    if (Hkv == 0 && Hq != 0) return fail(FP_ERR_SHAPE, "Hkv = 0 with Hq = %d", Hq);
    if (Hkv > 0 && Hq % Hkv != 0) return fail(FP_ERR_SHAPE, "Hq %d not a multiple of Hkv %d", Hq, Hkv);
    if (N % block != 0) return fail(FP_ERR_SHAPE, "N %d not a multiple of block %d", N, block);
    if (N / block > kMaxBlocks) return fail(FP_ERR_SHAPE, "N / block = %d exceeds %d", N / block, kMaxBlocks);
    const long long rows = (long long)B * Hq * (N / block);
    if (rows > 0x7FFFFFFFLL) return fail(FP_ERR_SHAPE, "too many query-block rows");
    return FP_OK;
}

bool empty_problem(int B, int Hq, int N) { return B == 0 || Hq == 0 || N == 0; }

// ------------------------------------------------------------ canonical consts
long double ln2_ld() { return 0.693147180559945309417232121458176568L; }

Canon make_canon(int d) {
    Canon K;
    long double pw = 1.0L, fact = 1.0L;
    for (int k = 0; k < 8; ++k) {
        if (k > 0) {
            pw *= ln2_ld();
            fact *= (long double)k;
        }
        K.e2[k] = (float)(pw / fact);
    }
    for (int k = 0; k < 11; ++k) K.lnc[k] = 1.0 / (double)(2 * k + 1);
    K.ln2 = (double)ln2_ld();
    K.sqrt_half = std::sqrt(0.5);
    const double log2e = (double)(1.0L / ln2_ld());
    K.C = (float)(log2e / std::sqrt((double)d));
    return K;
}

// ------------------------------------------------------------------ profiling
std::mutex g_prof_mu;
bool g_prof_on = false;
struct EvPair {
    hipEvent_t a, b;
    bool dense;
};
std::vector<EvPair> g_prof_events;
double g_prof_ms[2] = {0, 0};
long long g_prof_n[2] = {0, 0};

fp_status drain_profile_events() {
    for (auto& e : g_prof_events) {
        FP_HIP(hipEventSynchronize(e.b), "hipEventSynchronize");
        float ms = 0.f;
        FP_HIP(hipEventElapsedTime(&ms, e.a, e.b), "hipEventElapsedTime");
        g_prof_ms[e.dense ? 1 : 0] += ms;
        g_prof_n[e.dense ? 1 : 0] += 1;
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    g_prof_events.clear();
    return FP_OK;
}

void set_pool_threshold(int dev) {
    static std::mutex mu;
    static std::vector<int> done;
    std::lock_guard<std::mutex> g(mu);
    for (int x : done)
        if (x == dev) return;
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
        uint64_t thr = ~0ull;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    done.push_back(dev);
}

template <typename T>
fp_status palloc(fp_plan* p, T** ptr, size_t count) {
    void* q = nullptr;
    const size_t bytes = count * sizeof(T) > 0 ? count * sizeof(T) : 16;
    FP_HIP(hipMallocAsync(&q, bytes, p->stream), "hipMallocAsync (plan)");
    p->allocs.push_back(q);
    *ptr = (T*)q;
    return FP_OK;
}

void free_plan(fp_plan* p) {
    for (void* q : p->allocs) (void)hipFreeAsync(q, p->stream);
    p->allocs.clear();
    delete p;
}

fp_status attend_common(const void* q, const void* k, const void* v, void* o, fp_dtype dtype, int B, int Hq,
                        int Hkv, int N, int block, const fp_plan* plan, hipStream_t st) {
    const int nb = N / block;
    const size_t esz = dtype == FP_BF16 ? 2 : 4;
    int dev = 0;
    FP_HIP(hipGetDevice(&dev), "hipGetDevice");
    set_pool_threshold(dev);
    void* vt = nullptr;
    FP_HIP(hipMallocAsync(&vt, (size_t)B * Hkv * N * kHeadDim * esz, st), "hipMallocAsync (V^T)");
    hipError_t e = launch_transpose_v(v, vt, dtype == FP_BF16, B * Hkv, N, st);
    if (e != hipSuccess) {
        (void)hipFreeAsync(vt, st);
        return hip_fail(e, "transpose V");
    }
    AttnArgs a{};
    a.q = q;
    a.k = k;
    a.vt = vt;
    a.o = o;
    a.dtype_bf16 = dtype == FP_BF16;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.BS = block;
    a.nb = nb;
    a.tri = (long long)nb * (nb + 1) / 2;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)kHeadDim));
    if (plan) {
        a.lists = plan->dev.lists;
        a.counts = plan->dev.counts;
    }
    EvPair ev{};
    bool prof;
    {
        std::lock_guard<std::mutex> g(g_prof_mu);
        prof = g_prof_on;
    }
    if (prof) {
        FP_HIP(hipEventCreate(&ev.a), "hipEventCreate");
        FP_HIP(hipEventCreate(&ev.b), "hipEventCreate");
        ev.dense = plan == nullptr;
        FP_HIP(hipEventRecord(ev.a, st), "hipEventRecord");
    }
    e = launch_attention(a, st);
    if (prof) {
        FP_HIP(hipEventRecord(ev.b, st), "hipEventRecord");
        std::lock_guard<std::mutex> g(g_prof_mu);
        g_prof_events.push_back(ev);
    }
    (void)hipFreeAsync(vt, st);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return FP_OK;
}

}  // namespace

extern "C" {

const char* fp_status_str(fp_status s) {
    switch (s) {
        case FP_OK: return "FP_OK";
        case FP_ERR_INVALID_ARG: return "FP_ERR_INVALID_ARG";
        case FP_ERR_UNSUPPORTED: return "FP_ERR_UNSUPPORTED";
        case FP_ERR_SHAPE: return "FP_ERR_SHAPE";
        case FP_ERR_OOM: return "FP_ERR_OOM";
        case FP_ERR_HIP: return "FP_ERR_HIP";
    }
    return "FP_ERR_UNKNOWN";
}

const char* fp_last_error(void) { return g_err; }

fp_status fp_canonical_constants(int d, float* e2, double* lnc, double* ln2, double* sqrt_half, float* score_scale) {
    if (d <= 0) return fail(FP_ERR_INVALID_ARG, "d must be positive");
    const Canon K = make_canon(d);
    if (e2) memcpy(e2, K.e2, sizeof K.e2);
    if (lnc) memcpy(lnc, K.lnc, sizeof K.lnc);
    if (ln2) *ln2 = K.ln2;
    if (sqrt_half) *sqrt_half = K.sqrt_half;
    if (score_scale) *score_scale = K.C;
    return FP_OK;
}

fp_status fp_prefill_plan(const void* q, const void* k, fp_dtype dtype, int B, int Hq, int Hkv, int N, int d,
                          int block, float gamma, float tau, int min_budget, void* stream, fp_plan** out) {
    return fp_prefill_plan_ex(q, k, dtype, B, Hq, Hkv, N, d, block, gamma, tau, min_budget, nullptr, stream, out);
}

fp_status fp_prefill_plan_ex(const void* q, const void* k, fp_dtype dtype, int B, int Hq, int Hkv, int N, int d,
                             int block, float gamma, float tau, int min_budget, const fp_plan_options* options,
                             void* stream, fp_plan** out) {
    if (!out) return fail(FP_ERR_INVALID_ARG, "out is NULL");
    const int max_budget = options ? options->max_budget : 0;
    const int qa_selection = options ? options->qa_selection : FP_QA_FLATTENED;
    *out = nullptr;
    fp_status s = check_shape(dtype, B, Hq, Hkv, N, d, block);
    if (s != FP_OK) return s;
    if (!(gamma > 0.0f && gamma <= 1.0f)) return fail(FP_ERR_INVALID_ARG, "gamma %g outside (0, 1]", (double)gamma);
    if (!(tau >= 0.0f) || std::isinf(tau)) return fail(FP_ERR_INVALID_ARG, "tau %g must be finite and >= 0", (double)tau);
    if (min_budget < 0) return fail(FP_ERR_INVALID_ARG, "min_budget %d < 0", min_budget);
    if (max_budget < 0) return fail(FP_ERR_INVALID_ARG, "max_budget %d < 0", max_budget);
    if (qa_selection != FP_QA_FLATTENED && qa_selection != FP_QA_QUERYWISE)
        return fail(FP_ERR_INVALID_ARG, "qa_selection %d is not FP_QA_FLATTENED or FP_QA_QUERYWISE", qa_selection);
    {
        const long long floor_b = std::max(1LL, ((long long)min_budget + block - 1) / block);
        const long long cap_b = ((long long)max_budget + block - 1) / block;
        if (max_budget > 0 && cap_b < floor_b)
            return fail(FP_ERR_INVALID_ARG, "max_budget %d allows %lld blocks per row, min_budget needs %lld",
                        max_budget, cap_b, floor_b);
    }
    const bool empty = empty_problem(B, Hq, N);
    if (!empty && (!q || !k)) return fail(FP_ERR_INVALID_ARG, "q or k is NULL");

    fp_plan* p = new (std::nothrow) fp_plan();
    if (!p) return fail(FP_ERR_OOM, "host allocation failed");
    p->B = B; p->Hq = Hq; p->Hkv = Hkv; p->N = N; p->d = d; p->bs = block;
    p->nb = N / block; p->dtype = dtype; p->gamma = gamma; p->tau = tau; p->min_budget = min_budget;
    p->max_budget = max_budget;
    p->qa_selection = qa_selection;
    p->stream = (hipStream_t)stream;
    if (empty) {
        p->device = -1;
        memset(&p->dev, 0, sizeof p->dev);
        *out = p;
        return FP_OK;
    }
    hipError_t he = hipGetDevice(&p->device);
    if (he != hipSuccess) {
        delete p;
        return hip_fail(he, "hipGetDevice");
    }
    set_pool_threshold(p->device);

    PlanDev& P = p->dev;
    memset(&P, 0, sizeof P);
    const int BH = B * Hq, nb = p->nb;
    P.BH = BH; P.BS = block; P.N = N; P.nb = nb;
    P.tri = (long long)nb * (nb + 1) / 2;
    const double Gd = std::nearbyint((double)gamma * (double)(1 << kGammaShift));
    const unsigned long long G = (unsigned long long)Gd;
    P.mode_all = G >= (1ull << kGammaShift);
    P.floor_blocks = (min_budget + block - 1) / block;
    if (P.floor_blocks < 1) P.floor_blocks = 1;
    P.cap_blocks = (int)(((long long)max_budget + block - 1) / block);
    P.qa_querywise = qa_selection == FP_QA_QUERYWISE;
    P.G = G;

#define PALLOC(ptr, n)                          \
    do {                                        \
        fp_status s_ = palloc(p, &(ptr), (n));  \
        if (s_ != FP_OK) {                      \
            free_plan(p);                       \
            return s_;                          \
        }                                       \
    } while (0)
    PALLOC(P.pattern, (size_t)BH);
    PALLOC(P.djs, (size_t)BH);
    PALLOC(P.qbar, (size_t)BH * nb * kHeadDim);
    PALLOC(P.kbar, (size_t)B * Hkv * nb * kHeadDim);
    PALLOC(P.rowmax, (size_t)BH * block);
    PALLOC(P.rowsum, (size_t)BH * block);
    PALLOC(P.colsum, (size_t)BH * N);
    PALLOC(P.diagsum, (size_t)BH * N);
    PALLOC(P.atrue, (size_t)BH * nb);
    PALLOC(P.ahat, (size_t)BH * P.tri);
    PALLOC(P.sel, (size_t)2 * BH);
    PALLOC(P.hist, (size_t)2 * BH * kRadixBins);
    PALLOC(P.colblk, (size_t)BH * nb);
    PALLOC(P.diagA, (size_t)BH * nb);
    PALLOC(P.diagB, (size_t)BH * nb);
    PALLOC(P.colmass, P.cap_blocks > 0 ? (size_t)BH * nb : 0);
    PALLOC(P.diagmass, P.cap_blocks > 0 ? (size_t)BH * nb : 0);
    PALLOC(P.lists, (size_t)BH * P.tri);
    PALLOC(P.counts, (size_t)BH * nb);
    PALLOC(P.total_blocks, (size_t)BH);
#undef PALLOC

    PlanArgs a{};
    a.q = q; a.k = k; a.dtype_bf16 = dtype == FP_BF16;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv;
    a.tau = (double)tau;
    a.G = G;
    a.canon = make_canon(d);
    const int nchunks = (N + 255) / 256;
    void *s2 = nullptr, *pmax = nullptr, *rz = nullptr;
    hipStream_t st = p->stream;
    he = hipMallocAsync(&s2, (size_t)BH * block * N * sizeof(float), st);
    if (he == hipSuccess) he = hipMallocAsync(&pmax, (size_t)BH * nchunks * block * sizeof(float), st);
    if (he == hipSuccess) he = hipMallocAsync(&rz, (size_t)BH * block * sizeof(float), st);
    if (he == hipSuccess) {
        a.s2 = (float*)s2; a.pmax = (float*)pmax; a.rz = (float*)rz;
        he = launch_plan(a, P, st);
    }
    if (s2) (void)hipFreeAsync(s2, st);
    if (pmax) (void)hipFreeAsync(pmax, st);
    if (rz) (void)hipFreeAsync(rz, st);
    if (he != hipSuccess) {
        free_plan(p);
        return hip_fail(he, "planning");
    }
    *out = p;
    return FP_OK;
}

fp_status fp_prefill_attend(const fp_plan* plan, const void* q, const void* k, const void* v, void* o, void* stream) {
    if (!plan) return fail(FP_ERR_INVALID_ARG, "plan is NULL");
    if (empty_problem(plan->B, plan->Hq, plan->N)) return FP_OK;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID_ARG, "q, k, v or o is NULL");
    return attend_common(q, k, v, o, plan->dtype, plan->B, plan->Hq, plan->Hkv, plan->N, plan->bs, plan,
                         (hipStream_t)stream);
}

fp_status fp_dense_attend(const void* q, const void* k, const void* v, void* o, fp_dtype dtype, int B, int Hq,
                          int Hkv, int N, int d, int block, void* stream) {
    fp_status s = check_shape(dtype, B, Hq, Hkv, N, d, block);
    if (s != FP_OK) return s;
    if (empty_problem(B, Hq, N)) return FP_OK;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID_ARG, "q, k, v or o is NULL");
    return attend_common(q, k, v, o, dtype, B, Hq, Hkv, N, block, nullptr, (hipStream_t)stream);
}

fp_status fp_plan_info_get(const fp_plan* plan, fp_plan_info* out) {
    if (!plan || !out) return fail(FP_ERR_INVALID_ARG, "plan or out is NULL");
    fp_plan_info I{};
    I.B = plan->B; I.Hq = plan->Hq; I.Hkv = plan->Hkv; I.N = plan->N; I.d = plan->d;
    I.block = plan->bs; I.nb = plan->nb; I.dtype = plan->dtype; I.gamma = plan->gamma; I.tau = plan->tau;
    I.min_budget = plan->min_budget;
    I.max_budget = plan->max_budget;
    I.qa_selection = plan->qa_selection;
    const long long BH = (long long)plan->B * plan->Hq;
    I.dense_blocks = BH * plan->nb * (long long)(plan->nb + 1) / 2;
    if (BH > 0 && plan->N > 0) {
        FP_HIP(hipStreamSynchronize(plan->stream), "hipStreamSynchronize");
        std::vector<unsigned long long> per_head((size_t)BH);
        FP_HIP(hipMemcpy(per_head.data(), plan->dev.total_blocks, per_head.size() * sizeof(unsigned long long),
                         hipMemcpyDeviceToHost), "hipMemcpy");
        long long tot = 0;
        for (unsigned long long x : per_head) tot += (long long)x;
        I.total_blocks = tot;
        std::vector<unsigned char> pat((size_t)BH);
        FP_HIP(hipMemcpy(pat.data(), plan->dev.pattern, pat.size(), hipMemcpyDeviceToHost), "hipMemcpy");
        for (unsigned char c : pat) I.query_aware_heads += c == kPatternQueryAware;
    }
    *out = I;
    return FP_OK;
}

fp_status fp_plan_copy_out(const fp_plan* plan, unsigned char* pattern, double* djs, int* row_ptr, int* col_idx,
                           void* stream) {
    if (!plan) return fail(FP_ERR_INVALID_ARG, "plan is NULL");
    if ((row_ptr == nullptr) != (col_idx == nullptr)) return fail(FP_ERR_INVALID_ARG, "give both row_ptr and col_idx");
    const long long BH = (long long)plan->B * plan->Hq;
    const int nb = plan->nb;
    if (BH == 0 || plan->N == 0) {
        if (row_ptr) row_ptr[0] = 0;
        return FP_OK;
    }
    hipStream_t st = (hipStream_t)stream;
    FP_HIP(hipStreamSynchronize(plan->stream), "hipStreamSynchronize");
    if (pattern) FP_HIP(hipMemcpyAsync(pattern, plan->dev.pattern, (size_t)BH, hipMemcpyDeviceToHost, st), "copy pattern");
    if (djs) FP_HIP(hipMemcpyAsync(djs, plan->dev.djs, (size_t)BH * sizeof(double), hipMemcpyDeviceToHost, st), "copy djs");
    if (row_ptr) {
        std::vector<int> counts((size_t)BH * nb);
        const long long tri = plan->dev.tri;
        std::vector<int> lists((size_t)(BH * tri));
        FP_HIP(hipMemcpyAsync(counts.data(), plan->dev.counts, counts.size() * sizeof(int), hipMemcpyDeviceToHost, st),
               "copy counts");
        FP_HIP(hipMemcpyAsync(lists.data(), plan->dev.lists, lists.size() * sizeof(int), hipMemcpyDeviceToHost, st),
               "copy lists");
        FP_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");
        long long acc = 0;
        for (long long bh = 0; bh < BH; ++bh)
            for (int r = 0; r < nb; ++r) {
                const long long i = bh * nb + r;
                row_ptr[i] = (int)acc;
                const int c = counts[(size_t)i];
                memcpy(col_idx + acc, lists.data() + bh * tri + (long long)r * (r + 1) / 2, (size_t)c * sizeof(int));
                acc += c;
            }
        row_ptr[BH * nb] = (int)acc;
    }
    FP_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");
    return FP_OK;
}

fp_status fp_plan_copy_debug(const fp_plan* plan, int which, void* host_dst, size_t bytes) {
    if (!plan || !host_dst) return fail(FP_ERR_INVALID_ARG, "plan or destination is NULL");
    const PlanDev& P = plan->dev;
    const size_t BH = (size_t)plan->B * plan->Hq, nb = (size_t)plan->nb;
    const void* src = nullptr;
    size_t need = 0;
    switch (which) {
        case FP_DBG_QBAR: src = P.qbar; need = BH * nb * kHeadDim * 4; break;
        case FP_DBG_KBAR: src = P.kbar; need = (size_t)plan->B * plan->Hkv * nb * kHeadDim * 4; break;
        case FP_DBG_ROWMAX: src = P.rowmax; need = BH * plan->bs * 4; break;
        case FP_DBG_ROWSUM: src = P.rowsum; need = BH * plan->bs * 4; break;
        case FP_DBG_COLSUM: src = P.colsum; need = BH * plan->N * 4; break;
        case FP_DBG_DIAGSUM: src = P.diagsum; need = BH * plan->N * 4; break;
        case FP_DBG_ATRUE: src = P.atrue; need = BH * nb * 4; break;
        case FP_DBG_AHAT: src = P.ahat; need = BH * (size_t)P.tri * 4; break;
        case FP_DBG_COUNTS: src = P.counts; need = BH * nb * 4; break;
        default: return fail(FP_ERR_INVALID_ARG, "unknown debug item %d", which);
    }
    if (bytes != need) return fail(FP_ERR_INVALID_ARG, "item %d has %zu bytes, %zu given", which, need, bytes);
    if (need == 0) return FP_OK;
    FP_HIP(hipStreamSynchronize(plan->stream), "hipStreamSynchronize");
    FP_HIP(hipMemcpy(host_dst, src, need, hipMemcpyDeviceToHost), "hipMemcpy");
    return FP_OK;
}

void fp_plan_destroy(fp_plan* plan) {
    if (plan) free_plan(plan);
}

fp_status fp_profile_enable(int on) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_on = on != 0;
    return FP_OK;
}

fp_status fp_profile_read(double* sparse_ms, long long* sparse_launches, double* dense_ms, long long* dense_launches,
                          int reset) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    fp_status s = drain_profile_events();
    if (s != FP_OK) return s;
    if (sparse_ms) *sparse_ms = g_prof_ms[0];
    if (sparse_launches) *sparse_launches = g_prof_n[0];
    if (dense_ms) *dense_ms = g_prof_ms[1];
    if (dense_launches) *dense_launches = g_prof_n[1];
    if (reset) {
        g_prof_ms[0] = g_prof_ms[1] = 0;
        g_prof_n[0] = g_prof_n[1] = 0;
    }
    return FP_OK;
}

fp_status fp_probe_exp2(const float* x, float* y, long long n, void* stream) {
    if (n < 0 || (n > 0 && (!x || !y))) return fail(FP_ERR_INVALID_ARG, "bad probe arguments");
    hipError_t e = launch_probe_exp2(x, y, n, make_canon(kHeadDim), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "probe exp2");
    return FP_OK;
}

fp_status fp_probe_ln(const double* x, double* y, long long n, void* stream) {
    if (n < 0 || (n > 0 && (!x || !y))) return fail(FP_ERR_INVALID_ARG, "bad probe arguments");
    hipError_t e = launch_probe_ln(x, y, n, make_canon(kHeadDim), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "probe ln");
    return FP_OK;
}

fp_status fp_probe_sqrt(const double* x, double* y, long long n, void* stream) {
    if (n < 0 || (n > 0 && (!x || !y))) return fail(FP_ERR_INVALID_ARG, "bad probe arguments");
    hipError_t e = launch_probe_sqrt(x, y, n, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "probe sqrt");
    return FP_OK;
}

}  // extern "C"

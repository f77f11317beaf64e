// Host side of the C ABI declared in include/fp_prefill.h: argument
// validation (before any HIP call), plan ownership, stream-ordered workspace
// and kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <deque>
#include <mutex>
#include <new>
#include <vector>

#include "fp_launch.h"
#include "fp_prefill.h"

using namespace fp;

// One segment of a problem: heads that share one sequence length.  The
// [B, H, N, d] layout is one segment of B sequences; the packed [T, H, d]
// layout has one segment per non-empty sequence.
struct SegHost {
    int b0, nseq;            // first sequence, sequences in the segment
    int L, nb;               // tokens, blocks
    long long tri;           // nb (nb + 1) / 2
    long long qoff, koff;    // element offsets of the segment base in Q/O and K/V
};

struct fp_plan {
    int B, Hq, Hkv, N, d, bs, nb;     // N, nb: longest sequence
    fp_dtype dtype;
    float gamma, tau;
    int min_budget, max_budget, qa_selection, vs_granularity;
    int layout;
    long long tokens, rows, dense_blocks;
    std::vector<int> seqlens;
    TokStride qs, ks;
    std::vector<SegHost> segs;
    std::vector<PlanDev> dev;        // per segment (views into the buffers below)
    std::vector<AttnSeg> aseg_host;  // the attention segment table (host copy)
    AttnSeg* aseg;                   // ... on the device
    // whole-plan buffers; each segment owns a contiguous slice
    unsigned char* pattern;
    double* djs;
    unsigned long long* total_blocks;
    int* hperm;                      // attention order of the heads (see launch_head_order)
    int* lists;
    int* counts;
    int* colptr;                     // token-granular columns (vs_granularity = token), else null
    int* colidx;
    float *qbar, *kbar, *rowmax, *rowsum, *colsum, *diagsum, *atrue, *ahat;
    size_t n_qbar, n_kbar, n_rowmax, n_colsum, n_atrue, n_ahat, n_counts, n_lists, n_colptr;
    int device;
    hipStream_t stream;
    hipEvent_t ready;                // recorded on `stream` when planning is enqueued
    hipEvent_t used;                 // recorded after an attend on another stream
    struct {
        void* p = nullptr;           // every device buffer of the plan, carved from one cached block
        size_t bytes = 0;
        int dev = -1;
        hipEvent_t ev = nullptr;
    } mem;
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
fp_status check_common(fp_dtype dtype, int Hq, int Hkv, int d, int block) {
    if (dtype != FP_BF16 && dtype != FP_FP32) return fail(FP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (Hq < 0 || Hkv < 0) return fail(FP_ERR_INVALID_ARG, "negative size");
    if (d != 64 && d != 128) return fail(FP_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d);
    if (block != 64 && block != 128) return fail(FP_ERR_UNSUPPORTED, "block %d (supported: 64, 128)", block);
    if (Hkv == 0 && Hq != 0) return fail(FP_ERR_SHAPE, "Hkv = 0 with Hq = %d", Hq);
    if (Hkv > 0 && Hq % Hkv != 0) return fail(FP_ERR_SHAPE, "Hq %d not a multiple of Hkv %d", Hq, Hkv);
    return FP_OK;
}

fp_status check_length(int L, int block) {
    const long long nb = ((long long)L + block - 1) / block;
    if (nb > kMaxBlocks) return fail(FP_ERR_SHAPE, "sequence of %d tokens: %lld blocks exceed %d", L, nb, kMaxBlocks);
    return FP_OK;
}

fp_status check_shape(fp_dtype dtype, int B, int Hq, int Hkv, int N, int d, int block) {
    fp_status s = check_common(dtype, Hq, Hkv, d, block);
    if (s != FP_OK) return s;
    if (B < 0 || N < 0) return fail(FP_ERR_INVALID_ARG, "negative size");
    s = check_length(N, block);
    if (s != FP_OK) return s;
    const long long rows = (long long)B * Hq * ((N + block - 1) / block);
    if (rows > 0x7FFFFFFFLL) return fail(FP_ERR_SHAPE, "too many query-block rows");
    return FP_OK;
}

fp_status check_varlen(fp_dtype dtype, int nseq, const int* cu, int Hq, int Hkv, int d, int block) {
    fp_status s = check_common(dtype, Hq, Hkv, d, block);
    if (s != FP_OK) return s;
    if (nseq < 0) return fail(FP_ERR_INVALID_ARG, "nseq %d < 0", nseq);
    if (nseq == 0) return FP_OK;
    if (!cu) return fail(FP_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (cu[0] != 0) return fail(FP_ERR_INVALID_ARG, "cu_seqlens[0] = %d, must be 0", cu[0]);
    long long rows = 0;
    for (int b = 0; b < nseq; ++b) {
        if (cu[b + 1] < cu[b]) return fail(FP_ERR_INVALID_ARG, "cu_seqlens decreases at %d", b + 1);
        s = check_length(cu[b + 1] - cu[b], block);
        if (s != FP_OK) return s;
        rows += (long long)Hq * ((cu[b + 1] - cu[b] + block - 1) / block);
    }
    if (rows > 0x7FFFFFFFLL) return fail(FP_ERR_SHAPE, "too many query-block rows");
    return FP_OK;
}

// Segments of a [B, H, N, d] problem (one) or of a packed problem (one per
// non-empty sequence), with the token strides of Q/O and K/V.
void build_segments(int layout, int B, int N, const int* cu, int Hq, int Hkv, int d, int bs,
                    std::vector<SegHost>& segs, TokStride& qs, TokStride& ks) {
    segs.clear();
    const long long D = d;
    if (layout == FP_LAYOUT_BHND) {
        qs = TokStride{D, (long long)N * D, (long long)Hq * N * D};
        ks = TokStride{D, (long long)N * D, (long long)Hkv * N * D};
        if (B > 0 && Hq > 0 && N > 0) {
            const int nb = (N + bs - 1) / bs;
            segs.push_back(SegHost{0, B, N, nb, (long long)nb * (nb + 1) / 2, 0, 0});
        }
        return;
    }
    qs = TokStride{(long long)Hq * D, D, 0};
    ks = TokStride{(long long)Hkv * D, D, 0};
    if (Hq == 0) return;
    for (int b = 0; b < B; ++b) {
        const int L = cu[b + 1] - cu[b];
        if (L == 0) continue;
        const int nb = (L + bs - 1) / bs;
        segs.push_back(SegHost{b, 1, L, nb, (long long)nb * (nb + 1) / 2, (long long)cu[b] * Hq * D,
                               (long long)cu[b] * Hkv * D});
    }
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

// Adds up the recorded kernel times and releases every event, also when one
// of them cannot be read (that launch is then left out; the first failure is
// returned).
fp_status drain_profile_events() {
    fp_status s = FP_OK;
    for (auto& e : g_prof_events) {
        float ms = 0.f;
        hipError_t he = hipEventSynchronize(e.b);
        if (he == hipSuccess) he = hipEventElapsedTime(&ms, e.a, e.b);
        if (he == hipSuccess) {
            g_prof_ms[e.dense ? 1 : 0] += ms;
            g_prof_n[e.dense ? 1 : 0] += 1;
        } else if (s == FP_OK) {
            s = hip_fail(he, "profiling events");
        }
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    g_prof_events.clear();
    return s;
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

// ---------------------------------------------------------------------------
// Device memory cache.  On this runtime an allocation from the stream-ordered
// pool that reuses memory freed earlier, while the stream has not yet reached
// that free, makes the host wait until it has: a 256 MiB hipMallocAsync after
// a hipFreeAsync of the same size waited out the 6 ms of work queued before
// the free, and returned in 0.08 ms without the free.  A plan or an attend
// that allocated and freed per call therefore held its caller until the GPU
// drained, one call behind.  The library instead keeps the blocks it
// releases: a released block carries an event recorded on the stream of its
// last use, and a later call on any stream takes it after making its own
// stream wait on that event (a stream dependency, no host wait).  The cache
// holds at most kCacheLimit bytes (oldest blocks freed first, after their
// last use is complete) and fp_workspace_trim returns it to the runtime.
// ---------------------------------------------------------------------------
struct WsBlock {
    void* p = nullptr;
    size_t bytes = 0;
    int dev = -1;
    hipEvent_t ev = nullptr;    // recorded when the block was last released
};
std::mutex g_ws_mu;
std::deque<WsBlock> g_ws;       // released blocks, oldest first
size_t g_ws_bytes = 0;
constexpr size_t kCacheLimit = 16ull << 30;

// A cached block serves a request it exceeds by at most half (2 MiB for
// requests up to 1 MiB), so large blocks are not spent on small requests.
bool ws_fits(size_t have, size_t need) {
    return have >= need && (need <= (1u << 20) ? have <= (2u << 20) : have - need <= need / 2);
}

// Frees a block whose last use may still be queued: waits for that use on
// the host first, so the free (on the null stream) has nothing to wait for.
void ws_free_now(WsBlock& b) {
    if (b.ev) {
        (void)hipEventSynchronize(b.ev);
        (void)hipEventDestroy(b.ev);
    }
    (void)hipFreeAsync(b.p, nullptr);
    b = WsBlock{};
}

// A block of at least `bytes` on device `dev` for work enqueued on `st`.
hipError_t ws_get(size_t bytes, int dev, hipStream_t st, WsBlock* out) {
    bytes = bytes ? (bytes + 255) / 256 * 256 : 256;
    WsBlock b;
    {
        std::lock_guard<std::mutex> g(g_ws_mu);
        auto best = g_ws.end();
        for (auto it = g_ws.begin(); it != g_ws.end(); ++it)
            if (it->dev == dev && ws_fits(it->bytes, bytes) && (best == g_ws.end() || it->bytes < best->bytes))
                best = it;
        if (best != g_ws.end()) {
            b = *best;
            g_ws_bytes -= b.bytes;
            g_ws.erase(best);
        }
    }
    if (b.p) {
        const hipError_t e = hipStreamWaitEvent(st, b.ev, 0);
        if (e != hipSuccess) {
            ws_free_now(b);
            return e;
        }
        *out = b;
        return hipSuccess;
    }
    b.bytes = bytes;
    b.dev = dev;
    const hipError_t e = hipMallocAsync(&b.p, bytes, st);
    if (e != hipSuccess) return e;
    *out = b;
    return hipSuccess;
}

// Gives a block back once the work using it is enqueued on `st`.  When its
// last use cannot be marked, it is freed in the order of `st` instead (and
// the error returned); either way `b` is empty afterwards.
hipError_t ws_put(WsBlock& b, hipStream_t st) {
    if (!b.p) return hipSuccess;
    hipError_t e = hipSuccess;
    if (!b.ev) e = hipEventCreateWithFlags(&b.ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(b.ev, st);
    if (e != hipSuccess) {
        (void)hipFreeAsync(b.p, st);
        if (b.ev) (void)hipEventDestroy(b.ev);
        b = WsBlock{};
        return e;
    }
    std::vector<WsBlock> evict;
    {
        std::lock_guard<std::mutex> g(g_ws_mu);
        g_ws.push_back(b);
        g_ws_bytes += b.bytes;
        for (auto it = g_ws.begin(); g_ws_bytes > kCacheLimit && it != g_ws.end();) {
            if (it->dev == b.dev && it->p != b.p) {
                g_ws_bytes -= it->bytes;
                evict.push_back(*it);
                it = g_ws.erase(it);
            } else {
                ++it;
            }
        }
    }
    for (WsBlock& x : evict) ws_free_now(x);
    b = WsBlock{};
    return hipSuccess;
}

// Offsets of several buffers carved from one block (256-byte aligned).
struct Layout {
    std::vector<std::pair<void**, size_t>> items;
    size_t total = 0;
    template <typename T>
    void add(T** ptr, size_t count) {
        const size_t bytes = count * sizeof(T) > 0 ? count * sizeof(T) : 16;
        items.push_back({reinterpret_cast<void**>(ptr), total});
        total += (bytes + 255) / 256 * 256;
    }
    void assign(void* base) const {
        for (const auto& it : items) *it.first = static_cast<unsigned char*>(base) + it.second;
    }
};

void free_plan(fp_plan* p) {
    WsBlock b{p->mem.p, p->mem.bytes, p->mem.dev, p->mem.ev};
    (void)ws_put(b, p->stream);
    if (p->ready) (void)hipEventDestroy(p->ready);
    if (p->used) (void)hipEventDestroy(p->used);
    delete p;
}

// Sequences of a packed batch are planned concurrently on up to kPlanLanes
// streams (segment i on lane i % lanes), each lane with its own transient
// workspace and selection state; the caller's stream forks to the lanes and
// joins them with events.  The lane streams are created once per device and
// kept; they have the default priority.
constexpr int kPlanLanes = 4;

hipError_t lane_streams(hipStream_t* out) {
    static std::mutex mu;
    static std::vector<std::vector<hipStream_t>> pool;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)pool.size() <= dev) pool.resize(dev + 1);
    while ((int)pool[dev].size() < kPlanLanes) {
        hipStream_t s;
        e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e != hipSuccess) return e;
        pool[dev].push_back(s);
    }
    for (int i = 0; i < kPlanLanes; ++i) out[i] = pool[dev][i];
    return hipSuccess;
}

// Whether the attention kernel takes two query blocks per workgroup: bf16 at
// block 64, and bf16 dense causal rows at any block.
bool attention_pairs(int bs, fp_dtype dtype, bool dense) { return dtype == FP_BF16 && (bs == 64 || dense); }

// The attention segment table of a problem and the V^T workspace size.
void attention_table(const std::vector<SegHost>& segs, int Hq, int Hkv, int d, int bs, bool pair,
                     std::vector<AttnSeg>& t, long long& items, size_t& vt_elems, size_t& g_elems) {
    t.clear();
    items = 0;
    long long vt = 0, loff = 0, coff = 0, goff = 0, cpoff = 0, cioff = 0;
    for (const SegHost& g : segs) {
        AttnSeg a{};
        a.item0 = items;
        a.qoff = g.qoff;
        a.koff = g.koff;
        a.vtoff = vt;
        a.loff = loff;
        a.coff = coff;
        a.goff = goff;
        a.cpoff = cpoff;
        a.cioff = cioff;
        a.hoff = (long long)g.b0 * Hq;
        a.nseq = g.nseq;
        a.L = g.L;
        a.nb = g.nb;
        a.NT = g.nb * bs;
        a.npi = pair ? (g.nb + 1) / 2 : g.nb;
        t.push_back(a);
        const long long nbh = (long long)g.nseq * Hq;
        items += nbh * a.npi;
        vt += (long long)g.nseq * Hkv * d * a.NT;
        loff += nbh * g.tri;
        coff += nbh * g.nb;
        goff += nbh * d * a.NT;
        cpoff += nbh * (g.nb + 1);
        cioff += nbh * g.L;
    }
    vt_elems = (size_t)vt;
    g_elems = (size_t)goff;
}

// Device workspace of one attention call: V^T and, for token-granular
// plans, the gathered K rows and V^T columns.
struct AttendWork {
    void *vt = nullptr, *kg = nullptr, *vgt = nullptr;
    AttnSeg* dtab = nullptr;     // segment table allocated by the call (dense calls)
};

// Attention over the segments of a validated problem; `plan` is null for the
// dense baseline.  With `scratch` non-null the call allocates nothing: V^T
// and the gathered tiles are carved from those `scratch_bytes` bytes (the
// segment table is the plan's or must fit there too), no events are created
// and the profiling hooks are skipped.
fp_status attend_common(const void* q, const void* k, const void* v, void* o, fp_dtype dtype, int Hq, int Hkv,
                        int d, int block, const std::vector<SegHost>& segs, const TokStride& qs,
                        const TokStride& ks, const fp_plan* plan, hipStream_t st, void* scratch = nullptr,
                        size_t scratch_bytes = 0) {
    const size_t esz = dtype == FP_BF16 ? 2 : 4;
    std::vector<AttnSeg> table;
    long long items = 0;
    size_t vt_elems = 0, g_elems = 0;
    const bool gather = plan && plan->colptr;
    const bool pair = attention_pairs(block, dtype, plan == nullptr);
    attention_table(segs, Hq, Hkv, d, block, pair, table, items, vt_elems, g_elems);
    if (items == 0) return FP_OK;
    AttendWork w;
    WsBlock wblk;
    AttnSeg* dtab = plan ? plan->aseg : nullptr;
    hipError_t e = hipSuccess;
    if (scratch) {
        auto up = [](size_t x) { return (x + 255) / 256 * 256; };
        const size_t vt_b = up(vt_elems * esz), g_b = gather ? up(g_elems * esz) : 0;
        const size_t tab_b = dtab ? 0 : up(table.size() * sizeof(AttnSeg));
        const size_t need = vt_b + 2 * g_b + tab_b;
        if (need > scratch_bytes)
            return fail(FP_ERR_SHAPE, "attention needs %zu bytes of workspace; the allocation-free call has %zu",
                        need, scratch_bytes);
        unsigned char* base = (unsigned char*)scratch;
        w.vt = base;
        if (gather) {
            w.kg = base + vt_b;
            w.vgt = base + vt_b + g_b;
        }
        if (!dtab) dtab = (AttnSeg*)(base + vt_b + 2 * g_b);
    } else {
        int dev = 0;
        FP_HIP(hipGetDevice(&dev), "hipGetDevice");
        set_pool_threshold(dev);
        Layout wl;
        wl.add(reinterpret_cast<unsigned char**>(&w.vt), vt_elems * esz);
        if (gather) {
            wl.add(reinterpret_cast<unsigned char**>(&w.kg), g_elems * esz);
            wl.add(reinterpret_cast<unsigned char**>(&w.vgt), g_elems * esz);
        }
        if (!dtab) wl.add(&w.dtab, table.size());
        e = ws_get(wl.total, dev, st, &wblk);
        if (e == hipSuccess) {
            wl.assign(wblk.p);
            if (!dtab) dtab = w.dtab;
        }
    }
    // a plan made on another stream: wait for its kernels
    const bool cross = plan && plan->ready && st != plan->stream;
    if (e == hipSuccess && cross) e = hipStreamWaitEvent(st, plan->ready, 0);
    if (e == hipSuccess && dtab != (plan ? plan->aseg : nullptr))
        e = launch_upload(dtab, table.data(), table.size() * sizeof(AttnSeg), st);
    for (size_t i = 0; gather && i < segs.size() && e == hipSuccess; ++i)
        e = launch_gather_cols((const unsigned char*)k + (size_t)segs[i].koff * esz,
                               (const unsigned char*)v + (size_t)segs[i].koff * esz, ks, dtype == FP_BF16, d,
                               segs[i].nseq, Hq, Hkv, segs[i].L, segs[i].nb, table[i].NT,
                               plan->colptr + table[i].cpoff, plan->colidx + table[i].cioff,
                               (unsigned char*)w.kg + (size_t)table[i].goff * esz,
                               (unsigned char*)w.vgt + (size_t)table[i].goff * esz, st);
    for (size_t i = 0; i < segs.size() && e == hipSuccess; ++i)
        e = launch_transpose_v((const unsigned char*)v + (size_t)segs[i].koff * esz, ks,
                               (unsigned char*)w.vt + (size_t)table[i].vtoff * esz, dtype == FP_BF16, d,
                               segs[i].nseq, Hkv, segs[i].L, table[i].NT, st);
    AttnArgs a{};
    a.d = d;
    a.q = q;
    a.k = k;
    a.vt = w.vt;
    a.o = o;
    a.dtype_bf16 = dtype == FP_BF16;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.BS = block;
    a.pair = pair;
    a.qs = qs;
    a.ks = ks;
    a.segs = dtab;
    a.nseg = (int)table.size();
    a.items = items;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    if (plan) {
        a.lists = plan->lists;
        a.counts = plan->counts;
        a.hperm = plan->hperm;
    }
    if (gather) {
        a.colptr = plan->colptr;
        a.colidx = plan->colidx;
        a.kg = w.kg;
        a.vgt = w.vgt;
    }
    bool prof = false;
    if (!scratch) {
        std::lock_guard<std::mutex> g(g_prof_mu);
        prof = g_prof_on;
    }
    EvPair ev{};
    if (e == hipSuccess && prof) {
        ev.dense = plan == nullptr;
        e = hipEventCreate(&ev.a);
        if (e == hipSuccess) e = hipEventCreate(&ev.b);
        if (e == hipSuccess) e = hipEventRecord(ev.a, st);
    }
    if (e == hipSuccess) e = launch_attention(a, st);
    if (e == hipSuccess && prof) e = hipEventRecord(ev.b, st);
    if (e == hipSuccess && prof) {
        std::lock_guard<std::mutex> g(g_prof_mu);
        g_prof_events.push_back(ev);
    } else {
        if (ev.a) (void)hipEventDestroy(ev.a);
        if (ev.b) (void)hipEventDestroy(ev.b);
    }
    // a plan made on another stream: its buffers are released on its own
    // stream, so that stream waits for this call's kernels
    if (e == hipSuccess && cross) e = hipEventRecord(plan->used, st);
    if (e == hipSuccess && cross) e = hipStreamWaitEvent(plan->stream, plan->used, 0);
    if (!scratch) {
        const hipError_t re = ws_put(wblk, st);
        if (e == hipSuccess) e = re;
    }
    if (e != hipSuccess) return hip_fail(e, "attention");
    return FP_OK;
}

// FP_LOG=1: one line per plan and one per head on stderr (pattern, divergence,
// selected blocks and their share of the causal blocks).  Synchronizes the
// plan's stream; a plan that cannot be read is reported as such.
void log_plan(const fp_plan* p) {
    const char* env = std::getenv("FP_LOG");
    if (!env || std::strcmp(env, "1") != 0) return;
    std::fprintf(stderr, "[fp_prefill] plan: %d sequence(s), Hq %d, Hkv %d, longest %d tokens, d %d, block %d, gamma %g, "
                 "tau %g, min_budget %d, max_budget %d, %s, %s\n", p->B, p->Hq, p->Hkv, p->N, p->d, p->bs,
                 (double)p->gamma, (double)p->tau, p->min_budget, p->max_budget,
                 p->qa_selection == FP_QA_QUERYWISE ? "query-wise" : "flattened",
                 p->vs_granularity == FP_VS_TOKEN ? "token columns" : "block columns");
    if (p->segs.empty()) return;
    const size_t BH = (size_t)p->B * p->Hq;
    std::vector<unsigned char> pat(BH);
    std::vector<double> djs(BH);
    std::vector<unsigned long long> tot(BH);
    hipError_t e = hipStreamSynchronize(p->stream);
    if (e == hipSuccess) e = hipMemcpy(pat.data(), p->pattern, BH, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(djs.data(), p->djs, BH * sizeof(double), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(tot.data(), p->total_blocks, BH * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
        std::fprintf(stderr, "[fp_prefill] plan could not be read: %s\n", hipGetErrorString(e));
        return;
    }
    for (size_t bh = 0; bh < BH; ++bh) {
        const int b = (int)(bh / p->Hq), h = (int)(bh % p->Hq);
        const long long nb = ((long long)p->seqlens[(size_t)b] + p->bs - 1) / p->bs;
        const long long tri = nb * (nb + 1) / 2;
        std::fprintf(stderr, "[fp_prefill]   seq %d head %d: %s D %.6f blocks %llu / %lld (%.4f)\n", b, h,
                     pat[bh] == kPatternQueryAware ? "query-aware   " : "vertical-slash", djs[bh], tot[bh], tri,
                     tri ? (double)tot[bh] / (double)tri : 0.0);
    }
}

// Plan for every segment of a validated problem.
fp_status make_plan(const void* q, const void* k, fp_dtype dtype, int layout, int B, int N, const int* cu, int Hq,
                    int Hkv, int d, int block, float gamma, float tau, int min_budget,
                    const fp_plan_options* options, void* stream, fp_plan** out) {
    const int max_budget = options ? options->max_budget : 0;
    const int qa_selection = options ? options->qa_selection : FP_QA_FLATTENED;
    const int vs_granularity = options ? options->vs_granularity : FP_VS_BLOCK;
    if (!(gamma > 0.0f && gamma <= 1.0f)) return fail(FP_ERR_INVALID_ARG, "gamma %g outside (0, 1]", (double)gamma);
    if (!(tau >= 0.0f) || std::isinf(tau)) return fail(FP_ERR_INVALID_ARG, "tau %g must be finite and >= 0", (double)tau);
    if (min_budget < 0) return fail(FP_ERR_INVALID_ARG, "min_budget %d < 0", min_budget);
    if (max_budget < 0) return fail(FP_ERR_INVALID_ARG, "max_budget %d < 0", max_budget);
    if (qa_selection != FP_QA_FLATTENED && qa_selection != FP_QA_QUERYWISE)
        return fail(FP_ERR_INVALID_ARG, "qa_selection %d is not FP_QA_FLATTENED or FP_QA_QUERYWISE", qa_selection);
    if (vs_granularity != FP_VS_BLOCK && vs_granularity != FP_VS_TOKEN)
        return fail(FP_ERR_INVALID_ARG, "vs_granularity %d is not FP_VS_BLOCK or FP_VS_TOKEN", vs_granularity);
    {
        const long long floor_b = std::max(1LL, ((long long)min_budget + block - 1) / block);
        const long long cap_b = ((long long)max_budget + block - 1) / block;
        if (max_budget > 0 && cap_b < floor_b)
            return fail(FP_ERR_INVALID_ARG, "max_budget %d allows %lld blocks per row, min_budget needs %lld",
                        max_budget, cap_b, floor_b);
    }
    std::vector<SegHost> segs;
    TokStride qs, ks;
    build_segments(layout, B, N, cu, Hq, Hkv, d, block, segs, qs, ks);
    if (!segs.empty() && (!q || !k)) return fail(FP_ERR_INVALID_ARG, "q or k is NULL");

    fp_plan* p = new (std::nothrow) fp_plan();
    if (!p) return fail(FP_ERR_OOM, "host allocation failed");
    p->B = B; p->Hq = Hq; p->Hkv = Hkv; p->d = d; p->bs = block;
    p->dtype = dtype; p->gamma = gamma; p->tau = tau; p->min_budget = min_budget;
    p->max_budget = max_budget;
    p->qa_selection = qa_selection;
    p->vs_granularity = vs_granularity;
    p->layout = layout;
    p->stream = (hipStream_t)stream;
    p->qs = qs;
    p->ks = ks;
    p->segs = segs;
    p->seqlens.resize((size_t)B);
    for (int b = 0; b < B; ++b) p->seqlens[(size_t)b] = layout == FP_LAYOUT_BHND ? N : cu[b + 1] - cu[b];
    p->N = 0;
    for (int L : p->seqlens) p->N = std::max(p->N, L);
    if (B == 0) p->N = layout == FP_LAYOUT_BHND ? N : 0;
    p->nb = (p->N + block - 1) / block;
    p->tokens = layout == FP_LAYOUT_BHND ? (long long)B * N : (B > 0 ? (long long)cu[B] : 0);
    p->rows = 0;
    p->dense_blocks = 0;
    long long lists_n = 0;
    size_t n_qbar = 0, n_kbar = 0, n_rowmax = 0, n_colsum = 0, n_atrue = 0, n_ahat = 0, n_cp = 0;
    int max_bh = 0;
    const int lanes = (int)std::min<size_t>(segs.size(), kPlanLanes);
    size_t s2_max[kPlanLanes] = {}, pmax_max[kPlanLanes] = {}, rz_max[kPlanLanes] = {}, qt_max[kPlanLanes] = {};
    for (size_t si = 0; si < segs.size(); ++si) {
        const SegHost& g = segs[si];
        const int ln = (int)(si % kPlanLanes);
        const long long nbh = (long long)g.nseq * Hq;
        const int NS = (g.L + 255) / 256 * 256;
        p->rows += nbh * g.nb;
        p->dense_blocks += nbh * g.tri;
        lists_n += nbh * g.tri;
        n_qbar += (size_t)nbh * g.nb * d;
        n_kbar += (size_t)g.nseq * Hkv * g.nb * d;
        n_rowmax += (size_t)nbh * block;
        n_colsum += (size_t)nbh * g.L;
        n_atrue += (size_t)nbh * g.nb;
        n_ahat += (size_t)nbh * g.tri;
        n_cp += (size_t)nbh * (g.nb + 1);
        max_bh = std::max(max_bh, (int)nbh);
        s2_max[ln] = std::max(s2_max[ln], (size_t)nbh * block * NS);
        pmax_max[ln] = std::max(pmax_max[ln], (size_t)nbh * (NS / 256) * block);
        rz_max[ln] = std::max(rz_max[ln], (size_t)nbh * block);
        qt_max[ln] = std::max(qt_max[ln], (size_t)nbh * d * block);
    }
    p->n_qbar = n_qbar; p->n_kbar = n_kbar; p->n_rowmax = n_rowmax; p->n_colsum = n_colsum;
    p->n_atrue = n_atrue; p->n_ahat = n_ahat; p->n_counts = (size_t)p->rows; p->n_lists = (size_t)lists_n;
    const bool token = vs_granularity == FP_VS_TOKEN;
    p->n_colptr = token ? n_cp : 0;
    if (segs.empty()) {
        p->device = -1;
        log_plan(p);
        *out = p;
        return FP_OK;
    }
    hipError_t he = hipGetDevice(&p->device);
    if (he != hipSuccess) {
        delete p;
        return hip_fail(he, "hipGetDevice");
    }
    set_pool_threshold(p->device);
    const double Gd = std::nearbyint((double)gamma * (double)(1 << kGammaShift));
    const unsigned long long G = (unsigned long long)Gd;
    const size_t BHall = (size_t)B * Hq;
    const bool cap = max_budget > 0;

    // every device buffer of the plan, carved from one block of the cache
    Layout lay;
#define PALLOC(ptr, n) lay.add(&(ptr), (n))
    unsigned char *colblk, *diagA, *diagB, *diagT;
    float *colmass = nullptr, *diagmass = nullptr;
    int* colcount = nullptr;
    p->colptr = nullptr;
    p->colidx = nullptr;
    SelState *sel, *selk;
    unsigned long long* hist;
    AttnSeg* aseg;
    PALLOC(p->pattern, (BHall + 3) / 4 * 4);
    PALLOC(p->djs, BHall);
    PALLOC(p->total_blocks, BHall);
    PALLOC(p->hperm, BHall);
    PALLOC(p->qbar, n_qbar);
    PALLOC(p->kbar, n_kbar);
    PALLOC(p->rowmax, n_rowmax);
    PALLOC(p->rowsum, n_rowmax);
    PALLOC(p->colsum, n_colsum);
    PALLOC(p->diagsum, n_colsum);
    PALLOC(p->atrue, n_atrue);
    PALLOC(p->ahat, n_ahat);
    PALLOC(p->lists, (size_t)lists_n);
    PALLOC(p->counts, (size_t)p->rows);
    PALLOC(colblk, (size_t)p->rows);
    PALLOC(diagA, (size_t)p->rows);
    PALLOC(diagB, (size_t)p->rows);
    PALLOC(diagT, (size_t)p->rows);
    if (cap) {
        PALLOC(colmass, (size_t)p->rows);
        PALLOC(diagmass, (size_t)p->rows);
    }
    if (token) {
        PALLOC(colcount, (size_t)p->rows);
        PALLOC(p->colptr, n_cp);
        PALLOC(p->colidx, n_colsum);
    }
    PALLOC(sel, (size_t)2 * max_bh * lanes);
    PALLOC(selk, (size_t)kSelMaxPasses * 2 * max_bh * lanes);
    PALLOC(hist, (size_t)kSelHistBufs * 2 * max_bh * kRadixBins * lanes);
    PALLOC(aseg, segs.size());
#undef PALLOC
    {
        WsBlock blk;
        const hipError_t ae = ws_get(lay.total, p->device, p->stream, &blk);
        if (ae != hipSuccess) {
            free_plan(p);
            return hip_fail(ae, "device memory for the plan");
        }
        p->mem.p = blk.p;
        p->mem.bytes = blk.bytes;
        p->mem.dev = blk.dev;
        p->mem.ev = blk.ev;
        lay.assign(blk.p);
    }
    p->aseg = aseg;
    long long items = 0;
    size_t vt_elems = 0, g_elems = 0;
    attention_table(segs, Hq, Hkv, d, block, attention_pairs(block, dtype, false), p->aseg_host, items, vt_elems,
                    g_elems);
    hipStream_t st = p->stream;
    // heads of empty sequences keep pattern 0, divergence 0 and no blocks
    he = launch_zero3_u32((unsigned int*)p->pattern, (long long)(BHall + 3) / 4, (unsigned int*)p->djs,
                          2LL * (long long)BHall, (unsigned int*)p->total_blocks, 2LL * (long long)BHall, st);

    // per-segment views
    size_t o_qbar = 0, o_kbar = 0, o_rowmax = 0, o_colsum = 0, o_atrue = 0, o_ahat = 0, o_rows = 0, o_cp = 0;
    p->dev.resize(segs.size());
    for (size_t i = 0; i < segs.size(); ++i) {
        const SegHost& g = segs[i];
        const int nbh = g.nseq * Hq;
        PlanDev& P = p->dev[i];
        memset(&P, 0, sizeof P);
        P.BH = nbh; P.BS = block; P.L = g.L; P.NS = (g.L + 255) / 256 * 256; P.nb = g.nb;
        P.tail = g.L - (g.nb - 1) * block;
        P.tri = g.tri;
        P.mode_all = G >= (1ull << kGammaShift);
        P.floor_blocks = (int)std::min<long long>(kMaxBlocks, std::max(1LL, ((long long)min_budget + block - 1) / block));
        P.cap_blocks = (int)std::min<long long>(kMaxBlocks, ((long long)max_budget + block - 1) / block);
        P.qa_querywise = qa_selection == FP_QA_QUERYWISE;
        P.vs_token = token;
        P.G = G;
        P.pattern = p->pattern + (size_t)g.b0 * Hq;
        P.djs = p->djs + (size_t)g.b0 * Hq;
        P.total_blocks = p->total_blocks + (size_t)g.b0 * Hq;
        P.qbar = p->qbar + o_qbar;
        P.kbar = p->kbar + o_kbar;
        P.rowmax = p->rowmax + o_rowmax;
        P.rowsum = p->rowsum + o_rowmax;
        P.colsum = p->colsum + o_colsum;
        P.diagsum = p->diagsum + o_colsum;
        P.atrue = p->atrue + o_atrue;
        P.ahat = p->ahat + o_ahat;
        P.lists = p->lists + o_ahat;
        P.counts = p->counts + o_rows;
        P.colblk = colblk + o_rows;
        P.diagA = diagA + o_rows;
        P.diagB = diagB + o_rows;
        P.diagT = diagT + o_rows;
        if (cap) {
            P.colmass = colmass + o_rows;
            P.diagmass = diagmass + o_rows;
        }
        if (token) {
            P.colcount = colcount + o_rows;
            P.colptr = p->colptr + o_cp;
            P.colidx = p->colidx + o_colsum;
        }
        P.sel = sel + (size_t)2 * max_bh * (i % kPlanLanes);
        P.selk = selk + (size_t)kSelMaxPasses * 2 * max_bh * (i % kPlanLanes);
        P.hist = hist + (size_t)kSelHistBufs * 2 * max_bh * kRadixBins * (i % kPlanLanes);
        o_qbar += (size_t)nbh * g.nb * d;
        o_kbar += (size_t)g.nseq * Hkv * g.nb * d;
        o_rowmax += (size_t)nbh * block;
        o_colsum += (size_t)nbh * g.L;
        o_atrue += (size_t)nbh * g.nb;
        o_ahat += (size_t)nbh * g.tri;
        o_rows += (size_t)nbh * g.nb;
        o_cp += (size_t)nbh * (g.nb + 1);
    }

    // transient score workspace per lane, reused by the lane's segments in its stream order
    size_t o_s2[kPlanLanes + 1] = {}, o_pm[kPlanLanes + 1] = {}, o_rz[kPlanLanes + 1] = {}, o_qt[kPlanLanes + 1] = {};
    for (int j = 0; j < lanes; ++j) {
        o_s2[j + 1] = o_s2[j] + s2_max[j];
        o_pm[j + 1] = o_pm[j] + pmax_max[j];
        o_rz[j + 1] = o_rz[j] + rz_max[j];
        o_qt[j + 1] = o_qt[j] + qt_max[j];
    }
    float *s2 = nullptr, *pmax = nullptr, *rz = nullptr, *qt = nullptr;
    WsBlock tmp;
    {
        Layout tl;
        tl.add(&s2, o_s2[lanes]);
        tl.add(&pmax, o_pm[lanes]);
        tl.add(&rz, o_rz[lanes]);
        tl.add(&qt, o_qt[lanes]);
        if (he == hipSuccess) he = ws_get(tl.total, p->device, st, &tmp);
        if (he == hipSuccess) tl.assign(tmp.p);
    }
    hipStream_t ls[kPlanLanes];
    hipEvent_t ev[kPlanLanes + 1] = {};
    hipStream_t pool_streams[kPlanLanes];
    for (int j = 0; j < kPlanLanes; ++j) ls[j] = st;
    if (he == hipSuccess) he = lane_streams(pool_streams);
    // one segment: a lane stream carries its pooling kernels
    hipStream_t aux = lanes == 1 && he == hipSuccess ? pool_streams[0] : nullptr;
    if (lanes > 1 && he == hipSuccess) {
        for (int j = 0; j < kPlanLanes; ++j) ls[j] = pool_streams[j];
        for (int j = 0; j <= lanes && he == hipSuccess; ++j) he = hipEventCreateWithFlags(&ev[j], hipEventDisableTiming);
        if (he == hipSuccess) he = hipEventRecord(ev[lanes], st);     // fork
        for (int j = 0; j < lanes && he == hipSuccess; ++j) he = hipStreamWaitEvent(ls[j], ev[lanes], 0);
    }
    const size_t esz = dtype == FP_BF16 ? 2 : 4;
    const Canon canon = make_canon(d);
    for (size_t i = 0; i < segs.size() && he == hipSuccess; ++i) {
        const int ln = (int)(i % kPlanLanes);
        PlanArgs a{};
        a.d = d;
        a.q = (const unsigned char*)q + (size_t)segs[i].qoff * esz;
        a.k = (const unsigned char*)k + (size_t)segs[i].koff * esz;
        a.qs = qs;
        a.ks = ks;
        a.dtype_bf16 = dtype == FP_BF16;
        a.nseq = segs[i].nseq;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.tau = (double)tau;
        a.G = G;
        a.canon = canon;
        a.s2 = s2 + o_s2[ln];
        a.pmax = pmax + o_pm[ln];
        a.rz = rz + o_rz[ln];
        a.qt = qt + o_qt[ln];
        a.aux = aux;
        he = launch_plan(a, p->dev[i], ls[ln]);
    }
    if (lanes > 1) {
        // join: the caller's stream waits for every lane (also after a failure,
        // so the workspace is not freed under running kernels); a lane that
        // cannot be joined that way is finished here, and the call fails
        for (int j = 0; j < lanes; ++j) {
            hipError_t je = ev[j] ? hipEventRecord(ev[j], ls[j]) : hipErrorInvalidValue;
            if (je == hipSuccess) je = hipStreamWaitEvent(st, ev[j], 0);
            if (je != hipSuccess) {
                (void)hipStreamSynchronize(ls[j]);
                if (he == hipSuccess) he = je;
            }
        }
        for (int j = 0; j <= lanes; ++j)
            if (ev[j]) (void)hipEventDestroy(ev[j]);
    }
    if (he == hipSuccess) he = launch_head_order(p->total_blocks, p->hperm, (int)BHall, Hq / Hkv, st);
    // the attention's segment table (only attend reads it), after the plan's kernels
    if (he == hipSuccess) he = launch_upload(aseg, p->aseg_host.data(), segs.size() * sizeof(AttnSeg), st);
    if (he == hipSuccess) he = hipEventCreateWithFlags(&p->ready, hipEventDisableTiming);
    if (he == hipSuccess) he = hipEventCreateWithFlags(&p->used, hipEventDisableTiming);
    if (he == hipSuccess) he = hipEventRecord(p->ready, st);
    {
        // the score workspace goes back to the cache after the plan's kernels
        const hipError_t re = ws_put(tmp, st);
        if (he == hipSuccess) he = re;
    }
    if (he != hipSuccess) {
        free_plan(p);
        return hip_fail(he, "planning");
    }
    log_plan(p);
    *out = p;
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
    *out = nullptr;
    fp_status s = check_shape(dtype, B, Hq, Hkv, N, d, block);
    if (s != FP_OK) return s;
    return make_plan(q, k, dtype, FP_LAYOUT_BHND, B, N, nullptr, Hq, Hkv, d, block, gamma, tau, min_budget, options,
                     stream, out);
}

fp_status fp_prefill_plan_varlen(const void* q, const void* k, fp_dtype dtype, int nseq, const int* cu_seqlens,
                                 int Hq, int Hkv, int d, int block, float gamma, float tau, int min_budget,
                                 const fp_plan_options* options, void* stream, fp_plan** out) {
    if (!out) return fail(FP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    fp_status s = check_varlen(dtype, nseq, cu_seqlens, Hq, Hkv, d, block);
    if (s != FP_OK) return s;
    return make_plan(q, k, dtype, FP_LAYOUT_THD, nseq, 0, cu_seqlens, Hq, Hkv, d, block, gamma, tau, min_budget,
                     options, stream, out);
}

fp_status fp_prefill_attend(const fp_plan* plan, const void* q, const void* k, const void* v, void* o, void* stream) {
    if (!plan) return fail(FP_ERR_INVALID_ARG, "plan is NULL");
    if (plan->segs.empty()) return FP_OK;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID_ARG, "q, k, v or o is NULL");
    return attend_common(q, k, v, o, plan->dtype, plan->Hq, plan->Hkv, plan->d, plan->bs, plan->segs, plan->qs,
                         plan->ks, plan, (hipStream_t)stream);
}

fp_status fp_prefill_attend_noalloc(const fp_plan* plan, const void* q, const void* k, const void* v, void* o,
                                    void* stream) {
    if (!plan) return fail(FP_ERR_INVALID_ARG, "plan is NULL");
    if (plan->segs.empty()) return FP_OK;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID_ARG, "q, k, v or o is NULL");
    void* scr = nullptr;
    size_t bytes = 0;
    const hipError_t e = noalloc_scratch(&scr, &bytes);
    if (e != hipSuccess) return hip_fail(e, "workspace address of the allocation-free call");
    return attend_common(q, k, v, o, plan->dtype, plan->Hq, plan->Hkv, plan->d, plan->bs, plan->segs, plan->qs,
                         plan->ks, plan, (hipStream_t)stream, scr, bytes);
}

fp_status fp_dense_attend(const void* q, const void* k, const void* v, void* o, fp_dtype dtype, int B, int Hq,
                          int Hkv, int N, int d, int block, void* stream) {
    fp_status s = check_shape(dtype, B, Hq, Hkv, N, d, block);
    if (s != FP_OK) return s;
    if (empty_problem(B, Hq, N)) return FP_OK;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID_ARG, "q, k, v or o is NULL");
    std::vector<SegHost> segs;
    TokStride qs, ks;
    build_segments(FP_LAYOUT_BHND, B, N, nullptr, Hq, Hkv, d, block, segs, qs, ks);
    return attend_common(q, k, v, o, dtype, Hq, Hkv, d, block, segs, qs, ks, nullptr, (hipStream_t)stream);
}

fp_status fp_dense_attend_varlen(const void* q, const void* k, const void* v, void* o, fp_dtype dtype, int nseq,
                                 const int* cu_seqlens, int Hq, int Hkv, int d, int block, void* stream) {
    fp_status s = check_varlen(dtype, nseq, cu_seqlens, Hq, Hkv, d, block);
    if (s != FP_OK) return s;
    std::vector<SegHost> segs;
    TokStride qs, ks;
    build_segments(FP_LAYOUT_THD, nseq, 0, cu_seqlens, Hq, Hkv, d, block, segs, qs, ks);
    if (segs.empty()) return FP_OK;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID_ARG, "q, k, v or o is NULL");
    return attend_common(q, k, v, o, dtype, Hq, Hkv, d, block, segs, qs, ks, nullptr, (hipStream_t)stream);
}

fp_status fp_plan_info_get(const fp_plan* plan, fp_plan_info* out) {
    if (!plan || !out) return fail(FP_ERR_INVALID_ARG, "plan or out is NULL");
    fp_plan_info I{};
    I.B = plan->B; I.Hq = plan->Hq; I.Hkv = plan->Hkv; I.N = plan->N; I.d = plan->d;
    I.block = plan->bs; I.nb = plan->nb; I.dtype = plan->dtype; I.gamma = plan->gamma; I.tau = plan->tau;
    I.min_budget = plan->min_budget;
    I.max_budget = plan->max_budget;
    I.qa_selection = plan->qa_selection;
    I.vs_granularity = plan->vs_granularity;
    I.layout = plan->layout;
    I.tokens = plan->tokens;
    I.rows = plan->rows;
    I.dense_blocks = plan->dense_blocks;
    const long long BH = (long long)plan->B * plan->Hq;
    if (!plan->segs.empty()) {
        FP_HIP(hipStreamSynchronize(plan->stream), "hipStreamSynchronize");
        std::vector<unsigned long long> per_head((size_t)BH);
        FP_HIP(hipMemcpy(per_head.data(), plan->total_blocks, per_head.size() * sizeof(unsigned long long),
                         hipMemcpyDeviceToHost), "hipMemcpy");
        long long tot = 0;
        for (unsigned long long x : per_head) tot += (long long)x;
        I.total_blocks = tot;
        std::vector<unsigned char> pat((size_t)BH);
        FP_HIP(hipMemcpy(pat.data(), plan->pattern, pat.size(), hipMemcpyDeviceToHost), "hipMemcpy");
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
    if (plan->segs.empty()) {
        if (row_ptr) row_ptr[0] = 0;
        if (pattern) memset(pattern, 0, (size_t)BH);
        if (djs) memset(djs, 0, (size_t)BH * sizeof(double));
        return FP_OK;
    }
    hipStream_t st = (hipStream_t)stream;
    FP_HIP(hipStreamSynchronize(plan->stream), "hipStreamSynchronize");
    if (pattern) FP_HIP(hipMemcpyAsync(pattern, plan->pattern, (size_t)BH, hipMemcpyDeviceToHost, st), "copy pattern");
    if (djs) FP_HIP(hipMemcpyAsync(djs, plan->djs, (size_t)BH * sizeof(double), hipMemcpyDeviceToHost, st), "copy djs");
    if (row_ptr) {
        std::vector<int> counts(plan->n_counts);
        std::vector<int> lists(plan->n_lists);
        FP_HIP(hipMemcpyAsync(counts.data(), plan->counts, counts.size() * sizeof(int), hipMemcpyDeviceToHost, st),
               "copy counts");
        FP_HIP(hipMemcpyAsync(lists.data(), plan->lists, lists.size() * sizeof(int), hipMemcpyDeviceToHost, st),
               "copy lists");
        FP_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");
        long long acc = 0, row = 0, loff = 0;
        for (const SegHost& g : plan->segs) {
            const long long nbh = (long long)g.nseq * plan->Hq;
            for (long long bh = 0; bh < nbh; ++bh)
                for (int r = 0; r < g.nb; ++r, ++row) {
                    row_ptr[row] = (int)acc;
                    const int c = counts[(size_t)row];
                    memcpy(col_idx + acc, lists.data() + loff + bh * g.tri + (long long)r * (r + 1) / 2,
                           (size_t)c * sizeof(int));
                    acc += c;
                }
            loff += nbh * g.tri;
        }
        row_ptr[row] = (int)acc;
    }
    FP_HIP(hipStreamSynchronize(st), "hipStreamSynchronize");
    return FP_OK;
}

fp_status fp_plan_copy_debug(const fp_plan* plan, int which, void* host_dst, size_t bytes) {
    if (!plan || !host_dst) return fail(FP_ERR_INVALID_ARG, "plan or destination is NULL");
    const void* src = nullptr;
    size_t need = 0;
    switch (which) {
        case FP_DBG_QBAR: src = plan->qbar; need = plan->n_qbar * 4; break;
        case FP_DBG_KBAR: src = plan->kbar; need = plan->n_kbar * 4; break;
        case FP_DBG_ROWMAX: src = plan->rowmax; need = plan->n_rowmax * 4; break;
        case FP_DBG_ROWSUM: src = plan->rowsum; need = plan->n_rowmax * 4; break;
        case FP_DBG_COLSUM: src = plan->colsum; need = plan->n_colsum * 4; break;
        case FP_DBG_DIAGSUM: src = plan->diagsum; need = plan->n_colsum * 4; break;
        case FP_DBG_ATRUE: src = plan->atrue; need = plan->n_atrue * 4; break;
        case FP_DBG_AHAT: src = plan->ahat; need = plan->n_ahat * 4; break;
        case FP_DBG_COUNTS: src = plan->counts; need = plan->n_counts * 4; break;
        case FP_DBG_COLPTR: src = plan->colptr; need = plan->n_colptr * 4; break;
        case FP_DBG_COLIDX: src = plan->colidx; need = plan->colidx ? plan->n_colsum * 4 : 0; break;
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

fp_status fp_workspace_trim(void) {
    std::deque<WsBlock> blocks;
    {
        std::lock_guard<std::mutex> g(g_ws_mu);
        blocks.swap(g_ws);
        g_ws_bytes = 0;
    }
    hipError_t first = hipSuccess;
    int cur = -1;
    (void)hipGetDevice(&cur);
    std::vector<int> devs;
    for (WsBlock& b : blocks) {
        if (b.ev) {
            const hipError_t e = hipEventSynchronize(b.ev);
            if (e != hipSuccess && first == hipSuccess) first = e;
            (void)hipEventDestroy(b.ev);
        }
        // freed on the null stream of the block's own device
        if (b.dev != cur) (void)hipSetDevice(b.dev);
        (void)hipFreeAsync(b.p, nullptr);
        if (b.dev != cur && cur >= 0) (void)hipSetDevice(cur);
        if (std::find(devs.begin(), devs.end(), b.dev) == devs.end()) devs.push_back(b.dev);
    }
    for (int dev : devs) {
        hipMemPool_t pool;
        if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) (void)hipMemPoolTrimTo(pool, 0);
    }
    if (first != hipSuccess) return hip_fail(first, "waiting for the last use of a cached block");
    return FP_OK;
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
    hipError_t e = launch_probe_exp2(x, y, n, make_canon(kMaxHeadDim), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "probe exp2");
    return FP_OK;
}

fp_status fp_probe_ln(const double* x, double* y, long long n, void* stream) {
    if (n < 0 || (n > 0 && (!x || !y))) return fail(FP_ERR_INVALID_ARG, "bad probe arguments");
    hipError_t e = launch_probe_ln(x, y, n, make_canon(kMaxHeadDim), (hipStream_t)stream);
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

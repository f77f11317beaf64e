// Host stand-in for the HIP runtime calls and kernel launchers the host
// library (fp_api.cpp) makes, so that library can be built with address and
// undefined-behaviour sanitizers and exercised on a machine without a GPU.
// Test infrastructure only.
//
// "Device" memory is zero-filled host memory; streams and events are small
// host objects; kernel launches do nothing.  Every call whose failure the
// library handles counts as one fallible call; stub_fail_call(n) makes the
// n-th fallible call from now on fail (allocations with
// hipErrorOutOfMemory, everything else with hipErrorLaunchFailure).  Release
// calls (hipFree, hipFreeAsync, hipEventDestroy) never fail, and refuse
// pointers they did not hand out.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>

#include "fp_launch.h"

namespace {
std::mutex g_mu;
// registries that live until the process ends, so objects the library keeps
// for the whole process (its lane streams) stay reachable at exit
std::set<void*>& g_mem = *new std::set<void*>;
std::set<void*>& g_events = *new std::set<void*>;
std::set<void*>& g_streams = *new std::set<void*>;
long long g_calls = 0, g_fail_at = 0, g_bad_release = 0;
bool g_paused = false;

// One fallible call: true if it is the one chosen to fail.  While paused,
// calls are neither counted nor failed.
bool fail_now() {
    if (g_paused) return false;
    ++g_calls;
    return g_fail_at > 0 && g_calls == g_fail_at;
}
}  // namespace

extern "C" {
// The n-th fallible call from now fails (n = 0: none).
void stub_fail_call(long long n) {
    std::lock_guard<std::mutex> l(g_mu);
    g_fail_at = n > 0 ? g_calls + n : 0;
}
long long stub_calls() { return g_calls; }
// Stop (1) or resume (0) counting and failing calls.
void stub_pause(int on) {
    std::lock_guard<std::mutex> l(g_mu);
    g_paused = on != 0;
}
long long stub_live_memory() { return (long long)g_mem.size(); }
long long stub_live_events() { return (long long)g_events.size(); }
long long stub_live_streams() { return (long long)g_streams.size(); }
long long stub_bad_releases() { return g_bad_release; }
}

hipError_t hipGetDevice(int* device) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorNoDevice;
    *device = 0;
    return hipSuccess;
}

const char* hipGetErrorString(hipError_t e) {
    switch (e) {
        case hipSuccess: return "no error (stub)";
        case hipErrorOutOfMemory: return "out of memory (stub)";
        case hipErrorNoDevice: return "no device (stub)";
        default: return "failure (stub)";
    }
}

hipError_t hipDeviceGetDefaultMemPool(hipMemPool_t* pool, int) {
    *pool = nullptr;
    return hipSuccess;
}

hipError_t hipMemPoolSetAttribute(hipMemPool_t, hipMemPoolAttr, void*) { return hipSuccess; }

hipError_t hipMallocAsync(void** p, size_t bytes, hipStream_t) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorOutOfMemory;
    *p = std::calloc(1, bytes ? bytes : 1);
    if (!*p) return hipErrorOutOfMemory;
    g_mem.insert(*p);
    return hipSuccess;
}

hipError_t hipFreeAsync(void* p, hipStream_t) {
    std::lock_guard<std::mutex> l(g_mu);
    if (!g_mem.erase(p)) {
        ++g_bad_release;
        return hipErrorInvalidValue;
    }
    std::free(p);
    return hipSuccess;
}

hipError_t hipFree(void* p) {
    std::lock_guard<std::mutex> l(g_mu);
    if (!p) return hipSuccess;
    if (!g_mem.erase(p)) {
        ++g_bad_release;
        return hipErrorInvalidValue;
    }
    std::free(p);
    return hipSuccess;
}

hipError_t hipMemPoolTrimTo(hipMemPool_t, size_t) { return hipSuccess; }

// One device (0): switching to it always succeeds.
hipError_t hipSetDevice(int) { return hipSuccess; }

hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorOutOfMemory;
    void* h = std::malloc(16);
    g_streams.insert(h);
    *s = (hipStream_t)h;
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) {
    std::lock_guard<std::mutex> l(g_mu);
    return fail_now() ? hipErrorLaunchFailure : hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned int) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorLaunchFailure;
    return g_events.count((void*)e) ? hipSuccess : hipErrorInvalidResourceHandle;
}

static hipError_t make_event(hipEvent_t* e) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorOutOfMemory;
    void* h = std::malloc(16);
    g_events.insert(h);
    *e = (hipEvent_t)h;
    return hipSuccess;
}

hipError_t hipEventCreate(hipEvent_t* e) { return make_event(e); }
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return make_event(e); }

hipError_t hipEventDestroy(hipEvent_t e) {
    std::lock_guard<std::mutex> l(g_mu);
    if (!g_events.erase((void*)e)) {
        ++g_bad_release;
        return hipErrorInvalidResourceHandle;
    }
    std::free((void*)e);
    return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorLaunchFailure;
    return g_events.count((void*)e) ? hipSuccess : hipErrorInvalidResourceHandle;
}

hipError_t hipEventSynchronize(hipEvent_t) {
    std::lock_guard<std::mutex> l(g_mu);
    return fail_now() ? hipErrorLaunchFailure : hipSuccess;
}

hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorLaunchFailure;
    *ms = 1.0f;
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
    {
        std::lock_guard<std::mutex> l(g_mu);
        if (fail_now()) return hipErrorLaunchFailure;
    }
    if (bytes) std::memcpy(dst, src, bytes);
    return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
    {
        std::lock_guard<std::mutex> l(g_mu);
        if (fail_now()) return hipErrorLaunchFailure;
    }
    if (bytes) std::memcpy(dst, src, bytes);
    return hipSuccess;
}

// ------------------------------------------------------------ kernel launchers
namespace fp {

static hipError_t launch() {
    std::lock_guard<std::mutex> l(g_mu);
    return fail_now() ? hipErrorLaunchFailure : hipSuccess;
}

hipError_t launch_plan(const PlanArgs&, PlanDev&, hipStream_t) { return launch(); }
hipError_t launch_fill_u32(unsigned int*, unsigned int, long long, hipStream_t) { return launch(); }
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t) {
    const hipError_t e = launch();
    if (e == hipSuccess && bytes) std::memcpy(dst, src, bytes);
    return e;
}
hipError_t launch_zero3_u32(unsigned int*, long long, unsigned int*, long long, unsigned int*, long long, hipStream_t) {
    return launch();
}
hipError_t launch_probe_exp2(const float*, float*, long long, const Canon&, hipStream_t) { return launch(); }
hipError_t launch_probe_ln(const double*, double*, long long, const Canon&, hipStream_t) { return launch(); }
hipError_t launch_probe_sqrt(const double*, double*, long long, hipStream_t) { return launch(); }
hipError_t launch_transpose_v(const void*, const TokStride&, void*, int, int, int, int, int, int, hipStream_t) {
    return launch();
}
hipError_t launch_attention(const AttnArgs&, hipStream_t) { return launch(); }
hipError_t launch_head_order(const unsigned long long*, int*, int, int, hipStream_t) { return launch(); }
hipError_t launch_gather_cols(const void*, const void*, const TokStride&, int, int, int, int, int, int, int, int,
                              const int*, const int*, void*, void*, hipStream_t) {
    return launch();
}

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    static unsigned char* buf = nullptr;
    std::lock_guard<std::mutex> l(g_mu);
    if (fail_now()) return hipErrorInvalidSymbol;
    if (!buf) buf = (unsigned char*)std::calloc(1, kNoAllocScratchBytes);
    *ptr = buf;
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

}  // namespace fp

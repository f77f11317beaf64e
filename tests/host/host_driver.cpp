// Error-path driver for the host library built against the stub runtime
// (hip_stub.cpp), under address and undefined-behaviour sanitizers, on the
// CPU.  Test infrastructure only.
//
// Every scenario runs once as is (it must succeed and leave no stub memory,
// events or streams behind once the library's memory cache is trimmed) and
// then once with each of its fallible runtime calls failing in turn: the
// entry point must return FP_ERR_OOM (allocation failures) or FP_ERR_HIP, set
// a message, hand out no plan, and again leave nothing behind.  Destroying a
// plan cannot fail; its runtime calls are failed in turn separately, and must
// leave nothing behind either.  Host leaks are LeakSanitizer's to report at
// exit.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <vector>

#include "fp_prefill.h"

extern "C" {
void stub_fail_call(long long n);
void stub_pause(int on);
long long stub_calls();
long long stub_live_memory();
long long stub_live_events();
long long stub_live_streams();
long long stub_bad_releases();
// the stub's stream creation, for calls on a stream other than the plan's
int hipStreamCreateWithFlags(void** s, unsigned int flags);
}

namespace {

int g_failures = 0;
long long g_oom = 0, g_hip = 0;

#define EXPECT(cond, ...)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);              \
            std::fprintf(stderr, "\n");                     \
            ++g_failures;                                   \
        }                                                   \
    } while (0)

struct Live {
    long long mem, ev, st;
    bool operator==(const Live& o) const { return mem == o.mem && ev == o.ev && st == o.st; }
};
Live live() { return {stub_live_memory(), stub_live_events(), stub_live_streams()}; }

// One scenario: succeeds as is, fails cleanly with each fallible call failing.
// The last `best_effort` calls may fail without failing the scenario (they
// only serve logging), but must still leave nothing behind.
void sweep(const char* name, const std::function<fp_status()>& body, long long best_effort = 0) {
    EXPECT(fp_workspace_trim() == FP_OK, "%s: trim", name);
    const Live before = live();
    const long long c0 = stub_calls();
    const fp_status s = body();
    const long long n = stub_calls() - c0;
    EXPECT(fp_workspace_trim() == FP_OK, "%s: trim", name);
    EXPECT(s == FP_OK, "%s: status %s (%s)", name, fp_status_str(s), fp_last_error());
    EXPECT(live() == before, "%s: resources left after a successful run", name);
    EXPECT(n > 0, "%s: no fallible call", name);
    for (long long k = 1; k <= n; ++k) {
        stub_fail_call(k);
        const fp_status f = body();
        stub_fail_call(0);
        (void)fp_workspace_trim();
        const bool tail = k > n - best_effort;
        EXPECT(f == FP_ERR_OOM || f == FP_ERR_HIP || (tail && f == FP_OK), "%s: call %lld of %lld failing gave %s",
               name, k, n, fp_status_str(f));
        EXPECT(f == FP_OK || std::strlen(fp_last_error()) > 0, "%s: call %lld: no message", name, k);
        const Live after = live();
        EXPECT(after == before, "%s: call %lld failing left memory %lld events %lld streams %lld (before %lld %lld %lld)",
               name, k, after.mem, after.ev, after.st, before.mem, before.ev, before.st);
        if (f != FP_OK) (f == FP_ERR_OOM ? g_oom : g_hip) += 1;
    }
    std::printf("%-28s %3lld fallible calls, each failing cleanly\n", name, n);
}

// A plan call: on failure no plan is handed out; on success the plan is
// released, outside the swept calls (the stub neither counts nor fails them).
fp_status plan_and_release(const std::function<fp_status(fp_plan**)>& make) {
    fp_plan* p = reinterpret_cast<fp_plan*>(0x1);
    const fp_status s = make(&p);
    if (s != FP_OK) {
        EXPECT(p == nullptr, "a failed plan call handed out a plan");
        return s;
    }
    stub_pause(1);
    fp_plan_destroy(p);
    stub_pause(0);
    return s;
}

}  // namespace

int main() {
    // host buffers standing in for device tensors (the stub kernels never read them)
    std::vector<unsigned char> buf(1 << 22);
    void* q = buf.data();
    void* k = buf.data() + (1 << 20);
    void* v = buf.data() + (2 << 20);
    void* o = buf.data() + (3 << 20);
    void* other = nullptr;
    EXPECT(hipStreamCreateWithFlags(&other, 0) == 0, "stream");

    const int cu[5] = {0, 300, 300, 1000, 1001};
    fp_plan_options opt{};

    // warm-up: the library keeps its lane streams for later calls
    {
        fp_plan* p = nullptr;
        EXPECT(fp_prefill_plan_varlen(q, k, FP_BF16, 4, cu, 8, 2, 128, 128, 0.95f, 0.1f, 1024, nullptr, nullptr, &p) ==
                   FP_OK, "warm-up: %s", fp_last_error());
        fp_plan_destroy(p);
    }

    sweep("plan bf16 B=2 N=1000", [&] {
        return plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 2, 8, 2, 1000, 128, 128, 0.95f, 0.1f, 1024, nullptr, p);
        });
    });
    sweep("plan d64 block 64 options", [&] {
        opt.max_budget = 512;
        opt.qa_selection = FP_QA_QUERYWISE;
        opt.vs_granularity = FP_VS_TOKEN;
        return plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan_ex(q, k, FP_FP32, 1, 4, 4, 700, 64, 64, 0.9f, 0.1f, 128, &opt, nullptr, p);
        });
    });
    sweep("plan gamma 1", [&] {
        return plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 1, 4, 1, 512, 128, 128, 1.0f, 0.1f, 0, nullptr, p);
        });
    });
    sweep("plan varlen 4 sequences", [&] {
        return plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan_varlen(q, k, FP_BF16, 4, cu, 8, 2, 128, 128, 0.95f, 0.1f, 1024, nullptr, nullptr, p);
        });
    });

    sweep("plan with FP_LOG=1", [&] {
        setenv("FP_LOG", "1", 1);
        const fp_status st = plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 1, 4, 2, 300, 64, 64, 0.95f, 0.1f, 128, nullptr, p);
        });
        unsetenv("FP_LOG");
        return st;
    }, 4);   // the log's stream synchronization and three reads

    // destroying a plan with each of its runtime calls failing (giving the
    // plan's block back to the cache): nothing is left behind
    {
        auto make = [&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 2, 8, 2, 1000, 128, 128, 0.95f, 0.1f, 1024, nullptr, p);
        };
        EXPECT(fp_workspace_trim() == FP_OK, "trim");
        const Live before = live();
        fp_plan* d = nullptr;
        EXPECT(make(&d) == FP_OK, "plan for destroy: %s", fp_last_error());
        const long long c0 = stub_calls();
        fp_plan_destroy(d);
        const long long n = stub_calls() - c0;
        EXPECT(fp_workspace_trim() == FP_OK, "trim");
        EXPECT(live() == before, "destroy: resources left");
        for (long long kk = 1; kk <= n; ++kk) {
            d = nullptr;
            EXPECT(make(&d) == FP_OK, "plan for destroy: %s", fp_last_error());
            stub_fail_call(kk);
            fp_plan_destroy(d);
            stub_fail_call(0);
            (void)fp_workspace_trim();
            const Live after = live();
            EXPECT(after == before, "destroy: call %lld failing left memory %lld events %lld", kk, after.mem,
                   after.ev);
        }
        std::printf("%-28s %3lld fallible calls, each failing cleanly\n", "plan destroy", n);
    }

    // calls on an existing plan
    fp_plan* P = nullptr;
    EXPECT(fp_prefill_plan(q, k, FP_BF16, 2, 8, 2, 1000, 128, 128, 0.95f, 0.1f, 1024, nullptr, &P) == FP_OK, "plan");
    fp_plan* PT = nullptr;
    opt.vs_granularity = FP_VS_TOKEN;
    opt.max_budget = 0;
    opt.qa_selection = FP_QA_FLATTENED;
    EXPECT(fp_prefill_plan_ex(q, k, FP_BF16, 1, 4, 2, 1100, 128, 64, 0.95f, 0.1f, 256, &opt, nullptr, &PT) == FP_OK,
           "token plan");
    fp_plan* PV = nullptr;
    EXPECT(fp_prefill_plan_varlen(q, k, FP_FP32, 4, cu, 4, 2, 64, 64, 0.95f, 0.1f, 256, nullptr, nullptr, &PV) ==
               FP_OK, "varlen plan");

    sweep("attend", [&] { return fp_prefill_attend(P, q, k, v, o, nullptr); });
    sweep("attend on another stream", [&] { return fp_prefill_attend(P, q, k, v, o, other); });
    sweep("attend token columns", [&] { return fp_prefill_attend(PT, q, k, v, o, nullptr); });
    sweep("attend packed batch", [&] { return fp_prefill_attend(PV, q, k, v, o, nullptr); });
    sweep("attend allocation-free", [&] { return fp_prefill_attend_noalloc(PT, q, k, v, o, other); });
    // the second call takes the first one's block from the cache (its stream
    // waits on the block's release event); here on another stream
    sweep("attend twice (cache reuse)", [&] {
        const fp_status s = fp_prefill_attend(P, q, k, v, o, nullptr);
        return s != FP_OK ? s : fp_prefill_attend(P, q, k, v, o, other);
    });
    sweep("plan twice (cache reuse)", [&] {
        const fp_status s = plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 2, 8, 2, 1000, 128, 128, 0.95f, 0.1f, 1024, nullptr, p);
        });
        if (s != FP_OK) return s;
        return plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 2, 8, 2, 1000, 128, 128, 0.95f, 0.1f, 1024, nullptr, p);
        });
    });
    sweep("attend profiled", [&] {
        fp_profile_enable(1);
        fp_status s = fp_prefill_attend(P, q, k, v, o, nullptr);
        double sms = 0, dms = 0;
        long long sn = 0, dn = 0;
        const fp_status r = fp_profile_read(&sms, &sn, &dms, &dn, 1);
        fp_profile_enable(0);
        if (s == FP_OK) s = r;
        return s;
    });
    sweep("dense attend", [&] {
        return fp_dense_attend(q, k, v, o, FP_BF16, 2, 8, 2, 1000, 128, 128, nullptr);
    });
    sweep("dense attend varlen", [&] {
        return fp_dense_attend_varlen(q, k, v, o, FP_FP32, 4, cu, 4, 2, 64, 64, nullptr);
    });
    sweep("plan info", [&] {
        fp_plan_info info{};
        return fp_plan_info_get(P, &info);
    });
    sweep("plan copy out", [&] {
        std::vector<unsigned char> pat(16);
        std::vector<double> djs(16);
        std::vector<int> rp(2 * 8 * 8 + 1), ci(2 * 8 * 36 + 1);
        return fp_plan_copy_out(P, pat.data(), djs.data(), rp.data(), ci.data(), nullptr);
    });
    sweep("plan copy debug", [&] {
        std::vector<float> qbar(2 * 8 * 8 * 128);
        return fp_plan_copy_debug(P, FP_DBG_QBAR, qbar.data(), qbar.size() * sizeof(float));
    });

    // argument errors are caught before any runtime call and leave nothing behind
    {
        const Live before = live();
        auto no_calls = [&](const char* what, fp_status want, const std::function<fp_status()>& call) {
            const long long c0 = stub_calls();
            const fp_status s = call();
            EXPECT(s == want, "%s: %s, expected %s", what, fp_status_str(s), fp_status_str(want));
            EXPECT(stub_calls() == c0, "%s: %lld runtime call(s)", what, stub_calls() - c0);
        };
        fp_plan* p = nullptr;
        no_calls("null q", FP_ERR_INVALID_ARG, [&] {
            return fp_prefill_plan(nullptr, k, FP_BF16, 1, 4, 4, 1024, 128, 128, 0.95f, 0.1f, 1024, nullptr, &p);
        });
        no_calls("head dim 96", FP_ERR_UNSUPPORTED, [&] {
            return fp_prefill_plan(q, k, FP_BF16, 1, 4, 4, 1024, 96, 128, 0.95f, 0.1f, 1024, nullptr, &p);
        });
        no_calls("Hq not a multiple of Hkv", FP_ERR_SHAPE, [&] {
            return fp_prefill_plan(q, k, FP_BF16, 1, 6, 4, 1024, 128, 128, 0.95f, 0.1f, 1024, nullptr, &p);
        });
        const int bad[3] = {0, 10, 5};
        no_calls("decreasing cu_seqlens", FP_ERR_INVALID_ARG, [&] {
            return fp_prefill_plan_varlen(q, k, FP_BF16, 2, bad, 4, 4, 128, 128, 0.95f, 0.1f, 1024, nullptr, nullptr,
                                          &p);
        });
        opt.max_budget = 64;
        opt.vs_granularity = FP_VS_BLOCK;
        no_calls("cap below the floor", FP_ERR_INVALID_ARG, [&] {
            return fp_prefill_plan_ex(q, k, FP_BF16, 1, 4, 4, 1024, 128, 128, 0.95f, 0.1f, 1024, &opt, nullptr, &p);
        });
        no_calls("null plan", FP_ERR_INVALID_ARG, [&] { return fp_prefill_attend_noalloc(nullptr, q, k, v, o, nullptr); });
        no_calls("null output", FP_ERR_INVALID_ARG, [&] { return fp_prefill_attend(P, q, k, v, nullptr, nullptr); });
        EXPECT(live() == before, "argument errors left resources");
    }
    // the largest minimum budget: the block floor is computed without overflow
    sweep("plan min_budget INT_MAX", [&] {
        return plan_and_release([&](fp_plan** p) {
            return fp_prefill_plan(q, k, FP_BF16, 1, 4, 4, 1024, 128, 128, 0.95f, 0.1f, 2147483647, nullptr, p);
        });
    });

    fp_plan_destroy(P);
    fp_plan_destroy(PT);
    fp_plan_destroy(PV);
    EXPECT(fp_workspace_trim() == FP_OK, "final trim");
    EXPECT(stub_live_memory() == 0, "plan memory left: %lld", stub_live_memory());
    EXPECT(stub_live_events() == 0, "events left: %lld", stub_live_events());
    EXPECT(stub_bad_releases() == 0, "releases of unknown pointers: %lld", stub_bad_releases());
    EXPECT(g_oom > 0 && g_hip > 0, "failure kinds: %lld allocation, %lld other", g_oom, g_hip);
    std::printf("failing calls: %lld allocation (FP_ERR_OOM), %lld other (FP_ERR_HIP); %d check(s) failed\n", g_oom,
                g_hip, g_failures);
    return g_failures == 0 ? 0 : 1;
}

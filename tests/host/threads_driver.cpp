// Concurrency driver for the host library built against the stub runtime
// (hip_stub.cpp) with the thread sanitizer, on the CPU.  Test infrastructure
// only.
//
// Several host threads plan, attend (on their own stream and on the null
// stream, through the allocation-free entry point too), run the dense
// baseline, read plans back and destroy them, all at once, while another
// thread trims the library's memory cache and toggles the measurement hooks.
// Every call must succeed; the sanitizer reports any data race in the
// library's shared state (memory cache, lane streams, pool set-up,
// measurement events, the allocation-free workspace).
#include <atomic>
#include <cstdio>
#include <thread>
#include <vector>

#include "fp_prefill.h"

extern "C" {
long long stub_live_memory();
long long stub_live_events();
int hipStreamCreateWithFlags(void** s, unsigned int flags);
}

int main() {
    constexpr int kThreads = 6, kIters = 40;
    std::vector<unsigned char> buf(1 << 22);
    void* q = buf.data();
    void* k = buf.data() + (1 << 20);
    void* v = buf.data() + (2 << 20);
    std::atomic<int> failures{0};
    std::atomic<bool> done{false};
    const int cu[4] = {0, 300, 700, 1001};

    auto worker = [&](int t) {
        void* st = nullptr;
        if (hipStreamCreateWithFlags(&st, 0) != 0) {
            ++failures;
            return;
        }
        std::vector<unsigned char> obuf(1 << 20);
        void* o = obuf.data();
        for (int i = 0; i < kIters; ++i) {
            fp_plan* p = nullptr;
            const int N = 256 + 128 * ((t + i) % 7);
            fp_status s;
            if ((t + i) % 3 == 0)
                s = fp_prefill_plan_varlen(q, k, FP_BF16, 3, cu, 8, 2, 128, 128, 0.95f, 0.1f, 256, nullptr,
                                           (t % 2) ? st : nullptr, &p);
            else
                s = fp_prefill_plan(q, k, (t % 2) ? FP_FP32 : FP_BF16, 1, 8, 2, N, (i % 2) ? 64 : 128, 64, 0.9f,
                                    0.1f, 128, (t % 2) ? st : nullptr, &p);
            if (s != FP_OK) {
                std::fprintf(stderr, "thread %d iter %d: plan %s (%s)\n", t, i, fp_status_str(s), fp_last_error());
                ++failures;
                continue;
            }
            if ((s = fp_prefill_attend(p, q, k, v, o, st)) != FP_OK) ++failures;
            if ((s = fp_prefill_attend(p, q, k, v, o, nullptr)) != FP_OK) ++failures;
            if (i % 5 == 0 && (s = fp_prefill_attend_noalloc(p, q, k, v, o, st)) != FP_OK) ++failures;
            fp_plan_info info{};
            if (fp_plan_info_get(p, &info) != FP_OK) ++failures;
            fp_plan_destroy(p);
            if (i % 4 == 0 && fp_dense_attend(q, k, v, o, FP_BF16, 1, 8, 2, N, 128, 128, st) != FP_OK) ++failures;
        }
    };
    std::thread janitor([&] {
        int n = 0;
        while (!done.load()) {
            if (fp_workspace_trim() != FP_OK) ++failures;
            fp_profile_enable(n % 2);
            double a, b;
            long long c, d;
            if (fp_profile_read(&a, &c, &b, &d, 1) != FP_OK) ++failures;
            ++n;
            std::this_thread::yield();
        }
    });
    std::vector<std::thread> ts;
    for (int t = 0; t < kThreads; ++t) ts.emplace_back(worker, t);
    for (auto& t : ts) t.join();
    done = true;
    janitor.join();
    fp_profile_enable(0);
    double a, b;
    long long c, d;
    (void)fp_profile_read(&a, &c, &b, &d, 1);
    if (fp_workspace_trim() != FP_OK) ++failures;
    std::printf("threads %d x %d iterations: %d failure(s); live memory %lld, events %lld after trim\n", kThreads, kIters,
                failures.load(), stub_live_memory(), stub_live_events());
    return failures.load() == 0 && stub_live_memory() == 0 && stub_live_events() == 0 ? 0 : 1;
}

// Host-only driver for the split-KV planner (pkv_plan.cpp), built with the
// host compiler under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_plan_sanitized.py.  Seeded random batches (zero lengths, decode
// rows, chunks, whole prompts, sliding windows, every head shape, compact
// and capacity layouts) are planned into images of exactly the size the
// planner asks for, so that any write past them is reported.  Prints the
// number of plans made; exits non-zero on a failed status.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv_internal.h"

int main(int argc, char** argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 300;
    std::mt19937_64 rng(20261202);
    auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    int made = 0;
    for (int t = 0; t < cases; ++t) {
        const int B = uni(0, 60);
        std::vector<int32_t> ctx(B), ql(B);
        int64_t rows = 0;
        for (int s = 0; s < B; ++s) {
            ctx[s] = uni(0, 9) == 0 ? 0 : uni(1, 9000);
            int q = uni(0, 3) == 0 ? uni(2, 600) : 1;
            if (uni(0, 9) == 0) q = ctx[s];
            ql[s] = ctx[s] == 0 ? 0 : std::min(q, ctx[s]);
            rows += ql[s];
        }
        const int hkv = 1 << uni(0, 3);
        const int hq = hkv << uni(0, 3);
        const int d = uni(0, 1) ? 128 : 64;
        const int nq = uni(1, 600);
        const int window = uni(0, 2) == 0 ? uni(1, 5000) : 0;
        const float cap = uni(0, 3) == 0 ? 30.f : 0.f;
        const bool capacity = uni(0, 1) == 1;
        const int cap_seqs = capacity ? B + uni(0, 8) : -1;
        const int cap_tokens = capacity ? static_cast<int>(rows) + uni(0, 100) : -1;
        pkv_plan plan;
        int st = pkv::plan_host(ctx.data(), ql.data(), B, hq, hkv, d, nq, nullptr, 0, &plan, cap_seqs, cap_tokens,
                                cap, window);
        if (st != PKV_OK) {
            std::printf("case %d: status %d\n", t, st);
            return 1;
        }
        std::vector<unsigned char> image(static_cast<size_t>(plan.image_bytes));
        st = pkv::plan_host(ctx.data(), ql.data(), B, hq, hkv, d, nq, image.data(), image.size(), &plan, cap_seqs,
                            cap_tokens, cap, window);
        if (st != PKV_OK) {
            std::printf("case %d: status %d with the image\n", t, st);
            return 1;
        }
        size_t ws = 0, host = 0;
        if (capacity) {
            pkv::plan_bounds(cap_seqs, cap_tokens, hq, d, nq, &ws, &host);
            if (static_cast<size_t>(plan.workspace_bytes) > ws || static_cast<size_t>(plan.image_bytes) > host) {
                std::printf("case %d: plan exceeds the workspace bound\n", t);
                return 1;
            }
        }
        ++made;
    }
    std::printf("plans %d\n", made);
    return 0;
}

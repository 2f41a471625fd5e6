// Host-side fuzz driver for the library's CPU code (packer, planners, view-
// state cache directory), built with address and undefined-behaviour
// sanitizers by tests/test_host_sanitizers.py.  Random valid and invalid
// inputs; every call must return a status without touching memory outside
// the buffers it was given, and the size queries must match the filled
// outputs.  Exits non-zero on a failed check.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "linattn.h"

#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main() {
    std::mt19937 rng(12345);
    auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    for (int it = 0; it < 3000; ++it) {
        // ---- la_pack_pass_ext with random request shapes (some invalid)
        const int nr = uni(0, 6);
        std::vector<int32_t> vl(nr), bc(nr), er(nr);
        std::vector<int32_t> bl;
        for (int r = 0; r < nr; ++r) {
            vl[r] = uni(0, 5) == 0 ? 0 : uni(1, 400);
            bc[r] = uni(0, 4);
            er[r] = uni(-1, 5);
            for (int b = 0; b < bc[r]; ++b) bl.push_back(uni(0, 10) == 0 ? uni(-1, 0) : uni(1, 200));
        }
        const int G = uni(0, 9);
        la_pass_info info{};
        const bool use_er = uni(0, 1);
        la_status st = la_pack_pass_ext(nr, vl.data(), bc.data(), bl.data(), use_er ? er.data() : nullptr,
                                        LA_CHUNK, G, nullptr, nullptr, nullptr, nullptr, &info);
        if (st == LA_OK) {
            std::vector<int32_t> so(info.n_segments + 1), bp(info.n_segments), vo(info.n_segments);
            std::vector<int32_t> plan(info.plan_words);
            la_pass_info info2{};
            st = la_pack_pass_ext(nr, vl.data(), bc.data(), bl.data(), use_er ? er.data() : nullptr,
                                  LA_CHUNK, G, so.data(), bp.data(), vo.data(), plan.data(), &info2);
            CHECK(st == LA_OK);
            CHECK(info2.plan_words == info.plan_words && info2.n_segments == info.n_segments);
            CHECK(so[0] == 0 && so[info.n_segments] == info.n_tokens);
            for (int s = 0; s < info.n_segments; ++s) CHECK(so[s + 1] > so[s]);
            // the planner on the same table agrees
            la_pass_info info3{};
            CHECK(la_plan_segments(info.n_segments, so.data(), bp.data(), LA_CHUNK, G, nullptr,
                                   nullptr, &info3) == LA_OK);
            CHECK(info3.plan_words == info.plan_words);
            // attention items cover every token once
            std::vector<int32_t> ext_len(info.n_ext, 7);
            int32_t n_items = 0;
            CHECK(la_attn_plan(info.n_segments, so.data(), bp.data(), info.n_ext, ext_len.data(),
                               nullptr, &n_items) == LA_OK);
            std::vector<int32_t> items(size_t(n_items) * LA_ATTN_ITEM_WORDS);
            CHECK(la_attn_plan(info.n_segments, so.data(), bp.data(), info.n_ext, ext_len.data(),
                               items.data(), &n_items) == LA_OK);
            std::vector<int> cover(info.n_tokens, 0);
            for (int i = 0; i < n_items; ++i) {
                const int32_t* w = &items[size_t(i) * LA_ATTN_ITEM_WORDS];
                CHECK(w[1] >= 1 && w[1] <= LA_CHUNK && w[0] >= 0 && w[0] + w[1] <= info.n_tokens);
                for (int t = w[0]; t < w[0] + w[1]; ++t) ++cover[t];
            }
            for (int t = 0; t < info.n_tokens; ++t) CHECK(cover[t] == 1);
        } else {
            CHECK(st == LA_ERR_INVALID_ARG || st == LA_ERR_UNSUPPORTED);
        }
        // ---- la_plan_segments with random (often invalid) tables
        const int ns = uni(0, 6);
        std::vector<int32_t> so(ns + 1), bp(ns);
        so[0] = uni(0, 8) == 0 ? 1 : 0;
        for (int s = 0; s < ns; ++s) so[s + 1] = so[s] + uni(0, 100);
        for (int s = 0; s < ns; ++s) bp[s] = uni(-4, ns);
        la_pass_info pi{};
        const int g2 = uni(1, 4);   // the fill call must repeat the size query's arguments
        st = la_plan_segments(ns, so.data(), bp.data(), LA_CHUNK, g2, nullptr, nullptr, &pi);
        if (st == LA_OK) {
            std::vector<int32_t> vo(ns), plan(pi.plan_words);
            la_pass_info pi2{};
            CHECK(la_plan_segments(ns, so.data(), bp.data(), LA_CHUNK, g2, vo.data(), plan.data(),
                                   &pi2) == LA_OK);
            CHECK(pi2.plan_words == pi.plan_words);
        }
        int32_t n_items = 0;
        std::vector<int32_t> ext_len(4, uni(0, 3));
        (void)la_attn_plan(ns, so.data(), bp.data(), 4, ext_len.data(), nullptr, &n_items);
        // ---- cache directory: random operations
        la_state_cache* c = nullptr;
        const int cap = uni(1, 5);
        CHECK(la_cache_create(cap, &c) == LA_OK);
        for (int op = 0; op < 50; ++op) {
            int32_t row = -2;
            int64_t ev = -2;
            const int64_t id = uni(-1, 9);
            const int kind = uni(0, 3);
            switch (kind) {
                case 0: st = la_cache_lookup(c, id, &row); break;
                case 1: st = la_cache_reserve(c, id, &row, uni(0, 1) ? &ev : nullptr); break;
                case 2: st = la_cache_erase(c, id); break;
                default: {
                    int32_t n = -1;
                    st = la_cache_count(c, &n);
                    CHECK(n >= 0 && n <= cap);
                }
            }
            if (id < 0 && kind < 3) CHECK(st == LA_ERR_INVALID_ARG);   // count takes no id
            if (st == LA_OK && row != -2) CHECK(row >= -1 && row < cap);
        }
        CHECK(la_cache_destroy(c) == LA_OK);
    }
    std::printf("host fuzz: ok\n");
    return 0;
}

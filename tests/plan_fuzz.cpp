// Host-side fuzz of the planner (plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_sanitized.py: random and edge
// tensor lists, caps, world sizes and granules, including invalid ones, through
// every host entry point; the plan's invariants are checked on each valid plan.
// Usage: plan_fuzz <seed> <iterations>; prints "ok <plans>" on success.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "gsz_internal.h"

#define CHECK(c)                                                           \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::printf("FAIL %s at line %d (iteration %d)\n", #c, __LINE__, it); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

int main(int argc, char** argv) {
    const unsigned long long seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int iters = argc > 2 ? std::atoi(argv[2]) : 1000;
    std::mt19937_64 rng(seed);
    int valid = 0;
    for (int it = 0; it < iters; ++it) {
        const int T = (int)(rng() % 48);
        std::vector<int64_t> numel((size_t)T + 1);
        for (int t = 0; t < T; ++t) {
            switch (rng() % 7) {
                case 0: numel[t] = 0; break;
                case 1: numel[t] = 1 + (int64_t)(rng() % 7); break;
                case 2: numel[t] = (int64_t)(rng() % 5000); break;
                case 3: numel[t] = (int64_t)(rng() % (1u << 20)); break;
                case 4: numel[t] = (int64_t)1 << (rng() % 36); break;
                case 5: numel[t] = (int64_t)(rng() % 100) == 0 ? -1 : 4096; break;   // sometimes invalid
                default: numel[t] = (int64_t)(rng() % 100000); break;
            }
        }
        const int64_t cap = rng() % 16 == 0 ? (int64_t)(rng() % 3) - 1 : 1 + (int64_t)(rng() % (1u << 24));
        const int32_t P = rng() % 32 == 0 ? (int32_t)(rng() % 600) - 50 : 1 + (int32_t)(rng() % 256);
        const int32_t align = rng() % 32 == 0 ? (int32_t)(rng() % 3) - 1 : (rng() % 2 ? 64 : 1 + (int32_t)(rng() % 128));
        gsz_plan* p = reinterpret_cast<gsz_plan*>(&rng);   // must be overwritten
        const int rc = gsz_plan_create(T ? numel.data() : nullptr, T, cap, P, align, &p);
        if (rc != GSZ_OK) {
            CHECK(p == nullptr);
            CHECK(gsz_last_error()[0] != '\0');
            continue;
        }
        ++valid;
        gsz_plan_info info{};
        CHECK(gsz_plan_get_info(p, &info) == GSZ_OK);
        CHECK(info.n_tensors == T && info.world_size == P && info.align == align);
        int64_t psum = 0;
        for (int t = 0; t < T; ++t) psum += numel[t];
        CHECK(info.n_params == psum);
        CHECK(info.shard_len * P == info.flat_len);
        int64_t base = 0, shard = 0;
        std::vector<int> seen((size_t)T + 1, 0);
        for (int32_t b = 0; b < info.n_buckets; ++b) {
            gsz_bucket_info bi{};
            CHECK(gsz_plan_bucket(p, b, &bi) == GSZ_OK);
            CHECK(bi.base == base && bi.shard_off == shard);
            CHECK(bi.padded >= bi.n_elems && bi.padded % ((int64_t)P * align) == 0);
            CHECK(bi.chunk * P == bi.padded);
            int64_t off = bi.base;
            for (int k = 0; k < bi.n_tensors; ++k) {
                const int t = bi.first_tensor - k;
                CHECK(t >= 0 && t < T);
                int64_t fo = -1;
                int32_t tb = -1;
                CHECK(gsz_plan_tensor(p, t, &fo, &tb) == GSZ_OK);
                CHECK(fo == off && tb == b);
                off += numel[t];
                ++seen[t];
            }
            CHECK(off - bi.base == bi.n_elems);
            base += bi.padded;
            shard += bi.chunk;
        }
        CHECK(base == info.flat_len && shard == info.shard_len);
        for (int t = 0; t < T; ++t) CHECK(seen[t] == 1);
        gsz_bucket_info bi{};
        CHECK(gsz_plan_bucket(p, -1, &bi) != GSZ_OK && gsz_plan_bucket(p, info.n_buckets, &bi) != GSZ_OK);
        int64_t fo;
        int32_t tb;
        CHECK(gsz_plan_tensor(p, -1, &fo, &tb) != GSZ_OK && gsz_plan_tensor(p, T, &fo, &tb) != GSZ_OK);
        CHECK(gsz_plan_check(p, info.hash) == GSZ_OK);
        CHECK(gsz_plan_check(p, info.hash ^ 1) == GSZ_ERR_PLAN_MISMATCH);
        size_t ws = 0;
        CHECK(gsz_workspace_bytes(info.shard_len, &ws) == GSZ_OK && ws >= 8 * 1025);
        delete p;                                  // no device tables were made
    }
    // host entry points with hostile arguments
    int it = iters;
    size_t ws = 0;
    double d = 0;
    CHECK(gsz_workspace_bytes(-1, &ws) != GSZ_OK && gsz_workspace_bytes(5, nullptr) != GSZ_OK);
    CHECK(gsz_workspace_bytes((int64_t)1 << 62, &ws) == GSZ_OK);
    CHECK(gsz_ledger_bytes_per_param(0, 0, &d) != GSZ_OK && gsz_ledger_bytes_per_param(8, 4, &d) != GSZ_OK);
    CHECK(gsz_ledger_bytes_per_param(8, 2, nullptr) != GSZ_OK);
    CHECK(gsz_plan_get_info(nullptr, nullptr) != GSZ_OK);
    CHECK(gsz_plan_check(nullptr, 0) != GSZ_OK);
    for (int s = -12; s <= 2; ++s) CHECK(gsz_status_string(s) != nullptr);
    std::printf("ok %d\n", valid);
    return 0;
}

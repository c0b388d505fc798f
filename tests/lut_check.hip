// Host-only check of the plan lookup tables: for every plan read from stdin,
// the kernels' own lut_find (compiled here for the host) must give, for every
// position checked, the interval a brute-force scan gives -- the tensor of each
// pack tile (also within each launch batch of kPackBatch tensors) and the
// bucket of each shard index.  No GPU call is made.
//
// stdin, one plan per line: P align cap_bytes T numel_0 ... numel_{T-1}
// A plan whose tile or shard count exceeds 4M is checked at every position
// within 2 of an interval start or a cell edge, and at 200000 seeded others.
// Prints "ok <plans> <positions>" or the first mismatch (exit 1).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "gsz_device.h"

namespace {

int64_t g_checked = 0;

// The starts column of a table, copied out (the reference's own data).
std::vector<int64_t> column(const std::vector<int64_t>& tab, int off, int n) {
    std::vector<int64_t> c((size_t)n);
    for (int k = 0; k < n; ++k) c[(size_t)k] = tab[(size_t)k * 3 + off];
    return c;
}

bool check_one(const char* what, const gsz::Lut& lut, const std::vector<int64_t>& tab, int off,
               const std::vector<int64_t>& starts, int64_t total, int lo_min, int hi_max, int64_t x) {
    const int n = (int)starts.size();
    const int got = lut_find(reinterpret_cast<const uint64_t*>(lut.cells.data()), lut.shift,
                             tab.data() + off, 3, x, lo_min, hi_max);
    // reference: the largest k in [lo_min, min(hi_max, n - 1)] with starts[k] <= x
    const int hi = hi_max < n - 1 ? hi_max : n - 1;
    const int want = (int)(std::upper_bound(starts.begin() + lo_min, starts.begin() + hi + 1, x) -
                           starts.begin()) - 1;
    ++g_checked;
    if (got != want) {
        std::printf("MISMATCH %s: position %lld of %lld, bounds [%d, %d], n %d: lut %d, reference %d\n",
                    what, (long long)x, (long long)total, lo_min, hi_max, n, got, want);
        return false;
    }
    return true;
}

// Positions to check in [a, b): all of them when few, else those near the
// interval starts and cell edges plus seeded random ones.
std::vector<int64_t> positions(int64_t a, int64_t b, const std::vector<int64_t>& tab, int off, int n,
                               int shift, std::mt19937_64& rng) {
    std::vector<int64_t> xs;
    if (b - a <= (4 << 20)) {
        for (int64_t x = a; x < b; ++x) xs.push_back(x);
        return xs;
    }
    auto near = [&](int64_t c) {
        for (int64_t d = -2; d <= 2; ++d)
            if (c + d >= a && c + d < b) xs.push_back(c + d);
    };
    for (int k = 0; k < n; ++k) near(tab[(size_t)k * 3 + off]);
    for (int64_t c = (a >> shift) << shift; c < b; c += (int64_t)1 << shift) near(c);
    std::uniform_int_distribution<int64_t> u(a, b - 1);
    for (int i = 0; i < 200000; ++i) xs.push_back(u(rng));
    return xs;
}

}  // namespace

int main() {
    std::mt19937_64 rng(2026);
    int plans = 0;
    int P, align;
    long long cap;
    int T;
    while (std::scanf("%d %d %lld %d", &P, &align, &cap, &T) == 4) {
        std::vector<int64_t> numel(T);
        for (int t = 0; t < T; ++t) {
            long long v;
            if (std::scanf("%lld", &v) != 1) { std::printf("bad input\n"); return 2; }
            numel[t] = v;
        }
        gsz_plan* p = nullptr;
        if (gsz_plan_create(numel.data(), T, cap, P, align, &p) != GSZ_OK) {
            std::printf("plan rejected: %s\n", gsz_last_error());
            return 2;
        }
        const int B = (int)p->buckets.size();
        const int64_t tiles = T ? p->pack[(size_t)T * 3 + 2] : 0;
        const std::vector<int64_t> tile0 = column(p->pack, 2, T), shard0 = column(p->seg, 0, B);
        // pack: tile -> bucket-order tensor, over all tensors and within each launch batch
        for (int64_t x : positions(0, tiles, p->pack, 2, T, p->pack_lut.shift, rng))
            if (!check_one("pack", p->pack_lut, p->pack, 2, tile0, tiles, 0, T - 1, x)) return 1;
        for (int k0 = 0; k0 < T; k0 += gsz::kPackBatch) {
            const int nk = T - k0 < gsz::kPackBatch ? T - k0 : gsz::kPackBatch;
            const int64_t tb = p->pack[(size_t)k0 * 3 + 2], te = p->pack[(size_t)(k0 + nk) * 3 + 2];
            for (int64_t x : positions(tb, te, p->pack, 2, T, p->pack_lut.shift, rng))
                if (!check_one("pack batch", p->pack_lut, p->pack, 2, tile0, tiles, k0, k0 + nk - 1, x))
                    return 1;
        }
        // shard index -> bucket
        for (int64_t x : positions(0, p->shard_len, p->seg, 0, B, p->seg_lut.shift, rng))
            if (!check_one("seg", p->seg_lut, p->seg, 0, shard0, p->shard_len, 0, 0x7fffffff, x)) return 1;
        const size_t want_cells_t = tiles ? (size_t)(((tiles - 1) >> p->pack_lut.shift) + 1) : 0;
        const size_t want_cells_s = p->shard_len ? (size_t)(((p->shard_len - 1) >> p->seg_lut.shift) + 1) : 0;
        if (p->pack_lut.cells.size() != 2 * want_cells_t || p->seg_lut.cells.size() != 2 * want_cells_s ||
            want_cells_t > ((size_t)1 << gsz::kLutCellsLog2) || want_cells_s > ((size_t)1 << gsz::kLutCellsLog2)) {
            std::printf("MISMATCH table sizes: %zu/%zu cells for %lld tiles, %zu/%zu for %lld shard elements\n",
                        p->pack_lut.cells.size() / 2, want_cells_t, (long long)tiles,
                        p->seg_lut.cells.size() / 2, want_cells_s, (long long)p->shard_len);
            return 1;
        }
        delete p;                       // no device tables were made
        ++plans;
    }
    std::printf("ok %d %lld\n", plans, (long long)g_checked);
    return 0;
}

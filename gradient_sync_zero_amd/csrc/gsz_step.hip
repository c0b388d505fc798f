// Host half of the C ABI: argument checks, launch shapes and the entry points of
// include/gsz.h.  The kernels live in gsz_kernels_*.h (one header per part of
// the step, shared pieces in gsz_device.h), all compiled in this one
// translation unit.
//
// Pages cited (title, section): see gsz.h.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "gsz_device.h"
#include "gsz_internal.h"
#include "gsz_kernels_adamw.h"
#include "gsz_kernels_pack.h"
#include "gsz_kernels_reduce.h"

using gsz::set_error;

namespace {

// ------------------------------------------------------------ host side --

std::atomic<int> g_dev_state[64];   // 0 unknown, 1 gfx950, -1 other
std::atomic<int> g_dev_cus[64];     // compute units, set before g_dev_state

int hip_fail(const char* what, hipError_t e) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return GSZ_ERR_HIP;
}

// Current device, checked to be gfx950.
int current_device(int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= 64) { set_error("device index %d unsupported", dev); return GSZ_ERR_DEVICE; }
    int st = g_dev_state[dev].load();
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_dev_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1);
        g_dev_state[dev].store(st);
    }
    if (st != 1) { set_error("device %d is not gfx950 (MI355X); this library targets gfx950 only", dev); return GSZ_ERR_DEVICE; }
    *dev_out = dev;
    return GSZ_OK;
}

#ifdef GSZ_TEST_HOOKS
// Test builds only (libgsz_test.so, include/gsz_test.h): a process-wide cap on
// the blocks of grid-sized launches (0: the built-in caps), so that tests can
// run the block-striding path that otherwise only inputs of more than about
// 17e9 elements reach.  The product library has no such state.
std::atomic<int64_t> g_grid_limit{0};
// Which kernel the bf16 reduce at P > 16 uses: 0 the product's rule (use_burst),
// 1 always the burst kernel, 2 never (so that small test shards reach both).
std::atomic<int> g_reduce_path{0};
// The burst kernel's write window (period, window) in clock ticks; period 0:
// the product's choice (burst_write), else these, so that tests can reach
// every write policy: chunk writes (window 0), windows, every row at once
// (window >= period).
std::atomic<uint32_t> g_win_period{0}, g_win_window{0};
// Nonzero: bucket-flat reduces take the 64-bit-address path of the
// lane-contiguous kernel (kLayFlatWide) and AdamW's all-gather stores theirs,
// which otherwise only plans with buckets of over 2^29 elements reach.
std::atomic<int> g_force_flat_wide{0};
#endif

// Blocks of a one-tile-per-block launch over n_tiles tiles: at most `builtin`
// (the dispatch limit for the kernel's block size).
int tile_grid(int64_t n_tiles, int64_t builtin) {
    int64_t cap = builtin;
#ifdef GSZ_TEST_HOOKS
    const int64_t lim = g_grid_limit.load(std::memory_order_relaxed);
    if (lim > 0 && lim < builtin) cap = lim;
#endif
    if (n_tiles < 1) return 1;
    return (int)(n_tiles < cap ? n_tiles : cap);
}
int flat_grid(int64_t n_tiles) { return tile_grid(n_tiles, kMaxFlatGrid); }

// Partials of the reductions: grid blocks wrote ws[0, grid); sum them in a
// fixed order into *out (two stages when there are many).
void launch_finalize(double* ws, int64_t grid, double* out, hipStream_t stream) {
    if (grid > gsz::kFinalBlocks) {
        hipLaunchKernelGGL(k_finalize_ranges, dim3(gsz::kFinalBlocks), dim3(kBlock), 0, stream,
                           static_cast<const double*>(ws), grid, ws + grid);
        hipLaunchKernelGGL(k_finalize, dim3(1), dim3(kBlock), 0, stream,
                           static_cast<const double*>(ws + grid), (int64_t)gsz::kFinalBlocks, out);
    } else {
        hipLaunchKernelGGL(k_finalize, dim3(1), dim3(kBlock), 0, stream,
                           static_cast<const double*>(ws), grid, out);
    }
}

int launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(what, e);
    return GSZ_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// The fp32 constants of the update, each formed in double and rounded once.
AdamScalars adam_scalars(const gsz_adamw_hp& hp) {
    AdamScalars s;
    s.b1 = (float)hp.beta1;
    s.omb1 = (float)(1.0 - hp.beta1);
    s.b2 = (float)hp.beta2;
    s.omb2 = (float)(1.0 - hp.beta2);
    s.bc1 = (float)(1.0 - std::pow(hp.beta1, (double)hp.step));
    s.bc2 = (float)(1.0 - std::pow(hp.beta2, (double)hp.step));
    s.lr = (float)hp.lr;
    s.eps = (float)hp.eps;
    s.decay = (float)(1.0 - hp.lr * hp.weight_decay);
    return s;
}

// Checks a plan for a device call: uploaded to the current device, vector granule.
int check_plan(const gsz_plan* p, const char* who) {
    if (!p) { set_error("%s: NULL plan", who); return GSZ_ERR_INVALID_ARG; }
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (!p->d_seg || p->device != dev) {
        set_error("%s: plan has no device tables on device %d (call gsz_plan_upload)", who, dev);
        return GSZ_ERR_NOT_UPLOADED;
    }
    if (p->align % 8 != 0) {
        set_error("%s: device calls need align a multiple of 8 elements (plan has %d)", who, p->align);
        return GSZ_ERR_INVALID_ARG;
    }
    return GSZ_OK;
}

int check_owner(const gsz_plan* p, int32_t owner, const char* who) {
    if (owner < 0 || owner >= p->P) {
        set_error("%s: owner %d outside [0, %d)", who, owner, p->P);
        return GSZ_ERR_BAD_RANK;
    }
    return GSZ_OK;
}

// Calls f(std::integral_constant<int, PS>{}) with PS = P for the world sizes that
// have unrolled kernels and PS = 0 (the runtime-P loop) for every other P.  The
// bf16 reduces also unroll P = 3, 6, 24 and 96, where the runtime loop waits
// for its last (P-1) mod 8 contributions one at a time (measured on two machines:
// P = 3 7-9% faster unrolled, P = 6 2-5%, P = 24 1-2%, P = 96 0.5-6.5%; P = 12,
// 48 and 128 gained nothing); the fp32 reduce keeps the powers of two (unrolled
// at 48 or more it needs all 256 registers per lane).
template <bool kBf16 = false, class F>
void with_static_p(int P, F&& f) {
    switch (P) {
        case 2: f(std::integral_constant<int, 2>{}); return;
        case 4: f(std::integral_constant<int, 4>{}); return;
        case 8: f(std::integral_constant<int, 8>{}); return;
        case 16: f(std::integral_constant<int, 16>{}); return;
        case 32: f(std::integral_constant<int, 32>{}); return;
        case 64: f(std::integral_constant<int, 64>{}); return;
        default: break;
    }
    if constexpr (kBf16) {
        switch (P) {
            case 3: f(std::integral_constant<int, 3>{}); return;
            case 6: f(std::integral_constant<int, 6>{}); return;
            case 24: f(std::integral_constant<int, 24>{}); return;
            case 96: f(std::integral_constant<int, 96>{}); return;
            default: break;
        }
    }
    f(std::integral_constant<int, 0>{});
}

// Calls go(Lay{}) with Lay = std::integral_constant<int, lay> for the three
// contribution layouts.
template <class F>
void with_layout(int lay, F&& go) {
    if (lay == kLayFlat) go(std::integral_constant<int, kLayFlat>{});
    else if (lay == kLayCompact) go(std::integral_constant<int, kLayCompact>{});
    else go(std::integral_constant<int, kLayInterleaved>{});
}

// Launches k_reduce_mean<PS, ...> with the flags as template arguments (the
// combinations the entry points use): lay is a kLay* layout; outflat (the
// all-reduce's flat-position output) needs bucket-flat input.
template <int PS>
void launch_reduce(bool norm, int lay, dim3 grid, hipStream_t st, const RankPtrs& rp, int P,
                   float invP, int pow2, const int64_t* seg, const uint64_t* slut, int sshift,
                   int64_t owner, int64_t nvec, float* g, double* ws, bool outflat = false,
                   bool wire16 = false) {
    auto go = [&](auto nm, auto ly, auto of, auto w16) {
        hipLaunchKernelGGL((k_reduce_mean<PS, decltype(nm)::value, decltype(ly)::value,
                                          decltype(of)::value, decltype(w16)::value>),
                           grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, slut, sshift, owner,
                           nvec, g, ws);
    };
    using Y = std::true_type;
    using N = std::false_type;
    using Flat = std::integral_constant<int, kLayFlat>;
    auto layouts = [&](auto w16) {
        with_layout(lay, [&](auto ly) {
            if (norm) go(Y{}, ly, N{}, w16);
            else go(N{}, ly, N{}, w16);
        });
    };
    if (outflat) {
        if (norm) go(Y{}, Flat{}, Y{}, N{});
        else go(N{}, Flat{}, Y{}, N{});
    } else if (wire16) {
        layouts(Y{});
    } else {
        layouts(N{});
    }
}

// The largest world size of the lane-contiguous bf16 reduce (launch_reduce_lc).
constexpr int kLcMaxP = 16;

// The burst reduce (k_reduce_burst) serves bf16 contributions at every P above
// kLcMaxP on shards of at least kBurstMinElems elements: one block per CU, at
// most one per chunk.  Measured against the one-tile-per-block kernel on 64 GB
// of shard-compact contributions: 2-3% faster at P = 24, 32, 64 and 96 (the
// unrolled kernels) and 1.5-7% faster at P = 17, 33, 40, 48, 100, 128, 200 and
// 256 (the runtime-P loop, which in this kernel keeps 32 loads in flight and
// issues its last (P-1) mod 8 together; one at a time, as the tile kernel's
// loop does with more waves to hide them, it was up to 13% slower).  The bf16
// wire keeps the tile kernel: its rounding after every addition made the burst
// kernel 58% slower at P = 64 (36 ms against 22.7 ms on the 70B share).  Over
// shard sizes (P = 64 and 24): 4-12% faster from 2^23 to 2^27 elements, 3% at
// the 70B share's 1.08e9, and 13-70% slower at 2^22 and below, where the tile
// kernel has more blocks to spread over the chip.
constexpr int64_t kBurstMinElems = (int64_t)1 << 23;

bool use_burst(int P, int64_t S, bool wire16) {
#ifdef GSZ_TEST_HOOKS
    const int forced = g_reduce_path.load(std::memory_order_relaxed);
    if (forced == 1) return P > kLcMaxP;
    if (forced == 2) return false;
#endif
    return !wire16 && P > kLcMaxP && S >= kBurstMinElems;
}

// How the burst kernel writes g: with `chunked`, each chunk (or tail piece)
// by the whole block once it is reduced; else each wave writes the rows it
// holds when (100 MHz constant clock & (period - 1)) < window, or when its
// ring of kRingRows rows is full.  A wave fills its ring in about 250 * P
// ticks when the chip reads at 6.5 TB/s (16 rows of P KiB each at a CU's
// 25 GB/s shared by 4 waves), so a period of the largest power of two up to
// 256 * P has each ring written in a window before it fills, in 15% of the
// period.
//
// Measured against chunk writes on shard-compact contributions (P x S): the
// windows are 1.5-7% faster at P = 24-128 on 2^28 elements and 3% faster on
// the 70B share (P = 64, 1.08e9); at P = 32 and 64 also 2-6% faster on 2^26
// and 2^27.  Below 2^26 they are up to 6% slower, and 1-2.5% slower at
// P = 17-20 (equal at 2^28) and at P = 200-256, where writes are under 1% of
// the bytes: there the per-wave rings, which give up the block's lockstep
// over a chunk's rows, cost more than the windows save.
constexpr int kWinMinP = 24, kWinMaxP = 128;
constexpr int64_t kWinMinElems = (int64_t)1 << 27;
struct BurstWrite { int chunked; uint32_t period, window; };
BurstWrite burst_write(int P, int64_t S) {
#ifdef GSZ_TEST_HOOKS
    const uint32_t tp = g_win_period.load(std::memory_order_relaxed);
    if (tp > 0) {
        const uint32_t tw = g_win_window.load(std::memory_order_relaxed);
        return {tw == 0, tp, tw};
    }
#endif
    uint32_t period = 1;
    while (period * 2 <= 256u * (uint32_t)P) period *= 2;
    const bool windows = P >= kWinMinP && P <= kWinMaxP && S >= kWinMinElems;
    return {!windows, period, period * 3 / 20};
}

int burst_grid(int dev, int64_t S) {
    const int64_t chunks = (S + kBurstElems - 1) / kBurstElems;
    int64_t g = g_dev_cus[dev].load();
    if (g < 1) g = 1;
#ifdef GSZ_TEST_HOOKS
    const int64_t lim = g_grid_limit.load(std::memory_order_relaxed);
    if (lim > 0 && lim < g) g = lim;
#endif
    return (int)(chunks < g ? (chunks < 1 ? 1 : chunks) : g);
}

template <int PS>
void launch_reduce_burst(bool norm, int lay, bool wire16, dim3 grid, hipStream_t st,
                         const RankPtrs& rp, int P, float invP, int pow2, const int64_t* seg,
                         const uint64_t* slut, int sshift, int64_t owner, int64_t S, float* g,
                         double* ws) {
    const BurstWrite wr = burst_write(P, S);
    auto go = [&](auto nm, auto ly, auto w16) {
        hipLaunchKernelGGL((k_reduce_burst<PS, decltype(nm)::value, decltype(ly)::value,
                                           decltype(w16)::value>),
                           grid, dim3(kBlock), 0, st, rp, P, invP, pow2, seg, slut, sshift, owner,
                           S, g, ws, wr.chunked, wr.period - 1, wr.window);
    };
    auto layouts = [&](auto w16) {
        with_layout(lay, [&](auto ly) {
            if (norm) go(std::true_type{}, ly, w16);
            else go(std::false_type{}, ly, w16);
        });
    };
    if (wire16) layouts(std::true_type{});
    else layouts(std::false_type{});
}

// The largest flat span (last position - first position + 1) of a tile of T
// consecutive shard elements of owner r, over the shard's tiles.  Positions
// rise with the shard index, so only tiles that cross a bucket boundary span
// more than T.
int64_t max_tile_span(const gsz_plan* p, int64_t owner, int64_t T) {
    const std::vector<int64_t>& seg = p->seg;     // {shard_off, base, chunk} per bucket, then {S, 0, 0}
    const int64_t S = p->shard_len;
    const size_t B = seg.size() / 3 - 1;
    auto map = [&](int64_t i, size_t& b) {      // b: a bucket at or before i's, moved to i's
        while (b + 1 < B && seg[3 * (b + 1)] <= i) ++b;
        return i - seg[3 * b] + seg[3 * b + 1] + owner * seg[3 * b + 2];
    };
    int64_t best = S < T ? S : T;
    size_t b0 = 0;
    for (size_t b = 1; b < B; ++b) {
        const int64_t s0 = seg[3 * b];
        if (s0 >= S) break;
        const int64_t first = s0 / T * T;
        if (first == s0) continue;              // the tile starts in bucket b
        const int64_t last = (first + T < S ? first + T : S) - 1;
        size_t bb = b0;
        const int64_t lo = map(first, bb);
        b0 = bb;
        const int64_t hi = map(last, bb);
        if (hi - lo + 1 > best) best = hi - lo + 1;
    }
    return best;
}

// The layout the lane-contiguous kernel takes for bucket-flat contributions of
// esize bytes: kLayFlatWide when a 2048-element tile's offsets can reach 2^31
// bytes (its buffer descriptors take 32-bit offsets), else kLayFlat.
int flat_lay_for(const gsz_plan* p, int64_t owner, int64_t esize) {
#ifdef GSZ_TEST_HOOKS
    if (g_force_flat_wide.load(std::memory_order_relaxed)) return kLayFlatWide;
#endif
    return max_tile_span(p, owner, kRedTile) * esize >= ((int64_t)1 << 31) ? kLayFlatWide : kLayFlat;
}

// The lane-contiguous reduce (k_reduce_mean_lc) for bf16 contributions at
// P <= kLcMaxP (compile-time P for 2, 3, 4, 6, 8 and 16, its runtime-P loop for
// the others) and for fp32 contributions at every P.
// clen: elements of each contribution buffer (flat_len, S, or S * P for the
// interleaved receive buffer); lay may be kLayFlatWide (flat_lay_for).
template <typename T, int PS>
void launch_reduce_lc(bool norm, int lay, bool outflat, bool wire16, dim3 grid, hipStream_t st,
                      const RankPtrsT<T>& rp, int P, float invP, int pow2, const int64_t* seg,
                      const uint64_t* slut, int sshift, int64_t owner, int64_t S, int64_t clen,
                      float* g, double* ws) {
    const size_t lds = (int64_t)P * (int64_t)sizeof(T) >= kRedLcLdsMinBytes ? kRedLcLdsBytes : 0;
    auto go = [&](auto nm, auto ly, auto of, auto w16) {
        hipLaunchKernelGGL((k_reduce_mean_lc<T, PS, decltype(nm)::value, decltype(ly)::value,
                                             decltype(of)::value, decltype(w16)::value>),
                           grid, dim3(kBlock), lds, st, rp, P, invP, pow2, seg, slut, sshift, owner, S,
                           clen, g, ws);
    };
    using Y = std::true_type;
    using N = std::false_type;
    using Flat = std::integral_constant<int, kLayFlat>;
    using FlatWide = std::integral_constant<int, kLayFlatWide>;
    auto layouts = [&](auto w16) {
        auto pick = [&](auto ly) {
            if (norm) go(Y{}, ly, N{}, w16);
            else go(N{}, ly, N{}, w16);
        };
        if (lay == kLayFlatWide) pick(FlatWide{});
        else with_layout(lay, pick);
    };
    if constexpr (std::is_same<T, float>::value) {
        layouts(N{});                            // fp32 contributions: the reduce rows only
    } else {
        if (outflat) {
            if (lay == kLayFlatWide) {
                if (norm) go(Y{}, FlatWide{}, Y{}, N{});
                else go(N{}, FlatWide{}, Y{}, N{});
            } else {
                if (norm) go(Y{}, Flat{}, Y{}, N{});
                else go(N{}, Flat{}, Y{}, N{});
            }
        } else if (wire16) {
            layouts(Y{});
        } else {
            layouts(N{});
        }
    }
}

}  // namespace

// ---------------------------------------------------------------- C ABI --

#ifdef GSZ_TEST_HOOKS
extern "C" int gsz_test_set_grid_limit(int64_t max_blocks) {
    if (max_blocks < 0) {
        set_error("gsz_test_set_grid_limit: max_blocks %lld is negative", (long long)max_blocks);
        return GSZ_ERR_INVALID_ARG;
    }
    g_grid_limit.store(max_blocks, std::memory_order_relaxed);
    return GSZ_OK;
}

extern "C" int gsz_test_set_reduce_path(int32_t path) {
    if (path < 0 || path > 2) {
        set_error("gsz_test_set_reduce_path: path %d is not 0, 1 or 2", (int)path);
        return GSZ_ERR_INVALID_ARG;
    }
    g_reduce_path.store(path, std::memory_order_relaxed);
    return GSZ_OK;
}

extern "C" int gsz_test_max_tile_span(const gsz_plan* p, int32_t owner, int64_t tile, int64_t* out) {
    if (!p || !out || tile < 1) { set_error("gsz_test_max_tile_span: bad arguments"); return GSZ_ERR_INVALID_ARG; }
    if (owner < 0 || owner >= p->P) { set_error("gsz_test_max_tile_span: owner %d outside [0, %d)", owner, p->P); return GSZ_ERR_BAD_RANK; }
    *out = max_tile_span(p, owner, tile);
    return GSZ_OK;
}

extern "C" int gsz_test_set_flat_wide(int32_t on) {
    g_force_flat_wide.store(on != 0, std::memory_order_relaxed);
    return GSZ_OK;
}

extern "C" int gsz_test_set_burst_window(uint32_t period, uint32_t window) {
    if (period & (period - 1)) {
        set_error("gsz_test_set_burst_window: period %u is not 0 or a power of two", period);
        return GSZ_ERR_INVALID_ARG;
    }
    g_win_period.store(period, std::memory_order_relaxed);
    g_win_window.store(window, std::memory_order_relaxed);
    return GSZ_OK;
}
#endif

extern "C" int gsz_plan_upload(gsz_plan* p, void* dev_tables, size_t bytes, hipStream_t stream) {
    const char* who = "gsz_plan_upload";
    if (!p) { set_error("%s: NULL plan", who); return GSZ_ERR_INVALID_ARG; }
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    const size_t need = p->image.size() * sizeof(int64_t);
    if (!dev_tables) { set_error("%s: NULL device buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(dev_tables)) { set_error("%s: device buffer is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    if (bytes < need) {
        set_error("%s: device buffer of %zu bytes, the plan's tables need %zu (gsz_plan_device_bytes)",
                  who, bytes, need);
        return GSZ_ERR_SIZE;
    }
    std::lock_guard<std::mutex> lock(p->mu);
    // The source is the plan's own image, which lives as long as the plan, so
    // the copy may still be in flight when this returns.
    const hipError_t e = hipMemcpyAsync(dev_tables, p->image.data(), need, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail("gsz_plan_upload: hipMemcpyAsync", e);
    const size_t n_seg = p->seg.size(), n_pack = p->pack.size(), n_pads = p->pads.size();
    const size_t n_slut = p->seg_lut.cells.size() / 2;
    const int64_t* d = static_cast<const int64_t*>(dev_tables);
    p->device = dev;
    p->d_seg = d;
    p->d_pack = d + n_seg;
    p->d_pads = d + n_seg + n_pack;
    p->d_seg_lut = reinterpret_cast<const uint64_t*>(d + n_seg + n_pack + n_pads);
    p->d_pack_lut = reinterpret_cast<const uint64_t*>(d + n_seg + n_pack + n_pads + n_slut);
    return GSZ_OK;
}

namespace {

// Modes of run_pack beyond PackMode: the fp32 bucket buffer's first micro-batch
// (widen) and later ones (add).
constexpr int kPackF32 = 3, kAccumulateF32 = 4;

// Launches the pack kernel in `mode` over every tensor: ptrs is the host array of
// the T tensor pointers (sources for kPack/kAccumulate and the fp32 modes,
// destinations for kUnpack); flat is bf16 (uint16) or, in the fp32 modes, float.
int run_pack(const gsz_plan* p, const uint16_t* const* ptrs, void* flat, int mode,
             hipStream_t stream, const char* who) {
    int rc = check_plan(p, who);
    if (rc) return rc;
    const int T = (int)p->numel.size();
    if (p->flat_len == 0) return GSZ_OK;
    if (!flat || (T > 0 && !ptrs)) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(flat)) { set_error("%s: flat is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    for (int t = 0; t < T; ++t)
        if (p->numel[t] > 0 && !ptrs[t]) {
            set_error("%s: tensor pointer %d is NULL", who, t); return GSZ_ERR_INVALID_ARG;
        }
    for (int k0 = 0; k0 < T; k0 += gsz::kPackBatch) {
        const int nk = T - k0 < gsz::kPackBatch ? T - k0 : gsz::kPackBatch;
        PackPtrs pp{};
        for (int k = 0; k < nk; ++k) pp.p[k] = ptrs[T - 1 - (k0 + k)];
        const int64_t tb = p->pack[3 * k0 + 2], te = p->pack[3 * (k0 + nk) + 2];
        if (te == tb) continue;
        const int block = mode >= kPackF32 ? kF32Block : kPackBlock;
        const int grid = tile_grid(te - tb, kMaxWorkItems / block);
        uint16_t* f16 = static_cast<uint16_t*>(flat);
        float* f32 = static_cast<float*>(flat);
        if (mode == kPack)
            hipLaunchKernelGGL(k_pack<kPack>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, p->d_pack_lut, p->pack_lut.shift, k0, nk, tb, te, f16);
        else if (mode == kUnpack)
            hipLaunchKernelGGL(k_pack<kUnpack>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, p->d_pack_lut, p->pack_lut.shift, k0, nk, tb, te, f16);
        else if (mode == kAccumulate)
            hipLaunchKernelGGL(k_pack<kAccumulate>, dim3(grid), dim3(kPackBlock), 0, stream, pp, p->d_pack, p->d_pack_lut, p->pack_lut.shift, k0, nk, tb, te, f16);
        else if (mode == kPackF32)
            hipLaunchKernelGGL(k_pack_f32<false>, dim3(grid), dim3(kF32Block), 0, stream, pp, p->d_pack, p->d_pack_lut, p->pack_lut.shift, k0, nk, tb, te, f32);
        else
            hipLaunchKernelGGL(k_pack_f32<true>, dim3(grid), dim3(kF32Block), 0, stream, pp, p->d_pack, p->d_pack_lut, p->pack_lut.shift, k0, nk, tb, te, f32);
        if ((rc = launched(who))) return rc;
    }
    const int npad = (int)(p->pads.size() / 2);
    if (mode == kPack && npad > 0) {
        hipLaunchKernelGGL(k_zero_pads, dim3(npad), dim3(kBlock), 0, stream, p->d_pads,
                           static_cast<uint16_t*>(flat));
        if ((rc = launched(who))) return rc;
    }
    if (mode == kPackF32 && npad > 0) {
        hipLaunchKernelGGL(k_zero_pads_f32, dim3(npad), dim3(kBlock), 0, stream, p->d_pads,
                           static_cast<float*>(flat));
        if ((rc = launched(who))) return rc;
    }
    return GSZ_OK;
}

}  // namespace

extern "C" int gsz_bucket_pack(const gsz_plan* p, const uint16_t* const* grads, uint16_t* flat,
                               hipStream_t stream) {
    return run_pack(p, grads, flat, kPack, stream, "gsz_bucket_pack");
}

extern "C" int gsz_bucket_accumulate(const gsz_plan* p, const uint16_t* const* grads,
                                     uint16_t* flat, hipStream_t stream) {
    return run_pack(p, grads, flat, kAccumulate, stream, "gsz_bucket_accumulate");
}

extern "C" int gsz_bucket_pack_f32(const gsz_plan* p, const uint16_t* const* grads, float* flat32,
                                   hipStream_t stream) {
    return run_pack(p, grads, flat32, kPackF32, stream, "gsz_bucket_pack_f32");
}

extern "C" int gsz_bucket_accumulate_f32(const gsz_plan* p, const uint16_t* const* grads,
                                         float* flat32, hipStream_t stream) {
    return run_pack(p, grads, flat32, kAccumulateF32, stream, "gsz_bucket_accumulate_f32");
}

namespace {

// The shard reduce over bf16 contributions (wire16: rounding the partial sums
// to bf16) or, with f32in, over fp32 contributions; contrib holds P device
// pointers of the matching type.
int reduce_impl(const gsz_plan* p, int32_t owner, const void* const* contrib, int32_t layout,
                float* g, double* partial_out, void* ws, size_t ws_bytes, hipStream_t stream,
                bool wire16, bool f32in, const char* who) {
    int rc = check_plan(p, who);
    if (rc) return rc;
    if ((rc = check_owner(p, owner, who))) return rc;
    if (layout != GSZ_LAYOUT_BUCKET_FLAT && layout != GSZ_LAYOUT_SHARD_COMPACT &&
        layout != GSZ_LAYOUT_RANK_INTERLEAVED) {
        set_error("%s: unknown layout %d", who, layout); return GSZ_ERR_INVALID_ARG;
    }
    const int P = p->P;
    const int64_t S = p->shard_len;
    // The interleaved layout passes one receive buffer; the others P buffers.
    const bool ilv = layout == GSZ_LAYOUT_RANK_INTERLEAVED;
    const int n_ptrs = ilv ? 1 : P;
    if (partial_out) {
        size_t need = 0;
        gsz_workspace_bytes(S, &need);
        if (!ws || ws_bytes < need) { set_error("%s: workspace of %zu bytes required", who, need); return GSZ_ERR_SIZE; }
        if (misaligned(ws)) { set_error("%s: workspace is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    }
    if (S > 0) {
        if (!g || !contrib) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
        if (misaligned(g)) { set_error("%s: g is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
        for (int q = 0; q < n_ptrs; ++q) {
            if (!contrib[q]) { set_error("%s: contribution %d is NULL", who, q); return GSZ_ERR_INVALID_ARG; }
            if (misaligned(contrib[q])) { set_error("%s: contribution %d is not 16-byte aligned", who, q); return GSZ_ERR_MISALIGNED; }
        }
    }
    const int64_t nvec = S / 8;
    int grid = flat_grid((S + kRedTile - 1) / kRedTile);
    const int lay = layout == GSZ_LAYOUT_BUCKET_FLAT ? kLayFlat : ilv ? kLayInterleaved : kLayCompact;
    // Elements of each contribution buffer, and the layout the lane-contiguous
    // kernel takes (bucket-flat plans with very large buckets read through
    // 64-bit addresses).
    const int64_t clen = lay == kLayFlat ? p->flat_len : ilv ? S * P : S;
    const int lay_lc = lay == kLayFlat && S > 0 ? flat_lay_for(p, owner, f32in ? 4 : 2) : lay;
    // The bf16 reduce at P > kLcMaxP on a large shard runs the burst kernel,
    // whose grid is one block per CU (at most one per chunk).
    const bool burst = !f32in && use_burst(P, S, wire16);
    if (burst) grid = burst_grid(p->device, S);
    // p[k] = the contribution of rank (owner + 1 + k) mod P: its buffer, or its
    // piece of the first tile of the interleaved buffer.
    auto rank_ptr = [&](int k, size_t esize) -> const void* {
        const int q = (owner + 1 + k) % P;
        if (!ilv) return contrib[q];
        return static_cast<const char*>(contrib[0]) + (size_t)q * kIlvPiece * esize;
    };
    if (S > 0 && f32in) {
        RankPtrsF rp{};
        for (int k = 0; k < P; ++k) rp.p[k] = static_cast<const float*>(rank_ptr(k, sizeof(float)));
        const int pow2 = (P & (P - 1)) == 0;
        const float invP = pow2 ? 1.0f / (float)P : 0.0f;
        const bool norm = partial_out != nullptr;
        const uint64_t* slut = p->d_seg_lut;
        const int sshift = p->seg_lut.shift;
        double* wsd = static_cast<double*>(ws);
        with_static_p(P, [&](auto ps) {
            launch_reduce_lc<float, decltype(ps)::value>(norm, lay_lc, false, false, dim3(grid), stream,
                                                         rp, P, invP, pow2, p->d_seg, slut, sshift,
                                                         owner, S, clen, g, wsd);
        });
        if ((rc = launched(who))) return rc;
    } else if (S > 0) {
        RankPtrs rp{};
        for (int k = 0; k < P; ++k) rp.p[k] = static_cast<const uint16_t*>(rank_ptr(k, sizeof(uint16_t)));
        const int pow2 = (P & (P - 1)) == 0;
        const float invP = pow2 ? 1.0f / (float)P : 0.0f;
        const bool norm = partial_out != nullptr;
        const uint64_t* slut = p->d_seg_lut;
        const int sshift = p->seg_lut.shift;
        double* wsd = static_cast<double*>(ws);
        with_static_p<true>(P, [&](auto ps) {
            constexpr int PS = decltype(ps)::value;
            auto lc = [&](auto pc) {
                launch_reduce_lc<uint16_t, decltype(pc)::value>(
                    norm, lay_lc, false, wire16, dim3(grid), stream, rp, P, invP, pow2, p->d_seg, slut,
                    sshift, owner, S, clen, g, wsd);
            };
            auto wide = [&](auto pc) {
                if (burst)
                    launch_reduce_burst<decltype(pc)::value>(norm, lay, wire16, dim3(grid), stream, rp,
                                                             P, invP, pow2, p->d_seg, slut, sshift,
                                                             owner, S, g, wsd);
                else
                    launch_reduce<decltype(pc)::value>(norm, lay, dim3(grid), stream, rp, P, invP,
                                                       pow2, p->d_seg, slut, sshift, owner, nvec, g,
                                                       wsd, false, wire16);
            };
            if constexpr (PS > kLcMaxP) wide(ps);
            else if constexpr (PS > 0) lc(ps);
            else if (P <= kLcMaxP) lc(ps);
            else wide(ps);
        });
        if ((rc = launched(who))) return rc;
    }
    if (partial_out) {
        launch_finalize(static_cast<double*>(ws), S > 0 ? grid : 0, partial_out, stream);
        if ((rc = launched(who))) return rc;
    }
    return GSZ_OK;
}

}  // namespace

extern "C" int gsz_shard_reduce_mean(const gsz_plan* p, int32_t owner,
                                     const uint16_t* const* contrib, int32_t layout, float* g,
                                     double* partial_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, ws_bytes, stream, false, false, "gsz_shard_reduce_mean");
}

extern "C" int gsz_shard_reduce_mean_f32(const gsz_plan* p, int32_t owner,
                                         const float* const* contrib, int32_t layout, float* g,
                                         double* partial_out, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, ws_bytes, stream, false, true, "gsz_shard_reduce_mean_f32");
}

// ------------------------------------------- the allocation-free variant --

// Scratch of gsz_shard_reduce_mean_noalloc: the norm partials of one reduce
// (one fp64 per 2048 shard elements plus the 1024 second-stage sums), for
// shards of up to 2^31 elements.  Each device that runs the library holds its
// own copy for the life of the process.  Host code never passes this name to a
// kernel (on the host it is a stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchMaxShard = (int64_t)1 << 31;
constexpr int64_t kScratchDoubles = kScratchMaxShard / gsz::kRedElems + gsz::kFinalBlocks;
static __device__ __align__(256) double scratch[kScratchDoubles];

namespace {

std::mutex g_scratch_mu;
double* g_scratch_ptr[64];          // per device, set once under g_scratch_mu

// This device's copy of `scratch`, looked up on the first call on the device.
int scratch_for(int dev, double** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("gsz_shard_reduce_mean_noalloc: hipGetSymbolAddress", e);
        g_scratch_ptr[dev] = static_cast<double*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return GSZ_OK;
}

}  // namespace

extern "C" int gsz_shard_reduce_mean_noalloc(const gsz_plan* p, int32_t owner,
                                             const uint16_t* const* contrib, int32_t layout,
                                             float* g, double* partial_out, hipStream_t stream) {
    const char* who = "gsz_shard_reduce_mean_noalloc";
    if (!p) { set_error("%s: NULL plan", who); return GSZ_ERR_INVALID_ARG; }
    if (p->shard_len > kScratchMaxShard) {
        set_error("%s: shard of %lld elements exceeds this variant's limit of %lld (its scratch "
                  "is a fixed array); use gsz_shard_reduce_mean with a workspace",
                  who, (long long)p->shard_len, (long long)kScratchMaxShard);
        return GSZ_ERR_SIZE;
    }
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    double* ws = nullptr;
    if (partial_out && (rc = scratch_for(dev, &ws))) return rc;
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, partial_out ? kScratchDoubles * sizeof(double) : 0, stream,
                       false, false, who);
}

extern "C" int gsz_shard_reduce_mean_bf16_wire(const gsz_plan* p, int32_t owner,
                                               const uint16_t* const* contrib, int32_t layout,
                                               float* g, double* partial_out, void* ws,
                                               size_t ws_bytes, hipStream_t stream) {
    return reduce_impl(p, owner, reinterpret_cast<const void* const*>(contrib), layout, g,
                       partial_out, ws, ws_bytes, stream, true, false,
                       "gsz_shard_reduce_mean_bf16_wire");
}

extern "C" int gsz_shard_grad_sqnorm(const float* g, int64_t n, double* partial_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
    const char* who = "gsz_shard_grad_sqnorm";
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (n < 0 || !partial_out || (n > 0 && !g)) { set_error("%s: bad arguments", who); return GSZ_ERR_INVALID_ARG; }
    size_t need = 0;
    gsz_workspace_bytes(n, &need);
    if (!ws || ws_bytes < need) { set_error("%s: workspace of %zu bytes required", who, need); return GSZ_ERR_SIZE; }
    if (misaligned(ws) || (n > 0 && misaligned(g))) { set_error("%s: misaligned pointer", who); return GSZ_ERR_MISALIGNED; }
    int grid = 0;
    if (n > 0) {
        grid = flat_grid((n + kRedTile - 1) / kRedTile);
        hipLaunchKernelGGL(k_sqnorm, dim3(grid), dim3(kBlock), 0, stream, g, n, static_cast<double*>(ws));
        if ((rc = launched(who))) return rc;
    }
    launch_finalize(static_cast<double*>(ws), grid, partial_out, stream);
    return launched(who);
}

extern "C" int gsz_clip_coef(const double* partials, int32_t n_partials, float max_norm,
                             float* coef_out, float* norm_out, double* total_out,
                             hipStream_t stream) {
    const char* who = "gsz_clip_coef";
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (n_partials < 0 || (n_partials > 0 && !partials) || !coef_out) {
        set_error("%s: bad arguments", who); return GSZ_ERR_INVALID_ARG;
    }
    hipLaunchKernelGGL(k_clip, dim3(1), dim3(64), 0, stream, partials, n_partials, max_norm,
                       coef_out, norm_out, total_out);
    return launched(who);
}

extern "C" int gsz_shard_adamw_step(const gsz_plan* p, int32_t owner, float* master, float* m,
                                    float* v, const float* g, const float* coef,
                                    const gsz_adamw_hp* hp, uint16_t* gathered,
                                    uint16_t* shard_bf16, hipStream_t stream) {
    const char* who = "gsz_shard_adamw_step";
    int rc = check_plan(p, who);
    if (rc) return rc;
    if ((rc = check_owner(p, owner, who))) return rc;
    if (!hp || !coef) { set_error("%s: NULL hyperparameters or coefficient", who); return GSZ_ERR_INVALID_ARG; }
    if (hp->step < 1) { set_error("%s: step must be >= 1", who); return GSZ_ERR_INVALID_ARG; }
    if (!gathered && !shard_bf16) { set_error("%s: need gathered and/or shard_bf16 output", who); return GSZ_ERR_INVALID_ARG; }
    const int64_t S = p->shard_len;
    if (S == 0) return GSZ_OK;
    if (!master || !m || !v || !g) { set_error("%s: NULL state buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(master) || misaligned(m) || misaligned(v) || misaligned(g) ||
        (gathered && misaligned(gathered)) || (shard_bf16 && misaligned(shard_bf16))) {
        set_error("%s: a buffer is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED;
    }
    const AdamScalars s = adam_scalars(*hp);
    const dim3 grid(tile_grid((S + kAdamTile - 1) / kAdamTile, kMaxWorkItems / kAdamBlock));
    const uint64_t* slut = p->d_seg_lut;
    const int sshift = p->seg_lut.shift;
    // The bf16 all-gather stores take 32-bit offsets from each tile's first
    // position unless a tile's positions span 2^31 bytes or more.
    int gwide = gathered && max_tile_span(p, owner, kAdamTile) * 2 >= ((int64_t)1 << 31);
#ifdef GSZ_TEST_HOOKS
    if (g_force_flat_wide.load(std::memory_order_relaxed)) gwide = gathered != nullptr;
#endif
    const int64_t glen = p->flat_len;
    if (gathered && shard_bf16)
        hipLaunchKernelGGL((k_adamw<true, true>), grid, dim3(kAdamBlock), kAdamLdsBytes, stream, master, m, v, g, coef, s, p->d_seg, slut, sshift, (int64_t)owner, S, gathered, glen, gwide, shard_bf16);
    else if (gathered)
        hipLaunchKernelGGL((k_adamw<true, false>), grid, dim3(kAdamBlock), kAdamLdsBytes, stream, master, m, v, g, coef, s, p->d_seg, slut, sshift, (int64_t)owner, S, gathered, glen, gwide, shard_bf16);
    else
        hipLaunchKernelGGL((k_adamw<false, true>), grid, dim3(kAdamBlock), kAdamLdsBytes, stream, master, m, v, g, coef, s, p->d_seg, slut, sshift, (int64_t)owner, S, gathered, glen, gwide, shard_bf16);
    return launched(who);
}

extern "C" int gsz_allgather_layout_write(const gsz_plan* p, int32_t owner,
                                          const uint16_t* shard_bf16, uint16_t* gathered,
                                          hipStream_t stream) {
    const char* who = "gsz_allgather_layout_write";
    int rc = check_plan(p, who);
    if (rc) return rc;
    if ((rc = check_owner(p, owner, who))) return rc;
    const int64_t S = p->shard_len;
    if (S == 0) return GSZ_OK;
    if (!shard_bf16 || !gathered) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(shard_bf16) || misaligned(gathered)) { set_error("%s: misaligned buffer", who); return GSZ_ERR_MISALIGNED; }
    const int64_t nvec = S / 8;
    // The stores take 32-bit offsets from each tile's first all-gather position
    // unless a tile's positions span 2^31 bytes or more.
    int gwide = max_tile_span(p, owner, kRedTile) * 2 >= ((int64_t)1 << 31);
#ifdef GSZ_TEST_HOOKS
    if (g_force_flat_wide.load(std::memory_order_relaxed)) gwide = 1;
#endif
    hipLaunchKernelGGL(k_ag_write, dim3(flat_grid((S + kRedTile - 1) / kRedTile)), dim3(kBlock), 0, stream,
                       shard_bf16, p->d_seg, p->d_seg_lut, p->seg_lut.shift, (int64_t)owner, nvec,
                       gathered, p->flat_len, gwide);
    return launched(who);
}

extern "C" int gsz_bucket_unpack(const gsz_plan* p, const uint16_t* flat, uint16_t* const* params,
                                 hipStream_t stream) {
    return run_pack(p, const_cast<const uint16_t* const*>(params), const_cast<uint16_t*>(flat),
                    kUnpack, stream, "gsz_bucket_unpack");
}

extern "C" int gsz_allreduce_mean(const gsz_plan* p, const uint16_t* const* contrib, float* g_flat,
                                  double* partials, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* who = "gsz_allreduce_mean";
    int rc = check_plan(p, who);
    if (rc) return rc;
    const int P = p->P;
    const int64_t S = p->shard_len;
    if (partials) {
        size_t need = 0;
        gsz_workspace_bytes(S, &need);
        if (!ws || ws_bytes < need) { set_error("%s: workspace of %zu bytes required", who, need); return GSZ_ERR_SIZE; }
        if (misaligned(ws)) { set_error("%s: workspace is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    }
    if (S == 0) {
        if (partials)
            for (int c = 0; c < P; ++c) {
                launch_finalize(static_cast<double*>(ws), 0, partials + c, stream);
                if ((rc = launched(who))) return rc;
            }
        return GSZ_OK;
    }
    if (!g_flat || !contrib) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(g_flat)) { set_error("%s: g_flat is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED; }
    for (int q = 0; q < P; ++q) {
        if (!contrib[q]) { set_error("%s: contribution %d is NULL", who, q); return GSZ_ERR_INVALID_ARG; }
        if (misaligned(contrib[q])) { set_error("%s: contribution %d is not 16-byte aligned", who, q); return GSZ_ERR_MISALIGNED; }
    }
    const int64_t nvec = S / 8;
    const int grid = flat_grid((S + kRedTile - 1) / kRedTile);
    const dim3 gr(grid);
    const int pow2 = (P & (P - 1)) == 0;
    const float invP = pow2 ? 1.0f / (float)P : 0.0f;
    const uint64_t* slut = p->d_seg_lut;
    const int sshift = p->seg_lut.shift;
    const bool norm = partials != nullptr;
    double* wsd = static_cast<double*>(ws);
    const int64_t clen = p->flat_len;
    // chunk c of every bucket, summed in ring order ending at rank c; its norm
    // partial is finalized before the next launch reuses the workspace (stream order)
    for (int c = 0; c < P; ++c) {
        RankPtrs rp{};
        for (int k = 0; k < P; ++k) rp.p[k] = contrib[(c + 1 + k) % P];
        with_static_p<true>(P, [&](auto ps) {
            constexpr int PS = decltype(ps)::value;
            auto lc = [&](auto pc) {
                // g_flat takes 4-byte offsets relative to the tile, like the contributions
                launch_reduce_lc<uint16_t, decltype(pc)::value>(
                    norm, flat_lay_for(p, c, 4), true, false, gr, stream, rp, P, invP, pow2, p->d_seg,
                    slut, sshift, c, S, clen, g_flat, wsd);
            };
            auto wide = [&](auto pc) {
                launch_reduce<decltype(pc)::value>(norm, kLayFlat, gr, stream, rp, P, invP, pow2, p->d_seg,
                                                   slut, sshift, c, nvec, g_flat, wsd, true);
            };
            if constexpr (PS > kLcMaxP) wide(ps);
            else if constexpr (PS > 0) lc(ps);
            else if (P <= kLcMaxP) lc(ps);
            else wide(ps);
        });
        if ((rc = launched(who))) return rc;
        if (norm) {
            launch_finalize(wsd, grid, partials + c, stream);
            if ((rc = launched(who))) return rc;
        }
    }
    return GSZ_OK;
}

extern "C" int gsz_adamw_step(float* master, float* m, float* v, const float* g, int64_t n,
                              const float* coef, const gsz_adamw_hp* hp, uint16_t* out_bf16,
                              hipStream_t stream) {
    const char* who = "gsz_adamw_step";
    int dev = 0;
    int rc = current_device(&dev);
    if (rc) return rc;
    if (!hp || !coef || n < 0) { set_error("%s: bad arguments", who); return GSZ_ERR_INVALID_ARG; }
    if (hp->step < 1) { set_error("%s: step must be >= 1", who); return GSZ_ERR_INVALID_ARG; }
    if (n % 8 != 0) { set_error("%s: n must be a multiple of 8 (got %lld)", who, (long long)n); return GSZ_ERR_SIZE; }
    if (n == 0) return GSZ_OK;
    if (!master || !m || !v || !g || !out_bf16) { set_error("%s: NULL buffer", who); return GSZ_ERR_INVALID_ARG; }
    if (misaligned(master) || misaligned(m) || misaligned(v) || misaligned(g) || misaligned(out_bf16)) {
        set_error("%s: a buffer is not 16-byte aligned", who); return GSZ_ERR_MISALIGNED;
    }
    const AdamScalars s = adam_scalars(*hp);
    const int blocks = tile_grid((n + kAdamTile - 1) / kAdamTile, kMaxWorkItems / kAdamBlock);
    hipLaunchKernelGGL((k_adamw<false, true>), dim3(blocks), dim3(kAdamBlock), kAdamLdsBytes, stream, master, m, v, g,
                       coef, s, nullptr, nullptr, 0, (int64_t)0, n, nullptr, (int64_t)0, 0, out_bf16);
    return launched(who);
}

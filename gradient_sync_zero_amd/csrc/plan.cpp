// Host planner: buckets, padding, chunk ownership, device tables, plan hash.
//
// Rules (see gsz.h, gsz_plan_create): gradients are bucketed in reverse
// compute order ("Data parallelism in depth" §4.2, The Bucket mechanism; "Data
// Parallelism: DDP, ZeRO and FSDP", DDP section: roughly 25 MB buckets, reverse
// layer order); whole tensors only, a bucket closes once its bf16 bytes reach
// the cap; each bucket is zero-padded to a multiple of P*align so it splits
// into P equal chunks ("Data Parallelism: From Parameter Server to Ring
// All-Reduce" §5: the buffer cut into N equal chunks); rank r owns chunk r of
// every bucket.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "gsz_internal.h"

namespace gsz {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
}

const char* last_error() { return g_last_error.c_str(); }

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): offset basis 0xcbf29ce484222325, prime 0x100000001b3.
struct Fnv {
    uint64_t h = 0xcbf29ce484222325ull;
    void add(int64_t x) {
        uint64_t u = (uint64_t)x;
        for (int i = 0; i < 8; ++i) {
            h ^= (u >> (8 * i)) & 0xFFu;
            h *= 0x100000001b3ull;
        }
    }
};

}  // namespace

Lut build_lut(const std::vector<int64_t>& tab, int stride, int offset, int64_t n, int64_t total) {
    Lut lut;
    if (n <= 0 || total <= 0) return lut;
    while (((total - 1) >> lut.shift) + 1 > ((int64_t)1 << kLutCellsLog2)) ++lut.shift;
    const int64_t cells = ((total - 1) >> lut.shift) + 1;
    lut.cells.resize(2 * (size_t)cells);
    auto start = [&](int64_t k) { return tab[(size_t)(k * stride + offset)]; };
    int64_t lo = 0;   // largest k with start(k) <= x; both walks only move forward
    for (int64_t j = 0; j < cells; ++j) {
        const int64_t x = j << lut.shift;
        const int64_t y = std::min(x + ((int64_t)1 << lut.shift), total) - 1;
        while (lo + 1 < n && start(lo + 1) <= x) ++lo;
        int64_t hi = lo;
        while (hi + 1 < n && start(hi + 1) <= y) ++hi;
        lut.cells[2 * (size_t)j] = (int32_t)lo;
        lut.cells[2 * (size_t)j + 1] = (int32_t)hi;
    }
    return lut;
}

}  // namespace gsz

using gsz::set_error;

extern "C" int gsz_plan_create(const int64_t* numel, int32_t n_tensors, int64_t bucket_cap_bytes,
                               int32_t world_size, int32_t align_elems, gsz_plan** out) {
    if (!out) { set_error("gsz_plan_create: out is NULL"); return GSZ_ERR_INVALID_ARG; }
    *out = nullptr;
    if (n_tensors < 0 || (n_tensors > 0 && !numel)) {
        set_error("gsz_plan_create: bad tensor list (n_tensors %d, numel %s)", n_tensors,
                  numel ? "given" : "NULL");
        return GSZ_ERR_INVALID_ARG;
    }
    if (bucket_cap_bytes < 1 || world_size < 1 || world_size > GSZ_MAX_RANKS || align_elems < 1) {
        set_error("gsz_plan_create: got bucket_cap_bytes %lld, world_size %d, align %d; need "
                  "bucket_cap_bytes >= 1, 1 <= world_size <= %d, align >= 1",
                  (long long)bucket_cap_bytes, world_size, align_elems, GSZ_MAX_RANKS);
        return GSZ_ERR_INVALID_ARG;
    }
    // Sizes and offsets stay far from int64 overflow: at most 2^48 elements in
    // all (a 70B model has about 2^36), so padded lengths and byte counts fit.
    const int64_t kMaxTotal = (int64_t)1 << 48;
    int64_t total = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
        if (numel[t] < 0) {
            set_error("gsz_plan_create: tensor %d has negative size %lld", t, (long long)numel[t]);
            return GSZ_ERR_INVALID_ARG;
        }
        if (numel[t] > kMaxTotal - total) {
            set_error("gsz_plan_create: tensor sizes add up past 2^48 elements at tensor %d", t);
            return GSZ_ERR_SIZE;
        }
        total += numel[t];
    }

    gsz_plan* p = new (std::nothrow) gsz_plan();
    if (!p) { set_error("gsz_plan_create: out of host memory"); return GSZ_ERR_NO_MEMORY; }
    try {
        p->numel.assign(numel, numel + n_tensors);
        p->P = world_size;
        p->align = align_elems;
        p->cap = bucket_cap_bytes;
        p->tensor_off.assign(n_tensors, 0);
        p->tensor_bucket.assign(n_tensors, 0);

        const int64_t gran = (int64_t)world_size * align_elems;
        int64_t base = 0, shard_off = 0;
        int32_t t = n_tensors - 1;
        while (t >= 0) {
            gsz::Bucket bk{};
            bk.first_tensor = t;
            bk.base = base;
            int64_t n = 0;
            const int32_t b = (int32_t)p->buckets.size();
            while (t >= 0) {
                p->tensor_off[t] = base + n;
                p->tensor_bucket[t] = b;
                n += p->numel[t];
                ++bk.n_tensors;
                --t;
                if (2 * n >= bucket_cap_bytes) break;   // the bucket reached the cap
            }
            bk.n = n;
            bk.padded = (n + gran - 1) / gran * gran;
            bk.chunk = bk.padded / world_size;
            bk.shard_off = shard_off;
            p->buckets.push_back(bk);
            base += bk.padded;
            shard_off += bk.chunk;
            p->n_params += n;
            p->total_pad += bk.padded - n;
        }
        p->flat_len = base;
        p->shard_len = shard_off;

        gsz::Fnv h;
        h.add(world_size); h.add(align_elems); h.add(bucket_cap_bytes); h.add(n_tensors);
        for (int64_t n : p->numel) h.add(n);
        h.add((int64_t)p->buckets.size());
        for (const auto& bk : p->buckets) {
            h.add(bk.first_tensor); h.add(bk.n_tensors); h.add(bk.base); h.add(bk.n); h.add(bk.padded);
        }
        p->hash = h.h;

        // Device table images.
        const size_t B = p->buckets.size();
        p->seg.reserve(3 * (B + 1));
        for (const auto& bk : p->buckets) {
            p->seg.push_back(bk.shard_off); p->seg.push_back(bk.base); p->seg.push_back(bk.chunk);
        }
        p->seg.push_back(p->shard_len); p->seg.push_back(0); p->seg.push_back(0);

        p->pack.reserve(3 * ((size_t)n_tensors + 1));
        int64_t tiles = 0;
        for (int32_t k = 0; k < n_tensors; ++k) {
            const int32_t tt = n_tensors - 1 - k;
            p->pack.push_back(p->tensor_off[tt]);
            p->pack.push_back(p->numel[tt]);
            p->pack.push_back(tiles);
            tiles += (p->numel[tt] + gsz::kPackTile - 1) / gsz::kPackTile;
        }
        p->pack.push_back(0); p->pack.push_back(0); p->pack.push_back(tiles);

        for (const auto& bk : p->buckets)
            if (bk.padded > bk.n) { p->pads.push_back(bk.base + bk.n); p->pads.push_back(bk.padded - bk.n); }

        p->seg_lut = gsz::build_lut(p->seg, 3, 0, (int64_t)B, p->shard_len);
        p->pack_lut = gsz::build_lut(p->pack, 3, 2, n_tensors, tiles);

        // The device image: seg, pack, pads, the two lookup tables, 2 spare slots.
        const size_t n_slut = p->seg_lut.cells.size() / 2, n_plut = p->pack_lut.cells.size() / 2;
        const size_t fixed = p->seg.size() + p->pack.size() + p->pads.size();
        p->image.reserve(fixed + n_slut + n_plut + 2);
        p->image.insert(p->image.end(), p->seg.begin(), p->seg.end());
        p->image.insert(p->image.end(), p->pack.begin(), p->pack.end());
        p->image.insert(p->image.end(), p->pads.begin(), p->pads.end());
        p->image.resize(fixed + n_slut + n_plut + 2, 0);
        if (n_slut) std::memcpy(p->image.data() + fixed, p->seg_lut.cells.data(), n_slut * 8);
        if (n_plut) std::memcpy(p->image.data() + fixed + n_slut, p->pack_lut.cells.data(), n_plut * 8);
    } catch (const std::bad_alloc&) {
        delete p;
        set_error("gsz_plan_create: out of host memory");
        return GSZ_ERR_NO_MEMORY;
    }
    *out = p;
    return GSZ_OK;
}

extern "C" int gsz_plan_destroy(gsz_plan* p) {
    delete p;          // the device tables live in the caller's memory
    return GSZ_OK;
}

extern "C" int gsz_plan_get_info(const gsz_plan* p, gsz_plan_info* out) {
    if (!p || !out) { set_error("gsz_plan_get_info: NULL argument"); return GSZ_ERR_INVALID_ARG; }
    out->n_tensors = (int32_t)p->numel.size();
    out->n_buckets = (int32_t)p->buckets.size();
    out->world_size = p->P;
    out->align = p->align;
    out->bucket_cap_bytes = p->cap;
    out->flat_len = p->flat_len;
    out->shard_len = p->shard_len;
    out->n_params = p->n_params;
    out->hash = p->hash;
    return GSZ_OK;
}

extern "C" int gsz_plan_bucket(const gsz_plan* p, int32_t b, gsz_bucket_info* out) {
    if (!p || !out) { set_error("gsz_plan_bucket: NULL argument"); return GSZ_ERR_INVALID_ARG; }
    if (b < 0 || b >= (int32_t)p->buckets.size()) {
        set_error("gsz_plan_bucket: bucket %d out of range", b); return GSZ_ERR_INVALID_ARG;
    }
    const auto& bk = p->buckets[b];
    out->first_tensor = bk.first_tensor;
    out->n_tensors = bk.n_tensors;
    out->base = bk.base;
    out->n_elems = bk.n;
    out->padded = bk.padded;
    out->chunk = bk.chunk;
    out->shard_off = bk.shard_off;
    return GSZ_OK;
}

extern "C" int gsz_plan_tensor(const gsz_plan* p, int32_t t, int64_t* flat_offset, int32_t* bucket) {
    if (!p || !flat_offset || !bucket) { set_error("gsz_plan_tensor: NULL argument"); return GSZ_ERR_INVALID_ARG; }
    if (t < 0 || t >= (int32_t)p->numel.size()) {
        set_error("gsz_plan_tensor: tensor %d out of range", t); return GSZ_ERR_INVALID_ARG;
    }
    *flat_offset = p->tensor_off[t];
    *bucket = p->tensor_bucket[t];
    return GSZ_OK;
}

extern "C" int gsz_plan_check(const gsz_plan* p, uint64_t peer_hash) {
    if (!p) { set_error("gsz_plan_check: NULL plan"); return GSZ_ERR_INVALID_ARG; }
    if (p->hash != peer_hash) {
        set_error("gsz_plan_check: bucket plans differ (local %016llx, peer %016llx): ranks would "
                  "issue different collectives", (unsigned long long)p->hash,
                  (unsigned long long)peer_hash);
        return GSZ_ERR_PLAN_MISMATCH;
    }
    return GSZ_OK;
}

extern "C" int gsz_plan_device_bytes(const gsz_plan* p, size_t* out) {
    if (!p || !out) { set_error("gsz_plan_device_bytes: NULL argument"); return GSZ_ERR_INVALID_ARG; }
    *out = p->image.size() * sizeof(int64_t);
    return GSZ_OK;
}

extern "C" int gsz_ledger_bytes_per_param(int32_t P, int32_t zero_stage, double* out) {
    if (!out || P < 1 || zero_stage < 0 || zero_stage > 3) {
        set_error("gsz_ledger_bytes_per_param: need P >= 1, 0 <= zero_stage <= 3, out != NULL");
        return GSZ_ERR_INVALID_ARG;
    }
    // bf16 param 2, bf16 grad 2, fp32 master 4, first moment 4, second moment 4.
    const double param = 2, grad = 2, opt = 12;
    switch (zero_stage) {
        case 0: *out = param + grad + opt; break;
        case 1: *out = param + grad + opt / P; break;
        case 2: *out = param + (grad + opt) / P; break;
        default: *out = (param + grad + opt) / P; break;
    }
    return GSZ_OK;
}

extern "C" int gsz_workspace_bytes(int64_t n, size_t* out) {
    if (!out || n < 0) { set_error("gsz_workspace_bytes: bad argument"); return GSZ_ERR_INVALID_ARG; }
    *out = (size_t)(gsz::red_blocks(n) + gsz::kFinalBlocks) * sizeof(double);
    return GSZ_OK;
}

extern "C" const char* gsz_last_error(void) { return gsz::last_error(); }

extern "C" const char* gsz_status_string(int s) {
    switch (s) {
        case GSZ_OK: return "ok";
        case GSZ_ERR_INVALID_ARG: return "invalid argument";
        case GSZ_ERR_MISALIGNED: return "misaligned device pointer";
        case GSZ_ERR_SIZE: return "size mismatch";
        case GSZ_ERR_BAD_RANK: return "bad rank";
        case GSZ_ERR_PLAN_MISMATCH: return "plan mismatch";
        case GSZ_ERR_NOT_UPLOADED: return "plan not uploaded to this device";
        case GSZ_ERR_DEVICE: return "unsupported device";
        case GSZ_ERR_HIP: return "HIP error";
        case GSZ_ERR_NO_MEMORY: return "out of host memory";
        default: return "unknown status";
    }
}

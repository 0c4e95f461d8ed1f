// Adapter exchange: a residency cache of adapters over a pool.  Adapters
// live packed in host memory (the caller's, ideally pinned) and are copied
// into the pool's slab on demand, on a copy stream, while earlier batches
// run on the compute stream; the least recently used adapter that no
// outstanding batch holds is evicted to make room.  This is the prefetch /
// offload between CPU and GPU memory of the LoRAX pages ("Lorax" tool
// listing, "What is Lorax?": adapter exchange scheduling; "predibase/lorax"
// listing: adapter offloading, just-in-time weight loading).  Adapters are
// read-only, so offloading one drops its device copy and nothing moves back.
//
// The cache is a client of the pool's C ABI (reserve, upload_image,
// unregister); it adds stream ordering:
//   - the compute stream waits for the copies of the adapters it will read
//     (one event recorded on the copy stream after the last copy enqueued);
//   - a copy into an extent freed by an eviction waits for the batches that
//     read the evicted adapter (the fence recorded at their release).
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <deque>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include <hip/hip_runtime.h>

#include "lora_sgmv.h"
#include "sgmv_internal.h"

namespace {

lora_status err(lora_status st, const char *fmt, long long a = 0, long long b = 0) {
    char buf[256];
    snprintf(buf, sizeof buf, fmt, a, b);
    return lora::set_error(st, buf);
}

lora_status hip_err(hipError_t e, const char *what) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
    return lora::set_error(LORA_EHIP, buf);
}

struct Entry {
    int32_t rank = 0;
    float scale = 0.f;
    const void *image = nullptr;
    uint64_t bytes = 0;          // extent bytes: one image copy
    bool resident = false;
    bool held = false;           // named by the outstanding batch
    uint64_t tick = 0;           // last acquire or prefetch that named it
    uint64_t fence = 0;          // last released batch that read it (0: none)
};

}  // namespace

struct lora_cache {
    lora_pool *pool = nullptr;
    hipStream_t copy = nullptr;
    lora_pool_desc desc{};
    std::unordered_map<int32_t, Entry> entries;
    uint64_t tick = 0;
    uint64_t batches = 0;                              // released batches (fence ids 1..)
    std::deque<std::pair<uint64_t, hipEvent_t>> fences;  // pending fences, ascending id
    std::vector<int32_t> held;                         // the outstanding batch's adapters
    bool outstanding = false;
    bool copies_pending = false;                       // copies since the last compute wait
    hipEvent_t copied = nullptr;                       // recorded after the last copies
    int32_t resident = 0;
    uint64_t hits = 0, misses = 0, prefetched = 0, evictions = 0, bytes_up = 0;
};

namespace {

// Drop fences that have completed: waits on them are no-ops.
void prune_fences(lora_cache *c) {
    while (!c->fences.empty() && hipEventQuery(c->fences.front().second) == hipSuccess) {
        (void)hipEventDestroy(c->fences.front().second);
        c->fences.pop_front();
    }
}

hipEvent_t fence_event(lora_cache *c, uint64_t id) {
    for (auto &f : c->fences)
        if (f.first == id) return f.second;
    return nullptr;   // completed and pruned
}

// Evicts the least recently used resident adapter that the outstanding batch
// does not hold and that `keep` does not name; its last fence joins `wait`.
bool evict_one(lora_cache *c, const std::unordered_set<int32_t> &keep,
               std::vector<uint64_t> *wait) {
    int32_t victim = -1;
    uint64_t oldest = UINT64_MAX;
    for (auto &kv : c->entries) {
        const Entry &e = kv.second;
        if (!e.resident || e.held || keep.count(kv.first)) continue;
        if (e.tick < oldest || (e.tick == oldest && kv.first < victim)) {
            oldest = e.tick;
            victim = kv.first;
        }
    }
    if (victim < 0) return false;
    Entry &e = c->entries[victim];
    if (lora_pool_unregister(c->pool, victim) != LORA_OK) return false;
    e.resident = false;
    --c->resident;
    ++c->evictions;
    if (e.fence) wait->push_back(e.fence);
    return true;
}

// Makes `id` resident: reserve (evicting while the pool is full), make the
// copy stream wait for readers of the evicted extents, then copy the image.
// LORA_ENOSPC when nothing more can be evicted.
lora_status bring_in(lora_cache *c, int32_t id, const std::unordered_set<int32_t> &keep) {
    Entry &e = c->entries[id];
    std::vector<uint64_t> wait;
    for (;;) {
        const lora_status st = lora_pool_reserve(c->pool, id, e.rank, e.scale);
        if (st == LORA_OK) break;
        if (st != LORA_ENOSPC) return st;
        if (!evict_one(c, keep, &wait))
            return err(LORA_ENOSPC, "adapter %lld does not fit: every resident adapter is "
                                    "held by the batch (%lld resident)", id, c->resident);
    }
    prune_fences(c);
    std::sort(wait.begin(), wait.end());
    wait.erase(std::unique(wait.begin(), wait.end()), wait.end());
    for (uint64_t f : wait) {
        hipEvent_t ev = fence_event(c, f);
        if (!ev) continue;
        const hipError_t he = hipStreamWaitEvent(c->copy, ev, 0);
        if (he != hipSuccess) {
            (void)lora_pool_unregister(c->pool, id);
            return hip_err(he, "copy stream wait");
        }
    }
    const lora_status st = lora_pool_upload_image(c->pool, id, e.image, 1, c->copy);
    if (st != LORA_OK) {
        (void)lora_pool_unregister(c->pool, id);
        return st;
    }
    e.resident = true;
    ++c->resident;
    c->bytes_up += e.bytes;
    c->copies_pending = true;
    return LORA_OK;
}

}  // namespace

extern "C" {

lora_status lora_cache_create(lora_cache **out, lora_pool *p, void *copy_stream) {
    if (!out || !p) return err(LORA_EINVAL, "null output pointer or pool");
    lora_cache *c = new lora_cache();
    c->pool = p;
    c->copy = static_cast<hipStream_t>(copy_stream);
    lora_status st = lora_pool_get_desc(p, &c->desc);
    if (st != LORA_OK) {
        delete c;
        return st;
    }
    const hipError_t e = hipEventCreateWithFlags(&c->copied, hipEventDisableTiming);
    if (e != hipSuccess) {
        delete c;
        return hip_err(e, "event create");
    }
    *out = c;
    return LORA_OK;
}

lora_status lora_cache_destroy(lora_cache *c) {
    if (!c) return err(LORA_EINVAL, "null cache");
    for (auto &f : c->fences) (void)hipEventDestroy(f.second);
    if (c->copied) (void)hipEventDestroy(c->copied);
    delete c;
    return LORA_OK;
}

lora_status lora_cache_add(lora_cache *c, int32_t id, int32_t rank, float scale,
                           const void *image) {
    if (!c) return err(LORA_EINVAL, "null cache");
    if (id < 0) return err(LORA_EINVAL, "adapter id %lld < 0", id);
    if (!image) return err(LORA_EINVAL, "null image for adapter %lld", id);
    if (rank < 1 || rank > c->desc.r_max)
        return err(LORA_ERANK, "rank %lld not in 1..r_max=%lld", rank, c->desc.r_max);
    if (c->entries.count(id)) return err(LORA_EEXIST, "adapter %lld already added", id);
    if (lora_pool_query(c->pool, id, nullptr, nullptr, nullptr, nullptr) == LORA_OK)
        return err(LORA_EEXIST, "adapter %lld is registered in the pool already", id);
    Entry e;
    e.rank = rank;
    e.scale = scale;
    e.image = image;
    e.bytes = lora_pool_extent_bytes(&c->desc, rank);
    c->entries.emplace(id, e);
    return LORA_OK;
}

lora_status lora_cache_acquire(lora_cache *c, int32_t n, const int32_t *ids, void *compute_stream,
                               int32_t *num_uploaded) {
    if (!c) return err(LORA_EINVAL, "null cache");
    if (c->outstanding) return err(LORA_ESTATE, "the previous batch has not been released");
    if (n < 0 || (n > 0 && !ids)) return err(LORA_EINVAL, "bad id list (n = %lld)", n);
    std::unordered_set<int32_t> batch;
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0) continue;                  // no adapter
        if (!c->entries.count(ids[i])) return err(LORA_ENOENT, "adapter %lld was not added", ids[i]);
        batch.insert(ids[i]);
    }
    ++c->tick;
    int32_t up = 0;
    std::vector<int32_t> order;                    // first-appearance order
    {
        std::unordered_set<int32_t> seen;
        for (int32_t i = 0; i < n; ++i)
            if (ids[i] >= 0 && seen.insert(ids[i]).second) order.push_back(ids[i]);
    }
    for (int32_t id : order) {
        Entry &e = c->entries[id];
        if (e.resident) {
            ++c->hits;
        } else {
            const lora_status st = bring_in(c, id, batch);
            if (st != LORA_OK) return st;      // what was brought in stays resident, unheld
            ++c->misses;
            ++up;
        }
        e.tick = c->tick;
    }
    if (c->copies_pending) {
        hipError_t e = hipEventRecord(c->copied, c->copy);
        if (e == hipSuccess) e = hipStreamWaitEvent(static_cast<hipStream_t>(compute_stream), c->copied, 0);
        if (e != hipSuccess) return hip_err(e, "compute stream wait");
        c->copies_pending = false;
    }
    for (int32_t id : order) c->entries[id].held = true;
    c->held = order;
    c->outstanding = true;
    if (num_uploaded) *num_uploaded = up;
    return LORA_OK;
}

lora_status lora_cache_release(lora_cache *c, void *compute_stream) {
    if (!c) return err(LORA_EINVAL, "null cache");
    if (!c->outstanding) return err(LORA_ESTATE, "no batch is outstanding");
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev, static_cast<hipStream_t>(compute_stream));
    if (e != hipSuccess) {
        if (ev) (void)hipEventDestroy(ev);
        return hip_err(e, "batch fence");
    }
    const uint64_t id = ++c->batches;
    c->fences.emplace_back(id, ev);
    for (int32_t a : c->held) {
        Entry &en = c->entries[a];
        en.held = false;
        en.fence = id;
    }
    c->held.clear();
    c->outstanding = false;
    prune_fences(c);
    return LORA_OK;
}

lora_status lora_cache_prefetch(lora_cache *c, int32_t n, const int32_t *ids,
                                int32_t *num_uploaded) {
    if (!c) return err(LORA_EINVAL, "null cache");
    if (n < 0 || (n > 0 && !ids)) return err(LORA_EINVAL, "bad id list (n = %lld)", n);
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] >= 0 && !c->entries.count(ids[i]))
            return err(LORA_ENOENT, "adapter %lld was not added", ids[i]);
    ++c->tick;
    std::unordered_set<int32_t> keep;
    int32_t up = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = ids[i];
        if (id < 0 || !keep.insert(id).second) continue;
        Entry &e = c->entries[id];
        e.tick = c->tick;
        if (e.resident) continue;
        const lora_status st = bring_in(c, id, keep);
        if (st == LORA_ENOSPC) break;              // full of held or just-fetched adapters
        if (st != LORA_OK) return st;
        ++c->prefetched;
        ++up;
    }
    if (num_uploaded) *num_uploaded = up;
    return LORA_OK;
}

lora_status lora_cache_query(const lora_cache *c, int32_t id, int32_t *resident, int32_t *held) {
    if (!c) return err(LORA_EINVAL, "null cache");
    auto it = c->entries.find(id);
    if (it == c->entries.end()) return err(LORA_ENOENT, "adapter %lld was not added", id);
    if (resident) *resident = it->second.resident ? 1 : 0;
    if (held) *held = it->second.held ? 1 : 0;
    return LORA_OK;
}

lora_status lora_cache_stats(const lora_cache *c, int32_t *resident, uint64_t *hits,
                             uint64_t *misses, uint64_t *prefetched, uint64_t *evictions,
                             uint64_t *bytes_uploaded) {
    if (!c) return err(LORA_EINVAL, "null cache");
    if (resident) *resident = c->resident;
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (prefetched) *prefetched = c->prefetched;
    if (evictions) *evictions = c->evictions;
    if (bytes_uploaded) *bytes_uploaded = c->bytes_up;
    return LORA_OK;
}

}  // extern "C"

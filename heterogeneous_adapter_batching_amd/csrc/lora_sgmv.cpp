// Host side of the multi-adapter LoRA delta library: the adapter pool (slot
// table and extent allocator over a caller-owned HBM slab), the gather plan
// of a heterogeneous batch, and the C ABI declared in include/lora_sgmv.h.
//
// Nothing here allocates device memory.  Validation happens before anything
// is enqueued, so an error leaves every object as it was.
#include <algorithm>
#include <cmath>
#include <climits>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include <hip/hip_runtime.h>

#include "lora_sgmv.h"
#include "sgmv_internal.h"

using lora::BlockDesc;

namespace {

thread_local std::string g_last_error;

lora_status fail(lora_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

lora_status hip_fail(hipError_t e, const char *what) {
    return fail(LORA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

uint64_t round_up(uint64_t v, uint64_t m) { return (v + m - 1) / m * m; }

int32_t esize(int32_t dtype) { return dtype == LORA_BF16 ? 2 : 4; }

lora_status check_desc(const lora_pool_desc *d) {
    if (!d) return fail(LORA_EINVAL, "null pool descriptor");
    if (d->dtype != LORA_F32 && d->dtype != LORA_BF16)
        return fail(LORA_EDTYPE, "dtype %d is neither LORA_F32 nor LORA_BF16", d->dtype);
    if (d->num_layers < 1) return fail(LORA_EINVAL, "num_layers %d < 1", d->num_layers);
    if (d->num_proj < 1 || d->num_proj > LORA_MAX_PROJ)
        return fail(LORA_EINVAL, "num_proj %d not in 1..%d", d->num_proj, LORA_MAX_PROJ);
    for (int p = 0; p < d->num_proj; ++p) {
        if (d->h_in[p] < 8 || d->h_in[p] % 8 || d->h_out[p] < 8 || d->h_out[p] % 8)
            return fail(LORA_EINVAL, "projection %d: h_in %d / h_out %d must be positive "
                        "multiples of 8", p, d->h_in[p], d->h_out[p]);
    }
    if (d->rank_granule < 8 || d->rank_granule % 8)
        return fail(LORA_EINVAL, "rank_granule %d must be a positive multiple of 8",
                    d->rank_granule);
    if (d->r_max < 1 || d->r_max > LORA_MAX_RANK || d->r_max % d->rank_granule)
        return fail(LORA_EINVAL, "r_max %d must be a multiple of rank_granule %d and <= %d",
                    d->r_max, d->rank_granule, LORA_MAX_RANK);
    if (d->max_slots < 1) return fail(LORA_EINVAL, "max_slots %d < 1", d->max_slots);
    return LORA_OK;
}

// sum over projections of (h_in + h_out): the per-rank, per-layer element count
int64_t row_elems(const lora_pool_desc *d) {
    int64_t w = 0;
    for (int p = 0; p < d->num_proj; ++p) w += int64_t(d->h_in[p]) + d->h_out[p];
    return w;
}

// K elements of one 16-byte fragment over the 4 lane groups of an MFMA:
// A is stored in blocks of this many columns (see lora_pool_create)
int32_t kspan(int32_t dtype) { return dtype == LORA_BF16 ? 32 : 16; }

int64_t h_in_pad(const lora_pool_desc *d, int p) {
    return int64_t(round_up(uint64_t(d->h_in[p]), uint64_t(kspan(d->dtype))));
}

// the same sum with h_in padded to whole K-blocks: the stored layout
int64_t stored_row_elems(const lora_pool_desc *d) {
    int64_t w = 0;
    for (int p = 0; p < d->num_proj; ++p) w += h_in_pad(d, p) + d->h_out[p];
    return w;
}

int32_t pad_rank(const lora_pool_desc *d, int32_t r) {
    return int32_t(round_up(uint64_t(r), uint64_t(d->rank_granule)));
}

}  // namespace

struct Slot {
    int32_t rank;
    int32_t r_pad;
    float scale;
    uint64_t off;
    uint64_t bytes;
};

struct lora_pool {
    lora_pool_desc d;
    uint8_t *slab;
    uint64_t slab_bytes;
    std::unordered_map<int32_t, Slot> slots;
    std::map<uint64_t, uint64_t> free_list;  // offset -> bytes, coalesced
    uint64_t generation = 0;                  // bumped by unregister
    int64_t W = 0;                            // stored_row_elems(d)
    int64_t pre[LORA_MAX_PROJ + 1] = {};      // prefix of (h_in_pad + h_out) over projections

    // element offset multipliers of the A and B blocks of (layer, proj), in
    // units of r_pad elements
    int64_t coef_a(int layer, int p) const { return int64_t(layer) * W + pre[p]; }
    int64_t coef_b(int layer, int p) const { return coef_a(layer, p) + h_in_pad(&d, p); }

    bool alloc(uint64_t bytes, uint64_t *off) {
        for (auto it = free_list.begin(); it != free_list.end(); ++it) {
            if (it->second >= bytes) {
                *off = it->first;
                const uint64_t rest = it->second - bytes;
                const uint64_t roff = it->first + bytes;
                free_list.erase(it);
                if (rest) free_list.emplace(roff, rest);
                return true;
            }
        }
        return false;
    }

    void release(uint64_t off, uint64_t bytes) {
        auto it = free_list.emplace(off, bytes).first;
        auto nx = std::next(it);
        if (nx != free_list.end() && it->first + it->second == nx->first) {
            it->second += nx->second;
            free_list.erase(nx);
        }
        if (it != free_list.begin()) {
            auto pv = std::prev(it);
            if (pv->first + pv->second == it->first) {
                pv->second += it->second;
                free_list.erase(it);
            }
        }
    }
};

struct lora_plan {
    const lora_pool *pool = nullptr;
    uint64_t pool_generation = 0;
    int32_t T = 0;
    std::vector<int32_t> token_order;    // plan order: grouped adapter tokens, then the rest
    std::vector<int32_t> token_sigma;    // core index per plan-order row (-1: none)
    std::vector<float> token_weight;     // weight per plan-order row (weighted plans)
    bool weighted = false;
    int32_t max_sigma = -1;              // largest core index named
    std::vector<int32_t> token_group;    // per token row
    std::vector<int32_t> group_adapter, group_rank;
    // adapter blocks [0, nb_act): the long groups' [0, nb_long), then the
    // short groups' by padded rank; no-adapter blocks after
    std::vector<BlockDesc> blocks;
    int32_t nb_long = 0;
    std::vector<lora::TileDesc> tiles;   // rank tiles of the adapter blocks, in block order
    int32_t nb_act = 0, n_active = 0, max_block = 0, tt = 1, max_rpad = 0;

    // device image in the caller's workspace
    void *ws = nullptr;
    uint64_t ws_bytes = 0;
    int32_t max_proj = 0;
    uint64_t off_tok = 0, off_blocks = 0, off_tiles = 0, off_btok = 0, off_ttok = 0, off_tsig = 0,
             off_tw = 0, off_part = 0;
    uint64_t image_bytes = 0, part_bytes = 0;
    void *staging = nullptr;
    uint64_t staging_bytes = 0;
    hipEvent_t staged = nullptr;
    // the call whose shrink partials the workspace holds (sgmv_shrink_partials):
    // layer, projections and k-chunks; part_layer -1 = none
    mutable int32_t part_layer = -1, part_nproj = 0, part_c0 = 0;
    mutable int32_t part_projs[LORA_MAX_PROJ] = {};

    int32_t rt_total() const { return int32_t(tiles.size()); }
    int32_t nb_all() const { return int32_t(blocks.size()); }

    void layout(int32_t mp) {
        uint64_t o = 0;
        off_tok = o;     o = round_up(o + 4ull * std::max(T, 1), 256);
        off_blocks = o;  o = round_up(o + sizeof(BlockDesc) * std::max(nb_all(), 1), 256);
        off_tiles = o;   o = round_up(o + sizeof(lora::TileDesc) * std::max(rt_total(), 1), 256);
        off_btok = o;    o = round_up(o + 4ull * lora::kMaxBlockTokens * std::max(nb_all(), 1), 256);
        off_ttok = o;    o = round_up(o + 4ull * lora::kMaxBlockTokens * std::max(rt_total(), 1), 256);
        off_tsig = o;    o = round_up(o + 4ull * std::max(T, 1), 256);
        off_tw = o;      o = round_up(o + 4ull * std::max(T, 1), 256);
        image_bytes = o;
        part_bytes = 4ull * max_shrink_units(mp) * tt * lora::kTile * lora::kTile;
        off_part = o;    o = round_up(o + part_bytes, 256);
        ws_bytes = o;
    }

    // Most partial tiles of a shrink of up to mp projections under
    // shrink_geometry: nproj * rt_total * c0, with c0 at most
    // max(ceil(target / per_chunk), ceil(steps / frags)), where steps =
    // fragments of 4 waves over h_in.
    uint64_t max_shrink_units(int32_t mp) const {
        const lora_pool_desc &d = pool->d;
        const uint64_t span = 4ull * (16 / esize(d.dtype));
        int32_t h_in_max = 0;
        for (int i = 0; i < d.num_proj; ++i) h_in_max = std::max(h_in_max, d.h_in[i]);
        const uint64_t steps = (h_in_max + lora::kWaves * span - 1) / (lora::kWaves * span);
        const uint64_t frags = tt <= 2 ? lora::shrink_frags<1>() : lora::shrink_frags<4>();
        const uint64_t by_frags = (steps + frags - 1) / frags;
        uint64_t most = 0;
        const uint64_t rt = std::max(rt_total(), 1);
        for (int32_t np = 1; np <= mp; ++np) {
            // partial tiles = np * rt * c0, c0 from the workgroups per chunk:
            // np * rt, or rt for units over every projection (tt >= 2)
            const uint64_t per_chunk = (tt >= 2 && np > 1 && np <= 3 ? 1 : uint64_t(np)) * rt;
            const uint64_t by_target = (lora::kShrinkTargetGroups + per_chunk - 1) / per_chunk;
            most = std::max(most, uint64_t(np) * rt * std::max(by_target, by_frags));
        }
        return most;
    }
};

namespace {

// Host copy of one A block into its K-blocked place: A [rank][h_in] row-major
// -> dst [h_in_pad / span][r_pad][span]; dst is zero already.
void pack_a_host(const uint8_t *src, int32_t rank, uint64_t h_in, uint64_t hp, uint64_t span,
                 int32_t r_pad, uint64_t es, uint8_t *dst) {
    for (uint64_t kb = 0; kb < hp / span; ++kb) {
        const uint64_t cols = std::min<uint64_t>(span, h_in - std::min(h_in, kb * span));
        if (!cols) break;
        for (uint64_t j = 0; j < uint64_t(rank); ++j)
            std::memcpy(dst + ((kb * r_pad + j) * span) * es, src + (j * h_in + kb * span) * es,
                        cols * es);
    }
}

}  // namespace

namespace lora {
lora_status set_error(lora_status st, const char *msg) {
    g_last_error = msg;
    return st;
}
}  // namespace lora

// ------------------------------------------------------------------ C ABI ----
extern "C" {

const char *lora_last_error(void) { return g_last_error.c_str(); }

uint64_t lora_adapter_bytes(const lora_pool_desc *d, int32_t rank) {
    if (check_desc(d) != LORA_OK || rank < 1) return 0;
    return uint64_t(rank) * esize(d->dtype) * uint64_t(d->num_layers) * uint64_t(row_elems(d));
}

uint64_t lora_pool_extent_bytes(const lora_pool_desc *d, int32_t rank) {
    if (check_desc(d) != LORA_OK || rank < 1 || rank > d->r_max) return 0;
    return round_up(uint64_t(pad_rank(d, rank)) * esize(d->dtype) * uint64_t(d->num_layers) *
                    uint64_t(stored_row_elems(d)), 256);
}

lora_status lora_pool_create(lora_pool **out, const lora_pool_desc *d, void *slab,
                             uint64_t slab_bytes) {
    if (!out) return fail(LORA_EINVAL, "null output pointer");
    lora_status st = check_desc(d);
    if (st != LORA_OK) return st;
    if (!slab || (reinterpret_cast<uintptr_t>(slab) & 255))
        return fail(LORA_EINVAL, "slab must be a non-null, 256-byte aligned device pointer");
    lora_pool *p = new lora_pool();
    p->d = *d;
    p->slab = static_cast<uint8_t *>(slab);
    p->slab_bytes = slab_bytes / 256 * 256;
    if (p->slab_bytes) p->free_list.emplace(0, p->slab_bytes);
    p->W = stored_row_elems(d);
    for (int i = 0; i < d->num_proj; ++i) p->pre[i + 1] = p->pre[i] + h_in_pad(d, i) + d->h_out[i];
    *out = p;
    return LORA_OK;
}

lora_status lora_pool_destroy(lora_pool *p) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    delete p;
    return LORA_OK;
}

lora_status lora_pool_reserve(lora_pool *p, int32_t id, int32_t rank, float scale) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    if (id < 0) return fail(LORA_EINVAL, "adapter id %d < 0", id);
    if (rank < 1 || rank > p->d.r_max)
        return fail(LORA_ERANK, "rank %d not in 1..r_max=%d", rank, p->d.r_max);
    if (p->slots.count(id)) return fail(LORA_EEXIST, "adapter %d already registered", id);
    if (int32_t(p->slots.size()) >= p->d.max_slots)
        return fail(LORA_ENOSPC, "all %d slots in use", p->d.max_slots);
    const uint64_t bytes = lora_pool_extent_bytes(&p->d, rank);
    uint64_t off = 0;
    if (!p->alloc(bytes, &off))
        return fail(LORA_ENOSPC, "no free extent of %llu bytes in the slab",
                    (unsigned long long)bytes);
    p->slots.emplace(id, Slot{rank, pad_rank(&p->d, rank), scale, off, bytes});
    return LORA_OK;
}

lora_status lora_pool_upload(lora_pool *p, int32_t id, int32_t layer, int32_t proj,
                             const void *A, const void *B, int32_t src_on_host, void *stream) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    auto it = p->slots.find(id);
    if (it == p->slots.end()) return fail(LORA_ENOENT, "adapter %d not registered", id);
    if (layer < 0 || layer >= p->d.num_layers)
        return fail(LORA_EINVAL, "layer %d not in 0..%d", layer, p->d.num_layers - 1);
    if (proj < 0 || proj >= p->d.num_proj)
        return fail(LORA_EINVAL, "projection %d not in 0..%d", proj, p->d.num_proj - 1);
    if (!A || !B) return fail(LORA_EINVAL, "null weight pointer");
    if (!src_on_host && ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(B) & 15)))
        return fail(LORA_EINVAL, "device weight sources must be 16-byte aligned");
    const Slot &s = it->second;
    const uint64_t es = esize(p->d.dtype);
    const uint64_t h_in = p->d.h_in[proj], h_out = p->d.h_out[proj];
    const uint64_t span = kspan(p->d.dtype), hp = h_in_pad(&p->d, proj);
    uint8_t *a_dst = p->slab + s.off + uint64_t(s.r_pad) * es * p->coef_a(layer, proj);
    uint8_t *b_dst = p->slab + s.off + uint64_t(s.r_pad) * es * p->coef_b(layer, proj);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipMemcpyKind kind = src_on_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice;
    // A goes K-blocked: [h_in_pad / span][r_pad][span], zero padded, so the 16
    // rows x span columns one MFMA fragment reads are contiguous
    const uint64_t a_bytes = uint64_t(s.r_pad) * hp * es;
    hipError_t e;
    std::vector<uint8_t> a_blk;
    if (src_on_host) {
        a_blk.assign(a_bytes, 0);
        pack_a_host(static_cast<const uint8_t *>(A), s.rank, h_in, hp, span, s.r_pad, es,
                    a_blk.data());
        e = hipMemcpyAsync(a_dst, a_blk.data(), a_bytes, kind, st);
    } else {
        e = lora::launch_pack_a(p->d.dtype, A, s.rank, int32_t(h_in), a_dst, s.r_pad,
                                int32_t(hp), st);
    }
    if (e != hipSuccess) return hip_fail(e, "A upload");
    const uint64_t b_bytes = h_out * uint64_t(s.r_pad) * es;
    std::vector<uint8_t> padded;   // host source with padding: widen rows on the host
    if (s.r_pad == s.rank) {
        e = hipMemcpyAsync(b_dst, B, b_bytes, kind, st);
    } else if (src_on_host) {
        padded.assign(b_bytes, 0);
        const uint8_t *src = static_cast<const uint8_t *>(B);
        for (uint64_t o = 0; o < h_out; ++o)
            std::memcpy(padded.data() + o * s.r_pad * es, src + o * s.rank * es, s.rank * es);
        e = hipMemcpyAsync(b_dst, padded.data(), b_bytes, kind, st);
    } else {
        e = hipMemset2DAsync(b_dst + uint64_t(s.rank) * es, uint64_t(s.r_pad) * es, 0,
                             uint64_t(s.r_pad - s.rank) * es, h_out, st);
        if (e != hipSuccess) return hip_fail(e, "B pad columns");
        e = hipMemcpy2DAsync(b_dst, uint64_t(s.r_pad) * es, B, uint64_t(s.rank) * es,
                             uint64_t(s.rank) * es, h_out, kind, st);
    }
    if (e != hipSuccess) return hip_fail(e, "B upload");
    if (src_on_host) {
        e = hipStreamSynchronize(st);   // host sources must be consumed before returning
        if (e != hipSuccess) return hip_fail(e, "upload synchronize");
    }
    return LORA_OK;
}

lora_status lora_pool_unregister(lora_pool *p, int32_t id) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    auto it = p->slots.find(id);
    if (it == p->slots.end()) return fail(LORA_ENOENT, "adapter %d not registered", id);
    p->release(it->second.off, it->second.bytes);
    p->slots.erase(it);
    ++p->generation;
    return LORA_OK;
}

lora_status lora_pool_register(lora_pool *p, int32_t id, int32_t rank, float scale,
                               const void *const *A, const void *const *B,
                               int32_t src_on_host, void *stream) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    if (!A || !B) return fail(LORA_EINVAL, "null weight array");
    for (int i = 0; i < p->d.num_proj; ++i)
        if (!A[i] || !B[i]) return fail(LORA_EINVAL, "null weights for projection %d", i);
    lora_status st = lora_pool_reserve(p, id, rank, scale);
    if (st != LORA_OK) return st;
    const uint64_t es = esize(p->d.dtype);
    for (int l = 0; l < p->d.num_layers; ++l) {
        for (int i = 0; i < p->d.num_proj; ++i) {
            const uint8_t *a = static_cast<const uint8_t *>(A[i]) +
                               uint64_t(l) * rank * p->d.h_in[i] * es;
            const uint8_t *b = static_cast<const uint8_t *>(B[i]) +
                               uint64_t(l) * p->d.h_out[i] * rank * es;
            st = lora_pool_upload(p, id, l, i, a, b, src_on_host, stream);
            if (st != LORA_OK) {
                std::string msg = g_last_error;
                auto it = p->slots.find(id);   // undo the reservation (not a generation bump)
                p->release(it->second.off, it->second.bytes);
                p->slots.erase(it);
                g_last_error = msg;
                return st;
            }
        }
    }
    return LORA_OK;
}

lora_status lora_pack_adapter(const lora_pool_desc *d, int32_t rank, const void *const *A,
                              const void *const *B, void *image, uint64_t image_bytes) {
    lora_status st = check_desc(d);
    if (st != LORA_OK) return st;
    if (rank < 1 || rank > d->r_max)
        return fail(LORA_ERANK, "rank %d not in 1..r_max=%d", rank, d->r_max);
    if (!A || !B || !image) return fail(LORA_EINVAL, "null weight array or image");
    for (int i = 0; i < d->num_proj; ++i)
        if (!A[i] || !B[i]) return fail(LORA_EINVAL, "null weights for projection %d", i);
    const uint64_t need = lora_pool_extent_bytes(d, rank);
    if (image_bytes < need)
        return fail(LORA_EINVAL, "image of %llu bytes < extent of %llu",
                    (unsigned long long)image_bytes, (unsigned long long)need);
    const uint64_t es = esize(d->dtype), span = kspan(d->dtype);
    const int32_t r_pad = pad_rank(d, rank);
    const uint64_t W = uint64_t(stored_row_elems(d));
    uint8_t *img = static_cast<uint8_t *>(image);
    std::memset(img, 0, need);
    for (int l = 0; l < d->num_layers; ++l) {
        uint64_t pre = 0;   // (h_in_pad + h_out) of the projections before p
        for (int i = 0; i < d->num_proj; ++i) {
            const uint64_t h_in = d->h_in[i], h_out = d->h_out[i], hp = h_in_pad(d, i);
            uint8_t *a_dst = img + uint64_t(r_pad) * es * (uint64_t(l) * W + pre);
            uint8_t *b_dst = a_dst + uint64_t(r_pad) * es * hp;
            pack_a_host(static_cast<const uint8_t *>(A[i]) + uint64_t(l) * rank * h_in * es,
                        rank, h_in, hp, span, r_pad, es, a_dst);
            const uint8_t *b = static_cast<const uint8_t *>(B[i]) + uint64_t(l) * h_out * rank * es;
            for (uint64_t o = 0; o < h_out; ++o)
                std::memcpy(b_dst + o * r_pad * es, b + o * rank * es, rank * es);
            pre += hp + h_out;
        }
    }
    return LORA_OK;
}

lora_status lora_pool_upload_image(lora_pool *p, int32_t id, const void *image,
                                   int32_t src_on_host, void *stream) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    if (!image) return fail(LORA_EINVAL, "null image");
    auto it = p->slots.find(id);
    if (it == p->slots.end()) return fail(LORA_ENOENT, "adapter %d not registered", id);
    if (!src_on_host && (reinterpret_cast<uintptr_t>(image) & 15))
        return fail(LORA_EINVAL, "device images must be 16-byte aligned");
    const hipError_t e = hipMemcpyAsync(
        p->slab + it->second.off, image, it->second.bytes,
        src_on_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "image upload");
    return LORA_OK;
}

lora_status lora_pool_register_image(lora_pool *p, int32_t id, int32_t rank, float scale,
                                     const void *image, int32_t src_on_host, void *stream) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    if (!image) return fail(LORA_EINVAL, "null image");
    lora_status st = lora_pool_reserve(p, id, rank, scale);
    if (st != LORA_OK) return st;
    st = lora_pool_upload_image(p, id, image, src_on_host, stream);
    if (st != LORA_OK) {
        std::string msg = g_last_error;
        auto it = p->slots.find(id);   // undo the reservation (not a generation bump)
        p->release(it->second.off, it->second.bytes);
        p->slots.erase(it);
        g_last_error = msg;
    }
    return st;
}

lora_status lora_pool_get_desc(const lora_pool *p, lora_pool_desc *d) {
    if (!p || !d) return fail(LORA_EINVAL, "null pool or descriptor");
    *d = p->d;
    return LORA_OK;
}

lora_status lora_pool_query(const lora_pool *p, int32_t id, int32_t *rank, int32_t *r_pad,
                            float *scale, uint64_t *off) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    auto it = p->slots.find(id);
    if (it == p->slots.end()) return fail(LORA_ENOENT, "adapter %d not registered", id);
    if (rank) *rank = it->second.rank;
    if (r_pad) *r_pad = it->second.r_pad;
    if (scale) *scale = it->second.scale;
    if (off) *off = it->second.off;
    return LORA_OK;
}

lora_status lora_pool_stats(const lora_pool *p, int32_t *num, uint64_t *free_bytes) {
    if (!p) return fail(LORA_EINVAL, "null pool");
    if (num) *num = int32_t(p->slots.size());
    if (free_bytes) {
        uint64_t f = 0;
        for (auto &kv : p->free_list) f += kv.second;
        *free_bytes = f;
    }
    return LORA_OK;
}

// ------------------------------------------------------------------- plan ----
}  // extern "C"

namespace {
lora_status plan_create(lora_plan **out, const lora_pool *p, int32_t T, const int32_t *seg_starts,
                        const int32_t *seg_adapter, const int32_t *seg_sigma,
                        const float *seg_weight, int32_t S) {
    if (!out) return fail(LORA_EINVAL, "null output pointer");
    if (!p) return fail(LORA_EINVAL, "null pool");
    if (T < 0 || S < 0) return fail(LORA_ESEG, "negative token or segment count");
    if (!seg_starts || (S > 0 && !seg_adapter)) return fail(LORA_EINVAL, "null segment table");
    if (seg_starts[0] != 0) return fail(LORA_ESEG, "seg_starts[0] = %d, not 0", seg_starts[0]);
    if (seg_starts[S] != T)
        return fail(LORA_ESEG, "seg_starts[%d] = %d, not num_tokens %d", S, seg_starts[S], T);
    for (int32_t s = 0; s < S; ++s) {
        if (seg_starts[s + 1] < seg_starts[s])
            return fail(LORA_ESEG, "seg_starts decreases at segment %d", s);
        const int32_t id = seg_adapter[s];
        if (id < -1) return fail(LORA_ENOENT, "segment %d names adapter id %d", s, id);
        if (id >= 0 && !p->slots.count(id))
            return fail(LORA_ENOENT, "segment %d names unregistered adapter %d", s, id);
        if (seg_sigma && seg_sigma[s] < -1)
            return fail(LORA_EINVAL, "segment %d names core %d", s, seg_sigma[s]);
        if (seg_weight && !std::isfinite(seg_weight[s]))
            return fail(LORA_EINVAL, "segment %d has a weight that is not finite", s);
    }

    lora_plan *pl = new lora_plan();
    pl->pool = p;
    pl->pool_generation = p->generation;
    pl->T = T;
    pl->token_group.assign(T, -1);

    // groups in first-appearance order (segments with tokens only)
    std::unordered_map<int32_t, int32_t> gidx;
    std::vector<std::vector<int32_t>> members;
    for (int32_t s = 0; s < S; ++s) {
        const int32_t id = seg_adapter[s];
        if (id < 0 || seg_starts[s + 1] == seg_starts[s]) continue;
        auto it = gidx.find(id);
        int32_t g;
        if (it == gidx.end()) {
            g = int32_t(members.size());
            gidx.emplace(id, g);
            members.emplace_back();
            pl->group_adapter.push_back(id);
            pl->group_rank.push_back(p->slots.at(id).rank);
        } else {
            g = it->second;
        }
        for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) {
            members[g].push_back(t);
            pl->token_group[t] = g;
        }
    }
    std::vector<int32_t> idle;
    for (int32_t t = 0; t < T; ++t)
        if (pl->token_group[t] < 0) idle.push_back(t);

    // Two levels of blocks.  Shrink blocks: each group cut into near-equal
    // blocks of at most one 16-token tile (64 tokens, 4 tiles, for a long
    // group); the shrink reads the adapter's A once per shrink block and per
    // 16-rank tile of it (the rank tiles are its units).  Expand blocks: a
    // short group's shrink blocks are cut again into near-equal blocks of at
    // most kDecodeBlockTokens tokens, so that the decode expand's units move
    // about the same bytes whatever a group's size; a long group's are its
    // shrink blocks, for the MFMA expand.  An expand block names its shrink
    // block's first rank tile and its first token slot in it.
    size_t long_tokens = 0;
    for (auto &m : members)
        if (m.size() >= size_t(lora::kLongGroup)) long_tokens += m.size();
    const bool use_long = long_tokens >= size_t(lora::kMinLongTokens);
    std::vector<BlockDesc> long_blocks, short_blocks;
    auto cut = [](int32_t n, int32_t m, std::vector<int32_t> *sizes) {
        sizes->clear();
        const int32_t k = (n + m - 1) / m;
        for (int32_t i = 0; i < k; ++i) sizes->push_back(n / k + (i < n % k ? 1 : 0));
    };
    int32_t max_sblock = 0;
    std::vector<int32_t> ssz, esz;
    auto add_group = [&](const std::vector<int32_t> &toks, int32_t g, const Slot *sl) {
        const int32_t base = int32_t(pl->token_order.size());
        const int32_t rt = sl ? (sl->r_pad + lora::kTile - 1) / lora::kTile : 0;
        const bool lg = sl && use_long && toks.size() >= size_t(lora::kLongGroup);
        const int32_t smax = lg ? lora::kMaxBlockTokens : lora::kTile;
        const int32_t emax = lg ? lora::kMaxBlockTokens : lora::kDecodeBlockTokens;
        cut(int32_t(toks.size()), smax, &ssz);
        int32_t s0 = 0;
        for (int32_t sn : ssz) {
            const int32_t rt_before = int32_t(pl->tiles.size());
            for (int32_t i = 0; i < rt; ++i) {
                lora::TileDesc td{};
                td.tok_off = base + s0;
                td.n_tok = sn;
                td.r_pad = sl->r_pad;
                td.tile = i;
                td.block = g;
                td.ext_lo = uint32_t(sl->off & 0xffffffffu);
                td.ext_hi = uint32_t(sl->off >> 32);
                pl->tiles.push_back(td);
            }
            max_sblock = std::max(max_sblock, sn);
            cut(sn, emax, &esz);
            int32_t e0 = 0;
            for (int32_t en : esz) {
                BlockDesc bd{};
                bd.tok_off = base + s0 + e0;
                bd.n_tok = en;
                bd.r_pad = sl ? sl->r_pad : 0;
                bd.slot0 = e0;
                bd.scale = sl ? sl->scale : 0.f;
                bd.rt_before = rt_before;
                bd.ext_lo = sl ? uint32_t(sl->off & 0xffffffffu) : 0u;
                bd.ext_hi = sl ? uint32_t(sl->off >> 32) : 0u;
                (lg ? long_blocks : short_blocks).push_back(bd);
                pl->max_block = std::max(pl->max_block, en);
                e0 += en;
            }
            s0 += sn;
        }
        pl->token_order.insert(pl->token_order.end(), toks.begin(), toks.end());
    };
    for (int32_t g = 0; g < int32_t(members.size()); ++g)
        add_group(members[g], g, &p->slots.at(pl->group_adapter[g]));
    // The decode expand visits the short blocks by padded rank, largest first
    // (stable within a rank): its units are equal in bytes within a rank, the
    // costliest are dealt first, and the rank is uniform over a range of units.
    std::stable_sort(short_blocks.begin(), short_blocks.end(),
                     [](const BlockDesc &x, const BlockDesc &y) { return x.r_pad > y.r_pad; });
    pl->blocks = long_blocks;
    pl->blocks.insert(pl->blocks.end(), short_blocks.begin(), short_blocks.end());
    pl->nb_long = int32_t(long_blocks.size());
    pl->nb_act = int32_t(pl->blocks.size());
    pl->n_active = int32_t(pl->token_order.size());
    short_blocks.clear();
    add_group(idle, -1, nullptr);
    pl->blocks.insert(pl->blocks.end(), short_blocks.begin(), short_blocks.end());
    for (int32_t b = 0; b < pl->nb_act; ++b)
        pl->max_rpad = std::max(pl->max_rpad, pl->blocks[b].r_pad);
    const int32_t tiles = (std::max(max_sblock, pl->max_block) + lora::kTile - 1) / lora::kTile;
    pl->tt = tiles <= 1 ? 1 : tiles == 2 ? 2 : 4;
    // each row's core, in plan order
    std::vector<int32_t> row_sigma(T, -1);
    if (seg_sigma)
        for (int32_t s = 0; s < S; ++s)
            for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) row_sigma[t] = seg_sigma[s];
    pl->token_sigma.resize(T);
    for (int32_t i = 0; i < T; ++i) {
        pl->token_sigma[i] = row_sigma[pl->token_order[i]];
        pl->max_sigma = std::max(pl->max_sigma, pl->token_sigma[i]);
    }
    // and each row's weight, in plan order
    if (seg_weight) {
        std::vector<float> row_weight(T, 1.0f);
        for (int32_t s = 0; s < S; ++s)
            for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) row_weight[t] = seg_weight[s];
        pl->weighted = true;
        pl->token_weight.resize(T);
        for (int32_t i = 0; i < T; ++i) pl->token_weight[i] = row_weight[pl->token_order[i]];
    }
    *out = pl;
    return LORA_OK;
}
}  // namespace

extern "C" {

lora_status lora_plan_create(lora_plan **out, const lora_pool *p, int32_t T,
                             const int32_t *seg_starts, const int32_t *seg_adapter, int32_t S) {
    return plan_create(out, p, T, seg_starts, seg_adapter, nullptr, nullptr, S);
}

lora_status lora_plan_create_weighted(lora_plan **out, const lora_pool *p, int32_t T,
                                      const int32_t *seg_starts, const int32_t *seg_adapter,
                                      const float *seg_weight, int32_t S) {
    if (S > 0 && !seg_weight) return fail(LORA_EINVAL, "null weight table");
    return plan_create(out, p, T, seg_starts, seg_adapter, nullptr, seg_weight, S);
}

lora_status lora_plan_create_sigma(lora_plan **out, const lora_pool *p, int32_t T,
                                   const int32_t *seg_starts, const int32_t *seg_adapter,
                                   const int32_t *seg_sigma, int32_t S) {
    if (S > 0 && !seg_sigma) return fail(LORA_EINVAL, "null core table");
    return plan_create(out, p, T, seg_starts, seg_adapter, seg_sigma, nullptr, S);
}

lora_status lora_plan_destroy(lora_plan *pl) {
    if (!pl) return fail(LORA_EINVAL, "null plan");
    if (pl->staged) {
        (void)hipEventSynchronize(pl->staged);
        (void)hipEventDestroy(pl->staged);
    }
    if (pl->staging) (void)hipHostFree(pl->staging);
    delete pl;
    return LORA_OK;
}

uint64_t lora_plan_workspace_bytes(const lora_plan *pl, int32_t max_proj) {
    if (!pl || max_proj < 1 || max_proj > LORA_MAX_PROJ) return 0;
    lora_plan tmp;   // compute the layout without touching the plan
    tmp.pool = pl->pool;
    tmp.T = pl->T;
    tmp.blocks = pl->blocks;
    tmp.tiles = pl->tiles;
    tmp.nb_act = pl->nb_act;
    tmp.tt = pl->tt;
    tmp.layout(max_proj);
    return tmp.ws_bytes;
}

lora_status lora_plan_upload(lora_plan *pl, void *ws, uint64_t ws_bytes, int32_t max_proj,
                             void *stream) {
    if (!pl) return fail(LORA_EINVAL, "null plan");
    if (max_proj < 1 || max_proj > LORA_MAX_PROJ)
        return fail(LORA_EINVAL, "max_proj %d not in 1..%d", max_proj, LORA_MAX_PROJ);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255))
        return fail(LORA_EINVAL, "workspace must be a non-null, 256-byte aligned device pointer");
    const uint64_t need = lora_plan_workspace_bytes(pl, max_proj);
    if (ws_bytes < need)
        return fail(LORA_ESTATE, "workspace of %llu bytes < %llu needed",
                    (unsigned long long)ws_bytes, (unsigned long long)need);
    hipError_t e;
    if (pl->staged) {   // the previous image may still be in flight
        e = hipEventSynchronize(pl->staged);
        if (e != hipSuccess) return hip_fail(e, "plan staging wait");
    }
    lora_plan probe = lora_plan();   // layout of the new image
    probe.pool = pl->pool; probe.T = pl->T; probe.blocks = pl->blocks;
    probe.tiles = pl->tiles; probe.nb_act = pl->nb_act; probe.tt = pl->tt;
    probe.layout(max_proj);
    if (pl->staging_bytes < probe.image_bytes) {
        void *buf = nullptr;
        e = hipHostMalloc(&buf, probe.image_bytes, hipHostMallocDefault);
        if (e != hipSuccess) return hip_fail(e, "plan staging buffer");
        if (pl->staging) (void)hipHostFree(pl->staging);
        pl->staging = buf;
        pl->staging_bytes = probe.image_bytes;
    }
    if (!pl->staged) {
        e = hipEventCreateWithFlags(&pl->staged, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "plan staging event");
    }
    pl->layout(max_proj);
    pl->max_proj = max_proj;
    uint8_t *img = static_cast<uint8_t *>(pl->staging);
    std::memset(img, 0, pl->image_bytes);
    if (pl->T) std::memcpy(img + pl->off_tok, pl->token_order.data(), 4ull * pl->T);
    if (pl->T) std::memcpy(img + pl->off_tsig, pl->token_sigma.data(), 4ull * pl->T);
    if (pl->T && pl->weighted)
        std::memcpy(img + pl->off_tw, pl->token_weight.data(), 4ull * pl->T);
    if (!pl->blocks.empty())
        std::memcpy(img + pl->off_blocks, pl->blocks.data(), sizeof(BlockDesc) * pl->blocks.size());
    if (!pl->tiles.empty())
        std::memcpy(img + pl->off_tiles, pl->tiles.data(), sizeof(lora::TileDesc) * pl->tiles.size());
    {   // token rows of each block and of each rank tile, -1 padded
        int32_t *bt = reinterpret_cast<int32_t *>(img + pl->off_btok);
        for (int32_t b = 0; b < pl->nb_all(); ++b) {
            const BlockDesc &bd = pl->blocks[b];
            for (int32_t i = 0; i < lora::kMaxBlockTokens; ++i)
                bt[b * lora::kMaxBlockTokens + i] =
                    i < bd.n_tok ? pl->token_order[bd.tok_off + i] : -1;
        }
        int32_t *tt = reinterpret_cast<int32_t *>(img + pl->off_ttok);
        for (int32_t k = 0; k < pl->rt_total(); ++k) {
            const lora::TileDesc &td = pl->tiles[k];
            for (int32_t i = 0; i < lora::kMaxBlockTokens; ++i)
                tt[k * lora::kMaxBlockTokens + i] =
                    i < td.n_tok ? pl->token_order[td.tok_off + i] : -1;
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(ws, img, pl->image_bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "plan upload");
    e = hipEventRecord(pl->staged, st);
    if (e != hipSuccess) return hip_fail(e, "plan staging event record");
    pl->ws = ws;
    pl->part_layer = -1;               // a new workspace holds no partials
    return LORA_OK;
}

lora_status lora_plan_stats(const lora_plan *pl, int32_t *ng, int32_t *nb, int32_t *na,
                            int32_t *mb) {
    if (!pl) return fail(LORA_EINVAL, "null plan");
    if (ng) *ng = int32_t(pl->group_adapter.size());
    if (nb) *nb = pl->nb_all();
    if (na) *na = pl->n_active;
    if (mb) *mb = pl->max_block;
    return LORA_OK;
}

lora_status lora_plan_export(const lora_plan *pl, int32_t *order, int32_t *tgroup,
                             int32_t *gad, int32_t *grank) {
    if (!pl) return fail(LORA_EINVAL, "null plan");
    if (order && pl->T) std::memcpy(order, pl->token_order.data(), 4ull * pl->T);
    if (tgroup && pl->T) std::memcpy(tgroup, pl->token_group.data(), 4ull * pl->T);
    const size_t G = pl->group_adapter.size();
    if (gad && G) std::memcpy(gad, pl->group_adapter.data(), 4 * G);
    if (grank && G) std::memcpy(grank, pl->group_rank.data(), 4 * G);
    return LORA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------- sgmv ----
namespace {

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// bytes spanned by T rows of width `width` at leading dimension ld
uint64_t tensor_bytes(int32_t T, int64_t ld, int64_t width, int32_t es) {
    if (T <= 0) return 0;
    return (uint64_t(T - 1) * uint64_t(ld) + uint64_t(width)) * uint64_t(es);
}

struct CallCheck {
    int32_t h_in = 0;
    int32_t es = 0;
    int32_t vec = 0;   // elements per 16 bytes
};

lora_status check_call(const lora_pool *p, const lora_plan *pl, int32_t layer, int32_t nproj,
                       const int32_t *projs, CallCheck *cc) {
    if (!p || !pl) return fail(LORA_EINVAL, "null pool or plan");
    if (pl->pool != p) return fail(LORA_EINVAL, "plan was built for another pool");
    if (pl->pool_generation != p->generation)
        return fail(LORA_ESTATE, "an adapter was unregistered after the plan was built");
    if (!pl->ws) return fail(LORA_ESTATE, "plan has not been uploaded");
    if (layer < 0 || layer >= p->d.num_layers)
        return fail(LORA_EINVAL, "layer %d not in 0..%d", layer, p->d.num_layers - 1);
    if (nproj < 1 || nproj > pl->max_proj)
        return fail(LORA_EINVAL, "nproj %d not in 1..%d (plan uploaded for %d)", nproj,
                    pl->max_proj, pl->max_proj);
    if (!projs) return fail(LORA_EINVAL, "null projection list");
    for (int i = 0; i < nproj; ++i) {
        if (projs[i] < 0 || projs[i] >= p->d.num_proj)
            return fail(LORA_EINVAL, "projection %d not in 0..%d", projs[i], p->d.num_proj - 1);
        for (int k = 0; k < i; ++k)
            if (projs[k] == projs[i]) return fail(LORA_EINVAL, "projection %d listed twice", projs[i]);
        if (p->d.h_in[projs[i]] != p->d.h_in[projs[0]])
            return fail(LORA_EINVAL, "projections of one call must share h_in");
    }
    cc->h_in = p->d.h_in[projs[0]];
    cc->es = esize(p->d.dtype);
    cc->vec = 16 / cc->es;
    return LORA_OK;
}

lora_status check_y(const lora_pool *p, int32_t T, int32_t nproj, const int32_t *projs,
                    const int32_t *yoff, const void *y, int64_t ldy, const char *name,
                    const CallCheck &cc) {
    if (!yoff) return fail(LORA_EINVAL, "null y_offsets");
    if (!y || !aligned16(y)) return fail(LORA_EINVAL, "%s must be non-null and 16-byte aligned", name);
    if (ldy < 1 || ldy % 8 || ldy % cc.vec)
        return fail(LORA_EINVAL, "ld of %s (%lld) must be a positive multiple of 8", name,
                    (long long)ldy);
    if (tensor_bytes(T, ldy, ldy, cc.es) > lora::kMaxTensorBytes)
        return fail(LORA_EINVAL, "%s spans more than 2 GiB", name);
    for (int i = 0; i < nproj; ++i) {
        if (yoff[i] < 0 || yoff[i] % 8)
            return fail(LORA_EINVAL, "y_offsets[%d] = %d must be a non-negative multiple of 8", i,
                        yoff[i]);
        if (int64_t(yoff[i]) + p->d.h_out[projs[i]] > ldy)
            return fail(LORA_EINVAL, "slice of projection %d exceeds ld of %s", projs[i], name);
    }
    return LORA_OK;
}

// Shrink units over every projection of the call (one load of x for all of
// them) when blocks span several 16-token tiles, where x is most of the
// shrink's loads, for calls of up to kShrinkMaxUnitProj projections (each
// projection's A fragments are held in registers): the prefill shrink's
// average call went from 14.1 to 12.4 us.  Decode blocks (one tile) keep a
// unit per projection.
constexpr int32_t kShrinkMaxUnitProj = 3;
bool shrink_mp(const lora_plan *pl, int32_t nproj) {
    return pl->tt >= 2 && nproj > 1 && nproj <= kShrinkMaxUnitProj;
}

// k-chunking of the shrink: about kShrinkTargetGroups workgroups per launch, each
// wave loading at most `frags` fragments (all issued up front); chunks are a
// multiple of 4 fragment spans so the 4 waves split them evenly.
void shrink_geometry(const lora_plan *pl, int32_t nproj, int32_t h_in, int32_t span,
                     int32_t *kc, int32_t *c0) {
    // workgroups per k-chunk: one per rank tile and projection, or one per
    // rank tile for units over every projection
    const int64_t per_chunk = int64_t(shrink_mp(pl, nproj) ? 1 : nproj) *
                              std::max(pl->rt_total(), 1);
    const int32_t frags = pl->tt <= 2 ? lora::shrink_frags<1>() : lora::shrink_frags<4>();
    const int32_t steps = (h_in + lora::kWaves * span - 1) / (lora::kWaves * span);
    int64_t want = (lora::kShrinkTargetGroups + per_chunk - 1) / per_chunk;
    want = std::max<int64_t>(1, std::min<int64_t>(want, steps));
    const int32_t sper = std::min<int32_t>(frags, int32_t((steps + want - 1) / want));
    *kc = sper * lora::kWaves * span;
    *c0 = (h_in + *kc - 1) / *kc;
}

// workgroups launched for `units` dealt to the XCDs in groups of `gs`
int32_t grid_for(int32_t units, int32_t gs) {
    return int32_t(round_up(uint64_t(std::max(units, 0)), uint64_t(lora::kXcds) * gs));
}

lora_status run_shrink(const lora_pool *p, const lora_plan *pl, int32_t layer, int32_t nproj,
                       const int32_t *projs, const void *x, int64_t ldx, const CallCheck &cc,
                       hipStream_t st, int32_t *c0_out) {
    *c0_out = 0;
    // every shrink leaves its partials in the workspace: record whose they are
    pl->part_layer = -1;
    auto record = [&](int32_t c0) {
        pl->part_layer = layer;
        pl->part_nproj = nproj;
        pl->part_c0 = c0;
        for (int i = 0; i < nproj; ++i) pl->part_projs[i] = projs[i];
    };
    if (pl->nb_act == 0) {
        record(0);
        return LORA_OK;
    }
    lora::ShrinkArgs a{};
    const uint8_t *ws = static_cast<const uint8_t *>(pl->ws);
    a.slab = p->slab;
    a.tile_tok = reinterpret_cast<const int32_t *>(ws + pl->off_ttok);
    a.tiles = reinterpret_cast<const lora::TileDesc *>(ws + pl->off_tiles);
    a.partial = reinterpret_cast<float *>(const_cast<uint8_t *>(ws) + pl->off_part);
    a.x = x;
    a.ldx = ldx;
    for (int i = 0; i < nproj; ++i) a.coef_a[i] = p->coef_a(layer, projs[i]);
    a.nproj = nproj;
    a.h_in = cc.h_in;
    a.h_in_pad = int32_t(h_in_pad(&p->d, projs[0]));
    shrink_geometry(pl, nproj, cc.h_in, 4 * cc.vec, &a.kc, &a.c0);
    const bool mp = shrink_mp(pl, nproj);
    a.units = (mp ? 1 : nproj) * pl->rt_total() * a.c0;
    a.grid = grid_for(a.units, mp ? 1 : nproj);
    a.x_bytes = uint32_t(tensor_bytes(pl->T, ldx, cc.h_in, cc.es));
    const uint64_t need = 4ull * uint64_t(nproj) * pl->rt_total() * a.c0 * pl->tt * lora::kTile *
                          lora::kTile;
    if (need > lora::kMaxTensorBytes)   // the expands address the partials within 2 GiB
        return fail(LORA_EINVAL, "the call's shrink partials would span %llu bytes, more than "
                    "2 GiB: split the batch", (unsigned long long)need);
    if (need > pl->part_bytes)
        return fail(LORA_ESTATE, "partial buffer too small (%llu > %llu)",
                    (unsigned long long)need, (unsigned long long)pl->part_bytes);
    hipError_t e = lora::launch_shrink(p->d.dtype, pl->tt, mp, a, st);
    if (e != hipSuccess) return hip_fail(e, "shrink launch");
    *c0_out = a.c0;
    record(a.c0);
    return LORA_OK;
}

lora_status run_reduce(const lora_pool *p, const lora_plan *pl, int32_t nproj, int32_t c0,
                       float *v, int64_t ldv, hipStream_t st) {
    if (pl->nb_act == 0) return LORA_OK;
    lora::ReduceArgs a{};
    const uint8_t *ws = static_cast<const uint8_t *>(pl->ws);
    a.tok = reinterpret_cast<const int32_t *>(ws + pl->off_tok);
    a.blocks = reinterpret_cast<const BlockDesc *>(ws + pl->off_blocks);
    a.partial = reinterpret_cast<const float *>(ws + pl->off_part);
    a.partial_bytes = uint32_t(std::min<uint64_t>(pl->part_bytes, lora::kMaxTensorBytes));
    a.v = v;
    a.ldv = ldv;
    a.nb = pl->nb_act;
    a.nproj = nproj;
    a.c0 = c0;
    a.r_max = p->d.r_max;
    hipError_t e = lora::launch_reduce(pl->tt, a, st);
    if (e != hipSuccess) return hip_fail(e, "reduce launch");
    return LORA_OK;
}

// K-steps of the largest padded rank in the plan (the expand kernels are
// built for 1, 2 or 4)
int32_t plan_ksteps(const lora_pool *p, const lora_plan *pl) {
    const int32_t span = 4 * (16 / esize(p->d.dtype));
    int32_t ks = std::max(1, (pl->max_rpad + span - 1) / span);
    return ks == 3 ? 4 : ks;
}

// Cores of jointly compressed adapters for one call (kind 0: none).
struct Cores {
    const float *sigma = nullptr;
    int32_t kind = 0;
    int32_t count = 0;
};

// Checks the core table of a call against the plan and pool.
lora_status check_cores(const lora_plan *pl, const Cores &c) {
    if (c.kind != LORA_SIGMA_DIAG && c.kind != LORA_SIGMA_FULL)
        return fail(LORA_EINVAL, "core kind %d is neither diagonal nor full", c.kind);
    if (!c.sigma || !aligned16(c.sigma))
        return fail(LORA_EINVAL, "core table must be non-null and 16-byte aligned");
    if (c.count < 0 || pl->max_sigma >= c.count)
        return fail(LORA_EINVAL, "plan names core %d of a table of %d", pl->max_sigma, c.count);
    return LORA_OK;
}

// v source of the expand: the shrink partials of this call (c0 > 0), or a
// caller's v buffer
lora_status run_expand(const lora_pool *p, const lora_plan *pl, int32_t layer, int32_t nproj,
                       const int32_t *projs, const int32_t *yoff, int32_t c0, const float *v,
                       int64_t ldv, void *y, int64_t ldy, const void *base, int64_t ldb,
                       hipStream_t st, const Cores &cores = Cores()) {
    const int32_t nb = base ? pl->nb_all() : pl->nb_act;
    if (nb == 0) return LORA_OK;
    lora::ExpandArgs a{};
    const uint8_t *ws = static_cast<const uint8_t *>(pl->ws);
    a.slab = p->slab;
    a.tok = reinterpret_cast<const int32_t *>(ws + pl->off_tok);
    a.block_tok = reinterpret_cast<const int32_t *>(ws + pl->off_btok);
    a.blocks = reinterpret_cast<const BlockDesc *>(ws + pl->off_blocks);
    a.partial = c0 > 0 ? reinterpret_cast<const float *>(ws + pl->off_part) : nullptr;
    a.partial_bytes = uint32_t(std::min<uint64_t>(pl->part_bytes, lora::kMaxTensorBytes));
    a.c0 = c0;
    a.v = v;
    a.y = y;
    a.base = base;
    a.ldv = ldv;
    a.ldy = ldy;
    a.ldb = ldb;
    for (int i = 0; i < nproj; ++i) {
        a.coef_b[i] = p->coef_b(layer, projs[i]);
        a.h_out[i] = p->d.h_out[projs[i]];
        a.y_off[i] = yoff[i];
    }
    a.nproj = nproj;
    a.r_max = p->d.r_max;
    a.ptt = pl->tt;
    a.y_bytes = uint32_t(tensor_bytes(pl->T, ldy, ldy, esize(p->d.dtype)));
    a.base_bytes = base ? uint32_t(tensor_bytes(pl->T, ldb, ldb, esize(p->d.dtype))) : 0u;
    a.v_bytes = v ? uint32_t(tensor_bytes(pl->T, ldv, ldv, 4)) : 0u;
    if (pl->weighted) a.tok_w = reinterpret_cast<const float *>(ws + pl->off_tw);
    if (cores.kind) {
        const int64_t per = cores.kind == LORA_SIGMA_FULL ? int64_t(p->d.r_max) * p->d.r_max
                                                           : int64_t(p->d.r_max);
        a.sigma = cores.sigma;
        a.sigma_kind = cores.kind;
        a.tok_sig = reinterpret_cast<const int32_t *>(ws + pl->off_tsig);
        a.sig_stride = int64_t(p->d.num_layers) * p->d.num_proj * per;
        for (int i = 0; i < nproj; ++i)
            a.sig_off[i] = (int64_t(layer) * p->d.num_proj + projs[i]) * per;
    }
    // The long groups' blocks [0, nb_long) go to the MFMA expand, the rest
    // (short groups' blocks, then the blocks without an adapter) to the decode
    // expand: two launches on the stream when a batch has both.
    const int32_t nl = std::min(pl->nb_long, nb);
    if (nl > 0) {
        // K-steps of the largest padded rank fix the rows per wave (the wave
        // keeps 8 B fragments); 4 waves per workgroup; row chunks per wave:
        // about kTargetGroups workgroups per launch
        lora::ExpandArgs m = a;
        const int32_t ks = plan_ksteps(p, pl);
        const int64_t chunk_rows = int64_t(16 * lora::expand_tiles(ks)) * lora::kWaves;
        // token tiles per unit, and token slices per block
        const int32_t ttu = std::min<int32_t>(pl->tt, lora::kExpandUnitTiles);
        m.tslices = pl->tt / ttu;
        int64_t rows = 0;
        for (int i = 0; i < nproj; ++i) rows += m.h_out[i];
        m.chunks = int32_t(std::max<int64_t>(1, std::min<int64_t>(
            8, rows * nl * m.tslices / (chunk_rows * lora::kTargetGroups))));
        const int32_t rows_per_group = int32_t(chunk_rows) * m.chunks;
        m.oc_prefix[0] = 0;
        for (int i = 0; i < nproj; ++i)
            m.oc_prefix[i + 1] = m.oc_prefix[i] + (m.h_out[i] + rows_per_group - 1) / rows_per_group;
        for (int i = nproj; i < LORA_MAX_PROJ; ++i) m.oc_prefix[i + 1] = INT32_MAX;
        m.units = nl * m.tslices * m.oc_prefix[nproj];
        m.grid = grid_for(m.units, 1);
        const hipError_t e = lora::launch_expand(p->d.dtype, ttu, ks, m, st);
        if (e != hipSuccess) return hip_fail(e, "expand launch");
    }
    if (nb > nl) {
        // rank classes: runs of equal padded rank in block order (short
        // blocks by rank, largest first; then the blocks without an adapter)
        for (int k = 0; k < lora::kMaxClasses; ++k) a.cls_rb[k] = 0;
        if (nb >= (1 << 23)) return fail(LORA_ESTATE, "%d blocks: more than 2^23", nb);
        int32_t ncls = 0, units = 0, nvm = 1;
        for (int32_t b = nl; b < nb;) {
            const int32_t r = pl->blocks[b].r_pad;
            int32_t e = b;
            while (e < nb && pl->blocks[e].r_pad == r) ++e;
            if (ncls == lora::kMaxClasses)
                return fail(LORA_ESTATE, "more than %d rank classes", lora::kMaxClasses);
            const int32_t lg = lora::decode_unit_rows_log2(r, esize(p->d.dtype));
            int32_t upb = 0;
            for (int i = 0; i < nproj; ++i) upb += (a.h_out[i] + (1 << lg) - 1) >> lg;
            if (r > 0) nvm = std::max(nvm, lora::decode_nvt(r, esize(p->d.dtype)));
            a.cls_rb[ncls] = (b << 8) | r;
            a.cls_unit0[ncls] = units;
            units += (e - b) * upb;
            ++ncls;
            b = e;
        }
        for (int k = ncls; k <= lora::kMaxClasses; ++k) a.cls_unit0[k] = k == ncls ? units : INT32_MAX;
        a.units = units;
        a.grid = grid_for(a.units, 1);
        const hipError_t e = lora::launch_expand_decode(p->d.dtype, nvm, a, st);
        if (e != hipSuccess) return hip_fail(e, "expand launch");
    }
    return LORA_OK;
}

}  // namespace

extern "C" {

lora_status sgmv_shrink(const lora_pool *p, const lora_plan *pl, int32_t layer, int32_t nproj,
                        const int32_t *projs, const void *x, int64_t ldx, float *v, int64_t ldv,
                        void *stream) {
    CallCheck cc;
    lora_status st = check_call(p, pl, layer, nproj, projs, &cc);
    if (st != LORA_OK) return st;
    if (pl->T == 0) return LORA_OK;   // empty batch: nothing to read or write
    if (!x || !aligned16(x)) return fail(LORA_EINVAL, "x must be non-null and 16-byte aligned");
    if (ldx < cc.h_in || ldx % 8) return fail(LORA_EINVAL, "ldx %lld < h_in or not a multiple of 8",
                                               (long long)ldx);
    if (tensor_bytes(pl->T, ldx, cc.h_in, cc.es) > lora::kMaxTensorBytes)
        return fail(LORA_EINVAL, "x spans more than 2 GiB");
    if (!v || !aligned16(v)) return fail(LORA_EINVAL, "v must be non-null and 16-byte aligned");
    if (ldv < int64_t(nproj) * p->d.r_max || ldv % 4)
        return fail(LORA_EINVAL, "ldv %lld < nproj * r_max or not a multiple of 4", (long long)ldv);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t c0 = 0;
    st = run_shrink(p, pl, layer, nproj, projs, x, ldx, cc, hs, &c0);
    if (st != LORA_OK) return st;
    return run_reduce(p, pl, nproj, c0, v, ldv, hs);
}

lora_status sgmv_expand(const lora_pool *p, const lora_plan *pl, int32_t layer, int32_t nproj,
                        const int32_t *projs, const int32_t *yoff, const float *v, int64_t ldv,
                        void *y, int64_t ldy, void *stream) {
    CallCheck cc;
    lora_status st = check_call(p, pl, layer, nproj, projs, &cc);
    if (st != LORA_OK) return st;
    if (pl->T == 0) return LORA_OK;   // empty batch: nothing to read or write
    if (!v || !aligned16(v)) return fail(LORA_EINVAL, "v must be non-null and 16-byte aligned");
    if (ldv < int64_t(nproj) * p->d.r_max || ldv % 4)
        return fail(LORA_EINVAL, "ldv %lld < nproj * r_max or not a multiple of 4", (long long)ldv);
    if (tensor_bytes(pl->T, ldv, ldv, 4) > lora::kMaxTensorBytes)
        return fail(LORA_EINVAL, "v spans more than 2 GiB");
    st = check_y(p, pl->T, nproj, projs, yoff, y, ldy, "y", cc);
    if (st != LORA_OK) return st;
    return run_expand(p, pl, layer, nproj, projs, yoff, 0, v, ldv, y, ldy, nullptr, 0,
                      static_cast<hipStream_t>(stream));
}

lora_status sgmv_expand_sigma(const lora_pool *p, const lora_plan *pl, int32_t layer,
                              int32_t nproj, const int32_t *projs, const int32_t *yoff,
                              const float *v, int64_t ldv, const float *sigma, int32_t sigma_kind,
                              int32_t num_sigma, void *y, int64_t ldy, void *stream) {
    CallCheck cc;
    lora_status st = check_call(p, pl, layer, nproj, projs, &cc);
    if (st != LORA_OK) return st;
    const Cores cores{sigma, sigma_kind, num_sigma};
    st = check_cores(pl, cores);
    if (st != LORA_OK) return st;
    if (pl->T == 0) return LORA_OK;
    if (!v || !aligned16(v)) return fail(LORA_EINVAL, "v must be non-null and 16-byte aligned");
    if (ldv < int64_t(nproj) * p->d.r_max || ldv % 4)
        return fail(LORA_EINVAL, "ldv %lld < nproj * r_max or not a multiple of 4", (long long)ldv);
    if (tensor_bytes(pl->T, ldv, ldv, 4) > lora::kMaxTensorBytes)
        return fail(LORA_EINVAL, "v spans more than 2 GiB");
    st = check_y(p, pl->T, nproj, projs, yoff, y, ldy, "y", cc);
    if (st != LORA_OK) return st;
    return run_expand(p, pl, layer, nproj, projs, yoff, 0, v, ldv, y, ldy, nullptr, 0,
                      static_cast<hipStream_t>(stream), cores);
}

lora_status sgmv_fused(const lora_pool *p, const lora_plan *pl, int32_t layer, int32_t nproj,
                       const int32_t *projs, const int32_t *yoff, const void *x, int64_t ldx,
                       const void *base, int64_t ldb, void *y, int64_t ldy, void *stream) {
    return sgmv_fused_sigma(p, pl, layer, nproj, projs, yoff, x, ldx, nullptr, 0, 0, base, ldb,
                            y, ldy, stream);
}

lora_status sgmv_fused_sigma(const lora_pool *p, const lora_plan *pl, int32_t layer,
                             int32_t nproj, const int32_t *projs, const int32_t *yoff,
                             const void *x, int64_t ldx, const float *sigma, int32_t sigma_kind,
                             int32_t num_sigma, const void *base, int64_t ldb, void *y,
                             int64_t ldy, void *stream) {
    CallCheck cc;
    lora_status st = check_call(p, pl, layer, nproj, projs, &cc);
    if (st != LORA_OK) return st;
    if (pl->T == 0) return LORA_OK;   // empty batch: nothing to read or write
    if (!x || !aligned16(x)) return fail(LORA_EINVAL, "x must be non-null and 16-byte aligned");
    if (ldx < cc.h_in || ldx % 8) return fail(LORA_EINVAL, "ldx %lld < h_in or not a multiple of 8",
                                               (long long)ldx);
    if (tensor_bytes(pl->T, ldx, cc.h_in, cc.es) > lora::kMaxTensorBytes)
        return fail(LORA_EINVAL, "x spans more than 2 GiB");
    const Cores cores{sigma, sigma_kind, num_sigma};
    if (sigma_kind != 0 || sigma) {
        st = check_cores(pl, cores);
        if (st != LORA_OK) return st;
    }
    st = check_y(p, pl->T, nproj, projs, yoff, y, ldy, "y", cc);
    if (st != LORA_OK) return st;
    if (base) {
        st = check_y(p, pl->T, nproj, projs, yoff, base, ldb, "base", cc);
        if (st != LORA_OK) return st;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t c0 = 0;
    st = run_shrink(p, pl, layer, nproj, projs, x, ldx, cc, hs, &c0);
    if (st != LORA_OK) return st;
    return run_expand(p, pl, layer, nproj, projs, yoff, c0, nullptr, 0, y, ldy, base, ldb, hs,
                      cores);
}

lora_status sgmv_shrink_partials(const lora_pool *p, const lora_plan *pl, int32_t layer,
                                 int32_t nproj, const int32_t *projs, const void *x, int64_t ldx,
                                 void *stream) {
    CallCheck cc;
    lora_status st = check_call(p, pl, layer, nproj, projs, &cc);
    if (st != LORA_OK) return st;
    if (pl->T > 0) {
        if (!x || !aligned16(x)) return fail(LORA_EINVAL, "x must be non-null and 16-byte aligned");
        if (ldx < cc.h_in || ldx % 8)
            return fail(LORA_EINVAL, "ldx %lld < h_in or not a multiple of 8", (long long)ldx);
        if (tensor_bytes(pl->T, ldx, cc.h_in, cc.es) > lora::kMaxTensorBytes)
            return fail(LORA_EINVAL, "x spans more than 2 GiB");
    }
    int32_t c0 = 0;
    if (pl->T == 0) {                  // empty batch: nothing to read; the record alone
        pl->part_layer = layer;
        pl->part_nproj = nproj;
        pl->part_c0 = 0;
        for (int i = 0; i < nproj; ++i) pl->part_projs[i] = projs[i];
        return LORA_OK;
    }
    return run_shrink(p, pl, layer, nproj, projs, x, ldx, cc, static_cast<hipStream_t>(stream),
                      &c0);
}

lora_status sgmv_expand_partials(const lora_pool *p, const lora_plan *pl, int32_t layer,
                                 int32_t nproj, const int32_t *projs, const int32_t *yoff,
                                 const void *base, int64_t ldb, void *y, int64_t ldy,
                                 void *stream) {
    return sgmv_expand_partials_sigma(p, pl, layer, nproj, projs, yoff, nullptr, 0, 0, base, ldb,
                                      y, ldy, stream);
}

lora_status sgmv_expand_partials_sigma(const lora_pool *p, const lora_plan *pl, int32_t layer,
                                       int32_t nproj, const int32_t *projs, const int32_t *yoff,
                                       const float *sigma, int32_t sigma_kind, int32_t num_sigma,
                                       const void *base, int64_t ldb, void *y, int64_t ldy,
                                       void *stream) {
    CallCheck cc;
    lora_status st = check_call(p, pl, layer, nproj, projs, &cc);
    if (st != LORA_OK) return st;
    const Cores cores{sigma, sigma_kind, num_sigma};
    if (sigma_kind != 0 || sigma) {
        st = check_cores(pl, cores);
        if (st != LORA_OK) return st;
    }
    bool same = pl->part_layer == layer && pl->part_nproj == nproj;
    for (int i = 0; same && i < nproj; ++i) same = pl->part_projs[i] == projs[i];
    if (!same)
        return fail(LORA_ESTATE, "the plan's workspace holds no shrink partials of layer %d "
                                 "and these projections", layer);
    if (pl->T == 0) return LORA_OK;
    st = check_y(p, pl->T, nproj, projs, yoff, y, ldy, "y", cc);
    if (st != LORA_OK) return st;
    if (base) {
        st = check_y(p, pl->T, nproj, projs, yoff, base, ldb, "base", cc);
        if (st != LORA_OK) return st;
    }
    return run_expand(p, pl, layer, nproj, projs, yoff, pl->part_c0, nullptr, 0, y, ldy, base,
                      ldb, static_cast<hipStream_t>(stream), cores);
}

}  // extern "C"

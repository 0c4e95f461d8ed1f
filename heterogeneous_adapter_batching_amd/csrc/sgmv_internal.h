// Internal interface between the host library (pool, plan, C ABI) and the
// gfx950 kernels.  Not installed; the public interface is include/lora_sgmv.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "lora_sgmv.h"

namespace lora {

constexpr int kWaveSize = 64;
constexpr int kWaves = 4;                    // waves per 256-thread workgroup
constexpr int kTile = 16;                    // MFMA tile edge (rows, tokens)
constexpr int kMaxBlockTokens = 64;          // tokens per block: at most 4 token tiles
constexpr int kTargetGroups = 1024;          // workgroups aimed for per launch (4 per CU)
constexpr int kXcds = 8;                     // workgroup g runs on XCD g % 8

// One token block of one adapter group (or of the tokens without an adapter).
struct BlockDesc {
    int32_t tok_off;   // first entry of the block in the plan's token order
    int32_t n_tok;     // 1 .. kMaxBlockTokens
    int32_t r_pad;     // padded rank; 0 marks a block of tokens without an adapter
    int32_t rt;        // rank tiles of 16 rows: ceil(r_pad / 16)
    float scale;       // the adapter's scale
    int32_t group;     // group index (-1 for tokens without an adapter)
    uint32_t ext_lo;   // adapter extent byte offset in the slab, low and high words
    uint32_t ext_hi;
};
static_assert(sizeof(BlockDesc) == 32, "BlockDesc is 32 bytes");

// Shrink: one workgroup per unit (block b, k-chunk c, rank tile rt,
// projection i).  Units of a block are ordered with c outermost, so the units
// that read the same x chunk are consecutive; consecutive units are placed on
// one XCD.  The 4 waves split the chunk's K range and are summed through LDS
// in a fixed order; the unit writes one float32 partial tile
// [16 * TT token slots][16 ranks] at partial + unit * TT * 256.
struct ShrinkArgs {
    const uint8_t *slab;
    const int32_t *tok;          // plan token order
    const BlockDesc *blocks;
    const int32_t *rt_prefix;    // [nb + 1] prefix sums of BlockDesc::rt
    float *partial;
    const void *x;
    int64_t ldx;
    int64_t coef_a[LORA_MAX_PROJ];  // A block offset = extent + r_pad * esize * coef_a[i]
    int32_t nb;                  // adapter blocks
    int32_t nproj;
    int32_t h_in;
    int32_t kc;                  // k-chunk (elements, multiple of 4 fragment spans)
    int32_t c0;                  // number of k-chunks
    int32_t units;
    int32_t grid;                // workgroups launched: units rounded up to kXcds
};

// v from the shrink's partials, for the standalone shrink:
// v[t][i * r_max + j] = sum over chunks (j < r_pad), 0 for r_pad <= j < r_max.
struct ReduceArgs {
    const int32_t *tok;
    const BlockDesc *blocks;
    const int32_t *rt_prefix;
    const float *partial;
    float *v;
    int64_t ldv;
    int32_t nb;
    int32_t nproj;
    int32_t c0;
    int32_t r_max;
};

// Expand: one workgroup per unit (block b, projection i, chunk of 4 * ocw
// output rows).  The workgroup gathers its tokens' v into LDS once (summing
// the shrink partials in a fixed order, or reading a caller's v), then each
// wave streams the B rows of its ocw rows and writes y = y_in + s * (B v),
// rounded once.
struct ExpandArgs {
    const uint8_t *slab;
    const int32_t *tok;
    const BlockDesc *blocks;
    const int32_t *rt_prefix;
    const float *partial;        // non-null: v = sum of partials
    const float *v;              // else: caller's v [T][ldv]
    void *y;
    const void *base;            // nullable: y_in = base, else y_in = y
    int64_t ldv;
    int64_t ldy;
    int64_t ldb;
    int64_t coef_b[LORA_MAX_PROJ];  // B block offset = extent + r_pad * esize * coef_b[i]
    int32_t h_out[LORA_MAX_PROJ];
    int32_t y_off[LORA_MAX_PROJ];
    int32_t oc_prefix[LORA_MAX_PROJ + 1];  // row chunks of projections before i
    int32_t nb;                  // blocks launched over
    int32_t nproj;
    int32_t ocw;                 // output rows per wave (multiple of 32)
    int32_t c0;                  // partial chunks (when partial != null)
    int32_t units;
    int32_t grid;
    int32_t r_max;
};

// Kernel launchers (kernels.hip).  dtype is a lora_dtype; tt is the number of
// 16-token tiles of the largest block (1, 2 or 4).
hipError_t launch_shrink(int dtype, int tt, const ShrinkArgs &a, hipStream_t s);
hipError_t launch_reduce(int tt, const ReduceArgs &a, hipStream_t s);
hipError_t launch_expand(int dtype, int tt, const ExpandArgs &a, hipStream_t s);

}  // namespace lora

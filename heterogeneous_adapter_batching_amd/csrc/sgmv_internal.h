// Internal interface between the host library (pool, plan, C ABI) and the
// gfx950 kernels.  Not installed; the public interface is include/lora_sgmv.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "lora_sgmv.h"

namespace lora {

constexpr int kWaveSize = 64;
constexpr int kWavesPerGroup = 4;            // 256-thread workgroups of independent waves
constexpr int kTile = 16;                    // MFMA tile edge (rows, tokens)
constexpr int kMaxBlockTokens = 64;          // tokens per block: at most 4 token tiles
constexpr int kTargetWaves = 4096;           // work units aimed for per launch (16 per CU)

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

// Shrink: one wave per unit (block b, k-chunk c, rank tile rt, projection p),
// units of one block ordered with c outermost so the waves that share an x
// chunk are adjacent.  The last wave to finish a (block, projection) sums the
// k-chunk partials in a fixed order and writes v.
struct ShrinkArgs {
    const uint8_t *slab;
    const int32_t *tok;          // plan token order
    const BlockDesc *blocks;
    const int32_t *rt_prefix;    // [nb + 1] prefix sums of BlockDesc::rt
    uint32_t *counters;          // [nb][LORA_MAX_PROJ], zero between launches
    float *partial;              // [units][16 * TT tokens][16 ranks]
    const void *x;
    float *v;
    int64_t ldx;
    int64_t ldv;
    int64_t coef_a[LORA_MAX_PROJ];  // A block offset = extent + r_pad * esize * coef_a[i]
    int32_t nb;                  // adapter blocks
    int32_t nproj;
    int32_t h_in;
    int32_t kc;                  // k-chunk length (elements, multiple of the fragment span)
    int32_t c0;                  // number of k-chunks
    int32_t units;
    int32_t r_max;               // v column stride per projection
};

// Expand: one wave per unit (block b, projection i, o-chunk).  Reads v, streams
// the B rows of the chunk and writes y = y_in + s * (B v), rounded once.
struct ExpandArgs {
    const uint8_t *slab;
    const int32_t *tok;
    const BlockDesc *blocks;
    const float *v;
    void *y;
    const void *base;            // nullable: y_in = base, else y_in = y
    int64_t ldv;
    int64_t ldy;
    int64_t ldb;
    int64_t coef_b[LORA_MAX_PROJ];  // B block offset = extent + r_pad * esize * coef_b[i]
    int32_t h_out[LORA_MAX_PROJ];
    int32_t y_off[LORA_MAX_PROJ];
    int32_t oc_prefix[LORA_MAX_PROJ + 1];  // o-chunks of projections before i
    int32_t nb;                  // blocks launched over
    int32_t nproj;
    int32_t oc;                  // rows per o-chunk (multiple of 16)
    int32_t units;
    int32_t r_max;
};

// Kernel launchers (kernels.hip).  dtype is a lora_dtype; tt is the number of
// 16-token tiles of the largest block (1, 2 or 4).
hipError_t launch_shrink(int dtype, int tt, const ShrinkArgs &a, hipStream_t s);
hipError_t launch_expand(int dtype, int tt, const ExpandArgs &a, hipStream_t s);

}  // namespace lora

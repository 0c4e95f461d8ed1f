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
// Short groups are cut into blocks of at most kDecodeBlockTokens for the
// decode expand: every workgroup of its launch then moves about the same
// bytes (a popular adapter's group becomes several blocks instead of one
// heavy one), and it takes a whole block in one pass.  A group of at least
// kLongGroup tokens is long, and takes kMaxBlockTokens-token blocks and the
// MFMA expand, but only when the batch's long groups hold kMinLongTokens
// tokens between them: fewer 64-token blocks leave most of the chip idle in
// the MFMA expand's launch, and the decode cut does better.
constexpr int kDecodeBlockTokens = 4;
constexpr int kLongGroup = 48;
#ifndef LORA_MIN_LONG_TOKENS
#define LORA_MIN_LONG_TOKENS 1024
#endif
constexpr int kMinLongTokens = LORA_MIN_LONG_TOKENS;
constexpr int kValuTokens = kDecodeBlockTokens;  // token slots of the decode expand
// The shrink's chunk partials of one v entry are summed as kSumWays
// interleaved running sums (chunk c into sum c % kSumWays, in increasing c),
// then added in order: every kernel that sums them uses this one order.
constexpr int kSumWays = 4;
// rank classes of the decode expand: distinct padded ranks (multiples of 8)
// of the blocks, and 0 for tokens without an adapter
constexpr int kMaxClasses = LORA_MAX_RANK / 8 + 1;
constexpr int kTargetGroups = 1024;          // MFMA expand: workgroups aimed for per launch
// MFMA expand: 16-token tiles of a block per unit (a 64-token block is
// kMaxBlockTokens / (16 * kExpandUnitTiles) units over the same rows).  One
// tile a unit keeps the kernel near 150 VGPRs (3 waves a SIMD) where 4 tiles
// spilled into AGPRs at 1 wave: 4.5% faster per prefill step, 2 tiles 3.5%.
constexpr int kExpandUnitTiles = 1;
// Shrink: workgroups aimed for per launch.  Fewer, longer k-chunks win over
// more, shorter ones here (the expand then also sums fewer partials):
// measured on the full stack, 384 beat 1024 by 3.5% per step, and 256 beat
// 384 by 0.5% (the o call's 6 k-chunks become 4; 128 measured the same).
constexpr int kShrinkTargetGroups = 256;
constexpr int kXcds = 8;                     // workgroup g runs on XCD g % 8
// Activations and outputs are addressed through buffer resources whose
// out-of-range offset is 2^31: each such tensor spans at most 2 GiB.
constexpr uint64_t kMaxTensorBytes = 1ull << 31;

// One expand block: tokens of one adapter group (or tokens without an
// adapter) that share one pass over the adapter's B rows.
struct BlockDesc {
    int32_t tok_off;   // first entry of the block in the plan's token order
    int32_t n_tok;     // 1 .. kMaxBlockTokens
    int32_t r_pad;     // padded rank; 0 marks a block of tokens without an adapter
    int32_t slot0;     // token slot of its first token in its shrink block's partials
    float scale;       // the adapter's scale
    int32_t rt_before; // first rank tile of its shrink block (index into the tiles)
    uint32_t ext_lo;   // adapter extent byte offset in the slab, low and high words
    uint32_t ext_hi;
};
static_assert(sizeof(BlockDesc) == 32, "BlockDesc is 32 bytes");

// One rank tile (16 rows of A) of one shrink block: the shrink's unit of
// equal adapter bytes, whatever the adapter's rank.  tiles[rt_before + i] is
// tile i of a shrink block; its token rows are those of the shrink block.
struct TileDesc {
    int32_t tok_off;
    int32_t n_tok;
    int32_t r_pad;
    int32_t tile;      // rank tile index within the block
    int32_t block;     // group index
    int32_t pad1;
    uint32_t ext_lo;
    uint32_t ext_hi;
};
static_assert(sizeof(TileDesc) == 32, "TileDesc is 32 bytes");

// Shrink: one workgroup per unit (rank tile, k-chunk c, projection i), unit
// u = tile * nproj * c0 + c * nproj + i, so the projections that read the
// same x chunk are consecutive and are placed on one XCD.
// The 4 waves split the chunk's K range and are summed through LDS in a fixed
// order; the unit writes one float32 partial tile [16 * TT token slots][16
// ranks] at partial + u * TT * 256.
struct ShrinkArgs {
    const uint8_t *slab;
    const int32_t *tile_tok;     // [rt_total][kMaxBlockTokens] token rows, -1 padded
    const TileDesc *tiles;       // [rt_total]
    float *partial;
    const void *x;
    int64_t ldx;
    int64_t coef_a[LORA_MAX_PROJ];  // A block offset = extent + r_pad * esize * coef_a[i]
    int32_t nproj;
    int32_t h_in;
    int32_t h_in_pad;            // stored K: h_in rounded up to whole K-blocks
    int32_t kc;                  // k-chunk (elements): 4 waves x at most kShrinkFrags fragments
    int32_t c0;                  // number of k-chunks
    int32_t units;
    int32_t grid;                // workgroups launched: units rounded up to kXcds * nproj
    uint32_t x_bytes;            // buffer range (at most kMaxTensorBytes)
};

// fragments (16 bytes per lane) a shrink wave loads up front
template <int TT> constexpr int shrink_frags() { return TT <= 2 ? 8 : 4; }

// v from the shrink's partials, for the standalone shrink:
// v[t][i * r_max + j] = sum over chunks (j < r_pad), 0 for r_pad <= j < r_max.
struct ReduceArgs {
    const int32_t *tok;
    const BlockDesc *blocks;
    const float *partial;
    uint32_t partial_bytes;
    float *v;
    int64_t ldv;
    int32_t nb;
    int32_t nproj;
    int32_t c0;
    int32_t r_max;
};


// Expand: one workgroup per unit (block b, projection i, slice of 4 * ocw
// output rows; ocw = chunks * 16 * expand_tiles(ks)).  Each wave first issues the
// loads of all its B rows, then the workgroup gathers its tokens' v into LDS
// once (summing the shrink partials in a fixed order, or reading a caller's
// v), and each wave writes y = y_in + s * (B v), rounded once.
struct ExpandArgs {
    const uint8_t *slab;
    const int32_t *tok;          // plan token order
    const int32_t *block_tok;    // [nb][kMaxBlockTokens] token rows, -1 padded
    const BlockDesc *blocks;
    const float *partial;        // non-null: v = sum of partials
    const float *v;              // else: caller's v [T][ldv]
    uint32_t partial_bytes;
    void *y;
    const void *base;            // nullable: y_in = base, else y_in = y
    int64_t ldv;
    int64_t ldy;
    int64_t ldb;
    int64_t coef_b[LORA_MAX_PROJ];  // B block offset = extent + r_pad * esize * coef_b[i]
    int32_t h_out[LORA_MAX_PROJ];
    int32_t y_off[LORA_MAX_PROJ];
    int32_t oc_prefix[LORA_MAX_PROJ + 1];  // row chunks of projections before i
    int32_t tslices;             // MFMA expand: token slices of TT tiles per block
    int32_t nproj;
    int32_t chunks;              // row chunks per wave (16 * expand_tiles(ks) rows each)
    int32_t c0;                  // partial chunks (when partial != null)
    int32_t ptt;                 // 16-token tiles per shrink partial tile
    int32_t units;
    int32_t grid;
    int32_t r_max;
    uint32_t y_bytes;            // buffer ranges (each at most kMaxTensorBytes)
    uint32_t base_bytes;
    uint32_t v_bytes;            // range of a caller's v (when partial == null)
    // Jointly compressed adapters: sigma_kind 0 = none, 1 = diagonal cores,
    // 2 = full cores.  Token row tok_off + i of the plan order uses core
    // tok_sig[tok_off + i] (-1: none); core j of projection i of the call
    // starts at sigma + j * sig_stride + sig_off[i] (floats).
    const float *sigma;
    const int32_t *tok_sig;
    // Weighted plans: token row tok_off + i of the plan order scales its
    // delta by blk.scale * tok_w[tok_off + i] (null: by blk.scale).
    const float *tok_w;
    int64_t sig_stride;
    int64_t sig_off[LORA_MAX_PROJ];
    int32_t sigma_kind;
    // Decode expand: units by rank class.  Class k has units [cls_unit0[k],
    // cls_unit0[k + 1]) (unused entries INT32_MAX) over blocks from its first
    // one with one padded rank: cls_rb[k] = (first block << 8) | padded rank.
    // A block has, per projection i of the call, ceil(h_out[i] / rows) units
    // of rows = 1 << decode_unit_rows_log2(padded rank) output rows.
    int32_t cls_unit0[kMaxClasses + 1];
    int32_t cls_rb[kMaxClasses];
};

// Decode expand geometry.  A B row of r_pad elements is nv 16-byte vectors;
// the kernel is built for nvt = nv rounded up to a power of two, and a lane
// owns decode_rpl(nvt) rows of a step: 2 rows up to 64-byte rows, 1 row
// beyond, so one step of a wave streams 2-8 KB of B.  A wave's slice of a
// unit is one step; a unit is kWaves slices.  Units of 2 rows a lane beat
// 4 (fewer, longer workgroups) on every call of the full stack: 0.6-0.7 us
// less for the 4096-row projections, even for the 28672-row gate/up pair.
// Tokens without an adapter (r_pad 0) are copied 4 outputs a lane.
constexpr int decode_nvt(int r_pad, int esize) {
    int nv = (r_pad * esize + 15) / 16, t = 1;
    while (t < nv) t *= 2;
    return t;
}
constexpr int decode_rpl(int nvt) { return nvt >= 8 ? 1 : 2; }
constexpr int decode_wave_rows(int r_pad, int esize) {
    return r_pad == 0 ? 4 * kWaveSize : decode_rpl(decode_nvt(r_pad, esize)) * kWaveSize;
}
// log2 of a decode unit's rows, kWaves wave slices of decode_rpl rows per
// lane (1024 rows for r_pad 0); selects only, for the kernels' unit decode
constexpr int decode_unit_rows_log2(int r_pad, int esize) {
    return r_pad == 0 ? 10 : 8 + (decode_rpl(decode_nvt(r_pad, esize)) >= 4 ? 2
                                  : decode_rpl(decode_nvt(r_pad, esize)) == 2 ? 1 : 0);
}
constexpr bool decode_rows_agree() {
    for (int es = 2; es <= 4; es += 2)
        for (int r = 0; r <= LORA_MAX_RANK; r += 8)
            if ((1 << decode_unit_rows_log2(r, es)) != kWaves * decode_wave_rows(r, es)) return false;
    return true;
}
static_assert(decode_rows_agree(), "decode unit rows are kWaves wave slices");

// 16-row output tiles per expand wave, for kernels built for `ks` K-steps
// (ranks / (4 fragment elements)) at most: the wave keeps 8 B fragments.
constexpr int expand_tiles(int ks) { return ks >= 8 ? 1 : 8 / ks; }

// Sets the thread's last-error message (lora_last_error) and returns st.
lora_status set_error(lora_status st, const char *msg);

// Kernel launchers (kernels.hip).  dtype is a lora_dtype; tt is the number of
// 16-token tiles of the largest block (1, 2 or 4); ks the K-steps of the
// largest padded rank (bf16: 1 or 2, f32: 1, 2 or 4).
// mp: units of (rank tile, k-chunk) over every projection (tt 2 or 4, and
// 2 or 3 projections, only)
hipError_t launch_shrink(int dtype, int tt, bool mp, const ShrinkArgs &a, hipStream_t s);
// A [rank][h_in] row-major (device) -> K-blocked [h_in_pad / span][r_pad][span]
hipError_t launch_pack_a(int dtype, const void *src, int rank, int h_in, void *dst, int r_pad,
                         int h_in_pad, hipStream_t s);
hipError_t launch_reduce(int tt, const ReduceArgs &a, hipStream_t s);
hipError_t launch_expand(int dtype, int tt, int ks, const ExpandArgs &a, hipStream_t s);
// decode expand (every block of the plan within kValuTokens tokens)
// nvm: the largest decode_nvt of the launch's rank classes
hipError_t launch_expand_decode(int dtype, int nvm, const ExpandArgs &a, hipStream_t s);

}  // namespace lora

// Internal interface between the host library (pool, plan, C ABI) and the
// gfx950 kernels.  Not installed; the public interface is include/lora_sgmv.h.
#pragma once

#include <stddef.h>
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
// kDefaultLongGroup tokens is long, and takes kMaxBlockTokens-token blocks
// and the prefill kernel, but only when the batch's long groups hold
// kDefaultLongBatch tokens between them: fewer 64-token blocks leave most
// of the chip idle in the prefill kernel's launch, and the decode cut does
// better.  Both are defaults of a pool's plan options (lora_plan_opts).
constexpr int kDecodeBlockTokens = 4;
constexpr int kDefaultLongGroup = 48;
constexpr int kDefaultLongBatch = 1024;
constexpr int kValuTokens = kDecodeBlockTokens;  // token slots of the decode expand
// The shrink's chunk partials of one v entry are summed as kSumWays
// interleaved running sums (chunk c into sum c % kSumWays, in increasing c),
// then added in order: every kernel that sums them uses this one order.
constexpr int kSumWays = 4;
// rank classes of the decode expand: distinct padded ranks (multiples of 8)
// of the blocks, and 0 for tokens without an adapter
constexpr int kMaxClasses = LORA_MAX_RANK / 8 + 1;
// Prefill (long groups' blocks): one workgroup of kPrefillWaves waves per
// 16-token tile of a block, kPrefillTiles tiles per block, runs the whole
// delta of its tokens (see k_prefill).  16 waves fill a CU's 4 SIMDs with
// one workgroup.
#ifndef LORA_PREFILL_WAVES
#define LORA_PREFILL_WAVES 16
#endif
constexpr int kPrefillWaves = LORA_PREFILL_WAVES;
constexpr int kPrefillTiles = kMaxBlockTokens / kTile;
// Prefill launches aim for this many workgroups at least (by default): a
// launch with fewer tiles splits each tile's output rows over up to
// kPrefillMaxSplit workgroups (each then runs the A step of its tile itself).
constexpr int kDefaultPrefillGroups = 256;
constexpr int kPrefillMaxSplit = 4;
enum { kPrefillFused = 0, kPrefillShrink = 1, kPrefillExpand = 2 };
// Shrink: workgroups aimed for per launch (by default).  Fewer, longer
// k-chunks win over more, shorter ones here (the expand then also sums fewer
// partials): on the full stack 384 beat 1024 by 3.5% per step and 256 beat
// 384 by 0.5%; over the cost sweep (the full stack with 0-128 distinct
// adapters, and Zipf draws) 128 beat 256 by 7-8.5% for 1-8 distinct adapters
// and 1-2% for Zipf skews of 1.1-3, was never slower, and gives the full
// stack's calls the same k-chunks; 96, 64 and 32 lay between.
constexpr int kDefaultShrinkGroups = 128;
// upper limits of the launch targets a pool's plan options may set
constexpr int kMaxLaunchTarget = 1 << 16;
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

// What the debug build checks every unit against (see LORA_SGMV_DEBUG in
// kernels.hip): the slab's bytes (every adapter block a unit addresses lies
// inside), the tokens of the batch (every token row read from the plan lies
// in [0, num_tokens), -1 where a row may be absent) and the plan's rows
// (plan positions that index per-row tables lie in [0, num_rows)).
struct DebugBounds {
    uint64_t slab_bytes;
    int32_t num_tokens;
    int32_t num_rows;
};
// bits of the debug build's error word (lora_debug_checks)
enum : uint32_t { kDbgSlab = LORA_DEBUG_SLAB, kDbgToken = LORA_DEBUG_TOKEN,
                  kDbgRow = LORA_DEBUG_ROW };

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
    DebugBounds dbg;             // checked by the debug build only
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
    DebugBounds dbg;             // checked by the debug build only
};


// Decode expand: one workgroup per unit (see launch_expand_decode).  Each
// wave first issues the loads of its B rows, then the workgroup gathers its
// tokens' v into LDS once (summing the shrink partials in a fixed order, or
// reading a caller's v), and each wave writes y = y_in + s * (B v), rounded
// once.
struct ExpandArgs {
    const uint8_t *slab;
    const int32_t *tok;          // plan token order
    const int32_t *block_tok;    // [nb][kMaxBlockTokens] token rows, -1 padded
    const BlockDesc *blocks;
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
    int32_t nproj;
    int32_t c0;                  // partial chunks (when partial != null)
    int32_t ptt;                 // 16-token tiles per shrink partial tile
    int32_t units;               // (the grid is units rounded up to kXcds)
    int32_t r_max;
    uint32_t y_bytes;            // buffer ranges (each at most kMaxTensorBytes)
    uint32_t base_bytes;
    uint32_t v_bytes;            // range of a caller's v (when partial == null)
    uint32_t partial_bytes;
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
    DebugBounds dbg;             // checked by the debug build only
};

// Prefill: units are (long block, token tile, row part), unit u = (b *
// kPrefillTiles + tile) * osplit + part; the blocks [0, units / (kPrefillTiles
// * osplit)) of the plan are the long groups' blocks.  v rows (the shrink
// step's output, the expand step's input when it runs alone) are token rows
// of a caller's v, or plan positions (tok_off + i) of the workspace's region.
struct PrefillArgs {
    const uint8_t *slab;
    const int32_t *block_tok;    // [nb][kMaxBlockTokens] token rows, -1 padded
    const BlockDesc *blocks;
    const void *x;               // the shrink step's activations [T][ldx]
    void *y;                     // the expand step's output [T][ldy]
    const void *base;            // nullable: y_in = base, else y_in = y
    float *v;                    // v rows when a step runs alone
    const float *tok_w;          // weighted plans: per plan position (null: none)
    const float *sigma;          // cores of jointly compressed adapters
    const int32_t *tok_sig;      // core per plan position (-1: none)
    int64_t ldx;
    int64_t ldy;
    int64_t ldb;
    int64_t ldv;
    int64_t coef_a[LORA_MAX_PROJ];  // A block offset = extent + r_pad * esize * coef_a[i]
    int64_t coef_b[LORA_MAX_PROJ];  // B block offset = extent + r_pad * esize * coef_b[i]
    int64_t sig_stride;
    int64_t sig_off[LORA_MAX_PROJ];
    int32_t h_out[LORA_MAX_PROJ];
    int32_t y_off[LORA_MAX_PROJ];
    int32_t h_in;
    int32_t h_in_pad;            // stored K of A: h_in rounded up to whole K-blocks
    int32_t r_max;
    int32_t units;               // (the grid is units rounded up to kXcds)
    int32_t osplit;              // workgroups sharing a tile's output rows
    int32_t v_by_pos;            // v rows: plan positions (1) or token rows (0)
    int32_t sigma_kind;          // 0 none, 1 diagonal, 2 full (as ExpandArgs)
    uint32_t x_bytes;            // buffer ranges (each at most kMaxTensorBytes)
    uint32_t y_bytes;
    uint32_t base_bytes;
    DebugBounds dbg;             // checked by the debug build only
};

// Weighted merge of several adapters per request, in one pass: the shrink
// runs over every (token, slot) row as over the tokens of a plain plan (a
// row is the token's x row, grouped under its slot's adapter); the merge
// expand takes blocks of at most kValuTokens tokens of one segment (so the
// same slot adapters) and forms y = y_in + sum_k (w_k s_k) B_k v_k in float32,
// slot by slot in order, rounding y once.
constexpr int kMaxMerge = LORA_MAX_MERGE;

struct MergeSlot {
    uint32_t ext_lo, ext_hi;   // the slot adapter's extent
    int32_t r_pad;             // its padded rank; 0: an empty slot
    float scale;               // w * s, rounded to float32 once
};

struct MergeBlock {
    int32_t tok[kValuTokens];  // token rows, -1 padded
    int32_t n_tok;
    int32_t nslots;            // slots of the block's segment (<= kMaxMerge)
    int32_t pad[2];
    MergeSlot slot[kMaxMerge];
    // where row (token i, slot k) sits in the shrink's partials: the first
    // rank tile of its shrink block and its token slot in that block
    int32_t rt[kMaxMerge][kValuTokens];
    int32_t ps[kMaxMerge][kValuTokens];
};
static_assert(sizeof(MergeBlock) == 224, "MergeBlock is 224 bytes");
// the leading fields of a MergeBlock, which the merge expand copies whole
struct MergeHead {
    int32_t tok[kValuTokens];
    int32_t n_tok;
    int32_t nslots;
    int32_t pad[2];
};
static_assert(sizeof(MergeHead) == offsetof(MergeBlock, slot) &&
                  offsetof(MergeHead, nslots) == offsetof(MergeBlock, nslots),
              "MergeHead is the head of MergeBlock");

struct MergeArgs {
    const uint8_t *slab;
    const MergeBlock *mblocks;
    const float *partial;
    void *y;
    const void *base;            // nullable: y_in = base, else y_in = y
    int64_t ldy;
    int64_t ldb;
    int64_t coef_b[LORA_MAX_PROJ];
    int32_t h_out[LORA_MAX_PROJ];
    int32_t y_off[LORA_MAX_PROJ];
    int32_t nproj;
    int32_t c0;
    int32_t ptt;
    int32_t units;
    int32_t rows_log2;           // output rows of a unit (kWaves wave slices)
    uint32_t partial_bytes;
    uint32_t y_bytes;
    uint32_t base_bytes;
    DebugBounds dbg;             // checked by the debug build only
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

// Layout of a B block in the slab: h_out rows of r_pad elements, each row nv
// = r_pad * esize / 16 vectors of 16 bytes, permuted within slices of the
// decode expand's wave rows (64 * rpl rows, rpl = decode_rpl of the row's
// vector count; the last slice shorter).  In a slice of n rows the vectors
// run (i, v, l) with i < rpl, v < nv and l < n / rpl, vector v of row
// base + rpl * l + i at position (i * nv + v) * (n / rpl) + l: lane l of a
// wave holds rows base + rpl * l + i, so each of the wave's B loads (one i,
// one v) reads one contiguous run of n / rpl vectors.  The block's size is
// that of [h_out][r_pad].  sh = log2 rpl.
struct BLayout {
    int nv;
    int sh;
};
constexpr BLayout b_layout(int r_pad, int esize) {
    return BLayout{r_pad * esize / 16, decode_rpl(decode_nvt(r_pad, esize)) == 2 ? 1 : 0};
}
// byte offset of vector v of row o (o < h_out, v < nv) in its B block
constexpr uint32_t b_vec_off(BLayout b, int o, int v, int h_out) {
    const int base = o >> (6 + b.sh) << (6 + b.sh);
    const int n = h_out - base < (64 << b.sh) ? h_out - base : (64 << b.sh);
    const int q = o - base;
    return (uint32_t(base) * uint32_t(b.nv) +
            uint32_t(((q & b.sh) * b.nv + v) * (n >> b.sh) + (q >> b.sh))) * 16u;
}


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
// B [h_out][rank] row-major (device) -> the B block layout
// (b_vec_off), pad columns zero
hipError_t launch_pack_b(int dtype, const void *src, int rank, int h_out, void *dst, int r_pad,
                         hipStream_t s);
hipError_t launch_reduce(int tt, const ReduceArgs &a, hipStream_t s);
// prefill: mode kPrefillFused / kPrefillShrink / kPrefillExpand; np the
// call's projections (1..3); rtm the launch's largest rank tiles (1, 2 or 4);
// tpl the B row tiles per 16-byte load of the expand step: 4 or 2 when every
// long block's B row is one or two 16-byte vectors (rtm 1), else 1
hipError_t launch_prefill(int dtype, int mode, int np, int rtm, int tpl, const PrefillArgs &a,
                          int grid, hipStream_t s);
// decode expand (every block of the plan within kValuTokens tokens)
// nvm: the largest decode_nvt of the launch's rank classes
hipError_t launch_expand_decode(int dtype, int nvm, const ExpandArgs &a, int grid,
                                hipStream_t s);
// merge expand; nvm: the largest decode_nvt of the plan's slot adapters
// max_tok: the most tokens in one of the plan's merge blocks (1..kValuTokens)
hipError_t launch_expand_merge(int dtype, int nvm, int max_tok, const MergeArgs &a, int grid,
                               hipStream_t s);

// The library's static device scratch (sgmv_fused_static): the address of
// the current device's copy, found once per device, and its size in bytes.
constexpr uint64_t kStaticScratchBytes = uint64_t(LORA_STATIC_SCRATCH_MIB) << 20;
hipError_t static_scratch(void **ptr, uint64_t *bytes);

// Whether the kernels were built with LORA_SGMV_DEBUG, and the current
// device's debug error bits (after waiting for the device), cleared on request.
bool debug_build();
hipError_t debug_errors(uint32_t *bits, bool clear);

}  // namespace lora

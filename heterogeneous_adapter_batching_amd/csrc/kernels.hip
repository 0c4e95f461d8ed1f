// gfx950 kernels of the multi-adapter LoRA delta: shrink (v = A x) and expand
// (y = y_in + s * B v) over the groups of a heterogeneous batch.
//
// Both are thin dense contractions per adapter group (the segmented gather of
// SGMV: "Compress then Serve", rebuttal paragraph on Punica), and both are
// bound by HBM: a decode group streams its adapter's A and B rows once, a
// prefill group streams its token rows.  MFMA is used so that the arithmetic
// costs nothing next to the loads for any group size, not to reach a matrix
// throughput.
//
// Memory access: every global access is a buffer load or store through a
// wave-uniform resource whose size bounds the access; masked lanes use an
// out-of-range offset, which returns zero (loads) or is dropped (stores) by
// the hardware without touching memory.  So loads need no branch (the
// shrink's token rows excepted: lanes of absent rows are switched off, which
// spares the address path), and each wave issues all of its streaming loads
// before it waits for any.
//
// MFMA operand layout used throughout (16x16 output tile): lane l = 16 q + n
// holds row n of the left operand and column n of the right operand for the
// K-slice owned by lane group q; the 4 accumulators of lane l are output rows
// 4 q .. 4 q + 3 of column n.
//
// Precision: the A step's float32 intermediate ("Compress then Serve",
// rebuttal pseudocode, buffer of dtype float32) is kept exactly.  bf16 inputs
// multiply exactly inside the bf16 MFMA and sum in float32.  For the B step
// the float32 v is split into three bf16 pieces whose sum is v exactly, so
// B (h0 + h1 + h2) is the float32 product B v summed in float32.
#include <mutex>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "sgmv_internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int E = 8; };   // bf16 bit patterns
template <> struct Elem<float> { static constexpr int E = 4; };

// Buffer resources: raw (stride 0) with the byte size as the range.
constexpr uint32_t kOOB = 0x80000000u;        // offset of a masked lane: out of range
constexpr int kRsrcWord3 = 0x00020000;
// Non-temporal loads (early eviction from L2) for the shrink's A and the
// decode expand's B and y_in: each line is read whole by one instruction (the
// K-blocked A, the B block's row slices) and once; streaming B measured 2.7%
// faster per full-stack step and 5% on the multi-rank decode than the default
// policy, y_in 0.7% more on the full stack.  The shrink's partial sums keep
// the default policy (each is read by every unit of its block: 4.8% slower
// streamed).
// (While B rows were read 16 bytes a lane across 8 instructions the default
// policy was the faster one: the lines had to stay in L2 between the
// instructions.)  The prompt kernel reads B with the default policy: every
// token tile re-reads it from L2.
constexpr int kNT = 2;
// Outputs are stored at device scope (`sc1`, written through the L2): no
// dirty output lines are left for the kernel boundary to write back, which
// measured about 3% faster over the full stack than write-back stores.
constexpr int kOut = 16;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes),
                                             kRsrcWord3);
}
__device__ __forceinline__ uint32_t off_or_oob(bool ok, uint32_t off) { return ok ? off : kOOB; }

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
}
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kNT);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 bits (low half = a), rounded to nearest even by
// the hardware conversion (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c);

template <> __device__ __forceinline__ f32x4 mma<uint16_t>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// float32: the four elements of a lane's fragment are four consecutive K
// indices; MFMA m takes element m of both operands, so both sides see the
// same K permutation.
template <> __device__ __forceinline__ f32x4 mma<float>(u32x4 a, u32x4 b, f32x4 c) {
    const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ uint64_t extent(uint32_t lo, uint32_t hi) {
    return (uint64_t(hi) << 32) | lo;
}

// Debug build (LORA_SGMV_DEBUG): a unit checks every adapter block it
// addresses against the slab and every token row and plan position it reads
// against the batch; a failed check sets a bit of g_debug_errors and switches
// the access off (a zero-sized resource: the block reads as zeros; an absent
// row), so nothing outside the slab or the tensors is touched.  The release
// build compiles the checks out.
#ifdef LORA_SGMV_DEBUG
constexpr bool kDebug = true;
#else
constexpr bool kDebug = false;
#endif
__device__ uint32_t g_debug_errors;

// The byte range of the adapter block at slab offset `off`: `bytes`, or 0
// when it would leave the slab (debug build).
__device__ __forceinline__ uint32_t dbg_block(const DebugBounds &d, uint64_t off,
                                              uint64_t bytes) {
    if constexpr (kDebug) {
        if (off + bytes > d.slab_bytes) {
            atomicOr(&g_debug_errors, kDbgSlab);
            return 0u;
        }
    }
    return uint32_t(bytes);
}

// A token row from the plan: r, or -1 (absent) when it is outside [-1, T)
// (debug build).
__device__ __forceinline__ int dbg_token(const DebugBounds &d, int r) {
    if constexpr (kDebug) {
        if (r < -1 || r >= d.num_tokens) {
            atomicOr(&g_debug_errors, kDbgToken);
            return -1;
        }
    }
    return r;
}

// The token count of a descriptor whose rows [off, off + n) index per-row
// tables of the plan: n, or 0 when they leave the plan (debug build).
__device__ __forceinline__ int dbg_rows(const DebugBounds &d, int off, int n) {
    if constexpr (kDebug) {
        if (off < 0 || n < 0 || off + n > d.num_rows) {
            atomicOr(&g_debug_errors, kDbgRow);
            return 0;
        }
    }
    return n;
}

// Workgroup g runs on XCD g % kXcds.  Units are dealt to the XCDs in groups
// of `gs` consecutive units, round-robin: a group (e.g. the projections that
// read one x chunk) shares one L2, while consecutive groups, whose work may
// differ a lot (a popular adapter's block), spread over all XCDs and their
// links.  `grid` is a multiple of kXcds * gs.
__device__ __forceinline__ int xcd_unit(int gs) {
    const int g = blockIdx.x;
    const int x = g % kXcds, i = g / kXcds;
    return (i / gs) * (kXcds * gs) + x * gs + (i % gs);
}

// Workgroup g runs on XCD g % kXcds; here each XCD takes one contiguous range
// of ceil(units / kXcds) units, in order.  For the MFMA expand, whose units
// run block by block (token slices, then projections and row chunks), the
// units that read one token tile's shrink partials then share an L2, and so
// do the blocks of one adapter, which read the same B rows: with units dealt
// round-robin, a tile's partials were fetched once per XCD its units ran on
// (the prefill q/k/v expand fetched 1.4x its bytes).  Indices past `units`
// (at most kXcds - 1 of them, on the last XCDs) are idle.
__device__ __forceinline__ int xcd_range_unit(int units) {
    const int g = blockIdx.x;
    return (g % kXcds) * ((units + kXcds - 1) / kXcds) + g / kXcds;
}

// Reads plan memory (descriptors, token rows) through the constant address
// space, which promises that it stays unchanged for the whole dispatch: the
// plan workspace is written only by host uploads between launches, and the
// scalar cache is invalidated at each dispatch.  The dwords come in by
// scalar loads into SGPRs, so the unit's buffer resources are built in
// SGPRs (no loop around the buffer loads to make a VGPR descriptor
// uniform), and their wait counts apart from the vector loads.  3% per
// full-stack step against plain loads, which the compiler makes vector loads
// once a kernel may write memory.
template <typename D>
__device__ __forceinline__ D load_invariant(const D *p) {
    static_assert(sizeof(D) % 4 == 0, "whole dwords");
    typedef const __attribute__((address_space(4))) uint32_t *cptr;
    const cptr c = (cptr)p;
    D d;
    uint32_t *dst = reinterpret_cast<uint32_t *>(&d);
#pragma unroll
    for (int i = 0; i < int(sizeof(D) / 4); ++i) dst[i] = c[i];
    return d;
}

// Brings the whole kernel-argument block into the scalar cache in one
// round: one dword of every 32 bytes, loaded together and waited for once.
// The unit decode then reads its arguments in several dependent steps, each
// a scalar-cache hit instead of a trip to L2 or HBM (the arguments of a
// graph's kernels live in device memory).
template <typename Args>
__device__ __forceinline__ void warm_args() {
    typedef const __attribute__((address_space(4))) uint32_t *kptr;
    const kptr kp = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
    constexpr int N = int(sizeof(Args) + 31) / 32;
    static_assert(N <= 15, "at most 15 scalar loads in flight");
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = i < N ? kp[8 * i] : 0u;
    // every value live at once: the loads go out together, one wait
    asm volatile("" ::"s"(w[0]), "s"(w[1]), "s"(w[2]), "s"(w[3]), "s"(w[4]), "s"(w[5]),
                 "s"(w[6]), "s"(w[7]), "s"(w[8]), "s"(w[9]), "s"(w[10]), "s"(w[11]),
                 "s"(w[12]), "s"(w[13]), "s"(w[14]));
}

// ---------------------------------------------------------------- shrink ----
// NP > 1: a unit is (rank tile, k-chunk) and runs all NP projections of the
// call (a.nproj == NP) over one load of its x fragments: the A fragments of
// every projection, then x, all in flight together, then the projections'
// MFMAs and partial tiles one after the other (the same tiles as the
// per-projection units write).  For blocks of more than one 16-token tile,
// where x is most of the shrink's loads.
template <typename T, int TT, int NP>
__global__ __launch_bounds__(256) void k_shrink(const ShrinkArgs a) {
    constexpr bool MP = NP > 1;
    constexpr int E = Elem<T>::E;        // elements per 16-byte fragment
    constexpr int SPAN = 4 * E;          // K covered by one fragment over 4 lane groups
    constexpr int F = shrink_frags<TT>();
    __shared__ f32x4 red[kWaves][TT][kWaveSize];

    warm_args<ShrinkArgs>();
    const int u = xcd_unit(MP ? 1 : a.nproj);
    if (u >= a.units) return;            // whole workgroup: no barrier is skipped
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int n = lane & 15, q = lane >> 4;

    // unit -> (rank tile, chunk, projection): the descriptor and the token
    // rows of the tile load in parallel
    const int per = a.nproj * a.c0;
    const int key = MP ? u / a.c0 : u / per;
    int trow[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
        trow[tt] = dbg_token(a.dbg, a.tile_tok[key * kMaxBlockTokens + tt * kTile + n]);
    TileDesc td = load_invariant(a.tiles + key);
    if constexpr (kDebug)            // the tile's rows: inside the plan, at most TT tiles
        td.n_tok = min(dbg_rows(a.dbg, td.tok_off, td.n_tok), TT * kTile);
    int c, p0;
    if constexpr (MP) {
        c = u - key * a.c0;
        p0 = 0;
    } else {
        const int rem = u - key * per;
        c = rem / a.nproj;
        p0 = rem - (rem / a.nproj) * a.nproj;
    }

    // this wave's quarter of the chunk: at most F fragments
    const int kw = a.kc / kWaves;
    const int k_lo = c * a.kc + w * kw;
    const int k_hi = min(min(a.h_in, (c + 1) * a.kc), k_lo + kw);

    // A first: it depends on nothing but the descriptor.  A is K-blocked
    // [h_in_pad / SPAN][r_pad][SPAN], so the 16 rows x SPAN columns of one
    // fragment are one contiguous 1 KB (bf16) read.
    const int j = td.tile * kTile + n;
    const bool jv = j < td.r_pad;
    auto load_a = [&](int p, u32x4 (&af)[F]) {
        const uint64_t off = extent(td.ext_lo, td.ext_hi) +
                             uint64_t(td.r_pad) * sizeof(T) * uint64_t(a.coef_a[p]);
        const rsrc_t ar = make_rsrc(
            a.slab + off,
            dbg_block(a.dbg, off, uint64_t(td.r_pad) * uint64_t(a.h_in_pad) * sizeof(T)));
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int k = k_lo + f * SPAN + q * E;
            const uint32_t kb = uint32_t(k_lo / SPAN + f);
            af[f] = bload16_nt(ar, off_or_oob(jv && k < k_hi,
                                              ((kb * td.r_pad + j) * SPAN + q * E) * sizeof(T)));
        }
    };
    u32x4 af[NP][F];
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) load_a(p0 + pi, af[pi]);

    // then the token rows
    const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const int ntiles = (td.n_tok + kTile - 1) / kTile;   // wave-uniform
    u32x4 xf[TT][F];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = trow[tt];
        const bool tv = tt < ntiles && t >= 0;
        // lanes of absent token rows (a decode block holds 1-16 tokens of a
        // 16-row tile) are switched off rather than pointed out of range:
        // the address path then spends nothing on them (1.6% per decode
        // step, 2% per prefill step); the tile's loads still go out together
#pragma unroll
        for (int f = 0; f < F; ++f) xf[tt][f] = u32x4{0u, 0u, 0u, 0u};
        if (tv) {
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int k = k_lo + f * SPAN + q * E;
                xf[tt][f] = bload16(xr, off_or_oob(k < k_hi,
                                                   uint32_t(int64_t(t) * a.ldx + k) * sizeof(T)));
            }
        }
    }

#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
        f32x4 acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < F; ++f) {
            if (k_lo + f * SPAN >= k_hi) break;          // wave-uniform
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                if (tt < ntiles) acc[tt] = mma<T>(af[pi][f], xf[tt][f], acc[tt]);
        }

        // sum the 4 waves in a fixed order; lane holds ranks 4q..4q+3 of token n
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) red[w][tt][lane] = acc[tt];
        __syncthreads();
        // the partial tile of (rank tile, chunk, projection), as per-projection
        // units number them
        const int uu = key * per + c * a.nproj + p0 + pi;
        float *pt = a.partial + size_t(uu) * (TT * kTile * kTile);
        if constexpr (TT == 1) {
            // one token tile (decode blocks): wave 0 stores it, token slot n a
            // lane group; absent rows (a decode block fills 1-16 of the 16
            // slots) are never read, so their lanes are switched off (the
            // builds for 2-4 tiles keep the plain loop: this form held 4-6
            // more VGPRs there, one wave a SIMD fewer)
            if (w == 0 && ntiles > 0 && trow[0] >= 0) {
                const f32x4 s4 = red[0][0][lane] + red[1][0][lane] + red[2][0][lane] +
                                 red[3][0][lane];
                // partials are read once, by the next kernel
                __builtin_nontemporal_store(s4, reinterpret_cast<f32x4 *>(pt + n * kTile + q * 4));
            }
        } else {
            for (int i = threadIdx.x; i < ntiles * kWaveSize; i += kWaves * kWaveSize) {
                // token tiles past the block's last are never read: not stored
                const int tt = i / kWaveSize, ln = i % kWaveSize;
                const f32x4 s4 = red[0][tt][ln] + red[1][tt][ln] + red[2][tt][ln] + red[3][tt][ln];
                // partials are read once, by the next kernel
                __builtin_nontemporal_store(
                    s4, reinterpret_cast<f32x4 *>(pt + (tt * kTile + (ln & 15)) * kTile + (ln >> 4) * 4));
            }
        }
        if (MP) __syncthreads();                     // red is written again
    }
}

// Float offset of v entries (token slot `slot`, ranks j .. j + 3) of chunk 0
// in the shrink's partials, and the stride between chunks.  Unit u = (rank
// tile, chunk c, projection p) wrote tile u * ptt * 256: u = tile * nproj * c0
// + c * nproj + p, token slot s and rank i at s * 16 + i.
__device__ __forceinline__ uint32_t partial_off(int rt, int j, int slot, int p, int nproj, int c0,
                                                int ptt) {
    return uint32_t((rt + j / kTile) * nproj * c0 + p) * uint32_t(ptt * kTile * kTile) +
           uint32_t(slot * kTile + j % kTile);
}

// The whole chunk sum in the one order: the ways, then ((s0 + s1) + s2) + s3.
__device__ __forceinline__ f32x4 chunk_sum(rsrc_t pr, uint32_t off, uint32_t stride, int c0) {
    f32x4 w[kSumWays];
#pragma unroll
    for (int k = 0; k < kSumWays; ++k) w[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < c0; c += 8) {
        u32x4 part[8];
#pragma unroll
        for (int g = 0; g < 8; ++g)
            part[g] = bload16(pr, off_or_oob(c + g < c0, (off + uint32_t(c + g) * stride) * 4));
#pragma unroll
        for (int g = 0; g < 8; ++g)
            if (c + g < c0) w[g % kSumWays] += __builtin_bit_cast(f32x4, part[g]);
    }
    f32x4 s = w[0];
#pragma unroll
    for (int k = 1; k < kSumWays; ++k) s += w[k];
    return s;
}

// --------------------------------------------------------------- reduce -----
// One workgroup per (expand block, projection): v = sum of the chunk partials.
template <int TT>
__global__ __launch_bounds__(256) void k_reduce(const ReduceArgs a) {
    const int bp = blockIdx.x;
    const int b = bp / a.nproj, p = bp % a.nproj;
    BlockDesc blk = load_invariant(a.blocks + b);
    if constexpr (kDebug)
        blk.n_tok = min(dbg_rows(a.dbg, blk.tok_off, blk.n_tok), kMaxBlockTokens);
    const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
    const int quads = a.r_max / 4;
    for (int i = threadIdx.x; i < blk.n_tok * quads; i += blockDim.x) {
        const int ti = i / quads, j = (i % quads) * 4;
        f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < blk.r_pad)
            s4 = chunk_sum(pr, partial_off(blk.rt_before, j, blk.slot0 + ti, p, a.nproj, a.c0, TT),
                           uint32_t(a.nproj * TT * kTile * kTile), a.c0);
        const int t = dbg_token(a.dbg, a.tok[blk.tok_off + ti]);
        if (kDebug && t < 0) continue;
        *reinterpret_cast<f32x4 *>(a.v + int64_t(t) * a.ldv + int64_t(p) * a.r_max + j) = s4;
    }
}

// ---------------------------------------------------------------- expand ----
// v operand of one K-step for one token: bf16 pieces (3, summing to v
// exactly) or the float32 values themselves.
template <typename T> struct VOperand;

template <> struct VOperand<uint16_t> {
    static constexpr int kPieces = 3;
    u32x4 piece[3];
    // v = h0 + h1 + h2 exactly: each residual is exact in float32 and the
    // three 8-bit significands cover float32's 24.  Inf/NaN keep no residual.
    __device__ __forceinline__ void set(const float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = f[2 * i], b = f[2 * i + 1];
            const uint32_t w0 = bf16x2_rne(a, b);
            const float a1 = a - bf16_lo(w0), b1 = b - bf16_hi(w0);
            const uint32_t w1 = bf16x2_rne(a1, b1);
            const float a2 = a1 - bf16_lo(w1), b2 = b1 - bf16_hi(w1);
            uint32_t w2 = bf16x2_rne(a2, b2);
            uint32_t w1m = w1;
            if ((w0 & 0x7f80u) == 0x7f80u) { w1m &= 0xffff0000u; w2 &= 0xffff0000u; }
            if ((w0 & 0x7f800000u) == 0x7f800000u) { w1m &= 0xffffu; w2 &= 0xffffu; }
            piece[0][i] = w0;
            piece[1][i] = w1m;
            piece[2][i] = w2;
        }
    }
};

template <> struct VOperand<float> {
    static constexpr int kPieces = 1;
    u32x4 piece[1];
    __device__ __forceinline__ void set(const float (&f)[4]) {
        piece[0] = u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]),
                         __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};

// 4 consecutive outputs of one token: bf16 (8 bytes) or float32 (16 bytes)
template <typename T> struct Out4;
template <> struct Out4<uint16_t> {
    typedef u32x2 raw;
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, raw v) {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, int(off), 0, kOut);
    }
    static __device__ __forceinline__ void unpack(raw w, float (&o)[4]) {
        o[0] = bf16_lo(w[0]); o[1] = bf16_hi(w[0]);
        o[2] = bf16_lo(w[1]); o[3] = bf16_hi(w[1]);
    }
    static __device__ __forceinline__ raw pack(const float (&o)[4]) {
        return u32x2{bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3])};
    }
};
template <> struct Out4<float> {
    typedef u32x4 raw;
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, raw v) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, kOut);
    }
    static __device__ __forceinline__ void unpack(raw w, float (&o)[4]) {
        o[0] = __uint_as_float(w[0]); o[1] = __uint_as_float(w[1]);
        o[2] = __uint_as_float(w[2]); o[3] = __uint_as_float(w[3]);
    }
    static __device__ __forceinline__ raw pack(const float (&o)[4]) {
        return u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                     __float_as_uint(o[3])};
    }
};

// One output element: bf16 (2 bytes) or float32 (4 bytes).
template <typename T> struct Out1;
template <> struct Out1<uint16_t> {
    template <int AUX = 0>
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, AUX))
                               << 16);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(
            (unsigned short)(bf16x2_rne(v, 0.f) & 0xffffu), r, int(off), 0, kOut);
    }
};
template <> struct Out1<float> {
    template <int AUX = 0>
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, AUX));
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, int(off), 0, kOut);
    }
};

// The core step of jointly compressed adapters ("Compress then Serve",
// rebuttal pseudocode of add_lora_slice_with_sigma, step 2): each token's v
// (LDS rows [0, n_tok), ranks [0, r_pad)) becomes Sigma_j v with the token's
// core j, in float32, k ascending; a token without a core keeps v.  Full
// cores are r_max x r_max row-major, diagonal cores r_max values.  Up to
// MAXI entries per thread of NT threads.
template <int MAXI, int NT = kWaves * kWaveSize, typename Args>
__device__ __forceinline__ void apply_sigma(const Args &a, const BlockDesc &blk, int p,
                                            float (*vs)[LORA_MAX_RANK + 4]) {
    const int r = blk.r_pad;
    const int entries = blk.n_tok * r;
    float out[MAXI];
#pragma unroll
    for (int ii = 0; ii < MAXI; ++ii) {
        const int i = int(threadIdx.x) + ii * NT;
        out[ii] = 0.f;
        if (i < entries) {
            const int ti = i / r, j = i - (i / r) * r;
            const int sg = a.tok_sig[blk.tok_off + ti];
            float o = vs[ti][j];
            if (sg >= 0) {
                const float *core = a.sigma + int64_t(sg) * a.sig_stride + a.sig_off[p];
                if (a.sigma_kind == 1) {
                    o = core[j] * vs[ti][j];
                } else {
                    const f32x4 *row = reinterpret_cast<const f32x4 *>(core + int64_t(j) * a.r_max);
                    o = 0.f;
                    for (int k = 0; k < r; k += 4) {
                        const f32x4 c4 = row[k / 4];
                        o = __builtin_fmaf(c4[0], vs[ti][k], o);
                        o = __builtin_fmaf(c4[1], vs[ti][k + 1], o);
                        o = __builtin_fmaf(c4[2], vs[ti][k + 2], o);
                        o = __builtin_fmaf(c4[3], vs[ti][k + 3], o);
                    }
                }
            }
            out[ii] = o;
        }
    }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < MAXI; ++ii) {
        const int i = int(threadIdx.x) + ii * NT;
        if (i < entries) vs[i / r][i - (i / r) * r] = out[ii];
    }
    __syncthreads();
}

// v of a decode block (at most kValuTokens tokens) into LDS, in two parts so
// that its loads go out before the wave's B loads and its wait covers them
// alone (a wave's loads complete in issue order).  From the shrink's
// partials, thread (entry, way k) sums way k of the chunk sum of one v entry
// (4 ranks of one token) and the ways are added in order through LDS: the
// one chunk order.  Otherwise thread `entry` reads the entry from the
// caller's v.
struct VGather {
    u32x4 part[4];       // chunks k, k + 4, k + 8, k + 12 of way k (or the caller's entry)
    int e, k, ti, j;
    bool on;
};

template <bool Skip>
__device__ __forceinline__ void gather_issue(const ExpandArgs &a, const BlockDesc &blk,
                                             const int (&tr)[kValuTokens], int p, VGather &g) {
    const int quads = blk.r_pad / 4;                 // r_pad > 0
    const int entries = blk.n_tok * quads;           // <= kValuTokens * 16 = 64
    const int tid = int(threadIdx.x);
    if (a.partial) {
        g.k = tid % kSumWays;
        g.e = tid / kSumWays;
        g.on = g.e < entries;
        g.ti = g.e / quads;
        g.j = (g.e % quads) * 4;
        const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
        const uint32_t off = partial_off(blk.rt_before, g.j, blk.slot0 + g.ti, p, a.nproj, a.c0,
                                         a.ptt);
        const uint32_t stride = uint32_t(a.nproj * a.ptt * kTile * kTile);
        // Skip: a wave with no live entry (waves 1-3 of a block of at most
        // 16 entries) issues no load at all, by one wave-uniform branch, as a
        // masked lane still costs the address path.  These are the unit's
        // first loads, so the waits for the loads after them do not change.
        // 3-4.5% per full-stack expand; for wider rows (the rank-32 and -64
        // build) the multi-rank gate/up expand measured 0.9% slower, and a
        // branch per round of chunks as well raised that build past 64 VGPRs.
        if (!Skip || wave_id() * kWaveSize < entries * kSumWays) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = g.k + i * kSumWays;
                g.part[i] = bload16(pr, off_or_oob(g.on && c < a.c0, (off + uint32_t(c) * stride) * 4));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) g.part[i] = u32x4{0u, 0u, 0u, 0u};
        }
    } else {
        g.k = 0;
        g.e = tid;
        g.on = tid < entries;
        g.ti = g.on ? tid / quads : 0;
        g.j = (tid % quads) * 4;
        const rsrc_t vr = make_rsrc(a.v, a.v_bytes);
        // the entry's token row by selects (an indexed private array would
        // be placed in memory)
        const int row = g.ti == 0 ? tr[0] : g.ti == 1 ? tr[1] : g.ti == 2 ? tr[2] : tr[3];
        g.part[0] = bload16(vr, off_or_oob(g.on, uint32_t((int64_t(row) * a.ldv +
                                                           int64_t(p) * a.r_max + g.j) * 4)));
    }
}

__device__ __forceinline__ void gather_finish(const ExpandArgs &a, const BlockDesc &blk, int p,
                                              const VGather &g, float (*vs)[LORA_MAX_RANK + 4],
                                              f32x4 (*ways)[kSumWays]) {
    const int quads = blk.r_pad / 4;
    const int entries = blk.n_tok * quads;
    const int tid = int(threadIdx.x);
    if (a.partial) {
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (g.k + i * kSumWays < a.c0) s += __builtin_bit_cast(f32x4, g.part[i]);
        if (a.c0 > 4 * kSumWays) {                   // the rest of the way, in order
            const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
            const uint32_t off = partial_off(blk.rt_before, g.j, blk.slot0 + g.ti, p, a.nproj,
                                             a.c0, a.ptt);
            const uint32_t stride = uint32_t(a.nproj * a.ptt * kTile * kTile);
            for (int c = g.k + 4 * kSumWays; c < a.c0; c += kSumWays)
                s += __builtin_bit_cast(
                    f32x4, bload16(pr, off_or_oob(g.on, (off + uint32_t(c) * stride) * 4)));
        }
        if (g.on) ways[g.e][g.k] = s;
        __syncthreads();
        if (tid < entries) {
            const int ti = tid / quads, j = (tid % quads) * 4;
            f32x4 s4 = ways[tid][0];
#pragma unroll
            for (int w = 1; w < kSumWays; ++w) s4 += ways[tid][w];
            *reinterpret_cast<f32x4 *>(&vs[ti][j]) = s4;
        }
    } else if (g.on) {
        *reinterpret_cast<f32x4 *>(&vs[g.ti][g.j]) = __builtin_bit_cast(f32x4, g.part[0]);
    }
    __syncthreads();
}

// Decode expand on the vector ALUs, for one wave's slice [o_lo, o_hi) of a
// unit (one slice of the B block layout): lane owns rows o_lo + RPL * lane +
// i (i < RPL) and streams the NV 16-byte vectors of each B row (r_pad = nv *
// E values, nv <= NV), dotting them with every token's v (an LDS broadcast)
// in float32.  In the slab's B layout each (i, v) load of the wave is one
// contiguous run.  Loads go out in the order they are used: the v gather, B
// vector by vector, then y_in; so the dot products of the first vectors
// start while the rest arrive.  NT: the token slots the code is built for
// (the block's token count, or kValuTokens for a block of none), so that
// no y_in load or y store is issued for an absent slot.
template <typename T, int NV, bool Sig, int NT>
__device__ __forceinline__ void expand_valu(const ExpandArgs &a, const BlockDesc &blk,
                                            const int (&tr)[kValuTokens], int p, int o_lo,
                                            int o_hi, float (*vs)[LORA_MAX_RANK + 4],
                                            f32x4 (*ways)[kSumWays]) {
    static_assert(NT >= 1 && NT <= kValuTokens, "token slots of a decode block");
    constexpr int E = Elem<T>::E;
    constexpr int RPL = decode_rpl(NV);
    const int lane = threadIdx.x & 63;
    const int nv = blk.r_pad / E;                    // wave-uniform, <= NV
    const int nt = blk.n_tok;                        // wave-uniform, <= NT
    const int yoff = a.y_off[p];
    const uint64_t boff = extent(blk.ext_lo, blk.ext_hi) +
                          uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_b[p]);
    const rsrc_t br = make_rsrc(
        a.slab + boff,
        dbg_block(a.dbg, boff, uint64_t(a.h_out[p]) * uint64_t(blk.r_pad) * sizeof(T)));
    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const rsrc_t inr = a.base ? make_rsrc(a.base, a.base_bytes) : yr;
    const int64_t ld_in = a.base ? a.ldb : a.ldy;
    const uint32_t row_bytes = uint32_t(blk.r_pad) * sizeof(T);
    uint32_t in_row[NT], y_row[NT];                  // wave-uniform token rows (byte offsets)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const bool ok = t < nt && tr[t] >= 0;
        in_row[t] = ok ? uint32_t((int64_t(tr[t]) * ld_in + yoff) * sizeof(T)) : kOOB;
        y_row[t] = ok ? uint32_t((int64_t(tr[t]) * a.ldy + yoff) * sizeof(T)) : kOOB;
    }

    // PR (rows of at most 4 vectors, two rows a lane): a lane owns two
    // adjacent rows, so y_in and y of a token move 4 bytes a lane (bf16) in
    // one access instead of two of 2 bytes (1% per full-stack step).
    constexpr bool PR = RPL == 2;
    auto row_of = [&](int i) { return o_lo + RPL * lane + i; };
    VGather g;
    gather_issue<(NV <= 2)>(a, blk, tr, p, g);
    // the slice's vectors run (i, v, lane): vector v of the lane's row i at
    // ((i * nv + v) * lanes + lane) * 16 past the slice's first row
    const int lanes = (o_hi - o_lo) / RPL;          // o_hi - o_lo is a multiple of 8
    u32x4 bv[NV][RPL];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            bv[v][i] = bload16_nt(br, off_or_oob(lane < lanes && v < nv,
                                                 uint32_t(o_lo) * row_bytes +
                                                     uint32_t(((i * nv + v) * lanes + lane) * 16)));
    float yin[RPL][NT];
    if constexpr (PR) {
        const int row = row_of(0);
        const bool rok = row < o_hi;                 // o_hi is even: the pair is in or out
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t off = rok ? in_row[t] + uint32_t(row) * sizeof(T) : kOOB;
            if constexpr (sizeof(T) == 2) {
                const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(inr, int(off), 0, kNT);
                yin[0][t] = bf16_lo(w);
                yin[1][t] = bf16_hi(w);
            } else {
                const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(inr, int(off), 0, kNT);
                yin[0][t] = __uint_as_float(w[0]);
                yin[1][t] = __uint_as_float(w[1]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int row = row_of(i);
            const bool rok = row < o_hi;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                yin[i][t] =
                    Out1<T>::template load<kNT>(inr, rok ? in_row[t] + uint32_t(row) * sizeof(T) : kOOB);
        }
    }
    gather_finish(a, blk, p, g, vs, ways);
    if constexpr (Sig)
        apply_sigma<kValuTokens * LORA_MAX_RANK / (kWaves * kWaveSize)>(a, blk, p, vs);

    float d[RPL][NT];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) d[i][t] = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        // a wave-uniform guard rather than a loop exit, so the loop unrolls
        // fully and bv stays in registers
        if (v < nv) {
            // this vector's v one token at a time from LDS (broadcast
            // reads): E values live rather than every token's, 14 VGPRs
            // fewer (the rank-16 build at 8 waves a SIMD instead of 7),
            // 1.5% per full-stack step
            float f[RPL][E];
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                if constexpr (E == 8) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        f[i][2 * k] = bf16_lo(bv[v][i][k]);
                        f[i][2 * k + 1] = bf16_hi(bv[v][i][k]);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) f[i][k] = __uint_as_float(bv[v][i][k]);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < nt) {                        // wave-uniform
                    asm volatile("" ::: "memory");
                    float w[E];
#pragma unroll
                    for (int e = 0; e < E; e += 4) {
                        const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&vs[t][v * E + e]);
                        w[e] = w4[0]; w[e + 1] = w4[1]; w[e + 2] = w4[2]; w[e + 3] = w4[3];
                    }
#pragma unroll
                    for (int i = 0; i < RPL; ++i)
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            d[i][t] = __builtin_fmaf(f[i][e], w[e], d[i][t]);
                }
        }
    }
    // the delta's scale per token: the adapter's, times the token's weight
    // in a weighted plan (one float32 product)
    float sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        sc[t] = a.tok_w && t < nt ? blk.scale * a.tok_w[blk.tok_off + t] : blk.scale;
    if constexpr (PR) {
        const int row = row_of(0);
        const bool rok = row < o_hi;
#pragma unroll
        for (int t = 0; t < NT; ++t) {               // y_row[t] is kOOB for t >= nt
            const uint32_t off = rok ? y_row[t] + uint32_t(row) * sizeof(T) : kOOB;
            const float o0 = yin[0][t] + sc[t] * d[0][t], o1 = yin[1][t] + sc[t] * d[1][t];
            if constexpr (sizeof(T) == 2)
                __builtin_amdgcn_raw_buffer_store_b32(bf16x2_rne(o0, o1), yr, int(off), 0, kOut);
            else
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(o0), __float_as_uint(o1)},
                                                      yr, int(off), 0, kOut);
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int row = row_of(i);
            const bool rok = row < o_hi;
#pragma unroll
            for (int t = 0; t < NT; ++t)             // y_row[t] is kOOB for t >= nt
                Out1<T>::store(yr, rok ? y_row[t] + uint32_t(row) * sizeof(T) : kOOB,
                               yin[i][t] + sc[t] * d[i][t]);
        }
    }
}

// expand_valu built for the block's token count (a wave-uniform branch):
// a block of fewer tokens issues its y_in loads and y stores for those
// tokens only, instead of kValuTokens slots with the absent ones masked out
// of range (most decode blocks hold one token): 3.7% per full-stack step,
// 2.4% on the multi-rank decode.  Rows of 1-2 vectors only: below 4 tokens
// the builds for wider rows raise the kernel to 89-127 VGPRs (against
// 63-96, fewer waves a SIMD), and a single-token build for bf16 rows of 4
// vectors, which keeps 63, gave back the multi-rank gain.  The core step's
// build keeps one.
template <typename T, int NV, bool Sig>
__device__ __forceinline__ void expand_valu_nt(const ExpandArgs &a, const BlockDesc &blk,
                                               const int (&tr)[kValuTokens], int p, int o_lo,
                                               int o_hi, float (*vs)[LORA_MAX_RANK + 4],
                                               f32x4 (*ways)[kSumWays]) {
    static_assert(kValuTokens == 4 && NV <= 2, "builds per token count 1..4, rows of 1-2 vectors");
    if constexpr (Sig)
        return expand_valu<T, NV, Sig, kValuTokens>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    switch (blk.n_tok) {
    case 1: return expand_valu<T, NV, Sig, 1>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    case 2: return expand_valu<T, NV, Sig, 2>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    case 3: return expand_valu<T, NV, Sig, 3>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    default: return expand_valu<T, NV, Sig, kValuTokens>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    }
}

// Decode expand: plans whose blocks hold at most kValuTokens tokens.  A
// unit is (block, projection, kWaves slices of decode_wave_rows rows); the
// blocks are ordered by padded rank, and a unit's rank class, block,
// projection and slice follow from the kernel arguments alone, so the first
// loads are the block's descriptor and token rows (one round trip).
// Sig: the launch applies cores of jointly compressed adapters (a separate
// build, so the plain kernel keeps its registers).
// NVM: the largest count of 16-byte vectors per B row among the launch's
// rank classes; a build per bound, so that a batch of small ranks runs with
// the registers (and occupancy) of its own class rather than of rank 64.
template <typename T, bool Sig, int NVM>
__global__ __launch_bounds__(256) void k_expand_decode(const ExpandArgs a) {
    constexpr int VS = LORA_MAX_RANK + 4;
    __shared__ float vs[kValuTokens][VS];
    __shared__ f32x4 ways[kValuTokens * LORA_MAX_RANK / 4][kSumWays];

    warm_args<ExpandArgs>();
    const int u = xcd_unit(1);
    int cbase = 0, rb = a.cls_rb[0];
#pragma unroll
    for (int i = 1; i < kMaxClasses; ++i) {
        const int u0 = a.cls_unit0[i];
        if (u >= u0) { cbase = u0; rb = a.cls_rb[i]; }
    }
    const int nproj = a.nproj;
    int hout[LORA_MAX_PROJ];
#pragma unroll
    for (int i = 0; i < LORA_MAX_PROJ; ++i) hout[i] = a.h_out[i];
    if (u >= a.units) return;                        // whole workgroup
    const int r_pad = rb & 0xff;
    const int lg = decode_unit_rows_log2(r_pad, sizeof(T));
    int cnt[LORA_MAX_PROJ], upb = 0;
#pragma unroll
    for (int i = 0; i < LORA_MAX_PROJ; ++i) {
        cnt[i] = i < nproj ? (hout[i] + (1 << lg) - 1) >> lg : 0;
        upb += cnt[i];
    }
    const int ur = u - cbase;
    const int bi = ur / upb;
    const int rem = ur - bi * upb;
    const int b = (rb >> 8) + bi;
    int p = 0, first = 0, run = 0;                   // projection and its first unit
#pragma unroll
    for (int i = 0; i < LORA_MAX_PROJ; ++i) {
        if (i < nproj && rem >= run) { p = i; first = run; }
        run += cnt[i];
    }
    const int slice = rem - first;

    BlockDesc blk = load_invariant(a.blocks + b);
    const int4 bt4 = load_invariant(reinterpret_cast<const int4 *>(a.block_tok + b * kMaxBlockTokens));
    const int tr[kValuTokens] = {dbg_token(a.dbg, bt4.x), dbg_token(a.dbg, bt4.y),
                                 dbg_token(a.dbg, bt4.z), dbg_token(a.dbg, bt4.w)};
    static_assert(kValuTokens == 4, "token rows load as one int4");
    if constexpr (kDebug)            // the block's rows: inside the plan, at most 4
        blk.n_tok = min(dbg_rows(a.dbg, blk.tok_off, blk.n_tok), kValuTokens);

    int h_out = hout[0];
#pragma unroll
    for (int i = 1; i < LORA_MAX_PROJ; ++i) h_out = p == i ? hout[i] : h_out;
    const int wrows = 1 << (lg - 2);                 // rows of one wave slice
    const int o_lo = min(h_out, (slice * kWaves + wave_id()) * wrows);
    const int o_hi = min(h_out, o_lo + wrows);

    if (r_pad == 0) {                // tokens without an adapter: y = base, 4 outputs a lane
        if (!a.base) return;
        const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
        const rsrc_t br = make_rsrc(a.base, a.base_bytes);
        const int o = o_lo + 4 * (threadIdx.x & 63);
        const int yoff = a.y_off[p];
#pragma unroll
        for (int t = 0; t < kValuTokens; ++t) {
            const bool ok = t < blk.n_tok && o < o_hi;
            const auto v4 = Out4<T>::load(
                br, ok ? uint32_t((int64_t(tr[t]) * a.ldb + yoff + o) * sizeof(T)) : kOOB);
            Out4<T>::store(yr, ok ? uint32_t((int64_t(tr[t]) * a.ldy + yoff + o) * sizeof(T)) : kOOB,
                           v4);
        }
        return;
    }
    switch (decode_nvt(r_pad, sizeof(T))) {         // <= NVM for every class of the launch
    case 1: return expand_valu_nt<T, 1, Sig>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    case 2: if constexpr (NVM >= 2) return expand_valu_nt<T, 2, Sig>(a, blk, tr, p, o_lo, o_hi, vs, ways);
            return;
    case 4: if constexpr (NVM >= 4) return expand_valu<T, 4, Sig, kValuTokens>(a, blk, tr, p, o_lo, o_hi, vs, ways);
            return;
    case 8: if constexpr (NVM >= 8) return expand_valu<T, 8, Sig, kValuTokens>(a, blk, tr, p, o_lo, o_hi, vs, ways);
            return;
    default:
        if constexpr (sizeof(T) == 4 && NVM >= 16) return expand_valu<T, 16, Sig, kValuTokens>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    }
}

// Merge expand: y = y_in + sum_k (w_k s_k) B_k v_k for the tokens of a merge
// block (at most kValuTokens tokens of one segment, so the same slot
// adapters), slot by slot in order, in float32, rounded once.  A unit is
// (block, projection, kWaves wave slices of rows) as in the decode expand,
// and a lane owns the same rows o_lo + RPL * lane + i (i < RPL).  For each
// slot the v of the block's (token, slot) rows is gathered into LDS from the
// shrink's partials (the one chunk order: thread (entry, way) sums one way,
// the ways are added in order), the slot adapter's B rows stream in, and
// each lane adds the slot's scaled dot products to its running outputs,
// which start at y_in.  B keeps the default cache policy here: a block is
// one request, so a popular adapter's B rows are read by many blocks
// (streaming them was 2.4% slower per merged full-stack step).  Issuing slot
// k + 1's loads before slot k's gather and dot products held 96 VGPRs
// instead of 60, 5 waves a SIMD instead of 8, and was 6% slower.
template <typename T, int NVM> struct MergeLoads {
    static constexpr int RPL = decode_rpl(NVM);
    MergeSlot sl;
    u32x4 part[4];                // chunks kk, kk + 4, kk + 8, kk + 12 of the thread's way
    u32x4 bv[NVM][RPL];           // the lane's B rows, vector by vector
    uint32_t off;                 // the thread's v entry in the partials
    bool live;                    // a slot with an adapter
};

// NT: the token slots of the launch's blocks, 1 when every merge block of
// the plan holds one token (a decode batch: one request, one token), so
// that no y_in load, y store or LDS row is spent on absent slots.
template <typename T, int NVM, int NT>
__global__ __launch_bounds__(256) void k_expand_merge(const MergeArgs a) {
    static_assert(NT == 1 || NT == kValuTokens, "merge builds for 1 or kValuTokens tokens");
    constexpr int E = Elem<T>::E;
    constexpr int RPL = decode_rpl(NVM);
    constexpr int VS = LORA_MAX_RANK + 4;
    constexpr bool PR = RPL == 2;                    // two adjacent rows a lane
    __shared__ float vs[NT][VS];
    __shared__ f32x4 ways[NT * LORA_MAX_RANK / 4][kSumWays];

    warm_args<MergeArgs>();
    const int u = xcd_unit(1);
    if (u >= a.units) return;                        // whole workgroup
    const int nproj = a.nproj;
    const int lg = a.rows_log2;
    int hout[LORA_MAX_PROJ], cnt[LORA_MAX_PROJ], upb = 0;
#pragma unroll
    for (int i = 0; i < LORA_MAX_PROJ; ++i) {
        hout[i] = a.h_out[i];
        cnt[i] = i < nproj ? (hout[i] + (1 << lg) - 1) >> lg : 0;
        upb += cnt[i];
    }
    const int b = u / upb;
    const int rem = u - b * upb;
    int p = 0, first = 0, run = 0;
#pragma unroll
    for (int i = 0; i < LORA_MAX_PROJ; ++i) {
        if (i < nproj && rem >= run) { p = i; first = run; }
        run += cnt[i];
    }
    const int slice = rem - first;
    // the block's head (token rows and counts) as a private copy; the slot
    // entries are read from the plan at each slot (a private copy of the
    // whole block, indexed by the slot, would live in scratch memory)
    const MergeBlock *mbp = a.mblocks + b;
    MergeHead mb = load_invariant(reinterpret_cast<const MergeHead *>(mbp));
    if constexpr (kDebug) {          // token rows inside the batch, at most 4 of them
        mb.n_tok = min(max(mb.n_tok, 0), kValuTokens);
#pragma unroll
        for (int t = 0; t < kValuTokens; ++t) mb.tok[t] = dbg_token(a.dbg, mb.tok[t]);
    }
    if constexpr (NT < kValuTokens)  // the host launches this build for blocks of NT tokens
        mb.n_tok = min(mb.n_tok, NT);
    int h_out = hout[0];
#pragma unroll
    for (int i = 1; i < LORA_MAX_PROJ; ++i) h_out = p == i ? hout[i] : h_out;
    const int wrows = 1 << (lg - 2);
    const int o_lo = min(h_out, (slice * kWaves + wave_id()) * wrows);
    const int o_hi = min(h_out, o_lo + wrows);
    const int lane = threadIdx.x & 63;
    const int tid = int(threadIdx.x);
    const int yoff = a.y_off[p];
    auto row_of = [&](int i) { return o_lo + RPL * lane + i; };

    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const rsrc_t inr = a.base ? make_rsrc(a.base, a.base_bytes) : yr;
    const int64_t ld_in = a.base ? a.ldb : a.ldy;
    uint32_t in_row[NT], y_row[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const bool ok = t < mb.n_tok && mb.tok[t] >= 0;
        in_row[t] = ok ? uint32_t((int64_t(mb.tok[t]) * ld_in + yoff) * sizeof(T)) : kOOB;
        y_row[t] = ok ? uint32_t((int64_t(mb.tok[t]) * a.ldy + yoff) * sizeof(T)) : kOOB;
    }

    const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
    const uint32_t stride = uint32_t(a.nproj * a.ptt * kTile * kTile);
    const int kk = tid % kSumWays, e = tid / kSumWays;   // the thread's (entry, way)
    // the loads of slot k: its plan entry, its partials and its B rows
    auto issue = [&](int k, MergeLoads<T, NVM> &ld) {
        ld.live = false;
        if (k >= mb.nslots) return;                  // wave-uniform
        ld.sl = load_invariant(&mbp->slot[k]);
        if (ld.sl.r_pad == 0) return;                // an empty slot: wave-uniform
        ld.live = true;
        const int quads = ld.sl.r_pad / 4;
        const bool on = e < mb.n_tok * quads;
        const int ti = on ? e / quads : 0;
        const int j = on ? (e - ti * quads) * 4 : 0;
        // the row's place in the partials, by selects (an indexed private
        // array would be placed in memory)
        static_assert(kValuTokens == 4, "a slot's partial places load as one int4 each");
        const int4 rt4 = load_invariant(reinterpret_cast<const int4 *>(mbp->rt[k]));
        const int4 ps4 = load_invariant(reinterpret_cast<const int4 *>(mbp->ps[k]));
        const int rt = ti == 0 ? rt4.x : ti == 1 ? rt4.y : ti == 2 ? rt4.z : rt4.w;
        const int ps = ti == 0 ? ps4.x : ti == 1 ? ps4.y : ti == 2 ? ps4.z : ps4.w;
        ld.off = on ? partial_off(rt, j, ps, p, a.nproj, a.c0, a.ptt) : kOOB / 4;
        // one token: at most 16 entries, all in wave 0; waves 1-3 issue no
        // partial-sum load (a wave-uniform branch; a masked lane still costs
        // the address path)
        if (NT > 1 || wave_id() == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = kk + i * kSumWays;
                ld.part[i] = bload16(pr, off_or_oob(on && c < a.c0, (ld.off + uint32_t(c) * stride) * 4));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ld.part[i] = u32x4{0u, 0u, 0u, 0u};
        }
        const uint64_t boff = extent(ld.sl.ext_lo, ld.sl.ext_hi) +
                              uint64_t(ld.sl.r_pad) * sizeof(T) * uint64_t(a.coef_b[p]);
        const rsrc_t br = make_rsrc(a.slab + boff,
                                    dbg_block(a.dbg, boff, uint64_t(h_out) * uint64_t(ld.sl.r_pad) *
                                                               sizeof(T)));
        const int nv = ld.sl.r_pad / E;
        const BLayout bl = b_layout(ld.sl.r_pad, sizeof(T));   // the slot's B layout
#pragma unroll
        for (int v = 0; v < NVM; ++v)
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const int row = row_of(i);
                ld.bv[v][i] = bload16(br, off_or_oob(row < o_hi && v < nv,
                                                     b_vec_off(bl, row, v, h_out)));
            }
    };

    MergeLoads<T, NVM> cur;
    float acc[RPL][NT];                              // y_in, then the running outputs
    if constexpr (PR) {
        const int row = row_of(0);
        const bool rok = row < o_hi;                 // o_hi is even: the pair is in or out
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t off = rok ? in_row[t] + uint32_t(row) * sizeof(T) : kOOB;
            if constexpr (sizeof(T) == 2) {
                const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(inr, int(off), 0, kNT);
                acc[0][t] = bf16_lo(w);
                acc[1][t] = bf16_hi(w);
            } else {
                const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(inr, int(off), 0, kNT);
                acc[0][t] = __uint_as_float(w[0]);
                acc[1][t] = __uint_as_float(w[1]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int row = row_of(i);
            const bool rok = row < o_hi;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[i][t] = Out1<T>::template load<kNT>(
                    inr, rok ? in_row[t] + uint32_t(row) * sizeof(T) : kOOB);
        }
    }

#pragma unroll
    for (int k = 0; k < kMaxMerge; ++k) {
        if (k >= mb.nslots) break;                   // wave-uniform
        issue(k, cur);
        if (cur.live) {                              // wave-uniform
            const int quads = cur.sl.r_pad / 4;
            const int entries = mb.n_tok * quads;
            const bool on = e < entries;
            // finish the gather in the one chunk order
            f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kk + i * kSumWays < a.c0) s4 += __builtin_bit_cast(f32x4, cur.part[i]);
            for (int c = kk + 4 * kSumWays; c < a.c0; c += kSumWays)
                s4 += __builtin_bit_cast(
                    f32x4, bload16(pr, off_or_oob(on, (cur.off + uint32_t(c) * stride) * 4)));
            if (on) ways[e][kk] = s4;
            __syncthreads();
            if (tid < entries) {
                const int t2 = tid / quads, j2 = (tid - (tid / quads) * quads) * 4;
                f32x4 w4 = ways[tid][0];
#pragma unroll
                for (int w = 1; w < kSumWays; ++w) w4 += ways[tid][w];
                *reinterpret_cast<f32x4 *>(&vs[t2][j2]) = w4;
            }
            __syncthreads();
            // this slot's dot products, added to the running outputs
            const int nv = cur.sl.r_pad / E;
            float d[RPL][NT];
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int t = 0; t < NT; ++t) d[i][t] = 0.f;
#pragma unroll
            for (int v = 0; v < NVM; ++v) {
                if (v < nv) {                        // wave-uniform
                    float f[RPL][E];
#pragma unroll
                    for (int i = 0; i < RPL; ++i) {
                        if constexpr (E == 8) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                f[i][2 * q] = bf16_lo(cur.bv[v][i][q]);
                                f[i][2 * q + 1] = bf16_hi(cur.bv[v][i][q]);
                            }
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q) f[i][q] = __uint_as_float(cur.bv[v][i][q]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        if (t < mb.n_tok) {          // wave-uniform
                            float wv[E];
#pragma unroll
                            for (int q = 0; q < E; q += 4) {
                                const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&vs[t][v * E + q]);
                                wv[q] = w4[0]; wv[q + 1] = w4[1]; wv[q + 2] = w4[2]; wv[q + 3] = w4[3];
                            }
#pragma unroll
                            for (int i = 0; i < RPL; ++i)
#pragma unroll
                                for (int q = 0; q < E; ++q)
                                    d[i][t] = __builtin_fmaf(f[i][q], wv[q], d[i][t]);
                        }
                }
            }
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[i][t] = acc[i][t] + cur.sl.scale * d[i][t];
            __syncthreads();                         // vs and ways are written again
        }
    }
    if constexpr (PR) {
        const int row = row_of(0);
        const bool rok = row < o_hi;
#pragma unroll
        for (int t = 0; t < NT; ++t) {               // y_row[t] is kOOB for absent tokens
            const uint32_t off = rok ? y_row[t] + uint32_t(row) * sizeof(T) : kOOB;
            if constexpr (sizeof(T) == 2)
                __builtin_amdgcn_raw_buffer_store_b32(bf16x2_rne(acc[0][t], acc[1][t]), yr,
                                                      int(off), 0, kOut);
            else
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{__float_as_uint(acc[0][t]), __float_as_uint(acc[1][t])}, yr, int(off), 0,
                    kOut);
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int row = row_of(i);
            const bool rok = row < o_hi;
#pragma unroll
            for (int t = 0; t < NT; ++t)             // y_row[t] is kOOB for absent tokens
                Out1<T>::store(yr, rok ? y_row[t] + uint32_t(row) * sizeof(T) : kOOB, acc[i][t]);
        }
    }
}

// --------------------------------------------------------------- prefill ----
// The whole delta of one 16-token tile of a long group's block in one
// workgroup of kPrefillWaves waves, with nothing handed between kernels:
//
//  1. v = A x for each of the call's projections (the A step at scale 1.0,
//     "Compress then Serve", rebuttal pseudocode, step 1): the waves split
//     K into equal runs of K-blocks; each wave chains its MFMAs in K order,
//     loading the next batch of x and A fragments while it multiplies the
//     current one, and the waves' tiles are added in wave order through LDS.
//     v stays float32 in LDS.
//  2. y = y_in + s B v over every output row of the call's projections (step
//     3): the rows are split among the waves (and among the workgroups of a
//     tile when a launch has few tiles); each wave runs the MFMA expand's row
//     loop on its rows.
//
// A tile's x rows are read once from HBM and its y rows once each way, the
// adapter's A and B come from L2 (a group's tiles are consecutive units and
// xcd_range_unit keeps them on one XCD), and v never reaches memory.  MODE
// runs step 1 alone (v written to memory, the standalone shrink) or step 2
// alone (v read from memory), with the same arithmetic as the fused form.
//
// K-blocks per batch of the shrink step, for `pairs` (projection, rank tile)
// accumulators: a batch is FB x fragments and FB x pairs A fragments; two
// batches in flight stay within about 72 VGPRs.
#ifndef LORA_PREFILL_EARLY
#define LORA_PREFILL_EARLY 0
#endif
constexpr int prefill_kbatch(int pairs) { return pairs <= 1 ? 4 : pairs <= 3 ? 2 : 1; }
constexpr int prefill_ksm(int rtm, int e) {
    return (rtm * kTile + 4 * e - 1) / (4 * e) == 3 ? 4 : (rtm * kTile + 4 * e - 1) / (4 * e);
}
// Row tiles per chunk of the expand step: a wave holds B fragments for 8 /
// ksm row tiles of ksm K-steps each, halved so that two chunks in flight fit
// the 128 VGPRs of a 16-wave workgroup (whole pairs of tiles in bf16).
constexpr int prefill_otw(int ksm, int esize) {
    const int half = (ksm >= 8 ? 1 : 8 / ksm) / 2;
    return esize == 2 ? (half < 2 ? 2 : half) : (half < 1 ? 1 : half);
}

// The B step of a prefill workgroup for one wave: output rows of every
// projection of the call, this wave's share of each (whole 32-row pairs),
// visited as one run of OTW-tile chunks across the projections, so that two
// chunks are in flight at every step, also where one projection's rows end
// and the next one's begin.  Per chunk: the B rows (OTW 16-row tiles, TPL
// tiles per 16-byte load when r_pad packs them) and y_in of the tile's
// tokens, then the MFMAs against v (from LDS, in three bf16 pieces) and
// y = y_in + s B v, rounded once.  bf16 rows come in the pair order of the
// MFMA expand (a lane stores 8 consecutive outputs).
template <typename T, int NP, int KSM, int TPL, int OTW, int NBUF, bool EARLY, typename Before>
__device__ __forceinline__ void prefill_rows(const PrefillArgs &a, const BlockDesc &blk,
                                             int share, int shares, int n, int q, int trow,
                                             const int (&lrow)[2], float tsc,
                                             float (*vs)[kTile][LORA_MAX_RANK + 4],
                                             u32x4 *stage, Before before) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;
    constexpr int NL = TPL == 1 ? OTW * KSM : OTW / TPL;   // B loads per chunk
    constexpr int CH = OTW * kTile;                  // rows per chunk
    constexpr bool PAIR = sizeof(T) == 2;
    static_assert(!PAIR || OTW % 2 == 0, "row tiles of a chunk come in pairs");
    constexpr int NY = PAIR ? OTW / 2 : OTW;         // y_in loads per chunk
    // bf16 chunks of 4 row tiles: a token's 64 outputs are one 128-byte
    // line, so y_in and y move 8 tokens' whole lines per instruction (lane l:
    // token 8 j + l / 8 of instruction j, bytes 16 (l % 8)) and pass through
    // the wave's LDS rows (stage, 9 16-byte units a token: no bank
    // conflicts) to and from the MFMA layout; otherwise 16 tokens x 64 bytes
    // per instruction straight from the MFMA layout
    constexpr bool STAGE = PAIR && OTW == 4;
    constexpr int SROW = 9;                          // 16-byte units per staged token row
    typedef typename Out4<T>::raw raw;
    typedef typename std::conditional<PAIR, u32x4, raw>::type yraw;
    const int G = TPL == 1 ? 4 : 4 / TPL;            // vectors per row (packed)
    const int ks_n = (blk.r_pad + SPAN - 1) / SPAN;  // <= KSM

    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const rsrc_t inr = a.base ? make_rsrc(a.base, a.base_bytes) : yr;
    const int64_t ld_in = a.base ? a.ldb : a.ldy;
    const bool tv = trow >= 0;
    // an absent token's row offsets are out of range already
    const uint32_t in_row = tv ? uint32_t(int64_t(trow) * ld_in * sizeof(T)) : kOOB;
    const uint32_t y_row = tv ? uint32_t(int64_t(trow) * a.ldy * sizeof(T)) : kOOB;
    const int lane = n + kTile * q;
    uint32_t in_line[2], y_line[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        in_line[j] = lrow[j] >= 0 ? uint32_t(int64_t(lrow[j]) * ld_in * sizeof(T)) : kOOB;
        y_line[j] = lrow[j] >= 0 ? uint32_t(int64_t(lrow[j]) * a.ldy * sizeof(T)) : kOOB;
    }
    const int lane_tile = TPL == 1 ? 0 : q / G;
    const int lane_vec = TPL == 1 ? q : q % G;       // the lane's 16-byte vector of a B row
    const BLayout bl = b_layout(blk.r_pad, sizeof(T));
    auto brow = [&](int tile, int nn) {
        return PAIR ? (tile & ~1) * kTile + 8 * (nn >> 2) + 4 * (tile & 1) + (nn & 3)
                    : tile * kTile + nn;
    };

    // per-projection values by selects (an indexed array would be placed in
    // memory)
    auto sel = [](int p, auto v0, auto v1, auto v2) {
        return NP == 1 || p == 0 ? v0 : NP == 2 || p == 1 ? v1 : v2;
    };
    // this wave's rows [lo, hi) of each projection, in chunks
    int lo[NP], hi[NP], nch[NP];
    int total = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int h = a.h_out[p];
        const int rw = ((h + shares - 1) / shares + 2 * kTile - 1) / (2 * kTile) * (2 * kTile);
        lo[p] = min(h, share * rw);
        hi[p] = min(h, lo[p] + rw);
        nch[p] = (hi[p] - lo[p] + CH - 1) / CH;
        total += nch[p];
    }
    // chunk i -> (projection, first row); past the last chunk: past hi
    auto where = [&](int i, int &p, int &o0) {
        p = 0;
#pragma unroll
        for (int k = 0; k < NP - 1; ++k)
            if (p == k && i >= nch[k]) {
                i -= nch[k];
                p = k + 1;
            }
        o0 = sel(p, lo[0], lo[NP > 1 ? 1 : 0], lo[NP > 2 ? 2 : 0]) + i * CH;
    };

    auto load = [&](int i, u32x4 (&bf)[NL], yraw (&yin)[NY]) {
        int p, o0;
        where(i, p, o0);
        const int h = sel(p, a.h_out[0], a.h_out[1], a.h_out[2]);
        const int top = sel(p, hi[0], hi[NP > 1 ? 1 : 0], hi[NP > 2 ? 2 : 0]);
        const uint64_t boff = extent(blk.ext_lo, blk.ext_hi) +
                              uint64_t(blk.r_pad) * sizeof(T) *
                                  uint64_t(sel(p, a.coef_b[0], a.coef_b[1], a.coef_b[2]));
        const rsrc_t br = make_rsrc(a.slab + boff,
                                    dbg_block(a.dbg, boff, uint64_t(h) * uint64_t(blk.r_pad) *
                                                               sizeof(T)));
        const uint32_t yoff = uint32_t(sel(p, a.y_off[0], a.y_off[1], a.y_off[2])) * sizeof(T);
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int t = TPL == 1 ? l / KSM : l * TPL;
            const int ks = TPL == 1 ? l % KSM : 0;
            const int row = o0 + brow(t + lane_tile, n);
            const bool ok = i < total && row < top &&
                            (TPL > 1 || (ks < ks_n && ks * SPAN + q * E < blk.r_pad));
            bf[l] = bload16(br, off_or_oob(ok, b_vec_off(bl, row, lane_vec + ks * (SPAN / E), h)));
        }
#pragma unroll
        for (int oy = 0; oy < NY; ++oy) {
            if constexpr (STAGE) {
                const int o = o0 + 8 * (lane & 7);
                yin[oy] = bload16(inr, i < total && o < top
                                           ? in_line[oy] + yoff + uint32_t(o) * sizeof(T) : kOOB);
            } else {
                const int o = PAIR ? o0 + oy * 2 * kTile + 8 * q : o0 + oy * kTile + 4 * q;
                const uint32_t off =
                    i < total && o < top ? in_row + yoff + uint32_t(o) * sizeof(T) : kOOB;
                if constexpr (PAIR) yin[oy] = bload16(inr, off);
                else yin[oy] = Out4<T>::load(inr, off);
            }
        }
    };

    VOperand<T> vop[KSM];
    int vp = -1;                                     // projection whose v vop holds
    auto compute = [&](int i, const u32x4 (&bf)[NL], const yraw (&yin)[NY]) {
        int p, o0;
        where(i, p, o0);
        const int top = sel(p, hi[0], hi[NP > 1 ? 1 : 0], hi[NP > 2 ? 2 : 0]);
        const uint32_t yoff = uint32_t(sel(p, a.y_off[0], a.y_off[1], a.y_off[2])) * sizeof(T);
        if (p != vp) {                               // wave-uniform: v of projection p
            vp = p;
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
                float f[E];
                const int j0 = TPL == 1 ? ks * SPAN + q * E : (q % G) * E;
                const bool ok = tv && ks < ks_n && j0 < blk.r_pad;
                const int row = ok ? n : 0, col = ok ? j0 : 0;
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&vs[p][row][col + e]);
                    f[e] = ok ? w4[0] : 0.f; f[e + 1] = ok ? w4[1] : 0.f;
                    f[e + 2] = ok ? w4[2] : 0.f; f[e + 3] = ok ? w4[3] : 0.f;
                }
                vop[ks].set(f);
            }
        }
        // B v of row tile ot: D rows 4 q .. 4 q + 3 of the tile
        auto tile_acc = [&](int ot) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            if (TPL == 1) {
#pragma unroll
                for (int ks = 0; ks < KSM; ++ks) {
                    if (ks >= ks_n) continue;
#pragma unroll
                    for (int pc = VOperand<T>::kPieces - 1; pc >= 0; --pc)
                        acc = mma<T>(bf[ot * KSM + ks], vop[ks].piece[pc], acc);
                }
            } else {
                const bool mine = q / G == ot % TPL;     // lane groups of this tile
#pragma unroll
                for (int pc = VOperand<T>::kPieces - 1; pc >= 0; --pc) {
                    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
                    acc = mma<T>(bf[ot / TPL], mine ? vop[0].piece[pc] : z, acc);
                }
            }
            return acc;
        };
        if constexpr (STAGE) {                       // y_in rows into the MFMA layout
#pragma unroll
            for (int j = 0; j < NY; ++j) stage[(8 * j + (lane >> 3)) * SROW + (lane & 7)] = yin[j];
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int oy = 0; oy < NY; ++oy) {
            const int obase = o0 + oy * (PAIR ? 2 : 1) * kTile;
            if (!STAGE && obase >= top) break;       // wave-uniform
            if constexpr (PAIR) {
                const f32x4 a0 = tile_acc(2 * oy), a1 = tile_acc(2 * oy + 1);
                const int o = obase + 8 * q;
                const u32x4 wv = STAGE ? stage[n * SROW + 4 * oy + q] : yin[oy];
                float out[8];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    out[2 * k] = bf16_lo(wv[k]) + tsc * a0[2 * k];
                    out[2 * k + 1] = bf16_hi(wv[k]) + tsc * a0[2 * k + 1];
                    out[4 + 2 * k] = bf16_lo(wv[2 + k]) + tsc * a1[2 * k];
                    out[5 + 2 * k] = bf16_hi(wv[2 + k]) + tsc * a1[2 * k + 1];
                }
                const u32x4 pk = u32x4{bf16x2_rne(out[0], out[1]), bf16x2_rne(out[2], out[3]),
                                       bf16x2_rne(out[4], out[5]), bf16x2_rne(out[6], out[7])};
                if constexpr (STAGE)
                    stage[n * SROW + 4 * oy + q] = pk;
                else
                    __builtin_amdgcn_raw_buffer_store_b128(
                        pk, yr, int(o < top ? y_row + yoff + uint32_t(o) * sizeof(T) : kOOB), 0,
                        kOut);
            } else {
                const f32x4 acc = tile_acc(oy);
                const int o = obase + 4 * q;
                float in[4], out[4];
                Out4<T>::unpack(yin[oy], in);
#pragma unroll
                for (int k = 0; k < 4; ++k) out[k] = in[k] + tsc * acc[k];
                Out4<T>::store(yr, o < top ? y_row + yoff + uint32_t(o) * sizeof(T) : kOOB,
                               Out4<T>::pack(out));
            }
        }
        if constexpr (STAGE) {                       // y rows out of the MFMA layout
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < NY; ++j) {
                const int o = o0 + 8 * (lane & 7);
                __builtin_amdgcn_raw_buffer_store_b128(
                    stage[(8 * j + (lane >> 3)) * SROW + (lane & 7)], yr,
                    int(o < top ? y_line[j] + yoff + uint32_t(o) * sizeof(T) : kOOB), 0, kOut);
            }
            __builtin_amdgcn_wave_barrier();
        }
    };

    // a ring of NBUF chunks: the loads of NBUF - 1 chunks ahead are in flight
    // while a chunk is computed (loads past the last chunk are masked)
    u32x4 bf[NBUF][NL];
    yraw yin[NBUF][NY];
    if constexpr (EARLY) {
#pragma unroll
        for (int k = 0; k < NBUF - 1; ++k) load(k, bf[k], yin[k]);
        before();                                    // v into LDS meanwhile
    } else {
        before();
#pragma unroll
        for (int k = 0; k < NBUF - 1; ++k) load(k, bf[k], yin[k]);
    }
    for (int i = 0; i < total; i += NBUF) {
#pragma unroll
        for (int k = 0; k < NBUF; ++k) {
            if (i + k >= total) break;               // wave-uniform
            load(i + k + NBUF - 1, bf[(k + NBUF - 1) % NBUF], yin[(k + NBUF - 1) % NBUF]);
            compute(i + k, bf[k], yin[k]);
        }
    }
}

template <typename T, int NP, int RTM, int MODE, int TPLK>
__global__ __launch_bounds__(kPrefillWaves * kWaveSize, 4) void k_prefill(const PrefillArgs a) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;
    constexpr int W = kPrefillWaves;
    constexpr int NT = W * kWaveSize;
    constexpr int VS = LORA_MAX_RANK + 4;
    constexpr int PAIRS = NP * RTM;
    constexpr int FB = prefill_kbatch(PAIRS);
    constexpr bool DB = PAIRS <= 8;
    constexpr int KSM = prefill_ksm(RTM, E);
    constexpr int OTW = prefill_otw(KSM, int(sizeof(T)));
#ifndef LORA_PREFILL_NBUF
#define LORA_PREFILL_NBUF 2
#endif
    constexpr int NBUF = sizeof(T) == 2 && KSM == 1 ? LORA_PREFILL_NBUF : 2;
    __shared__ float vs[NP][kTile][VS];
    __shared__ f32x4 red[MODE == kPrefillExpand ? 1 : 2][W][kWaveSize];
    // per wave: 16 staged token rows of 9 16-byte units (bf16 x lines of the
    // A step, y_in and y lines of the B step)
    __shared__ u32x4 stage[W][kTile * 9];

    warm_args<PrefillArgs>();
    const int u = xcd_range_unit(a.units);
    if (u >= a.units) return;                        // whole workgroup
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int n = lane & 15, q = lane >> 4;
    // unit -> (block, token tile, row part)
    const int part = u % a.osplit;
    const int bt = u / a.osplit;
    const int b = bt / kPrefillTiles, tile = bt % kPrefillTiles;
    BlockDesc blk = load_invariant(a.blocks + b);
    if constexpr (kDebug)            // the block's rows: inside the plan, at most one block
        blk.n_tok = min(dbg_rows(a.dbg, blk.tok_off, blk.n_tok), kMaxBlockTokens);
    const int off = tile * kTile;
    if (off >= blk.n_tok) return;                    // whole workgroup: an empty tile
    blk.tok_off += off;
    blk.slot0 += off;
    blk.n_tok = min(kTile, blk.n_tok - off);
    // the tile's 16 token rows (-1 past n_tok) by scalar loads, which go out
    // with the descriptor's; each lane then picks its own row by selects, so
    // no vector round trip precedes the first loads
    struct Rows { int32_t r[kTile]; };
    Rows rows = load_invariant(reinterpret_cast<const Rows *>(a.block_tok) +
                               (b * kMaxBlockTokens + off) / kTile);
    if constexpr (kDebug) {
#pragma unroll
        for (int k = 0; k < kTile; ++k) rows.r[k] = dbg_token(a.dbg, rows.r[k]);
    }
    int trow = rows.r[0];
#pragma unroll
    for (int k = 1; k < kTile; ++k) trow = n == k ? rows.r[k] : trow;
    // token rows of the lines layout (staged loads and stores): token
    // 8 j + lane / 8 of instruction j = 0, 1
    int lrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = 8 * j + (lane >> 3);
        lrow[j] = rows.r[0];
#pragma unroll
        for (int k = 1; k < kTile; ++k) lrow[j] = t == k ? rows.r[k] : lrow[j];
    }

    // step 1 (v = A x into LDS), for the fused and shrink-only forms
    auto step1 = [&]() {
        if constexpr (MODE != kPrefillExpand) {
            // ---- step 1: v = A x, K split over the waves
            const int nkb = (a.h_in + SPAN - 1) / SPAN;
            const int per_w = (nkb + W - 1) / W;
            const int kb0 = min(nkb, w * per_w), kb1 = min(nkb, kb0 + per_w);
            const int rtn = (blk.r_pad + kTile - 1) / kTile;   // rank tiles, <= RTM
            const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
            // an absent token's row offset is out of range already (kOOB + k
            // bytes stays at or above 2^31)
            const uint32_t xrow = trow >= 0 ? uint32_t(int64_t(trow) * a.ldx * sizeof(T)) : kOOB;
            rsrc_t ar[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const uint64_t aoff = extent(blk.ext_lo, blk.ext_hi) +
                                      uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_a[p]);
                ar[p] = make_rsrc(a.slab + aoff,
                                  dbg_block(a.dbg, aoff, uint64_t(blk.r_pad) *
                                                             uint64_t(a.h_in_pad) * sizeof(T)));
            }
            f32x4 acc[NP][RTM];
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int rt = 0; rt < RTM; ++rt) acc[p][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

            // bf16 batches of whole K-block pairs: x moves as 8 tokens' 128-byte
            // lines per instruction (two K-blocks of a token) and passes through
            // the wave's LDS rows into the MFMA layout, instead of 16 tokens x
            // 64 bytes per instruction
            constexpr bool STAGEX = sizeof(T) == 2 && FB % 2 == 0;
            uint32_t xline[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                xline[j] = lrow[j] >= 0 ? uint32_t(int64_t(lrow[j]) * a.ldx * sizeof(T)) : kOOB;
            u32x4 *xs = stage[w];
            // a batch: K-blocks kb .. kb + FB - 1 (masked past kb1, so the loads
            // need no branch); A is K-blocked [h_in_pad / SPAN][r_pad][SPAN]
            auto load = [&](int kb, u32x4 (&xf)[FB], u32x4 (&af)[NP][RTM][FB]) {
#pragma unroll
                for (int f = 0; f < FB; ++f) {
                    const bool ok = kb + f < kb1;
                    const int k = (kb + f) * SPAN + q * E;
#pragma unroll
                    for (int p = 0; p < NP; ++p)
#pragma unroll
                        for (int rt = 0; rt < RTM; ++rt) {
                            const int j = rt * kTile + n;
                            af[p][rt][f] = bload16(
                                ar[p], off_or_oob(ok && j < blk.r_pad,
                                                  uint32_t(((kb + f) * blk.r_pad + j) * SPAN + q * E) *
                                                      sizeof(T)));
                        }
                    if constexpr (STAGEX) {
                        // instruction f: K-blocks kb + 2 (f / 2) and the next,
                        // tokens 8 (f % 2) .. + 7, 16 bytes at 16 (lane % 8)
                        const int b2 = kb + 2 * (f / 2);
                        const int kk = b2 * SPAN + 8 * (lane & 7);
                        const bool okl = b2 + ((lane & 7) >> 2) < kb1 && kk < a.h_in;
                        xf[f] = bload16_nt(xr, okl ? xline[f % 2] + uint32_t(kk) * sizeof(T)
                                                   : kOOB);
                    } else {
                        xf[f] = bload16_nt(xr, ok && k < a.h_in ? xrow + uint32_t(k) * sizeof(T)
                                                                : kOOB);
                    }
                }
            };
            auto mult = [&](int kb, const u32x4 (&xl)[FB], const u32x4 (&af)[NP][RTM][FB]) {
                u32x4 xf[FB];
                if constexpr (STAGEX) {
                    // lines into the MFMA layout: token n, K-block kb + f, the
                    // 16 bytes of lane group q
#pragma unroll
                    for (int f2 = 0; f2 < FB; f2 += 2) {
                        xs[(lane >> 3) * 9 + (lane & 7)] = xl[f2];
                        xs[(8 + (lane >> 3)) * 9 + (lane & 7)] = xl[f2 + 1];
                        __builtin_amdgcn_wave_barrier();
                        xf[f2] = xs[n * 9 + q];
                        xf[f2 + 1] = xs[n * 9 + 4 + q];
                        __builtin_amdgcn_wave_barrier();
                    }
                } else {
#pragma unroll
                    for (int f = 0; f < FB; ++f) xf[f] = xl[f];
                }
#pragma unroll
                for (int f = 0; f < FB; ++f) {
                    if (kb + f >= kb1) break;            // wave-uniform
#pragma unroll
                    for (int p = 0; p < NP; ++p)
#pragma unroll
                        for (int rt = 0; rt < RTM; ++rt)
                            if (rt < rtn) acc[p][rt] = mma<T>(af[p][rt][f], xf[f], acc[p][rt]);
                }
            };
            u32x4 xa[FB], aa[NP][RTM][FB];
            if constexpr (DB) {
                u32x4 xb[FB], ab[NP][RTM][FB];
                load(kb0, xa, aa);
                for (int kb = kb0; kb < kb1; kb += 2 * FB) {
                    load(kb + FB, xb, ab);
                    mult(kb, xa, aa);
                    if (kb + FB >= kb1) break;
                    load(kb + 2 * FB, xa, aa);
                    mult(kb + FB, xb, ab);
                }
            } else {
                for (int kb = kb0; kb < kb1; kb += FB) {
                    load(kb, xa, aa);
                    mult(kb, xa, aa);
                }
            }

            // the waves' tiles added in wave order: lane (n, q) holds ranks
            // 4 q .. 4 q + 3 of token n; two LDS buffers in turn, one barrier a pair
            int k = 0;
#pragma unroll
            for (int pr = 0; pr < PAIRS; ++pr) {
                const int p = pr / RTM, rt = pr % RTM;
                if (rt >= rtn) continue;                 // uniform over the workgroup
                red[k & 1][w][lane] = acc[p][rt];
                __syncthreads();
                if (threadIdx.x < kTile * kTile) {
                    const int ln = threadIdx.x >> 2, e = threadIdx.x & 3;
                    float s = red[k & 1][0][ln][e];
#pragma unroll
                    for (int ww = 1; ww < W; ++ww) s += red[k & 1][ww][ln][e];
                    vs[p][ln & 15][rt * kTile + 4 * (ln >> 4) + e] = s;
                }
                ++k;
            }
            __syncthreads();
        }
    };
    if constexpr (MODE == kPrefillShrink) {
        step1();
        // v rows of the tile's tokens: r_max entries per projection,
        // zero past the padded rank
        const int quads = a.r_max / 4;
        for (int i = threadIdx.x; i < blk.n_tok * NP * quads; i += NT) {
            const int ti = i / (NP * quads), rem = i - ti * (NP * quads);
            const int p = rem / quads, j = (rem - p * quads) * 4;
            const f32x4 s4 = j < blk.r_pad ? *reinterpret_cast<const f32x4 *>(&vs[p][ti][j])
                                           : f32x4{0.f, 0.f, 0.f, 0.f};
            const int64_t row = a.v_by_pos ? int64_t(blk.tok_off + ti)
                                           : int64_t(a.block_tok[b * kMaxBlockTokens + off + ti]);
            if (kDebug && (a.v_by_pos ? dbg_rows(a.dbg, int(row), 1) == 0
                                      : dbg_token(a.dbg, int(row)) < 0))
                continue;
            *reinterpret_cast<f32x4 *>(a.v + row * a.ldv + int64_t(p) * a.r_max + j) = s4;
        }
    } else {
        // v in LDS (step 1, or the tile's v rows from memory), cores applied;
        // run by the expand step once its first loads are out
        auto before = [&]() {
            if constexpr (MODE == kPrefillFused) {
                step1();
            } else {
                // v of the tile's tokens from memory
                const int quads = blk.r_pad / 4;
                for (int i = threadIdx.x; i < blk.n_tok * NP * quads; i += NT) {
                    const int ti = i / (NP * quads), rem = i - ti * (NP * quads);
                    const int p = rem / quads, j = (rem - p * quads) * 4;
                    const int64_t row = a.v_by_pos ? int64_t(blk.tok_off + ti)
                                                   : int64_t(a.block_tok[b * kMaxBlockTokens + off + ti]);
                    if (kDebug && (a.v_by_pos ? dbg_rows(a.dbg, int(row), 1) == 0
                                              : dbg_token(a.dbg, int(row)) < 0)) {
                        *reinterpret_cast<f32x4 *>(&vs[p][ti][j]) = f32x4{0.f, 0.f, 0.f, 0.f};
                        continue;
                    }
                    *reinterpret_cast<f32x4 *>(&vs[p][ti][j]) = *reinterpret_cast<const f32x4 *>(
                        a.v + row * a.ldv + int64_t(p) * a.r_max + j);
                }
                __syncthreads();
            }
            if (a.sigma_kind) {
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    apply_sigma<kTile * LORA_MAX_RANK / NT, NT>(a, blk, p, vs[p]);
            }
        };
        const float tsc =
            a.tok_w && n < blk.n_tok ? blk.scale * a.tok_w[blk.tok_off + n] : blk.scale;
        // each projection's rows in kPrefillWaves * osplit shares of whole
        // 32-row pairs; share part * W + w is this wave's
        const int shares = W * a.osplit, share = part * W + w;
        // the first chunks' loads go out before step 1 where the registers
        // allow (up to 4 accumulator tiles)
        constexpr bool EARLY = LORA_PREFILL_EARLY && PAIRS <= 4;
        prefill_rows<T, NP, KSM, TPLK, OTW, NBUF, EARLY>(a, blk, share, shares, n, q, trow, lrow,
                                                         tsc, vs, stage[w], before);
    }
}

// ----------------------------------------------------------------- pack ----
// A [rank][h_in] (row-major, device) -> K-blocked [h_in_pad / SPAN][r_pad][SPAN]
// with zeros in the pad rows and columns; one thread per 16-byte vector.
template <typename T>
__global__ __launch_bounds__(256) void k_pack_a(const T *src, int rank, int h_in, T *dst,
                                                int r_pad, int h_in_pad) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;
    const int vecs = h_in_pad / E * r_pad;             // 16-byte vectors of the block
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= vecs) return;
    const int kb = i / (r_pad * 4), rem = i % (r_pad * 4);
    const int j = rem / 4, c = (rem % 4) * E;
    const int k = kb * SPAN + c;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (j < rank && k < h_in) v = *reinterpret_cast<const u32x4 *>(src + int64_t(j) * h_in + k);
    *reinterpret_cast<u32x4 *>(dst + (int64_t(kb) * r_pad + j) * SPAN + c) = v;
}

// B [h_out][rank] (row-major, device) -> the slab's B block layout (row
// slices of permuted 16-byte vectors, b_vec_off) with zeros in the pad
// columns; one thread per 16-byte vector, read element by element (rank
// need not fill whole vectors).
template <typename T>
__global__ __launch_bounds__(256) void k_pack_b(const T *src, int rank, int h_out, T *dst,
                                                int r_pad) {
    constexpr int E = Elem<T>::E;
    const BLayout bl = b_layout(r_pad, sizeof(T));
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= h_out * bl.nv) return;
    const int o = i / bl.nv, v = i % bl.nv;
    T e[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int j = v * E + k;
        e[k] = j < rank ? src[int64_t(o) * rank + j] : T(0);
    }
    u32x4 w;
    __builtin_memcpy(&w, e, sizeof w);
    *reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(dst) + b_vec_off(bl, o, v, h_out)) = w;
}

template <typename T>
hipError_t shrink_dispatch(int tt, bool mp, const ShrinkArgs &a, hipStream_t s) {
    const dim3 grid(a.grid), block(kWaves * kWaveSize);
    const int np = mp ? a.nproj : 1;
    switch (tt * 4 + np) {
    case 1 * 4 + 1: hipLaunchKernelGGL((k_shrink<T, 1, 1>), grid, block, 0, s, a); break;
    case 2 * 4 + 1: hipLaunchKernelGGL((k_shrink<T, 2, 1>), grid, block, 0, s, a); break;
    case 2 * 4 + 2: hipLaunchKernelGGL((k_shrink<T, 2, 2>), grid, block, 0, s, a); break;
    case 2 * 4 + 3: hipLaunchKernelGGL((k_shrink<T, 2, 3>), grid, block, 0, s, a); break;
    case 4 * 4 + 1: hipLaunchKernelGGL((k_shrink<T, 4, 1>), grid, block, 0, s, a); break;
    case 4 * 4 + 2: hipLaunchKernelGGL((k_shrink<T, 4, 2>), grid, block, 0, s, a); break;
    case 4 * 4 + 3: hipLaunchKernelGGL((k_shrink<T, 4, 3>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// kernels built: TPL (B rows packed per load) 2 or 4 only for launches whose
// long blocks all have one padded rank of 1 or 2 vectors (RTM 1), and only
// for the modes with an expand step
template <typename T, int MODE, int TPL>
hipError_t prefill_np(int np, int rtm, const PrefillArgs &a, int g, hipStream_t s) {
    const dim3 grid(g), block(kPrefillWaves * kWaveSize);
#define LORA_PREFILL(NP, RTM)                                                                      \
    case NP * 8 + RTM:                                                                            \
        hipLaunchKernelGGL((k_prefill<T, NP, RTM, MODE, TPL>), grid, block, 0, s, a);             \
        break;
    if constexpr (TPL == 1) {
        switch (np * 8 + rtm) {
            LORA_PREFILL(1, 1) LORA_PREFILL(1, 2) LORA_PREFILL(1, 4)
            LORA_PREFILL(2, 1) LORA_PREFILL(2, 2) LORA_PREFILL(2, 4)
            LORA_PREFILL(3, 1) LORA_PREFILL(3, 2) LORA_PREFILL(3, 4)
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (np * 8 + rtm) {
            LORA_PREFILL(1, 1) LORA_PREFILL(2, 1) LORA_PREFILL(3, 1)
        default: return hipErrorInvalidValue;
        }
    }
#undef LORA_PREFILL
    return hipGetLastError();
}

template <typename T>
hipError_t prefill_modes(int mode, int np, int rtm, int tpl, const PrefillArgs &a, int g,
                         hipStream_t s) {
    if (mode == kPrefillShrink) return prefill_np<T, kPrefillShrink, 1>(np, rtm, a, g, s);
    if (mode != kPrefillFused && mode != kPrefillExpand) return hipErrorInvalidValue;
    const bool fused = mode == kPrefillFused;
    switch (tpl) {
    case 1: return fused ? prefill_np<T, kPrefillFused, 1>(np, rtm, a, g, s)
                         : prefill_np<T, kPrefillExpand, 1>(np, rtm, a, g, s);
    case 2: return fused ? prefill_np<T, kPrefillFused, 2>(np, rtm, a, g, s)
                         : prefill_np<T, kPrefillExpand, 2>(np, rtm, a, g, s);
    case 4: return fused ? prefill_np<T, kPrefillFused, 4>(np, rtm, a, g, s)
                         : prefill_np<T, kPrefillExpand, 4>(np, rtm, a, g, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Scratch for callers that cannot allocate (sgmv_fused_static): the shrink
// partials of such a call.  Each device holds its own copy at its own address
// until the process ends; host code must never pass the array's name to a
// kernel or a copy (in host code it is a host-side stand-in), only the
// address hipGetSymbolAddress gives for the current device, found once per
// device and kept.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void **ptr, uint64_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kStaticScratchBytes;
    return hipSuccess;
}

bool debug_build() { return kDebug; }

hipError_t debug_errors(uint32_t *bits, bool clear) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    uint32_t v = 0;
    e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_errors), sizeof(v), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    if (clear) {
        const uint32_t zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_debug_errors), &zero, sizeof(zero), 0,
                              hipMemcpyHostToDevice);
        if (e != hipSuccess) return e;
    }
    *bits = v;
    return hipSuccess;
}

hipError_t launch_shrink(int dtype, int tt, bool mp, const ShrinkArgs &a, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    return dtype == LORA_BF16 ? shrink_dispatch<uint16_t>(tt, mp, a, s)
                              : shrink_dispatch<float>(tt, mp, a, s);
}

hipError_t launch_pack_a(int dtype, const void *src, int rank, int h_in, void *dst, int r_pad,
                         int h_in_pad, hipStream_t s) {
    const int e = dtype == LORA_BF16 ? 8 : 4;
    const int vecs = h_in_pad / e * r_pad;
    const dim3 grid((vecs + 255) / 256), block(256);
    if (dtype == LORA_BF16)
        hipLaunchKernelGGL(k_pack_a<uint16_t>, grid, block, 0, s,
                           static_cast<const uint16_t *>(src), rank, h_in,
                           static_cast<uint16_t *>(dst), r_pad, h_in_pad);
    else
        hipLaunchKernelGGL(k_pack_a<float>, grid, block, 0, s, static_cast<const float *>(src),
                           rank, h_in, static_cast<float *>(dst), r_pad, h_in_pad);
    return hipGetLastError();
}

hipError_t launch_pack_b(int dtype, const void *src, int rank, int h_out, void *dst, int r_pad,
                         hipStream_t s) {
    const int es = dtype == LORA_BF16 ? 2 : 4;
    const int vecs = h_out * (r_pad * es / 16);
    const dim3 grid((vecs + 255) / 256), block(256);
    if (dtype == LORA_BF16)
        hipLaunchKernelGGL(k_pack_b<uint16_t>, grid, block, 0, s,
                           static_cast<const uint16_t *>(src), rank, h_out,
                           static_cast<uint16_t *>(dst), r_pad);
    else
        hipLaunchKernelGGL(k_pack_b<float>, grid, block, 0, s, static_cast<const float *>(src),
                           rank, h_out, static_cast<float *>(dst), r_pad);
    return hipGetLastError();
}

hipError_t launch_reduce(int tt, const ReduceArgs &a, hipStream_t s) {
    if (a.nb <= 0) return hipSuccess;
    const dim3 grid(a.nb * a.nproj), block(kWaves * kWaveSize);
    switch (tt) {
    case 1: hipLaunchKernelGGL((k_reduce<1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_reduce<2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_reduce<4>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool Sig>
void expand_decode_nvm(int nvm, dim3 grid, dim3 block, const ExpandArgs &a, hipStream_t s) {
    if (nvm <= 1) hipLaunchKernelGGL((k_expand_decode<T, Sig, 1>), grid, block, 0, s, a);
    else if (nvm <= 2) hipLaunchKernelGGL((k_expand_decode<T, Sig, 2>), grid, block, 0, s, a);
    else if (nvm <= 4) hipLaunchKernelGGL((k_expand_decode<T, Sig, 4>), grid, block, 0, s, a);
    else if (nvm <= 8) hipLaunchKernelGGL((k_expand_decode<T, Sig, 8>), grid, block, 0, s, a);
    else if constexpr (sizeof(T) == 4) hipLaunchKernelGGL((k_expand_decode<T, Sig, 16>), grid, block, 0, s, a);
}

hipError_t launch_expand_decode(int dtype, int nvm, const ExpandArgs &a, int g, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    const dim3 grid(g), block(kWaves * kWaveSize);
    if (dtype == LORA_BF16) {
        if (nvm > 8) return hipErrorInvalidValue;
        if (a.sigma_kind) expand_decode_nvm<uint16_t, true>(nvm, grid, block, a, s);
        else expand_decode_nvm<uint16_t, false>(nvm, grid, block, a, s);
    } else {
        if (nvm > 16) return hipErrorInvalidValue;
        if (a.sigma_kind) expand_decode_nvm<float, true>(nvm, grid, block, a, s);
        else expand_decode_nvm<float, false>(nvm, grid, block, a, s);
    }
    return hipGetLastError();
}

template <typename T, int NT>
hipError_t expand_merge_t(int nvm, dim3 grid, dim3 block, const MergeArgs &a, hipStream_t s) {
    if (nvm <= 1) hipLaunchKernelGGL((k_expand_merge<T, 1, NT>), grid, block, 0, s, a);
    else if (nvm <= 2) hipLaunchKernelGGL((k_expand_merge<T, 2, NT>), grid, block, 0, s, a);
    else if (nvm <= 4) hipLaunchKernelGGL((k_expand_merge<T, 4, NT>), grid, block, 0, s, a);
    else if (nvm <= 8) hipLaunchKernelGGL((k_expand_merge<T, 8, NT>), grid, block, 0, s, a);
    else if constexpr (sizeof(T) == 4) hipLaunchKernelGGL((k_expand_merge<T, 16, NT>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_expand_merge(int dtype, int nvm, int max_tok, const MergeArgs &a, int grid,
                               hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    if (max_tok < 1 || max_tok > kValuTokens) return hipErrorInvalidValue;
    const dim3 g(grid), block(kWaves * kWaveSize);
    const bool one = max_tok == 1;
    if (dtype == LORA_BF16) {
        if (nvm > 8) return hipErrorInvalidValue;
        return one ? expand_merge_t<uint16_t, 1>(nvm, g, block, a, s)
                   : expand_merge_t<uint16_t, kValuTokens>(nvm, g, block, a, s);
    }
    if (nvm > 16) return hipErrorInvalidValue;
    return one ? expand_merge_t<float, 1>(nvm, g, block, a, s)
               : expand_merge_t<float, kValuTokens>(nvm, g, block, a, s);
}

hipError_t launch_prefill(int dtype, int mode, int np, int rtm, int tpl, const PrefillArgs &a,
                          int grid, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    if (tpl != 1 && rtm != 1) return hipErrorInvalidValue;
    return dtype == LORA_BF16 ? prefill_modes<uint16_t>(mode, np, rtm, tpl, a, grid, s)
                              : prefill_modes<float>(mode, np, rtm, tpl, a, grid, s);
}

}  // namespace lora

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
// Non-temporal loads (early eviction from L2) for the shrink's A only.  The
// expands load B with the default policy: the blocks of one adapter read the
// same B rows at about the same time on one XCD, and keeping the lines in L2
// measured 3.8% faster per decode step (2% per prefill step) than streaming
// them; for A the default policy was about 3% slower.
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
    for (int tt = 0; tt < TT; ++tt) trow[tt] = a.tile_tok[key * kMaxBlockTokens + tt * kTile + n];
    const TileDesc td = load_invariant(a.tiles + key);
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
        const rsrc_t ar = make_rsrc(
            a.slab + extent(td.ext_lo, td.ext_hi) +
                uint64_t(td.r_pad) * sizeof(T) * uint64_t(a.coef_a[p]),
            uint32_t(td.r_pad) * uint32_t(a.h_in_pad) * sizeof(T));
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
        for (int i = threadIdx.x; i < ntiles * kWaveSize; i += kWaves * kWaveSize) {
            // token tiles past the block's last are never read: not stored
            const int tt = i / kWaveSize, ln = i % kWaveSize;
            const f32x4 s4 = red[0][tt][ln] + red[1][tt][ln] + red[2][tt][ln] + red[3][tt][ln];
            // partials are read once, by the next kernel
            __builtin_nontemporal_store(
                s4, reinterpret_cast<f32x4 *>(pt + (tt * kTile + (ln & 15)) * kTile + (ln >> 4) * 4));
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
    const BlockDesc blk = load_invariant(a.blocks + b);
    const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
    const int quads = a.r_max / 4;
    for (int i = threadIdx.x; i < blk.n_tok * quads; i += blockDim.x) {
        const int ti = i / quads, j = (i % quads) * 4;
        f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < blk.r_pad)
            s4 = chunk_sum(pr, partial_off(blk.rt_before, j, blk.slot0 + ti, p, a.nproj, a.c0, TT),
                           uint32_t(a.nproj * TT * kTile * kTile), a.c0);
        const int t = a.tok[blk.tok_off + ti];
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

// The expand's per-workgroup context: the block, its token rows and the
// wave's output rows.
struct ExpandCtx {
    int b, p, w, n, q;
    int o_lo, o_hi, yoff, h_out, ks_n, ntiles;
    float scale;
    float tsc[4];     // the scale of this lane's token in each 16-token tile
};

// One output element: bf16 (2 bytes) or float32 (4 bytes).
template <typename T> struct Out1;
template <> struct Out1<uint16_t> {
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, 0))
                               << 16);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(
            (unsigned short)(bf16x2_rne(v, 0.f) & 0xffffu), r, int(off), 0, kOut);
    }
};
template <> struct Out1<float> {
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, int(off), 0, kOut);
    }
};

// v of the block's tokens into LDS, once per workgroup: from the shrink's
// chunk partials (summed in the one chunk order) or a caller's v.
template <int TT>
__device__ __forceinline__ void gather_v(const ExpandArgs &a, const BlockDesc &blk, int p,
                                         float (*vs)[LORA_MAX_RANK + 4]) {
    const int quads = blk.r_pad / 4;
    if (a.partial) {
        const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
        const uint32_t stride = uint32_t(a.nproj * a.ptt * kTile * kTile);
        for (int i = threadIdx.x; i < blk.n_tok * quads; i += kWaves * kWaveSize) {
            const int ti = i / quads, j = (i % quads) * 4;
            *reinterpret_cast<f32x4 *>(&vs[ti][j]) = chunk_sum(
                pr, partial_off(blk.rt_before, j, blk.slot0 + ti, p, a.nproj, a.c0, a.ptt),
                stride, a.c0);
        }
    } else {
        for (int i = threadIdx.x; i < blk.n_tok * quads; i += kWaves * kWaveSize) {
            const int ti = i / quads, j = (i % quads) * 4;
            const int t = a.tok[blk.tok_off + ti];
            *reinterpret_cast<f32x4 *>(&vs[ti][j]) = *reinterpret_cast<const f32x4 *>(
                a.v + int64_t(t) * a.ldv + int64_t(p) * a.r_max + j);
        }
    }
}

// The core step of jointly compressed adapters ("Compress then Serve",
// rebuttal pseudocode of add_lora_slice_with_sigma, step 2): each token's v
// (LDS rows [0, n_tok), ranks [0, r_pad)) becomes Sigma_j v with the token's
// core j, in float32, k ascending; a token without a core keeps v.  Full
// cores are r_max x r_max row-major, diagonal cores r_max values.  Up to
// MAXI entries per thread.
template <int MAXI>
__device__ __forceinline__ void apply_sigma(const ExpandArgs &a, const BlockDesc &blk, int p,
                                            float (*vs)[LORA_MAX_RANK + 4]) {
    const int r = blk.r_pad;
    const int entries = blk.n_tok * r;
    float out[MAXI];
#pragma unroll
    for (int ii = 0; ii < MAXI; ++ii) {
        const int i = int(threadIdx.x) + ii * kWaves * kWaveSize;
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
        const int i = int(threadIdx.x) + ii * kWaves * kWaveSize;
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = g.k + i * kSumWays;
            g.part[i] = bload16(pr, off_or_oob(g.on && c < a.c0, (off + uint32_t(c) * stride) * 4));
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
// unit: lane owns rows o_lo + lane + 64 i (i < RPL) and streams the NV
// 16-byte vectors of each B row (r_pad = nv * E values, nv <= NV), dotting
// them with every token's v (an LDS broadcast) in float32.  Loads go out in
// the order they are used: the v gather, B vector by vector, then y_in; so
// the dot products of the first vectors start while the rest arrive.
template <typename T, int NV, bool Sig, bool PRW>
__device__ __forceinline__ void expand_valu(const ExpandArgs &a, const BlockDesc &blk,
                                            const int (&tr)[kValuTokens], int p, int o_lo,
                                            int o_hi, float (*vs)[LORA_MAX_RANK + 4],
                                            f32x4 (*ways)[kSumWays]) {
    constexpr int E = Elem<T>::E;
    constexpr int RPL = decode_rpl(NV);
    constexpr int NT = kValuTokens;
    const int lane = threadIdx.x & 63;
    const int nv = blk.r_pad / E;                    // wave-uniform, <= NV
    const int nt = blk.n_tok;                        // wave-uniform, <= NT
    const int yoff = a.y_off[p];
    const rsrc_t br = make_rsrc(
        a.slab + extent(blk.ext_lo, blk.ext_hi) +
            uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_b[p]),
        uint32_t(a.h_out[p]) * uint32_t(blk.r_pad) * sizeof(T));
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

    // PR (builds for B rows of at most 2 vectors): a lane owns two adjacent
    // rows, so y_in and y of a token move 4 bytes a lane (bf16) in one
    // access instead of two of 2 bytes, and the kernel holds 48 VGPRs
    // instead of 54: 1% per full-stack step.  Wider rows keep rows a wave
    // apart (paired, their B loads would stride 128 bytes a lane; 1% slower
    // on the multi-rank decode).
    constexpr bool PR = PRW && RPL == 2;
    auto row_of = [&](int i) { return PR ? o_lo + 2 * lane + i : o_lo + i * kWaveSize + lane; };
    VGather g;
    gather_issue(a, blk, tr, p, g);
    u32x4 bv[NV][RPL];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int row = row_of(i);
            bv[v][i] = bload16(br, off_or_oob(row < o_hi && v < nv,
                                              uint32_t(row) * row_bytes + v * 16));
        }
    float yin[RPL][NT];
    if constexpr (PR) {
        const int row = row_of(0);
        const bool rok = row < o_hi;                 // o_hi is even: the pair is in or out
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t off = rok ? in_row[t] + uint32_t(row) * sizeof(T) : kOOB;
            if constexpr (sizeof(T) == 2) {
                const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(inr, int(off), 0, 0);
                yin[0][t] = bf16_lo(w);
                yin[1][t] = bf16_hi(w);
            } else {
                const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(inr, int(off), 0, 0);
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
                yin[i][t] = Out1<T>::load(inr, rok ? in_row[t] + uint32_t(row) * sizeof(T) : kOOB);
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

// Expand of one workgroup for blocks whose padded rank packs TPL row tiles
// into one 16-byte load per lane (TPL = 4: r_pad = E / 2 ... see below), or
// TPL = 1 (one tile per load and K-step).  Row chunks of OTW tiles are
// double-buffered: the next chunk's B rows and y_in are in flight while the
// current chunk is computed.
//
// Packing: a 16-row tile of B is 16 * r_pad elements.  With G = r_pad / E
// 16-byte vectors per row and G in {1, 2}, one load of 64 lanes covers
// TPL = 4 / G consecutive tiles: lane group q reads vector q % G of tile
// q / G.  The MFMA of tile t then takes v only in the lane groups holding
// tile t (zero elsewhere), which selects tile t's rows.
template <typename T, int TT, int KSM, int TPL>
__device__ __forceinline__ void expand_body(const ExpandArgs &a, const BlockDesc &blk,
                                            const ExpandCtx &c, const int (&trow)[TT],
                                            const bool (&tv)[TT], float (*vs)[LORA_MAX_RANK + 4]) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;
    constexpr int OTW = expand_tiles(KSM);           // tiles per chunk
    constexpr int NL = TPL == 1 ? OTW * KSM : OTW / TPL;   // loads per chunk
    constexpr int CH = OTW * kTile;                  // rows per chunk
    const int G = TPL == 1 ? 4 : 4 / TPL;            // vectors per row (packed)
    typedef typename Out4<T>::raw raw;

    const rsrc_t br = make_rsrc(
        a.slab + extent(blk.ext_lo, blk.ext_hi) +
            uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_b[c.p]),
        uint32_t(c.h_out) * uint32_t(blk.r_pad) * sizeof(T));
    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const rsrc_t inr = a.base ? make_rsrc(a.base, a.base_bytes) : yr;
    const int64_t ld_in = a.base ? a.ldb : a.ldy;

    // Byte offsets hoisted out of the row loops: a masked token's row offset
    // is already out of range (kOOB + o * size stays >= 2^31, below 2^32).
    uint32_t in_row[TT], y_row[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        in_row[tt] = tv[tt] ? uint32_t((int64_t(trow[tt]) * ld_in + c.yoff) * sizeof(T)) : kOOB;
        y_row[tt] = tv[tt] ? uint32_t((int64_t(trow[tt]) * a.ldy + c.yoff) * sizeof(T)) : kOOB;
    }
    const uint32_t row_bytes = uint32_t(blk.r_pad) * sizeof(T);
    // this lane's tile within a load and element offset within its B row
    const int lane_tile = TPL == 1 ? 0 : c.q / G;
    const uint32_t lane_col = uint32_t(TPL == 1 ? c.q * E : (c.q % G) * E) * sizeof(T);
    // bf16: within each pair of row tiles the B rows are taken in the order
    // that leaves a lane 8 consecutive outputs (4 from each tile of the
    // pair), so y_in and y move 16 bytes a lane: tile T's MFMA row n is
    // output row 16 (T & ~1) + 8 (n / 4) + 4 (T & 1) + n % 4 of the chunk.
    constexpr bool PAIR = sizeof(T) == 2;
    static_assert(!PAIR || OTW % 2 == 0, "row tiles of a chunk come in pairs");
    auto brow = [&](int tile, int n) {
        return PAIR ? (tile & ~1) * kTile + 8 * (n >> 2) + 4 * (tile & 1) + (n & 3)
                    : tile * kTile + n;
    };
    constexpr int NY = PAIR ? OTW / 2 : OTW;         // y_in loads per token tile and chunk
    typedef typename std::conditional<PAIR, u32x4, raw>::type yraw;

    auto load = [&](int o0, u32x4 (&bf)[NL], yraw (&yin)[NY][TT]) {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int t = TPL == 1 ? l / KSM : l * TPL;          // first tile of the load
            const int ks = TPL == 1 ? l % KSM : 0;
            const int row = o0 + brow(t + lane_tile, c.n);
            const bool ok = row < c.o_hi &&
                            (TPL > 1 || (ks < c.ks_n && ks * SPAN + c.q * E < blk.r_pad));
            bf[l] = bload16(br, off_or_oob(ok, uint32_t(row) * row_bytes + lane_col +
                                                   uint32_t(ks * SPAN) * sizeof(T)));
        }
#pragma unroll
        for (int oy = 0; oy < NY; ++oy) {
            const int o = PAIR ? o0 + oy * 2 * kTile + 8 * c.q : o0 + oy * kTile + 4 * c.q;
            const uint32_t oo = uint32_t(o) * sizeof(T);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if constexpr (PAIR)
                    yin[oy][tt] = bload16(inr, o < c.o_hi ? in_row[tt] + oo : kOOB);
                else
                    yin[oy][tt] = Out4<T>::load(inr, o < c.o_hi ? in_row[tt] + oo : kOOB);
            }
        }
    };

    u32x4 bfA[NL], bfB[NL];
    yraw yinA[NY][TT], yinB[NY][TT];
    load(c.o_lo, bfA, yinA);

    gather_v<TT>(a, blk, c.p, vs);
    __syncthreads();
    if (a.sigma_kind)
        apply_sigma<TT * kTile * LORA_MAX_RANK / (kWaves * kWaveSize)>(a, blk, c.p, vs);
    if (c.o_lo >= c.o_hi) return;

    // v operand per (token tile, K-step); packed blocks have one K-step
    VOperand<T> vop[TT][KSM];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks) {
            float f[E];
            const int j0 = TPL == 1 ? ks * SPAN + c.q * E : (c.q % G) * E;
            const bool ok = tv[tt] && ks < c.ks_n && j0 < blk.r_pad;
            const int row = ok ? tt * kTile + c.n : 0;
            const int col = ok ? j0 : 0;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&vs[row][col + e]);
                f[e] = ok ? w4[0] : 0.f; f[e + 1] = ok ? w4[1] : 0.f;
                f[e + 2] = ok ? w4[2] : 0.f; f[e + 3] = ok ? w4[3] : 0.f;
            }
            vop[tt][ks].set(f);
        }
    }

    // B v of row tile ot for token tile tt: D rows 4q .. 4q + 3 of the tile
    auto tile_acc = [&](int ot, int tt, const u32x4 (&bf)[NL]) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        if (TPL == 1) {
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
                if (ks >= c.ks_n) continue;
#pragma unroll
                for (int pc = VOperand<T>::kPieces - 1; pc >= 0; --pc)
                    acc = mma<T>(bf[ot * KSM + ks], vop[tt][ks].piece[pc], acc);
            }
        } else {
            const bool mine = c.q / G == ot % TPL;   // lane groups of this tile
#pragma unroll
            for (int pc = VOperand<T>::kPieces - 1; pc >= 0; --pc) {
                const u32x4 vp = vop[tt][0].piece[pc];
                const u32x4 z = u32x4{0u, 0u, 0u, 0u};
                acc = mma<T>(bf[ot / TPL], mine ? vp : z, acc);
            }
        }
        return acc;
    };

    auto compute = [&](int o0, const u32x4 (&bf)[NL], const yraw (&yin)[NY][TT]) {
#pragma unroll
        for (int oy = 0; oy < NY; ++oy) {
            const int obase = o0 + oy * (PAIR ? 2 : 1) * kTile;
            if (obase >= c.o_hi) break;              // wave-uniform
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt >= c.ntiles) continue;        // wave-uniform
                if constexpr (PAIR) {
                    // tiles 2 oy and 2 oy + 1: this lane's outputs 8 q .. 8 q + 7
                    const f32x4 a0 = tile_acc(2 * oy, tt, bf);
                    const f32x4 a1 = tile_acc(2 * oy + 1, tt, bf);
                    const int o = obase + 8 * c.q;
                    const u32x4 w = yin[oy][tt];
                    float out[8];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        out[2 * i] = bf16_lo(w[i]) + c.tsc[tt] * a0[2 * i];
                        out[2 * i + 1] = bf16_hi(w[i]) + c.tsc[tt] * a0[2 * i + 1];
                        out[4 + 2 * i] = bf16_lo(w[2 + i]) + c.tsc[tt] * a1[2 * i];
                        out[5 + 2 * i] = bf16_hi(w[2 + i]) + c.tsc[tt] * a1[2 * i + 1];
                    }
                    const u32x4 pk = u32x4{bf16x2_rne(out[0], out[1]), bf16x2_rne(out[2], out[3]),
                                           bf16x2_rne(out[4], out[5]), bf16x2_rne(out[6], out[7])};
                    __builtin_amdgcn_raw_buffer_store_b128(
                        pk, yr, int(o < c.o_hi ? y_row[tt] + uint32_t(o) * sizeof(T) : kOOB), 0,
                        kOut);
                } else {
                    const f32x4 acc = tile_acc(oy, tt, bf);
                    const int o = obase + 4 * c.q;
                    float in[4], out[4];
                    Out4<T>::unpack(yin[oy][tt], in);
#pragma unroll
                    for (int i = 0; i < 4; ++i) out[i] = in[i] + c.tsc[tt] * acc[i];
                    Out4<T>::store(yr, o < c.o_hi ? y_row[tt] + uint32_t(o) * sizeof(T) : kOOB,
                                   Out4<T>::pack(out));
                }
            }
        }
    };

    for (int o0 = c.o_lo; o0 < c.o_hi; o0 += 2 * CH) {
        if (o0 + CH < c.o_hi) load(o0 + CH, bfB, yinB);
        compute(o0, bfA, yinA);
        const int o1 = o0 + CH;
        if (o1 >= c.o_hi) break;
        if (o1 + CH < c.o_hi) load(o1 + CH, bfA, yinA);
        compute(o1, bfB, yinB);
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

    const BlockDesc blk = load_invariant(a.blocks + b);
    const int4 bt4 = load_invariant(reinterpret_cast<const int4 *>(a.block_tok + b * kMaxBlockTokens));
    const int tr[kValuTokens] = {bt4.x, bt4.y, bt4.z, bt4.w};
    static_assert(kValuTokens == 4, "token rows load as one int4");

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
    case 1: return expand_valu<T, 1, Sig, (NVM <= 2)>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    case 2: if constexpr (NVM >= 2) return expand_valu<T, 2, Sig, (NVM <= 2)>(a, blk, tr, p, o_lo, o_hi, vs, ways);
            return;
    case 4: if constexpr (NVM >= 4) return expand_valu<T, 4, Sig, (NVM <= 2)>(a, blk, tr, p, o_lo, o_hi, vs, ways);
            return;
    case 8: if constexpr (NVM >= 8) return expand_valu<T, 8, Sig, (NVM <= 2)>(a, blk, tr, p, o_lo, o_hi, vs, ways);
            return;
    default:
        if constexpr (sizeof(T) == 4 && NVM >= 16) return expand_valu<T, 16, Sig, (NVM <= 2)>(a, blk, tr, p, o_lo, o_hi, vs, ways);
    }
}

template <typename T, int TT, int KSM>
__global__ __launch_bounds__(256) void k_expand(const ExpandArgs a) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;
    constexpr int OTW = expand_tiles(KSM);
    constexpr int VS = LORA_MAX_RANK + 4;            // LDS row stride of v (floats)
    __shared__ float vs[TT * kTile][VS];

    warm_args<ExpandArgs>();
    const int u = xcd_unit(1);
    if (u >= a.units) return;                        // whole workgroup
    const int lane = threadIdx.x & 63;
    ExpandCtx c;
    c.w = wave_id();
    c.n = lane & 15;
    c.q = lane >> 4;
    // unit -> (block, token slice, projection, row chunk)
    const int upb = a.oc_prefix[a.nproj];
    const int per_block = a.tslices * upb;
    c.b = u / per_block;
    const int rs = u - c.b * per_block;
    const int ts = rs / upb;
    const int rem = rs - ts * upb;
    c.p = 0;
    while (rem >= a.oc_prefix[c.p + 1]) ++c.p;
    const int oc = rem - a.oc_prefix[c.p];
    // the slice's tokens as a block of their own: its first token, its first
    // slot in the shrink block and its token count
    BlockDesc blk = load_invariant(a.blocks + c.b);
    const int off = ts * TT * kTile;
    if (off >= blk.n_tok) return;                    // whole workgroup: an empty slice
    blk.tok_off += off;
    blk.slot0 += off;
    blk.n_tok = min(TT * kTile, blk.n_tok - off);
    int trow[TT];                                    // token rows, -1 padded
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
        trow[tt] = a.block_tok[c.b * kMaxBlockTokens + off + tt * kTile + c.n];
    c.h_out = a.h_out[c.p];
    const int rows_w = a.chunks * OTW * kTile;       // rows of this wave
    c.o_lo = min(c.h_out, (oc * kWaves + c.w) * rows_w);
    c.o_hi = min(c.h_out, c.o_lo + rows_w);
    c.yoff = a.y_off[c.p];
    c.ks_n = (blk.r_pad + SPAN - 1) / SPAN;          // wave-uniform, <= KSM
    c.ntiles = (blk.n_tok + kTile - 1) / kTile;
    c.scale = blk.scale;
    bool tv[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) tv[tt] = tt < c.ntiles && trow[tt] >= 0;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int i = tt * kTile + c.n;
        c.tsc[tt] = a.tok_w && tt < TT && i < blk.n_tok ? blk.scale * a.tok_w[blk.tok_off + i]
                                                       : blk.scale;
    }

    if (blk.r_pad == 0) {            // tokens without an adapter: y = base
        if (!a.base) return;
        const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
        const rsrc_t br = make_rsrc(a.base, a.base_bytes);
        for (int o0 = c.o_lo; o0 < c.o_hi; o0 += kTile) {
            const int o = o0 + 4 * c.q;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const bool ok = tv[tt] && o < c.o_hi;
                const auto v4 = Out4<T>::load(
                    br, off_or_oob(ok, uint32_t(int64_t(trow[tt]) * a.ldb + c.yoff + o) * sizeof(T)));
                Out4<T>::store(
                    yr, off_or_oob(ok, uint32_t(int64_t(trow[tt]) * a.ldy + c.yoff + o) * sizeof(T)),
                    v4);
            }
        }
        return;
    }

    // rows of 16-byte vectors: 1 or 2 per row pack 4 or 2 tiles into one load
    if constexpr (KSM == 1) {
        const int g = blk.r_pad / E;
        if (g == 1) return expand_body<T, TT, KSM, 4>(a, blk, c, trow, tv, vs);
        if (g == 2) return expand_body<T, TT, KSM, 2>(a, blk, c, trow, tv, vs);
    }
    expand_body<T, TT, KSM, 1>(a, blk, c, trow, tv, vs);
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

template <typename T, int KSM>
hipError_t expand_dispatch_ks(int tt, const ExpandArgs &a, hipStream_t s) {
    const dim3 grid(a.grid), block(kWaves * kWaveSize);
    switch (tt) {
    case 1: hipLaunchKernelGGL((k_expand<T, 1, KSM>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_expand<T, 2, KSM>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_expand<T, 4, KSM>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

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

hipError_t launch_expand_decode(int dtype, int nvm, const ExpandArgs &a, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    const dim3 grid(a.grid), block(kWaves * kWaveSize);
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

hipError_t launch_expand(int dtype, int tt, int ks, const ExpandArgs &a, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    if (dtype == LORA_BF16) {
        if (ks == 1) return expand_dispatch_ks<uint16_t, 1>(tt, a, s);
        if (ks == 2) return expand_dispatch_ks<uint16_t, 2>(tt, a, s);
        return hipErrorInvalidValue;
    }
    if (ks == 1) return expand_dispatch_ks<float, 1>(tt, a, s);
    if (ks == 2) return expand_dispatch_ks<float, 2>(tt, a, s);
    if (ks == 4) return expand_dispatch_ks<float, 4>(tt, a, s);
    return hipErrorInvalidValue;
}

}  // namespace lora

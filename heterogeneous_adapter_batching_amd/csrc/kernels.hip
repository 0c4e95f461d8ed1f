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
// the hardware without touching memory.  So no load sits behind a branch,
// and each wave issues all of its streaming loads before it waits for any.
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
constexpr int kNT = 2;                        // non-temporal: streamed once

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

// float -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

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

// Workgroup g runs on XCD g % kXcds.  Give each XCD a contiguous range of
// units, so units that share operands (the x chunk of one block, the partials
// of one block) meet in one L2.
__device__ __forceinline__ int xcd_unit(int grid) {
    const int g = blockIdx.x;
    return (g % kXcds) * (grid / kXcds) + g / kXcds;
}

// ---------------------------------------------------------------- shrink ----
template <typename T, int TT>
__global__ __launch_bounds__(256) void k_shrink(const ShrinkArgs a) {
    constexpr int E = Elem<T>::E;        // elements per 16-byte fragment
    constexpr int SPAN = 4 * E;          // K covered by one fragment over 4 lane groups
    constexpr int F = shrink_frags<TT>();
    __shared__ f32x4 red[kWaves][TT][kWaveSize];

    const int u = xcd_unit(a.grid);
    if (u >= a.units) return;            // whole workgroup: no barrier is skipped
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int n = lane & 15, q = lane >> 4;

    // unit -> (rank tile, chunk, projection): the descriptor and the token
    // rows of the tile load in parallel
    const int per = a.nproj * a.c0;
    const int key = u / per;
    int trow[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) trow[tt] = a.tile_tok[key * kMaxBlockTokens + tt * kTile + n];
    const TileDesc td = a.tiles[key];
    const int rem = u - key * per;
    const int c = rem / a.nproj, p = rem - (rem / a.nproj) * a.nproj;

    // this wave's quarter of the chunk: at most F fragments
    const int kw = a.kc / kWaves;
    const int k_lo = c * a.kc + w * kw;
    const int k_hi = min(min(a.h_in, (c + 1) * a.kc), k_lo + kw);

    // A rows first: they depend on nothing but the descriptor
    const rsrc_t ar = make_rsrc(
        a.slab + extent(td.ext_lo, td.ext_hi) +
            uint64_t(td.r_pad) * sizeof(T) * uint64_t(a.coef_a[p]),
        uint32_t(td.r_pad) * uint32_t(a.h_in) * sizeof(T));
    const int j = td.tile * kTile + n;
    const bool jv = j < td.r_pad;
    u32x4 af[F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
        const int k = k_lo + f * SPAN + q * E;
        af[f] = bload16_nt(ar, off_or_oob(jv && k < k_hi,
                                          (uint32_t(j) * uint32_t(a.h_in) + k) * sizeof(T)));
    }

    // then the token rows
    const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const int ntiles = (td.n_tok + kTile - 1) / kTile;   // wave-uniform
    u32x4 xf[TT][F];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = trow[tt];
        const bool tv = tt < ntiles && t >= 0;
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const int k = k_lo + f * SPAN + q * E;
            xf[tt][f] = bload16(xr, off_or_oob(tv && k < k_hi,
                                               uint32_t(int64_t(t) * a.ldx + k) * sizeof(T)));
        }
    }

    f32x4 acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < F; ++f) {
        if (k_lo + f * SPAN >= k_hi) break;              // wave-uniform
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            if (tt < ntiles) acc[tt] = mma<T>(af[f], xf[tt][f], acc[tt]);
    }

    // sum the 4 waves in a fixed order; lane holds ranks 4q..4q+3 of token n
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) red[w][tt][lane] = acc[tt];
    __syncthreads();
    float *pt = a.partial + size_t(u) * (TT * kTile * kTile);
    for (int i = threadIdx.x; i < TT * kWaveSize; i += kWaves * kWaveSize) {
        const int tt = i / kWaveSize, ln = i % kWaveSize;
        const f32x4 s4 = red[0][tt][ln] + red[1][tt][ln] + red[2][tt][ln] + red[3][tt][ln];
        *reinterpret_cast<f32x4 *>(pt + (tt * kTile + (ln & 15)) * kTile + (ln >> 4) * 4) = s4;
    }
}

// partial tile of (rank tile, chunk, projection) for an adapter block
__device__ __forceinline__ const float *partial_tile(const float *partial, int tt_tiles,
                                                     int rt_before, int tile, int c, int p,
                                                     int nproj, int c0) {
    const int u = (rt_before + tile) * nproj * c0 + c * nproj + p;
    return partial + size_t(u) * (tt_tiles * kTile * kTile);
}

// --------------------------------------------------------------- reduce -----
// One workgroup per (adapter block, projection): v = sum of the chunk partials.
template <int TT>
__global__ __launch_bounds__(256) void k_reduce(const ReduceArgs a) {
    const int bp = blockIdx.x;
    const int b = bp / a.nproj, p = bp % a.nproj;
    const BlockDesc blk = a.blocks[b];
    const int quads = a.r_max / 4;
    for (int i = threadIdx.x; i < blk.n_tok * quads; i += blockDim.x) {
        const int ti = i / quads, j = (i % quads) * 4;
        f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < blk.r_pad) {
            for (int c = 0; c < a.c0; ++c)
                s4 += *reinterpret_cast<const f32x4 *>(
                    partial_tile(a.partial, TT, blk.rt_before, j / kTile, c, p, a.nproj, a.c0) +
                    ti * kTile + j % kTile);
        }
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
    __device__ __forceinline__ void set(const float (&f)[8]) {
        uint32_t h[3][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h0 = bf16_rne(f[e]);
            const float r1 = f[e] - bf16_to_f32(h0);
            const bool fin = (h0 & 0x7f80u) != 0x7f80u;   // Inf/NaN: no residual
            const uint32_t h1 = fin ? bf16_rne(r1) : 0u;
            const float r2 = r1 - bf16_to_f32(h1);
            const uint32_t h2 = fin ? bf16_rne(r2) : 0u;
            h[0][e] = h0; h[1][e] = h1; h[2][e] = h2;
        }
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
            piece[pc] = u32x4{h[pc][0] | (h[pc][1] << 16), h[pc][2] | (h[pc][3] << 16),
                              h[pc][4] | (h[pc][5] << 16), h[pc][6] | (h[pc][7] << 16)};
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
        __builtin_amdgcn_raw_buffer_store_b64(v, r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void unpack(raw w, float (&o)[4]) {
        o[0] = __uint_as_float(w[0] << 16); o[1] = __uint_as_float(w[0] & 0xffff0000u);
        o[2] = __uint_as_float(w[1] << 16); o[3] = __uint_as_float(w[1] & 0xffff0000u);
    }
    static __device__ __forceinline__ raw pack(const float (&o)[4]) {
        return u32x2{bf16_rne(o[0]) | (bf16_rne(o[1]) << 16),
                     bf16_rne(o[2]) | (bf16_rne(o[3]) << 16)};
    }
};
template <> struct Out4<float> {
    typedef u32x4 raw;
    static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    }
    static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, raw v) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, 0);
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

template <typename T, int TT, int KSM>
__global__ __launch_bounds__(256) void k_expand(const ExpandArgs a) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;                      // ranks per K-step
    constexpr int OTW = expand_tiles(KSM);           // 16-row tiles per wave
    constexpr int VS = LORA_MAX_RANK + 4;            // LDS row stride of v (floats)
    __shared__ float vs[TT * kTile][VS];

    const int u = xcd_unit(a.grid);
    if (u >= a.units) return;                        // whole workgroup
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int n = lane & 15, q = lane >> 4;

    const int upb = a.oc_prefix[a.nproj];
    const int b = u / upb;
    const int rem = u - b * upb;
    int p = 0;
    while (rem >= a.oc_prefix[p + 1]) ++p;
    const int oc = rem - a.oc_prefix[p];
    int trow[TT];                                    // token rows, -1 padded
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) trow[tt] = a.block_tok[b * kMaxBlockTokens + tt * kTile + n];
    const BlockDesc blk = a.blocks[b];
    const int h_out = a.h_out[p];
    const int o_lo = min(h_out, (oc * kWaves + w) * (OTW * kTile));
    const int o_hi = min(h_out, o_lo + OTW * kTile);
    const int yoff = a.y_off[p];
    const int ks_n = (blk.r_pad + SPAN - 1) / SPAN;  // wave-uniform, <= KSM

    // B rows of this wave first: they depend on nothing but the descriptor
    const rsrc_t br = make_rsrc(
        a.slab + extent(blk.ext_lo, blk.ext_hi) +
            uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_b[p]),
        uint32_t(h_out) * uint32_t(blk.r_pad) * sizeof(T));
    u32x4 bf[OTW][KSM];
#pragma unroll
    for (int ot = 0; ot < OTW; ++ot) {
        const int orow = o_lo + ot * kTile + n;
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks) {
            const int j0 = ks * SPAN + q * E;
            bf[ot][ks] = bload16_nt(br, off_or_oob(ks < ks_n && orow < o_hi && j0 < blk.r_pad,
                                                   uint32_t(orow * blk.r_pad + j0) * sizeof(T)));
        }
    }

    // then y_in (base, or y itself) of every output tile
    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const rsrc_t inr = a.base ? make_rsrc(a.base, a.base_bytes) : yr;
    const int64_t ld_in = a.base ? a.ldb : a.ldy;
    const int ntiles = (blk.n_tok + kTile - 1) / kTile;
    bool tv[TT];
    typename Out4<T>::raw yin[OTW][TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        tv[tt] = tt < ntiles && trow[tt] >= 0;
#pragma unroll
        for (int ot = 0; ot < OTW; ++ot) {
            const int o = o_lo + ot * kTile + 4 * q;
            yin[ot][tt] = Out4<T>::load(
                inr, off_or_oob(tv[tt] && o < o_hi,
                                uint32_t(int64_t(trow[tt]) * ld_in + yoff + o) * sizeof(T)));
        }
    }

    if (blk.r_pad == 0) {            // tokens without an adapter: y = base
        if (!a.base) return;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
            for (int ot = 0; ot < OTW; ++ot) {
                const int o = o_lo + ot * kTile + 4 * q;
                Out4<T>::store(yr, off_or_oob(tv[tt] && o < o_hi,
                                              uint32_t(int64_t(trow[tt]) * a.ldy + yoff + o) *
                                                  sizeof(T)),
                               yin[ot][tt]);
            }
        }
        return;
    }

    // v of the block's tokens into LDS, once per workgroup: the chunk partials
    // of each (token, 4 ranks) are loaded 8 at a time, then summed in order
    const int quads = blk.r_pad / 4;
    if (a.partial) {
        const rsrc_t pr = make_rsrc(a.partial, a.partial_bytes);
        constexpr int G = 8;
        for (int i = threadIdx.x; i < blk.n_tok * quads; i += kWaves * kWaveSize) {
            const int ti = i / quads, j = (i % quads) * 4;
            const uint32_t base_f = uint32_t((blk.rt_before + j / kTile) * a.nproj * a.c0 + p) *
                                        (TT * kTile * kTile) + ti * kTile + j % kTile;
            const uint32_t stride_f = uint32_t(a.nproj) * (TT * kTile * kTile);
            f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int c0 = 0; c0 < a.c0; c0 += G) {
                u32x4 part[G];
#pragma unroll
                for (int g = 0; g < G; ++g)
                    part[g] = bload16(pr, off_or_oob(c0 + g < a.c0,
                                                     (base_f + uint32_t(c0 + g) * stride_f) * 4));
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if (c0 + g < a.c0) s4 += __builtin_bit_cast(f32x4, part[g]);
            }
            *reinterpret_cast<f32x4 *>(&vs[ti][j]) = s4;
        }
    } else {
        for (int i = threadIdx.x; i < blk.n_tok * quads; i += kWaves * kWaveSize) {
            const int ti = i / quads, j = (i % quads) * 4;
            const int t = a.tok[blk.tok_off + ti];
            *reinterpret_cast<f32x4 *>(&vs[ti][j]) = *reinterpret_cast<const f32x4 *>(
                a.v + int64_t(t) * a.ldv + int64_t(p) * a.r_max + j);
        }
    }
    __syncthreads();
    if (o_lo >= o_hi) return;

    // v operand per (token tile, K-step)
    VOperand<T> vop[TT][KSM];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int ks = 0; ks < KSM; ++ks) {
            float f[E];
            const int j0 = ks * SPAN + q * E;
            const bool ok = tv[tt] && ks < ks_n && j0 < blk.r_pad;
            const int row = ok ? tt * kTile + n : 0;
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

    const float s = blk.scale;
#pragma unroll
    for (int ot = 0; ot < OTW; ++ot) {
        const int obase = o_lo + ot * kTile;
        if (obase >= o_hi) break;                    // wave-uniform
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            if (tt >= ntiles) continue;              // wave-uniform
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSM; ++ks) {
                if (ks >= ks_n) continue;
#pragma unroll
                for (int pc = VOperand<T>::kPieces - 1; pc >= 0; --pc)
                    acc = mma<T>(bf[ot][ks], vop[tt][ks].piece[pc], acc);
            }
            const int o = obase + 4 * q;             // 4 consecutive outputs of token n
            float in[4], out[4];
            Out4<T>::unpack(yin[ot][tt], in);
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = in[i] + s * acc[i];
            Out4<T>::store(yr, off_or_oob(tv[tt] && o < o_hi,
                                          uint32_t(int64_t(trow[tt]) * a.ldy + yoff + o) *
                                              sizeof(T)),
                           Out4<T>::pack(out));
        }
    }
}

template <typename T>
hipError_t shrink_dispatch(int tt, const ShrinkArgs &a, hipStream_t s) {
    const dim3 grid(a.grid), block(kWaves * kWaveSize);
    switch (tt) {
    case 1: hipLaunchKernelGGL((k_shrink<T, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_shrink<T, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_shrink<T, 4>), grid, block, 0, s, a); break;
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

hipError_t launch_shrink(int dtype, int tt, const ShrinkArgs &a, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    return dtype == LORA_BF16 ? shrink_dispatch<uint16_t>(tt, a, s)
                              : shrink_dispatch<float>(tt, a, s);
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

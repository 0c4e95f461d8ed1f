// gfx950 kernels of the multi-adapter LoRA delta: shrink (v = A x) and expand
// (y = y_in + s * B v) over the groups of a heterogeneous batch.
//
// Both are thin dense contractions per adapter group (the segmented gather of
// SGMV: "Compress then Serve", rebuttal paragraph on Punica), and both are
// bound by HBM: a decode group streams its adapter's A and B rows once, a
// prefill group streams its token rows.  MFMA is used so that the arithmetic
// costs nothing next to the loads for any group size, not to reach a matrix
// throughput; the loads are 16-byte per lane and each wave streams whole rows.
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

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int E = 8; };   // bf16 bit patterns
template <> struct Elem<float> { static constexpr int E = 4; };

__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    // adapter rows are read once per launch: do not keep them in the caches
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
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

__device__ __forceinline__ uint64_t extent(const BlockDesc &b) {
    return (uint64_t(b.ext_hi) << 32) | b.ext_lo;
}

// Workgroup g runs on XCD g % kXcds.  Give each XCD a contiguous range of
// units, so units that share operands (the x chunk of one block, the partials
// of one block) meet in one L2.
__device__ __forceinline__ int xcd_unit(int grid) {
    const int g = blockIdx.x;
    return (g % kXcds) * (grid / kXcds) + g / kXcds;
}

// unit -> block: the largest b with rt_prefix[b] <= key (rt_prefix[nb] > key)
__device__ __forceinline__ int find_block(const int32_t *rt_prefix, int nb, int key) {
    int lo = 0, hi = nb;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (rt_prefix[mid] <= key) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------- shrink ----
template <typename T, int TT>
__global__ __launch_bounds__(256) void k_shrink(const ShrinkArgs a) {
    constexpr int E = Elem<T>::E;        // elements per 16-byte fragment
    constexpr int SPAN = 4 * E;          // K covered by one fragment over 4 lane groups
    constexpr int UNROLL = 4;
    __shared__ f32x4 red[kWaves][TT][kWaveSize];

    const int u = xcd_unit(a.grid);
    if (u >= a.units) return;            // whole workgroup: no barrier is skipped
    const int lane = threadIdx.x & 63;
    const int w = wave_id();
    const int n = lane & 15, q = lane >> 4;

    // unit -> (block, chunk, rank tile, projection)
    const int per = a.nproj * a.c0;
    const int b = find_block(a.rt_prefix, a.nb, u / per);
    const BlockDesc blk = a.blocks[b];
    int rem = u - a.rt_prefix[b] * per;
    const int p = rem % a.nproj;
    rem /= a.nproj;
    const int rt = rem % blk.rt;
    const int c = rem / blk.rt;

    // operands: rank row j of A (left), token rows (right)
    const T *ablk = reinterpret_cast<const T *>(
        a.slab + extent(blk) + uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_a[p]));
    const int j = rt * kTile + n;
    const bool jv = j < blk.r_pad;
    const T *arow = ablk + int64_t(jv ? j : 0) * a.h_in;
    const T *xrow[TT];
    bool tv[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int ti = tt * kTile + n;
        tv[tt] = ti < blk.n_tok;
        const int t = tv[tt] ? a.tok[blk.tok_off + ti] : 0;
        xrow[tt] = reinterpret_cast<const T *>(a.x) + int64_t(t) * a.ldx;
    }
    const int ntiles = (blk.n_tok + kTile - 1) / kTile;   // wave-uniform

    // this wave's quarter of the chunk
    const int kw = a.kc / kWaves;
    const int k_chunk_end = min(a.h_in, (c + 1) * a.kc);
    const int k_lo = c * a.kc + w * kw;
    const int k_hi = min(k_chunk_end, k_lo + kw);
    f32x4 acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = k_lo; kb < k_hi; kb += SPAN * UNROLL) {
        u32x4 af[UNROLL], xf[TT][UNROLL];
#pragma unroll
        for (int f = 0; f < UNROLL; ++f) {
            const int k = kb + f * SPAN + q * E;
            const bool kv = k < k_hi;
            af[f] = u32x4{0u, 0u, 0u, 0u};
            if (jv && kv) af[f] = ld16_stream(arow + k);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                xf[tt][f] = u32x4{0u, 0u, 0u, 0u};
                if (tt < ntiles && tv[tt] && kv) xf[tt][f] = ld16(xrow[tt] + k);
            }
        }
#pragma unroll
        for (int f = 0; f < UNROLL; ++f) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                if (tt < ntiles) acc[tt] = mma<T>(af[f], xf[tt][f], acc[tt]);
        }
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

// --------------------------------------------------------------- reduce -----
// One workgroup per (adapter block, projection): v = sum of the chunk partials.
template <int TT>
__global__ __launch_bounds__(256) void k_reduce(const ReduceArgs a) {
    const int bp = blockIdx.x;
    const int b = bp / a.nproj, p = bp % a.nproj;
    const BlockDesc blk = a.blocks[b];
    const int per = a.nproj * a.c0;
    const int ubase = a.rt_prefix[b] * per;
    const int quads = a.r_max / 4;
    for (int i = threadIdx.x; i < blk.n_tok * quads; i += blockDim.x) {
        const int ti = i / quads, j = (i % quads) * 4;
        f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < blk.r_pad) {
            const int rt = j / kTile, jj = j % kTile;
            for (int c = 0; c < a.c0; ++c) {
                const int u = ubase + (c * blk.rt + rt) * a.nproj + p;
                s4 += *reinterpret_cast<const f32x4 *>(
                    a.partial + size_t(u) * (TT * kTile * kTile) + ti * kTile + jj);
            }
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

template <typename T> struct OutVec;
template <> struct OutVec<uint16_t> {   // 4 bf16 = 8 bytes
    static __device__ __forceinline__ void load(const void *p, float (&o)[4]) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
        o[0] = __uint_as_float(w[0] << 16); o[1] = __uint_as_float(w[0] & 0xffff0000u);
        o[2] = __uint_as_float(w[1] << 16); o[3] = __uint_as_float(w[1] & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(void *p, const float (&o)[4]) {
        const u32x2 w = u32x2{bf16_rne(o[0]) | (bf16_rne(o[1]) << 16),
                              bf16_rne(o[2]) | (bf16_rne(o[3]) << 16)};
        *reinterpret_cast<u32x2 *>(p) = w;
    }
    static __device__ __forceinline__ void copy(const void *src, void *dst) {
        *reinterpret_cast<u32x2 *>(dst) = *reinterpret_cast<const u32x2 *>(src);
    }
};
template <> struct OutVec<float> {      // 4 float = 16 bytes
    static __device__ __forceinline__ void load(const void *p, float (&o)[4]) {
        const f32x4 w = *reinterpret_cast<const f32x4 *>(p);
        o[0] = w[0]; o[1] = w[1]; o[2] = w[2]; o[3] = w[3];
    }
    static __device__ __forceinline__ void store(void *p, const float (&o)[4]) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{o[0], o[1], o[2], o[3]};
    }
    static __device__ __forceinline__ void copy(const void *src, void *dst) {
        *reinterpret_cast<f32x4 *>(dst) = *reinterpret_cast<const f32x4 *>(src);
    }
};

template <typename T, int TT>
__global__ __launch_bounds__(256) void k_expand(const ExpandArgs a) {
    constexpr int E = Elem<T>::E;
    constexpr int SPAN = 4 * E;                      // ranks per K-step
    constexpr int KS = (LORA_MAX_RANK + SPAN - 1) / SPAN;
    constexpr int OT = 2;                            // o-tiles per iteration
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
    const BlockDesc blk = a.blocks[b];
    const int h_out = a.h_out[p];
    const int o_lo = min(h_out, (oc * kWaves + w) * a.ocw);
    const int o_hi = min(h_out, o_lo + a.ocw);
    const int ntiles = (blk.n_tok + kTile - 1) / kTile;
    const int yoff = a.y_off[p];

    int trow[TT];
    bool tv[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int ti = tt * kTile + n;
        tv[tt] = ti < blk.n_tok;
        trow[tt] = tv[tt] ? a.tok[blk.tok_off + ti] : 0;
    }
    T *y = reinterpret_cast<T *>(a.y);
    const T *base = reinterpret_cast<const T *>(a.base);

    if (blk.r_pad == 0) {            // tokens without an adapter: y = base
        if (!base) return;
        for (int o0 = o_lo; o0 < o_hi; o0 += kTile) {
            const int o = o0 + 4 * q;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt < ntiles && tv[tt] && o < o_hi)
                    OutVec<T>::copy(base + int64_t(trow[tt]) * a.ldb + yoff + o,
                                    y + int64_t(trow[tt]) * a.ldy + yoff + o);
            }
        }
        return;
    }

    // v of the block's tokens into LDS, once per workgroup
    const int quads = blk.r_pad / 4;
    if (a.partial) {
        const int per = a.nproj * a.c0;
        const int ubase = a.rt_prefix[b] * per;
        for (int i = threadIdx.x; i < blk.n_tok * quads; i += kWaves * kWaveSize) {
            const int ti = i / quads, j = (i % quads) * 4;
            const int rt = j / kTile, jj = j % kTile;
            f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < a.c0; ++c) {
                const int uu = ubase + (c * blk.rt + rt) * a.nproj + p;
                s4 += *reinterpret_cast<const f32x4 *>(
                    a.partial + size_t(uu) * (TT * kTile * kTile) + ti * kTile + jj);
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
    const int ks_n = (blk.r_pad + SPAN - 1) / SPAN;  // wave-uniform
    VOperand<T> vop[TT][KS];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float f[E];
            const int j0 = ks * SPAN + q * E;
            const bool ok = tt < ntiles && tv[tt] && ks < ks_n && j0 < blk.r_pad;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                f32x4 w4 = f32x4{0.f, 0.f, 0.f, 0.f};
                if (ok) w4 = *reinterpret_cast<const f32x4 *>(&vs[tt * kTile + n][j0 + e]);
                f[e] = w4[0]; f[e + 1] = w4[1]; f[e + 2] = w4[2]; f[e + 3] = w4[3];
            }
            vop[tt][ks].set(f);
        }
    }

    const T *bblk = reinterpret_cast<const T *>(
        a.slab + extent(blk) + uint64_t(blk.r_pad) * sizeof(T) * uint64_t(a.coef_b[p]));
    const float s = blk.scale;

    for (int o0 = o_lo; o0 < o_hi; o0 += kTile * OT) {
        u32x4 bf[OT][KS];
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
            const int orow = o0 + ot * kTile + n;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int j0 = ks * SPAN + q * E;
                bf[ot][ks] = u32x4{0u, 0u, 0u, 0u};
                if (ks < ks_n && orow < o_hi && j0 < blk.r_pad)
                    bf[ot][ks] = ld16_stream(bblk + int64_t(orow) * blk.r_pad + j0);
            }
        }
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) {
            const int obase = o0 + ot * kTile;
            if (obase >= o_hi) break;
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (tt >= ntiles) continue;
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks >= ks_n) continue;
#pragma unroll
                    for (int pc = VOperand<T>::kPieces - 1; pc >= 0; --pc)
                        acc = mma<T>(bf[ot][ks], vop[tt][ks].piece[pc], acc);
                }
                const int o = obase + 4 * q;     // 4 consecutive outputs of token n
                if (tv[tt] && o < o_hi) {
                    T *yp = y + int64_t(trow[tt]) * a.ldy + yoff + o;
                    float in[4];
                    if (base) OutVec<T>::load(base + int64_t(trow[tt]) * a.ldb + yoff + o, in);
                    else OutVec<T>::load(yp, in);
                    float out[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) out[i] = in[i] + s * acc[i];
                    OutVec<T>::store(yp, out);
                }
            }
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

template <typename T>
hipError_t expand_dispatch(int tt, const ExpandArgs &a, hipStream_t s) {
    const dim3 grid(a.grid), block(kWaves * kWaveSize);
    switch (tt) {
    case 1: hipLaunchKernelGGL((k_expand<T, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_expand<T, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_expand<T, 4>), grid, block, 0, s, a); break;
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

hipError_t launch_expand(int dtype, int tt, const ExpandArgs &a, hipStream_t s) {
    if (a.units <= 0) return hipSuccess;
    return dtype == LORA_BF16 ? expand_dispatch<uint16_t>(tt, a, s)
                              : expand_dispatch<float>(tt, a, s);
}

}  // namespace lora

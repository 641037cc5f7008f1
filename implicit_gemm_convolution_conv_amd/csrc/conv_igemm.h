// Pieces shared by every implicit-GEMM conv kernel for gfx950 (CDNA4): vector
// types, MFMA accumulator types, the workgroup -> output tile schedule and the
// output transform of the epilogue.
//
// The convolution is one GEMM: rows are output positions m = (n, od, oh, ow),
// columns are output channels k, the reduction runs over (t, r, s, c) with c
// fastest, the layout of the packed filter and of NDHWC activations (FlyDSL
// PR #860, PR summary: A is gathered from the activations per tile, B is a
// plain KTRSC matrix). Point-output shapes (MIOpen PR #10912) use the same
// GEMM with the filter as A and the flattened images as B.
#pragma once

#include "igconv_internal.h"

namespace igc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 16-byte load from an address that is only known to be 4-byte aligned.
typedef int i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int MF>
struct AccType {
    using type = f32x4;
};
template <>
struct AccType<32> {
    using type = f32x16;
};

// Quad q (4 consecutive rows of one column) of an accumulator block.
template <int MF>
__device__ inline f32x4 quad(const typename AccType<MF>::type &acc, int q)
{
    if constexpr (MF == 16) {
        return acc;
    } else {
        return f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    }
}

template <bool BIG>
struct OffType {
    using type = int32_t;
};
template <>
struct OffType<true> {
    using type = int64_t;
};

// Workgroup -> output tile. Workgroups are handed to the 8 XCDs round-robin,
// so block b runs on XCD b % 8; renumber so that consecutive logical tiles
// share an XCD (and its L2), then walk the tiles in groups of group_m tile
// rows, all columns of a group before the next group.
__device__ inline void tile_coords(const ConvParams &p, int bid, int &tm, int &tn)
{
    const int nblk = p.tiles_m * p.tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int q = nblk >> 3, r = nblk & 7;
    const int lin = xcd * q + min(xcd, r) + idx;
    const int gsz = p.group_m * p.tiles_n;
    const int g = p.div_gsz.div(lin);
    const int first = g * p.group_m;
    const int rows = min(p.tiles_m - first, p.group_m);
    const int in = lin - g * gsz;
    if (rows == p.group_m) {
        tn = p.div_gm.div(in);
    } else {  // the last, shorter group
        tn = in / rows;
    }
    tm = first + in - tn * rows;
    if (p.tap_stride > 0) {  // temporal raster: the group's tiles one tap apart, within whole blocks
        const int blk = p.group_m * p.tap_stride;
        if (tm < p.div_blk.div(p.tiles_m) * blk) {
            const int b = p.div_blk.div(tm), r = tm - b * blk;
            const int gi = p.div_gm.div(r), c = r - gi * p.group_m;  // group gi of the block, member c
            tm = b * blk + c * p.tap_stride + gi;
        }
    }
}

__device__ inline void tile_coords(const ConvParams &p, int &tm, int &tn) { tile_coords(p, blockIdx.x, tm, tn); }

// Have the scalar loads of the parameters a workgroup's setup reads issued
// together at kernel entry. Left alone, the compiler loads each field where
// it is first used and waits for it there, one memory round trip per field:
// about 0.9 us before the first operand load of the point-output kernel.
__device__ __attribute__((always_inline)) inline void preload_setup_params(const ConvParams &p)
{
    asm volatile("" ::"s"(p.tiles_m), "s"(p.tiles_n), "s"(p.group_m), "s"(p.tap_stride), "s"(p.splits),
                 "s"(p.ksplit), "s"(p.tail_first), "s"(p.tail_splits), "s"(p.div_gsz.m), "s"(p.div_gsz.l),
                 "s"(p.div_gm.m), "s"(p.div_gm.l), "s"(p.div_blk.m), "s"(p.div_blk.l));
    asm volatile("" ::"s"(p.x), "s"(p.w), "s"(p.M), "s"(p.Ncol), "s"(p.Rk), "s"(p.ldw), "s"(p.nk), "s"(p.P),
                 "s"(p.div_P.m), "s"(p.div_P.l), "s"(p.div_HW.m), "s"(p.div_HW.l), "s"(p.div_Wo.m), "s"(p.div_Wo.l));
}

// Two fp32 values -> their bf16 bits (a in the low half), rounded to nearest
// even by gfx950's packed conversion (one v_cvt_pk_bf16_f32). Over all 2^32
// fp32 bit patterns it gives the bits of the software rounding it replaces,
// (u + 0x7fff + lsb) >> 16 with NaN -> (u >> 16) | 0x40, NaNs included.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __attribute__((always_inline)) inline uint32_t bf16_pack2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __attribute__((always_inline)) inline uint32_t f32_to_bf16_rne(float f) { return bf16_pack2(f, 0.0f) & 0xffffu; }

// Output transform of every epilogue: y = bf16(acc * scale + bias[k]), the
// scale s_x * s_w for fp8 and 1 for bf16, the bias (fp32, one per output
// channel) only when given. With p.amax set it also keeps the running maximum
// of |y| over the values this lane stores (non-negative floats order like
// their bits, so the maximum of bf16 bits & 0x7fff) and flush() merges the
// wave's maximum into *p.amax as fp32 bits. EXTRAS = false compiles the bias
// and amax out: kernels pick the instance once per launch (with_epilogue), so
// a call without extras runs the plain epilogue with no per-element tests.
template <bool EXTRAS>
struct Epilogue {
    float sc;
    const float *bias;
    unsigned *amax;
    unsigned m = 0;

    __device__ Epilogue(const ConvParams &p, bool fp8)
        : sc(fp8 ? p.scales[0] * p.scales[2] : 1.0f), bias(p.bias), amax(p.amax) {}

    // bf16 bits of the output of channel k
    __device__ __attribute__((always_inline)) uint32_t one(float acc, int k)
    {
        float v = acc * sc;
        if constexpr (EXTRAS) {
            if (bias)
                v += bias[k];
        }
        const uint32_t r = f32_to_bf16_rne(v);
        if constexpr (EXTRAS) {
            if (amax)
                m = max(m, r & 0x7fffu);
        }
        return r;
    }
    // four outputs of channel k, packed for one 8-byte store
    __device__ __attribute__((always_inline)) u32x2 four(const f32x4 &acc, int k)
    {
        float b = 0.0f;
        if constexpr (EXTRAS)
            b = bias ? bias[k] : 0.0f;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = acc[e] * sc;
            if constexpr (EXTRAS) {
                if (bias)
                    v[e] += b;
            }
        }
        const u32x2 r = {bf16_pack2(v[0], v[1]), bf16_pack2(v[2], v[3])};
        if constexpr (EXTRAS) {
            if (amax)
                m = max(m, max(max(r[0] & 0x7fffu, (r[0] >> 16) & 0x7fffu), max(r[1] & 0x7fffu, (r[1] >> 16) & 0x7fffu)));
        }
        return r;
    }
    // four outputs of channels k .. k + 3 (point output: channels are the rows)
    __device__ __attribute__((always_inline)) u32x2 four_channels(const f32x4 &acc, int k)
    {
        uint32_t r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = one(acc[e], k + e);
        return u32x2{r[0] | (r[1] << 16), r[2] | (r[3] << 16)};
    }
    // every lane of the wave calls this once, after its last store
    __device__ __attribute__((always_inline)) void flush()
    {
        if constexpr (EXTRAS) {
            if (!amax)
                return;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1)
                m = max(m, (unsigned)__shfl_xor((int)m, off));
            if ((threadIdx.x & 63) == 0)
                atomicMax(amax, m << 16);
        }
    }
};

// Run body(ep) with the epilogue instance this launch needs.
template <typename F>
__device__ __attribute__((always_inline)) inline void with_epilogue(const ConvParams &p, bool fp8, F &&body)
{
    if (p.bias || p.amax) {
        Epilogue<true> ep(p, fp8);
        body(ep);
        ep.flush();
    } else {
        Epilogue<false> ep(p, fp8);
        body(ep);
    }
}

}  // namespace igc

// Implicit-GEMM forward convolution kernel for gfx950 (CDNA4), bf16 and fp8.
//
// The convolution is one GEMM: rows are output positions m = (n, od, oh, ow),
// columns are output channels k, the reduction runs over (t, r, s, c) with c
// fastest, the layout of the packed filter and of NDHWC activations (FlyDSL
// PR #860, PR summary: A is gathered from the activations per tile, B is a
// plain KTRSC matrix). Point-output shapes (MIOpen PR #10912) use the same
// kernel with the filter as A and the flattened images as B.
//
// Per workgroup: a BM x BN fp32 accumulator tile split over WM x WN waves,
// each wave owning (BM/WM) x (BN/WN) as 16x16 MFMA blocks. Each reduction step
// covers 128 bytes of k per row (64 bf16 or 128 fp8) and is staged in LDS,
// double-buffered: the global loads of step s+1 are in flight while step s
// feeds the MFMAs. LDS rows are 128 bytes (eight 16-byte chunks); chunk q of
// row r is stored in slot q ^ (r & 7) so that the MFMA fragment reads (16 rows,
// one chunk each) hit distinct banks.
//
// Zero padding: an im2col tap outside the input box, a row past M and a
// reduction index past C*T*R*S are loaded as zero (predicated loads), so the
// MFMAs need no masking.
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
    const int g = lin / gsz;
    const int first = g * p.group_m;
    const int rows = min(p.tiles_m - first, p.group_m);
    const int in = lin - g * gsz;
    tm = first + in % rows;
    tn = in / rows;
    if (p.tap_stride > 0) {  // temporal raster: the group's tiles one tap apart, within whole blocks
        const int blk = p.group_m * p.tap_stride;
        if (tm < p.tiles_m / blk * blk) {
            const int b = tm / blk, r = tm - b * blk;
            const int gi = r / p.group_m, c = r - gi * p.group_m;  // group gi of the block, member c
            tm = b * blk + c * p.tap_stride + gi;
        }
    }
}

__device__ inline void tile_coords(const ConvParams &p, int &tm, int &tn) { tile_coords(p, blockIdx.x, tm, tn); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ inline uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

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
        uint32_t r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = acc[e] * sc;
            if constexpr (EXTRAS) {
                if (bias)
                    v += b;
            }
            r[e] = f32_to_bf16_rne(v);
            if constexpr (EXTRAS) {
                if (amax)
                    m = max(m, r[e] & 0x7fffu);
            }
        }
        return u32x2{r[0] | (r[1] << 16), r[2] | (r[3] << 16)};
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

template <int BM, int BN, int WM, int WN, int MF, int DT, int MODE, bool BIG, bool CBLK>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void conv_igemm_kernel(ConvParams p)
{
    using Off = typename OffType<BIG>::type;
    constexpr int THREADS = WM * WN * 64;
    constexpr int ESZ = DT == DT_FP8 ? 1 : 2;  // bytes per element
    constexpr int CH = 16 / ESZ;               // elements per 16-byte chunk
    constexpr int TKE = 8 * CH;                // elements per reduction step (128 bytes)
    constexpr int RSTEP = THREADS / 8;         // tile rows covered by one pass of the loaders
    constexpr int AIT = BM / RSTEP;            // A rows loaded per thread
    constexpr int BIT = BN / RSTEP;            // B rows loaded per thread
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int STAGE = (BM + BN) * 128;
    static_assert(BM % RSTEP == 0 && BN % RSTEP == 0 && AIT >= 1 && BIT >= 1, "loader split");
    static_assert(RSTEP % 8 == 0, "a thread's rows must share (row & 7)");
    static_assert(MF == 16 || MF == 32, "MFMA block size");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "MFMA blocks");
    static_assert(2 * STAGE <= 160 * 1024, "LDS budget");
    static_assert(MODE != MODE_POINT || !CBLK, "point mode reduces in natural order");

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int jc = tid & 7;            // chunk column this thread loads
    const int r0 = tid >> 3;           // its first tile row
    const int slot = (jc ^ (r0 & 7)) * 16;  // its swizzled LDS slot (same for all its rows)

    const char *xb = static_cast<const char *>(p.x);
    const char *wb = static_cast<const char *>(p.w);

    // ---------------------------------------------------------------- A rows
    // im2col modes: per row, the input origin (id0, ih0, iw0) and the element
    // offset of (n, id0, ih0, iw0, c=0); rows past M get an origin far outside
    // the box so that every tap fails the bounds check.
    int a_id0[AIT], a_ih0[AIT], a_iw0[AIT];
    Off a_base[AIT];
    const char *a_row[AIT];  // point mode: filter rows
    bool a_ok[AIT];
    if constexpr (MODE != MODE_POINT) {
        const int hw = p.Ho * p.Wo;
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            const int m = m0 + r0 + i * RSTEP;
            if (m < p.M) {
                const int nimg = m / p.P;
                const int sp = m - nimg * p.P;
                const int od = sp / hw;
                const int rem = sp - od * hw;
                const int oh = rem / p.Wo;
                const int ow = rem - oh * p.Wo;
                a_id0[i] = od * p.sd - p.pd;
                a_ih0[i] = oh * p.sh - p.ph;
                a_iw0[i] = ow * p.sw - p.pw;
                if constexpr (MODE == MODE_TEMPORAL)  // Ho == H, Wo == W: the (h, w) index carries over
                    a_base[i] = (((Off)nimg * p.D + a_id0[i]) * (Off)(p.H * p.W) + rem) * (Off)p.C;
                else
                    a_base[i] = ((((Off)nimg * p.D + a_id0[i]) * p.H + a_ih0[i]) * (Off)p.W + a_iw0[i]) * (Off)p.C;
            } else {
                a_id0[i] = a_ih0[i] = a_iw0[i] = -(1 << 29);
                a_base[i] = 0;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            const int k = m0 + r0 + i * RSTEP;  // filter row
            a_ok[i] = k < p.M;
            a_row[i] = wb + (a_ok[i] ? (int64_t)k * p.ldw * ESZ : 0);
        }
    }

    // ---------------------------------------------------------------- B rows
    const char *b_row[BIT];
    bool b_ok[BIT];
#pragma unroll
    for (int i = 0; i < BIT; ++i) {
        const int n = n0 + r0 + i * RSTEP;
        b_ok[i] = n < p.Ncol;
        if constexpr (MODE == MODE_POINT)  // image n, flattened: Rk elements
            b_row[i] = xb + (b_ok[i] ? (int64_t)n * p.Rk * ESZ : 0);
        else  // filter row n
            b_row[i] = wb + (b_ok[i] ? (int64_t)n * p.ldw * ESZ : 0);
    }

    // ---------------------------------------------------------- k position
    // This thread's chunk starts at reduction index kc of the packed filter;
    // for the im2col modes also channel c and tap (t, r, s).
    int kc, c = 0, t = 0, r = 0, s = 0;
    bool kval = true;
    if constexpr (MODE == MODE_POINT || !CBLK) {
        kc = jc * CH;
        if constexpr (MODE != MODE_POINT) {
            c = kc % p.C;
            const int tap = kc / p.C;
            s = tap % p.S;
            r = (tap / p.S) % p.R;
            t = tap / (p.S * p.R);
            kval = kc < p.Rk;
        }
    } else {  // channel block outer, taps inner: C % TKE == 0
        c = jc * CH;
        kc = c;
    }
    Off tapoff = 0;  // x offset of tap (t, r, s) plus c, relative to a row origin
    auto update_tapoff = [&]() {
        if constexpr (MODE == MODE_TEMPORAL)
            tapoff = (Off)(t * p.dd) * (Off)(p.H * p.W) * (Off)p.C + c;
        else if constexpr (MODE == MODE_GENERIC)
            tapoff = (((Off)(t * p.dd) * p.H + r * p.dh) * (Off)p.W + s * p.dw) * (Off)p.C + c;
    };
    update_tapoff();

    auto advance = [&]() {
        if constexpr (MODE == MODE_POINT) {
            kc += TKE;
        } else if constexpr (CBLK) {
            if (++s == p.S) {
                s = 0;
                if (++r == p.R) {
                    r = 0;
                    if (++t == p.T) {
                        t = 0;
                        c += TKE;
                    }
                }
            }
            kc = ((t * p.R + r) * p.S + s) * p.C + c;
            update_tapoff();
        } else {
            kc += TKE;
            kval = kc < p.Rk;
            c += TKE;
            while (c >= p.C) {
                c -= p.C;
                if (++s == p.S) {
                    s = 0;
                    if (++r == p.R) {
                        r = 0;
                        ++t;
                    }
                }
            }
            update_tapoff();
        }
    };

    // ---------------------------------------------------------- global loads
    i32x4 areg[AIT], breg[BIT];
    auto load_tiles = [&]() {
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            i32x4 v = {0, 0, 0, 0};
            if constexpr (MODE == MODE_POINT) {
                if (a_ok[i])
                    v = *reinterpret_cast<const i32x4 *>(a_row[i] + (int64_t)kc * ESZ);
            } else {
                bool ok;
                if constexpr (MODE == MODE_TEMPORAL) {
                    ok = kval && (unsigned)(a_id0[i] + t * p.dd) < (unsigned)p.D;
                } else {
                    ok = kval && (unsigned)(a_id0[i] + t * p.dd) < (unsigned)p.D &&
                         (unsigned)(a_ih0[i] + r * p.dh) < (unsigned)p.H &&
                         (unsigned)(a_iw0[i] + s * p.dw) < (unsigned)p.W;
                }
                if (ok)
                    v = *reinterpret_cast<const i32x4 *>(xb + (a_base[i] + tapoff) * ESZ);
            }
            areg[i] = v;
        }
#pragma unroll
        for (int i = 0; i < BIT; ++i) {
            i32x4 v = {0, 0, 0, 0};
            if constexpr (MODE == MODE_POINT) {
                // image rows are only 4-byte aligned and end at Rk (no padding)
                if (b_ok[i]) {
                    const char *ptr = b_row[i] + (int64_t)kc * ESZ;
                    if (kc + CH <= p.Rk) {
                        const i32x4_a4 u = *reinterpret_cast<const i32x4_a4 *>(ptr);
                        v = i32x4{u[0], u[1], u[2], u[3]};
                    } else if (kc < p.Rk) {
                        const int nbytes = (p.Rk - kc) * ESZ;  // a multiple of 4
                        for (int q = 0; q < 4; ++q)
                            if (4 * q < nbytes)
                                v[q] = *reinterpret_cast<const int *>(ptr + 4 * q);
                    }
                }
            } else {
                if (b_ok[i])
                    v = *reinterpret_cast<const i32x4 *>(b_row[i] + (int64_t)kc * ESZ);
            }
            breg[i] = v;
        }
    };

    auto store_tiles = [&](char *st) {
#pragma unroll
        for (int i = 0; i < AIT; ++i)
            *reinterpret_cast<i32x4 *>(st + (r0 + i * RSTEP) * 128 + slot) = areg[i];
        char *bs = st + BM * 128;
#pragma unroll
        for (int i = 0; i < BIT; ++i)
            *reinterpret_cast<i32x4 *>(bs + (r0 + i * RSTEP) * 128 + slot) = breg[i];
    };

    // ---------------------------------------------------------------- MFMA
    // MF = 16: 16x16 blocks (bf16 16x16x32, fp8 16x16x128), a lane owns rows
    //          4*(lane/16) + 0..3 of column lane%16 of each block.
    // MF = 32: 32x32 blocks (bf16 32x32x16, fp8 32x32x64), a lane owns rows
    //          8*q + 4*(lane/32) + 0..3 (q = 0..3) of column lane%32.
    // A lane's operand fragment is one row (column) of its block, lane % MF,
    // and 16 (bf16) or 32 (fp8) bytes of k; A and B take the same k bytes, so
    // which bytes a lane holds does not change the product.
    using AccT = typename AccType<MF>::type;
    AccT acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
            acc[a][b] = AccT{};

    const int lrow = lane & (MF - 1), lgrp = lane / MF, lsw = lane & 7;
    auto compute = [&](const char *st) {
        const char *aw = st + (wm * WTM + lrow) * 128;
        const char *bw = st + BM * 128 + (wn * WTN + lrow) * 128;
        constexpr int GROUPS = 64 / MF;            // lane groups per block (k split)
        constexpr int CPL = DT == DT_BF16 ? 1 : 2;  // 16-byte chunks per lane per MFMA
        constexpr int SUB = 8 / (GROUPS * CPL);     // MFMAs per block per reduction step
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            // chunks of this lane: (h * GROUPS + lgrp) * CPL + 0..CPL-1
            const int c0 = (h * GROUPS + lgrp) * CPL;
            const int sl0 = (c0 ^ lsw) * 16;
            const int sl1 = ((c0 + 1) ^ lsw) * 16;
            if constexpr (DT == DT_BF16) {
                bf16x8 bf[FN];
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    bf[b] = *reinterpret_cast<const bf16x8 *>(bw + b * MF * 128 + sl0);
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8 *>(aw + a * MF * 128 + sl0);
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        if constexpr (MF == 16)
                            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[b], acc[a][b], 0, 0, 0);
                        else
                            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[b], acc[a][b], 0, 0, 0);
                    }
                }
            } else {
                i32x8 bf[FN];
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const i32x4 lo = *reinterpret_cast<const i32x4 *>(bw + b * MF * 128 + sl0);
                    const i32x4 hi = *reinterpret_cast<const i32x4 *>(bw + b * MF * 128 + sl1);
                    bf[b] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const i32x4 lo = *reinterpret_cast<const i32x4 *>(aw + a * MF * 128 + sl0);
                    const i32x4 hi = *reinterpret_cast<const i32x4 *>(aw + a * MF * 128 + sl1);
                    const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        // operand formats 0/0: both E4M3; zero scale operands select the unscaled MFMA
                        if constexpr (MF == 16)
                            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b], acc[a][b], 0, 0,
                                                                                         0, 0, 0, 0);
                        else
                            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[b], acc[a][b], 0, 0,
                                                                                        0, 0, 0, 0);
                    }
                }
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    load_tiles();
    store_tiles(smem);
    __syncthreads();
    for (int ks = 0; ks < p.nk; ++ks) {
        const bool more = ks + 1 < p.nk;
        if (more) {
            advance();
            load_tiles();
        }
        compute(smem + (ks & 1) * STAGE);
        if (more)
            store_tiles(smem + ((ks + 1) & 1) * STAGE);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // Each lane holds groups of 4 consecutive GEMM rows of one column ("quads").
    uint16_t *yb = static_cast<uint16_t *>(p.y);
    with_epilogue(p, DT == DT_FP8, [&](auto &ep) __attribute__((always_inline)) {
        constexpr int QUADS = MF / 16 * (MF / 16);  // 1 (16x16) or 4 (32x32) per block
#pragma unroll
        for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int q = 0; q < QUADS; ++q) {
                // first of the 4 consecutive GEMM rows of this quad
                const int row = m0 + wm * WTM + a * MF + (MF == 16 ? 4 * lgrp : 8 * q + 4 * lgrp);
                if constexpr (MODE != MODE_POINT) {
                    int nimg = 0, sp = 0;
                    if (row < p.M) {
                        nimg = row / p.P;
                        sp = row - nimg * p.P;
                    }
                    const bool vec = (p.P & 3) == 0 && row + 3 < p.M;  // 4 rows in one image, 8-byte aligned
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        const int col = n0 + wn * WTN + b * MF + lrow;  // output channel
                        if (row >= p.M || col >= p.K)
                            continue;
                        const f32x4 v = quad<MF>(acc[a][b], q);
                        if (vec) {
                            *reinterpret_cast<u32x2 *>(yb + ((Off)nimg * p.K + col) * (Off)p.P + sp) = ep.four(v, col);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int m = row + e;
                                if (m < p.M) {
                                    const int n2 = m / p.P;
                                    const int sp2 = m - n2 * p.P;
                                    yb[((Off)n2 * p.K + col) * (Off)p.P + sp2] = (uint16_t)ep.one(v[e], col);
                                }
                            }
                        }
                    }
                } else {
                    // rows are output channels, columns are images: y[n][k] is contiguous in k
                    const bool vec = (p.K & 3) == 0 && row + 3 < p.M;
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        const int col = n0 + wn * WTN + b * MF + lrow;  // image
                        if (row >= p.M || col >= p.Ncol)
                            continue;
                        const f32x4 v = quad<MF>(acc[a][b], q);
                        uint16_t *dst = yb + (Off)col * p.K + row;
                        if (vec) {
                            *reinterpret_cast<u32x2 *>(dst) = ep.four_channels(v, row);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (row + e < p.M)
                                    dst[e] = (uint16_t)ep.one(v[e], row + e);
                        }
                    }
                }
            }
        }
    });
}

// Launch helper for one dtype: picks the instantiation for (tile, mode, big, cblock).
template <int DT>
hipError_t launch_conv_dt(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
#define IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_, BIG_, CBLK_)                                                  \
    do {                                                                                                       \
        hipLaunchKernelGGL((conv_igemm_kernel<BM_, BN_, WM_, WN_, MF_, DT, MODE_, BIG_, CBLK_>), grid,         \
                           dim3(WM_ * WN_ * 64), 0, stream, p);                                                \
        return hipGetLastError();                                                                              \
    } while (0)
#define IGC_MODES(BM_, BN_, WM_, WN_, MF_)                                                                     \
    do {                                                                                                       \
        if (mode == MODE_POINT) {                                                                              \
            if (big) IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_POINT, true, false);                             \
            IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_POINT, false, false);                                     \
        }                                                                                                      \
        if (mode == MODE_TEMPORAL) {                                                                           \
            if (big) {                                                                                         \
                if (cblock) IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_TEMPORAL, true, true);                    \
                IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_TEMPORAL, true, false);                               \
            }                                                                                                  \
            if (cblock) IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_TEMPORAL, false, true);                       \
            IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_TEMPORAL, false, false);                                  \
        }                                                                                                      \
        if (big) {                                                                                             \
            if (cblock) IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_GENERIC, true, true);                         \
            IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_GENERIC, true, false);                                    \
        }                                                                                                      \
        if (cblock) IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_GENERIC, false, true);                            \
        IGC_LAUNCH(BM_, BN_, WM_, WN_, MF_, MODE_GENERIC, false, false);                                       \
    } while (0)
    switch (tile) {
    case 0: IGC_MODES(256, 256, 2, 4, 16);
    case 1: IGC_MODES(128, 128, 2, 2, 16);
    case 2: IGC_MODES(64, 64, 2, 2, 16);
    case 3: IGC_MODES(256, 256, 2, 4, 32);
    case 4: IGC_MODES(128, 128, 2, 2, 32);
    default: IGC_MODES(64, 64, 2, 2, 32);
    }
#undef IGC_MODES
#undef IGC_LAUNCH
}

}  // namespace igc

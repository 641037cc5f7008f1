// Implicit-GEMM forward convolution, im2col paths, with a multi-stage
// direct-to-LDS pipeline (gfx950 global_load_lds_dwordx4).
//
// Rows = output positions, columns = output channels, reduction over
// (t, r, s, c) with c fastest. The operand tiles go from global memory
// straight into LDS without passing through registers, as the async
// global->LDS pipeline of FlyDSL PR #860 does (async DMA commit). Freed of
// staging registers, the ring holds S stages of 128 bytes of k per row, so a
// load is issued S-1 reduction steps before its data are consumed, which
// hides L2-miss latency that a one-step register prefetch exposes.
//
// An LDS-DMA instruction writes lane i's 16 bytes at base + 16 * i: one wave
// instruction fills 8 consecutive 128-byte rows. The LDS layout (chunk q of
// row r at slot q ^ (r & 7)) is therefore produced by choosing which chunk
// each lane fetches. Zero padding: a lane whose tap falls outside the
// input box (or whose row is past M, or whose reduction index is past
// C*T*R*S) fetches a 16-byte zero line instead.
//
// Point-output mode (MIOpen PR #10912: one GEMM over the batch) uses the
// filter as A and the flattened images as B. Image rows end at C*T*R*S
// elements with no padding and are only 4-byte aligned; the one chunk that
// straddles a row's end is fetched as zeros by the DMA and then overwritten
// from registers with its valid bytes before the last step is consumed.
//
// Split reduction (split-K, for grids of output tiles too small to occupy the
// GPU; FlyDSL PR #860 chooses it only when the tile grid under-fills the
// device): with p.splits > 1 the grid holds p.splits workgroups per tile, each
// runs a contiguous range of reduction steps from its own start position and
// stores unscaled fp32 sums; launch_splitk_reduce adds the slices in split
// order, scales and rounds to bf16.
#pragma once

#include <type_traits>

#include "conv_igemm.h"

namespace igc {

// Sixteen zero bytes: the source of every padding chunk.
__device__ __attribute__((aligned(16))) const int kZeroLine[4] = {0, 0, 0, 0};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// Epilogue through LDS for a whole tile: the rings are idle after the last
// step, so the workgroup writes its bf16 outputs there as [column][row]
// (column stride 2 * BM + 16 bytes), then every lane stores 16 bytes: 8
// consecutive rows of one column, so that each column's 2 * BM bytes of y go
// out as whole 128-byte lines. The direct epilogue writes 32-byte pieces of
// lines from 4 separate instructions. Same output transform as Epilogue
// (y = bf16(acc * scale [+ bias])); the amax of y, when asked for, is folded
// from the bf16 values as they leave LDS.
// im2col tiles (rows = positions, columns = channels): needs P % 8 == 0
// (16-byte aligned rows), the tile's rows in one image and all its columns
// below K. Point tiles (POINT: rows = channels, columns = images, y[n][k]
// contiguous in k with rows of p.K): needs p.K % 8 == 0 and the whole tile
// inside the GEMM. The callers check that and otherwise store directly.
template <int BM, int BN, int WM, int WN, int MF, int DT, bool POINT>
__device__ __attribute__((always_inline)) inline void store_tile_lds(
    const typename AccType<MF>::type (&acc)[BM / WM / MF][BN / WN / MF], const ConvParams &p, int m0, int n0,
    int wm, int wn, int lane, char *smem)
{
    constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / MF, FN = WTN / MF;
    constexpr int CS = 2 * BM + 16;      // bytes per column in LDS
    constexpr int NT = WM * WN * 64;     // threads
    constexpr int PIECES = BM * 2 / 16;  // 16-byte pieces per column
    static_assert(MF == 16, "16x16 MFMA blocks");
    static_assert((BN * PIECES) % NT == 0, "whole rounds of pieces");
    const int lrow = lane & 15, lgrp = lane >> 4;
    const float sc = DT == DT_FP8 ? p.scales[0] * p.scales[2] : 1.0f;
    __syncthreads();  // every wave has finished reading the rings
    auto put = [&](auto with_bias) __attribute__((always_inline)) {
        constexpr bool BIAS = decltype(with_bias)::value;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int col = wn * WTN + b * MF + lrow;
                const int row = wm * WTM + a * MF + 4 * lgrp;
                const f32x4 v = quad<MF>(acc[a][b], 0);
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t[e] = v[e] * sc;
                    if constexpr (BIAS)
                        t[e] += p.bias[POINT ? m0 + row + e : n0 + col];  // bias of the output channel
                }
                *reinterpret_cast<u32x2 *>(smem + col * CS + row * 2) = u32x2{bf16_pack2(t[0], t[1]), bf16_pack2(t[2], t[3])};
            }
    };
    if (p.bias)
        put(std::true_type{});
    else
        put(std::false_type{});
    __syncthreads();
    const int nimg = POINT ? 0 : p.div_P.div(m0);
    const int sp0 = POINT ? 0 : m0 - nimg * p.P;
    uint16_t *yb = static_cast<uint16_t *>(p.y);
    unsigned m = 0;
#pragma unroll
    for (int it = 0; it < BN * PIECES / NT; ++it) {
        const int idx = it * NT + (int)threadIdx.x;
        const int col = idx / PIECES, piece = idx - col * PIECES;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(smem + col * CS + piece * 16);
        const int64_t off = POINT ? (int64_t)(n0 + col) * p.K + m0 + piece * 8
                                  : ((int64_t)nimg * p.K + n0 + col) * p.P + sp0 + piece * 8;
        // streaming store: y is not read again by this kernel, and lines that bypass L2 need no
        // write-back when the kernel ends (the 24 MB output of the 9500-image patch embed lands about 1 us sooner)
        __builtin_nontemporal_store(v, reinterpret_cast<i32x4 *>(yb + off));
#pragma unroll
        for (int q = 0; q < 4; ++q)
            m = max(m, max((unsigned)v[q] & 0x7fffu, ((unsigned)v[q] >> 16) & 0x7fffu));
    }
    if (p.amax) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            m = max(m, (unsigned)__shfl_xor((int)m, off));
        if (lane == 0)
            atomicMax(p.amax, m << 16);
    }
}

template <int BM, int BN, int WM, int WN, int MF, int DT, int MODE, bool BIG, bool CBLK, int S, int KB = 128>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void conv_igemm_dma_kernel(ConvParams p)
{
    using Off = typename OffType<BIG>::type;
    constexpr int NW = WM * WN;                // waves
    constexpr int ESZ = DT == DT_FP8 ? 1 : 2;  // bytes per element
    constexpr int CH = 16 / ESZ;               // elements per 16-byte chunk
    constexpr int TKE = KB / ESZ;              // elements per reduction step
    constexpr int RPI = 1024 / KB;             // rows filled by one DMA instruction (64 lanes x 16 B)
    constexpr int CPR = KB / 16;               // 16-byte chunks per row
    constexpr int AIT = BM / (RPI * NW);       // A row groups per wave
    constexpr int BIT = BN / (RPI * NW);
    constexpr int LPS = AIT + BIT;             // LDS-DMA loads per thread per stage
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int STAGE = (BM + BN) * KB;
    static_assert(MODE != MODE_POINT || !CBLK, "point mode reduces in natural order");
    static_assert(KB == 128, "128-byte steps");
    static_assert(AIT >= 1 && BIT >= 1 && BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "loader split");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "MFMA blocks");
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS budget");
    static_assert(LPS * (S - 2) < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    preload_setup_params(p);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the LDS destinations go to M0
    const int wm = wave % WM, wn = wave / WM;

    // Split reduction: workgroups [j * tiles, (j + 1) * tiles) run split j of every tile.
    const int ntiles = p.tiles_m * p.tiles_n;
    const int split = p.splits > 1 ? (int)blockIdx.x / ntiles : 0;
    const int kbeg = split * p.ksplit;  // first reduction step of this workgroup
    int tm, tn;
    tile_coords(p, (int)blockIdx.x - split * ntiles, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // This lane's row within each RPI-row group and the chunk it fetches there:
    // chunk q of a row sits at slot q ^ (row & 7).
    const int lr = lane / CPR;
    const int jc = (lane & 7) ^ (lane >> 3);

    const char *xb = static_cast<const char *>(p.x);
    const char *wb = static_cast<const char *>(p.w);
    const char *zero = reinterpret_cast<const char *>(kZeroLine);
    asm volatile("" : "+v"(zero));  // held in registers: otherwise rebuilt (s_getpc and an add) before every load

    // ---------------------------------------------------------------- A rows
    // im2col modes: input origin of each row; point mode: filter rows (rows
    // past M load row M - 1, whose results are never stored).
    int a_id0[AIT], a_ih0[AIT], a_iw0[AIT];
    Off a_base[AIT];
    const char *a_row[AIT];
    if constexpr (MODE == MODE_POINT) {
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            const int k = min(m0 + RPI * (wave + i * NW) + lr, p.M - 1);
            a_row[i] = wb + (int64_t)k * p.ldw * ESZ;
        }
    } else {
        const int hw = p.Ho * p.Wo;
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            const int m = m0 + RPI * (wave + i * NW) + lr;
            if (m < p.M) {
                const int nimg = p.div_P.div(m);
                const int sp = m - nimg * p.P;
                const int od = p.div_HW.div(sp);
                const int rem = sp - od * hw;
                const int oh = p.div_Wo.div(rem);
                const int ow = rem - oh * p.Wo;
                a_id0[i] = od * p.sd - p.pd;
                a_ih0[i] = oh * p.sh - p.ph;
                a_iw0[i] = ow * p.sw - p.pw;
                if constexpr (MODE == MODE_TEMPORAL)
                    a_base[i] = (((Off)nimg * p.D + a_id0[i]) * (Off)(p.H * p.W) + rem) * (Off)p.C;
                else
                    a_base[i] = ((((Off)nimg * p.D + a_id0[i]) * p.H + a_ih0[i]) * (Off)p.W + a_iw0[i]) * (Off)p.C;
            } else {
                a_id0[i] = a_ih0[i] = a_iw0[i] = -(1 << 29);
                a_base[i] = 0;
            }
        }
    }
    // ---------------------------------------------------------------- B rows (filter)
    const char *b_row[BIT];
#pragma unroll
    for (int i = 0; i < BIT; ++i) {
        const int n = n0 + RPI * (wave + i * NW) + lr;
        if constexpr (MODE == MODE_POINT)  // image n: Rk elements (columns past Ncol load image Ncol - 1)
            b_row[i] = xb + (int64_t)min(n, p.Ncol - 1) * p.Rk * ESZ;
        else  // filter row n (rows past Ncol load row Ncol - 1, whose results are never stored)
            b_row[i] = wb + (int64_t)min(n, p.Ncol - 1) * p.ldw * ESZ;
    }
    // point mode: valid bytes of the chunk that straddles the end of an image row
    i32x4 tailv[BIT];
    unsigned tail_mask = 0;

    // ---------------------------------------------------------------- k position of the next issue
    // Channel-block order: channel block (TKE channels, one 128-byte line per
    // tap) outer, then the tap. The position starts at step kbeg.
    int kc, c = 0, t = 0, r = 0, s = 0;
    bool kval = true;
    int cbase = 0;
    if constexpr (MODE == MODE_POINT) {
        kc = kbeg * TKE + jc * CH;
    } else if constexpr (!CBLK) {
        kc = kbeg * TKE + jc * CH;
        c = kc % p.C;
        const int tap = kc / p.C;
        s = tap % p.S;
        r = (tap / p.S) % p.R;
        t = tap / (p.S * p.R);
        kval = kc < p.Rk;
    } else {
        const int taps = p.T * p.R * p.S;
        const int tap = kbeg % taps;  // step = channel block * taps + tap
        cbase = kbeg / taps * TKE;
        s = tap % p.S;
        r = (tap / p.S) % p.R;
        t = tap / (p.S * p.R);
        c = cbase + jc * CH;
        kc = ((t * p.R + r) * p.S + s) * p.C + c;
    }
    Off tapoff = 0;
    auto update_tapoff = [&]() {
        if constexpr (MODE == MODE_POINT)
            return;
        else if constexpr (MODE == MODE_TEMPORAL)
            tapoff = (Off)(t * p.dd) * (Off)(p.H * p.W) * (Off)p.C + c;
        else
            tapoff = (((Off)(t * p.dd) * p.H + r * p.dh) * (Off)p.W + s * p.dw) * (Off)p.C + c;
    };
    update_tapoff();
    auto advance = [&]() {
        if constexpr (MODE == MODE_POINT) {
            kc += TKE;
            return;
        } else if constexpr (CBLK) {
            if (++s == p.S) {
                s = 0;
                if (++r == p.R) {
                    r = 0;
                    if (++t == p.T) {
                        t = 0;
                        cbase += TKE;
                    }
                }
            }
            c = cbase + jc * CH;
            kc = ((t * p.R + r) * p.S + s) * p.C + c;
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
        }
        update_tapoff();
    };

    // Issue one reduction step into LDS stage st: A then B, one instruction per 16-row group.
    auto issue = [&](int st) __attribute__((always_inline)) {
        char *stage = smem + st * STAGE;
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            if constexpr (MODE == MODE_POINT) {
                const char *src = a_row[i] + (int64_t)kc * ESZ;
                __builtin_amdgcn_global_load_lds(
                    src, (__attribute__((address_space(3))) void *)(stage + RPI * (wave + i * NW) * KB), 16, 0, 0);
                continue;
            }
            // the tests combined without short circuit, so that the choice is one select and no branch
            // (the generic step went from 273 to 185 instructions on the 128x128 tile: -10 to -23 % on
            // 3x3x3 grids of the 128x128 and 64x64 tiles)
            bool ok;
            if constexpr (MODE == MODE_TEMPORAL) {
                ok = kval & ((unsigned)(a_id0[i] + t * p.dd) < (unsigned)p.D);
            } else {
                ok = kval & ((unsigned)(a_id0[i] + t * p.dd) < (unsigned)p.D) &
                     ((unsigned)(a_ih0[i] + r * p.dh) < (unsigned)p.H) &
                     ((unsigned)(a_iw0[i] + s * p.dw) < (unsigned)p.W);
            }
            const char *src = ok ? xb + (a_base[i] + tapoff) * ESZ : zero;
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(stage + RPI * (wave + i * NW) * KB), 16, 0, 0);
        }
        char *bst = stage + BM * KB;
#pragma unroll
        for (int i = 0; i < BIT; ++i) {
            const char *src = zero;
            if constexpr (MODE == MODE_POINT) {
                if (kc + CH <= p.Rk) {
                    src = b_row[i] + (int64_t)kc * ESZ;
                } else if (kc < p.Rk) {  // straddles the row end: keep its valid words
                    const int nwords = (p.Rk - kc) * ESZ / 4;
                    const int *w4 = reinterpret_cast<const int *>(b_row[i] + (int64_t)kc * ESZ);
                    i32x4 v = {0, 0, 0, 0};
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        if (q < nwords)
                            v[q] = w4[q];
                    tailv[i] = v;
                    tail_mask |= 1u << i;
                }
            } else {
                src = b_row[i] + (int64_t)kc * ESZ;
            }
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(bst + RPI * (wave + i * NW) * KB), 16, 0, 0);
        }
    };

    // Point mode, a step that lies inside every image row: no straddle test and
    // no zero line, so no divergent branch. (The source pointer goes through a
    // named variable: passing the sum straight to the builtin made the host pass
    // drop the kernel's launch stub.)
    auto issue_whole = [&](int st) __attribute__((always_inline)) {
        char *stage = smem + st * STAGE;
#pragma unroll
        for (int i = 0; i < AIT; ++i) {
            const char *src = a_row[i] + (int64_t)kc * ESZ;
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(stage + RPI * (wave + i * NW) * KB), 16, 0, 0);
        }
        char *bst = stage + BM * KB;
#pragma unroll
        for (int i = 0; i < BIT; ++i) {
            const char *src = b_row[i] + (int64_t)kc * ESZ;
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(bst + RPI * (wave + i * NW) * KB), 16, 0, 0);
        }
    };

    // ---------------------------------------------------------------- MFMA
    using AccT = typename AccType<MF>::type;
    AccT acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
            acc[a][b] = AccT{};

    const int lrow = lane & (MF - 1), lgrp = lane / MF, lsw = lane & 7;
    auto compute = [&](const char *st, auto &&hook) {
        const char *aw = st + (wm * WTM + lrow) * KB;
        const char *bw = st + BM * KB + (wn * WTN + lrow) * KB;
        constexpr int GROUPS = 64 / MF;
        constexpr int CPL = DT == DT_BF16 ? 1 : 2;
        constexpr int SUB = CPR / (GROUPS * CPL);
        static_assert(SUB >= 1, "step too short for this MFMA");
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            const int c0 = (h * GROUPS + lgrp) * CPL;
            const int sl0 = (c0 ^ lsw) * 16;
            const int sl1 = ((c0 + 1) ^ lsw) * 16;
            if constexpr (DT == DT_BF16) {
                bf16x8 bf[FN];
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    bf[b] = *reinterpret_cast<const bf16x8 *>(bw + b * MF * KB + sl0);
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const bf16x8 af = *reinterpret_cast<const bf16x8 *>(aw + a * MF * KB + sl0);
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        if constexpr (MF == 16)
                            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[b], acc[a][b], 0, 0, 0);
                        else
                            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[b], acc[a][b], 0, 0, 0);
                    }
                    hook(h * FM + a);
                }
            } else {
                i32x8 bf[FN];
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const i32x4 lo = *reinterpret_cast<const i32x4 *>(bw + b * MF * KB + sl0);
                    const i32x4 hi = *reinterpret_cast<const i32x4 *>(bw + b * MF * KB + sl1);
                    bf[b] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const i32x4 lo = *reinterpret_cast<const i32x4 *>(aw + a * MF * KB + sl0);
                    const i32x4 hi = *reinterpret_cast<const i32x4 *>(aw + a * MF * KB + sl1);
                    const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        if constexpr (MF == 16)
                            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[b], acc[a][b], 0, 0,
                                                                                         0, 0, 0, 0);
                        else
                            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[b], acc[a][b], 0, 0,
                                                                                        0, 0, 0, 0);
                    }
                    hook(h * FM + a);
                }
            }
        }
    };

    // ---------------------------------------------------------------- pipeline
    // Stage ks lives in slot ks % S. Before computing step ks every thread
    // waits until its own loads of step ks have landed (later steps may stay
    // in flight), then the barrier makes all threads' data visible and
    // guarantees that step ks-1's slot is no longer read, so step ks+S-1 can be
    // issued into it.
    const int nk = p.splits > 1 ? min(p.nk - kbeg, p.ksplit) : p.nk;  // steps of this workgroup
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
        if (st < nk) {
            issue(st);
            if (st + 1 < nk)
                advance();
        }
    }
    int ks = 0;
    if constexpr (MODE == MODE_POINT && S == 2) {
        // Point output, two-stage ring: while the next step lies inside every image row
        // ((kbeg + ks + 2) * TKE <= Rk), a lean step with branch-free loads (c2: 121 instead of
        // 325 instructions per step; patch embed -7 %, its backward GEMMs -4 to -9 %).
        const int lean = min(nk - 1, p.Rk / TKE - kbeg - 1);
        for (; ks < lean; ++ks) {
            wait_vmcnt<0>();
            asm volatile("s_barrier" ::: "memory");
            const int st = (ks + 1) & 1;
            compute(smem + (ks & 1) * STAGE, [&](int row) __attribute__((always_inline)) {
                if (row == 0)
                    issue_whole(st);
            });
            if (ks + 2 < nk)
                advance();
        }
    }
    for (; ks < nk; ++ks) {
        const int ahead = nk - 1 - ks;  // steps issued after ks, capped at S-2
        if (ahead >= S - 2) {
            wait_vmcnt<LPS * (S - 2)>();
        } else if constexpr (S > 3) {
            if (ahead == 1)
                wait_vmcnt<LPS>();
            else
                wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        asm volatile("s_barrier" ::: "memory");
        if constexpr (MODE == MODE_POINT) {
            // The straddling chunks belong to the last step (p.nk = ceil(Rk / TKE)); its
            // DMA wrote zeros there, which have landed: overwrite them, then publish.
            if (kbeg + ks == p.nk - 1 && (p.Rk % CH) != 0) {
                char *bst = smem + (ks % S) * STAGE + BM * KB;
#pragma unroll
                for (int i = 0; i < BIT; ++i)
                    if (tail_mask & (1u << i))
                        *reinterpret_cast<i32x4 *>(bst + RPI * (wave + i * NW) * KB + 16 * lane) = tailv[i];
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
        }
        if constexpr (MODE == MODE_POINT) {
            // Point output: the next step's loads go out after this step's first MFMA row rather than in
            // front of it (one A fragment feeds few MFMAs here, and the issue delayed the first of them).
            // Measured on the patch embed (back to back, C = 3 / 6 / 12: -1.5 / -5 / -7 %) and its
            // backward GEMMs (equal); spreading the issue over all rows of the step instead left the last
            // loads too little time with a two-stage ring (backward data +24 %).
            const bool more = ks + S - 1 < nk;
            const int st = (ks + S - 1) % S;
            compute(smem + (ks % S) * STAGE, [&](int row) __attribute__((always_inline)) {
                if (more && row == 0)
                    issue(st);
            });
            if (more && ks + S < nk)
                advance();
        } else {
            if (ks + S - 1 < nk) {
                issue((ks + S - 1) % S);
                if (ks + S < nk)
                    advance();
            }
            compute(smem + (ks % S) * STAGE, [](int) {});
        }
    }

    // ---------------------------------------------------------------- epilogue
    // emit(put4, put1) walks this lane's outputs: put4(off, v, k) for 4
    // consecutive elements from element offset off (4 positions of channel k,
    // or channels k .. k + 3 in point mode), put1 for single ones.
    auto emit = [&](auto &&put4, auto &&put1) __attribute__((always_inline)) {
        constexpr int QUADS = MF / 16 * (MF / 16);
#pragma unroll
        for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int q = 0; q < QUADS; ++q) {
                const int row = m0 + wm * WTM + a * MF + (MF == 16 ? 4 * lgrp : 8 * q + 4 * lgrp);
                if constexpr (MODE == MODE_POINT) {
                    // rows are output channels, columns are images: y[n][k] is contiguous in k
                    const bool vec = (p.K & 3) == 0 && row + 3 < p.M;
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        const int col = n0 + wn * WTN + b * MF + lrow;
                        if (row >= p.M || col >= p.Ncol)
                            continue;
                        const f32x4 v = quad<MF>(acc[a][b], q);
                        const Off dst = (Off)col * p.K + row;
                        if (vec) {
                            put4(dst, v, row);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (row + e < p.M)
                                    put1(dst + e, v[e], row + e);
                        }
                    }
                    continue;
                }
                int nimg = 0, sp = 0;
                if (row < p.M) {
                    nimg = row / p.P;
                    sp = row - nimg * p.P;
                }
                const bool vec = (p.P & 3) == 0 && row + 3 < p.M;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int col = n0 + wn * WTN + b * MF + lrow;
                    if (row >= p.M || col >= p.K)
                        continue;
                    const f32x4 v = quad<MF>(acc[a][b], q);
                    if (vec) {
                        put4(((Off)nimg * p.K + col) * (Off)p.P + sp, v, col);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = row + e;
                            if (m < p.M) {
                                const int n2 = m / p.P;
                                const int sp2 = m - n2 * p.P;
                                put1(((Off)n2 * p.K + col) * (Off)p.P + sp2, v[e], col);
                            }
                        }
                    }
                }
            }
        }
    };
    if (p.splits > 1) {
        // a split workgroup stores its raw fp32 sums at the same element offsets of its slice of
        // the partial buffer (16-byte aligned runs); the reduction pass applies the epilogue
        float *pb = p.part + (int64_t)split * ((int64_t)p.M * p.Ncol);
        emit([&](Off off, const f32x4 &v, int) __attribute__((always_inline)) { *reinterpret_cast<f32x4 *>(pb + off) = v; },
             [&](Off off, float v, int) __attribute__((always_inline)) { pb[off] = v; });
    } else {
        // whole tiles go out through the idle LDS ring in full 128-byte lines
        constexpr int NT = WM * WN * 64;
        constexpr bool LDS_EPI = MF == 16 && S * STAGE >= BN * (2 * BM + 16) && (BN * (BM / 8)) % NT == 0;
        if constexpr (LDS_EPI) {
            const bool whole = MODE == MODE_POINT
                                   ? (p.K & 7) == 0 && m0 + BM <= p.M && n0 + BN <= p.Ncol
                                   : (p.P & 7) == 0 && m0 + BM <= p.M && n0 + BN <= p.K && m0 / p.P == (m0 + BM - 1) / p.P;
            if (whole) {
                store_tile_lds<BM, BN, WM, WN, MF, DT, MODE == MODE_POINT>(acc, p, m0, n0, wm, wn, lane, smem);
                return;
            }
        }
        uint16_t *yb = static_cast<uint16_t *>(p.y);
        with_epilogue(p, DT == DT_FP8, [&](auto &ep) __attribute__((always_inline)) {
            emit(
                [&](Off off, const f32x4 &v, int k) __attribute__((always_inline)) {
                    if constexpr (MODE == MODE_POINT)
                        *reinterpret_cast<u32x2 *>(yb + off) = ep.four_channels(v, k);
                    else
                        *reinterpret_cast<u32x2 *>(yb + off) = ep.four(v, k);
                },
                [&](Off off, float v, int k) __attribute__((always_inline)) { yb[off] = (uint16_t)ep.one(v, k); });
        });
    }
}

#define IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_, BIG_, CBLK_)                                              \
    do {                                                                                                       \
        hipLaunchKernelGGL((conv_igemm_dma_kernel<BM_, BN_, WM_, WN_, MF_, DT, MODE_, BIG_, CBLK_, S_, KB_>),   \
                           grid, dim3(WM_ * WN_ * 64), 0, stream, p);                                          \
        return hipGetLastError();                                                                              \
    } while (0)
#define IGC_DMODES(BM_, BN_, WM_, WN_, MF_, S_)                                                                \
    do {                                                                                                       \
        if (mode == MODE_POINT) {                                                                              \
            if (big) IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_POINT, true, false);                        \
            IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_POINT, false, false);                                \
        }                                                                                                      \
        if (mode == MODE_TEMPORAL) {                                                                           \
            if (big) {                                                                                         \
                if (cblock) IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_TEMPORAL, true, true);               \
                IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_TEMPORAL, true, false);                          \
            }                                                                                                  \
            if (cblock) IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_TEMPORAL, false, true);                  \
            IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_TEMPORAL, false, false);                             \
        }                                                                                                      \
        if (big) {                                                                                             \
            if (cblock) IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_GENERIC, true, true);                    \
            IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_GENERIC, true, false);                               \
        }                                                                                                      \
        if (cblock) IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_GENERIC, false, true);                       \
        IGC_DLAUNCH(BM_, BN_, WM_, WN_, MF_, S_, MODE_GENERIC, false, false);                                  \
    } while (0)
// Launch of one direct-to-LDS tile shape (kTiles[TILE], stages > 0) for one
// dtype, every (mode, 64-bit offsets, channel-block order) variant. Each
// conv_dma_*.hip unit instantiates a few tiles (IGC_DMA_INSTANTIATE) so that
// the units compile in parallel; conv_dma.hip dispatches on the tile index.
template <int DT, int TILE>
hipError_t launch_conv_dma_tile(const ConvParams &p, Mode mode, bool big, bool cblock, hipStream_t stream)
{
    constexpr TileShape T = kTiles[TILE];
    static_assert(T.stages > 0 && T.sb == 0, "direct-to-LDS tiles only");
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n * p.splits));
    constexpr int KB_ = T.kb;
    IGC_DMODES(T.bm, T.bn, T.wm, T.wn, T.mf, T.stages);
    return hipErrorInvalidValue;  // not reached: IGC_DMODES returns on every path
}

#define IGC_DMA_INSTANTIATE(DT_, TILE_)                                                                       \
    template hipError_t launch_conv_dma_tile<DT_, TILE_>(const ConvParams &, Mode, bool, bool, hipStream_t)
#define IGC_DMA_EXTERN(DT_, TILE_)                                                                            \
    extern template hipError_t launch_conv_dma_tile<DT_, TILE_>(const ConvParams &, Mode, bool, bool, hipStream_t)

#undef IGC_DMODES
#undef IGC_DLAUNCH

}  // namespace igc

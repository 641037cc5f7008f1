// Implicit-GEMM forward convolution with an LDS-resident input window.
//
// In the im2col GEMM every input pixel feeds up to T*R*S rows of A (one per
// filter tap), so a kernel that gathers A tiles tap by tap streams each pixel
// from L2 that many times. Here a workgroup owns 256 consecutive output
// positions of one output plane (n, od) and 256 output channels; for each
// 64-byte channel block it copies the input box those positions touch (T
// input planes x win_h rows x win_w columns, zero where the box leaves the
// input) into LDS once, by direct-to-LDS loads, and every tap's A fragments
// are read from that box at a tap-dependent pixel offset. Only the filter
// tile (B) is streamed per step, through a 4-stage direct-to-LDS ring.
//
// Pixel p of the box holds 64 bytes (4 chunks of 16); chunk q sits in slot
// q ^ ((p >> 1) & 3), so 8 consecutive pixels read by 8 lanes hit distinct
// banks. Filter rows use the same 64-byte layout as conv_igemm_dma_kernel.
#pragma once

#include "conv_igemm_dma.h"

namespace igc {

constexpr int kWinBytes = 96 * 1024;  // input box; the filter ring takes 4 x 16 KB of the 160 KB

template <int MF, int DT, bool BIG>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void conv_win_kernel(ConvParams p)
{
    using Off = typename OffType<BIG>::type;
    constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NW = 8, S = 4;
    constexpr int ESZ = DT == DT_FP8 ? 1 : 2;
    constexpr int CH = 16 / ESZ;               // elements per 16-byte chunk
    constexpr int KB = 64;                     // bytes of k per row per step
    constexpr int TKE = KB / ESZ;              // channels per block (one reduction step per tap)
    constexpr int BIT = BN / (16 * NW);        // filter DMA instructions per thread per step
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int BSTAGE = BN * KB;
    static_assert(S * BSTAGE + kWinBytes <= 160 * 1024, "LDS budget");
    static_assert(MF == 32 || DT == DT_BF16, "fp8 needs 128-byte k per 16x16 MFMA: use 32x32 blocks");

    __shared__ __attribute__((aligned(1024))) char win[kWinBytes];
    __shared__ __attribute__((aligned(1024))) char bring[S * BSTAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    int tm, tn;
    tile_coords(p, tm, tn);
    const int plane = tm / p.tpp;  // n * Do + od
    const int jt = tm - plane * p.tpp;
    const int nimg = plane / p.Do, od = plane - nimg * p.Do;
    const int P2 = p.Ho * p.Wo;
    const int q0 = jt * BM;  // first output position of the tile within its plane
    const int qend = min(q0 + BM, P2);
    const int oh_lo = q0 / p.Wo;
    const int n0 = tn * BN;
    const int whw = p.win_h * p.win_w;  // pixels per input plane of the box
    const int ntaps = p.T * p.R * p.S;

    const char *xb = static_cast<const char *>(p.x);
    const char *wb = static_cast<const char *>(p.w);
    const char *zero = reinterpret_cast<const char *>(kZeroLine);

    // ---------------------------------------------------------------- the input box
    auto fill_window = [&](int cb) {
        for (int j = 0; j < p.win_nwi; ++j) {
            const int g = (j * NW + wave) * 64 + lane;  // 16-byte slot this lane fills
            const int pix = g >> 2;
            const int q = (g & 3) ^ ((pix >> 1) & 3);   // chunk stored in that slot
            const char *src = zero;
            if (pix < p.T * whw) {
                const int ts = pix / whw;
                const int rem = pix - ts * whw;
                const int row = rem / p.win_w;
                const int col = rem - row * p.win_w;
                const int id = od * p.sd - p.pd + ts * p.dd;
                const int ih = oh_lo * p.sh - p.ph + row;
                const int iw = col - p.pw;
                if ((unsigned)id < (unsigned)p.D && (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W)
                    src = xb + (((((Off)nimg * p.D + id) * p.H + ih) * (Off)p.W + iw) * (Off)p.C + cb * TKE + q * CH) *
                                   ESZ;
            }
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(win + (j * NW + wave) * 1024), 16, 0, 0);
        }
    };

    // ---------------------------------------------------------------- filter ring
    const int lr = lane >> 2;
    const int jc = (lane & 3) ^ ((lane >> 3) & 3);
    const char *b_row[BIT];
#pragma unroll
    for (int i = 0; i < BIT; ++i) {
        const int n = n0 + 16 * (wave + i * NW) + lr;
        b_row[i] = n < p.Ncol ? wb + (int64_t)n * p.ldw * ESZ : nullptr;
    }
    int tap_i = 0, cb_i = 0;  // reduction step of the next filter issue
    auto issue_b = [&](int st) {
        char *bst = bring + st * BSTAGE;
        const int kc = tap_i * p.C + cb_i * TKE + jc * CH;
#pragma unroll
        for (int i = 0; i < BIT; ++i) {
            const char *src = b_row[i] ? b_row[i] + (int64_t)kc * ESZ : zero;
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(bst + 16 * (wave + i * NW) * KB), 16, 0, 0);
        }
        if (++tap_i == ntaps) {
            tap_i = 0;
            ++cb_i;
        }
    };

    // ---------------------------------------------------------------- A fragment rows
    // Box pixel of each of this lane's A rows at tap (0, 0, 0); rows past the
    // plane's end read pixel 0 (their results are not stored).
    const int lrow = lane & (MF - 1), lgrp = lane / MF, lsw = (lane >> 1) & 3;
    int pbase[FM];
#pragma unroll
    for (int a = 0; a < FM; ++a) {
        int q = q0 + wm * WTM + a * MF + lrow;
        if (q >= qend)
            q = q0;
        const int oh = q / p.Wo;
        const int ow = q - oh * p.Wo;
        pbase[a] = (oh - oh_lo) * p.sh * p.win_w + ow * p.sw;
    }

    using AccT = typename AccType<MF>::type;
    AccT acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
            acc[a][b] = AccT{};

    auto compute = [&](const char *bst, int tpix) {
        const char *bw = bst + (wn * WTN + lrow) * KB;
        constexpr int GROUPS = 64 / MF;
        constexpr int CPL = DT == DT_BF16 ? 1 : 2;
        constexpr int SUB = (KB / 16) / (GROUPS * CPL);
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
                    const int pix = pbase[a] + tpix;
                    const bf16x8 af =
                        *reinterpret_cast<const bf16x8 *>(win + pix * KB + ((c0 ^ ((pix >> 1) & 3)) << 4));
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
                    const i32x4 lo = *reinterpret_cast<const i32x4 *>(bw + b * MF * KB + sl0);
                    const i32x4 hi = *reinterpret_cast<const i32x4 *>(bw + b * MF * KB + sl1);
                    bf[b] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const int pix = pbase[a] + tpix;
                    const int sw = (pix >> 1) & 3;
                    const i32x4 lo = *reinterpret_cast<const i32x4 *>(win + pix * KB + ((c0 ^ sw) << 4));
                    const i32x4 hi = *reinterpret_cast<const i32x4 *>(win + pix * KB + (((c0 + 1) ^ sw) << 4));
                    const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                    for (int b = 0; b < FN; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[b], acc[a][b], 0, 0, 0, 0,
                                                                                    0, 0);
                }
            }
        }
    };

    // ---------------------------------------------------------------- pipeline
    // Step ks = (channel block, tap). The box changes once per channel block:
    // every wave stops reading it (barrier), it is refilled, and all loads in
    // flight are drained before the next barrier. Within a block, filter step
    // ks+3 is issued while step ks is consumed.
    const int nk = p.nk;
    fill_window(0);
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < nk)
            issue_b(st);
    int t = 0, r = 0, s = 0;  // tap of the step being consumed
    for (int ks = 0; ks < nk; ++ks) {
        const bool new_block = ks > 0 && t == 0 && r == 0 && s == 0;
        if (ks == 0) {
            wait_vmcnt<0>();
            asm volatile("s_barrier" ::: "memory");
        } else if (new_block) {
            asm volatile("s_barrier" ::: "memory");  // nobody reads the old box any more
            fill_window(ks / ntaps);
            wait_vmcnt<0>();
            asm volatile("s_barrier" ::: "memory");
        } else {
            const int ahead = nk - 1 - ks;
            if (ahead >= S - 2)
                wait_vmcnt<BIT * (S - 2)>();
            else if (ahead == 1)
                wait_vmcnt<BIT>();
            else
                wait_vmcnt<0>();
            asm volatile("s_barrier" ::: "memory");
        }
        if (ks + S - 1 < nk)
            issue_b((ks + S - 1) % S);
        compute(bring + (ks % S) * BSTAGE, t * whw + r * p.dh * p.win_w + s * p.dw);
        if (++s == p.S) {
            s = 0;
            if (++r == p.R) {
                r = 0;
                if (++t == p.T)
                    t = 0;
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    uint16_t *yb = static_cast<uint16_t *>(p.y);
    constexpr int QUADS = MF / 16 * (MF / 16);
    const Off ybase = ((Off)nimg * p.K) * (Off)p.P + (Off)od * P2;  // + k * P + q
    with_epilogue(p, DT == DT_FP8, [&](auto &ep) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int qd = 0; qd < QUADS; ++qd) {
                const int q = q0 + wm * WTM + a * MF + (MF == 16 ? 4 * lgrp : 8 * qd + 4 * lgrp);
                const bool vec = (P2 & 3) == 0 && q + 3 < qend;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int col = n0 + wn * WTN + b * MF + lrow;
                    if (q >= qend || col >= p.K)
                        continue;
                    const f32x4 v = quad<MF>(acc[a][b], qd);
                    uint16_t *dst = yb + ybase + (Off)col * p.P + q;
                    if (vec) {
                        *reinterpret_cast<u32x2 *>(dst) = ep.four(v, col);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (q + e < qend)
                                dst[e] = (uint16_t)ep.one(v[e], col);
                    }
                }
            }
        }
    });
}

template <int DT>
hipError_t launch_conv_win_dt(const ConvParams &p, int tile, bool big, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(512);
    if constexpr (DT == DT_BF16) {
        if (tile == 16) {
            if (big)
                hipLaunchKernelGGL((conv_win_kernel<16, DT, true>), grid, block, 0, stream, p);
            else
                hipLaunchKernelGGL((conv_win_kernel<16, DT, false>), grid, block, 0, stream, p);
            return hipGetLastError();
        }
    }
    if (tile == 17) {
        if (big)
            hipLaunchKernelGGL((conv_win_kernel<32, DT, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((conv_win_kernel<32, DT, false>), grid, block, 0, stream, p);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace igc

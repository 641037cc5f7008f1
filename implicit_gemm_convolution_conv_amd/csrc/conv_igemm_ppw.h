// Implicit-GEMM forward convolution, generic im2col path: ping-pong wave
// groups with activation rows shared across the S taps of a filter row.
//
// The ping-pong schedule, tile, filter ring and reduction order of
// conv_igemm_pp_kernel, hence bit-identical outputs. What changes is how the
// activations reach LDS. In channel-block order the S steps of one filter
// row (t, r) read, for tile row m, the input pixels iw = ow*sw - pw + s*dw of
// one input row: successive taps s are the same pixels shifted by dw. So
// instead of S im2col tiles of 256 rows, one window is loaded per
// (channel block, t, r): for every output row (n, od, oh) that the tile's 256
// output positions touch, the input pixels iw = -pw .. -pw + Wwin - 1 of input
// row (n, od*sd - pd + t*dd, oh*sh - ph + r*dh), Wwin = (Wo-1)*sw + (S-1)*dw + 1,
// one 128-byte row per pixel and channel block. Tile row m at tap s reads
// window row j(m) * Wwin + ow(m) * sw + s * dw, j(m) = its output row within
// the window. For the 3x3x3 / Wo=45 headline shape a window is 7 x 47 rows
// (41 KB) and serves three steps, in place of 3 x 32 KB.
//
// Rings: two window slots of up to kWinRows rows (44 KB each), two filter
// slots of 32 KB. Group 1 issues window w+1 during the first step of window
// w (its slot held window w-1, last read in Q2 of the step before) and waits
// for it in Q2 of the last step of window w; group 0 issues the filter as in
// conv_igemm_pp_kernel. Window rows whose pixel is padding (or past the last
// output row) are routed past the buffer and read as zeros.
#pragma once

#include "conv_igemm_pp.h"

namespace igc {

constexpr int kWinRows = 352;  // window rows per slot (128 bytes each)

// N window rows of one lane (rows first + i * stride of the window of the
// tile whose first output row is g0): the byte offset of the row's pixel at
// t = r = 0 and chunk `chunk`, and a mask of the filter rows (t, r) at which
// the pixel lies inside the input (16 bits per row, two rows per register).
template <int N, int ESZ>
struct WinRows {
    unsigned off[N];              // wraps for rows above or left of the input
    unsigned valid[(N + 1) / 2];  // row i: bits 16 * (i & 1) + t * R + r

    __device__ __attribute__((always_inline)) void init(const ConvParams &p, int g0, int first, int stride, int chunk, int64_t xbase)
    {
        const int glast = p.N * p.Do * p.Ho - 1;
#pragma unroll
        for (int i = 0; i < (N + 1) / 2; ++i)
            valid[i] = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int wr = first + i * stride;
            const int j = wr / p.win_cols;
            const int col = wr - j * p.win_cols;
            const int g = min(g0 + j, glast);
            const int oh = g % p.Ho;
            const int q = g / p.Ho;
            const int od = q % p.Do;
            const int n = q / p.Do;
            const int id0 = od * p.sd - p.pd, ih0 = oh * p.sh - p.ph, iw = col - p.pw;
            off[i] = (unsigned)(((((int64_t)n * p.D + id0) * p.H + ih0) * (int64_t)p.W + iw) * p.C * ESZ - xbase) +
                     (unsigned)(chunk * 16);
            const bool colok = (unsigned)iw < (unsigned)p.W && wr < p.win_rows && g0 + j <= glast;
            unsigned v = 0;
            for (int t = 0; t < p.T; ++t)
                for (int r = 0; r < p.R; ++r)
                    if (colok && (unsigned)(id0 + t * p.dd) < (unsigned)p.D && (unsigned)(ih0 + r * p.dh) < (unsigned)p.H)
                        v |= 1u << (t * p.R + r);
            valid[i / 2] |= v << (16 * (i & 1));
        }
    }
    __device__ bool ok(int i, unsigned tr) const { return (valid[i / 2] >> (16 * (i & 1) + tr)) & 1u; }
};

// Filter row (t, r) and channel block of one window, uniform.
template <int TKE>
struct WPos {
    int r = 0, t = 0, cb = 0;

    __device__ void advance(const ConvParams &p)
    {
        const bool rw = ++r == p.R;
        r = rw ? 0 : r;
        t += rw;
        const bool tw = t == p.T;
        t = tw ? 0 : t;
        cb += tw ? TKE : 0;
    }
    template <int ESZ>
    __device__ unsigned shift(const ConvParams &p) const
    {
        return (unsigned)((((t * p.dd) * p.H + r * p.dh) * p.W) * p.C + cb) * ESZ;
    }
};

template <int DT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void conv_igemm_ppw_kernel(ConvParams p)
{
    constexpr int BM = 256, BN = 256, MF = 16, KB = 128;
    constexpr int ESZ = DT == DT_FP8 ? 1 : 2;
    constexpr int TKE = KB / ESZ;
    constexpr int RPI = 1024 / KB;               // rows per DMA instruction
    constexpr int IT = BN / (RPI * 4);           // filter DMA instructions per group-0 wave per step
    constexpr int IW = kWinRows / (RPI * 4);     // window DMA instructions per group-1 wave (upper bound)
    constexpr int WTM = 128, WTN = 64;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int WSLOT = kWinRows * KB, BSTAGE = BN * KB;
    constexpr bool SLICES = DT == DT_BF16;
    constexpr int HA = SLICES ? FM : FM / 2;
    static_assert(2 * WSLOT + 2 * BSTAGE <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) char smem[2 * WSLOT + 2 * BSTAGE];
    char *const as = smem;
    char *const bs = smem + 2 * WSLOT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, wl = wave & 3;
    const int wm = wl & 1, wn = (wl >> 1) + 2 * g;

    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int g0 = m0 / p.Wo;  // first output row of the tile

    const int lr = lane >> 3;
    const int jc = (lane & 7) ^ (lane >> 3);

    WinRows<IW, ESZ> wrows;
    FilterRows<IT, ESZ> brows;
    const int64_t xbase = tile_x_base<ESZ>(p, m0);
    if (g)
        wrows.init(p, g0, RPI * wl + lr, RPI * 4, jc, xbase);
    else
        brows.init(p, n0 + RPI * wl + lr, RPI * 4, jc);
    const __amdgpu_buffer_rsrc_t xr = tile_x_rsrc(p, xbase);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(p.w, p.wbytes);
    KPos<TKE> kb;
    WPos<TKE> kw;
    const int nwi = (p.win_rows + RPI * 4 - 1) / (RPI * 4);  // window instructions this wave may need

    // window instruction i (rows RPI * (wl + 4 i) + lr) of the next window into slot st
    auto issue_w = [&](int st, int i, unsigned sh) {
        if (i < nwi && RPI * (wl + 4 * i) < p.win_rows) {
            const unsigned tr = (unsigned)(kw.t * p.R + kw.r);
            const unsigned off = wrows.ok(i, tr) ? wrows.off[i] + sh : kPastEnd;
            buffer_to_lds16(xr, as + st * WSLOT + RPI * (wl + 4 * i) * KB, off);
        }
    };
    auto issue_w_all = [&](int st) {
        const unsigned sh = kw.template shift<ESZ>(p);
#pragma unroll
        for (int i = 0; i < IW; ++i)
            issue_w(st, i, sh);
        kw.advance(p);
    };
    auto issue_b = [&](int st, int i, unsigned sh) {
        buffer_to_lds16(wr, bs + st * BSTAGE + RPI * (wl + 4 * i) * KB, brows.off[i] + sh);
    };
    auto issue_b_step = [&](int st) {
        const unsigned sh = kb.template b_shift<ESZ>(p);
#pragma unroll
        for (int i = 0; i < IT; ++i)
            issue_b(st, i, sh);
        kb.advance(p);
    };

    using AccT = typename AccType<MF>::type;
    using Frag = FragT<DT>;
    AccT acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
            acc[a][b] = AccT{};
    Frag af[HA], bf[FN];

    const int lrow = lane & (MF - 1), lgrp = lane / MF, lsw = lane & 7;
    // window row of this lane's tile row in each A fragment at tap s = 0
    // (below 2^16: two per register)
    unsigned wbase[FM / 2];
#pragma unroll
    for (int a = 0; a < FM; ++a) {
        const int m = min(m0 + wm * WTM + a * MF + lrow, p.M - 1);
        const int gm = m / p.Wo;
        const unsigned row = (unsigned)((gm - g0) * p.win_cols + (m - gm * p.Wo) * p.sw);
        if (a & 1)
            wbase[a / 2] |= row << 16;
        else
            wbase[a / 2] = row;
    }
    auto wrow = [&](int a) -> int { return (int)((wbase[a / 2] >> (16 * (a & 1))) & 0xffffu); };
    // Memory phase: fragments of half q of the step at tap s, window slot ws, filter slot sb.
    auto read_half = [&](int ws, int s, int sb, int q) {
        const char *bw = bs + sb * BSTAGE + (wn * WTN + lrow) * KB;
        if (SLICES || q == 0) {
#pragma unroll
            for (int b = 0; b < FN; ++b)
                bf[b] = lds_frag<DT, MF>(bw + b * MF * KB, SLICES ? q : 0, lgrp, lsw);
        }
        const char *wbuf = as + ws * WSLOT;
        const int sd = s * p.dw;
#pragma unroll
        for (int i = 0; i < HA; ++i) {
            const int row = wrow(SLICES ? i : q * HA + i) + sd;
            af[i] = lds_frag<DT, MF>(wbuf + row * KB, SLICES ? q : 0, lgrp, row & 7);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    auto compute_half = [&](int q, auto &&hook) {
#pragma unroll
        for (int i = 0; i < HA; ++i) {
#pragma unroll
            for (int b = 0; b < FN; ++b)
                mfma_acc<DT, MF>(af[i], bf[b], acc[SLICES ? i : q * HA + i][b]);
            hook(i);
        }
    };
    auto no_issue = [](int) {};
    auto spread = [&](auto &&one, int n) {
        return [&, n](int i) {
#pragma unroll
            for (int j = 0; j < n; ++j)
                if (j * HA / n == i)
                    one(j);
        };
    };

    const int nk = p.nk;
    const int S = p.S;
    const int nwin = nk / S;
    if (!g) {
        issue_b_step(0);
        if (nk > 1)
            issue_b_step(1);
        wait_vmcnt<0>();
        phase_barrier();
        read_half(0, 0, 0, 0);
        phase_barrier();
        int ws = 0, s = 0, sb = 0;  // window slot, tap and filter slot of step ks
        for (int ks = 0; ks < nk; ++ks) {
            const int sb1 = sb ^ 1;
            const int s1 = s + 1 == S ? 0 : s + 1, ws1 = s + 1 == S ? ws ^ 1 : ws;  // step ks+1
            {  // Q0: B(ks+1) into the filter slot of step ks-1
                const bool go = ks >= 1 && ks + 1 < nk;
                const unsigned sh = kb.template b_shift<ESZ>(p);
                compute_half(0, spread(
                                    [&](int j) {
                                        if (go)
                                            issue_b(sb1, j, sh);
                                    },
                                    IT));
                if (go)
                    kb.advance(p);
            }
            phase_barrier();
            read_half(ws, s, sb, 1);  // Q1
            phase_barrier();
            compute_half(1, no_issue);  // Q2
            wait_vmcnt<0>();  // B(ks+1)
            phase_barrier();
            if (ks + 1 < nk)  // Q3
                read_half(ws1, s1, sb1, 0);
            phase_barrier();
            ws = ws1;
            s = s1;
            sb = sb1;
        }
    } else {
        issue_w_all(0);
        if (nwin > 1)
            issue_w_all(1);
        wait_vmcnt<0>();
        phase_barrier();
        phase_barrier();
        int ws = 0, s = 0, sb = 0, w = 0;  // window slot, tap, filter slot, window of step ks
        for (int ks = 0; ks < nk; ++ks) {
            read_half(ws, s, sb, 0);  // Q0
            phase_barrier();
            {  // Q1: on the first step of window w >= 1, window w+1 into the slot of window w-1
                const bool go = s == 0 && w >= 1 && w + 1 < nwin;
                const unsigned sh = kw.template shift<ESZ>(p);
                compute_half(0, spread(
                                    [&](int j) {
                                        if (go)
                                            issue_w(ws ^ 1, j, sh);
                                    },
                                    IW));
                if (go)
                    kw.advance(p);
            }
            phase_barrier();
            read_half(ws, s, sb, 1);  // Q2
            if (s == S - 1)
                wait_vmcnt<0>();  // window w+1 is read from Q3 on
            phase_barrier();
            compute_half(1, no_issue);  // Q3
            phase_barrier();
            sb ^= 1;
            if (++s == S) {
                s = 0;
                ws ^= 1;
                ++w;
            }
        }
    }

    store_tile_ncdhw<MF, FM, FN, DT>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane);
}

template <int DT>
hipError_t launch_conv_ppw(const ConvParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL((conv_igemm_ppw_kernel<DT>), dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace igc

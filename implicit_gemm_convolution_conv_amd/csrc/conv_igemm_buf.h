// Implicit-GEMM forward convolution, im2col paths in channel-block order, with
// buffer-addressed direct-to-LDS loads and one LDS ring per operand.
//
// Same GEMM and LDS layout as conv_igemm_dma_kernel (rows = output positions,
// columns = output channels, reduction over (t, r, s, c) with the channel
// block outermost), with three changes to the load side:
//
//  * Loads go through buffer resources (buffer_load_dwordx4 ... lds). An
//    offset past the end of a buffer reads as zeros without touching memory,
//    so a padding tap only has to select an out-of-range offset: the address
//    of a row is one 32-bit add per step and no zero line or branch is needed.
//    Rows past the end of the GEMM are clamped to the last row; they load real
//    data whose results are never stored.
//  * The filter (B) and the activations (A) have rings of their own (SB and
//    SA stages), so the LDS budget can give the operand whose loads take
//    longer the deeper ring: B is issued SB-1 steps ahead, A SA-1 steps ahead.
//  * The loads of a step can be spread over the MFMA rows of the step before
//    (SPREAD rows), so that their address arithmetic issues in the shadow of
//    the matrix instructions instead of in front of them.
//
// Reduction step ks: wait until this thread's loads of step ks have landed,
// barrier (all loads of step ks visible, step ks-1's slots no longer read),
// then compute step ks while issuing A(ks+SA-1) and B(ks+SB-1) into the slots
// step ks-1 used. The multi-stage async global->LDS pipeline follows FlyDSL
// PR #860 (async DMA commit); the channel-block reduction order and the
// temporal-only mode follow the same PR's 3D-conv kernels.
#pragma once

#include <type_traits>

#include "conv_igemm_dma.h"

namespace igc {

// Offset past the end of every buffer the kernel reads (buffers are < 2^31 bytes).
constexpr unsigned kPastEnd = 0x80000000u;

// Raw buffer resource over [base, base + bytes). Dword 3 = 0x00020000: 32-bit
// data format, no swizzle, offsets checked against `bytes`.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Byte offset in x of the first input plane that any row of the tile starting
// at output row m0 can read: plane od*sd - pd of the row's image, clamped to
// [0, D-1]. Every valid tap of rows m0.. lies at or above it (later rows have
// later planes or later images); the plan checks that they lie below it + 2^31.
template <int ESZ>
__device__ inline int64_t tile_x_base(const ConvParams &p, int m0)
{
    const int nimg = p.div_P.div(m0);
    const int od = p.div_HW.div(m0 - nimg * p.P);
    const int id = min(max(0, od * p.sd - p.pd), p.D - 1);
    return ((int64_t)nimg * p.D + id) * ((int64_t)p.H * p.W) * p.C * ESZ;
}

// Buffer over x seen from the tile's base: at most 2^31 - 16 bytes, so the
// out-of-range offset kPastEnd is always past it.
__device__ inline __amdgpu_buffer_rsrc_t tile_x_rsrc(const ConvParams &p, int64_t xbase)
{
    const int64_t left = p.xbytes - xbase;
    return buffer_rsrc(static_cast<const char *>(p.x) + xbase, (int)(left < 0x7ffffff0 ? left : 0x7ffffff0));
}

// 16 bytes per lane from buffer offset `off` into LDS at lds + 16 * lane.
__device__ inline void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, char *lds, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

// Reduction position in channel-block order: channel block cb (TKE channels,
// one 128-byte line per row) outer, then tap (t, r, s). Every field is
// uniform across the workgroup.
template <int TKE>
struct KPos {
    int s = 0, r = 0, t = 0, cb = 0;
    int tap = 0;  // (t * R + r) * S + s

    __device__ void advance(const ConvParams &p)
    {
        ++tap;
        ++s;
        const bool sw = s == p.S;
        s = sw ? 0 : s;
        r += sw;
        const bool rw = r == p.R;
        r = rw ? 0 : r;
        t += rw;
        const bool tw = t == p.T;
        t = tw ? 0 : t;
        tap = tw ? 0 : tap;
        cb += tw ? TKE : 0;
    }
    // Position of reduction step `step` (advance() applied `step` times from zero).
    __device__ void seek(const ConvParams &p, int step)
    {
        const int taps = p.T * p.R * p.S;
        const int cbi = step / taps;
        tap = step - cbi * taps;
        s = tap % p.S;
        r = (tap / p.S) % p.R;
        t = tap / (p.S * p.R);
        cb = cbi * TKE;
    }
    // Bytes from an input row's origin to this tap and channel block.
    template <int MODE, int ESZ>
    __device__ unsigned a_shift(const ConvParams &p) const
    {
        const int c = cb;
        if constexpr (MODE == MODE_TEMPORAL)
            return (unsigned)((t * p.dd) * (p.H * p.W) * p.C + c) * ESZ;
        else
            return (unsigned)((((t * p.dd) * p.H + r * p.dh) * p.W + s * p.dw) * p.C + c) * ESZ;
    }
    // Bytes from a packed filter row's start to this reduction step.
    template <int ESZ>
    __device__ unsigned b_shift(const ConvParams &p) const
    {
        return (unsigned)((((t * p.R + r) * p.S + s) * p.C + cb) * ESZ);
    }
};

// N im2col rows of one lane (rows first + i * stride, clamped to M - 1): the
// input origin (d, h, w) of each and its byte offset from xbase at channel
// chunk `chunk`.
template <int N, int MODE, int ESZ>
struct ImRows {
    int d[N], h[N], w[N];
    unsigned off[N];  // wraps for padded origins; valid taps land in range

    __device__ __attribute__((always_inline)) void init(const ConvParams &p, int first, int stride, int chunk, int64_t xbase)
    {
        const int hw = p.Ho * p.Wo;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int m = min(first + i * stride, p.M - 1);
            const int nimg = p.div_P.div(m);
            const int sp = m - nimg * p.P;
            const int od = p.div_HW.div(sp);
            const int rem = sp - od * hw;
            const int oh = p.div_Wo.div(rem);
            const int ow = rem - oh * p.Wo;
            d[i] = od * p.sd - p.pd;
            h[i] = oh * p.sh - p.ph;
            w[i] = ow * p.sw - p.pw;
            int64_t pos;
            if constexpr (MODE == MODE_TEMPORAL)
                pos = ((int64_t)nimg * p.D + d[i]) * ((int64_t)p.H * p.W) + rem;
            else
                pos = (((int64_t)nimg * p.D + d[i]) * p.H + h[i]) * (int64_t)p.W + w[i];
            off[i] = (unsigned)(pos * p.C * ESZ - xbase) + (unsigned)(chunk * 16);
        }
    }
    // Buffer offset of row i at reduction position k (shift = k.a_shift): past
    // the end of the buffer when the tap falls outside the input box.
    template <int TKE>
    __device__ unsigned at(const ConvParams &p, int i, const KPos<TKE> &k, unsigned shift) const
    {
        bool ok = (unsigned)(d[i] + k.t * p.dd) < (unsigned)p.D;
        if constexpr (MODE == MODE_GENERIC)
            ok = ok & ((unsigned)(h[i] + k.r * p.dh) < (unsigned)p.H) & ((unsigned)(w[i] + k.s * p.dw) < (unsigned)p.W);
        return ok ? off[i] + shift : kPastEnd;
    }
};

// As ImRows, for filters of at most 32 taps: each row keeps a bit mask of
// the taps that fall inside the input box instead of its origin (two
// registers per row instead of four).
template <int N, int MODE, int ESZ>
struct ImRowsMasked {
    unsigned off[N];
    unsigned valid[N];  // bit (t * R + r) * S + s: that tap reads inside the input box

    __device__ __attribute__((always_inline)) void init(const ConvParams &p, int first, int stride, int chunk, int64_t xbase)
    {
        ImRows<N, MODE, ESZ> rows;
        rows.init(p, first, stride, chunk, xbase);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            off[i] = rows.off[i];
            unsigned md = 0, mh = 0, mw = 0;  // per-axis validity
            for (int t = 0; t < p.T; ++t)
                md |= (unsigned)((unsigned)(rows.d[i] + t * p.dd) < (unsigned)p.D) << t;
            for (int r = 0; r < p.R; ++r)
                mh |= (unsigned)(MODE == MODE_TEMPORAL || (unsigned)(rows.h[i] + r * p.dh) < (unsigned)p.H) << r;
            for (int s = 0; s < p.S; ++s)
                mw |= (unsigned)(MODE == MODE_TEMPORAL || (unsigned)(rows.w[i] + s * p.dw) < (unsigned)p.W) << s;
            unsigned v = 0;
            for (int t = 0; t < p.T; ++t)
                for (int r = 0; r < p.R; ++r)
                    if (((md >> t) & (mh >> r)) & 1u)
                        v |= mw << ((t * p.R + r) * p.S);
            valid[i] = v;
        }
    }
    template <int TKE>
    __device__ unsigned at(const ConvParams &, int i, const KPos<TKE> &k, unsigned shift) const
    {
        return ((valid[i] >> k.tap) & 1u) ? off[i] + shift : kPastEnd;
    }
};

// N packed-filter rows of one lane (rows first + i * stride, clamped to Ncol - 1).
template <int N, int ESZ>
struct FilterRows {
    unsigned off[N];

    __device__ __attribute__((always_inline)) void init(const ConvParams &p, int first, int stride, int chunk)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int n = min(first + i * stride, p.Ncol - 1);
            off[i] = (unsigned)n * (unsigned)(p.ldw * ESZ) + (unsigned)(chunk * 16);
        }
    }
};

// Slot-of-chunk swizzle of a 128-byte LDS row r (chunk q sits at slot
// q ^ lds_swizzle(r)): r & 7 keeps the 16 rows that a bf16 fragment read
// touches (one 16-byte chunk per lane) free of bank conflicts, as the LDS
// counters show (0.15 % of the active cycles on the 3x3x3 workload). fp8
// fragments read two adjacent chunks per lane; for them the row's bit 3 also
// flips the slot, which measured 3.5 % faster on the 3x1x1 fp8 workload
// (2.05 -> 1.98 ms) and would cost bf16 4-5 %.
template <int DT>
__device__ __attribute__((always_inline)) inline int lds_swizzle(int r)
{
    return DT == DT_FP8 ? ((r & 7) ^ ((r >> 3) & 1)) : (r & 7);
}

// MFMA operand fragment of one lane: 8 bf16 or 32 fp8 values along k.
template <int DT>
using FragT = typename std::conditional<DT == DT_BF16, bf16x8, i32x8>::type;

// The fragment of k-slice h of the LDS row at rowp (KB-byte rows, chunk q at
// slot q ^ lsw): lane group lgrp holds chunk(s) (h * GROUPS + lgrp) * CPL.
template <int DT, int MF>
__device__ inline FragT<DT> lds_frag(const char *rowp, int h, int lgrp, int lsw)
{
    constexpr int GROUPS = 64 / MF, CPL = DT == DT_BF16 ? 1 : 2;
    const int c0 = (h * GROUPS + lgrp) * CPL;
    if constexpr (DT == DT_BF16) {
        return *reinterpret_cast<const bf16x8 *>(rowp + ((c0 ^ lsw) * 16));
    } else {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(rowp + ((c0 ^ lsw) * 16));
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(rowp + (((c0 + 1) ^ lsw) * 16));
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

template <int DT, int MF>
__device__ inline void mfma_acc(const FragT<DT> &af, const FragT<DT> &bf, typename AccType<MF>::type &c)
{
    if constexpr (DT == DT_BF16) {
        if constexpr (MF == 16)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, c, 0, 0, 0);
    } else {
        if constexpr (MF == 16)
            c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf, c, 0, 0, 0, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, c, 0, 0, 0, 0, 0, 0);
    }
}

// Epilogue: one wave's FM x FN MFMA blocks of the tile at (row0, col0) to bf16
// NCDHW y through Epilogue (scale s_x * s_w for fp8, bias, amax). Four
// consecutive rows of one column go out as one 8-byte store when they share
// an image and P % 4 == 0.
template <int MF, int FM, int FN, int DT>
__device__ __attribute__((always_inline)) inline void store_tile_ncdhw(const typename AccType<MF>::type (&acc)[FM][FN], const ConvParams &p,
                                        int row0, int col0, int lane)
{
    const int lrow = lane & (MF - 1), lgrp = lane / MF;
    uint16_t *yb = static_cast<uint16_t *>(p.y);
    with_epilogue(p, DT == DT_FP8, [&](auto &ep) __attribute__((always_inline)) {
        constexpr int QUADS = MF / 16 * (MF / 16);
#pragma unroll
        for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int q = 0; q < QUADS; ++q) {
                const int row = row0 + a * MF + (MF == 16 ? 4 * lgrp : 8 * q + 4 * lgrp);
                int nimg = 0, sp = 0;
                if (row < p.M) {
                    nimg = row / p.P;
                    sp = row - nimg * p.P;
                }
                const bool vec = (p.P & 3) == 0 && row + 3 < p.M;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int col = col0 + b * MF + lrow;
                    if (row >= p.M || col >= p.K)
                        continue;
                    const f32x4 v = quad<MF>(acc[a][b], q);
                    if (vec) {
                        *reinterpret_cast<u32x2 *>(yb + ((int64_t)nimg * p.K + col) * p.P + sp) = ep.four(v, col);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = row + e;
                            if (m < p.M) {
                                const int n2 = m / p.P;
                                const int sp2 = m - n2 * p.P;
                                yb[((int64_t)n2 * p.K + col) * p.P + sp2] = (uint16_t)ep.one(v[e], col);
                            }
                        }
                    }
                }
            }
        }
    });
}

template <int BM, int BN, int WM, int WN, int MF, int DT, int MODE, int SA, int SB, int KB, int SPREAD, int PF = 1,
          bool BPF = false>
__global__ __launch_bounds__(WM *WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void conv_igemm_buf_kernel(ConvParams p)
{
    constexpr int NW = WM * WN;                // waves
    constexpr int ESZ = DT == DT_FP8 ? 1 : 2;  // bytes per element
    constexpr int TKE = KB / ESZ;              // elements per reduction step
    constexpr int RPI = 1024 / KB;             // rows filled by one DMA instruction (64 lanes x 16 B)
    constexpr int CPR = KB / 16;               // 16-byte chunks per row
    constexpr int AIT = BM / (RPI * NW);       // A row groups per wave
    constexpr int BIT = BN / (RPI * NW);
    constexpr int LPS = AIT + BIT;             // DMA instructions per thread per step
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int ASTAGE = BM * KB, BSTAGE = BN * KB;
    constexpr int GROUPS = 64 / MF;            // lane groups along k in one MFMA operand
    constexpr int CPL = DT == DT_BF16 ? 1 : 2; // 16-byte chunks per lane per MFMA operand
    constexpr int SUB = CPR / (GROUPS * CPL);  // MFMA k-slices per step
    constexpr int ROWS = SUB * FM;             // MFMA rows (FN instructions each) per step
    static_assert(MODE == MODE_GENERIC || MODE == MODE_TEMPORAL, "im2col modes only");
    static_assert(KB == 128, "128-byte steps");
    static_assert(AIT >= 1 && BIT >= 1 && BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "loader split");
    static_assert(SUB >= 1, "step too short for this MFMA");
    static_assert(SA >= 2 && SB >= 2, "ring depths");
    static_assert(SA * ASTAGE + SB * BSTAGE <= 160 * 1024, "LDS budget");
    static_assert(SPREAD >= 0 && SPREAD <= ROWS, "spread within one step");
    static_assert(PF >= 1 && PF <= 3, "A fragment prefetch distance");

    __shared__ __attribute__((aligned(1024))) char smem[SA * ASTAGE + SB * BSTAGE];
    char *const as = smem;
    char *const bs = smem + SA * ASTAGE;

    preload_setup_params(p);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;

    // Tail split: the workgroups from p.tail_first on share the last, partial
    // round's tiles, p.tail_splits per tile, each over a contiguous range of
    // reduction steps; they leave fp32 partial sums for tail_reduce.
    int bid = (int)blockIdx.x, split = -1, kbeg = 0, nk = p.nk;
    if (p.tail_splits > 1 && bid >= p.tail_first) {
        const int t = bid - p.tail_first;
        const int tile = t / p.tail_splits;
        split = t - tile * p.tail_splits;
        bid = p.tail_first + tile;
        kbeg = (int)((int64_t)split * p.nk / p.tail_splits);
        nk = (int)((int64_t)(split + 1) * p.nk / p.tail_splits) - kbeg;
    }
    int tm, tn;
    tile_coords(p, bid, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // This lane's row within each RPI-row group and the chunk it fetches there:
    // row r keeps chunk q at slot q ^ lds_swizzle<DT>(r); a DMA instruction
    // fills rows 8 * (wave + j * NW) + lr, so r & 7 = lr and (r >> 3) & 1 = wave & 1.
    const int lr = lane / CPR;
    const int jc = (lane & 7) ^ lds_swizzle<DT>(lr | ((wave & 1) << 3));

    const int64_t xbase = tile_x_base<ESZ>(p, m0);
    const __amdgpu_buffer_rsrc_t xr = tile_x_rsrc(p, xbase);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(p.w, p.wbytes);

    ImRows<AIT, MODE, ESZ> arows;
    arows.init(p, m0 + RPI * wave + lr, RPI * NW, jc, xbase);
    FilterRows<BIT, ESZ> brows;
    brows.init(p, n0 + RPI * wave + lr, RPI * NW, jc);

    // One DMA instruction: A row group i (or B row group i - AIT) of the step at k into ring slot st.
    auto issue = [&](int j, int st, const KPos<TKE> &k, unsigned ash, unsigned bsh) {
        if (j < AIT)
            buffer_to_lds16(xr, as + st * ASTAGE + RPI * (wave + j * NW) * KB, arows.at(p, j, k, ash));
        else
            buffer_to_lds16(wr, bs + st * BSTAGE + RPI * (wave + (j - AIT) * NW) * KB, brows.off[j - AIT] + bsh);
    };

    // ---------------------------------------------------------------- MFMA
    using AccT = typename AccType<MF>::type;
    using Frag = FragT<DT>;
    AccT acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
            acc[a][b] = AccT{};

    const int lrow = lane & (MF - 1), lgrp = lane / MF, lsw = lds_swizzle<DT>(lrow);
    auto frag = [&](const char *rowp, int h) -> Frag { return lds_frag<DT, MF>(rowp, h, lgrp, lsw); };
    // One step from slots (sa, sb); hook(row) runs after MFMA row `row` (0..ROWS-1).
    // A fragments are read PF rows ahead of their MFMAs; with BPF the B
    // fragments of the next k-slice are read while the last rows of this one run.
    auto compute = [&](int sa, int sb, auto &&hook) {
        const char *aw = as + sa * ASTAGE + (wm * WTM + lrow) * KB;
        const char *bw = bs + sb * BSTAGE + (wn * WTN + lrow) * KB;
        Frag bf[2][FN];
#pragma unroll
        for (int b = 0; b < FN; ++b)
            bf[0][b] = frag(bw + b * MF * KB, 0);
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            const int cb = BPF ? (h & 1) : 0;
            if (!BPF && h > 0) {
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    bf[0][b] = frag(bw + b * MF * KB, h);
            }
            Frag af[PF + 1];
#pragma unroll
            for (int q = 0; q < PF; ++q)
                if (q < FM)
                    af[q] = frag(aw + q * MF * KB, h);
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                if (a + PF < FM)
                    af[(a + PF) % (PF + 1)] = frag(aw + (a + PF) * MF * KB, h);
                if (BPF && h + 1 < SUB && a == (FM > 2 ? FM - 2 : 0)) {
#pragma unroll
                    for (int b = 0; b < FN; ++b)
                        bf[cb ^ 1][b] = frag(bw + b * MF * KB, h + 1);
                }
#pragma unroll
                for (int b = 0; b < FN; ++b)
                    mfma_acc<DT, MF>(af[a % (PF + 1)], bf[cb][b], acc[a][b]);
                hook(h * FM + a);
            }
        }
    };

    // ---------------------------------------------------------------- pipeline
    // The operand with the deeper ring (the lead) is issued further ahead; in
    // each step the other one (the trail) is issued first, so that waiting for
    // the trail's loads of a step never waits for loads issued after them.
    constexpr bool A_FIRST = SA <= SB;
    constexpr int SMIN = SA < SB ? SA : SB, SMAX = SA < SB ? SB : SA;
    constexpr int FIRST_IT = A_FIRST ? AIT : BIT;
    // Loads issued after this thread's last load of step ks, in steady state:
    // the lead's loads of the step that issued the trail's part of ks (when the
    // rings differ), plus SMIN-2 whole steps.
    constexpr int AHEAD = (SA == SB ? 0 : LPS - FIRST_IT) + (SMIN - 2) * LPS;
    static_assert(AHEAD < 64, "vmcnt range");
    KPos<TKE> ka, kb;  // next A and B steps to issue
    if (kbeg > 0) {
        ka.seek(p, kbeg);
        kb.seek(p, kbeg);
    }
    // j-th DMA instruction of a step in issue order (A rows then B rows, or B then A).
    auto issue_j = [&](int j, int sta, int stb, unsigned ash, unsigned bsh) {
        const bool is_a = A_FIRST ? j < AIT : j >= BIT;
        const int row = A_FIRST ? (is_a ? j : j - AIT) : (is_a ? j - BIT : j);
        if (is_a)
            issue(row, sta, ka, ash, 0);
        else
            issue(AIT + row, stb, kb, 0, bsh);
    };
    auto issue_a_step = [&](int st) {
        const unsigned sh = ka.template a_shift<MODE, ESZ>(p);
#pragma unroll
        for (int j = 0; j < AIT; ++j)
            issue(j, st, ka, sh, 0);
        ka.advance(p);
    };
    auto issue_b_step = [&](int st) {
        const unsigned sh = kb.template b_shift<ESZ>(p);
#pragma unroll
        for (int j = AIT; j < LPS; ++j)
            issue(j, st, kb, 0, sh);
        kb.advance(p);
    };
    // issue the step's parts that exist (A(ks+SA-1) if < nk, B(ks+SB-1) if < nk) in ring order
    auto issue_parts = [&](int ja, int jb, int sta, int stb) {
        if (A_FIRST) {
            if (ja >= 0 && ja < nk)
                issue_a_step(sta);
            if (jb >= 0 && jb < nk)
                issue_b_step(stb);
        } else {
            if (jb >= 0 && jb < nk)
                issue_b_step(stb);
            if (ja >= 0 && ja < nk)
                issue_a_step(sta);
        }
    };
    // Prologue: the issues of the virtual steps -(SMAX-1) .. -1, in steady-state order.
#pragma unroll
    for (int j = -(SMAX - 1); j < 0; ++j) {
        const int ja = j + SA - 1, jb = j + SB - 1;
        issue_parts(ja, jb, ja >= 0 ? ja % SA : 0, jb >= 0 ? jb % SB : 0);
    }
    int ks = 0;
    int sa = 0, sb = 0;                  // slots of step ks
    int ia = SA - 1, ib = SB - 1;        // slots the step's issues go to
    // Steady state: every step issues both parts.
    for (; ks < nk - SMAX + 1; ++ks) {
        wait_vmcnt<AHEAD>();
        asm volatile("s_barrier" ::: "memory");
        const unsigned ash = ka.template a_shift<MODE, ESZ>(p), bsh = kb.template b_shift<ESZ>(p);
        const int sta = ia, stb = ib;
        if constexpr (SPREAD == 0) {
#pragma unroll
            for (int j = 0; j < LPS; ++j)
                issue_j(j, sta, stb, ash, bsh);
            compute(sa, sb, [](int) {});
        } else {
            compute(sa, sb, [&](int row) {
#pragma unroll
                for (int j = 0; j < LPS; ++j)
                    if (j * SPREAD / LPS == row)
                        issue_j(j, sta, stb, ash, bsh);
            });
        }
        ka.advance(p);
        kb.advance(p);
        sa = sa + 1 == SA ? 0 : sa + 1;
        sb = sb + 1 == SB ? 0 : sb + 1;
        ia = ia + 1 == SA ? 0 : ia + 1;
        ib = ib + 1 == SB ? 0 : ib + 1;
    }
    // Drain: the last SMAX-1 steps (or all of a short reduction) wait for everything.
    for (; ks < nk; ++ks) {
        wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
        issue_parts(ks + SA - 1, ks + SB - 1, ia, ib);
        compute(sa, sb, [](int) {});
        sa = sa + 1 == SA ? 0 : sa + 1;
        sb = sb + 1 == SB ? 0 : sb + 1;
        ia = ia + 1 == SA ? 0 : ia + 1;
        ib = ib + 1 == SB ? 0 : ib + 1;
    }

    if (split >= 0) {  // tail split: unscaled fp32 sums, [column][row] per tile and split
        float *dst = p.part + ((int64_t)(bid - p.tail_first) * p.tail_splits + split) * (BM * BN);
        const int lrow2 = lane & (MF - 1), lgrp2 = lane / MF;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
#pragma unroll
                for (int q = 0; q < MF / 16 * (MF / 16); ++q) {
                    const int col = wn * WTN + b * MF + lrow2;
                    const int row = wm * WTM + a * MF + (MF == 16 ? 4 * lgrp2 : 8 * q + 4 * lgrp2);
                    *reinterpret_cast<f32x4 *>(dst + col * BM + row) = quad<MF>(acc[a][b], q);
                }
        return;
    }
    // whole tile inside one image, 16-byte aligned rows: stage the outputs through the idle rings
    constexpr bool LDS_EPI = MF == 16 && SA * ASTAGE + SB * BSTAGE >= BN * (2 * BM + 16);
    if constexpr (LDS_EPI) {
        if ((p.P & 7) == 0 && m0 + BM <= p.M && n0 + BN <= p.K && m0 / p.P == (m0 + BM - 1) / p.P) {
            store_tile_lds<BM, BN, WM, WN, MF, DT, false>(acc, p, m0, n0, wm, wn, lane, smem);
            return;
        }
    }
    store_tile_ncdhw<MF, FM, FN, DT>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane);
}

// Launch helper for one dtype: the buffer-addressed tiles of kTiles (sb > 0).
template <int DT>
hipError_t launch_conv_buf_dt(const ConvParams &p, int tile, Mode mode, hipStream_t stream)
{
    const int ntiles = p.tiles_m * p.tiles_n;  // tail split: the tail tiles take tail_splits workgroups each
    const dim3 grid((unsigned)(p.tail_splits > 1 ? p.tail_first + (ntiles - p.tail_first) * p.tail_splits : ntiles));
#define IGC_BLAUNCH(BM_, BN_, WM_, WN_, MF_, SA_, SB_, KB_, SP_, ...)                                          \
    do {                                                                                                   \
        if (mode == MODE_TEMPORAL)                                                                         \
            hipLaunchKernelGGL((conv_igemm_buf_kernel<BM_, BN_, WM_, WN_, MF_, DT, MODE_TEMPORAL, SA_, SB_, KB_, \
                                                      SP_, ##__VA_ARGS__>),                                  \
                               grid, dim3(WM_ * WN_ * 64), 0, stream, p);                                  \
        else                                                                                               \
            hipLaunchKernelGGL((conv_igemm_buf_kernel<BM_, BN_, WM_, WN_, MF_, DT, MODE_GENERIC, SA_, SB_, KB_,  \
                                                      SP_, ##__VA_ARGS__>),                                  \
                               grid, dim3(WM_ * WN_ * 64), 0, stream, p);                                  \
        return hipGetLastError();                                                                          \
    } while (0)
    switch (tile) {
    case TILE_BUF: IGC_BLAUNCH(256, 256, 2, 4, 16, 3, 2, 128, 8);
    case TILE_BUF_AHEAD: IGC_BLAUNCH(256, 256, 2, 4, 16, 3, 2, 128, 8, 2, true);
    case TILE_BUF_128:  // loads over the step's 8 (bf16) or 4 (fp8) MFMA rows
        if constexpr (DT == DT_FP8)
            IGC_BLAUNCH(128, 128, 2, 2, 16, 3, 2, 128, 4);
        else
            IGC_BLAUNCH(128, 128, 2, 2, 16, 3, 2, 128, 8);
    default: break;
    }
    return hipErrorInvalidValue;
#undef IGC_BLAUNCH
}

}  // namespace igc

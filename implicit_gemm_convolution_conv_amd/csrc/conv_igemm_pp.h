// Implicit-GEMM forward convolution, im2col paths: ping-pong wave groups.
//
// Same tile (256x256, 8 waves of 128x64), LDS rings (activations 3 x 32 KB,
// filter 2 x 32 KB, 128-byte steps), buffer addressing and reduction order as
// conv_igemm_buf_kernel, so the outputs are bit-identical; what changes is
// the schedule. The waves form two groups of four (waves 0-3 and 4-7), one
// wave of each group on every SIMD. A step's MFMA work is cut in two halves
// (bf16: its two 32-element k-slices; fp8: the two halves of the row
// blocks). Each group alternates between a compute phase (one half's MFMAs
// with every operand already in registers, no memory instruction) and a
// memory phase (the LDS fragment reads of its next half, plus DMA issue).
// The groups are one phase apart and a workgroup barrier separates phases,
// so on every SIMD one wave runs MFMAs while the other reads LDS: the matrix
// unit stays fed across barriers and load latency.
//
// Group 0 (tile columns 0-127) issues the filter DMA, group 1 (columns
// 128-255) the activation DMA, each from inside a compute phase, one DMA
// instruction after each row of MFMAs. Phases of step ks:
//   Q0: g0 computes half 0 of ks,         g1 reads half 0 of ks
//       issues B(ks+1)
//   Q1: g0 reads half 1 of ks             g1 computes half 0 of ks, issues A(ks+2)
//   Q2: g0 computes half 1 of ks,         g1 reads half 1 of ks,
//       waits for its B(ks+1)                 waits for its A(ks+1)
//   Q3: g0 reads half 0 of ks+1           g1 computes half 1 of ks
// Step ks's slots are read from Q3 of ks-1 to Q2 of ks. A(ks+2) goes to the
// activation slot of step ks-1 (last read in Q2 of ks-1), B(ks+1) to the
// filter slot of step ks-1 (last read in Q2 of ks-1). The waits before the
// Q2 barrier make step ks+1 visible to the reads from Q3 on. The alternating
// compute / memory wave groups follow the ping-pong schedules used for
// MI355X GEMMs; the rings and the reduction order follow FlyDSL PR #860
// (async DMA commit, 3D-conv kernels).
#pragma once

#include "conv_igemm_buf.h"

namespace igc {

// Phase boundary: a workgroup barrier that no instruction is scheduled across.
__device__ inline void phase_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int DT, int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void conv_igemm_pp_kernel(ConvParams p)
{
    constexpr int BM = 256, BN = 256, MF = 16, KB = 128, SA = 3, SB = 2;
    constexpr int ESZ = DT == DT_FP8 ? 1 : 2;
    constexpr int TKE = KB / ESZ;
    constexpr int RPI = 1024 / KB;             // rows per DMA instruction
    constexpr int IT = BM / (RPI * 4);         // DMA instructions per issuing wave per step
    constexpr int WTM = 128, WTN = 64;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int ASTAGE = BM * KB, BSTAGE = BN * KB;
    constexpr bool SLICES = DT == DT_BF16;     // halves are k-slices (bf16) or row-block halves (fp8)
    constexpr int HA = SLICES ? FM : FM / 2;   // A fragments per half
    static_assert(MODE == MODE_GENERIC || MODE == MODE_TEMPORAL, "im2col modes only");
    static_assert(SA * ASTAGE + SB * BSTAGE <= 160 * 1024, "LDS budget");
    static_assert(SA * ASTAGE + SB * BSTAGE >= BN * (2 * BM + 16), "room for the LDS-staged epilogue");

    __shared__ __attribute__((aligned(1024))) char smem[SA * ASTAGE + SB * BSTAGE];
    char *const as = smem;
    char *const bs = smem + SA * ASTAGE;

    preload_setup_params(p);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2, wl = wave & 3;
    const int wm = wl & 1, wn = (wl >> 1) + 2 * g;  // 128-row half, 64-column quarter of the tile

    // Tail split (as in conv_igemm_buf_kernel): workgroups from p.tail_first on
    // run a contiguous step range of a tail tile and leave fp32 partial sums.
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

    // rows 8 * (wl + 4 i) + lr: r & 7 = lr, (r >> 3) & 1 = wl & 1 (lds_swizzle)
    const int lr = lane >> 3;
    const int jc = (lane & 7) ^ lds_swizzle<DT>(lr | ((wl & 1) << 3));

    // group 1 loads activation rows, group 0 filter rows: RPI * (wl + 4 i) + lr
    ImRowsMasked<IT, MODE, ESZ> arows;  // the plan keeps T * R * S <= 32 on this kernel
    FilterRows<IT, ESZ> brows;
    const int64_t xbase = tile_x_base<ESZ>(p, m0);
    if (g)
        arows.init(p, m0 + RPI * wl + lr, RPI * 4, jc, xbase);
    else
        brows.init(p, n0 + RPI * wl + lr, RPI * 4, jc);
    const __amdgpu_buffer_rsrc_t xr = tile_x_rsrc(p, xbase);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(p.w, p.wbytes);
    KPos<TKE> ka, kb;  // next activation / filter step to issue
    if (kbeg > 0) {
        ka.seek(p, kbeg);
        kb.seek(p, kbeg);
    }

    // DMA instruction i of an activation / filter step into ring slot st.
    auto issue_a = [&](int st, int i, unsigned sh) {
        buffer_to_lds16(xr, as + st * ASTAGE + RPI * (wl + 4 * i) * KB, arows.at(p, i, ka, sh));
    };
    auto issue_b = [&](int st, int i, unsigned sh) {
        buffer_to_lds16(wr, bs + st * BSTAGE + RPI * (wl + 4 * i) * KB, brows.off[i] + sh);
    };
    auto issue_a_step = [&](int st) {
        const unsigned sh = ka.template a_shift<MODE, ESZ>(p);
#pragma unroll
        for (int i = 0; i < IT; ++i)
            issue_a(st, i, sh);
        ka.advance(p);
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

    const int lrow = lane & (MF - 1), lgrp = lane / MF, lsw = lds_swizzle<DT>(lrow);
    // Memory phase: fragments of half q of the step in slots (sa, sb).
    auto read_half = [&](int sa, int sb, int q) {
        const char *aw = as + sa * ASTAGE + (wm * WTM + lrow) * KB;
        const char *bw = bs + sb * BSTAGE + (wn * WTN + lrow) * KB;
        if (SLICES || q == 0) {
#pragma unroll
            for (int b = 0; b < FN; ++b)
                bf[b] = lds_frag<DT, MF>(bw + b * MF * KB, SLICES ? q : 0, lgrp, lsw);
        }
#pragma unroll
        for (int i = 0; i < HA; ++i)
            af[i] = lds_frag<DT, MF>(aw + (SLICES ? i : q * HA + i) * MF * KB, SLICES ? q : 0, lgrp, lsw);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    // Compute phase: the MFMAs of half q; hook(i) runs after the MFMAs of A
    // fragment i (the step's DMA instructions go there, between matrix ops).
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
    // IT DMA instructions spread over the HA fragment rows of a compute phase
    auto spread = [&](auto &&one) {
        return [&](int i) {
#pragma unroll
            for (int j = 0; j < IT; ++j)
                if (j * HA / IT == i)
                    one(j);
        };
    };

    // Each group runs its own copy of the loop (the group is fixed per wave);
    // both execute the same barriers: two in the prologue, four per step.
    // DMA instructions issue inside compute phases, between MFMA rows: the
    // filter step ks+2 in group 0's Q0 of step ks+1 (its slot is free once
    // Q2 of ks is over), the activation step ks+2 in group 1's Q1 of ks.
    if (!g) {
        // Prologue: filter steps 0 and 1 land (and, from group 1, activation
        // steps 0 and 1), then this group reads half 0 of step 0.
        issue_b_step(0);
        if (nk > 1)
            issue_b_step(1);
        wait_vmcnt<0>();
        phase_barrier();
        read_half(0, 0, 0);
        phase_barrier();
        int sa = 0, sb = 0;  // slots of step ks
        for (int ks = 0; ks < nk; ++ks) {
            const int sa1 = sa + 1 == SA ? 0 : sa + 1, sb1 = sb ^ 1;  // slots of step ks+1
            {  // Q0: B(ks+1) into the slot of step ks-1
                const bool go = ks >= 1 && ks + 1 < nk;
                const unsigned sh = kb.template b_shift<ESZ>(p);
                compute_half(0, spread([&](int j) {
                    if (go)
                        issue_b(sb1, j, sh);
                }));
                if (go)
                    kb.advance(p);
            }
            phase_barrier();
            read_half(sa, sb, 1);  // Q1
            phase_barrier();
            compute_half(1, no_issue);  // Q2
            wait_vmcnt<0>();  // B(ks+1), this wave's latest filter issue
            phase_barrier();
            if (ks + 1 < nk)  // Q3
                read_half(sa1, sb1, 0);
            phase_barrier();
            sa = sa1;
            sb = sb1;
        }
    } else {
        issue_a_step(0);
        if (nk > 1)
            issue_a_step(1);
        wait_vmcnt<0>();
        phase_barrier();
        phase_barrier();
        int sa = 0, sb = 0;
        for (int ks = 0; ks < nk; ++ks) {
            const int sa1 = sa + 1 == SA ? 0 : sa + 1, sb1 = sb ^ 1;
            const int sa2 = sa1 + 1 == SA ? 0 : sa1 + 1;  // activation slot of step ks+2
            read_half(sa, sb, 0);  // Q0
            phase_barrier();
            {  // Q1: A(ks+2) into the slot of step ks-1
                const bool go = ks + 2 < nk;
                const unsigned sh = ka.template a_shift<MODE, ESZ>(p);
                compute_half(0, spread([&](int j) {
                    if (go)
                        issue_a(sa2, j, sh);
                }));
                if (go)
                    ka.advance(p);
            }
            phase_barrier();
            read_half(sa, sb, 1);  // Q2
            if (ks + 2 < nk)
                wait_vmcnt<IT>();  // A(ks+1) landed, A(ks+2) may still be in flight
            else
                wait_vmcnt<0>();
            phase_barrier();
            compute_half(1, no_issue);  // Q3
            phase_barrier();
            sa = sa1;
            sb = sb1;
        }
    }

    if (split >= 0) {  // tail split: unscaled fp32 sums, [column][row] per tile and split
        float *dst = p.part + ((int64_t)(bid - p.tail_first) * p.tail_splits + split) * (BM * BN);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
                *reinterpret_cast<f32x4 *>(dst + (wn * WTN + b * MF + lrow) * BM + wm * WTM + a * MF + 4 * lgrp) =
                    quad<MF>(acc[a][b], 0);
        return;
    }
    // whole tile inside one image, 16-byte aligned rows: stage the outputs through the idle rings
    if ((p.P & 7) == 0 && m0 + BM <= p.M && n0 + BN <= p.K && m0 / p.P == (m0 + BM - 1) / p.P) {
        store_tile_lds<BM, BN, 2, 4, MF, DT, false>(acc, p, m0, n0, wm, wn, lane, smem);
        return;
    }
    store_tile_ncdhw<MF, FM, FN, DT>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane);
}

template <int DT>
hipError_t launch_conv_pp(const ConvParams &p, Mode mode, hipStream_t stream)
{
    const int ntiles = p.tiles_m * p.tiles_n;  // tail split: the tail tiles take tail_splits workgroups each
    const dim3 grid((unsigned)(p.tail_splits > 1 ? p.tail_first + (ntiles - p.tail_first) * p.tail_splits : ntiles));
    if (mode == MODE_TEMPORAL)
        hipLaunchKernelGGL((conv_igemm_pp_kernel<DT, MODE_TEMPORAL>), grid, dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((conv_igemm_pp_kernel<DT, MODE_GENERIC>), grid, dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace igc

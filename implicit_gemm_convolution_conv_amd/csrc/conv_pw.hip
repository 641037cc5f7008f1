// 1x1x1 convolution straight from NCDHW activations (no transpose).
//
// With a 1x1x1 filter, stride 1 and no padding, the convolution of image n is
// the GEMM Y_n[k][s] = sum_c W[k][c] * X_n[c][s] over the S = D*H*W positions.
// FlyDSL PR #860 routes this shape to a plain matmul precisely because the
// im2col path would first pay an NCDHW->NDHWC transpose of the whole tensor
// (the PR's 1x1x1 measurement in its "Performance" section); here the GEMM
// reads NCDHW x as it is. Its operands for the matrix cores must hold eight
// consecutive channels per lane, while X_n is contiguous along s, so the
// transpose happens inside LDS:
//
//  * A step covers TK channels (32 in the launched kernel). The x tile of a
//    workgroup is TK channel rows x BM positions (2*BM bytes per row), filled
//    by direct-to-LDS loads; the 16-byte chunk q of row c sits at slot
//    q ^ (2 * ((c >> 3) & 3)), so the 16-bit reads below (16 consecutive
//    positions of four rows 8 apart) hit distinct banks.
//  * A lane's A fragment (tile row s, channels c0..c0+7) is eight 16-bit LDS
//    reads down one column; B fragments (the filter, rows of TK channels)
//    are 16-byte reads of the usual swizzled layout.
//  * 4 waves, each BM/4 positions x 64 output channels (16x16x32 bf16 MFMA),
//    a ring of NS stages of (2*BM + 128) * TK bytes; y[n][k][s] is written 4
//    positions (8 bytes) per lane.
//
// The kernel streams x once per 64 output channels and is HBM-bound for the
// shapes it targets (few output channels, many positions).
#include "conv_igemm_buf.h"

namespace igc {

namespace {

constexpr int kPwBN = 64;  // output channels per tile

// 16 bytes per lane from global src into LDS at lds + 16 * lane.
__device__ inline void global_to_lds16(const char *src, char *lds)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// BM positions per tile (4 waves of BM/4), TK channels per reduction step
// (32 or 64: one or two 32-channel MFMA slices), NS ring stages.
template <int BM, int TK, int NS>
__global__ __launch_bounds__(256) void conv_pw_ncdhw_kernel(ConvParams p)
{
    constexpr int ROWB = BM * 2;                 // bytes per x tile row (one channel)
    constexpr int CPRX = BM / 8;                 // 16-byte chunks per x row
    constexpr int RPIX = CPRX >= 64 ? 1 : 64 / CPRX;  // x rows per DMA instruction
    constexpr int XIT = TK * ROWB / 1024 / 4;    // x DMA instructions per wave per step
    constexpr int XSTAGE = TK * ROWB;
    constexpr int WROWB = TK * 2;                // bytes per filter tile row
    constexpr int WSTAGE = kPwBN * WROWB;
    constexpr int WRPI = 1024 / WROWB;           // filter rows per DMA instruction
    constexpr int WIT = kPwBN / WRPI / 4;        // filter DMA instructions per wave per step
    constexpr int STAGE = XSTAGE + WSTAGE;
    constexpr int SB = BM / 64;                  // 16-position blocks per wave
    constexpr int LPS = XIT + WIT;               // DMA instructions per thread per step
    constexpr int SLICES = TK / 32;
    static_assert(BM == 128 || BM == 256 || BM == 512, "tile rows");
    static_assert(TK == 32 || TK == 64, "reduction step");
    static_assert(XIT >= 1 && WIT >= 1, "loader split");
    static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // block -> (image, position tile, channel tile); channel tiles of one position tile are adjacent (L2 reuse of x)
    const int tk = blockIdx.x % p.tiles_n;
    const int rest = blockIdx.x / p.tiles_n;
    const int tiles_s = (p.P + BM - 1) / BM;
    const int n = rest / tiles_s;
    const int s0 = (rest - n * tiles_s) * BM;
    const int k0 = tk * kPwBN;
    const int S = p.P, C = p.C, K = p.K;

    const char *xb = static_cast<const char *>(p.x);
    const char *wb = static_cast<const char *>(p.w);
    const char *zero = reinterpret_cast<const char *>(kZeroLine);

    // x DMA: instruction i of this wave fills the RPIX tile rows from RPIX * (wave + 4 i) on (one 1 KB row for
    // BM = 512; 64 / (BM / 8) rows of BM / 8 lanes each otherwise)
    const int xr_sub = CPRX >= 64 ? 0 : lane / CPRX, xslot = CPRX >= 64 ? lane : lane % CPRX;
    // filter DMA: instruction i fills rows WRPI*(wave + 4 i) .. +WRPI-1; 128-byte rows keep chunk q at slot
    // q ^ (row & 7), 64-byte rows at q ^ ((row >> 1) & 3)
    const int wrow_l = lane / (WROWB / 16);
    const int wchunk = WROWB == 128 ? ((lane & 7) ^ (lane >> 3)) : ((lane & 3) ^ ((lane >> 3) & 3));
    const char *wrow[WIT];
#pragma unroll
    for (int i = 0; i < WIT; ++i) {
        const int k = min(k0 + WRPI * (wave + 4 * i) + wrow_l, K - 1);
        wrow[i] = wb + (int64_t)k * p.ldw * 2 + wchunk * 16;
    }

    auto issue = [&](int step, int st) {
        char *xs = smem + st * STAGE;
        char *ws = xs + XSTAGE;
        const int c0 = step * TK;
#pragma unroll
        for (int i = 0; i < XIT; ++i) {
            const int row = RPIX * (wave + 4 * i) + xr_sub;
            const int c = c0 + row;
            const int q = xslot ^ (2 * ((row >> 3) & 3));
            // S % 8 == 0: a chunk lies wholly inside or wholly past the row's S positions
            const char *src = c < C && s0 + 8 * q < S ? xb + (((int64_t)n * C + c) * S + s0) * 2 + q * 16 : zero;
            global_to_lds16(src, xs + RPIX * (wave + 4 * i) * ROWB);
        }
#pragma unroll
        for (int i = 0; i < WIT; ++i)
            global_to_lds16(wrow[i] + (int64_t)c0 * 2, ws + WRPI * (wave + 4 * i) * WROWB);
    };

    f32x4 acc[SB][4];
#pragma unroll
    for (int b = 0; b < SB; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            acc[b][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lrow = lane & 15, lgrp = lane >> 4;
    auto compute = [&](int st) {
        const char *xs = smem + st * STAGE;
        const char *ws = xs + XSTAGE;
#pragma unroll
        for (int h = 0; h < SLICES; ++h) {
            bf16x8 wf[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int row = 16 * kb + lrow;
                wf[kb] = lds_frag<DT_BF16, 16>(ws + row * WROWB, h, lgrp, WROWB == 128 ? (row & 7) : ((row >> 1) & 3));
            }
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int s = (BM / 4) * wave + 16 * b + lrow;  // tile row of this lane
                const int cbase = 32 * h + 8 * lgrp;
                bf16x8 xf;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = cbase + j;
                    const int slot = (s >> 3) ^ (2 * ((c >> 3) & 3));
                    xf[j] = *reinterpret_cast<const __bf16 *>(xs + c * ROWB + slot * 16 + (s & 7) * 2);
                }
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    acc[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wf[kb], acc[b][kb], 0, 0, 0);
            }
        }
    };

    const int nk = p.nk;
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
        if (st < nk)
            issue(st, st);
    for (int ks = 0; ks < nk; ++ks) {
        // steps issued after ks and possibly still in flight: min(NS - 2, nk - 1 - ks)
        const int ahead = nk - 1 - ks;
        if (ahead >= NS - 2)
            wait_vmcnt<LPS * (NS - 2)>();
        else if (NS > 3 && ahead == 1)
            wait_vmcnt<LPS>();
        else
            wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
        if (ks + NS - 1 < nk)
            issue(ks + NS - 1, (ks + NS - 1) % NS);
        compute(ks % NS);
    }

    // y[n][k][s]: lane holds positions 4*lgrp..+3 of each 16-row block for output channel lrow of each column block
    uint16_t *yb = static_cast<uint16_t *>(p.y);
    with_epilogue(p, false, [&](auto &ep) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int s = s0 + (BM / 4) * wave + 16 * b + 4 * lgrp;
            if (s >= S)
                continue;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int k = k0 + 16 * kb + lrow;
                if (k >= K)
                    continue;
                *reinterpret_cast<u32x2 *>(yb + ((int64_t)n * K + k) * S + s) = ep.four(acc[b][kb], k);
            }
        }
    });
}

}  // namespace

hipError_t launch_conv_pw(const ConvParams &p, hipStream_t stream)
{
    // 512 positions x 64 output channels, 32-channel steps, 4 stages: the fastest of the shapes measured on
    // the 14 GB 512 -> 48 workload (256 or 512 positions, 32 or 64 channels per step, 2 to 4 stages)
    hipLaunchKernelGGL((conv_pw_ncdhw_kernel<512, 32, 4>), dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace igc

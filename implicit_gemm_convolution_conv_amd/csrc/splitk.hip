// Second pass of the split reduction: y = bf16(scale * sum of the fp32 slices + bias).
//
// The direct-to-LDS conv kernel, run with p.splits > 1, leaves `splits` slices
// of unscaled fp32 sums, each indexed like y. This pass adds them in split
// order (so the result does not depend on scheduling), then applies the
// epilogue of the unsplit kernels (Epilogue: s_x * s_w for fp8, the channel's
// bias, bf16 rounding to nearest even, the amax of y). It streams
// splits * 4 + 2 bytes per output element and is bound by HBM bandwidth;
// 4 consecutive elements per lane (16-byte loads, one 8-byte store) when the
// element count is a multiple of 4. Element i of y belongs to channel
// (i / P) % K, which also covers point output (P = 1, y[n][k]).
#include <algorithm>

#include "conv_igemm.h"

namespace igc {

namespace {

__global__ __launch_bounds__(256) void splitk_reduce_kernel(ConvParams p)
{
    const int64_t ynum = (int64_t)p.M * p.Ncol;
    const float *part = p.part;
    const int splits = p.splits;
    uint16_t *y = static_cast<uint16_t *>(p.y);
    const int64_t step = (int64_t)gridDim.x * 256 * 4;
    const bool vec = (ynum & 3) == 0;
    const bool same_k = (p.P & 3) == 0;  // 4 consecutive elements (from a multiple of 4) share a channel
    with_epilogue(p, p.scales != nullptr, [&](auto &ep) __attribute__((always_inline)) {
        for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < ynum; i += step) {
            if (vec) {
                f32x4 acc = *reinterpret_cast<const f32x4 *>(part + i);
                for (int j = 1; j < splits; ++j)
                    acc += *reinterpret_cast<const f32x4 *>(part + (int64_t)j * ynum + i);
                u32x2 pk;
                if (same_k) {
                    pk = ep.four(acc, (int)((i / p.P) % p.K));
                } else {
                    uint32_t r[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        r[e] = ep.one(acc[e], (int)(((i + e) / p.P) % p.K));
                    pk = u32x2{r[0] | (r[1] << 16), r[2] | (r[3] << 16)};
                }
                *reinterpret_cast<u32x2 *>(y + i) = pk;
            } else {
                for (int e = 0; e < 4 && i + e < ynum; ++e) {
                    float a = part[i + e];
                    for (int j = 1; j < splits; ++j)
                        a += part[(int64_t)j * ynum + i + e];
                    y[i + e] = (uint16_t)ep.one(a, (int)(((i + e) / p.P) % p.K));
                }
            }
        }
    });
}

// Tail split, second pass: block (x, t) sums 4 consecutive rows of one column
// of tail tile t per lane over its splits, in split order, and stores them
// through the epilogue like the direct store of the conv kernels (8 bytes
// when the 4 rows share an image and P % 4 == 0).
__global__ __launch_bounds__(256) void tail_reduce_kernel(ConvParams p, int bm, int bn)
{
    const int t = blockIdx.y;
    int tm, tn;
    tile_coords(p, p.tail_first + t, tm, tn);
    const int quad = blockIdx.x * 256 + threadIdx.x;  // bm / 4 quads per column
    const int col_l = quad / (bm / 4), row_l = (quad - col_l * (bm / 4)) * 4;
    const bool live = col_l < bn;
    const int64_t tsz = (int64_t)bm * bn;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
        const float *src = p.part + (int64_t)t * p.tail_splits * tsz + (int64_t)col_l * bm + row_l;
        acc = *reinterpret_cast<const f32x4 *>(src);
        for (int j = 1; j < p.tail_splits; ++j)
            acc += *reinterpret_cast<const f32x4 *>(src + j * tsz);
    }
    const int row = tm * bm + row_l, col = tn * bn + col_l;
    uint16_t *yb = static_cast<uint16_t *>(p.y);
    with_epilogue(p, p.scales != nullptr, [&](auto &ep) __attribute__((always_inline)) {
        if (!live || row >= p.M || col >= p.K)
            return;
        const int nimg = row / p.P, sp = row - nimg * p.P;
        if ((p.P & 3) == 0 && row + 3 < p.M) {
            *reinterpret_cast<u32x2 *>(yb + ((int64_t)nimg * p.K + col) * p.P + sp) = ep.four(acc, col);
        } else {
            for (int e = 0; e < 4; ++e) {
                const int m = row + e;
                if (m < p.M) {
                    const int n2 = m / p.P, sp2 = m - n2 * p.P;
                    yb[((int64_t)n2 * p.K + col) * p.P + sp2] = (uint16_t)ep.one(acc[e], col);
                }
            }
        }
    });
}

__global__ void amax_clear_kernel(float *out)
{
    if (threadIdx.x == 0)
        *out = 0.0f;
}

}  // namespace

hipError_t launch_splitk_reduce(const ConvParams &p, hipStream_t stream)
{
    const int64_t ynum = (int64_t)p.M * p.Ncol;
    const int64_t blocks = std::min<int64_t>((ynum + 1023) / 1024, 8192);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_tail_reduce(const ConvParams &p, int bm, int bn, int ntail, hipStream_t stream)
{
    const int quads = bm / 4 * bn;
    hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)((quads + 255) / 256), (unsigned)ntail), dim3(256), 0, stream,
                       with_divisors(p), bm, bn);
    return hipGetLastError();
}

hipError_t launch_amax_zero(float *amax, hipStream_t stream)
{
    hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(64), 0, stream, amax);
    return hipGetLastError();
}

}  // namespace igc

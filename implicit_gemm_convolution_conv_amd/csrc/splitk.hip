// Second pass of the split reduction: y = bf16(scale * sum of the fp32 slices).
//
// The direct-to-LDS conv kernel, run with p.splits > 1, leaves `splits` slices
// of unscaled fp32 sums, each indexed like y. This pass adds them in split
// order (so the result does not depend on scheduling), multiplies by
// s_x * s_w for fp8 (the one scale the unsplit epilogue applies) and rounds to
// bf16 to nearest even. It streams splits * 4 + 2 bytes per output element and
// is bound by HBM bandwidth; 4 consecutive elements per lane (16-byte loads,
// one 8-byte store) when the element count is a multiple of 4.
#include <algorithm>

#include "conv_igemm.h"

namespace igc {

namespace {

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *part, int splits, int64_t ynum,
                                                            const float *scales, uint16_t *y)
{
    const float sc = scales ? scales[0] * scales[2] : 1.0f;
    const int64_t step = (int64_t)gridDim.x * 256 * 4;
    const bool vec = (ynum & 3) == 0;
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < ynum; i += step) {
        if (vec) {
            f32x4 acc = *reinterpret_cast<const f32x4 *>(part + i);
            for (int j = 1; j < splits; ++j)
                acc += *reinterpret_cast<const f32x4 *>(part + (int64_t)j * ynum + i);
            acc *= sc;
            const u32x2 pk = {f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16),
                              f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16)};
            *reinterpret_cast<u32x2 *>(y + i) = pk;
        } else {
            for (int e = 0; e < 4 && i + e < ynum; ++e) {
                float a = part[i + e];
                for (int j = 1; j < splits; ++j)
                    a += part[(int64_t)j * ynum + i + e];
                y[i + e] = (uint16_t)f32_to_bf16_rne(a * sc);
            }
        }
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const float *part, int splits, int64_t ynum, const float *scales, void *y,
                                hipStream_t stream)
{
    const int64_t blocks = std::min<int64_t>((ynum + 1023) / 1024, 8192);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, stream, part,
                       splits, ynum, scales, static_cast<uint16_t *>(y));
    return hipGetLastError();
}

}  // namespace igc

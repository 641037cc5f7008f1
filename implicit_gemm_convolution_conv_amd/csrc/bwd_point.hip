// Operand preparation for the point-output gradients.
//
// MIOpen PR #10912 computes both gradients of a point-output convolution
// (input extent equal to the filter extent, stride equal to the filter, so one
// output position per image) as one GEMM over the batch (PR body):
//   backward data     dx[n][j] = sum_k dy[n][k] * w[k][j]
//   backward weights  dw[k][j] = sum_n dy[n][k] * x[n][j]
// with j over the C*T*R*S elements of an image, in the activation layout's
// order. Both run on the point-output GEMM kernel (MODE_POINT), which wants
// both operands with the reduction index contiguous:
//  * backward data reduces over k: the filter is repacked once as
//    w_t[j][k] (pack_w_t_kernel), dy rows are used as they are;
//  * backward weights reduces over n, the slow index of both dy and x: both
//    are transposed into the workspace as [k][n] and [j][n] rows of ldn
//    elements, zero-filled from N to ldn (transpose_pad_kernel). The pass is
//    bound by HBM bandwidth: 2 bytes read and 2 written per element.
#include <algorithm>

#include "conv_igemm.h"

namespace igc {

namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// dst[c][r] = src[r][c] for r < rows, c < cols; dst[c][r] = 0 for rows <= r < ld.
// One workgroup per 64 x 64 block (64 rows r of src x 64 columns c), 256 threads.
// Loads: consecutive lanes read consecutive 4-byte pairs of one src row (EVEN:
// cols even and src 4-byte aligned), else consecutive 2-byte elements, so each
// wave instruction reads whole 128-byte row segments. Stores: 8 lanes per dst
// row, 16 bytes (8 consecutive r) each; dst rows of ld elements, ld % 8 == 0,
// dst 16-byte aligned.
template <bool EVEN>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t *src, uint16_t *dst, int64_t rows,
                                                            int64_t cols, int64_t ld)
{
    __shared__ uint16_t tile[64][66];  // [r][c]; the 66-element pitch spreads the column reads over banks
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
    if (EVEN) {
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {  // 8 rows per pass, 32 lanes x 2 elements per row
            const int lr = pass * 8 + (tid >> 5), lc = (tid & 31) * 2;
            const int64_t r = r0 + lr, c = c0 + lc;
            uint32_t u = 0;
            if (r < rows && c < cols)  // c even, cols even: the pair is whole
                u = *reinterpret_cast<const uint32_t *>(src + r * cols + c);
            *reinterpret_cast<uint32_t *>(&tile[lr][lc]) = u;
        }
    } else {
#pragma unroll
        for (int pass = 0; pass < 16; ++pass) {  // 4 rows per pass, 64 lanes x 1 element per row
            const int lr = pass * 4 + (tid >> 6), lc = tid & 63;
            const int64_t r = r0 + lr, c = c0 + lc;
            tile[lr][lc] = (r < rows && c < cols) ? src[r * cols + c] : (uint16_t)0;
        }
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {  // 32 dst rows per pass, 8 lanes x 16 bytes per row
        const int lc = pass * 32 + (tid >> 3), q = tid & 7;
        const int64_t c = c0 + lc, r = r0 + 8 * q;
        if (c >= cols || r >= ld)
            continue;
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = tile[8 * q + e][lc];  // rows past `rows` were loaded as 0
        *reinterpret_cast<u16x8 *>(dst + c * ld + r) = v;
    }
}

// w_t[j][k] = w[k][c][t][r][s] with j = ((c * T + t) * R + r) * S + s (channel-first
// activations) or ((t * R + r) * S + s) * C + c (channel-last); zero for K <= k < ldk.
__global__ __launch_bounds__(256) void pack_w_t_kernel(const uint16_t *w, uint16_t *wt, int64_t K, int64_t C,
                                                       int64_t T, int64_t R, int64_t S, int64_t ldk,
                                                       bool channel_last)
{
    const int64_t rk = C * T * R * S;
    const int64_t total = rk * ldk;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t j = i / ldk, k = i - j * ldk;
        uint16_t v = 0;
        if (k < K) {
            int64_t c, tap;  // tap = (t * R + r) * S + s
            if (channel_last) {
                c = j % C;
                tap = j / C;
            } else {
                c = j / (T * R * S);
                tap = j - c * (T * R * S);
            }
            v = w[(k * C + c) * (T * R * S) + tap];
        }
        wt[i] = v;
    }
}

}  // namespace

hipError_t launch_transpose_pad(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t cols, int64_t ld,
                                hipStream_t stream)
{
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((ld + 63) / 64));
    const bool even = (cols & 1) == 0 && (reinterpret_cast<uintptr_t>(src) & 3) == 0;
    if (even)
        hipLaunchKernelGGL(transpose_pad_kernel<true>, grid, dim3(256), 0, stream, src, dst, rows, cols, ld);
    else
        hipLaunchKernelGGL(transpose_pad_kernel<false>, grid, dim3(256), 0, stream, src, dst, rows, cols, ld);
    return hipGetLastError();
}

hipError_t launch_pack_w_t(const uint16_t *w, uint16_t *wt, int64_t K, int64_t C, int64_t T, int64_t R, int64_t S,
                           int64_t ldk, bool channel_last, hipStream_t stream)
{
    const int64_t total = C * T * R * S * ldk;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_w_t_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, stream, w, wt, K,
                       C, T, R, S, ldk, channel_last);
    return hipGetLastError();
}

}  // namespace igc

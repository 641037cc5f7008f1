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

// One operand of the transpose pass: dst[c][r] = src[r][c] for r < rows, c < cols, and dst[c][r] = 0 for
// rows <= r < ld (ld % 64 == 0, dst 16-byte aligned); v = 8 when cols % 8 == 0 and src is 16-byte aligned,
// 4 when cols % 4 == 0 and src is 8-byte aligned, else 1: the elements one row load takes.
struct TransposeOp {
    const uint16_t *src;
    uint16_t *dst;
    int64_t rows, cols, ld;
    int v;
    int blocks_x;  // workgroups along the columns: ceil(cols / 256)
};

// Both operands of the backward-weights GEMM in one launch (workgroups [0, a.blocks_x * ld / 64) transpose
// a, the rest b). Register transpose, no LDS and no barrier, as the activation pack does it: a lane reads 8 src
// rows x 8 columns, transposes them in registers and writes 8 dst rows x 8 elements, one 16-byte store each.
// In a wave, lanes side by side cover 8 x 8 = 64 src rows and lanes 8 apart 64 columns, so each load
// instruction reads whole 128-byte pieces of 8 src rows (with 16-byte loads) and each store writes whole
// 128-byte pieces of 8 dst rows; a workgroup (4 waves) covers 64 rows x 256 columns.
__global__ __launch_bounds__(256) void transpose_pad_kernel(TransposeOp a, TransposeOp b)
{
    const int64_t na = (int64_t)a.blocks_x * (a.ld / 64);
    const bool first = (int64_t)blockIdx.x < na;
    const TransposeOp op = first ? a : b;
    const int64_t blk = first ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - na;
    const int64_t bx = blk % op.blocks_x, by = blk / op.blocks_x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r = by * 64 + (lane & 7) * 8;                                  // this lane's 8 src rows
    const int64_t c = (bx * 4 + wave) * 64 + (int64_t)(lane >> 3) * 8;            // and 8 columns
    if (c >= op.cols || r >= op.ld)
        return;
    const int64_t rows = op.rows, cols = op.cols;
    const int nc = cols - c < 8 ? (int)(cols - c) : 8;  // columns in range (a multiple of v when v > 1)
    uint32_t v[8][4];  // v[i][q]: src row r + i, columns c + 2q (low half) and c + 2q + 1 (high half)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[i][q] = 0u;
        if (r + i >= rows)
            continue;
        const uint16_t *row = op.src + (r + i) * cols + c;
        if (op.v == 8) {
            const i32x4 t = *reinterpret_cast<const i32x4 *>(row);  // nc == 8: cols % 8 == 0
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[i][q] = (uint32_t)t[q];
        } else if (op.v == 4) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (4 * h < nc) {
                    const uint2 t = *reinterpret_cast<const uint2 *>(row + 4 * h);
                    v[i][2 * h] = t.x;
                    v[i][2 * h + 1] = t.y;
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = 2 * q < nc ? row[2 * q] : 0u;
                const uint32_t hi = 2 * q + 1 < nc ? row[2 * q + 1] : 0u;
                v[i][q] = lo | (hi << 16);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (e >= nc)
            break;
        i32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // src rows r + 2q and r + 2q + 1 at column c + e
            const uint32_t lo = v[2 * q][e >> 1], hi = v[2 * q + 1][e >> 1];
            o[q] = (e & 1) ? (int)((lo >> 16) | (hi & 0xffff0000u)) : (int)((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<i32x4 *>(op.dst + (c + e) * op.ld + r) = o;  // ld % 8 == 0, r % 8 == 0: aligned
    }
}

TransposeOp transpose_op(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t cols, int64_t ld)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(src);
    const int v = (cols % 8 == 0 && a % 16 == 0) ? 8 : (cols % 4 == 0 && a % 8 == 0) ? 4 : 1;
    return TransposeOp{src, dst, rows, cols, ld, v, (int)((cols + 255) / 256)};
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

hipError_t launch_transpose_pad2(const uint16_t *src_a, uint16_t *dst_a, int64_t cols_a, const uint16_t *src_b,
                                 uint16_t *dst_b, int64_t cols_b, int64_t rows, int64_t ld, hipStream_t stream)
{
    const TransposeOp a = transpose_op(src_a, dst_a, rows, cols_a, ld), b = transpose_op(src_b, dst_b, rows, cols_b, ld);
    const int64_t blocks = ((int64_t)a.blocks_x + b.blocks_x) * (ld / 64);
    hipLaunchKernelGGL(transpose_pad_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b);
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

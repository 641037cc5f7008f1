// Operand preparation kernels: per-tensor amax and fp8 scales, the activation
// pack (NCDHW -> NDHWC transpose, optionally to fp8 E4M3FN) and the filter
// pack (KCTRS -> K x crs_pad rows in the activation's channel order).
//
// These kernels move data and are bound by HBM bandwidth: each reads and
// writes every element once, with 16-byte global accesses on both sides
// (the fp8 pack writes 16-byte runs of codes, never single bytes).
#include "igconv_internal.h"

namespace igc {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ amax
// Non-negative floats order like their bit patterns, so the maximum of
// |bf16| is the maximum of (bits & 0x7fff); as fp32 bits it is that << 16.

__global__ void amax_zero_kernel(float *out)
{
    if (threadIdx.x == 0)
        *out = 0.0f;
}

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t *t, int64_t n, unsigned *out)
{
    const int64_t nvec = n >> 3;  // 8 bf16 per 16-byte load
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned m = 0;
    const i32x4 *tv = reinterpret_cast<const i32x4 *>(t);
    for (int64_t i = gid; i < nvec; i += stride) {
        const i32x4 v = tv[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned u = (unsigned)v[q];
            m = max(m, max(u & 0x7fffu, (u >> 16) & 0x7fffu));
        }
    }
    for (int64_t i = nvec * 8 + gid; i < n; i += stride)
        m = max(m, (unsigned)(t[i] & 0x7fffu));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        m = max(m, (unsigned)__shfl_xor((int)m, off));
    __shared__ unsigned red[4];
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = max(max(red[0], red[1]), max(red[2], red[3]));
        atomicMax(out, m << 16);
    }
}

hipError_t launch_amax(const uint16_t *t, int64_t n, float *amax, hipStream_t stream)
{
    hipLaunchKernelGGL(amax_zero_kernel, dim3(1), dim3(64), 0, stream, amax);
    const int64_t want = ((n >> 3) + 255) / 256;
    const unsigned blocks = (unsigned)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
    hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(256), 0, stream, t, n, reinterpret_cast<unsigned *>(amax));
    return hipGetLastError();
}

// ------------------------------------------------------------------ scales

__global__ void fp8_scales_kernel(const float *amax, float *pair)
{
    if (threadIdx.x != 0)
        return;
    const float a = *amax;
    float s = 1.0f, inv = 1.0f;
    if (a > 0.0f) {
        s = __fdiv_rn(a, 448.0f);    // largest finite E4M3FN value
        inv = __fdiv_rn(448.0f, a);
    }
    pair[0] = s;
    pair[1] = inv;
}

hipError_t launch_fp8_scales(const float *amax, float *pair, hipStream_t stream)
{
    hipLaunchKernelGGL(fp8_scales_kernel, dim3(1), dim3(64), 0, stream, amax, pair);
    return hipGetLastError();
}

// ------------------------------------------------------------------ E4M3FN encode
// Round to nearest even, saturating at +-448, NaN -> 0x7F | sign; subnormals
// (|v| < 2^-6) are multiples of 2^-9.
__device__ inline uint32_t e4m3_rne_sat(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u)
        return sign | 0x7fu;
    if (a >= 0x43e00000u)  // |v| >= 448
        return sign | 0x7eu;
    if (a < 0x3c800000u) {  // |v| < 2^-6: code = round(|v| * 2^9), exact scaling, 0..8
        const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
        return sign | (uint32_t)q;
    }
    // normal: keep 3 of the 23 mantissa bits, ties to even, then rebias 127 -> 7
    a += 0x7ffffu + ((a >> 20) & 1u);
    return sign | ((a >> 20) - (120u << 3));
}

// ------------------------------------------------------------------ activation pack
// One workgroup transposes a 64 (channels) x 64 (spatial) tile of one image
// through LDS. Reads are 16-byte pieces of channel rows (8 spatial), writes
// are 16-byte pieces of spatial rows (8 bf16 or 16 fp8 channels).
template <bool FP8, bool VEC_S>
__global__ __launch_bounds__(256) void pack_x_kernel(const uint16_t *x, void *out, int64_t C, int64_t S,
                                                     int64_t cblocks, int64_t sblocks, const float *pair)
{
    __shared__ uint32_t tile[64][65];
    const int64_t b = blockIdx.x;
    const int64_t sb = b % sblocks;
    const int64_t rest = b / sblocks;
    const int64_t cb = rest % cblocks;
    const int64_t n = rest / cblocks;
    const int64_t c0 = cb * 64, s0 = sb * 64;
    const int tid = threadIdx.x;

    {  // load: thread -> channel row (tid / 8 + 32 p), spatial piece (tid % 8)
        const int sc = (tid & 7) * 8;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int cl = (tid >> 3) + 32 * p;
            const int64_t c = c0 + cl;
            const int64_t s = s0 + sc;
            if (c >= C)
                continue;
            const uint16_t *src = x + (n * C + c) * S + s;
            if (VEC_S) {
                if (s < S) {
                    const i32x4 v = *reinterpret_cast<const i32x4 *>(src);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        tile[cl][sc + 2 * q] = (uint32_t)v[q] & 0xffffu;
                        tile[cl][sc + 2 * q + 1] = (uint32_t)v[q] >> 16;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (s + e < S)
                        tile[cl][sc + e] = src[e];
            }
        }
    }
    __syncthreads();

    if (!FP8) {  // store: thread -> spatial row (tid / 8 + 32 p), 8 channels (tid % 8)
        const int cc = (tid & 7) * 8;
        uint16_t *o = static_cast<uint16_t *>(out);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int sl = (tid >> 3) + 32 * p;
            const int64_t s = s0 + sl, c = c0 + cc;
            if (s >= S || c >= C)
                continue;
            i32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = (int)(tile[cc + 2 * q][sl] | (tile[cc + 2 * q + 1][sl] << 16));
            *reinterpret_cast<i32x4 *>(o + (n * S + s) * C + c) = v;
        }
    } else {  // store: thread -> spatial row (tid / 4), 16 channels (tid % 4)
        const float inv = pair[1];
        const int cc = (tid & 3) * 16;
        const int sl = tid >> 2;
        const int64_t s = s0 + sl, c = c0 + cc;
        if (s < S && c < C) {
            i32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t wd = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f = __uint_as_float(tile[cc + 4 * q + e][sl] << 16) * inv;
                    wd |= e4m3_rne_sat(f) << (8 * e);
                }
                v[q] = (int)wd;
            }
            *reinterpret_cast<i32x4 *>(static_cast<uint8_t *>(out) + (n * S + s) * C + c) = v;
        }
    }
}

hipError_t launch_pack_x(const uint16_t *x, void *out, int64_t N, int64_t C, int64_t S, Dtype dt,
                         const float *pair, hipStream_t stream)
{
    const int64_t cblocks = (C + 63) / 64, sblocks = (S + 63) / 64;
    const dim3 grid((unsigned)(N * cblocks * sblocks));
    const bool vec = (S % 8) == 0;
    if (dt == DT_FP8) {
        if (vec)
            hipLaunchKernelGGL((pack_x_kernel<true, true>), grid, dim3(256), 0, stream, x, out, C, S, cblocks,
                               sblocks, pair);
        else
            hipLaunchKernelGGL((pack_x_kernel<true, false>), grid, dim3(256), 0, stream, x, out, C, S, cblocks,
                               sblocks, pair);
    } else {
        if (vec)
            hipLaunchKernelGGL((pack_x_kernel<false, true>), grid, dim3(256), 0, stream, x, out, C, S, cblocks,
                               sblocks, pair);
        else
            hipLaunchKernelGGL((pack_x_kernel<false, false>), grid, dim3(256), 0, stream, x, out, C, S, cblocks,
                               sblocks, pair);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ filter pack
// out[k][col], col < ldw: the element of w[k] at reduction index col in
// (t, r, s, c) order (channel_last) or (c, t, r, s) order; zero past C*T*R*S.
template <bool FP8>
__global__ __launch_bounds__(256) void pack_w_kernel(const uint16_t *w, void *out, int64_t K, int64_t C, int64_t T,
                                                     int64_t R, int64_t S, int64_t ldw, bool channel_last,
                                                     const float *pair)
{
    const int64_t total = K * ldw;
    const int64_t rk = C * T * R * S;
    const int64_t taps = T * R * S;
    const float inv = FP8 ? pair[1] : 1.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = i / ldw, col = i - k * ldw;
        uint32_t bits = 0;
        if (col < rk) {
            int64_t c, tap;
            if (channel_last) {
                tap = col / C;
                c = col - tap * C;
            } else {
                c = col / taps;
                tap = col - c * taps;
            }
            bits = w[(k * C + c) * taps + tap];  // w[k][c][t][r][s], taps flattened (t, r, s)
        }
        if (FP8)
            static_cast<uint8_t *>(out)[i] = (uint8_t)e4m3_rne_sat(__uint_as_float(bits << 16) * inv);
        else
            static_cast<uint16_t *>(out)[i] = (uint16_t)bits;
    }
}

hipError_t launch_pack_w(const uint16_t *w, void *out, int64_t K, int64_t C, int64_t T, int64_t R, int64_t S,
                         int64_t ldw, bool channel_last, Dtype dt, const float *pair, hipStream_t stream)
{
    const int64_t total = K * ldw;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    if (dt == DT_FP8)
        hipLaunchKernelGGL(pack_w_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, w, out, K, C, T, R, S,
                           ldw, channel_last, pair);
    else
        hipLaunchKernelGGL(pack_w_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, w, out, K, C, T, R,
                           S, ldw, channel_last, pair);
    return hipGetLastError();
}

}  // namespace igc

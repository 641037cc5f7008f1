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
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ amax
// Non-negative floats order like their bit patterns, so the maximum of
// |bf16| is the maximum of (bits & 0x7fff); as fp32 bits it is that << 16.

__global__ void amax_zero_kernel(float *out)
{
    if (threadIdx.x == 0)
        *out = 0.0f;
}

// Each lane keeps eight independent 16-byte loads in flight per round and
// folds them with packed 16-bit maxima; the grid covers the CUs 16 times.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t *t, int64_t n, unsigned *out)
{
    constexpr int U = 8;
    const int64_t nvec = n >> 3;  // 8 bf16 per 16-byte load
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const i32x4 *tv = reinterpret_cast<const i32x4 *>(t);
    us2 mx = {0, 0};
    int64_t i = gid;
    for (; i + (U - 1) * stride < nvec; i += U * stride) {
        i32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(tv + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, (unsigned)v[u][q] & 0x7fff7fffu));
    }
    for (; i < nvec; i += stride) {
        const i32x4 v = tv[i];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, (unsigned)v[q] & 0x7fff7fffu));
    }
    unsigned m = mx[0] > mx[1] ? mx[0] : mx[1];
    for (int64_t j = nvec * 8 + gid; j < n; j += stride)
        m = max(m, (unsigned)(t[j] & 0x7fffu));
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
// Register transpose, no LDS and no barrier. A lane reads CPT channel rows x
// 8 spatial positions (one 16-byte load per row when S % 8 == 0), transposes
// them in registers and writes 8 spatial rows x CPT channels (one 16-byte
// store per row: 8 bf16 values or 16 fp8 codes). Eight lanes side by side
// along channels and eight along space make every load and every store of a
// wave cover whole 128-byte lines: 8 channel rows x 128 bytes on the read
// side, 8 spatial rows x 128 bytes on the write side. A workgroup (4 waves)
// covers 8*CPT channels x 256 spatial positions.
//
// Block order, measured on MI355X: bf16 walks the channel blocks of one
// spatial range together (whole output rows written side by side) with
// nontemporal stores; fp8 walks the spatial blocks of one channel block.
//
// fp8 codes: a lane first takes the largest |bf16| it holds. When that value
// times |inv| is below 448, no product can saturate or be NaN, and the
// hardware conversion (round to nearest even into E4M3FN) gives the code;
// otherwise the lane encodes with e4m3_rne_sat. Both give the same bits
// wherever both apply.
template <bool FP8, bool VEC_S>
__global__ __launch_bounds__(256) void pack_x_kernel(const uint16_t *x, void *out, int64_t C, int64_t S,
                                                     int64_t cblocks, int64_t sblocks, const float *pair)
{
    constexpr int CPT = FP8 ? 16 : 8;  // channels per lane
    constexpr int CB = 8 * CPT;        // channels per workgroup
    const int64_t b = blockIdx.x;
    int64_t sb, cb, n;
    if (FP8) {
        sb = b % sblocks;
        const int64_t r = b / sblocks;
        cb = r % cblocks;
        n = r / cblocks;
    } else {
        cb = b % cblocks;
        const int64_t r = b / cblocks;
        sb = r % sblocks;
        n = r / sblocks;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = cb * CB + (lane & 7) * CPT;  // C % CPT == 0: all CPT channels in range or none
    const int64_t s = sb * 256 + wave * 64 + (lane >> 3) * 8;
    if (c >= C || s >= S)
        return;
    const int ns = S - s < 8 ? (int)(S - s) : 8;  // spatial positions in range (8 unless at the ragged end)

    uint32_t r[CPT][4];  // r[i][q]: channel c + i, positions s + 2q (low half) and s + 2q + 1 (high half)
    const uint16_t *src = x + (n * C + c) * S + s;
    if (VEC_S) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const i32x4 v = *reinterpret_cast<const i32x4 *>(src + i * S);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[i][q] = (uint32_t)v[q];
        }
    } else {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = 2 * q < ns ? src[i * S + 2 * q] : 0u;
                const uint32_t hi = 2 * q + 1 < ns ? src[i * S + 2 * q + 1] : 0u;
                r[i][q] = lo | (hi << 16);
            }
    }

    if (!FP8) {
        uint16_t *o = static_cast<uint16_t *>(out) + (n * S + s) * C + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (e >= ns)
                break;
            i32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // channels 2q, 2q+1 at position e
                const uint32_t lo = r[2 * q][e >> 1], hi = r[2 * q + 1][e >> 1];
                v[q] = (e & 1) ? (int)((lo >> 16) | (hi & 0xffff0000u)) : (int)((lo & 0xffffu) | (hi << 16));
            }
            __builtin_nontemporal_store(v, reinterpret_cast<i32x4 *>(o + e * C));
        }
    } else {
        const float inv = pair[1];
        us2 mx = {0, 0};
#pragma unroll
        for (int i = 0; i < CPT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, r[i][q] & 0x7fff7fffu));
        const uint32_t m16 = mx[0] > mx[1] ? mx[0] : mx[1];
        // false for NaN too (a NaN input or inv makes the comparison false)
        const bool hw = __uint_as_float(m16 << 16) * __builtin_fabsf(inv) < 448.0f;
        uint8_t *o = static_cast<uint8_t *>(out) + (n * S + s) * C + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (e >= ns)
                break;
            i32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // channels 4q .. 4q+3 at position e
                float f[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wd = r[4 * q + j][e >> 1];
                    f[j] = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16)) * inv;
                }
                if (hw) {
                    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                    v[q] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pk, true);
                } else {
                    v[q] = (int)(e4m3_rne_sat(f[0]) | (e4m3_rne_sat(f[1]) << 8) | (e4m3_rne_sat(f[2]) << 16) |
                                 (e4m3_rne_sat(f[3]) << 24));
                }
            }
            *reinterpret_cast<i32x4 *>(o + e * C) = v;
        }
    }
}

hipError_t launch_pack_x(const uint16_t *x, void *out, int64_t N, int64_t C, int64_t S, Dtype dt,
                         const float *pair, hipStream_t stream)
{
    const int64_t cb_ch = dt == DT_FP8 ? 128 : 64;
    const int64_t cblocks = (C + cb_ch - 1) / cb_ch, sblocks = (S + 255) / 256;
    if (N * cblocks * sblocks > (int64_t(1) << 24))  // a dispatch holds at most 2^32 work-items
        return hipErrorInvalidValue;
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
// Each thread writes one 16-byte run of a packed row (16 fp8 codes or 8 bf16
// values; ldw is a multiple of 64, so a run never crosses a row): whole
// 16-byte stores, as Primus-Turbo PR #399 found fp8 operand preparation to
// need (its fp8 scatter-store coalescing commit), rather than single bytes.
template <bool FP8>
__global__ __launch_bounds__(256) void pack_w_kernel(const uint16_t *w, void *out, int64_t K, int64_t C, int64_t T,
                                                     int64_t R, int64_t S, int64_t ldw, bool channel_last,
                                                     const float *pair)
{
    constexpr int E = FP8 ? 16 : 8;  // elements per 16-byte run
    const int64_t runs = ldw / E;     // runs per packed row
    const int64_t total = K * runs;
    const int64_t rk = C * T * R * S;
    const int64_t taps = T * R * S;
    const float inv = FP8 ? pair[1] : 1.0f;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = q / runs, col0 = (q - k * runs) * E;
        uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int64_t col = col0 + e;
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
                word[e / 4] |= e4m3_rne_sat(__uint_as_float(bits << 16) * inv) << (8 * (e % 4));
            else
                word[e / 2] |= bits << (16 * (e % 2));
        }
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<u32x4 *>(static_cast<char *>(out) + q * 16) = u32x4{word[0], word[1], word[2], word[3]};
    }
}

hipError_t launch_pack_w(const uint16_t *w, void *out, int64_t K, int64_t C, int64_t T, int64_t R, int64_t S,
                         int64_t ldw, bool channel_last, Dtype dt, const float *pair, hipStream_t stream)
{
    const int64_t total = K * ldw / (dt == DT_FP8 ? 16 : 8);
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

// Internal declarations shared by the host library and the kernel translation
// units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace igc {

enum Mode { MODE_GENERIC = 0, MODE_TEMPORAL = 1, MODE_POINT = 2 };
enum Dtype { DT_BF16 = 0, DT_FP8 = 1 };

// Tile shapes: rows x cols of the GEMM tile, waves along rows x cols, MFMA
// block edge (16: 16x16 blocks), LDS stages and bytes of k per row per
// reduction step (kb: 128 = 64 bf16 / 128 fp8; 64 = 32 bf16 channels for the
// NCDHW 1x1x1 kernel). sb == 0: global-address direct-to-LDS kernel, one ring
// of `stages` stages shared by both operands. sb > 0: buffer-addressed
// direct-to-LDS kernel (channel-block order, im2col modes): activations in a
// ring of `stages` stages, filter in a ring of sb.
struct TileShape {
    int bm, bn, wm, wn, mf, stages, kb;
    int sb = 0;
};

// The tiles the planner chooses from (the index is the tile id of the plan
// string and of the conv_debug_force test hook).
enum TileId {
    TILE_DMA_256 = 0,       // global-address, 256x256: large grids the buffer tiles cannot take, point output
    TILE_DMA_128 = 1,       // global-address, 128x128, two workgroups per CU: grids of 64..159 large tiles
    TILE_DMA_64 = 2,        // global-address, 64x64, 4-stage ring: small grids, split reductions
    TILE_DMA_256x192 = 3,   // global-address, 256x192 (bf16): point-output grids that 256x192 fills best
    TILE_BUF = 4,           // buffer-addressed 256x256, activations two steps ahead: temporal filters
    TILE_BUF_AHEAD = 5,     // as TILE_BUF, A fragments read two MFMA rows ahead: bf16 generic path
    TILE_BUF_PINGPONG = 6,  // as TILE_BUF, two wave groups alternating compute and LDS phases: long fp8 reductions
    TILE_PW = 7,            // 1x1x1 filters on NCDHW bf16 activations (conv_pw.hip)
    TILE_BUF_128 = 8,       // buffer-addressed 128x128, two workgroups per CU: grids of about half a round
};
constexpr int kNumTiles = 9;
constexpr bool is_pointwise_tile(int t) { return t == TILE_PW; }
constexpr TileShape kTiles[kNumTiles] = {
    {256, 256, 2, 4, 16, 2, 128},     // 8 waves of 128x64, 2 x 64 KB ring
    {128, 128, 2, 2, 16, 2, 128},     // 4 waves of 64x64, 2 x 32 KB ring
    {64, 64, 2, 2, 16, 4, 128},       // 4 waves of 32x32, 4 x 16 KB ring
    {256, 192, 4, 2, 16, 2, 128},     // 8 waves of 64x96, 2 x 56 KB ring
    {256, 256, 2, 4, 16, 3, 128, 2},  // rings of 3 (activations) and 2 (filter) x 32 KB, loads over 8 of 16 MFMA rows
    {256, 256, 2, 4, 16, 3, 128, 2},
    {256, 256, 2, 4, 16, 3, 128, 2},
    {512, 64, 4, 1, 16, 4, 64},       // 512 positions x 64 output channels, 32-channel steps, 4 x 36 KB
    {128, 128, 2, 2, 16, 3, 128, 2},  // 4 waves of 64x64, rings of 3 + 2 x 16 KB (80 KB: two per CU)
};

// Quotient by a divisor fixed for a launch, with one multiply-high instead of
// an integer division sequence: the round-up method of Granlund and Montgomery
// ("Division by invariant integers using multiplication", PLDI 1994). With
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the 33-bit factor
// f = 2^32 + m satisfies 2^(32+l) < f * d <= 2^(32+l) + d, so for
// 0 <= n < 2^31, n / d = floor(n * f / 2^(32+l)) = (mulhi(n, m) + n) >> l,
// and the sum stays below 2^32.
struct FastDiv {
    unsigned m = 1, l = 0;  // d = 1

    __host__ void set(long long d)
    {
        d = d < 1 ? 1 : d;
        l = 0;
        while ((1ll << l) < d)
            ++l;
        m = (unsigned)((((1ull << l) - (unsigned long long)d) << 32) / (unsigned long long)d + 1);
    }
    __host__ __device__ __attribute__((always_inline)) int div(int n) const
    {
        const unsigned hi = (unsigned)(((unsigned long long)(unsigned)n * m) >> 32);
        return (int)((hi + (unsigned)n) >> l);
    }
};

// Everything a conv kernel needs, passed by value as kernel arguments.
struct ConvParams {
    const void *x;          // activations (NDHWC for im2col modes; rows of the B operand for point mode)
    const void *w;          // packed filter, K rows of ldw elements
    void *y;                // bf16 NCDHW output
    const float *scales;    // fp8: {s_x, inv_x, s_w, inv_w}; null for bf16
    int N, C, D, H, W;
    int K, T, R, S;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int Do, Ho, Wo;
    int P;                  // Do*Ho*Wo
    int M;                  // GEMM rows   (im2col: N*P, point: K)
    int Ncol;               // GEMM cols   (im2col: K,   point: N)
    int Rk;                 // reduction length C*T*R*S
    int ldw;                // packed filter row length (crs_pad)
    int nk;                 // reduction steps
    int tiles_m, tiles_n;   // grid of output tiles
    int group_m;            // grouped raster height (tiles along M sharing an L2 working set)
    // buffer-addressed kernels: byte size of x (any size: each tile rebases its
    // buffer at the first input plane it can read) and of the packed filter (< 2^31)
    int64_t xbytes;
    int wbytes;
    // split reduction (direct-to-LDS kernels): `splits` workgroups per output
    // tile, split j runs reduction steps [j * ksplit, min(nk, (j + 1) * ksplit))
    // and stores its unscaled fp32 sums at part + j * (elements of y), indexed
    // like y; splits == 1: no split, y written directly
    int splits, ksplit;
    float *part;
    // tail split (buffer-addressed kernels): with tail_splits > 1, the tiles
    // from linear index tail_first on (the last, partial round) each run as
    // tail_splits workgroups over contiguous step ranges; workgroup
    // tail_first + t * tail_splits + j stores its unscaled fp32 sums of tile
    // tail_first + t at part + (t * tail_splits + j) * BM * BN, [column][row]
    int tail_first, tail_splits;
    // temporal raster (0 = off): within each block of group_m * tap_stride
    // M-tiles, the group_m tiles a raster group walks together are tap_stride
    // tiles apart (about H*W / BM: one temporal tap), so that each tile's next
    // tap reads the window its neighbour in the group reads at the current one
    int tap_stride;
    // fused epilogue extras (null = off): fp32 bias per output channel added
    // before rounding; max |y| merged into *amax as fp32 bits (zeroed before
    // the launch)
    const float *bias;
    unsigned *amax;
    // divisors of the tile walk and the row decode (with_divisors fills them)
    FastDiv div_P, div_HW, div_Wo;  // P, Ho * Wo, Wo
    FastDiv div_gsz, div_gm;        // group_m * tiles_n, group_m
    FastDiv div_blk;                // group_m * tap_stride (temporal raster block)
};

// p with its divisor fields set from its sizes; every launch of a kernel that
// takes ConvParams passes the result.
inline ConvParams with_divisors(const ConvParams &p)
{
    ConvParams q = p;
    q.div_P.set(p.P);
    q.div_HW.set((long long)p.Ho * p.Wo);
    q.div_Wo.set(p.Wo);
    q.div_gsz.set((long long)p.group_m * p.tiles_n);
    q.div_gm.set(p.group_m);
    q.div_blk.set(p.tap_stride > 0 ? (long long)p.group_m * p.tap_stride : 1);
    return q;
}

// One launch of the implicit-GEMM kernel selected by (tile, mode, dtype,
// 64-bit addressing, channel-block-outer reduction order).
hipError_t launch_conv(const ConvParams &p, int tile, Mode mode, Dtype dt, bool big, bool cblock,
                       hipStream_t stream);
// Reduction step of a tile in bytes of k per row.
constexpr int step_bytes(const TileShape &t) { return t.kb; }
constexpr bool is_buffer(const TileShape &t) { return t.sb > 0; }

// 1x1x1 filter, unit stride, no padding, NCDHW bf16 x: one GEMM per image
// over the D*H*W positions, reading x untransposed (tiles of 256 positions x
// 64 output channels: tiles_m = N * ceil(P / 256), tiles_n = ceil(K / 64)).
hipError_t launch_conv_pw(const ConvParams &p, hipStream_t stream);

// y[i] = bf16(sum over j < splits of part[j * ynum + i], in order j = 0, 1, ...
// times s_x * s_w for fp8 (scales non-null) plus the bias of i's channel),
// ynum = M * Ncol; the amax of y as in the conv epilogues;
// in point-output layout (y[n][k], K per row) channel = i % K, else (i / P) % K
hipError_t launch_splitk_reduce(const ConvParams &p, hipStream_t stream);
hipError_t launch_amax_zero(float *amax, hipStream_t stream);
// Second pass of the tail split: sums each tail tile's partials in split order
// and applies the epilogue (tiles of bm x bn).
hipError_t launch_tail_reduce(const ConvParams &p, int bm, int bn, int ntail, hipStream_t stream);

// dst_a[c][r] = src_a[r][c] and dst_b[c][r] = src_b[r][c] (src rows of cols_a / cols_b bf16, `rows` rows
// each), dst rows of ld >= rows elements (ld a multiple of 64), zero past rows; one launch for both
hipError_t launch_transpose_pad2(const uint16_t *src_a, uint16_t *dst_a, int64_t cols_a, const uint16_t *src_b,
                                 uint16_t *dst_b, int64_t cols_b, int64_t rows, int64_t ld, hipStream_t stream);

// w_t[j][k]: the filter transposed, j in the activation layout's (c, t, r, s) or (t, r, s, c) order
hipError_t launch_pack_w_t(const uint16_t *w, uint16_t *wt, int64_t K, int64_t C, int64_t T, int64_t R, int64_t S,
                           int64_t ldk, bool channel_last, hipStream_t stream);

hipError_t launch_amax(const uint16_t *t, int64_t n, float *amax, hipStream_t stream);
hipError_t launch_fp8_scales(const float *amax, float *pair, hipStream_t stream);
hipError_t launch_pack_x(const uint16_t *x, void *out, int64_t N, int64_t C, int64_t S, Dtype dt,
                         const float *pair, hipStream_t stream);
hipError_t launch_pack_w(const uint16_t *w, void *out, int64_t K, int64_t C, int64_t T, int64_t R, int64_t S,
                         int64_t ldw, bool channel_last, Dtype dt, const float *pair, hipStream_t stream);

}  // namespace igc

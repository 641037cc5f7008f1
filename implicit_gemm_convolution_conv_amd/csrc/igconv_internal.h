// Internal declarations shared by the host library and the kernel translation
// units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace igc {

enum Mode { MODE_GENERIC = 0, MODE_TEMPORAL = 1, MODE_POINT = 2 };
enum Dtype { DT_BF16 = 0, DT_FP8 = 1 };

// Tile shapes: rows x cols of the GEMM tile, waves along rows x cols, MFMA
// block edge (16: 16x16 blocks; 32: 32x32 blocks, which need fewer operand
// registers per lane), LDS stages and bytes of k per row per reduction step
// (kb: 128 = 64 bf16 / 128 fp8, 64 = 32 bf16 / 64 fp8). stages == 0:
// register-staged kernel, two LDS buffers. stages > 0: direct-to-LDS ring of
// that many stages; fp8 with 64-byte steps needs 32x32 blocks.
// stages < 0: input-window kernel: the activations a tile needs for one
// 64-byte channel block sit in LDS once and serve every filter tap; the
// filter streams through a ring of -stages stages (64 bytes of k per step).
// sb > 0: buffer-addressed direct-to-LDS kernel (channel-block order, im2col
// modes): activations in a ring of `stages` stages, filter in a ring of sb.
struct TileShape {
    int bm, bn, wm, wn, mf, stages, kb;
    int sb = 0;
};
constexpr int kNumTiles = 42;
// tiles 35..39: the NCDHW 1x1x1 kernel (conv_pw.hip), chosen by its path only
constexpr int kPointwiseFirst = 35, kPointwiseLast = 39;
constexpr bool is_pointwise_tile(int t) { return t >= kPointwiseFirst && t <= kPointwiseLast; }
constexpr TileShape kTiles[kNumTiles] = {
    {256, 256, 2, 4, 16, 0, 128},  // 8 waves, 128x64 per wave: large grids
    {128, 128, 2, 2, 16, 0, 128},  // 4 waves, 64x64 per wave
    {64, 64, 2, 2, 16, 0, 128},    // 4 waves, 32x32 per wave: small grids
    {256, 256, 2, 4, 32, 0, 128},
    {128, 128, 2, 2, 32, 0, 128},
    {64, 64, 2, 2, 32, 0, 128},
    {256, 256, 2, 4, 16, 4, 64},   // direct-to-LDS, 4 x 32 KB ring
    {256, 256, 2, 4, 32, 4, 64},
    {128, 128, 2, 2, 16, 4, 64},   // direct-to-LDS, 4 x 16 KB ring
    {128, 128, 2, 2, 32, 4, 64},
    {128, 128, 2, 2, 16, 8, 64},   // direct-to-LDS, 8 x 16 KB ring: latency-bound short reductions
    {64, 64, 2, 2, 16, 4, 64},     // direct-to-LDS, 4 x 8 KB ring, many blocks per CU
    {128, 128, 2, 2, 32, 8, 64},
    {64, 64, 2, 2, 32, 4, 64},
    {256, 256, 2, 2, 16, 4, 64},   // direct-to-LDS, 4 waves of 128x128 (256 accumulators per lane)
    {256, 256, 2, 2, 32, 4, 64},
    {256, 256, 2, 4, 16, -4, 64},  // input window in LDS + 4-stage filter ring (full 3D filters)
    {256, 256, 2, 4, 32, -4, 64},
    {256, 128, 2, 2, 16, 3, 64},   // direct-to-LDS, 3 x 24 KB ring: two workgroups per CU
    {256, 128, 2, 2, 32, 3, 64},
    {128, 256, 2, 2, 16, 3, 64},
    {256, 256, 2, 4, 16, 2, 128},  // direct-to-LDS, 2 x 64 KB ring, 128-byte steps
    {256, 256, 2, 4, 32, 2, 128},
    {128, 128, 2, 2, 16, 4, 128},  // direct-to-LDS, 4 x 32 KB ring, 128-byte steps: short reductions
    {128, 128, 2, 2, 16, 2, 128},  // two workgroups per CU
    {256, 128, 2, 4, 16, 2, 128},
    {64, 64, 2, 2, 16, 4, 128},    // small grids
    {256, 256, 2, 4, 16, 2, 128, 2},  // buffer-addressed: rings of 2 x 32 KB, loads over 8 of 16 MFMA rows
    {256, 256, 2, 4, 16, 2, 128, 3},  // filter ring 3 x 32 KB (issued two steps ahead)
    {256, 256, 2, 4, 16, 3, 128, 2},  // activation ring 3 x 32 KB (two steps ahead): large-grid default
    {256, 256, 2, 4, 16, 3, 128, 2},  // as 29, loads over all 16 MFMA rows (bf16 only)
    {256, 256, 2, 4, 16, 3, 128, 2},  // as 29, A fragments two rows ahead, next k-slice's B read early
    {256, 256, 2, 4, 16, 3, 64, 5},   // 64-byte steps: rings of 3 and 5 x 16 KB (bf16 only)
    {256, 256, 2, 4, 16, 3, 128, 2},  // as 29, ping-pong wave groups (compute / memory phases)
    {256, 256, 2, 4, 16, 2, 128, 2},  // as 33, activation windows shared by the S taps of a filter row
    {256, 64, 4, 1, 16, 3, 128},      // 1x1x1 on NCDHW x: 256 positions x 64 output channels, 64-channel steps
    {256, 64, 4, 1, 16, 2, 128},      // 2 stages of 40 KB: two workgroups per CU
    {512, 64, 4, 1, 16, 4, 64},       // 512 positions (1 KB per channel row), 32-channel steps, 4 x 36 KB
    {512, 64, 4, 1, 16, 2, 64},       // two workgroups per CU
    {256, 64, 4, 1, 16, 4, 64},       // 256 positions, 32-channel steps, 4 x 20 KB: two workgroups per CU
    {256, 192, 2, 4, 16, 2, 128},     // direct-to-LDS, 2 x 56 KB ring: grids of 192..256 tiles of 256x256
    {256, 256, 2, 4, 16, 3, 128, 2},  // as 29, persistent: one workgroup per CU walks its tiles as one step stream
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
    int pairs;              // direct-to-LDS channel-block order: reduction steps per 128-byte line (1 or 2)
    // input-window kernel: tiles never cross an output plane (n, od)
    int tpp;                // M tiles per output plane = ceil(Ho*Wo / BM)
    int win_h, win_w;       // window rows / columns (input pixels) per plane slot
    int win_nwi;            // window DMA instructions per thread per channel block
    // buffer-addressed kernels: byte size of x (any size: each tile rebases its
    // buffer at the first input plane it can read) and of the packed filter (< 2^31)
    int64_t xbytes;
    int wbytes;
    // tap-shared activation windows: input pixels per output row, rows per window
    int win_cols, win_rows;
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
};

// One launch of the implicit-GEMM kernel selected by (tile, mode, dtype,
// 64-bit addressing, channel-block-outer reduction order).
hipError_t launch_conv(const ConvParams &p, int tile, Mode mode, Dtype dt, bool big, bool cblock,
                       hipStream_t stream);
// Reduction step of a tile in bytes of k per row.
constexpr int step_bytes(const TileShape &t) { return t.kb; }
constexpr bool is_window(const TileShape &t) { return t.stages < 0; }
constexpr bool is_buffer(const TileShape &t) { return t.sb > 0; }

// 1x1x1 filter, unit stride, no padding, NCDHW bf16 x: one GEMM per image
// over the D*H*W positions, reading x untransposed (tiles of 256 positions x
// 64 output channels: tiles_m = N * ceil(P / 256), tiles_n = ceil(K / 64)).
hipError_t launch_conv_pw(const ConvParams &p, int variant, hipStream_t stream);

// y[i] = bf16(sum over j < splits of part[j * ynum + i], in order j = 0, 1, ...
// times s_x * s_w for fp8 (scales non-null) plus the bias of i's channel),
// ynum = M * Ncol; the amax of y as in the conv epilogues;
// in point-output layout (y[n][k], K per row) channel = i % K, else (i / P) % K
hipError_t launch_splitk_reduce(const ConvParams &p, hipStream_t stream);
hipError_t launch_amax_zero(float *amax, hipStream_t stream);
// Second pass of the tail split: sums each tail tile's partials in split order
// and applies the epilogue (tiles of bm x bn).
hipError_t launch_tail_reduce(const ConvParams &p, int bm, int bn, int ntail, hipStream_t stream);

// dst[c][r] = src[r][c] (src rows of `cols` bf16), dst rows of ld >= rows elements, zero past rows
hipError_t launch_transpose_pad(const uint16_t *src, uint16_t *dst, int64_t rows, int64_t cols, int64_t ld,
                                hipStream_t stream);
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

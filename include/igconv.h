/*
 * igconv -- forward implicit-GEMM convolution for MI355X (gfx950), C ABI.
 *
 * What is computed. conv_fwd evaluates 3D forward convolution (a
 * cross-correlation with zero padding, stride and dilation; 2D and 1D are the
 * D = T = 1 and H = R = 1 special cases) as one implicit GEMM: rows
 * M = N*Do*Ho*Wo output positions, columns = K output channels, reduction
 * C*T*R*S over channel and filter tap, as described for the bf16 and fp8
 * conv3d kernels of FlyDSL PR #860 ("[Kernel] fp8 conv3d: 8-wave GEMM
 * pipeline + BIG_IN fix", PR summary and the commits on the async
 * global->LDS pipeline, the temporal-only 3x1x1 decode, the vec4 epilogue
 * and the large-tensor rebase). Point-output shapes (stride equal to the
 * filter, zero padding, unit dilation, input extent equal to the filter
 * extent, hence a 1x1x1 output) are one plain GEMM over the batch with no
 * im2col, as in MIOpen PR #10912 (PR body; channel-last is valid because a
 * batch slice of x and a row of w enumerate C*T*R*S in the same order).
 *
 *   y[n,k,od,oh,ow] = sum_{c,t,r,s} x[n,c,od*sd-pd+t*dd, oh*sh-ph+r*dh,
 *                                      ow*sw-pw+s*dw] * w[k,c,t,r,s]
 *   Do = (D + 2*pd - dd*(T-1) - 1)/sd + 1   (likewise Ho, Wo)
 *
 * Arithmetic: bf16 operands, or fp8 E4M3FN operands with one fp32 scale per
 * tensor (s = amax/448); fp32 accumulation; y is bf16 (round to nearest even)
 * of acc, or of acc * (s_x * s_w) for fp8.
 *
 * Conventions for every entry point:
 *  - Shapes are plain arrays: xshape = {N, C, D, H, W} (logical, whatever the
 *    memory layout), wshape = {K, C, T, R, S}; stride, pad, dilation =
 *    {d, h, w}. 2D callers pass D = T = 1, pad_d = 0; 1D also H = R = 1.
 *  - Every pointer argument named *_dev or a tensor (x, w, y, ...) is DEVICE
 *    memory owned by the caller; the library allocates nothing, keeps no
 *    pointer after the call returns, never synchronises and enqueues all work
 *    on `stream` (a hipStream_t; NULL = the null stream) in call order.
 *  - Tensors must be contiguous in the stated layout and 16-byte aligned.
 *  - Return value: IGC_OK, or a negative status. All validation runs before any
 *    GPU work: on error nothing is enqueued and conv_last_error() describes the
 *    reason. IGC_ERR_HIP reports a failed kernel launch. No C++ exception
 *    crosses this interface. All entry points are thread-safe; the error text
 *    is per thread, and so are the settings of the conv_debug_force* test
 *    hooks (a forced plan applies to the calls of the thread that set it).
 */
#ifndef IGCONV_H
#define IGCONV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define IGC_API __attribute__((visibility("default")))
#else
#define IGC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* status */
#define IGC_OK 0
#define IGC_ERR_INVALID (-1)     /* bad pointer, shape or argument */
#define IGC_ERR_UNSUPPORTED (-2) /* valid convolution this library does not run */
#define IGC_ERR_ALIGN (-3)       /* pointer not 16-byte aligned */
#define IGC_ERR_HIP (-4)         /* HIP runtime error while enqueuing */

/* operand type (dtype) */
#define IGC_BF16 0
#define IGC_FP8_E4M3FN 1

/* activation memory layout (x_layout) */
#define IGC_NCDHW 0
#define IGC_NDHWC 1

/* tile ids reported by conv_plan ("tile_id=") / forced by conv_debug_force */
#define IGC_TILE_AUTO (-1)
#define IGC_TILE_DMA_256 0       /* global-address direct-to-LDS 256x256: grids the buffer tiles cannot take */
#define IGC_TILE_DMA_128 1       /* global-address direct-to-LDS 128x128, two workgroups per CU */
#define IGC_TILE_DMA_64 2        /* global-address direct-to-LDS 64x64, 4-stage ring: small grids */
#define IGC_TILE_DMA_256x192 3   /* global-address direct-to-LDS 256x192 (bf16): point-output grids */
#define IGC_TILE_BUF 4           /* buffer-addressed 256x256, lockstep waves: temporal filters */
#define IGC_TILE_BUF_AHEAD 5     /* as IGC_TILE_BUF, fragments read further ahead: bf16 generic filters */
#define IGC_TILE_BUF_PINGPONG 6  /* as IGC_TILE_BUF, two wave groups in compute / LDS phases: long fp8 reductions */
#define IGC_TILE_PW 7            /* 1x1x1 filter on NCDHW bf16 activations */
#define IGC_TILE_BUF_128 8       /* buffer-addressed 128x128, two workgroups per CU: grids of about half a round */

/* execution path reported by conv_plan / forced by conv_debug_force */
#define IGC_PATH_AUTO 0
#define IGC_PATH_GENERIC 1  /* im2col decode of every tap */
#define IGC_PATH_TEMPORAL 2 /* T x 1 x 1 filter: one bounds check per row (time axis only) */
#define IGC_PATH_POINT 3    /* point output: plain GEMM over the batch */
#define IGC_PATH_POINTWISE 4 /* 1x1x1 filter on NCDHW bf16 activations: per-image GEMM, no transpose */

/*
 * Output extent {Do, Ho, Wo} by the formula above. Host only.
 * IGC_ERR_INVALID when a size is non-positive, C differs between x and w, a
 * stride or dilation is < 1, a pad is < 0, or the filter does not fit.
 */
IGC_API int conv_out_dims(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3],
                  const int32_t pad[3], const int32_t dilation[3], int64_t out_dhw[3]);

/*
 * Row length (elements) of the packed filter that conv_pack_w writes and
 * conv_fwd reads: C*T*R*S rounded up to the reduction step (64 elements for
 * bf16, 128 for fp8), the zero-padded "crs_pad" of FlyDSL PR #860 (commit
 * generalising the 8-wave fp8 kernel to N-/K-partial and tiny-K shapes).
 * The packed filter is K rows of this length. Host only. <= 0 on bad input.
 */
IGC_API int64_t conv_packed_w_cols(const int64_t wshape[5], int dtype);

/*
 * amax_dev[0] = max |t[i]| over `numel` bf16 values (exact; a NaN input makes
 * it NaN). amax_dev: one device float, overwritten. numel >= 1.
 * The per-tensor fp8 scale of each operand is derived from this maximum.
 */
IGC_API int conv_amax(const void *t_bf16, int64_t numel, float *amax_dev, void *stream);

/*
 * scale_pair_dev[0..1] = {s, inv} = {amax/448, 448/amax}, each a correctly
 * rounded fp32 division of amax_dev[0]; {1, 1} when amax is 0.
 * 448 is the largest finite E4M3FN value (FlyDSL PR #860 runs its fp8 kernel
 * on E4M3FN operands, PR summary).
 */
IGC_API int conv_fp8_scales(const float *amax_dev, float *scale_pair_dev, void *stream);

/*
 * Activation pack: x (bf16, NCDHW) -> x_out in NDHWC, as bf16 (a pure
 * transpose, bit-exact) or as fp8 E4M3FN codes q = E4M3FN(fp32(v * inv)),
 * round to nearest even, saturating at +-448, inv = scale_pair_dev[1].
 * This is the NCDHW->NDHWC transpose and the bf16->fp8 pack that FlyDSL
 * PR #860 runs before its conv kernels (large-tensor rebase commit; the fp8
 * kernel's tiled transpose). Requires C % 8 == 0 (bf16) or C % 16 == 0 (fp8).
 * scale_pair_dev is ignored (may be NULL) for bf16. x and x_out must not
 * overlap. Tensors above 2^31 elements are supported.
 */
IGC_API int conv_pack_x(const void *x_ncdhw_bf16, void *x_out, const int64_t xshape[5], int dtype,
                const float *scale_pair_dev, void *stream);

/*
 * Filter pack: w (bf16, KCTRS) -> w_packed, K rows of conv_packed_w_cols()
 * elements, columns zero-filled past C*T*R*S. Column order follows the
 * activation layout conv_fwd will see: (t, r, s, c) with c fastest for
 * x_layout = IGC_NDHWC, (c, t, r, s) for IGC_NCDHW (point-output only).
 * fp8: codes of fp32(w * inv), inv = scale_pair_dev[1], as in conv_pack_x.
 */
IGC_API int conv_pack_w(const void *w_kctrs_bf16, void *w_packed, const int64_t wshape[5], int dtype, int x_layout,
                const float *scale_pair_dev, void *stream);

/*
 * Forward convolution y = conv(x, w).
 *  x        activations, dtype operands, layout x_layout. The im2col paths
 *           (generic, temporal) need IGC_NDHWC with C % 8 == 0 (bf16) or
 *           C % 16 == 0 (fp8); the point-output path takes either layout.
 *           A 1x1x1 filter with unit stride and no padding on IGC_NCDHW bf16
 *           activations with D*H*W % 8 == 0 runs as one GEMM per image that
 *           reads x as it is (IGC_PATH_POINTWISE): the route FlyDSL PR #860
 *           takes for 1x1x1 filters to avoid the NCDHW->NDHWC transpose
 *           (PR description, "Performance"). w_packed then comes from
 *           conv_pack_w with x_layout = IGC_NCDHW.
 *  w_packed filter from conv_pack_w with the same dtype and x_layout.
 *  y        bf16 output, NCDHW {N, K, Do, Ho, Wo}; every element is written.
 *  scales_dev  fp8 only: device float[4] = {s_x, inv_x, s_w, inv_w} (the two
 *           conv_fp8_scales pairs); y = bf16(acc * (s_x * s_w)). NULL for bf16.
 * y must not overlap x or w_packed. Output rows M = N*Do*Ho*Wo must be
 * < 2^31; x and y above 2^31 elements are supported (32-bit buffer windows
 * rebased per output tile while a tile's reach stays below 2^31 bytes,
 * 64-bit offsets beyond). Returns IGC_ERR_UNSUPPORTED for a shape no path
 * accepts (the message says which requirement failed).
 */
IGC_API int conv_fwd(const void *x, const void *w_packed, void *y, const int64_t xshape[5], const int64_t wshape[5],
             const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout,
             const float *scales_dev, void *stream);

/*
 * Forward convolution with a caller-provided device workspace, for output-tile
 * grids too small to occupy the GPU (few output positions and channels, long
 * reductions). Same arguments, layouts, result and errors as conv_fwd, plus:
 *  workspace_dev    device memory owned by the caller, 16-byte aligned, or
 *                   NULL (then workspace_bytes must be 0); only read and
 *                   written by work enqueued on `stream` by this call.
 *  workspace_bytes  its size. When the plan splits the reduction (split-K)
 *                   into `splits` ranges, each range's fp32 sums take
 *                   4 * N*K*Do*Ho*Wo bytes; the split count is lowered to what
 *                   fits, and with room for fewer than two ranges the call
 *                   runs exactly as conv_fwd.
 * A split run enqueues two kernels: the conv kernel (one workgroup per tile
 * and range, unscaled fp32 sums into the workspace) and a pass that adds the
 * ranges in a fixed order, scales (fp8) and rounds to bf16 into y. Results
 * are deterministic but may differ from conv_fwd's in the last bit (another
 * summation order). The split is chosen only where the grid of output tiles
 * under-fills the GPU, as FlyDSL PR #860's split-K selection does (its rule
 * that the under-fill test alone decides).
 * Tail split: on the 256x256 buffer-addressed tiles, when the grid's last
 * round of tiles fills at most half of the GPU's 256 CUs, each of its r tiles
 * runs as S workgroups over 1/S of the reduction (S = 256 / r, 2..8), using
 * r * S * 256 * 256 * 4 bytes of workspace, and a second pass adds them in a
 * fixed order for those tiles only; every other tile is computed and stored
 * as by conv_fwd. Without that much room the call runs exactly as conv_fwd.
 */
IGC_API int conv_fwd_ws(const void *x, const void *w_packed, void *y, const int64_t xshape[5],
                const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3],
                int dtype, int x_layout, const float *scales_dev, void *workspace_dev, size_t workspace_bytes,
                void *stream);

/*
 * Forward convolution with fused epilogue extras; otherwise as conv_fwd_ws
 * (workspace_dev NULL and workspace_bytes 0: as conv_fwd).
 *  bias_dev    NULL, or device fp32[K]: y = bf16(acc * (s_x * s_w) + bias[k])
 *              (bf16: bf16(acc + bias[k])), the bias added in fp32 before the
 *              one rounding. FlyDSL PR #860 tests its fp8 conv with a bias
 *              (PR summary, the gemm8w test cases).
 *  y_amax_dev  NULL, or device fp32[1]: receives max |y| over the bf16 values
 *              written to y (the per-tensor amax conv_amax would compute on
 *              y, as the input of a next fp8 convolution's conv_fp8_scales),
 *              without a second pass over y. It is cleared on `stream` first.
 * Both must be 4-byte aligned. The amax is merged with atomic maxima of
 * fp32 bit patterns: calls that share y_amax_dev must not overlap.
 */
IGC_API int conv_fwd_ex(const void *x, const void *w_packed, void *y, const int64_t xshape[5],
                const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3],
                int dtype, int x_layout, const float *scales_dev, const float *bias_dev, float *y_amax_dev,
                void *workspace_dev, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): conv_fwd_ex
 * with its workspace taken from a static device array of the library instead
 * of the caller. Same arguments, layouts, plan, result and errors as
 * conv_fwd_ex with a workspace of conv_fwd_workspace_bytes bytes (bit for bit
 * the same output), without the workspace arguments. Allocates nothing: the
 * scratch is a 64 MiB `__device__` array, one per GPU the library runs on,
 * held until the process ends; its device address is looked up once per
 * device (the current one) on the first call that needs it.
 * Limit: a plan whose workspace exceeds 64 MiB returns IGC_ERR_UNSUPPORTED
 * before any work is enqueued (automatic plans need at most 64 MiB on a
 * 256-CU device; a forced split can need more). The scratch keeps the last
 * call's partial sums and needs no clearing (every value is written before
 * it is read). Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * ordered by the caller.
 */
IGC_API int conv_fwd_noalloc(const void *x, const void *w_packed, void *y, const int64_t xshape[5],
                const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3],
                int dtype, int x_layout, const float *scales_dev, const float *bias_dev, float *y_amax_dev,
                void *stream);

/*
 * Workspace bytes conv_fwd_ws would use for these arguments with unlimited
 * room: splits * 4 * N*K*Do*Ho*Wo when it splits the reduction, r * S * 256 *
 * 256 * 4 for a tail split, else 0.
 * Negative status (as conv_fwd) for invalid arguments. Host only.
 */
IGC_API int64_t conv_fwd_workspace_bytes(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3],
                const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout);

/*
 * Gradients of point-output convolutions (input extent equal to the filter
 * extent, no padding, unit dilation: one output position per image), each one
 * GEMM over the batch as in MIOpen PR #10912 (PR body: backward data and
 * backward weights for patch-embedding shapes). bf16 operands, fp32
 * accumulation, one bf16 rounding. An image of x (and of dx) is then the
 * C*T*R*S elements in the layout's order: (c, t, r, s) for IGC_NCDHW, (t, r,
 * s, c) for IGC_NDHWC; dy is {N, K, 1, 1, 1}, i.e. [N][K]. Other geometries
 * return IGC_ERR_UNSUPPORTED, fp8 too.
 *
 * conv_packed_w_t_cols: row length of the transposed filter, K rounded up to 64.
 * conv_pack_w_t: w_t[j][k] = w[k][c][t][r][s] for the backward-data GEMM, j in
 *   x_layout's element order, rows of conv_packed_w_t_cols elements with zeros
 *   from K on (a one-time, per-filter preparation).
 * conv_bwd_data: dx[n][j] = sum_k dy[n][k] * w[k][j]; dx has x's shape and
 *   layout, every element written. Needs K even (4-byte aligned dy rows).
 * conv_bwd_weight: dw[k][j] = sum_n dy[n][k] * x[n][j], written as bf16 in
 *   filter order: KCTRS for IGC_NCDHW, K x (T, R, S, C) for IGC_NDHWC. The
 *   reduction runs over n, the slow index of x and dy, so both are first
 *   transposed into the workspace (x^T and dy^T, rows padded to a multiple of
 *   64 images with zeros); where the grid of output tiles under-fills the GPU
 *   the batch is also split as in conv_fwd_ws, fp32 slices in the workspace.
 *   The workspace must hold at least the two transposes; the split count is
 *   lowered to what the rest holds.
 * conv_bwd_weight_workspace_bytes: the bytes conv_bwd_weight uses with
 *   unlimited room (negative status for invalid arguments). Host only.
 */
IGC_API int64_t conv_packed_w_t_cols(const int64_t wshape[5]);
IGC_API int conv_pack_w_t(const void *w_kctrs_bf16, void *w_t, const int64_t wshape[5], int x_layout, void *stream);
IGC_API int conv_bwd_data(const void *dy, const void *w_t, void *dx, const int64_t xshape[5],
                const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3],
                int dtype, int x_layout, void *stream);
IGC_API int64_t conv_bwd_weight_workspace_bytes(const int64_t xshape[5], const int64_t wshape[5],
                const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout);
IGC_API int conv_bwd_weight(const void *x, const void *dy, void *dw, const int64_t xshape[5],
                const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3],
                int dtype, int x_layout, void *workspace_dev, size_t workspace_bytes, void *stream);

/*
 * Describe, without running anything, the path and tile conv_fwd would use
 * for these arguments: writes a one-line text such as
 * "path=generic tile_id=5 tile=256x256 waves=8 ... order=cblock big=0 grid=6752 ..."
 * into buf (NUL-terminated, truncated to len). Same validation and return
 * codes as conv_fwd. Host only.
 */
IGC_API int conv_plan(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3],
              const int32_t dilation[3], int dtype, int x_layout, char *buf, size_t len);

/* As conv_plan, for conv_fwd_ws with a workspace of workspace_bytes (the text
 * ends with the split count, reduction steps per split and "tail=r/S": the
 * tail tiles and their splits, 0/1 without a tail split). Host only. */
IGC_API int conv_plan_ws(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3],
                 const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout, size_t workspace_bytes,
                 char *buf, size_t len);

/*
 * Test hooks. Each setting is per thread (it applies to the later conv_fwd*,
 * conv_plan* and workspace-size calls of the calling thread only) and stays
 * until that thread changes it. They exist for tests and tuning runs, not for
 * production callers.
 *
 * conv_debug_force: force the path (IGC_PATH_*), the tile (IGC_TILE_*, -1 =
 * automatic) and the grouped-raster height in tiles (0 = automatic). A forced
 * path or tile that does not apply to a shape makes conv_fwd return
 * IGC_ERR_UNSUPPORTED.
 */
IGC_API int conv_debug_force(int path, int tile, int group_m);

/* Test hook: force the split count of conv_fwd_ws / conv_plan_ws (0 =
 * automatic, 1 = never split; more is capped by the reduction steps and the
 * workspace). A split on a tile that cannot split returns IGC_ERR_UNSUPPORTED. */
IGC_API int conv_debug_force_splits(int splits);

/* Test hook: plan as if the device had `cus` compute units (0 = the device's
 * own count), so that small problems have a partial last round of 256x256
 * tiles for conv_fwd_ws to split. */
IGC_API int conv_debug_force_grid(int cus);

/* Test and tuning hook: -1 turns the temporal raster off (raster groups of
 * consecutive M tiles on temporal filters too), 0 restores the automatic
 * choice (groups of tiles one temporal tap apart). */
IGC_API int conv_debug_force_tap_raster(int mode);

/* Text of the last error on this thread ("" if none). Valid until the next call. */
IGC_API const char *conv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IGCONV_H */

// C-ABI entry points: validation, path and tile selection, launch.
//
// Nothing here allocates device memory or synchronises; every launch goes to
// the caller's stream. Validation finishes before the first launch, so an
// error return leaves the stream untouched.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <cstdlib>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "igconv.h"
#include "igconv_internal.h"
#include "tile_table.h"

namespace igc {
hipError_t launch_conv_dma_bf16(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream);
hipError_t launch_conv_dma_fp8(const ConvParams &p, int tile, Mode mode, bool big, bool cblock, hipStream_t stream);

hipError_t launch_conv_buf_bf16(const ConvParams &p, int tile, Mode mode, hipStream_t stream);
hipError_t launch_conv_buf_fp8(const ConvParams &p, int tile, Mode mode, hipStream_t stream);

hipError_t launch_conv(const ConvParams &plan, int tile, Mode mode, Dtype dt, bool big, bool cblock,
                       hipStream_t stream)
{
    const ConvParams p = with_divisors(plan);
    if (is_pointwise_tile(tile))
        return launch_conv_pw(p, stream);
    if (is_buffer(kTiles[tile]))
        return dt == DT_FP8 ? launch_conv_buf_fp8(p, tile, mode, stream) : launch_conv_buf_bf16(p, tile, mode, stream);
    return dt == DT_FP8 ? launch_conv_dma_fp8(p, tile, mode, big, cblock, stream)
                        : launch_conv_dma_bf16(p, tile, mode, big, cblock, stream);
}
}  // namespace igc

namespace {

using namespace igc;

thread_local std::string g_err;
// Test hooks (conv_debug_force*): per thread, so that forcing a plan in one
// thread never changes the plans of calls made by another.
thread_local int g_force_path = IGC_PATH_AUTO;
thread_local int g_force_tile = -1;
thread_local int g_force_group_m = 0;
thread_local int g_force_splits = 0;
thread_local int g_force_cus = 0;
thread_local int g_force_tap_raster = 0;

constexpr int64_t kI32Max = 2147483647;

// Compute units of the current device: the workgroups of 256x256 tiles (one
// per CU, their rings fill its LDS) that run at once. Queried once per device;
// 256, an MI355X's count, where no device answers (host-only planning calls on
// a machine without one). conv_debug_force_grid stands in another count.
int64_t device_cus()
{
    if (g_force_cus > 0)
        return g_force_cus;
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0)
        return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}
// Element offsets up to this bound use 32-bit arithmetic in the conv kernel;
// larger tensors switch to 64-bit offsets (invalid im2col taps may compute an
// offset up to one tensor beyond the valid range before being masked).
constexpr int64_t kSmallTensor = int64_t(1) << 30;

// Device scratch of conv_fwd_noalloc, one copy per GPU, held until the process
// ends. 64 MiB is the largest workspace an automatic plan asks for on a
// 256-CU device: a split-K grid fills at most one round of 256x256 fp32 tiles
// (256 x 256 KB), and a tail split at most r * S <= 256 of them.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per device
// (the current one) and kept: host code passes this pointer, never the
// array's name, which on the host is only a stand-in for the symbol. Null if
// the lookup fails.
void *scratch_ptr()
{
    static std::mutex mu;
    static void *ptrs[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return IGC_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Geometry {
    int64_t N, C, D, H, W, K, T, R, S;
    int64_t sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int64_t Do, Ho, Wo;
};

int check_geometry(const int64_t *xs, const int64_t *ws, const int32_t *st, const int32_t *pad,
                   const int32_t *dil, Geometry &g)
{
    if (!xs || !ws || !st || !pad || !dil)
        return fail(IGC_ERR_INVALID, "null shape/stride/pad/dilation array");
    g.N = xs[0]; g.C = xs[1]; g.D = xs[2]; g.H = xs[3]; g.W = xs[4];
    g.K = ws[0]; g.T = ws[2]; g.R = ws[3]; g.S = ws[4];
    for (int i = 0; i < 5; ++i) {
        if (xs[i] < 1 || xs[i] > kI32Max)
            return fail(IGC_ERR_INVALID, "xshape[%d] = %lld must be in [1, 2^31)", i, (long long)xs[i]);
        if (ws[i] < 1 || ws[i] > kI32Max)
            return fail(IGC_ERR_INVALID, "wshape[%d] = %lld must be in [1, 2^31)", i, (long long)ws[i]);
    }
    if (ws[1] != xs[1])
        return fail(IGC_ERR_INVALID, "channel mismatch: x has C=%lld, w has C=%lld", (long long)xs[1],
                    (long long)ws[1]);
    for (int i = 0; i < 3; ++i) {
        if (st[i] < 1)
            return fail(IGC_ERR_INVALID, "stride[%d] = %d must be >= 1", i, st[i]);
        if (dil[i] < 1)
            return fail(IGC_ERR_INVALID, "dilation[%d] = %d must be >= 1", i, dil[i]);
        if (pad[i] < 0)
            return fail(IGC_ERR_INVALID, "pad[%d] = %d must be >= 0", i, pad[i]);
    }
    g.sd = st[0]; g.sh = st[1]; g.sw = st[2];
    g.pd = pad[0]; g.ph = pad[1]; g.pw = pad[2];
    g.dd = dil[0]; g.dh = dil[1]; g.dw = dil[2];
    const int64_t ed = g.D + 2 * g.pd - g.dd * (g.T - 1) - 1;
    const int64_t eh = g.H + 2 * g.ph - g.dh * (g.R - 1) - 1;
    const int64_t ew = g.W + 2 * g.pw - g.dw * (g.S - 1) - 1;
    if (ed < 0 || eh < 0 || ew < 0)
        return fail(IGC_ERR_INVALID, "filter (dilated) does not fit the padded input");
    g.Do = ed / g.sd + 1;
    g.Ho = eh / g.sh + 1;
    g.Wo = ew / g.sw + 1;
    return IGC_OK;
}

// Upper bound on the bytes between a tile's x base (the first input plane its
// first row can read, see tile_x_base) and the end of the last input plane any
// of its 256 rows can read.
int64_t buffer_x_span(const Geometry &g, int esz)
{
    const int64_t plane = g.H * g.W * g.C * esz;
    const int64_t hw = g.Ho * g.Wo;
    const int64_t k = 255 / hw + 2;                          // output planes past the first one
    int64_t planes = k * g.sd + (g.T - 1) * g.dd + 1;        // tile inside one image
    if (g.N > 1) {
        const int64_t P = g.Do * hw;
        if (P <= 256 + 2 * hw)                               // a tile can hold whole images
            planes = std::max(planes, (256 / P + 3) * g.D);
        else                                                 // the tail of one image, the head of the next
            planes = std::max(planes, g.D - std::min(g.D - 1, std::max<int64_t>(0, (g.Do - 1 - k) * g.sd - g.pd)) +
                                          std::min(g.D, k * g.sd + (g.T - 1) * g.dd + 1));
    }
    return planes * plane;
}

int64_t packed_cols(int64_t rk, int dtype) { return (rk + (dtype == IGC_FP8_E4M3FN ? 127 : 63)) / (dtype == IGC_FP8_E4M3FN ? 128 : 64) * (dtype == IGC_FP8_E4M3FN ? 128 : 64); }

struct Plan {
    int path;  // IGC_PATH_*
    int tile;
    bool big, cblock;
    int64_t xspan;  // bound on a tile's reach into x from its buffer base
    int64_t ws_need = 0;  // workspace bytes the planned split uses (split reduction or tail split)
    ConvParams p;
};

// Point output (MIOpen PR #10912): stride irrelevant once the input extent
// equals the filter extent with no padding and unit dilation -- one output
// position per image, a plain GEMM over the batch.
bool is_point(const Geometry &g)
{
    return g.pd == 0 && g.ph == 0 && g.pw == 0 && g.dd == 1 && g.dh == 1 && g.dw == 1 && g.D == g.T &&
           g.H == g.R && g.W == g.S;
}

// 1x1x1 filter with unit stride and no padding (dilation is irrelevant): y of
// image n is W (K x C) times x_n (C x D*H*W), so NCDHW activations need no
// transpose (FlyDSL PR #860 sends this shape to a plain matmul for that reason,
// PR description "Performance").
bool is_pointwise(const Geometry &g)
{
    return g.T == 1 && g.R == 1 && g.S == 1 && g.sd == 1 && g.sh == 1 && g.sw == 1 && g.pd == 0 && g.ph == 0 &&
           g.pw == 0;
}

// Temporal-only filter (FlyDSL PR #860, 3x1x1 fast decode): the (h, w) index
// of an output position is its input index, only the time axis has taps.
bool is_temporal(const Geometry &g)
{
    return g.R == 1 && g.S == 1 && g.ph == 0 && g.pw == 0 && g.sh == 1 && g.sw == 1;
}

// Tile of a point-output GEMM (forward point path and the backward GEMMs): one
// round of tiles on the GPU is what these grids take, so the tile shape that
// fills the round best wins, among 256x256, 256x192 (bf16) and 128x128 (two
// per CU); grids too small for 128x128 tiles take 64x64 as elsewhere.
// Measured on MI355X with the 9500-image patch embed: forward (1280 x 9500
// over 588) 256x192 27.7 us, 256x256 33.5 us, 128x128 34 us; backward data
// (588 x 9500 over 1280) 128x128 27.8 us, 256x192 38 us, 256x256 46.6 us.
int point_tile(int64_t M, int64_t Ncol, bool bf16)
{
    auto nblocks = [&](int t) {
        return (M + kTiles[t].bm - 1) / kTiles[t].bm * ((Ncol + kTiles[t].bn - 1) / kTiles[t].bn);
    };
    const int64_t cus = device_cus();
    if (nblocks(TILE_DMA_256) >= 2 * cus)
        return TILE_DMA_256;
    if (nblocks(TILE_DMA_256) < cus * 5 / 8 && nblocks(TILE_DMA_128) < cus)
        return TILE_DMA_64;
    int best = TILE_DMA_256;
    double best_fill = 0.0;
    for (int t : {TILE_DMA_256, TILE_DMA_256x192, TILE_DMA_128}) {
        if (t == TILE_DMA_256x192 && !bf16)
            continue;
        const int64_t slots = kTiles[t].bm * kTiles[t].bn > 128 * 128 ? cus : 2 * cus;  // resident workgroups
        const int64_t n = nblocks(t), rounds = (n + slots - 1) / slots;
        const double fill = (double)n / (double)(rounds * slots);
        if (fill > best_fill + 1e-9) {
            best = t;
            best_fill = fill;
        }
    }
    return best;
}

// Nearest swept shape (tile_table.h) of the same element size and path: distance |log2| of the ratio of
// 256x256 tiles per CU plus |log2| of the ratio of 128-byte reduction steps, at most kSweptReach. Returns
// its fastest tile if runs(tile), else its runner-up if runs(it), else -1.
template <typename Runs>
int swept_tile(int esz, int path, double tiles_per_cu, int64_t steps, Runs &&runs)
{
    const SweptShape *best = nullptr;
    double bd = 0.0;
    for (int i = 0; i < kNumSwept; ++i) {
        const SweptShape &e = kSwept[i];
        if (e.esz != esz || e.path != path)
            continue;
        const double d = std::fabs(std::log2(std::max(tiles_per_cu, 1e-6) / e.tiles_per_cu)) +
                         std::fabs(std::log2((double)std::max<int64_t>(steps, 1) / e.steps));
        if (!best || d < bd) {
            best = &e;
            bd = d;
        }
    }
    if (!best || bd > kSweptReach)
        return -1;
    if (runs(best->tile))
        return best->tile;
    if (best->second >= 0 && runs(best->second))
        return best->second;
    return -1;
}

int make_plan(const int64_t *xs, const int64_t *ws, const int32_t *st, const int32_t *pad, const int32_t *dil,
              int dtype, int x_layout, Plan &pl)
{
    Geometry g;
    int rc = check_geometry(xs, ws, st, pad, dil, g);
    if (rc)
        return rc;
    if (dtype != IGC_BF16 && dtype != IGC_FP8_E4M3FN)
        return fail(IGC_ERR_INVALID, "dtype %d is neither IGC_BF16 nor IGC_FP8_E4M3FN", dtype);
    if (x_layout != IGC_NCDHW && x_layout != IGC_NDHWC)
        return fail(IGC_ERR_INVALID, "x_layout %d is neither IGC_NCDHW nor IGC_NDHWC", x_layout);
    const int esz = dtype == IGC_FP8_E4M3FN ? 1 : 2;
    const int chunk = 16 / esz;

    const int forced = g_force_path;
    const bool pointwise_ok = is_pointwise(g) && x_layout == IGC_NCDHW && dtype == IGC_BF16;
    int path;
    if (forced == IGC_PATH_AUTO) {
        path = is_point(g) ? IGC_PATH_POINT
                           : (pointwise_ok ? IGC_PATH_POINTWISE : (is_temporal(g) ? IGC_PATH_TEMPORAL : IGC_PATH_GENERIC));
    } else {
        path = forced;
        if (path == IGC_PATH_POINT && !is_point(g))
            return fail(IGC_ERR_UNSUPPORTED, "forced point-output path does not apply to this shape");
        if (path == IGC_PATH_TEMPORAL && !is_temporal(g))
            return fail(IGC_ERR_UNSUPPORTED, "forced temporal path needs a Tx1x1 filter, h/w stride 1, pad 0");
        if (path == IGC_PATH_POINTWISE && !pointwise_ok)
            return fail(IGC_ERR_UNSUPPORTED,
                        "forced pointwise path needs a 1x1x1 filter, unit stride, no padding, NCDHW bf16 activations");
        if (path < IGC_PATH_GENERIC || path > IGC_PATH_POINTWISE)
            return fail(IGC_ERR_INVALID, "forced path %d unknown", path);
    }

    const int64_t rk = g.C * g.T * g.R * g.S;
    const int64_t ldw = packed_cols(rk, dtype);
    const int64_t P = g.Do * g.Ho * g.Wo;
    const int64_t xnum = g.N * g.C * g.D * g.H * g.W;
    const int64_t ynum = g.N * g.K * P;
    if (rk > kI32Max - 256 || ldw * g.K / g.K != ldw)
        return fail(IGC_ERR_UNSUPPORTED, "reduction length C*T*R*S = %lld too large", (long long)rk);
    if (g.K * ldw * esz >= (int64_t(1) << 32))
        return fail(IGC_ERR_UNSUPPORTED, "packed filter of %lld bytes exceeds 2^32", (long long)(g.K * ldw * esz));

    ConvParams &p = pl.p;
    p = ConvParams{};
    p.splits = 1;
    p.N = (int)g.N; p.C = (int)g.C; p.D = (int)g.D; p.H = (int)g.H; p.W = (int)g.W;
    p.K = (int)g.K; p.T = (int)g.T; p.R = (int)g.R; p.S = (int)g.S;
    p.sd = (int)g.sd; p.sh = (int)g.sh; p.sw = (int)g.sw;
    p.pd = (int)g.pd; p.ph = (int)g.ph; p.pw = (int)g.pw;
    p.dd = (int)g.dd; p.dh = (int)g.dh; p.dw = (int)g.dw;
    p.Do = (int)g.Do; p.Ho = (int)g.Ho; p.Wo = (int)g.Wo;
    p.Rk = (int)rk;
    p.ldw = (int)ldw;
    p.xbytes = xnum * esz;
    p.wbytes = (int)std::min<int64_t>(g.K * ldw * esz, kI32Max);

    if (path == IGC_PATH_POINTWISE) {
        const int64_t S = g.D * g.H * g.W;
        const int ft = g_force_tile;
        if (ft >= 0 && !is_pointwise_tile(ft))
            return fail(IGC_ERR_UNSUPPORTED, "the pointwise path runs tile %d only (forced %d)", (int)TILE_PW, ft);
        const int pt = TILE_PW;
        const int bm = kTiles[pt].bm;
        if (S % 8 != 0)
            return fail(IGC_ERR_UNSUPPORTED, "pointwise path needs D*H*W %% 8 == 0 (16-byte rows), D*H*W = %lld",
                        (long long)S);
        if (g.N * S > kI32Max || S > kI32Max)
            return fail(IGC_ERR_UNSUPPORTED, "output rows N*D*H*W = %lld exceed 2^31", (long long)(g.N * S));
        const int64_t tiles = g.N * ((S + bm - 1) / bm) * ((g.K + 63) / 64);
        if (tiles > kI32Max)
            return fail(IGC_ERR_UNSUPPORTED, "grid of %lld tiles too large", (long long)tiles);
        p.P = (int)S;
        p.M = (int)(g.N * S);
        p.Ncol = (int)g.K;
        p.nk = (int)((g.C + kTiles[pt].kb / 2 - 1) / (kTiles[pt].kb / 2));  // kb bytes = kb/2 channels per step
        p.tiles_m = (int)(g.N * ((S + bm - 1) / bm));
        p.tiles_n = (int)((g.K + 63) / 64);
        p.group_m = 1;
        p.ksplit = p.nk;
        pl.path = path;
        pl.tile = pt;
        pl.big = xnum > kSmallTensor || ynum > kSmallTensor;
        pl.cblock = false;
        pl.xspan = 0;
        return IGC_OK;
    }
    if (path == IGC_PATH_POINT) {
        if ((rk * esz) % 4 != 0)
            return fail(IGC_ERR_UNSUPPORTED, "point-output path needs image rows of a multiple of 4 bytes (C*T*R*S*%d = %lld)",
                        esz, (long long)(rk * esz));
        p.P = 1;
        p.M = (int)g.K;
        p.Ncol = (int)g.N;
    } else {
        if (x_layout != IGC_NDHWC)
            return fail(IGC_ERR_UNSUPPORTED, "im2col paths need NDHWC activations (pack them with conv_pack_x)");
        if (g.C % chunk != 0)
            return fail(IGC_ERR_UNSUPPORTED, "im2col paths need C %% %d == 0 for %s (C = %lld)", chunk,
                        esz == 1 ? "fp8" : "bf16", (long long)g.C);
        const int64_t M = g.N * P;
        if (M > kI32Max || P > kI32Max)
            return fail(IGC_ERR_UNSUPPORTED, "output rows N*Do*Ho*Wo = %lld exceed 2^31", (long long)M);
        p.P = (int)P;
        p.M = (int)M;
        p.Ncol = (int)g.K;
    }
    pl.path = path;
    pl.big = xnum > kSmallTensor || ynum > kSmallTensor;
    pl.xspan = buffer_x_span(g, esz);

    // Tile: the largest whose grid still covers the 256 CUs at least twice
    // (256x256) or once (128x128), else 64x64.
    auto nblocks = [&](int t) {
        return ((int64_t)p.M + kTiles[t].bm - 1) / kTiles[t].bm * (((int64_t)p.Ncol + kTiles[t].bn - 1) / kTiles[t].bn);
    };
    int tile = g_force_tile;
    if (is_pointwise_tile(tile))
        return fail(IGC_ERR_UNSUPPORTED, "tile %d is the pointwise path's kernel", tile);
    const int64_t cus = device_cus();
    if (tile < 0 || tile >= kNumTiles) {
        // Size rule (the fallback where no swept shape is near). Measured on
        // MI355X: the 256x256 direct-to-LDS tile with 128-byte steps (16x16 MFMA
        // blocks, bf16 and fp8) is the fastest whenever its grid reaches ~160
        // workgroups (5/8 of the CUs); smaller grids take the 128x128 (two
        // workgroups per CU) or 64x64 (4-stage ring) direct-to-LDS tiles. The
        // point-output path picks the tile that fills one round best.
        // A long reduction on a grid that 64x64 tiles would fill too far to split (the split needs a grid
        // below half the CUs) but 128x128 tiles would not: 128x128 with its split. Measured (fp8 3x3x3,
        // C1024 on 4x16x16 / C2048 on 4x8x8): 32 / 45 us against 88 / 173 us for 64x64 unsplit.
        const int64_t steps = (rk * esz + 127) / 128;
        const bool split128 = steps >= 64 && 2 * nblocks(TILE_DMA_64) >= cus && 2 * nblocks(TILE_DMA_128) < cus;
        tile = path == IGC_PATH_POINT
                   ? point_tile(p.M, p.Ncol, esz == 2)
                   : (nblocks(TILE_DMA_256) >= cus * 5 / 8
                          ? TILE_DMA_256
                          : (nblocks(TILE_DMA_128) >= cus || split128 ? TILE_DMA_128 : TILE_DMA_64));
        // Where the whole-channel-block im2col order applies and each tile's
        // reach into x (and the whole packed filter) fits a 2^31-byte buffer
        // range, a buffer-addressed 256x256 tile replaces the large tile:
        // activations issued two steps ahead (3 x 32 KB ring), the filter one
        // step ahead (2 x 32 KB).
        const bool buffer_ok = path != IGC_PATH_POINT && g.C % (128 / esz) == 0 &&
                               buffer_x_span(g, esz) < 0x7ffffff0 && g.K * ldw * esz < (int64_t(1) << 31);
        // In this rule every buffer-addressable grid takes TILE_BUF: on every swept shape where the buffer
        // tiles run, the lockstep tile was the fastest of them or within 0.3 % (the ping-pong wave groups
        // 2-10 % slower on fp8, 10 % on bf16; TILE_BUF_AHEAD level or up to 3 % slower).
        if (tile == TILE_DMA_256 && buffer_ok)
            tile = TILE_BUF;
        // The measured choice replaces that rule where a swept shape is near: the winner (or, if it
        // cannot run this shape, the runner-up) of the nearest shape of the same dtype and path in
        // tile_table.h, which sweep.py writes from timing every tile on one GPU.
        if (path == IGC_PATH_GENERIC || path == IGC_PATH_TEMPORAL) {
            const int taps = (int)(g.T * g.R * g.S);
            auto runs = [&](int t) {
                if (is_buffer(kTiles[t]))
                    return buffer_ok && (t != TILE_BUF_PINGPONG || taps <= 32);
                if (t == TILE_DMA_256x192)
                    return esz == 2;
                return t == TILE_DMA_256 || t == TILE_DMA_128 || t == TILE_DMA_64;
            };
            const int t = swept_tile(esz, path, (double)nblocks(TILE_DMA_256) / (double)cus,
                                     (rk * esz + 127) / 128, runs);
            if (t >= 0)
                tile = t;
        }
    } else {
        if (esz == 1 && tile == TILE_DMA_256x192)
            return fail(IGC_ERR_UNSUPPORTED, "tile %d is a bf16-only tile", tile);
        if (is_buffer(kTiles[tile])) {
            if (path == IGC_PATH_POINT)
                return fail(IGC_ERR_UNSUPPORTED, "tile %d (buffer-addressed) runs the im2col paths only", tile);
            if (g.C % (kTiles[tile].kb / esz) != 0)
                return fail(IGC_ERR_UNSUPPORTED, "tile %d needs C %% %d == 0", tile, kTiles[tile].kb / esz);
            if (buffer_x_span(g, esz) >= 0x7ffffff0 || g.K * ldw * esz >= (int64_t(1) << 31))
                return fail(IGC_ERR_UNSUPPORTED,
                            "tile %d needs each tile's reach into x and the packed filter below 2^31 bytes", tile);
            if (tile == TILE_BUF_PINGPONG && g.T * g.R * g.S > 32)
                return fail(IGC_ERR_UNSUPPORTED, "tile %d keeps a 32-bit tap mask per row: at most 32 filter taps",
                            tile);
        }
    }
    pl.tile = tile;
    const TileShape ts = kTiles[tile];
    const int tke = step_bytes(ts) / esz;  // elements per reduction step
    if (path == IGC_PATH_POINT) {
        p.nk = (int)((rk + tke - 1) / tke);  // no step made only of the filter's zero padding
        pl.cblock = false;
    } else {
        pl.cblock = (g.C % tke) == 0;
        p.nk = pl.cblock ? (int)(g.T * g.R * g.S * (g.C / tke)) : (int)(ldw / tke);
    }
    const int64_t tm = ((int64_t)p.M + ts.bm - 1) / ts.bm;
    const int64_t tn = ((int64_t)p.Ncol + ts.bn - 1) / ts.bn;
    if (tm * tn > kI32Max)
        return fail(IGC_ERR_UNSUPPORTED, "grid of %lld tiles too large", (long long)(tm * tn));
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    // Workgroups resident on one XCD (an eighth of the CUs): one 256x256 or two smaller tiles per CU.
    const int resident = (int)(cus / 8) * (ts.bm * ts.bn >= 256 * 256 ? 1 : 2);
    p.group_m = (int)std::max<int64_t>(1, resident / tn);
    if (path == IGC_PATH_POINT)  // few tile rows: all of them per column, so an image block is fetched once per XCD
        p.group_m = (int)std::max<int64_t>(p.group_m, std::min<int64_t>(tm, 8));
    if (g_force_group_m > 0)
        p.group_m = g_force_group_m;
    // Temporal filters on the buffer tiles: a tile's taps read activation windows H*W rows apart, ~56 tiles
    // on c5, which a raster of consecutive tiles re-fetches from beyond L2 once per tap. Raster groups of
    // tiles one tap apart share those windows instead (tile_coords).
    p.tap_stride = 0;
    if (path == IGC_PATH_TEMPORAL && is_buffer(ts) && g.T > 1) {
        const int64_t stride = (g.H * g.W * g.dd + ts.bm / 2) / ts.bm;
        if (stride >= 2 && tm >= (int64_t)p.group_m * stride && g_force_tap_raster >= 0)
            p.tap_stride = (int)stride;
    }
    p.ksplit = p.nk;
    return IGC_OK;
}

// Split reduction (split-K). FlyDSL PR #860 splits the reduction only when the
// grid of output tiles under-fills the GPU (its split-K selection rule: the
// under-fill test decides, a long reduction alone does not). Here: the
// global-address direct-to-LDS kernels, grids below half the CUs, and at least
// 5 reduction steps per split (about the ring depth: shorter splits are mostly
// pipeline fill); enough splits to fill the GPU once (one workgroup of 256x256
// per CU, two of the smaller tiles, which pair on a CU), at most 32, and no
// more than the workspace holds (splits * elements of y fp32 values).
// Measured on MI355X (bf16, 64x64 tiles): the 1024x64x1728 GEMM of a
// 64-channel 3x3x3 conv on 4x16x16 goes from 19.0 to 11.7 us, a 512-channel
// 3x3 conv on 7x7 from 42 to 15 us. Returns the split count (1 = none) with
// p.ksplit set, or a negative status for a forced split the tile cannot run.
bool splits_tile(int tile) { return !is_buffer(kTiles[tile]) && !is_pointwise_tile(tile); }

int plan_splits(Plan &pl, size_t ws_bytes)
{
    ConvParams &p = pl.p;
    const int64_t ynum = (int64_t)p.M * p.Ncol;
    const int64_t cap = std::min<int64_t>(ws_bytes / 4 / ynum, 64);
    const int forced = g_force_splits;
    int splits = 1;
    if (forced > 0) {
        if (forced > 1 && !splits_tile(pl.tile))
            return fail(IGC_ERR_UNSUPPORTED, "tile %d does not split the reduction (direct-to-LDS tiles only)",
                        pl.tile);
        splits = (int)std::min<int64_t>(std::min(forced, p.nk), cap);
    } else if (splits_tile(pl.tile)) {
        const int64_t grid = (int64_t)p.tiles_m * p.tiles_n;
        const TileShape &t = kTiles[pl.tile];
        const int64_t cus = device_cus();
        const int64_t slots = t.bm * t.bn >= 256 * 256 ? cus : 2 * cus;  // workgroups the GPU holds at once
        if (2 * grid < cus)
            splits = (int)std::min<int64_t>(std::min<int64_t>(std::min<int64_t>(slots / grid, p.nk / 5), 32), cap);
    }
    splits = std::max(splits, 1);
    p.ksplit = (p.nk + splits - 1) / splits;
    p.splits = (p.nk + p.ksplit - 1) / p.ksplit;  // every split holds at least one step
    pl.ws_need = p.splits > 1 ? (int64_t)p.splits * ynum * 4 : 0;
    // Tail split (buffer-addressed tiles; a round is one 256x256 workgroup per CU,
    // or two 128x128 ones): when the last round of tiles fills at most half of
    // the slots, its tiles run as S workgroups each over 1/S of the reduction,
    // S = slots / tail tiles (at most 8, at least 8 steps per split), and a
    // second pass adds the partials; only for reductions of at least 96 steps.
    // The last round then takes about 1/S of a tile's time instead of a whole
    // one. The one-GPU share of c3 (844 tiles: 3 rounds + 76) is the case this
    // is for. Needs the workspace; conv_debug_force_splits(1) turns it off.
    p.tail_first = 0;
    p.tail_splits = 0;
    if (p.splits == 1 && forced != 1 && is_buffer(kTiles[pl.tile])) {
        const TileShape &t = kTiles[pl.tile];
        const int64_t ntiles = (int64_t)p.tiles_m * p.tiles_n;
        const int64_t slots = t.bm * t.bn >= 256 * 256 ? device_cus() : 2 * device_cus();
        const int64_t full = ntiles / slots * slots, r = ntiles - full;
        const int64_t S = std::min<int64_t>(std::min<int64_t>(r > 0 ? slots / r : 0, 8), p.nk / 8);
        const int64_t need = r * S * t.bm * t.bn * 4;
        // at least 96 steps per tile: on 48-step tiles (c5s) the second pass cost more than the split saved
        if (p.nk >= 96 && full > 0 && r > 0 && 2 * r <= slots && S >= 2 && (size_t)need <= ws_bytes) {
            p.tail_first = (int)full;
            p.tail_splits = (int)S;
            pl.ws_need = need;
        }
    }
    return p.splits;
}

// One point-mode GEMM, out[col][row] = sum_r A[row][r] * B[col][r] with A rows
// of ldw elements (zero from Rk on), B rows of Rk elements (4-byte aligned) and
// out rows of ldo elements: the backward GEMMs of point-output shapes (the
// forward point path is the case A = filter, B = images, ldo = K). The tile
// follows the forward rule for grids of this size; a forced tile applies if it
// is a register or global-address direct-to-LDS tile.
int plan_point_gemm(int64_t M, int64_t Ncol, int64_t Rk, int64_t ldw, int64_t ldo, Plan &pl, bool long_split = false)
{
    if (M > kI32Max || Ncol > kI32Max || Rk > kI32Max - 256 || ldw > kI32Max || ldo > kI32Max ||
        M * ldo > (int64_t(1) << 62) / 2)
        return fail(IGC_ERR_UNSUPPORTED, "GEMM of %lld x %lld over %lld too large", (long long)M, (long long)Ncol,
                    (long long)Rk);
    ConvParams &p = pl.p;
    p = ConvParams{};
    p.splits = 1;
    p.N = 1;
    p.K = (int)ldo;
    p.M = (int)M;
    p.Ncol = (int)Ncol;
    p.Rk = (int)Rk;
    p.ldw = (int)ldw;
    p.P = 1;
    p.Do = p.Ho = p.Wo = 1;
    int tile = g_force_tile;
    if (tile < 0 || tile >= kNumTiles || is_buffer(kTiles[tile]) || is_pointwise_tile(tile)) {
        tile = point_tile(M, Ncol, true);
        // A long reduction that will be split (backward weights over the batch): 128x128 tiles, then
        // enough splits to fill the GPU; measured on the 9500-image patch embed (588 x 1280 over 9536):
        // 128x128 with 8 splits 51.5 us, 64x64 with 4-10 splits 61-64 us.
        if (long_split && tile == TILE_DMA_64 && Rk >= 32 * 64)
            tile = TILE_DMA_128;
    }
    const TileShape ts = kTiles[tile];
    const int tke = step_bytes(ts) / 2;
    p.nk = (int)((Rk + tke - 1) / tke);
    p.ksplit = p.nk;
    const int64_t tm = (M + ts.bm - 1) / ts.bm, tn = (Ncol + ts.bn - 1) / ts.bn;
    if (tm * tn > kI32Max)
        return fail(IGC_ERR_UNSUPPORTED, "grid of %lld tiles too large", (long long)(tm * tn));
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    const int64_t resident = device_cus() / 8 * (ts.bm * ts.bn >= 256 * 256 ? 1 : 2);
    p.group_m = (int)std::max<int64_t>({(int64_t)1, resident / tn, std::min<int64_t>(tm, 8)});
    if (g_force_group_m > 0)
        p.group_m = g_force_group_m;
    pl.path = IGC_PATH_POINT;
    pl.tile = tile;
    pl.big = Ncol * ldo > kSmallTensor;  // 64-bit output offsets
    pl.cblock = false;
    pl.xspan = 0;
    return IGC_OK;
}

// Shared checks of the point-output gradient entry points: a point-output
// geometry (input extent = filter extent, no padding, unit dilation), bf16.
int check_point_grad(const char *fn, const int64_t *xs, const int64_t *ws, const int32_t *st, const int32_t *pad,
                     const int32_t *dil, int dtype, int x_layout, Geometry &g)
{
    int rc = check_geometry(xs, ws, st, pad, dil, g);
    if (rc)
        return rc;
    if (dtype != IGC_BF16)
        return fail(dtype == IGC_FP8_E4M3FN ? IGC_ERR_UNSUPPORTED : IGC_ERR_INVALID, "%s: bf16 only (dtype %d)", fn,
                    dtype);
    if (x_layout != IGC_NCDHW && x_layout != IGC_NDHWC)
        return fail(IGC_ERR_INVALID, "%s: x_layout %d is neither IGC_NCDHW nor IGC_NDHWC", fn, x_layout);
    if (!is_point(g))
        return fail(IGC_ERR_UNSUPPORTED,
                    "%s: needs a point-output shape (input extent equal to the filter extent, no padding, unit "
                    "dilation)", fn);
    return IGC_OK;
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Backward weights workspace: x^T [R][ldn] and dy^T [K][ldn] (bf16), each
// 256-byte aligned, then the split slices (fp32, K * R each).
struct WgradLayout {
    int64_t ldn, xt_off, dyt_off, part_off, base_bytes;
};

WgradLayout wgrad_layout(const Geometry &g)
{
    WgradLayout L;
    const int64_t rk = g.C * g.T * g.R * g.S;
    L.ldn = align_up(g.N, 64);
    L.xt_off = 0;
    L.dyt_off = align_up(rk * L.ldn * 2, 256);
    L.part_off = L.dyt_off + align_up(g.K * L.ldn * 2, 256);
    L.base_bytes = L.part_off;
    return L;
}

const char *path_name(int path)
{
    switch (path) {
    case IGC_PATH_POINTWISE: return "pointwise";
    case IGC_PATH_POINT: return "point";
    case IGC_PATH_TEMPORAL: return "temporal";
    default: return "generic";
    }
}

}  // namespace


extern "C" {

int conv_out_dims(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3],
                  const int32_t dilation[3], int64_t out_dhw[3])
{
    Geometry g;
    int rc = check_geometry(xshape, wshape, stride, pad, dilation, g);
    if (rc)
        return rc;
    if (!out_dhw)
        return fail(IGC_ERR_INVALID, "null out_dhw");
    out_dhw[0] = g.Do;
    out_dhw[1] = g.Ho;
    out_dhw[2] = g.Wo;
    return ok();
}

int64_t conv_packed_w_cols(const int64_t wshape[5], int dtype)
{
    if (!wshape || (dtype != IGC_BF16 && dtype != IGC_FP8_E4M3FN))
        return IGC_ERR_INVALID;
    for (int i = 1; i < 5; ++i)
        if (wshape[i] < 1 || wshape[i] > kI32Max)
            return IGC_ERR_INVALID;
    const int64_t rk = wshape[1] * wshape[2] * wshape[3] * wshape[4];
    if (rk > kI32Max - 256)
        return IGC_ERR_INVALID;
    return packed_cols(rk, dtype);
}

int conv_amax(const void *t_bf16, int64_t numel, float *amax_dev, void *stream)
{
    if (!t_bf16 || !amax_dev)
        return fail(IGC_ERR_INVALID, "conv_amax: null pointer");
    if (numel < 1)
        return fail(IGC_ERR_INVALID, "conv_amax: numel = %lld must be >= 1", (long long)numel);
    if (!aligned16(t_bf16))
        return fail(IGC_ERR_ALIGN, "conv_amax: tensor not 16-byte aligned");
    if (launch_amax(static_cast<const uint16_t *>(t_bf16), numel, amax_dev, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return fail(IGC_ERR_HIP, "conv_amax: launch failed");
    return ok();
}

int conv_fp8_scales(const float *amax_dev, float *scale_pair_dev, void *stream)
{
    if (!amax_dev || !scale_pair_dev)
        return fail(IGC_ERR_INVALID, "conv_fp8_scales: null pointer");
    if (launch_fp8_scales(amax_dev, scale_pair_dev, static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_fp8_scales: launch failed");
    return ok();
}

int conv_pack_x(const void *x_ncdhw_bf16, void *x_out, const int64_t xshape[5], int dtype,
                const float *scale_pair_dev, void *stream)
{
    if (!x_ncdhw_bf16 || !x_out || !xshape)
        return fail(IGC_ERR_INVALID, "conv_pack_x: null pointer");
    if (dtype != IGC_BF16 && dtype != IGC_FP8_E4M3FN)
        return fail(IGC_ERR_INVALID, "conv_pack_x: bad dtype %d", dtype);
    if (dtype == IGC_FP8_E4M3FN && !scale_pair_dev)
        return fail(IGC_ERR_INVALID, "conv_pack_x: fp8 needs scale_pair_dev");
    for (int i = 0; i < 5; ++i)
        if (xshape[i] < 1 || xshape[i] > kI32Max)
            return fail(IGC_ERR_INVALID, "conv_pack_x: xshape[%d] = %lld out of range", i, (long long)xshape[i]);
    if (!aligned16(x_ncdhw_bf16) || !aligned16(x_out))
        return fail(IGC_ERR_ALIGN, "conv_pack_x: tensors must be 16-byte aligned");
    const int64_t C = xshape[1], S = xshape[2] * xshape[3] * xshape[4];
    const int need = dtype == IGC_FP8_E4M3FN ? 16 : 8;
    if (C % need != 0)
        return fail(IGC_ERR_UNSUPPORTED, "conv_pack_x: needs C %% %d == 0 (C = %lld)", need, (long long)C);
    const int64_t blocks = xshape[0] * ((C + 63) / 64) * ((S + 63) / 64);
    if (blocks > kI32Max)
        return fail(IGC_ERR_UNSUPPORTED, "conv_pack_x: tensor too large");
    if (launch_pack_x(static_cast<const uint16_t *>(x_ncdhw_bf16), x_out, xshape[0], C, S,
                      dtype == IGC_FP8_E4M3FN ? DT_FP8 : DT_BF16, scale_pair_dev,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_pack_x: launch failed");
    return ok();
}

int conv_pack_w(const void *w_kctrs_bf16, void *w_packed, const int64_t wshape[5], int dtype, int x_layout,
                const float *scale_pair_dev, void *stream)
{
    if (!w_kctrs_bf16 || !w_packed || !wshape)
        return fail(IGC_ERR_INVALID, "conv_pack_w: null pointer");
    if (dtype != IGC_BF16 && dtype != IGC_FP8_E4M3FN)
        return fail(IGC_ERR_INVALID, "conv_pack_w: bad dtype %d", dtype);
    if (x_layout != IGC_NCDHW && x_layout != IGC_NDHWC)
        return fail(IGC_ERR_INVALID, "conv_pack_w: bad x_layout %d", x_layout);
    if (dtype == IGC_FP8_E4M3FN && !scale_pair_dev)
        return fail(IGC_ERR_INVALID, "conv_pack_w: fp8 needs scale_pair_dev");
    for (int i = 0; i < 5; ++i)
        if (wshape[i] < 1 || wshape[i] > kI32Max)
            return fail(IGC_ERR_INVALID, "conv_pack_w: wshape[%d] = %lld out of range", i, (long long)wshape[i]);
    if (!aligned16(w_kctrs_bf16) || !aligned16(w_packed))
        return fail(IGC_ERR_ALIGN, "conv_pack_w: tensors must be 16-byte aligned");
    const int64_t ldw = conv_packed_w_cols(wshape, dtype);
    if (ldw <= 0)
        return fail(IGC_ERR_INVALID, "conv_pack_w: reduction too large");
    if (launch_pack_w(static_cast<const uint16_t *>(w_kctrs_bf16), w_packed, wshape[0], wshape[1], wshape[2],
                      wshape[3], wshape[4], ldw, x_layout == IGC_NDHWC, dtype == IGC_FP8_E4M3FN ? DT_FP8 : DT_BF16,
                      scale_pair_dev, static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_pack_w: launch failed");
    return ok();
}

int conv_fwd_ex(const void *x, const void *w_packed, void *y, const int64_t xshape[5], const int64_t wshape[5],
                const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout,
                const float *scales_dev, const float *bias_dev, float *y_amax_dev, void *workspace_dev,
                size_t workspace_bytes, void *stream)
{
    Plan pl;
    int rc = make_plan(xshape, wshape, stride, pad, dilation, dtype, x_layout, pl);
    if (rc)
        return rc;
    if (!x || !w_packed || !y)
        return fail(IGC_ERR_INVALID, "conv_fwd: null tensor pointer");
    if (dtype == IGC_FP8_E4M3FN && !scales_dev)
        return fail(IGC_ERR_INVALID, "conv_fwd: fp8 needs scales_dev = {s_x, inv_x, s_w, inv_w}");
    if (!aligned16(x) || !aligned16(w_packed) || !aligned16(y))
        return fail(IGC_ERR_ALIGN, "conv_fwd: x, w_packed and y must be 16-byte aligned");
    if (workspace_bytes && !workspace_dev)
        return fail(IGC_ERR_INVALID, "conv_fwd_ws: null workspace with workspace_bytes = %zu", workspace_bytes);
    if (workspace_dev && !aligned16(workspace_dev))
        return fail(IGC_ERR_ALIGN, "conv_fwd_ws: workspace must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(bias_dev) | reinterpret_cast<uintptr_t>(y_amax_dev)) & 3u)
        return fail(IGC_ERR_ALIGN, "conv_fwd_ex: bias and amax must be 4-byte aligned fp32");
    rc = plan_splits(pl, workspace_dev ? workspace_bytes : 0);
    if (rc < 0)
        return rc;
    pl.p.x = x;
    pl.p.w = w_packed;
    pl.p.y = y;
    pl.p.scales = dtype == IGC_FP8_E4M3FN ? scales_dev : nullptr;
    pl.p.part = pl.p.splits > 1 || pl.p.tail_splits > 1 ? static_cast<float *>(workspace_dev) : nullptr;
    pl.p.bias = bias_dev;
    pl.p.amax = reinterpret_cast<unsigned *>(y_amax_dev);
    const Mode mode = pl.path == IGC_PATH_POINT ? MODE_POINT : (pl.path == IGC_PATH_TEMPORAL ? MODE_TEMPORAL : MODE_GENERIC);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (y_amax_dev && launch_amax_zero(y_amax_dev, st) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_fwd_ex: amax clear launch failed");
    if (launch_conv(pl.p, pl.tile, mode, dtype == IGC_FP8_E4M3FN ? DT_FP8 : DT_BF16, pl.big, pl.cblock, st) !=
        hipSuccess)
        return fail(IGC_ERR_HIP, "conv_fwd: kernel launch failed");
    if (pl.p.splits > 1 && launch_splitk_reduce(pl.p, st) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_fwd_ws: split reduction launch failed");
    if (pl.p.tail_splits > 1 &&
        launch_tail_reduce(pl.p, kTiles[pl.tile].bm, kTiles[pl.tile].bn,
                           pl.p.tiles_m * pl.p.tiles_n - pl.p.tail_first, st) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_fwd_ws: tail reduction launch failed");
    return ok();
}

int conv_fwd_ws(const void *x, const void *w_packed, void *y, const int64_t xshape[5], const int64_t wshape[5],
                const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout,
                const float *scales_dev, void *workspace_dev, size_t workspace_bytes, void *stream)
{
    return conv_fwd_ex(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev, nullptr,
                       nullptr, workspace_dev, workspace_bytes, stream);
}

int conv_fwd_noalloc(const void *x, const void *w_packed, void *y, const int64_t xshape[5],
                     const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3],
                     int dtype, int x_layout, const float *scales_dev, const float *bias_dev, float *y_amax_dev,
                     void *stream)
{
    Plan pl;
    int rc = make_plan(xshape, wshape, stride, pad, dilation, dtype, x_layout, pl);
    if (rc)
        return rc;
    rc = plan_splits(pl, SIZE_MAX);
    if (rc < 0)
        return rc;
    const int64_t need = pl.ws_need;
    if (need > (int64_t)kScratchBytes)
        return fail(IGC_ERR_UNSUPPORTED, "conv_fwd_noalloc: the plan needs %lld bytes of workspace, the static "
                    "scratch holds %zu", (long long)need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_ptr();
        if (!ws)
            return fail(IGC_ERR_HIP, "conv_fwd_noalloc: device address of the static scratch not available");
    }
    // the same plan as conv_fwd_ws with conv_fwd_workspace_bytes of workspace: every fp32 partial the
    // split writes is written before it is read, so nothing in the scratch needs clearing
    return conv_fwd_ex(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev, bias_dev,
                       y_amax_dev, ws, (size_t)need, stream);
}

int conv_fwd(const void *x, const void *w_packed, void *y, const int64_t xshape[5], const int64_t wshape[5],
             const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout,
             const float *scales_dev, void *stream)
{
    return conv_fwd_ws(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev, nullptr, 0,
                       stream);
}

int64_t conv_fwd_workspace_bytes(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3],
                                 const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout)
{
    Plan pl;
    int rc = make_plan(xshape, wshape, stride, pad, dilation, dtype, x_layout, pl);
    if (rc)
        return rc;
    rc = plan_splits(pl, SIZE_MAX);
    if (rc < 0)
        return rc;
    ok();
    return pl.ws_need;
}

int conv_plan_ws(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3],
                 const int32_t dilation[3], int dtype, int x_layout, size_t workspace_bytes, char *buf, size_t len)
{
    Plan pl;
    int rc = make_plan(xshape, wshape, stride, pad, dilation, dtype, x_layout, pl);
    if (rc)
        return rc;
    rc = plan_splits(pl, workspace_bytes);
    if (rc < 0)
        return rc;
    if (buf && len) {
        const TileShape ts = kTiles[pl.tile];
        snprintf(buf, len,
                 "path=%s tile_id=%d tile=%dx%d waves=%d mfma=%dx%d stages=%d bstages=%d kstep=%d order=%s big=%d "
                 "grid=%d group_m=%d nk=%d loads=%s schedule=%s xspan=%lld splits=%d ksplit=%d tail=%d/%d tap=%d",
                 path_name(pl.path), pl.tile, ts.bm, ts.bn, ts.wm * ts.wn, ts.mf, ts.mf, ts.stages,
                 is_buffer(ts) ? ts.sb : ts.stages, step_bytes(ts) / (dtype == IGC_FP8_E4M3FN ? 1 : 2),
                 pl.cblock ? "cblock" : "linear", pl.big ? 1 : 0, pl.p.tiles_m * pl.p.tiles_n, pl.p.group_m, pl.p.nk,
                 is_buffer(ts) ? "buffer-lds" : "global-lds", pl.tile == TILE_BUF_PINGPONG ? "pingpong" : "lockstep",
                 pl.path == IGC_PATH_POINT ? 0LL : (long long)pl.xspan, pl.p.splits, pl.p.ksplit,
                 pl.p.tail_splits > 1 ? pl.p.tiles_m * pl.p.tiles_n - pl.p.tail_first : 0,
                 pl.p.tail_splits > 1 ? pl.p.tail_splits : 1, pl.p.tap_stride);
    }
    return ok();
}

int conv_plan(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3], const int32_t pad[3],
              const int32_t dilation[3], int dtype, int x_layout, char *buf, size_t len)
{
    return conv_plan_ws(xshape, wshape, stride, pad, dilation, dtype, x_layout, 0, buf, len);
}

int conv_debug_force(int path, int tile, int group_m)
{
    if (path < IGC_PATH_AUTO || path > IGC_PATH_POINTWISE)
        return fail(IGC_ERR_INVALID, "conv_debug_force: unknown path %d", path);
    if (tile < -1 || tile >= kNumTiles)
        return fail(IGC_ERR_INVALID, "conv_debug_force: tile %d not in [-1, %d)", tile, kNumTiles);
    if (group_m < 0)
        return fail(IGC_ERR_INVALID, "conv_debug_force: group_m %d < 0", group_m);
    g_force_path = path;
    g_force_tile = tile;
    g_force_group_m = group_m;
    return ok();
}

int64_t conv_packed_w_t_cols(const int64_t wshape[5])
{
    if (!wshape)
        return IGC_ERR_INVALID;
    for (int i = 0; i < 5; ++i)
        if (wshape[i] < 1 || wshape[i] > kI32Max)
            return IGC_ERR_INVALID;
    return align_up(wshape[0], 64);
}

int conv_pack_w_t(const void *w_kctrs_bf16, void *w_t, const int64_t wshape[5], int x_layout, void *stream)
{
    if (!w_kctrs_bf16 || !w_t || !wshape)
        return fail(IGC_ERR_INVALID, "conv_pack_w_t: null pointer");
    if (x_layout != IGC_NCDHW && x_layout != IGC_NDHWC)
        return fail(IGC_ERR_INVALID, "conv_pack_w_t: bad x_layout %d", x_layout);
    for (int i = 0; i < 5; ++i)
        if (wshape[i] < 1 || wshape[i] > kI32Max)
            return fail(IGC_ERR_INVALID, "conv_pack_w_t: wshape[%d] = %lld out of range", i, (long long)wshape[i]);
    if (!aligned16(w_kctrs_bf16) || !aligned16(w_t))
        return fail(IGC_ERR_ALIGN, "conv_pack_w_t: tensors must be 16-byte aligned");
    const int64_t ldk = align_up(wshape[0], 64), rk = wshape[1] * wshape[2] * wshape[3] * wshape[4];
    if (rk > kI32Max || rk * ldk * 2 >= (int64_t(1) << 32))
        return fail(IGC_ERR_UNSUPPORTED, "conv_pack_w_t: transposed filter of %lld x %lld too large", (long long)rk,
                    (long long)ldk);
    if (launch_pack_w_t(static_cast<const uint16_t *>(w_kctrs_bf16), static_cast<uint16_t *>(w_t), wshape[0],
                        wshape[1], wshape[2], wshape[3], wshape[4], ldk, x_layout == IGC_NDHWC,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_pack_w_t: launch failed");
    return ok();
}

int conv_bwd_data(const void *dy, const void *w_t, void *dx, const int64_t xshape[5], const int64_t wshape[5],
                  const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout,
                  void *stream)
{
    Geometry g;
    int rc = check_point_grad("conv_bwd_data", xshape, wshape, stride, pad, dilation, dtype, x_layout, g);
    if (rc)
        return rc;
    if (!dy || !w_t || !dx)
        return fail(IGC_ERR_INVALID, "conv_bwd_data: null tensor pointer");
    if (!aligned16(dy) || !aligned16(w_t) || !aligned16(dx))
        return fail(IGC_ERR_ALIGN, "conv_bwd_data: dy, w_t and dx must be 16-byte aligned");
    if (g.K % 2 != 0)
        return fail(IGC_ERR_UNSUPPORTED, "conv_bwd_data: dy rows of K = %lld bf16 must be 4-byte aligned (K even)",
                    (long long)g.K);
    const int64_t rk = g.C * g.T * g.R * g.S;
    Plan pl;
    // dx[n][j] = sum_k w_t[j][k] * dy[n][k]: A = w_t (rows j, ldk), B = dy rows (K elements), dx rows of rk
    rc = plan_point_gemm(rk, g.N, g.K, align_up(g.K, 64), rk, pl);
    if (rc)
        return rc;
    pl.p.x = dy;
    pl.p.w = w_t;
    pl.p.y = dx;
    if (launch_conv(pl.p, pl.tile, MODE_POINT, DT_BF16, pl.big, false, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return fail(IGC_ERR_HIP, "conv_bwd_data: kernel launch failed");
    return ok();
}

// Shared by conv_bwd_weight and its workspace query: the GEMM plan, its split
// count for `room` bytes of slices, and the workspace layout.
int plan_wgrad(const int64_t *xs, const int64_t *ws, const int32_t *st, const int32_t *pad, const int32_t *dil,
               int dtype, int x_layout, size_t room, Plan &pl, WgradLayout &L)
{
    Geometry g;
    int rc = check_point_grad("conv_bwd_weight", xs, ws, st, pad, dil, dtype, x_layout, g);
    if (rc)
        return rc;
    L = wgrad_layout(g);
    const int64_t rk = g.C * g.T * g.R * g.S;
    if (L.ldn > kI32Max - 256 || rk * L.ldn * 2 >= (int64_t(1) << 32) || g.K * L.ldn * 2 >= (int64_t(1) << 32))
        return fail(IGC_ERR_UNSUPPORTED, "conv_bwd_weight: transposed operands above 2^32 bytes");
    // dw[k][j] = sum_n xt[j][n] * dyt[k][n]: A = x^T (rows j), B = dy^T (rows k), both rows of ldn (zeros past N)
    rc = plan_point_gemm(rk, g.K, L.ldn, L.ldn, rk, pl, room > 0);
    if (rc)
        return rc;
    rc = plan_splits(pl, room);
    return rc < 0 ? rc : IGC_OK;
}

int64_t conv_bwd_weight_workspace_bytes(const int64_t xshape[5], const int64_t wshape[5], const int32_t stride[3],
                                        const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout)
{
    Plan pl;
    WgradLayout L;
    int rc = plan_wgrad(xshape, wshape, stride, pad, dilation, dtype, x_layout, SIZE_MAX, pl, L);
    if (rc)
        return rc;
    ok();
    return L.base_bytes + (pl.p.splits > 1 ? (int64_t)pl.p.splits * pl.p.M * pl.p.Ncol * 4 : 0);
}

int conv_bwd_weight(const void *x, const void *dy, void *dw, const int64_t xshape[5], const int64_t wshape[5],
                    const int32_t stride[3], const int32_t pad[3], const int32_t dilation[3], int dtype, int x_layout,
                    void *workspace_dev, size_t workspace_bytes, void *stream)
{
    Plan pl;
    WgradLayout L;
    Geometry g;
    int rc = check_point_grad("conv_bwd_weight", xshape, wshape, stride, pad, dilation, dtype, x_layout, g);
    if (rc)
        return rc;
    if (!x || !dy || !dw || !workspace_dev)
        return fail(IGC_ERR_INVALID, "conv_bwd_weight: null pointer");
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dw) || !aligned16(workspace_dev))
        return fail(IGC_ERR_ALIGN, "conv_bwd_weight: x, dy, dw and the workspace must be 16-byte aligned");
    L = wgrad_layout(g);
    if ((int64_t)workspace_bytes < L.base_bytes)
        return fail(IGC_ERR_INVALID, "conv_bwd_weight: workspace of %zu bytes, needs at least %lld", workspace_bytes,
                    (long long)L.base_bytes);
    rc = plan_wgrad(xshape, wshape, stride, pad, dilation, dtype, x_layout, workspace_bytes - L.base_bytes, pl, L);
    if (rc)
        return rc;
    char *wsb = static_cast<char *>(workspace_dev);
    uint16_t *xt = reinterpret_cast<uint16_t *>(wsb + L.xt_off);
    uint16_t *dyt = reinterpret_cast<uint16_t *>(wsb + L.dyt_off);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t rk = g.C * g.T * g.R * g.S;
    // x is [N][rk] in either layout (a point-output image is rk contiguous elements), dy is [N][K]
    if (launch_transpose_pad2(static_cast<const uint16_t *>(x), xt, rk, static_cast<const uint16_t *>(dy), dyt, g.K,
                              g.N, L.ldn, st) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_bwd_weight: transpose launch failed");
    pl.p.x = dyt;
    pl.p.w = xt;
    pl.p.y = dw;
    pl.p.part = pl.p.splits > 1 ? reinterpret_cast<float *>(wsb + L.part_off) : nullptr;
    if (launch_conv(pl.p, pl.tile, MODE_POINT, DT_BF16, pl.big, false, st) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_bwd_weight: kernel launch failed");
    if (pl.p.splits > 1 && launch_splitk_reduce(pl.p, st) != hipSuccess)
        return fail(IGC_ERR_HIP, "conv_bwd_weight: split reduction launch failed");
    return ok();
}

int conv_debug_force_grid(int cus)
{
    if (cus < 0)
        return fail(IGC_ERR_INVALID, "conv_debug_force_grid: compute units %d < 0", cus);
    g_force_cus = cus;
    return ok();
}

int conv_debug_force_tap_raster(int mode)
{
    if (mode != -1 && mode != 0)
        return fail(IGC_ERR_INVALID, "conv_debug_force_tap_raster: mode %d is neither -1 (off) nor 0 (automatic)", mode);
    g_force_tap_raster = mode;
    return ok();
}

int conv_debug_force_splits(int splits)
{
    if (splits < 0)
        return fail(IGC_ERR_INVALID, "conv_debug_force_splits: splits %d < 0", splits);
    g_force_splits = splits;
    return ok();
}

const char *conv_last_error(void) { return g_err.c_str(); }

}  // extern "C"

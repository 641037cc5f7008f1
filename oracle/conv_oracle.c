/*
 * Plain CPU oracle for forward convolution -- TEST INFRASTRUCTURE ONLY.
 *
 * Nothing in the product library links, includes or calls this file. Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark load
 * it (through oracle/oracle.py). It shares no source, header, table or helper
 * with the GPU path.
 *
 * What it computes (every routine is the textbook definition, written for a
 * reader to check by eye, with no blocking, fusion or reordering):
 *
 *  - conv3d forward as a cross-correlation with zero padding, the operation
 *    that FlyDSL PR #860 ("[Kernel] fp8 conv3d: 8-wave GEMM pipeline + BIG_IN
 *    fix") checks its implicit-GEMM kernels against (torch conv3d, see the
 *    commit adding the large_shape regression test) and that MIOpen PR #10912
 *    reduces to a single GEMM for the point-output case (PR body). For every
 *    output element it sums x * w over channel c and filter taps (t, r, s):
 *        y[n,k,od,oh,ow] = sum_{c,t,r,s} X(n,c,od*sd-pd+t*dd, oh*sh-ph+r*dh,
 *                                          ow*sw-pw+s*dw) * W(k,c,t,r,s)
 *    with X = 0 outside the input box. Seven nested loops, fp64 accumulation,
 *    int64 indices.
 *  - the two gradients of that map, which MIOpen PR #10912 turns into one GEMM
 *    each for point-output shapes (backward data and backward weights, PR
 *    body): with y = conv(x, w) and an incoming gradient dy of y's shape,
 *        dx[n,c,d,h,w] = sum of dy[n,k,od,oh,ow] * W(k,c,t,r,s) over every
 *                        (k, od, oh, ow, t, r, s) whose tap reads (d, h, w)
 *        dw[k,c,t,r,s] = sum over (n, od, oh, ow) of dy[n,k,od,oh,ow] *
 *                        X(n,c,od*sd-pd+t*dd, oh*sh-ph+r*dh, ow*sw-pw+s*dw)
 *    (the adjoints of the forward map in x and in w), fp64, for any geometry.
 *  - the operand encodings the pages use: bf16 (top half of binary32, round to
 *    nearest even) and OCP fp8 E4M3FN (sign, 4-bit exponent with bias 7, 3-bit
 *    mantissa, subnormals, no infinities, S.1111.111 = NaN, max finite 448),
 *    which FlyDSL PR #860 names as the fp8 format its kernel accepts natively
 *    (PR summary, "Design"); per-tensor scale = amax / 448.
 *
 * Parity status of every routine is recorded in the test suite's pins; none is
 * unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Scalar encodings                                                         */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> exact double (bf16 is the upper 16 bits of binary32). */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary32 -> bf16 bits, round to nearest, ties to even on the 16 dropped bits. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep it a (quiet) NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent when the mantissa is all ones */
    return (uint16_t)upper;
}

/* E4M3FN code -> value, from the format definition. */
double oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xf;
    int m = code & 0x7;
    double v;
    if (e == 0xf && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/*
 * value -> E4M3FN code: the nearest representable value, ties to the code with
 * an even mantissa, values beyond the largest finite value clamp to +-448
 * (saturating conversion), NaN -> 0x7F with the input's sign. The search runs
 * over the 127 non-negative finite codes, which are ordered by value.
 */
uint8_t oracle_e4m3_encode(float f)
{
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (isnan(f))
        return (uint8_t)(sign | 0x7f);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7e);
    /* lo = largest code whose value is <= a (code 0 has value 0 <= a). */
    int lo = 0, hi = 0x7e;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int up = lo + 1; /* a < 448 so lo < 0x7e and up is finite */
    double dlo = a - oracle_e4m3_decode((uint8_t)lo);
    double dup = oracle_e4m3_decode((uint8_t)up) - a;
    int code;
    if (dlo < dup)
        code = lo;
    else if (dup < dlo)
        code = up;
    else
        code = (lo % 2 == 0) ? lo : up; /* tie: even mantissa (= even code) */
    return (uint8_t)(sign | code);
}

/* Element-wise array forms of the three encodings above. */
void oracle_f32_to_bf16_array(const float *f, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(f[i]);
}

void oracle_e4m3_encode_array(const float *f, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(f[i]);
}

void oracle_e4m3_decode_array(const uint8_t *q, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_decode(q[i]);
}

/* ------------------------------------------------------------------------ */
/* Per-tensor fp8 scaling: s = amax/448, q = E4M3FN(fp32(v * (448/amax)))     */
/* ------------------------------------------------------------------------ */

float oracle_amax_bf16(const uint16_t *v, int64_t n)
{
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double a = fabs(bf16_bits_to_double(v[i]));
        if (a > m)
            m = a;
    }
    return (float)m; /* a bf16 magnitude is exactly representable in binary32 */
}

/* {s, inv} = {amax/448, 448/amax}, each one correctly rounded binary32
 * division; an all-zero tensor gets {1, 1}. */
void oracle_fp8_scales(float amax, float *s, float *inv)
{
    if (!(amax > 0.0f)) {
        *s = 1.0f;
        *inv = 1.0f;
        return;
    }
    volatile float a = amax; /* keep the two divisions in binary32 */
    *s = a / 448.0f;
    *inv = 448.0f / a;
}

/* q[i] = E4M3FN(fp32(bf16 v[i] * inv)); the product is one binary32 multiply. */
void oracle_quantize_e4m3(const uint16_t *v, int64_t n, float inv, uint8_t *q)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        volatile float p = (float)bf16_bits_to_double(v[i]) * inv;
        q[i] = oracle_e4m3_encode(p);
    }
}

/* ------------------------------------------------------------------------ */
/* Convolution                                                              */
/* ------------------------------------------------------------------------ */

enum { ORACLE_F64 = 0, ORACLE_BF16 = 1, ORACLE_E4M3 = 2 };
enum { ORACLE_NCDHW = 0, ORACLE_NDHWC = 1 };

/* Operand element as a double: plain value, bf16 bits, or fp8 code * scale. */
static double operand(int kind, const void *p, int64_t i, double scale)
{
    switch (kind) {
    case ORACLE_BF16:
        return bf16_bits_to_double(((const uint16_t *)p)[i]);
    case ORACLE_E4M3:
        return oracle_e4m3_decode(((const uint8_t *)p)[i]) * scale;
    default:
        return ((const double *)p)[i];
    }
}

typedef struct {
    int xkind, xlayout, wkind;
    const void *x, *w;
    double sx, sw;
    int64_t N, C, D, H, W, K, T, R, S;
    int64_t sd, sh, sw_, pd, ph, pw, dd, dh, dw;
    int64_t Do, Ho, Wo;
} conv_problem;

static int64_t x_index(const conv_problem *p, int64_t n, int64_t c, int64_t d, int64_t h, int64_t w)
{
    if (p->xlayout == ORACLE_NDHWC)
        return (((n * p->D + d) * p->H + h) * p->W + w) * p->C + c;
    return (((n * p->C + c) * p->D + d) * p->H + h) * p->W + w;
}

/* One output element, the definition: sum over c, t, r, s of X * W. */
static double conv_point(const conv_problem *p, int64_t n, int64_t k, int64_t od, int64_t oh, int64_t ow)
{
    double acc = 0.0;
    for (int64_t c = 0; c < p->C; ++c)
        for (int64_t t = 0; t < p->T; ++t)
            for (int64_t r = 0; r < p->R; ++r)
                for (int64_t s = 0; s < p->S; ++s) {
                    int64_t id = od * p->sd - p->pd + t * p->dd;
                    int64_t ih = oh * p->sh - p->ph + r * p->dh;
                    int64_t iw = ow * p->sw_ - p->pw + s * p->dw;
                    if (id < 0 || id >= p->D || ih < 0 || ih >= p->H || iw < 0 || iw >= p->W)
                        continue; /* zero padding */
                    double xv = operand(p->xkind, p->x, x_index(p, n, c, id, ih, iw), p->sx);
                    int64_t wi = (((k * p->C + c) * p->T + t) * p->R + r) * p->S + s;
                    double wv = operand(p->wkind, p->w, wi, p->sw);
                    acc += xv * wv;
                }
    return acc;
}

static int setup(conv_problem *p, int xkind, const void *x, int xlayout, double sx, int wkind, const void *w,
                 double sw, const int64_t xs[5], const int64_t ws[5], const int32_t st[3], const int32_t pad[3],
                 const int32_t dil[3])
{
    p->xkind = xkind; p->x = x; p->xlayout = xlayout; p->sx = sx;
    p->wkind = wkind; p->w = w; p->sw = sw;
    p->N = xs[0]; p->C = xs[1]; p->D = xs[2]; p->H = xs[3]; p->W = xs[4];
    p->K = ws[0]; p->T = ws[2]; p->R = ws[3]; p->S = ws[4];
    p->sd = st[0]; p->sh = st[1]; p->sw_ = st[2];
    p->pd = pad[0]; p->ph = pad[1]; p->pw = pad[2];
    p->dd = dil[0]; p->dh = dil[1]; p->dw = dil[2];
    if (ws[1] != p->C || p->sd < 1 || p->sh < 1 || p->sw_ < 1 || p->dd < 1 || p->dh < 1 || p->dw < 1)
        return -1;
    /* output extent: floor((in + 2*pad - dil*(k-1) - 1) / stride) + 1 */
    int64_t nd = p->D + 2 * p->pd - p->dd * (p->T - 1) - 1;
    int64_t nh = p->H + 2 * p->ph - p->dh * (p->R - 1) - 1;
    int64_t nw = p->W + 2 * p->pw - p->dw * (p->S - 1) - 1;
    if (nd < 0 || nh < 0 || nw < 0)
        return -1;
    p->Do = nd / p->sd + 1;
    p->Ho = nh / p->sh + 1;
    p->Wo = nw / p->sw_ + 1;
    return 0;
}

/* Output extent (Do, Ho, Wo); returns -1 when the filter does not fit. */
int oracle_out_dims(const int64_t xs[5], const int64_t ws[5], const int32_t st[3], const int32_t pad[3],
                    const int32_t dil[3], int64_t out[3])
{
    conv_problem p;
    if (setup(&p, ORACLE_F64, 0, 0, 1.0, ORACLE_F64, 0, 1.0, xs, ws, st, pad, dil))
        return -1;
    out[0] = p.Do; out[1] = p.Ho; out[2] = p.Wo;
    return 0;
}

/* Full output, y in NCDHW (N, K, Do, Ho, Wo), fp64. */
int oracle_conv3d(int xkind, const void *x, int xlayout, double sx, int wkind, const void *w, double sw,
                  const int64_t xs[5], const int64_t ws[5], const int32_t st[3], const int32_t pad[3],
                  const int32_t dil[3], double *y)
{
    conv_problem p;
    if (setup(&p, xkind, x, xlayout, sx, wkind, w, sw, xs, ws, st, pad, dil))
        return -1;
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int64_t n = 0; n < p.N; ++n)
        for (int64_t k = 0; k < p.K; ++k)
            for (int64_t od = 0; od < p.Do; ++od)
                for (int64_t oh = 0; oh < p.Ho; ++oh)
                    for (int64_t ow = 0; ow < p.Wo; ++ow)
                        y[(((n * p.K + k) * p.Do + od) * p.Ho + oh) * p.Wo + ow] =
                            conv_point(&p, n, k, od, oh, ow);
    return 0;
}

/*
 * Sampled output: y[i] = output element at pts[i] = (n, k, od, oh, ow).
 */
int oracle_conv3d_points(int xkind, const void *x, int xlayout, double sx, int wkind, const void *w, double sw,
                         const int64_t xs[5], const int64_t ws[5], const int32_t st[3], const int32_t pad[3],
                         const int32_t dil[3], const int64_t *pts, int64_t npts, double *y)
{
    conv_problem p;
    if (setup(&p, xkind, x, xlayout, sx, wkind, w, sw, xs, ws, st, pad, dil))
        return -1;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t *q = pts + 5 * i;
        if (q[0] < 0 || q[0] >= p.N || q[1] < 0 || q[1] >= p.K || q[2] < 0 || q[2] >= p.Do || q[3] < 0 ||
            q[3] >= p.Ho || q[4] < 0 || q[4] >= p.Wo)
            return -2;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t *q = pts + 5 * i;
        y[i] = conv_point(&p, q[0], q[1], q[2], q[3], q[4]);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gradients                                                                */
/* ------------------------------------------------------------------------ */

/* dy element (NCDHW, N x K x Do x Ho x Wo) */
static double dy_at(const conv_problem *p, int dykind, const void *dy, int64_t n, int64_t k, int64_t od, int64_t oh,
                    int64_t ow)
{
    return operand(dykind, dy, (((n * p->K + k) * p->Do + od) * p->Ho + oh) * p->Wo + ow, 1.0);
}

/* Output index o that a tap at offset tap*dil reads input index i from: o*st - pad + tap*dil == i. */
static int64_t tap_source(int64_t i, int64_t tap, int64_t st, int64_t pad, int64_t dil, int64_t out)
{
    int64_t num = i + pad - tap * dil;
    if (num < 0 || num % st != 0 || num / st >= out)
        return -1;
    return num / st;
}

/*
 * Gradient with respect to x: dx (N, C, D, H, W) in the layout xlayout. Every
 * input element gathers the dy elements whose receptive field reads it.
 */
int oracle_conv3d_bwd_data(int dykind, const void *dy, int wkind, const void *w, int xlayout, const int64_t xs[5],
                           const int64_t ws[5], const int32_t st[3], const int32_t pad[3], const int32_t dil[3],
                           double *dx)
{
    conv_problem p;
    if (setup(&p, ORACLE_F64, 0, xlayout, 1.0, wkind, w, 1.0, xs, ws, st, pad, dil))
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t n = 0; n < p.N; ++n)
        for (int64_t c = 0; c < p.C; ++c)
            for (int64_t d = 0; d < p.D; ++d)
                for (int64_t h = 0; h < p.H; ++h)
                    for (int64_t x = 0; x < p.W; ++x) {
                        double acc = 0.0;
                        for (int64_t k = 0; k < p.K; ++k)
                            for (int64_t t = 0; t < p.T; ++t) {
                                int64_t od = tap_source(d, t, p.sd, p.pd, p.dd, p.Do);
                                if (od < 0)
                                    continue;
                                for (int64_t r = 0; r < p.R; ++r) {
                                    int64_t oh = tap_source(h, r, p.sh, p.ph, p.dh, p.Ho);
                                    if (oh < 0)
                                        continue;
                                    for (int64_t s = 0; s < p.S; ++s) {
                                        int64_t ow = tap_source(x, s, p.sw_, p.pw, p.dw, p.Wo);
                                        if (ow < 0)
                                            continue;
                                        int64_t wi = (((k * p.C + c) * p.T + t) * p.R + r) * p.S + s;
                                        acc += dy_at(&p, dykind, dy, n, k, od, oh, ow) * operand(p.wkind, w, wi, 1.0);
                                    }
                                }
                            }
                        dx[x_index(&p, n, c, d, h, x)] = acc;
                    }
    return 0;
}

/*
 * Gradient with respect to w: dw (K, C, T, R, S). Every filter element sums
 * dy times the input element its tap reads, over images and output positions.
 */
int oracle_conv3d_bwd_weight(int xkind, const void *x, int xlayout, int dykind, const void *dy, const int64_t xs[5],
                             const int64_t ws[5], const int32_t st[3], const int32_t pad[3], const int32_t dil[3],
                             double *dw)
{
    conv_problem p;
    if (setup(&p, xkind, x, xlayout, 1.0, ORACLE_F64, 0, 1.0, xs, ws, st, pad, dil))
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t k = 0; k < p.K; ++k)
        for (int64_t c = 0; c < p.C; ++c)
            for (int64_t t = 0; t < p.T; ++t)
                for (int64_t r = 0; r < p.R; ++r)
                    for (int64_t s = 0; s < p.S; ++s) {
                        double acc = 0.0;
                        for (int64_t n = 0; n < p.N; ++n)
                            for (int64_t od = 0; od < p.Do; ++od)
                                for (int64_t oh = 0; oh < p.Ho; ++oh)
                                    for (int64_t ow = 0; ow < p.Wo; ++ow) {
                                        int64_t id = od * p.sd - p.pd + t * p.dd;
                                        int64_t ih = oh * p.sh - p.ph + r * p.dh;
                                        int64_t iw = ow * p.sw_ - p.pw + s * p.dw;
                                        if (id < 0 || id >= p.D || ih < 0 || ih >= p.H || iw < 0 || iw >= p.W)
                                            continue; /* zero padding */
                                        acc += dy_at(&p, dykind, dy, n, k, od, oh, ow) *
                                               operand(p.xkind, x, x_index(&p, n, c, id, ih, iw), 1.0);
                                    }
                        dw[(((k * p.C + c) * p.T + t) * p.R + r) * p.S + s] = acc;
                    }
    return 0;
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Plain CPU oracle for grouped 1D/2D convolution backward-weight (wgrad).
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP path in grouped_convolution_backward_amd/.
 *
 * What it computes (Composable Kernel doxygen page, "grouped_convolution_
 * backward_weight_kernel.hpp": the NWGC/GKXC/NWGK and NHWGC/GKYXC/NHWGK
 * argument constructors fix the three layouts and the per-group base offsets
 * group_stride_a = K, group_stride_b = C, group_stride_c = K*C*prod(filter);
 * the operator() comment "conv_bwd_weight = Out * In = Weight" fixes the
 * operands). With per-group channel counts cpg = C/G and kpg = K/G:
 *
 *   dW[g,k,y,x,c] = sum_{n<N} sum_{ho<Ho} sum_{wo<Wo}
 *                     [0 <= hi < Hi and 0 <= wi < Wi]
 *                     * dY[n,ho,wo,g,k] * X[n,hi,wi,g,c],
 *   hi = ho*s_h - pl_h + y*d_h,   wi = wo*s_w - pl_w + x*d_w.
 *
 * 1D drops the h axis (Hi = Ho = Y = 1). Every bf16/fp16 input is widened to
 * fp64 (exact) and each output element is one fp64 sum in ascending
 * (n, ho, wo) order, so the result is deterministic. Alongside dW it returns
 * sum |dY*X| per element, which scales the acceptance bound.
 *
 * Readings where the pages are silent (each listed in the design doc):
 *   - C and K are totals; cpg = C/G and kpg = K/G must be whole.
 *   - Ho = floor((Hi + pl + ph - d*(Y-1) - 1)/s) + 1; only the left pad
 *     enters the input index, the right pad only sizes Ho.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Mirrors the fields of the problem; every field is int64 so that the
 * Python side can fill it with a flat array. */
typedef struct {
    int64_t ndim;          /* 1 or 2 */
    int64_t G, N, C, K;    /* C, K are totals over all groups */
    int64_t in_len[2];     /* (Hi, Wi); 1D uses in_len[0] only */
    int64_t filt_len[2];   /* (Y, X) */
    int64_t stride[2];
    int64_t dilation[2];
    int64_t pad_lo[2];
    int64_t pad_hi[2];
    int64_t in_dtype;      /* 0 = bf16, 1 = fp16 */
} oracle_problem;

enum { ORC_BF16 = 0, ORC_FP16 = 1 };

/* bf16 is the top half of an IEEE binary32; widening is a shift. */
static double widen_bf16(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double widen_fp16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* zero or subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Spatial extents in (h, w) order; a 1D problem is a 2D one with h of size 1. */
typedef struct {
    int64_t Hi, Wi, Y, X, sh, sw, dh, dw, ph, pw, Ho, Wo;
} geom;

static int make_geom(const oracle_problem* p, geom* g)
{
    int64_t hi_pad = 0, wi_pad = 0;
    if (p->ndim == 2) {
        g->Hi = p->in_len[0];   g->Wi = p->in_len[1];
        g->Y = p->filt_len[0];  g->X = p->filt_len[1];
        g->sh = p->stride[0];   g->sw = p->stride[1];
        g->dh = p->dilation[0]; g->dw = p->dilation[1];
        g->ph = p->pad_lo[0];   g->pw = p->pad_lo[1];
        hi_pad = p->pad_lo[0] + p->pad_hi[0];
        wi_pad = p->pad_lo[1] + p->pad_hi[1];
    } else if (p->ndim == 1) {
        g->Hi = 1; g->Y = 1; g->sh = 1; g->dh = 1; g->ph = 0;
        g->Wi = p->in_len[0];  g->X = p->filt_len[0];
        g->sw = p->stride[0];  g->dw = p->dilation[0];
        g->pw = p->pad_lo[0];
        wi_pad = p->pad_lo[0] + p->pad_hi[0];
    } else {
        return -1;
    }
    if (g->sh < 1 || g->sw < 1 || g->dh < 1 || g->dw < 1) return -1;
    {
        int64_t nh = g->Hi + hi_pad - g->dh * (g->Y - 1) - 1;
        int64_t nw = g->Wi + wi_pad - g->dw * (g->X - 1) - 1;
        if (nh < 0 || nw < 0) return -1;
        g->Ho = nh / g->sh + 1;
        g->Wo = nw / g->sw + 1;
    }
    return 0;
}

/* Output spatial size; returns -1 for an invalid problem. */
int oracle_out_len(const oracle_problem* p, int64_t* ho, int64_t* wo)
{
    geom g;
    if (make_geom(p, &g)) return -1;
    *ho = g.Ho;
    *wo = g.Wo;
    return 0;
}

static double* widen_all(const uint16_t* src, int64_t n, int64_t dtype)
{
    double* d = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!d) return NULL;
    for (int64_t i = 0; i < n; ++i)
        d[i] = dtype == ORC_FP16 ? widen_fp16(src[i]) : widen_bf16(src[i]);
    return d;
}

/* One output element: the sum over (n, ho, wo) in ascending order. */
static void one_element(const geom* g, int64_t N, int64_t C, int64_t K,
                        const double* xs, const double* dys,
                        int64_t gi, int64_t cpg, int64_t kt,
                        int64_t y, int64_t x, int64_t c,
                        double* acc_out, double* abs_out)
{
    double acc = 0.0, ab = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t ho = 0; ho < g->Ho; ++ho) {
            int64_t hi = ho * g->sh - g->ph + y * g->dh;
            if (hi < 0 || hi >= g->Hi) continue;
            for (int64_t wo = 0; wo < g->Wo; ++wo) {
                int64_t wi = wo * g->sw - g->pw + x * g->dw;
                if (wi < 0 || wi >= g->Wi) continue;
                double dy = dys[((n * g->Ho + ho) * g->Wo + wo) * K + kt];
                double xv = xs[((n * g->Hi + hi) * g->Wi + wi) * C + gi * cpg + c];
                double prod = dy * xv;
                acc += prod;
                ab += fabs(prod);
            }
        }
    *acc_out = acc;
    *abs_out = ab;
}

/*
 * Full dW in GKYXC order (k_tot = g*kpg + k outer, then y, x, c), fp64.
 * x: N*Hi*Wi*C 16-bit patterns; dy: N*Ho*Wo*K 16-bit patterns.
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 on a bad problem
 * or allocation failure.
 */
int oracle_wgrad(const oracle_problem* p, const uint16_t* x, const uint16_t* dy,
                 double* dw, double* absdw, int nthreads)
{
    geom g;
    if (make_geom(p, &g)) return -1;
    if (p->G < 1 || p->C % p->G || p->K % p->G || p->N < 0) return -1;
    const int64_t cpg = p->C / p->G, kpg = p->K / p->G;
    const int64_t nx = p->N * g.Hi * g.Wi * p->C;
    const int64_t ndy = p->N * g.Ho * g.Wo * p->K;
    double* xs = widen_all(x, nx, p->in_dtype);
    double* dys = widen_all(dy, ndy, p->in_dtype);
    if (!xs || !dys) { free(xs); free(dys); return -1; }
    const int64_t per_k = g.Y * g.X * cpg;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t kt = 0; kt < p->K; ++kt) {
        const int64_t gi = kt / kpg;
        for (int64_t y = 0; y < g.Y; ++y)
            for (int64_t xx = 0; xx < g.X; ++xx)
                for (int64_t c = 0; c < cpg; ++c) {
                    int64_t e = kt * per_k + (y * g.X + xx) * cpg + c;
                    one_element(&g, p->N, p->C, p->K, xs, dys, gi, cpg, kt, y, xx, c,
                                &dw[e], &absdw[e]);
                }
    }
    free(xs);
    free(dys);
    return 0;
}

/*
 * The same sums for a list of flat GKYXC indices only (for full-size
 * problems, where the whole dW would take too long on the CPU).
 */
int oracle_wgrad_sampled(const oracle_problem* p, const uint16_t* x, const uint16_t* dy,
                         int64_t nidx, const int64_t* idx, double* dw, double* absdw,
                         int nthreads)
{
    geom g;
    if (make_geom(p, &g)) return -1;
    if (p->G < 1 || p->C % p->G || p->K % p->G || p->N < 0) return -1;
    const int64_t cpg = p->C / p->G, kpg = p->K / p->G;
    const int64_t nx = p->N * g.Hi * g.Wi * p->C;
    const int64_t ndy = p->N * g.Ho * g.Wo * p->K;
    const int64_t total = p->K * g.Y * g.X * cpg;
    for (int64_t i = 0; i < nidx; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;
    double* xs = widen_all(x, nx, p->in_dtype);
    double* dys = widen_all(dy, ndy, p->in_dtype);
    if (!xs || !dys) { free(xs); free(dys); return -1; }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t i = 0; i < nidx; ++i) {
        int64_t e = idx[i];
        int64_t c = e % cpg;
        int64_t t = e / cpg;
        int64_t xx = t % g.X;  t /= g.X;
        int64_t y = t % g.Y;
        int64_t kt = t / g.Y;
        one_element(&g, p->N, p->C, p->K, xs, dys, kt / kpg, cpg, kt, y, xx, c,
                    &dw[i], &absdw[i]);
    }
    free(xs);
    free(dys);
    return 0;
}

/* Widening of a buffer of 16-bit patterns, exposed so that tests can pin it. */
int oracle_widen(const uint16_t* src, int64_t n, int64_t dtype, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORC_FP16 ? widen_fp16(src[i]) : widen_bf16(src[i]);
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

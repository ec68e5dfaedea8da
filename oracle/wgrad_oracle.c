/*
 * Plain CPU oracle for grouped 1D/2D convolution backward-weight (wgrad).
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP path in grouped_convolution_backward_amd/.
 *
 * What it computes (Composable Kernel doxygen page, "grouped_convolution_
 * backward_weight_kernel.hpp": the NWGC/GKXC/NWGK, NHWGC/GKYXC/NHWGK and
 * NDHWGC/GKZYXC/NDHWGK argument constructors fix the layouts and the
 * per-group base offsets group_stride_a = K, group_stride_b = C,
 * group_stride_c = K*C*prod(filter); the comment in operator() fixes the
 * operands: the weight gradient is formed from the output gradient and the
 * input). With per-group
 * channel counts cpg = C/G and kpg = K/G:
 *
 *   dW[g,k,z,y,x,c] = sum_{n<N} sum_{do<Do} sum_{ho<Ho} sum_{wo<Wo}
 *                       [0 <= di < Di and 0 <= hi < Hi and 0 <= wi < Wi]
 *                       * dY[n,do,ho,wo,g,k] * X[n,di,hi,wi,g,c],
 *   di = do*s_d - pl_d + z*d_d,  hi = ho*s_h - pl_h + y*d_h,
 *   wi = wo*s_w - pl_w + x*d_w.
 *
 * 2D drops the d axis (Di = Do = Z = 1) and 1D the h axis as well. Every
 * bf16/fp16 input is widened to fp64 (exact) and each output element is one
 * fp64 sum in ascending (n, do, ho, wo) order, so the result is
 * deterministic. Alongside dW it returns sum |dY*X| per element, which
 * scales the acceptance bound.
 *
 * Readings where the pages are silent:
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

/* Threads of the last parallel loop (for tests). Each call sets its thread
 * count with a num_threads clause on its own loop, never through the global
 * OpenMP setting, so one call's request does not leak into the next. */
static int g_last_threads = 1;

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Called from each iteration of a parallel loop: every thread of the team
 * records the team size (the same value), so it is set even when some
 * threads get no iteration. */
static void note_threads(void)
{
#ifdef _OPENMP
    const int n = omp_get_num_threads();
#pragma omp atomic write
    g_last_threads = n;
#else
    g_last_threads = 1;
#endif
}

/* Mirrors the fields of the problem; every field is int64 so that the
 * Python side can fill it with a flat array. */
typedef struct {
    int64_t ndim;          /* 1, 2 or 3 */
    int64_t G, N, C, K;    /* C, K are totals over all groups */
    int64_t in_len[3];     /* the first ndim of (Di, Hi, Wi), outermost first:
                              3D (Di, Hi, Wi), 2D (Hi, Wi), 1D (Wi) */
    int64_t filt_len[3];   /* likewise (Z, Y, X) */
    int64_t stride[3];
    int64_t dilation[3];
    int64_t pad_lo[3];
    int64_t pad_hi[3];
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

/* Spatial extents along (d, h, w); missing leading axes have size 1. */
typedef struct {
    int64_t in[3], f[3], s[3], dl[3], pl[3], out[3];
} geom;

static int make_geom(const oracle_problem* p, geom* g)
{
    if (p->ndim < 1 || p->ndim > 3) return -1;
    const int64_t lead = 3 - p->ndim;   /* axes the problem does not have */
    for (int a = 0; a < 3; ++a) {
        if (a < lead) {
            g->in[a] = 1; g->f[a] = 1; g->s[a] = 1; g->dl[a] = 1; g->pl[a] = 0;
            g->out[a] = 1;
            continue;
        }
        const int i = a - (int)lead;
        g->in[a] = p->in_len[i];  g->f[a] = p->filt_len[i];
        g->s[a] = p->stride[i];   g->dl[a] = p->dilation[i];
        g->pl[a] = p->pad_lo[i];
        if (g->s[a] < 1 || g->dl[a] < 1) return -1;
        int64_t span = g->in[a] + p->pad_lo[i] + p->pad_hi[i] - g->dl[a] * (g->f[a] - 1) - 1;
        if (span < 0) return -1;
        g->out[a] = span / g->s[a] + 1;
    }
    return 0;
}

/* Output spatial sizes along (d, h, w) (1 for axes the problem does not
 * have); returns -1 for an invalid problem. */
int oracle_out_len(const oracle_problem* p, int64_t* od, int64_t* oh, int64_t* ow)
{
    geom g;
    if (make_geom(p, &g)) return -1;
    *od = g.out[0];
    *oh = g.out[1];
    *ow = g.out[2];
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

/* One output element: the sum over (n, do, ho, wo) in ascending order;
 * (z, y, x) is the filter tap. */
static void one_element(const geom* g, int64_t N, int64_t C, int64_t K,
                        const double* xs, const double* dys,
                        int64_t gi, int64_t cpg, int64_t kt,
                        int64_t z, int64_t y, int64_t x, int64_t c,
                        double* acc_out, double* abs_out)
{
    const int64_t Di = g->in[0], Hi = g->in[1], Wi = g->in[2];
    const int64_t Do = g->out[0], Ho = g->out[1], Wo = g->out[2];
    double acc = 0.0, ab = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t od = 0; od < Do; ++od) {
            int64_t di = od * g->s[0] - g->pl[0] + z * g->dl[0];
            if (di < 0 || di >= Di) continue;
            for (int64_t ho = 0; ho < Ho; ++ho) {
                int64_t hi = ho * g->s[1] - g->pl[1] + y * g->dl[1];
                if (hi < 0 || hi >= Hi) continue;
                for (int64_t wo = 0; wo < Wo; ++wo) {
                    int64_t wi = wo * g->s[2] - g->pl[2] + x * g->dl[2];
                    if (wi < 0 || wi >= Wi) continue;
                    double dy = dys[(((n * Do + od) * Ho + ho) * Wo + wo) * K + kt];
                    double xv = xs[(((n * Di + di) * Hi + hi) * Wi + wi) * C + gi * cpg + c];
                    double prod = dy * xv;
                    acc += prod;
                    ab += fabs(prod);
                }
            }
        }
    *acc_out = acc;
    *abs_out = ab;
}

/*
 * Full dW in GK[Z]YXC order (k_tot = g*kpg + k outer, then z, y, x, c), fp64.
 * x: N*Di*Hi*Wi*C 16-bit patterns; dy: N*Do*Ho*Wo*K 16-bit patterns.
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
    const int64_t nx = p->N * g.in[0] * g.in[1] * g.in[2] * p->C;
    const int64_t ndy = p->N * g.out[0] * g.out[1] * g.out[2] * p->K;
    double* xs = widen_all(x, nx, p->in_dtype);
    double* dys = widen_all(dy, ndy, p->in_dtype);
    if (!xs || !dys) { free(xs); free(dys); return -1; }
    const int64_t Z = g.f[0], Y = g.f[1], X = g.f[2];
    const int64_t per_k = Z * Y * X * cpg;
    const int nt = pick_threads(nthreads);
    (void)nt;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int64_t kt = 0; kt < p->K; ++kt) {
        note_threads();
        const int64_t gi = kt / kpg;
        for (int64_t z = 0; z < Z; ++z)
            for (int64_t y = 0; y < Y; ++y)
                for (int64_t xx = 0; xx < X; ++xx)
                    for (int64_t c = 0; c < cpg; ++c) {
                        int64_t e = kt * per_k + ((z * Y + y) * X + xx) * cpg + c;
                        one_element(&g, p->N, p->C, p->K, xs, dys, gi, cpg, kt, z, y, xx, c,
                                    &dw[e], &absdw[e]);
                    }
    }
    free(xs);
    free(dys);
    return 0;
}

/*
 * The same sums for a list of flat GK[Z]YXC indices only (for full-size
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
    const int64_t nx = p->N * g.in[0] * g.in[1] * g.in[2] * p->C;
    const int64_t ndy = p->N * g.out[0] * g.out[1] * g.out[2] * p->K;
    const int64_t Z = g.f[0], Y = g.f[1], X = g.f[2];
    const int64_t total = p->K * Z * Y * X * cpg;
    for (int64_t i = 0; i < nidx; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -1;
    double* xs = widen_all(x, nx, p->in_dtype);
    double* dys = widen_all(dy, ndy, p->in_dtype);
    if (!xs || !dys) { free(xs); free(dys); return -1; }
    const int nt = pick_threads(nthreads);
    (void)nt;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int64_t i = 0; i < nidx; ++i) {
        note_threads();
        int64_t e = idx[i];
        int64_t c = e % cpg;
        int64_t t = e / cpg;
        int64_t xx = t % X;  t /= X;
        int64_t y = t % Y;   t /= Y;
        int64_t z = t % Z;
        int64_t kt = t / Z;
        one_element(&g, p->N, p->C, p->K, xs, dys, kt / kpg, cpg, kt, z, y, xx, c,
                    &dw[i], &absdw[i]);
    }
    free(xs);
    free(dys);
    return 0;
}

/*
 * Backward data (dgrad) of the same convolution, fp64: the input gradient
 *
 *   dX[n,di,hi,wi,g,c] = sum_{k<kpg} sum_{z,y,x} [do, ho, wo exist]
 *                          dY[n,do,ho,wo,g,k] * W[g,k,z,y,x,c]
 *
 * where (do, ho, wo) is the output position whose tap (z, y, x) reads
 * (di, hi, wi): do = (di + pl_d - z*d_d) / s_d when that division is exact
 * and 0 <= do < Do, likewise for h and w. It is the adjoint of the forward
 * convolution's map X -> Y for a fixed W (the Composable Kernel page's
 * backward-weight kernel computes the other adjoint, W -> Y for a fixed X).
 * w: K*Z*Y*X*(C/G) 16-bit patterns in GK[Z]YXC order; dy: N*Do*Ho*Wo*K.
 * dx and absdx hold N*Di*Hi*Wi*C doubles (NDHWGC order). Each element is one
 * fp64 sum in ascending (k, z, y, x) order. Returns 0, or -1 on a bad
 * problem or allocation failure.
 */
int oracle_dgrad(const oracle_problem* p, const uint16_t* dy, const uint16_t* w,
                 double* dx, double* absdx, int nthreads)
{
    geom g;
    if (make_geom(p, &g)) return -1;
    if (p->G < 1 || p->C % p->G || p->K % p->G || p->N < 0) return -1;
    const int64_t cpg = p->C / p->G, kpg = p->K / p->G;
    const int64_t Di = g.in[0], Hi = g.in[1], Wi = g.in[2];
    const int64_t Do = g.out[0], Ho = g.out[1], Wo = g.out[2];
    const int64_t Z = g.f[0], Y = g.f[1], X = g.f[2];
    const int64_t ndy = p->N * Do * Ho * Wo * p->K;
    const int64_t nw = p->K * Z * Y * X * cpg;
    double* dys = widen_all(dy, ndy, p->in_dtype);
    double* ws = widen_all(w, nw, p->in_dtype);
    if (!dys || !ws) { free(dys); free(ws); return -1; }
    const int64_t rows = p->N * Di * Hi * Wi;
    const int nt = pick_threads(nthreads);
    (void)nt;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        note_threads();
        int64_t t = r;
        const int64_t wi = t % Wi;  t /= Wi;
        const int64_t hi = t % Hi;  t /= Hi;
        const int64_t di = t % Di;
        const int64_t n = t / Di;
        for (int64_t gi = 0; gi < p->G; ++gi)
            for (int64_t c = 0; c < cpg; ++c) {
                double acc = 0.0, ab = 0.0;
                for (int64_t k = 0; k < kpg; ++k) {
                    const int64_t kt = gi * kpg + k;
                    for (int64_t z = 0; z < Z; ++z) {
                        const int64_t nd = di + g.pl[0] - z * g.dl[0];
                        if (nd < 0 || nd % g.s[0]) continue;
                        const int64_t od = nd / g.s[0];
                        if (od >= Do) continue;
                        for (int64_t y = 0; y < Y; ++y) {
                            const int64_t nh = hi + g.pl[1] - y * g.dl[1];
                            if (nh < 0 || nh % g.s[1]) continue;
                            const int64_t ho = nh / g.s[1];
                            if (ho >= Ho) continue;
                            for (int64_t x = 0; x < X; ++x) {
                                const int64_t nwv = wi + g.pl[2] - x * g.dl[2];
                                if (nwv < 0 || nwv % g.s[2]) continue;
                                const int64_t wo = nwv / g.s[2];
                                if (wo >= Wo) continue;
                                const double a = dys[(((n * Do + od) * Ho + ho) * Wo + wo) * p->K + kt];
                                const double b = ws[(((kt * Z + z) * Y + y) * X + x) * cpg + c];
                                acc += a * b;
                                ab += fabs(a * b);
                            }
                        }
                    }
                }
                dx[r * p->C + gi * cpg + c] = acc;
                absdx[r * p->C + gi * cpg + c] = ab;
            }
    }
    free(dys);
    free(ws);
    return 0;
}

/* Widening of a buffer of 16-bit patterns, exposed so that tests can pin it. */
int oracle_widen(const uint16_t* src, int64_t n, int64_t dtype, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == ORC_FP16 ? widen_fp16(src[i]) : widen_bf16(src[i]);
    return 0;
}

/* Threads the last oracle_wgrad / oracle_wgrad_sampled / oracle_dgrad loop ran on. */
int oracle_last_threads(void)
{
    return g_last_threads;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

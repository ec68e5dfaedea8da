/*
 * Runs the CPU oracle (oracle/wgrad_oracle.c) on one problem for the
 * sanitizer build:
 *
 *   oracle_driver <op> <nthreads> <in.bin> <out.bin> ndim G N C K in_len[3]
 *                 filt_len[3] stride[3] dilation[3] pad_lo[3] pad_hi[3] in_dtype
 *
 * op 0: wgrad; in.bin holds the X bits then the dY bits (uint16), out.bin
 * receives dW then sum|dY*X| (float64, GK[Z]YXC). op 1: dgrad; in.bin holds
 * dY then W, out.bin receives dX then sum|dY*W|. The element counts come
 * from the problem (oracle_out_len). Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int64_t ndim, G, N, C, K;
    int64_t in_len[3], filt_len[3], stride[3], dilation[3], pad_lo[3], pad_hi[3];
    int64_t in_dtype;
} problem;

int oracle_wgrad(const problem*, const uint16_t*, const uint16_t*, double*, double*, int);
int oracle_dgrad(const problem*, const uint16_t*, const uint16_t*, double*, double*, int);
int oracle_out_len(const problem*, int64_t*, int64_t*, int64_t*);

int main(int argc, char** argv)
{
    if (argc != 5 + 24) return 2;
    const int op = atoi(argv[1]), nt = atoi(argv[2]);
    problem p;
    int64_t* f = &p.ndim;
    for (int i = 0; i < 24; ++i) f[i] = atoll(argv[5 + i]);
    int64_t od, oh, ow;
    if (oracle_out_len(&p, &od, &oh, &ow)) return 3;
    int64_t in_sp = 1, out_sp = 1, taps = 1;
    for (int i = 0; i < p.ndim; ++i) {
        in_sp *= p.in_len[i];
        taps *= p.filt_len[i];
    }
    const int64_t ol[3] = {od, oh, ow};
    for (int i = 3 - (int)p.ndim; i < 3; ++i) out_sp *= ol[i];
    const int64_t nx = p.N * in_sp * p.C, ndy = p.N * out_sp * p.K, nw = p.K * taps * (p.C / p.G);
    const int64_t na = op == 0 ? nx : ndy, nb = op == 0 ? ndy : nw, nout = op == 0 ? nw : nx;
    uint16_t* in = malloc(sizeof(uint16_t) * (size_t)(na + nb + 1));
    double* out = malloc(sizeof(double) * (size_t)(2 * nout + 1));
    if (!in || !out) return 4;
    FILE* fi = fopen(argv[3], "rb");
    if (!fi || fread(in, sizeof(uint16_t), (size_t)(na + nb), fi) != (size_t)(na + nb)) return 5;
    fclose(fi);
    const int rc = op == 0 ? oracle_wgrad(&p, in, in + na, out, out + nout, nt)
                           : oracle_dgrad(&p, in, in + na, out, out + nout, nt);
    if (rc) return 6;
    FILE* fo = fopen(argv[4], "wb");
    if (!fo || fwrite(out, sizeof(double), (size_t)(2 * nout), fo) != (size_t)(2 * nout)) return 7;
    fclose(fo);
    free(in);
    free(out);
    return 0;
}

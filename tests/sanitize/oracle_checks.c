/* Runs every entry point of the fp64 oracle (oracle/oracle.c) on small
 * seeded inputs, edge shapes included (one token, one channel, one state,
 * H != W grids, more threads than units). Built with gcc under
 * -fsanitize=address,undefined by tests/test_sanitizers.py: an out-of-bounds
 * access, a use after free, a leak or undefined behaviour aborts the run.
 * Values are checked elsewhere (the oracle's pins); here only that every call
 * succeeds and returns finite numbers. Test infrastructure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_scan_ex_f64(int batch, int dim, int dstate, long L, long H, long W, int ndir,
                       const int* order, const double* u, int per_direction, const double* delta,
                       const double* z, const double* B, const double* C, int bc_per_direction,
                       const double* A, const double* Dskip, const double* dt_bias,
                       int delta_softplus, double* y, int nthreads);
int oracle_vim_bidir_f64(int batch, int dim, int dstate, long L, const double* u,
                         const double* delta, const double* z, const double* B, const double* C,
                         const double* A, const double* Dskip, const double* dt_bias,
                         int delta_softplus, double* y, int nthreads);
int oracle_cross4_f64(int batch, int dim, int dstate, long H, long W, const double* u,
                      const double* delta, const double* z, const double* B, const double* C,
                      const double* A, const double* Dskip, const double* dt_bias,
                      int delta_softplus, double* y, int nthreads);
int oracle_s6_1d_f64(int batch, int dim, int dstate, long L, int reverse, const double* u,
                     const double* delta, const double* z, const double* B, const double* C,
                     const double* A, const double* Dskip, const double* dt_bias,
                     int delta_softplus, double* y, int nthreads);
int oracle_vim_conv_f64(int batch, int dim, int dstate, long L, const double* x,
                        const double* conv_w, const double* conv_b, const double* delta,
                        const double* z, const double* B, const double* C, const double* A,
                        const double* Dskip, const double* dt_bias, int delta_softplus,
                        double* y, int nthreads);
int oracle_vim_bidir_grad_f64(int batch, int dim, int dstate, long L, const double* u,
                              const double* delta, const double* z, const double* B,
                              const double* C, const double* A, const double* Dskip,
                              const double* dt_bias, int delta_softplus, const double* g,
                              double* du, double* ddelta, double* dz, double* dB, double* dC,
                              double* dA, double* dD, double* dbias, int nthreads);
int oracle_linear_f64(int batch, int M, int K, long L, const double* W, const double* in,
                      const double* bias, const double* residual, double* out);
int oracle_dt_proj_f64(int batch, int dim, long L, const double* dt, const double* w,
                       double* delta);

static uint64_t state = 0x9e3779b97f4a7c15ull;

static double uniform(void)     /* splitmix64, mapped to [-1, 1) */
{
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

/* an exactly sized heap array, so that any read past the end is caught */
static double* arr(long n, double scale, double shift)
{
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!a) { fprintf(stderr, "out of memory\n"); exit(2); }
    for (long i = 0; i < n; ++i) a[i] = shift + scale * uniform();
    return a;
}

static void finite(const double* a, long n, const char* what)
{
    for (long i = 0; i < n; ++i)
        if (!isfinite(a[i])) { fprintf(stderr, "%s: non-finite output at %ld\n", what, i); exit(1); }
}

static void ok(int rc, const char* what)
{
    if (rc != 0) { fprintf(stderr, "%s: status %d\n", what, rc); exit(1); }
}

/* one shape through every scan entry point */
static void shape(int batch, int dim, int N, long H, long W, int threads)
{
    const long L = H * W, e = (long)batch * dim * L;
    double* u = arr(2 * e, 1.0, 0.0);           /* two copies for the per-direction form */
    double* dl = arr(2 * e, 0.5, 0.0);
    double* z = arr(e, 1.0, 0.0);
    double* B = arr((long)batch * 4 * N * L, 1.0, 0.0);
    double* C = arr((long)batch * 4 * N * L, 1.0, 0.0);
    double* A = arr(4L * dim * N, 0.5, -1.0);
    double* D = arr(4L * dim, 1.0, 0.0);
    double* bias = arr(4L * dim, 1.0, -3.0);
    double* cw = arr(2L * dim * 3, 0.6, 0.0);
    double* cb = arr(2L * dim, 0.2, 0.0);
    double* g = arr(e, 1.0, 0.0);
    double* y = arr(e, 0.0, 0.0);
    ok(oracle_vim_bidir_f64(batch, dim, N, L, u, dl, z, B, C, A, D, bias, 1, y, threads), "vim");
    finite(y, e, "vim");
    ok(oracle_vim_bidir_f64(batch, dim, N, L, u, dl, NULL, B, C, A, NULL, NULL, 3, y, threads),
       "vim zoh");
    finite(y, e, "vim zoh");
    ok(oracle_cross4_f64(batch, dim, N, H, W, u, dl, z, B, C, A, D, bias, 1, y, threads), "cross4");
    finite(y, e, "cross4");
    ok(oracle_s6_1d_f64(batch, dim, N, L, 1, u, dl, z, B, C, A, D, bias, 1, y, threads), "1d");
    finite(y, e, "1d");
    const int order[2] = {0, 1};
    ok(oracle_scan_ex_f64(batch, dim, N, L, 0, 0, 2, order, u, 3, dl, z, B, C, 1, A, D, bias, 1,
                          y, threads), "per-direction");
    finite(y, e, "per-direction");
    ok(oracle_vim_conv_f64(batch, dim, N, L, u, cw, cb, dl, z, B, C, A, D, bias, 1, y, threads),
       "conv");
    finite(y, e, "conv");
    double* du = arr(e, 0.0, 0.0);
    double* dd = arr(e, 0.0, 0.0);
    double* dz = arr(e, 0.0, 0.0);
    double* dB = arr((long)batch * N * L, 0.0, 0.0);
    double* dC = arr((long)batch * N * L, 0.0, 0.0);
    double* dA = arr(2L * dim * N, 0.0, 0.0);
    double* dD = arr(2L * dim, 0.0, 0.0);
    double* db = arr(2L * dim, 0.0, 0.0);
    ok(oracle_vim_bidir_grad_f64(batch, dim, N, L, u, dl, z, B, C, A, D, bias, 1, g, du, dd, dz,
                                 dB, dC, dA, dD, db, threads), "grad");
    finite(du, e, "grad du");
    finite(dB, (long)batch * N * L, "grad dB");
    finite(dA, 2L * dim * N, "grad dA");
    double* Wt = arr((long)dim * dim, 0.3, 0.0);
    ok(oracle_linear_f64(batch, dim, dim, L, Wt, u, D, z, y), "linear");
    finite(y, e, "linear");
    ok(oracle_dt_proj_f64(batch, dim, L, g, D, y), "dt_proj");
    double* to_free[] = {u, dl, z, B, C, A, D, bias, cw, cb, g, y, du, dd, dz, dB, dC, dA, dD, db, Wt};
    for (size_t i = 0; i < sizeof(to_free) / sizeof(to_free[0]); ++i) free(to_free[i]);
}

int main(void)
{
    shape(1, 1, 1, 1, 1, 1);        /* one token, one channel, one state */
    shape(2, 3, 16, 5, 7, 4);       /* H != W, more threads than some loops have units */
    shape(1, 2, 8, 9, 4, 16);       /* more threads than units */
    shape(3, 5, 12, 1, 33, 2);      /* a one-row grid */
    /* arguments the oracle must refuse without touching memory */
    const int bad_order[1] = {7};
    double one = 1.0;
    if (oracle_scan_ex_f64(1, 1, 1, 1, 1, 1, 1, bad_order, &one, 0, &one, NULL, &one, &one, 0,
                           &one, NULL, NULL, 1, &one, 1) != -1) {
        fprintf(stderr, "bad order accepted\n");
        return 1;
    }
    printf("oracle checks ok\n");
    return 0;
}

/*
 * oracle.c -- plain fp64 CPU reference of the selective scan (S6) that Vision
 * Mamba runs forward and backward and VMamba runs in four cross-scan orders.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load or call this library. The HIP
 * product path never links, imports or calls it, and it shares no code,
 * header or table with that path.
 *
 * Everything below is the sequential definition written out, step by step,
 * in double precision, with no blocking, fusion or reordering beyond what the
 * definition states. Sources (all on "Vision Mamba Guide: Efficient
 * Bidirectional SSM & VMamba", aifetchly blog, unless noted):
 *
 *  - Continuous-Time State Space Equations: y = C h + D x, D a scalar skip.
 *  - Discretization via Zero-Order Hold: A_bar = exp(delta A); B_bar is
 *    approximated by delta B (the form the page's code uses), or, on
 *    request, the exact hold (exp(delta A) - 1) / A B the same section states
 *    first; recurrence h_t = A_bar h_{t-1} + B_bar x_t, read-out y_t = C h_t.
 *  - The Selective State Space (S6) Mechanism box: delta_t = softplus(...),
 *    B_t, C_t input dependent, so A_bar and B_bar change with t.
 *  - PyTorch code, SimpleSelectiveSSM.forward: h starts at zero, A is
 *    diagonal (one decay per state), B_t and C_t are shared by all channels.
 *  - 2. The Bidirectional Mamba Block: forward pass over tokens 1..N+1,
 *    backward pass from N+1 down to 1; gated fusion
 *    (y_f + y_b) * sigma(z) with sigma the SiLU.
 *  - VMamba, 1. Cross-Scan Traversal and the CrossScan2D code: four orders
 *    (row-major, its reverse, column-major, its reverse); 3. Cross-Merge:
 *    every sequence mapped back to (h, w) and the four maps summed.
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reason in the design notes):
 *  - D is applied per direction (y_k += D_k u); D = 0 disables it.
 *  - delta_raw + dt_bias goes through softplus when bit 0 of the flags
 *    word (the delta_softplus argument) is set; bit 1 selects the exact
 *    zero-order-hold B_bar.
 *  - Vim directions share u, delta_raw, z, B and C (spatial order); VMamba
 *    directions share u, delta_raw (spatial order) and have their own B and C,
 *    stored in each direction's scan order.
 *  - The gate, when z is given, multiplies the merged sum by z * sigmoid(z).
 *
 * Build: gcc -O2 -fPIC -shared oracle.c -o liboracle.so -lm -lpthread
 * (no -ffast-math: every operation is IEEE double).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* Direction kinds: the order in which a direction visits the tokens. */
enum { ORD_FORWARD = 0, ORD_REVERSE = 1, ORD_COLUMN = 2, ORD_COLUMN_REVERSE = 3 };

/* Token index (row-major, p = i*W + j) visited at scan step t.
 * ORD_COLUMN walks down each column from the top, columns left to right,
 * which is what the page's x.permute(0, 3, 2, 1).reshape(B, L, C) produces. */
static long visit(int order, long t, long L, long H, long W)
{
    switch (order) {
    case ORD_FORWARD: return t;
    case ORD_REVERSE: return L - 1 - t;
    case ORD_COLUMN: return (t % H) * W + t / H;
    default: { long r = L - 1 - t; return (r % H) * W + r / H; }
    }
}

/* softplus(x) = log(1 + e^x), written in the form that neither overflows
 * nor loses the small result for very negative x. */
static double softplus(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

#define PER_DIR_U 1
#define PER_DIR_DELTA 2

typedef struct {
    int batch, dim, dstate;
    long L, H, W;
    int ndir;
    const int* order;       /* [ndir] */
    const double *u, *delta, *z, *B, *C, *A, *Dskip, *dt_bias;
    int bc_per_direction;   /* 0: B, C are [batch][dstate][L] in token order;
                               1: [batch][ndir][dstate][L] in scan order */
    int per_direction;      /* bit 0 (PER_DIR_U): u is [ndir][batch][dim][L], one per
                               direction, else [batch][dim][L], shared; bit 1
                               (PER_DIR_DELTA): the same for delta_raw */
    int delta_softplus;
    int zoh;                /* B_bar = (exp(delta A) - 1) / A B, else delta B */
    double* y;
    /* work split */
    long unit_begin, unit_end;
} job_t;

/* One (batch, channel) unit: every direction's recurrence, then the merge
 * and the gate, for all tokens of that unit. */
static void run_unit(const job_t* J, long unit, double* h, double* acc)
{
    const long b = unit / J->dim, d = unit % J->dim;
    const long L = J->L, N = J->dstate;
    const long copy = (long)J->batch * J->dim * L;       /* elements of one direction's copy */
    double* y = J->y + (b * J->dim + d) * L;

    for (long p = 0; p < L; ++p) acc[p] = 0.0;

    for (int k = 0; k < J->ndir; ++k) {
        const double* u = J->u + ((J->per_direction & PER_DIR_U) ? k * copy : 0)
                          + (b * J->dim + d) * L;
        const double* dl = J->delta + ((J->per_direction & PER_DIR_DELTA) ? k * copy : 0)
                           + (b * J->dim + d) * L;
        const double* A = J->A + ((long)k * J->dim + d) * N;
        const double Dk = J->Dskip ? J->Dskip[(long)k * J->dim + d] : 0.0;
        const double bias = J->dt_bias ? J->dt_bias[(long)k * J->dim + d] : 0.0;
        const double *Bk, *Ck;
        if (J->bc_per_direction) {
            Bk = J->B + ((long)b * J->ndir + k) * N * L;
            Ck = J->C + ((long)b * J->ndir + k) * N * L;
        } else {
            Bk = J->B + (long)b * N * L;
            Ck = J->C + (long)b * N * L;
        }
        for (long n = 0; n < N; ++n) h[n] = 0.0;           /* zero initial state */
        for (long t = 0; t < L; ++t) {
            const long p = visit(J->order[k], t, L, J->H, J->W);
            /* index of this step's B_t, C_t row entry */
            const long q = J->bc_per_direction ? t : p;
            const double x = dl[p] + bias;
            const double delta = J->delta_softplus ? softplus(x) : x;
            double yk = 0.0;
            for (long n = 0; n < N; ++n) {
                const double Abar = exp(delta * A[n]);              /* exp(delta A) */
                double Bbar_x = delta * Bk[n * L + q] * u[p];       /* delta B x */
                if (J->zoh)   /* exact hold: (exp(delta A) - 1) / A B x; delta B x at A = 0 */
                    Bbar_x = (A[n] != 0.0 ? expm1(A[n] * delta) / A[n] : delta) * Bk[n * L + q] * u[p];
                h[n] = Abar * h[n] + Bbar_x;
                yk += Ck[n * L + q] * h[n];                         /* C_t h_t */
            }
            yk += Dk * u[p];                                        /* D x_t */
            acc[p] += yk;                                           /* merge by sum */
        }
    }
    for (long p = 0; p < L; ++p) {
        double v = acc[p];
        if (J->z) {
            const double zz = J->z[(b * J->dim + d) * L + p];
            v *= zz / (1.0 + exp(-zz));                             /* SiLU gate */
        }
        y[p] = v;
    }
}

static void* worker(void* arg)
{
    const job_t* J = (const job_t*)arg;
    double* h = (double*)malloc(sizeof(double) * (size_t)J->dstate);
    double* acc = (double*)malloc(sizeof(double) * (size_t)J->L);
    if (!h || !acc) { free(h); free(acc); return (void*)1; }
    for (long unit = J->unit_begin; unit < J->unit_end; ++unit) run_unit(J, unit, h, acc);
    free(h);
    free(acc);
    return NULL;
}

/* Generic entry: ndir directions with the given visiting orders; u and
 * delta_raw each shared or one per direction (per_direction bits PER_DIR_U,
 * PER_DIR_DELTA). The guide's Vim block code gives each branch its own conv
 * and its own SimpleSelectiveSSM projections, hence its own u, delta, B, C.
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_scan_ex_f64(int batch, int dim, int dstate, long L, long H, long W,
                       int ndir, const int* order, const double* u, int per_direction,
                       const double* delta, const double* z, const double* B, const double* C,
                       int bc_per_direction, const double* A, const double* Dskip,
                       const double* dt_bias, int delta_softplus, double* y, int nthreads)
{
    if (batch < 0 || dim < 0 || dstate < 1 || L < 0 || ndir < 1 || !order) return -1;
    if (batch == 0 || dim == 0 || L == 0) return 0;
    if (!u || !delta || !B || !C || !A || !y) return -1;
    for (int k = 0; k < ndir; ++k) {
        if (order[k] < 0 || order[k] > 3) return -1;
        if (order[k] >= ORD_COLUMN && (H < 1 || W < 1 || H * W != L)) return -1;
    }
    const long units = (long)batch * dim;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        job_t* J = &jobs[i];
        J->batch = batch; J->dim = dim; J->dstate = dstate;
        J->L = L; J->H = H; J->W = W; J->ndir = ndir; J->order = order;
        J->u = u; J->delta = delta; J->z = z; J->B = B; J->C = C;
        J->A = A; J->Dskip = Dskip; J->dt_bias = dt_bias;
        J->bc_per_direction = bc_per_direction;
        J->delta_softplus = delta_softplus & 1;
        J->zoh = (delta_softplus & 2) != 0;
        J->per_direction = per_direction & (PER_DIR_U | PER_DIR_DELTA);
        J->y = y;
        J->unit_begin = units * i / nthreads;
        J->unit_end = units * (i + 1) / nthreads;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &jobs[i]) != 0) break;
        started = i;
    }
    if (worker(&jobs[0]) != NULL) rc = -2;
    for (int i = 1; i <= started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -2;
    }
    /* units a failed pthread_create left undone run on this thread */
    for (int i = started + 1; i < nthreads; ++i)
        if (worker(&jobs[i]) != NULL) rc = -2;
    free(jobs);
    free(th);
    return rc;
}

/* The shared-u scan (the Vim and VMamba entries below use it). */
int oracle_scan_f64(int batch, int dim, int dstate, long L, long H, long W,
                    int ndir, const int* order, const double* u, const double* delta,
                    const double* z, const double* B, const double* C, int bc_per_direction,
                    const double* A, const double* Dskip, const double* dt_bias,
                    int delta_softplus, double* y, int nthreads)
{
    return oracle_scan_ex_f64(batch, dim, dstate, L, H, W, ndir, order, u, 0, delta, z, B, C,
                              bc_per_direction, A, Dskip, dt_bias, delta_softplus, y, nthreads);
}

/* Depthwise Conv1d with kernel 3, padding 1 and a bias, as the guide's
 * BidirectionalVisionMambaBlock applies it (conv_f, conv_b; PyTorch's Conv1d
 * is a cross-correlation): out[t] = bias + w[0] in[t-1] + w[1] in[t] +
 * w[2] in[t+1], with in[-1] = in[L] = 0. */
static void conv3(const double* in, long L, const double* w, double bias, double* out)
{
    for (long t = 0; t < L; ++t) {
        const double left = t > 0 ? in[t - 1] : 0.0;
        const double right = t + 1 < L ? in[t + 1] : 0.0;
        out[t] = bias + w[0] * left + w[1] * in[t] + w[2] * right;
    }
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* Vim with its front end: u_f = silu(conv_f(x)) feeds the forward scan and
 * u_b = silu(conv_b(flip(x))), in the flipped order, feeds the backward scan
 * (the guide's "1. Forward Branch" and "2. Backward Branch (Reverse
 * sequence)"); the D skip of each direction uses its own u. conv_w is
 * [2][dim][3], conv_b [2][dim] (NULL: no bias). u_b is stored back in token
 * order (u_b[p] is the value the backward scan reads at token p). */
int oracle_vim_conv_f64(int batch, int dim, int dstate, long L, const double* x,
                        const double* conv_w, const double* conv_b, const double* delta,
                        const double* z, const double* B, const double* C, const double* A,
                        const double* Dskip, const double* dt_bias, int delta_softplus,
                        double* y, int nthreads)
{
    if (batch < 0 || dim < 0 || L < 0 || !x || !conv_w) return -1;
    if (batch == 0 || dim == 0 || L == 0) return 0;
    const long rows = (long)batch * dim;
    double* u = (double*)malloc(sizeof(double) * (size_t)(2 * rows * L));
    double* rev = (double*)malloc(sizeof(double) * (size_t)L);
    double* c = (double*)malloc(sizeof(double) * (size_t)L);
    if (!u || !rev || !c) { free(u); free(rev); free(c); return -2; }
    for (long r = 0; r < rows; ++r) {
        const long d = r % dim;
        const double* xr = x + r * L;
        /* forward branch */
        conv3(xr, L, conv_w + d * 3, conv_b ? conv_b[d] : 0.0, c);
        for (long p = 0; p < L; ++p) u[r * L + p] = silu(c[p]);
        /* backward branch: flip, convolve, SiLU; step t of the flipped
         * sequence is token L-1-t */
        for (long t = 0; t < L; ++t) rev[t] = xr[L - 1 - t];
        conv3(rev, L, conv_w + ((long)dim + d) * 3, conv_b ? conv_b[dim + d] : 0.0, c);
        for (long t = 0; t < L; ++t) u[(rows + r) * L + (L - 1 - t)] = silu(c[t]);
    }
    free(rev);
    free(c);
    const int order[2] = {ORD_FORWARD, ORD_REVERSE};
    const int rc = oracle_scan_ex_f64(batch, dim, dstate, L, 0, 0, 2, order, u, 1, delta, z, B,
                                      C, 0, A, Dskip, dt_bias, delta_softplus, y, nthreads);
    free(u);
    return rc;
}

/* Vim bidirectional scan: forward and backward over the same tensors
 * (B, C: [batch][dstate][L]); A: [2][dim][dstate]; Dskip, dt_bias: [2][dim]. */
int oracle_vim_bidir_f64(int batch, int dim, int dstate, long L, const double* u,
                         const double* delta, const double* z, const double* B,
                         const double* C, const double* A, const double* Dskip,
                         const double* dt_bias, int delta_softplus, double* y, int nthreads)
{
    static const int order[2] = { ORD_FORWARD, ORD_REVERSE };
    return oracle_scan_f64(batch, dim, dstate, L, 0, 0, 2, order, u, delta, z, B, C, 0,
                           A, Dskip, dt_bias, delta_softplus, y, nthreads);
}

/* VMamba four-direction cross-scan on an H x W grid (L = H*W, row-major).
 * B, C: [batch][4][dstate][L], each direction's rows in its scan order. */
int oracle_cross4_f64(int batch, int dim, int dstate, long H, long W, const double* u,
                      const double* delta, const double* z, const double* B,
                      const double* C, const double* A, const double* Dskip,
                      const double* dt_bias, int delta_softplus, double* y, int nthreads)
{
    static const int order[4] = { ORD_FORWARD, ORD_REVERSE, ORD_COLUMN, ORD_COLUMN_REVERSE };
    return oracle_scan_f64(batch, dim, dstate, H * W, H, W, 4, order, u, delta, z, B, C, 1,
                           A, Dskip, dt_bias, delta_softplus, y, nthreads);
}

/* One direction (reverse = 0: forward, 1: backward) over [batch][dstate][L]
 * B, C; A: [dim][dstate]; Dskip, dt_bias: [dim]. */
int oracle_s6_1d_f64(int batch, int dim, int dstate, long L, int reverse, const double* u,
                     const double* delta, const double* z, const double* B, const double* C,
                     const double* A, const double* Dskip, const double* dt_bias,
                     int delta_softplus, double* y, int nthreads)
{
    const int order[1] = { reverse ? ORD_REVERSE : ORD_FORWARD };
    return oracle_scan_f64(batch, dim, dstate, L, 0, 0, 1, order, u, delta, z, B, C, 0,
                           A, Dskip, dt_bias, delta_softplus, y, nthreads);
}

/* ------------------------------------------------------------------------
 * Gradient of the Vim scan (oracle_vim_bidir_f64) with respect to every
 * input, for an upstream gradient g of y. Reverse-mode differentiation of
 * the definition above, per direction k in its own step order t
 * (p = token visited at step t, q = the B/C entry of that step):
 *   out[p]  = s[p] * silu(z[p]),  s[p] = sum_k y_k[p]
 *   gs[p]   = g[p] * silu(z[p]);  dz[p] = g[p] * s[p] * silu'(z[p])
 *   lam_t   = gs[p] C_t + e_{t+1} lam_{t+1}        (lam after the last step = 0)
 *   dC_t   += gs[p] h_t;  dB_t += lam_t * delta_t * u[p]
 *   du[p]  += gs[p] D_k + sum_n lam_t delta_t B_t
 *   ddelta_t = sum_n lam_t (h_{t-1} e_t A + B_t u[p])
 *   dA_k   += lam_t h_{t-1} e_t delta_t;  dD_k += gs[p] u[p]
 *   dx_t    = ddelta_t * sigmoid(x_t) (softplus' ; 1 without softplus),
 *             x_t = delta_raw[p] + dt_bias_k
 *   ddelta_raw[p] += dx_t;  ddt_bias_k += dx_t
 * with e_t = exp(delta_t A) and h the forward states (kept per unit).
 * B and C are shared by every channel, so dB and dC sum over channels and
 * directions; A, D and dt_bias sum over batch rows.
 * ------------------------------------------------------------------------ */
typedef struct {
    int batch, dim, dstate;
    long L;
    const double *u, *delta, *z, *B, *C, *A, *Dskip, *dt_bias, *g;
    int delta_softplus;
    double *du, *ddelta, *dz;                 /* [batch][dim][L], written per unit */
    double *dB, *dC;                          /* [batch][dstate][L], this thread's sums */
    double *dA, *dD, *dbias;                  /* [2][dim][dstate], [2][dim], this thread's sums */
    long unit_begin, unit_end;
} grad_job_t;

static double sigmoid(double x)
{
    return x >= 0.0 ? 1.0 / (1.0 + exp(-x)) : exp(x) / (1.0 + exp(x));
}

static int grad_unit(const grad_job_t* J, long unit)
{
    const long b = unit / J->dim, d = unit % J->dim;
    const long L = J->L, N = J->dstate, row = (b * J->dim + d) * L;
    const double *u = J->u + row, *dl = J->delta + row, *g = J->g + row;
    const double *Bb = J->B + b * N * L, *Cb = J->C + b * N * L;
    double *du = J->du + row, *ddl = J->ddelta + row, *dz = J->dz + row;
    double *dBb = J->dB + b * N * L, *dCb = J->dC + b * N * L;
    /* forward states h_t (both directions) and deltas, kept for the reverse pass */
    double* hs = (double*)malloc(sizeof(double) * (size_t)(2 * L * N));
    double* dts = (double*)malloc(sizeof(double) * (size_t)(2 * L));
    double* s = (double*)malloc(sizeof(double) * (size_t)L);
    double* gs = (double*)malloc(sizeof(double) * (size_t)L);
    double* lam = (double*)malloc(sizeof(double) * (size_t)N);
    if (!hs || !dts || !s || !gs || !lam) {
        free(hs); free(dts); free(s); free(gs); free(lam);
        return -2;
    }
    for (long p = 0; p < L; ++p) s[p] = 0.0;
    for (int k = 0; k < 2; ++k) {
        const double* A = J->A + ((long)k * J->dim + d) * N;
        const double Dk = J->Dskip ? J->Dskip[(long)k * J->dim + d] : 0.0;
        const double bias = J->dt_bias ? J->dt_bias[(long)k * J->dim + d] : 0.0;
        double* h = hs + (long)k * L * N;
        for (long t = 0; t < L; ++t) {
            const long p = k == 0 ? t : L - 1 - t;
            const double x = bias + dl[p];
            const double delta = !J->delta_softplus ? x : softplus(x);
            dts[(long)k * L + t] = delta;
            double yk = Dk * u[p];
            for (long n = 0; n < N; ++n) {
                const double prev = t > 0 ? h[(t - 1) * N + n] : 0.0;
                h[t * N + n] = exp(A[n] * delta) * prev + delta * Bb[n * L + p] * u[p];
                yk += Cb[n * L + p] * h[t * N + n];
            }
            s[p] += yk;
        }
    }
    /* gate */
    for (long p = 0; p < L; ++p) {
        if (J->z) {
            const double zz = J->z[row + p], sg = sigmoid(zz);
            gs[p] = g[p] * zz * sg;
            dz[p] = g[p] * s[p] * sg * (1.0 + zz * (1.0 - sg));
        } else {
            gs[p] = g[p];
            dz[p] = 0.0;
        }
        du[p] = 0.0;
        ddl[p] = 0.0;
    }
    /* reverse pass, per direction */
    for (int k = 0; k < 2; ++k) {
        const double* A = J->A + ((long)k * J->dim + d) * N;
        const double Dk = J->Dskip ? J->Dskip[(long)k * J->dim + d] : 0.0;
        const double bias = J->dt_bias ? J->dt_bias[(long)k * J->dim + d] : 0.0;
        const double* h = hs + (long)k * L * N;
        double* dA = J->dA + ((long)k * J->dim + d) * N;
        for (long n = 0; n < N; ++n) lam[n] = 0.0;
        double next_delta = 0.0;                       /* delta_{t+1} */
        for (long t = L - 1; t >= 0; --t) {
            const long p = k == 0 ? t : L - 1 - t;
            const double delta = dts[(long)k * L + t];
            double ddelta = 0.0, dupart = 0.0;
            for (long n = 0; n < N; ++n) {
                const double e_next = t + 1 < L ? exp(next_delta * A[n]) : 0.0;
                lam[n] = gs[p] * Cb[n * L + p] + e_next * lam[n];
                const double hprev = t > 0 ? h[(t - 1) * N + n] : 0.0;
                const double e = exp(A[n] * delta);
                dCb[n * L + p] += gs[p] * h[t * N + n];
                dBb[n * L + p] += lam[n] * delta * u[p];
                dupart += lam[n] * delta * Bb[n * L + p];
                ddelta += lam[n] * (hprev * e * A[n] + Bb[n * L + p] * u[p]);
                dA[n] += lam[n] * hprev * e * delta;
            }
            du[p] += gs[p] * Dk + dupart;
            if (J->dD) J->dD[(long)k * J->dim + d] += gs[p] * u[p];
            const double x = bias + dl[p];
            const double dx = ddelta * (J->delta_softplus ? sigmoid(x) : 1.0);
            ddl[p] += dx;
            if (J->dbias) J->dbias[(long)k * J->dim + d] += dx;
            next_delta = delta;
        }
    }
    free(hs); free(dts); free(s); free(gs); free(lam);
    return 0;
}

static void* grad_worker(void* arg)
{
    const grad_job_t* J = (const grad_job_t*)arg;
    for (long unit = J->unit_begin; unit < J->unit_end; ++unit)
        if (grad_unit(J, unit) != 0) return (void*)1;
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 * Every output is overwritten. Dskip, dt_bias and z may be NULL (zeros / no
 * gate); dD and dbias are then still returned (the gradient at 0). */
int oracle_vim_bidir_grad_f64(int batch, int dim, int dstate, long L, const double* u,
                              const double* delta, const double* z, const double* B,
                              const double* C, const double* A, const double* Dskip,
                              const double* dt_bias, int delta_softplus, const double* g,
                              double* du, double* ddelta, double* dz, double* dB, double* dC,
                              double* dA, double* dD, double* dbias, int nthreads)
{
    if (batch < 1 || dim < 1 || dstate < 1 || L < 1) return -1;
    if (!u || !delta || !B || !C || !A || !g || !du || !ddelta || !dz || !dB || !dC || !dA ||
        !dD || !dbias)
        return -1;
    const long units = (long)batch * dim;
    const size_t nbc = (size_t)batch * dstate * L, na = (size_t)2 * dim * dstate,
                 nd = (size_t)2 * dim;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)units;
    grad_job_t* jobs = (grad_job_t*)calloc((size_t)nthreads, sizeof(grad_job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    /* per-thread sums of the shared gradients */
    double* acc = (double*)calloc((size_t)nthreads * (2 * nbc + na + 2 * nd), sizeof(double));
    if (!jobs || !th || !acc) { free(jobs); free(th); free(acc); return -2; }
    for (int i = 0; i < nthreads; ++i) {
        grad_job_t* J = &jobs[i];
        double* a = acc + (size_t)i * (2 * nbc + na + 2 * nd);
        J->batch = batch; J->dim = dim; J->dstate = dstate; J->L = L;
        J->u = u; J->delta = delta; J->z = z; J->B = B; J->C = C; J->A = A;
        J->Dskip = Dskip; J->dt_bias = dt_bias; J->g = g; J->delta_softplus = delta_softplus;
        J->du = du; J->ddelta = ddelta; J->dz = dz;
        J->dB = a; J->dC = a + nbc; J->dA = a + 2 * nbc; J->dD = a + 2 * nbc + na;
        J->dbias = a + 2 * nbc + na + nd;
        J->unit_begin = units * i / nthreads;
        J->unit_end = units * (i + 1) / nthreads;
    }
    int rc = 0, started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, grad_worker, &jobs[i]) != 0) break;
        started = i;
    }
    if (grad_worker(&jobs[0]) != NULL) rc = -2;
    for (int i = 1; i <= started; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) rc = -2;
    }
    for (int i = started + 1; i < nthreads; ++i)
        if (grad_worker(&jobs[i]) != NULL) rc = -2;
    /* sum the threads' shared gradients */
    for (size_t j = 0; j < nbc; ++j) { dB[j] = 0.0; dC[j] = 0.0; }
    for (size_t j = 0; j < na; ++j) dA[j] = 0.0;
    for (size_t j = 0; j < nd; ++j) { dD[j] = 0.0; dbias[j] = 0.0; }
    for (int i = 0; i < nthreads; ++i) {
        const double* a = acc + (size_t)i * (2 * nbc + na + 2 * nd);
        for (size_t j = 0; j < nbc; ++j) { dB[j] += a[j]; dC[j] += a[nbc + j]; }
        for (size_t j = 0; j < na; ++j) dA[j] += a[2 * nbc + j];
        for (size_t j = 0; j < nd; ++j) {
            dD[j] += a[2 * nbc + na + j];
            dbias[j] += a[2 * nbc + na + nd + j];
        }
    }
    free(jobs); free(th); free(acc);
    return rc;
}

/* ------------------------------------------------------------------------
 * The linear maps around the scan. "1. PyTorch Implementation of the
 * Bidirectional Vision Mamba Block": SimpleSelectiveSSM's x_proj
 * (Linear(d_model, 2 d_state + 1), no bias) gives B, C and the one-wide dt;
 * dt_proj (Linear(1, d_model)) widens dt to one value per channel before the
 * softplus; the block's out_proj (Linear(d_model, d_model)) maps the fused
 * output, and the residual is added. nn.Linear computes out = in W^T + b; in
 * the channel-major layout [batch][features][L] used here that is, per
 * batch row and token t,
 *     out[b][m][t] = sum_k W[m][k] in[b][k][t] + bias[m] (+ residual[b][m][t]).
 * W is [M][K] as nn.Linear stores it. bias and residual may be NULL. */
int oracle_linear_f64(int batch, int M, int K, long L, const double* W, const double* in,
                      const double* bias, const double* residual, double* out)
{
    if (batch < 0 || M < 0 || K < 0 || L < 0) return -1;
    if (!W || !in || !out) return -1;
    for (long b = 0; b < batch; ++b)
        for (long m = 0; m < M; ++m)
            for (long t = 0; t < L; ++t) {
                double s = 0.0;
                for (long k = 0; k < K; ++k) s += W[m * K + k] * in[(b * K + k) * L + t];
                if (bias) s += bias[m];
                if (residual) s += residual[(b * M + m) * L + t];
                out[(b * M + m) * L + t] = s;
            }
    return 0;
}

/* dt_proj with the bias left to the scan (its dt_bias, added before the
 * softplus): delta_raw[b][d][t] = w[d] dt[b][t], the one-input Linear. */
int oracle_dt_proj_f64(int batch, int dim, long L, const double* dt, const double* w,
                       double* delta)
{
    if (batch < 0 || dim < 0 || L < 0 || !dt || !w || !delta) return -1;
    for (long b = 0; b < batch; ++b)
        for (long d = 0; d < dim; ++d)
            for (long t = 0; t < L; ++t)
                delta[(b * dim + d) * L + t] = w[d] * dt[b * L + t];
    return 0;
}

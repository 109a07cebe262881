/*
 * CPU oracle, plain C.  TEST INFRASTRUCTURE ONLY: loaded by tests/, by
 * __graft_entry__.smoke() and by the cpu_baseline leg of bench.py, never by
 * the product path.  It shares no code or header with the HIP library.
 *
 * Build (done by __graft_entry__.build() and oracle/build.py):
 *   gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC \
 *       -o oracle/libssmoracle.so oracle/ref_cpu.c -lm
 * -ffp-contract=off keeps every a*b+c as two rounded operations unless
 * fmaf() is written explicitly, which the fp32 replay below relies on.
 *
 * Pages cited:
 *   [Scan page]    "Hardware-aware parallel associative scan for Mamba"
 *                  (http://www.pwwt.cn/news/6375169/)
 *   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
 *                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x) in the overflow-safe form max(x,0) + log1p(e^-|x|)
 * ([Scan page] §1.2: delta is made positive with softplus). */
static double softplus_d(double x) {
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* silu(z) = z / (1 + e^-z) ([Mamba-2 page] §4.1 names the SiLU gate). */
static double silu_d(double z) {
    return z / (1.0 + exp(-z));
}

/*
 * Selective-scan forward, float64 arithmetic on float32 inputs, for a set of
 * (batch, channel) rows.  Row r uses batch row_b[r] and channel row_d[r];
 * u_rows/delta_rows/z_rows hold that row's L inputs contiguously.  For every
 * step t ([Scan page] §1.1-§1.2):
 *     x = delta + bias;  dt = softplus(x) or x
 *     h[n] = exp(dt*A[d,n]) * h[n] + dt * B[b,n,t] * u       (h_0 = 0)
 *     y = sum_n C[b,n,t]*h[n] + D[d]*u;  y *= silu(z) if gated
 * Outputs y[r, t] (float64) and last_state[r, n] = h_L (float64); either may
 * be NULL.  Rows are independent; OpenMP splits them statically over
 * nthreads threads (nthreads <= 0: runtime default).  Returns 0, or 1 on a
 * bad argument.
 */
int ssm_oracle_fwd_rows_h0(const float *u_rows, const float *delta_rows, const float *z_rows,
                           const int64_t *row_b, const int64_t *row_d, int64_t nrows,
                           const float *A, const float *B, const float *C, const float *D,
                           const float *delta_bias, int delta_softplus,
                           int64_t batch, int64_t dim, int64_t dstate, int64_t L,
                           const double *h0_rows, int64_t chunk, double *bounds,
                           double *y, double *last_state, int nthreads);

int ssm_oracle_fwd_rows(const float *u_rows, const float *delta_rows, const float *z_rows,
                        const int64_t *row_b, const int64_t *row_d, int64_t nrows,
                        const float *A, const float *B, const float *C, const float *D,
                        const float *delta_bias, int delta_softplus,
                        int64_t batch, int64_t dim, int64_t dstate, int64_t L,
                        double *y, double *last_state, int nthreads) {
    return ssm_oracle_fwd_rows_h0(u_rows, delta_rows, z_rows, row_b, row_d, nrows, A, B, C, D, delta_bias,
                                  delta_softplus, batch, dim, dstate, L, NULL, 0, NULL, y, last_state, nthreads);
}

/*
 * The same recurrence started from a given state and keeping the state at
 * every chunk boundary ([Scan page] §2.1: h_t = A_t h_0 + B_t for any start
 * state; [Mamba-2 page] §4.3: the chunked recomputation keeps h at every
 * chunk boundary).  h0_rows: [nrows, dstate] or NULL (zero).  With chunk > 0
 * and bounds non-NULL, bounds[r, k, n] (k = 0 .. ceil(L/chunk) - 1) is the
 * state after step min((k+1)*chunk, L) - 1.
 */
int ssm_oracle_fwd_rows_h0(const float *u_rows, const float *delta_rows, const float *z_rows,
                           const int64_t *row_b, const int64_t *row_d, int64_t nrows,
                           const float *A, const float *B, const float *C, const float *D,
                           const float *delta_bias, int delta_softplus,
                           int64_t batch, int64_t dim, int64_t dstate, int64_t L,
                           const double *h0_rows, int64_t chunk, double *bounds,
                           double *y, double *last_state, int nthreads) {
    if (!u_rows || !delta_rows || !row_b || !row_d || !A || !B || !C) return 1;
    if (nrows < 0 || batch <= 0 || dim <= 0 || dstate <= 0 || L < 0 || chunk < 0) return 1;
    if (bounds && chunk == 0) return 1;
    const int64_t K = chunk > 0 ? (L + chunk - 1) / chunk : 0;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_b[r] < 0 || row_b[r] >= batch || row_d[r] < 0 || row_d[r] >= dim) return 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = row_b[r], d = row_d[r];
        double *h = (double *)calloc((size_t)dstate, sizeof(double));
        if (!h) { bad = 1; continue; }
        if (h0_rows)
            for (int64_t n = 0; n < dstate; ++n) h[n] = h0_rows[r * dstate + n];
        const float *ur = u_rows + r * L;
        const float *dr = delta_rows + r * L;
        const float *zr = z_rows ? z_rows + r * L : NULL;
        const double bias = delta_bias ? (double)delta_bias[d] : 0.0;
        const double Dd = D ? (double)D[d] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double uu = (double)ur[t];
            const double x = (double)dr[t] + bias;
            const double dt = delta_softplus ? softplus_d(x) : x;
            double acc = 0.0;
            for (int64_t n = 0; n < dstate; ++n) {
                const double a = exp(dt * (double)A[d * dstate + n]);
                const double bb = dt * (double)B[(b * dstate + n) * L + t] * uu;
                h[n] = a * h[n] + bb;
                acc += (double)C[(b * dstate + n) * L + t] * h[n];
            }
            acc += Dd * uu;
            if (zr) acc *= silu_d((double)zr[t]);
            if (y) y[r * L + t] = acc;
            if (bounds && ((t + 1) % chunk == 0 || t + 1 == L))
                for (int64_t n = 0; n < dstate; ++n) bounds[(r * K + t / chunk) * dstate + n] = h[n];
        }
        if (last_state)
            for (int64_t n = 0; n < dstate; ++n) last_state[r * dstate + n] = h[n];
        free(h);
    }
    return bad ? 1 : 0;
}

/*
 * Gradients of the selective scan (reverse-mode chain rule of the forward
 * above), float64, for the whole [batch, dim, L] problem.  The loss is
 * sum(dy * y) + sum(dlast * last_state); dlast and h0 may be NULL (zero).
 * Per (batch, channel) chain the forward is run keeping every state, then
 * the steps are walked back ([Scan page] §4.2 and [Mamba-2 page] §4.3
 * recompute the same states chunk by chunk; here all are kept):
 *     gs = dy*silu(z) (dy without gate);  dz = dy*s*silu'(z), s = C.h + D u
 *     g_t = C_t gs_t + a_{t+1} g_{t+1}  (g after the last step = dlast)
 *     dC[b,n,t] += gs_t h_t[n];  dB[b,n,t] += g_t[n] dt_t u_t
 *     du_t = D gs_t + dt_t sum_n g_t[n] B[b,n,t]
 *     ddt_t = sum_n g_t[n] (A[d,n] a_t[n] h_{t-1}[n] + B[b,n,t] u_t)
 *     dA[d,n] += g_t[n] a_t[n] h_{t-1}[n] dt_t;  dD[d] += gs_t u_t
 *     ddelta_t = ddt_t * sigmoid(x_t) with softplus, else ddt_t
 *     ddelta_bias[d] += ddelta_t;  dh0 = a_0 g_0
 * Outputs (all float64, all required except dz, which is required iff z is
 * given): du, ddelta, dz [b,d,L]; dA [d,n]; dB, dC [b,n,L]; dD, dbias [d];
 * dh0 [b,d,n].  Channels run in parallel (OpenMP, static); the sums over
 * channels (dB, dC) go through per-thread buffers added in thread order.
 * Returns 0, or 1 on a bad argument or allocation failure.
 */
int ssm_oracle_bwd(const float *u, const float *delta, const float *A, const float *B, const float *C,
                   const float *D, const float *z, const float *delta_bias, int delta_softplus,
                   const float *h0, const float *dy, const float *dlast,
                   int64_t batch, int64_t dim, int64_t dstate, int64_t L,
                   double *du, double *ddelta, double *dz, double *dA, double *dB, double *dC,
                   double *dD, double *dbias, double *dh0, int nthreads) {
    if (!u || !delta || !A || !B || !C || !dy) return 1;
    if (!du || !ddelta || !dA || !dB || !dC || !dD || !dbias || !dh0) return 1;
    if ((z != NULL) != (dz != NULL)) return 1;
    if (batch <= 0 || dim <= 0 || dstate <= 0 || L <= 0) return 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    const int maxth = omp_get_max_threads();
#else
    (void)nthreads;
    const int maxth = 1;
#endif
    const size_t bcn = (size_t)(batch * dstate * L);
    double *partB = (double *)calloc((size_t)maxth * bcn, sizeof(double));
    double *partC = (double *)calloc((size_t)maxth * bcn, sizeof(double));
    if (!partB || !partC) { free(partB); free(partC); return 1; }
    int bad = 0, nth_used = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#pragma omp single
        nth_used = omp_get_num_threads();
#else
        const int tid = 0;
#endif
        double *pB = partB + (size_t)tid * bcn;
        double *pC = partC + (size_t)tid * bcn;
        double *hs = (double *)malloc((size_t)(L + 1) * (size_t)dstate * sizeof(double));
        double *aa = (double *)malloc((size_t)L * (size_t)dstate * sizeof(double));
        double *dts = (double *)malloc((size_t)L * sizeof(double));
        double *gss = (double *)malloc((size_t)L * sizeof(double));
        double *g = (double *)malloc((size_t)dstate * sizeof(double));
        if (!hs || !aa || !dts || !gss || !g) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t d = 0; d < dim; ++d) {
            if (!hs || !aa || !dts || !gss || !g) continue;
            const double bias = delta_bias ? (double)delta_bias[d] : 0.0;
            const double Dd = D ? (double)D[d] : 0.0;
            double sumD = 0.0, sumBias = 0.0;
            for (int64_t n = 0; n < dstate; ++n) dA[d * dstate + n] = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                const int64_t row = (b * dim + d) * L;
                /* forward, keeping h_t for every t (hs[t+1]) and a_t */
                for (int64_t n = 0; n < dstate; ++n)
                    hs[n] = h0 ? (double)h0[(b * dim + d) * dstate + n] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const double uu = (double)u[row + t];
                    const double x = (double)delta[row + t] + bias;
                    const double dt = delta_softplus ? softplus_d(x) : x;
                    dts[t] = dt;
                    double s = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const double a = exp(dt * (double)A[d * dstate + n]);
                        aa[t * dstate + n] = a;
                        const double hn = a * hs[t * dstate + n] + dt * (double)B[(b * dstate + n) * L + t] * uu;
                        hs[(t + 1) * dstate + n] = hn;
                        s += (double)C[(b * dstate + n) * L + t] * hn;
                    }
                    s += Dd * uu;
                    const double gy = (double)dy[row + t];
                    if (z) {
                        const double zz = (double)z[row + t];
                        const double sg = 1.0 / (1.0 + exp(-zz));
                        gss[t] = gy * zz * sg;
                        dz[row + t] = gy * s * sg * (1.0 + zz * (1.0 - sg));
                    } else {
                        gss[t] = gy;
                    }
                }
                /* reverse */
                for (int64_t n = 0; n < dstate; ++n)
                    g[n] = dlast ? (double)dlast[(b * dim + d) * dstate + n] : 0.0;
                for (int64_t t = L - 1; t >= 0; --t) {
                    const double uu = (double)u[row + t];
                    const double dt = dts[t];
                    const double gs = gss[t];
                    double r = 0.0, w = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const double a_next = (t + 1 < L) ? aa[(t + 1) * dstate + n] : 1.0;
                        const double Bv = (double)B[(b * dstate + n) * L + t];
                        const double Cv = (double)C[(b * dstate + n) * L + t];
                        g[n] = Cv * gs + a_next * g[n];
                        pC[(b * dstate + n) * L + t] += gs * hs[(t + 1) * dstate + n];
                        pB[(b * dstate + n) * L + t] += g[n] * dt * uu;
                        r += g[n] * Bv;
                        const double ga = g[n] * aa[t * dstate + n] * hs[t * dstate + n];
                        w += ga * (double)A[d * dstate + n];
                        dA[d * dstate + n] += ga * dt;
                    }
                    du[row + t] = Dd * gs + dt * r;
                    const double ddt = w + uu * r;
                    double dd = ddt;
                    if (delta_softplus) {
                        const double x = (double)delta[row + t] + bias;
                        dd = ddt / (1.0 + exp(-x));
                    }
                    ddelta[row + t] = dd;
                    sumBias += dd;
                    sumD += gs * uu;
                }
                for (int64_t n = 0; n < dstate; ++n)
                    dh0[(b * dim + d) * dstate + n] = aa[n] * g[n];
            }
            dD[d] = sumD;
            dbias[d] = sumBias;
        }
        free(hs); free(aa); free(dts); free(gss); free(g);
    }
    if (!bad) {
        for (size_t i = 0; i < bcn; ++i) {
            double sb = 0.0, sc = 0.0;
            for (int th = 0; th < nth_used; ++th) {
                sb += partB[(size_t)th * bcn + i];
                sc += partC[(size_t)th * bcn + i];
            }
            dB[i] = sb;
            dC[i] = sc;
        }
    }
    free(partB); free(partC);
    return bad ? 1 : 0;
}

/*
 * Serial float32 left fold with an explicit fused multiply-add:
 *     A_t = a_t * A_{t-1},  H_t = fmaf(a_t, H_{t-1}, b_t),  (A, H) from (1, 0).
 * This is the plain serial order of the recurrence in [Scan page] §2.1.
 */
void affine_scan_serial_f32(const float *a, const float *b, float *out_a, float *out_b,
                            int64_t rows, int64_t L) {
    for (int64_t r = 0; r < rows; ++r) {
        float P = 1.0f, H = 0.0f;
        for (int64_t t = 0; t < L; ++t) {
            const float at = a[r * L + t], bt = b[r * L + t];
            P = at * P;
            H = fmaf(at, H, bt);
            if (out_a) out_a[r * L + t] = P;
            out_b[r * L + t] = H;
        }
    }
}

/* (a2, b2) o (a1, b1) = (a2*a1, a2*b1 + b2) with the second part fused
 * ([Mamba-2 page] §2.2 composition, evaluated in float32). */
typedef struct { float p, h; } pair_f32;
static pair_f32 comp(pair_f32 later, pair_f32 earlier) {
    pair_f32 r;
    r.p = later.p * earlier.p;
    r.h = fmaf(later.p, earlier.h, later.h);
    return r;
}

/*
 * float32 replay of a blocked scan order: T items per lane, `lanes` lanes per
 * wave (64 on the GPU), W waves per block; chunk = lanes*W*T items.
 * The order, stated without reference to any implementation:
 *   For each row, chunks are taken in order with a carry that starts at the
 *   identity (1, 0).  Item j of lane l of wave w in chunk k is at index
 *   k*chunk + (w*lanes + l)*T + j; indices >= L are identities.
 *   1. Each lane folds its T items left to right starting from its first
 *      item (no identity in front): (P, H) <- (a_j, b_j) o (P, H).
 *   2. Inclusive lane scan of those lane totals inside each wave, in rounds.
 *      Rounds d = 1, 2, 4, 8: lane l takes lane l-d when (l mod 16) >= d and
 *      the identity otherwise.  Round 16: lanes whose index has bit 4 set take
 *      the last lane of the previous group of 16 (lane 16*floor(l/16) - 1),
 *      others the identity.  Round 32: lanes >= 32 take lane 31, others the
 *      identity.  In every round all lanes read the values of the previous
 *      round and compute own o taken (the identity is composed too).
 *      With fewer than 64 lanes the same rules run on the lanes present, and
 *      a lane whose partner index does not exist takes the identity.
 *   3. The exclusive prefix of lane l is the inclusive value of lane l-1.
 *   4. acc = carry; for v = 0..w-1: acc = total(v) o acc, where total(v) is the
 *      inclusive value of the last lane of wave v.  The lane's start state is
 *      excl o acc for l >= 1 and acc for l = 0.  After the chunk the carry
 *      becomes total(W-1) o ... o total(0) o carry, folded in that order.
 *   5. Each lane re-folds its items from its start state:
 *      (A, H) <- (a_j, b_j) o (A, H), writing A and H for indices < L.
 * lanes must be a power of two <= 64.  Returns 0, or 1 on bad parameters.
 */
int affine_scan_replay_f32(const float *a, const float *b, float *out_a, float *out_b,
                           int64_t rows, int64_t L, int T, int lanes, int W) {
    if (T <= 0 || W <= 0 || lanes <= 0 || lanes > 64 || (lanes & (lanes - 1))) return 1;
    const int64_t per_chunk = (int64_t)lanes * W * T;
    const int nl = lanes * W;
    pair_f32 *tot = (pair_f32 *)malloc(sizeof(pair_f32) * (size_t)nl);
    pair_f32 *nxt = (pair_f32 *)malloc(sizeof(pair_f32) * (size_t)nl);
    if (!tot || !nxt) { free(tot); free(nxt); return 1; }
    const pair_f32 ident = {1.0f, 0.0f};
    for (int64_t r = 0; r < rows; ++r) {
        const float *ar = a + r * L, *br = b + r * L;
        pair_f32 carry = ident;
        for (int64_t base = 0; base < L; base += per_chunk) {
            /* 1. lane-local folds */
            for (int g = 0; g < nl; ++g) {
                pair_f32 acc = ident;
                for (int j = 0; j < T; ++j) {
                    const int64_t i = base + (int64_t)g * T + j;
                    pair_f32 it = ident;
                    if (i < L) { it.p = ar[i]; it.h = br[i]; }
                    acc = (j == 0) ? it : comp(it, acc);
                }
                tot[g] = acc;
            }
            /* 2. rounds inside each wave */
            for (int w = 0; w < W; ++w) {
                pair_f32 *v = tot + (size_t)w * lanes;
                pair_f32 *o = nxt + (size_t)w * lanes;
                static const int rounds[6] = {1, 2, 4, 8, 16, 32};
                for (int q = 0; q < 6; ++q) {
                    const int d = rounds[q];
                    for (int l = 0; l < lanes; ++l) {
                        int src = -1;
                        if (d <= 8) {
                            if ((l % 16) >= d) src = l - d;
                        } else if (d == 16) {
                            if (l & 16) src = 16 * (l / 16) - 1;
                        } else {
                            if (l >= 32) src = 31;
                        }
                        pair_f32 taken = ident;
                        if (src >= 0 && src < lanes) taken = v[src];
                        o[l] = comp(v[l], taken);
                    }
                    for (int l = 0; l < lanes; ++l) v[l] = o[l];
                }
            }
            /* 3.-5. start states and the re-fold */
            pair_f32 acc = carry;
            for (int w = 0; w < W; ++w) {
                pair_f32 *v = tot + (size_t)w * lanes;
                for (int l = 0; l < lanes; ++l) {
                    pair_f32 st = (l == 0) ? acc : comp(v[l - 1], acc);
                    for (int j = 0; j < T; ++j) {
                        const int64_t i = base + ((int64_t)w * lanes + l) * T + j;
                        pair_f32 it = ident;
                        if (i < L) { it.p = ar[i]; it.h = br[i]; }
                        st = comp(it, st);
                        if (i < L) {
                            if (out_a) out_a[r * L + i] = st.p;
                            out_b[r * L + i] = st.h;
                        }
                    }
                }
                acc = comp(v[lanes - 1], acc);
            }
            carry = acc;
        }
    }
    free(tot);
    free(nxt);
    return 0;
}

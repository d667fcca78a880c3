/*
 * ssd_oracle.c -- plain, slow, fp64 CPU reference for the Mamba-2 SSD
 * chunked forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, calls or
 * executes this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * constant with the HIP implementation.
 *
 * Sources (cited by page title and section):
 *   [P1] "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in
 *        NVIDIA CUDA Tile" (trishampatil.com)
 *   [P2] the Chinese rendering of the same NVIDIA / Jane Street write-up
 *        (zhiding.cn), section "Mamba-2架构", where the display formulas
 *        survive.
 *
 * What is computed.  Per batch b and head h (group g = h / (H/G)):
 *
 *   S_t = exp(A_h * dt_t) * S_{t-1} + dt_t * x_t B_t^T        (P x N)
 *   y_t = S_t C_t + D_h * x_t
 *
 * [P1 "The Mamba-2 Recurrence"; P2 "Mamba-2架构", the recurrence pair].
 * The state is the outer product x B^T, so S has shape (P, N): one row per
 * element of x_t, one column per element of B_t.  y_t reads the state after
 * token t's update: [P2] writes it so in the recurrence pair, its expansion
 * of y_{t+i} includes the b_{t+i} x_{t+i}^T term, and the causal mask of
 * both kernels keeps the diagonal ([P1 "Kernel 3: compute_out"]).  A second
 * line of [P2] that reads h_{t-1} contradicts all three and is taken as a
 * typo.
 *
 * Chunking only decides where states are sampled: states[b,h,c] is the state
 * before the first token of chunk c, so states[b,h,0] is the initial state
 * [P1 "Kernel 2: fwd_pass_state": the state is stored at the top of every
 * chunk iteration, before the update]; final is the state after the last
 * token.  A ragged last chunk (seqlen % chunk != 0) needs no special case in
 * the recurrence.
 *
 * The stage-1 quantity is the per-chunk inclusive cumulative sum of
 * a_t = A_h dt_t, pre-scaled by log2(e) so later stages can use exp2
 * [P1 "Kernel 1: chunk_cumsum"].
 *
 * Inputs are float32 arrays holding the exact values the GPU receives (bf16
 * values are exactly representable in float32), except the initial state,
 * which is double so a state carried out of one call can be fed back
 * unrounded; all arithmetic is double.
 * Outputs are written per (batch, head) pair in a compact layout: pair k of
 * the `pairs` list (index b*H + h), or pair k = b*H + h when pairs == NULL.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* log2(e) as printed in [P1 "Kernel 1: chunk_cumsum"]. */
static const double kLog2e = 1.4426950408889634;

/* g[k][t] for pair k: log2(e) * sum_{s = T*floor(t/T)}^{t} A_h * dt[b,s,h].
 * g has shape [npairs, seqlen]. */
void oracle_chunk_cumsum(const float *dt, const float *A, double *g,
                         int64_t batch, int64_t seqlen, int64_t nheads,
                         int64_t chunk, const int64_t *pairs, int64_t npairs)
{
    if (pairs == NULL) npairs = batch * nheads;
    for (int64_t k = 0; k < npairs; ++k) {
        int64_t bh = pairs ? pairs[k] : k;
        int64_t b = bh / nheads, h = bh % nheads;
        double run = 0.0;
        for (int64_t t = 0; t < seqlen; ++t) {
            if (t % chunk == 0) run = 0.0;   /* the sum restarts per chunk */
            run += (double)A[h] * (double)dt[(b * seqlen + t) * nheads + h];
            g[k * seqlen + t] = kLog2e * run;
        }
    }
}

/* One token of the recurrence on state S (P x N, row-major), emitting y_t
 * into yt (length P) when yt != NULL. */
static void recurrence_step(double *S, const float *xt, double dtt, double ah,
                            const float *Bt, const float *Ct, double Dh,
                            double *yt, int64_t P, int64_t N)
{
    const double decay = exp(ah * dtt);
    for (int64_t p = 0; p < P; ++p) {
        const double u = dtt * (double)xt[p];
        double *row = S + p * N;
        for (int64_t n = 0; n < N; ++n)
            row[n] = decay * row[n] + u * (double)Bt[n];
    }
    if (yt) {
        for (int64_t p = 0; p < P; ++p) {
            const double *row = S + p * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += row[n] * (double)Ct[n];
            yt[p] = acc + Dh * (double)xt[p];
        }
    }
}

/*
 * Full forward by the literal recurrence.
 *   x [b,L,H,P], dt [b,L,H], A [H], B,C [b,L,G,N], D [H] (float),
 *   init [b,H,P,N] (double; may be NULL: zero state).
 * Outputs (any may be NULL), per pair k:
 *   y      [npairs, L, P]
 *   states [npairs, nc, P, N]   (state before chunk c)
 *   final  [npairs, P, N]
 */
void oracle_forward(const float *x, const float *dt, const float *A,
                    const float *B, const float *C, const float *D,
                    const double *init, double *y, double *states,
                    double *final_state, int64_t batch, int64_t seqlen,
                    int64_t nheads, int64_t headdim, int64_t dstate,
                    int64_t ngroups, int64_t chunk, const int64_t *pairs,
                    int64_t npairs, int nthreads)
{
    const int64_t L = seqlen, H = nheads, P = headdim, N = dstate;
    const int64_t G = ngroups, hpg = H / G, nc = (L + chunk - 1) / chunk;
    if (pairs == NULL) npairs = batch * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t k = 0; k < npairs; ++k) {
        const int64_t bh = pairs ? pairs[k] : k;
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        double *S = (double *)malloc(sizeof(double) * P * N);
        if (init) {
            memcpy(S, init + (b * H + h) * P * N, sizeof(double) * P * N);
        } else {
            memset(S, 0, sizeof(double) * P * N);
        }
        for (int64_t t = 0; t < L; ++t) {
            if (states && t % chunk == 0)
                memcpy(states + (k * nc + t / chunk) * P * N, S,
                       sizeof(double) * P * N);
            const int64_t tok = b * L + t;
            recurrence_step(S, x + (tok * H + h) * P, (double)dt[tok * H + h],
                            (double)A[h], B + (tok * G + g) * N,
                            C + (tok * G + g) * N, (double)D[h],
                            y ? y + (k * L + t) * P : NULL, P, N);
        }
        if (final_state) memcpy(final_state + k * P * N, S,
                                sizeof(double) * P * N);
        free(S);
    }
}

/*
 * Chunk outputs from given per-chunk starting states: for every chunk c the
 * recurrence restarts from states_in[k][c] and runs through the chunk's
 * tokens, emitting y.  This is what the output stage computes from the state
 * pass's results [P1 "Step 2: Compute a Chunk of Outputs from One State";
 * P1 "Kernel 3: compute_out"].  With states_in equal to oracle_forward's
 * states it reproduces oracle_forward's y.
 *   states_in [npairs, nc, P, N] (double), y [npairs, L, P].
 */
void oracle_chunk_out(const float *x, const float *dt, const float *A,
                      const float *B, const float *C, const float *D,
                      const double *states_in, double *y, int64_t batch,
                      int64_t seqlen, int64_t nheads, int64_t headdim,
                      int64_t dstate, int64_t ngroups, int64_t chunk,
                      const int64_t *pairs, int64_t npairs, int nthreads)
{
    const int64_t L = seqlen, H = nheads, P = headdim, N = dstate;
    const int64_t G = ngroups, hpg = H / G, nc = (L + chunk - 1) / chunk;
    if (pairs == NULL) npairs = batch * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t k = 0; k < npairs; ++k) {
        const int64_t bh = pairs ? pairs[k] : k;
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        double *S = (double *)malloc(sizeof(double) * P * N);
        for (int64_t c = 0; c < nc; ++c) {
            memcpy(S, states_in + (k * nc + c) * P * N,
                   sizeof(double) * P * N);
            const int64_t t1 = (c + 1) * chunk < L ? (c + 1) * chunk : L;
            for (int64_t t = c * chunk; t < t1; ++t) {
                const int64_t tok = b * L + t;
                recurrence_step(S, x + (tok * H + h) * P,
                                (double)dt[tok * H + h], (double)A[h],
                                B + (tok * G + g) * N, C + (tok * G + g) * N,
                                (double)D[h], y + (k * L + t) * P, P, N);
            }
        }
        free(S);
    }
}

/*
 * Causal depthwise 1-D convolution, the Mamba-2 block step upstream of the
 * SSD (page 3, the Helion hackathon gallery, its causal_conv1d entries: each
 * channel is convolved on its own with a short filter of W taps, the input
 * padded with zeros on the left):
 *   out[b,d,t] = bias[d] + sum_{k=0}^{W-1} weight[d,k] * x[b,d,t-W+1+k],
 * where x at a negative time index is zero.  No activation is applied (the
 * page's formula has none).
 *   x, out [batch, dim, seqlen]; weight [dim, width]; bias [dim] or NULL.
 */
void oracle_causal_conv1d(const float *x, const float *weight, const float *bias,
                          double *out, int64_t batch, int64_t dim,
                          int64_t seqlen, int64_t width)
{
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const float *row = x + (b * dim + d) * seqlen;
            double *o = out + (b * dim + d) * seqlen;
            for (int64_t t = 0; t < seqlen; ++t) {
                double acc = bias ? (double)bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k) {
                    const int64_t s = t - width + 1 + k;
                    if (s >= 0) acc += (double)weight[d * width + k] * (double)row[s];
                }
                o[t] = acc;
            }
        }
    }
}

/*
 * Gated DeltaNet, chunked forward: the inter-chunk state pass (chunk_fwd_h)
 * and the output (chunk_fwd_o), taken in the order the Helion hackathon
 * gallery states them (page 3, its gated_deltanet_chunk_fwd_h and
 * gated_deltanet_chunk_fwd_o entries).  The state h is K x V per (b, h) and
 * chunks have C tokens; per chunk c with tokens t in [t0, t1):
 *   h_out[b,h,c] = h                                       (1) store h
 *   v_new[t] = u[t] - w[t] h           (row vectors, 1xV)  (2)
 *   h = exp(g_last) h + sum_t k[t]^T (exp(g_last - g[t]) v_new[t])   (3)-(5)
 * with g_last = g at the chunk's last token (the last valid token of a
 * ragged chunk).  g is the chunk-local cumulative sum of the log-gates
 * (natural log, so exp), as the gate exp(g_last - g_t) implies; w and u are
 * the WY-transformed keys and values (inputs here).  Output, per chunk:
 *   o[t] = scale * ( exp(g[t]) q[t] h_out[b,h,c]
 *                    + sum_{j in chunk, j <= t} (q[t] . k[j]) exp(g[t] - g[j]) v_new[j] )
 * (the gallery's inter + intra terms; scale = 1 is its formula as written).
 * Layouts: q, k, w [b, L, H, K]; u, v_new, o [b, L, H, V]; g [b, L, H];
 * h0 and final [b, H, K, V]; h_out [b, H, NT, K, V], NT = ceil(L / C).
 * h0 and final may be NULL (zero initial state / not wanted).
 */
void oracle_gdn_chunk_fwd_h(const float *k, const float *w, const float *u,
                            const float *g, const double *h0, double *h_out,
                            double *v_new, double *final_state, int64_t batch,
                            int64_t seqlen, int64_t nheads, int64_t dk,
                            int64_t dv, int64_t chunk, int nthreads)
{
    const int64_t nt = (seqlen + chunk - 1) / chunk;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int64_t bh = 0; bh < batch * nheads; ++bh) {
        const int64_t b = bh / nheads, hd = bh % nheads;
        double *h = (double *)malloc((size_t)(dk * dv) * sizeof(double));
        double *vn = (double *)malloc((size_t)(chunk * dv) * sizeof(double));
        for (int64_t i = 0; i < dk * dv; ++i) h[i] = h0 ? h0[bh * dk * dv + i] : 0.0;
        for (int64_t c = 0; c < nt; ++c) {
            const int64_t t0 = c * chunk;
            const int64_t t1 = t0 + chunk < seqlen ? t0 + chunk : seqlen;
            memcpy(h_out + (bh * nt + c) * dk * dv, h, (size_t)(dk * dv) * sizeof(double));
            for (int64_t t = t0; t < t1; ++t) {
                const int64_t row = (b * seqlen + t) * nheads + hd;
                for (int64_t j = 0; j < dv; ++j) {
                    double acc = (double)u[row * dv + j];
                    for (int64_t i = 0; i < dk; ++i)
                        acc -= (double)w[row * dk + i] * h[i * dv + j];
                    vn[(t - t0) * dv + j] = acc;
                    v_new[row * dv + j] = acc;
                }
            }
            const double gl = (double)g[(b * seqlen + t1 - 1) * nheads + hd];
            const double decay = exp(gl);
            for (int64_t i = 0; i < dk * dv; ++i) h[i] *= decay;
            for (int64_t t = t0; t < t1; ++t) {
                const int64_t row = (b * seqlen + t) * nheads + hd;
                const double gate = exp(gl - (double)g[row]);
                for (int64_t i = 0; i < dk; ++i) {
                    const double ki = (double)k[row * dk + i] * gate;
                    for (int64_t j = 0; j < dv; ++j) h[i * dv + j] += ki * vn[(t - t0) * dv + j];
                }
            }
        }
        if (final_state)
            memcpy(final_state + bh * dk * dv, h, (size_t)(dk * dv) * sizeof(double));
        free(h);
        free(vn);
    }
}

void oracle_gdn_chunk_fwd_o(const float *q, const float *k, const double *v_new,
                            const double *h_out, const float *g, double *o,
                            double scale, int64_t batch, int64_t seqlen,
                            int64_t nheads, int64_t dk, int64_t dv,
                            int64_t chunk, int nthreads)
{
    const int64_t nt = (seqlen + chunk - 1) / chunk;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int64_t bh = 0; bh < batch * nheads; ++bh) {
        const int64_t b = bh / nheads, hd = bh % nheads;
        for (int64_t t = 0; t < seqlen; ++t) {
            const int64_t c = t / chunk, t0 = c * chunk;
            const int64_t row = (b * seqlen + t) * nheads + hd;
            const double *hc = h_out + (bh * nt + c) * dk * dv;
            const double gt = (double)g[row];
            for (int64_t j = 0; j < dv; ++j) {
                double inter = 0.0;
                for (int64_t i = 0; i < dk; ++i) inter += (double)q[row * dk + i] * hc[i * dv + j];
                double intra = 0.0;
                for (int64_t s = t0; s <= t; ++s) {
                    const int64_t rs = (b * seqlen + s) * nheads + hd;
                    double qk = 0.0;
                    for (int64_t i = 0; i < dk; ++i)
                        qk += (double)q[row * dk + i] * (double)k[rs * dk + i];
                    intra += qk * exp(gt - (double)g[rs]) * v_new[rs * dv + j];
                }
                o[row * dv + j] = scale * (exp(gt) * inter + intra);
            }
        }
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

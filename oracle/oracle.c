/*
 * oracle.c -- plain, sequential, double-precision CPU oracle of the RG-LRU
 * hot path (causal depthwise Conv1D of width 4 followed by the RG-LRU).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
 * baseline may load this library.  It shares no code, header, table or helper
 * with the GPU library; the only thing both sides share is the seeded input
 * generator, which holds none of the method's arithmetic.
 *
 * Every input is the exact stored value the GPU receives (fp32, or bf16
 * widened), passed here as double; all arithmetic is IEEE double.  Each
 * output is computed straight from its definition: no blocking, fusion or
 * reordering beyond what the definition states.  OpenMP only spreads
 * independent outputs over threads; every output is computed by one thread
 * in the order written.
 *
 * Sources (page titles as published; sections / equations on them):
 *  [G]  "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention"
 *       - "Formulation of the RG-LRU Gating Mechanism": recurrence gate,
 *         input gate, dynamic diagonal decay, state update and output
 *         equations, and the log-space form of the decay.
 *       - "Temporal Filtering via Separable 1D Convolutions": depthwise
 *         conv of width 4 on branch 1.
 *       - "Block-Diagonal Sharding for Zero-Communication Tensor
 *         Parallelism": W_a and W_x are block-diagonal.
 *       - the PyTorch listing under "End-to-End Implementation" (module
 *         RGLRU: forward with prev_state / last_state, step; module
 *         RecurrentBlock: Conv1d with padding k-1, groups = width, keep the
 *         first T outputs).
 *  [W]  "Griffin" (wiki note), section "Gated Linear Recurrence".
 *  [L]  "Griffin" (wiki note), section "Residual Block View": the pre-norm
 *       residual layer x~ = x + TemporalMix(RMSNorm(x)), y = x~ + MLP(RMSNorm(x~));
 *       module page "transformer_lens.model_bridge.supported_architectures.
 *       recurrent_gemma", "Architecture overview": temporal_pre_norm,
 *       channel_pre_norm, gated MLP gate_proj / up_proj / down_proj with
 *       GELU-tanh, RMSNorm applying (1 + weight).
 *  [N]  "Griffin" (wiki note), section "Local Attention Path": the window
 *       N(t) = {i : t - w < i <= t} and y_t = sum over N(t) of
 *       softmax_i(q_t . k_i) v_i; [G] "Local Sliding-Window Multi-Query
 *       Attention (MQA)" (one key head and one value head shared by all query
 *       heads) and "Bounding the Key-Value Cache Footprint" (the cache holds
 *       at most W positions, the oldest evicted ring-buffer fashion).
 *
 * Readings where the pages are silent or disagree (each is stated where used):
 *  R1  gates are block-diagonal with K = D/H; W[h][o][j] multiplies input
 *      channel hK+j into output channel hK+o (z = W x, W stored [out][in]).
 *  R2  1 - a^2 is computed exactly as -expm1(2*l) with no clamp (the state
 *      update equation has none; the listing's clamp at 1e-7 never binds on
 *      the workloads and would hide the r -> 0 limit the pages describe).
 *  R3  conv tap k (k = 0..3) multiplies u[t-3+k]; tap 3 is the current token
 *      (cross-correlation with 3 zero/history slots on the left, first T
 *      outputs kept).  The history holds the 3 previous pre-conv inputs,
 *      oldest first; absent history means zeros.
 *  R4  absent h0 means zeros (the listing starts from zeros without
 *      prev_state).  State is double here.
 *  R5  the backward is the exact derivative of the forward above (the pages
 *      state no backward); dh_last is an optional extra upstream gradient on
 *      the final state.
 *  R8  the residual layer (Hawk layer, temporal mixer = the recurrent block):
 *      RMSNorm(x) = x / sqrt(mean_d x^2 + eps) * (1 + w) with eps = 1e-6 (not
 *      on the pages); gated MLP = down(GELU_tanh(gate x) * (up x)) without
 *      biases, GELU_tanh(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)));
 *      the MLP width is the caller's (not on the pages).
 *  R9  the attention residual layer: q, k, v are bias-free projections of
 *      RMSNorm(x) (Hq query heads, one key and one value head); rotary
 *      embedding ([G] "Local Sliding-Window Multi-Query Attention (MQA)":
 *      standard RoPE on queries and keys; module page: partial rotary) turns
 *      dimension pairs (j, j + rot/2), j < rot/2, of each head by the angle
 *      p * base^(-2j/rot) at position p, leaving dimensions >= rot as they are;
 *      the output projection is bias-free; the MLP half is that of R8.
 *  R6  the recurrent block ([G] "Non-Linear Multiplicative Gating with GeLU"
 *      and the listing's RecurrentBlock): out = proj_out(y * GeLU(proj_in_2
 *      x)), y the RG-LRU of conv(proj_in_1 x); linear layers without bias,
 *      weights stored [out][in]; GeLU is the exact one, 0.5 v (1 + erf(v /
 *      sqrt 2)), which is what the listing's F.gelu computes (the pages also
 *      show a tanh form for the MLP, not for this merge); the residual add is
 *      the decoder layer's, outside the block.
 *  R7  local attention: the scores carry a caller-given scale (the page's
 *      formula shows none; the workloads pass 1/sqrt(d_head)); the inputs q,
 *      k are taken after any rotary embedding (positional encoding is the
 *      attention block's, outside this operation); the ring slot of position
 *      p is p mod W.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX3(a, b, c, B_, C_) ((((size_t)(a)) * (B_) + (size_t)(b)) * (C_) + (size_t)(c))

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* sigma(z) = 1 / (1 + e^-z)   ([G] notation under the formulation) */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* softplus(v) = log(1 + e^v), written so that neither branch overflows */
static double softplus(double v)
{
    return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

/* Pre-conv input at position tau of stream b, channel d: positions -3..-1
 * come from the history (oldest first), 0..T-1 from u.  (R3) */
static double u_at(const double *u, const double *hist_in, int T, int D,
                   int b, int tau, int d)
{
    if (tau >= 0) return u[IDX3(b, tau, d, T, D)];
    if (!hist_in) return 0.0;
    return hist_in[IDX3(b, 3 + tau, d, 3, D)];
}

/* a1: causal depthwise Conv1D, width 4, with bias ([G] "Temporal Filtering
 * via Separable 1D Convolutions"; listing: Conv1d(padding = 3, groups = D),
 * first T outputs).  x[b][t][d] = cb[d] + sum_k cw[d][k] * u[t-3+k].
 * hist_out[b][j][d] = pre-conv input at position T-3+j. */
void oracle_conv1d(int B, int T, int D, const double *u, const double *cw,
                   const double *cb, const double *hist_in, double *x,
                   double *hist_out)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int d = 0; d < D; ++d) {
                double acc = cb ? cb[d] : 0.0;
                for (int k = 0; k < 4; ++k)
                    acc += cw[(size_t)d * 4 + k] * u_at(u, hist_in, T, D, b, t - 3 + k, d);
                x[IDX3(b, t, d, T, D)] = acc;
            }
    if (hist_out)
        for (int b = 0; b < B; ++b)
            for (int j = 0; j < 3; ++j)
                for (int d = 0; d < D; ++d)
                    hist_out[IDX3(b, j, d, 3, D)] = u_at(u, hist_in, T, D, b, T - 3 + j, d);
}

/* a2: gates ([G] recurrence-gate and input-gate equations; block-diagonal
 * per "Block-Diagonal Sharding"; reading R1).
 * r = sigma(W_a x + b_a), i = sigma(W_x x + b_x) per token, block by block. */
void oracle_gates(int B, int T, int D, int H, const double *x,
                  const double *Wa, const double *ba, const double *Wx,
                  const double *bx, double *r, double *i)
{
    const int K = D / H;
    const long rows = (long)B * T;
    #pragma omp parallel for schedule(static)
    for (long row = 0; row < rows; ++row) {
        const double *xr = x + (size_t)row * D;
        for (int h = 0; h < H; ++h)
            for (int o = 0; o < K; ++o) {
                const int d = h * K + o;
                double za = ba ? ba[d] : 0.0, zx = bx ? bx[d] : 0.0;
                const double *wa = Wa + ((size_t)h * K + o) * K;
                const double *wx = Wx + ((size_t)h * K + o) * K;
                for (int j = 0; j < K; ++j) {
                    za += wa[j] * xr[h * K + j];
                    zx += wx[j] * xr[h * K + j];
                }
                r[(size_t)row * D + d] = sigmoid(za);
                i[(size_t)row * D + d] = sigmoid(zx);
            }
    }
}

/* a3: decay and normalisation ([G] dynamic diagonal decay a_t = a^(c r_t)
 * with a = sigma(Lambda), in the page's log-space form
 * log a_t = -c r_t softplus(-Lambda); the factor sqrt(1 - a_t^2) of the
 * state-update equation, reading R2). */
void oracle_decay(long N, int D, double c, const double *r, const double *Lambda,
                  double *a, double *beta)
{
    #pragma omp parallel for schedule(static)
    for (long n = 0; n < N; ++n)
        for (int d = 0; d < D; ++d) {
            const double s = softplus(-Lambda[d]);
            const double l = -c * r[(size_t)n * D + d] * s;
            a[(size_t)n * D + d] = exp(l);
            beta[(size_t)n * D + d] = sqrt(-expm1(2.0 * l));
        }
}

/* a3 + a4: the diagonal linear scan ([G] state-update and output equations;
 * [W] "Gated Linear Recurrence").  Per lane (b, d), sequentially in t:
 * h_t = a_t h_{t-1} + sqrt(1 - a_t^2) i_t x_t, y_t = h_t, h_last = h_{T-1}.
 * h_{-1} = h0[b][d] (zeros if h0 is NULL, reading R4). */
void oracle_scan(int B, int T, int D, double c, const double *x, const double *r,
                 const double *i, const double *Lambda, const double *h0,
                 double *y, double *h_last)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int d = 0; d < D; ++d) {
            const double s = softplus(-Lambda[d]);
            double h = h0 ? h0[(size_t)b * D + d] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t e = IDX3(b, t, d, T, D);
                const double l = -c * r[e] * s;
                const double a = exp(l);
                const double beta = sqrt(-expm1(2.0 * l));
                h = a * h + beta * i[e] * x[e];
                if (y) y[e] = h;
            }
            if (h_last) h_last[(size_t)b * D + d] = h;
        }
}

/* a5: the whole forward, u -> y: conv, gates, scan (each as above). */
void oracle_fwd(int B, int T, int D, int H, double c, const double *u,
                const double *cw, const double *cb, const double *hist_in,
                const double *Wa, const double *ba, const double *Wx,
                const double *bx, const double *Lambda, const double *h0,
                double *y, double *h_last, double *hist_out)
{
    const size_t n = (size_t)B * T * D;
    double *x = malloc(n * sizeof(double));
    double *r = malloc(n * sizeof(double));
    double *i = malloc(n * sizeof(double));
    if (cw) oracle_conv1d(B, T, D, u, cw, cb, hist_in, x, hist_out);
    else memcpy(x, u, n * sizeof(double));
    oracle_gates(B, T, D, H, x, Wa, ba, Wx, bx, r, i);
    oracle_scan(B, T, D, c, x, r, i, Lambda, h0, y, h_last);
    free(x); free(r); free(i);
}

/* a6: one decode step = the forward with T = 1, the conv history and the
 * state read and written back ([G] listing, RGLRU.step: new state
 * a_t h + sqrt(1 - a_t^2) i_t x_t, returned twice; the conv history is
 * reading R3).  hist [B][3][D] and h [B][D] are in/out. */
void oracle_step(int B, int D, int H, double c, const double *u_t,
                 const double *cw, const double *cb, const double *Wa,
                 const double *ba, const double *Wx, const double *bx,
                 const double *Lambda, double *hist, double *h, double *y_t)
{
    double *hist_new = malloc((size_t)B * 3 * D * sizeof(double));
    double *h_new = malloc((size_t)B * D * sizeof(double));
    oracle_fwd(B, 1, D, H, c, u_t, cw, cb, hist, Wa, ba, Wx, bx, Lambda, h,
               y_t, h_new, hist_new);
    memcpy(hist, hist_new, (size_t)B * 3 * D * sizeof(double));
    memcpy(h, h_new, (size_t)B * D * sizeof(double));
    free(hist_new); free(h_new);
}

/* a7: backward of a5 by the chain rule (reading R5).  Given g_t = dL/dy_t and
 * optional dh_last = dL/dh_{T-1}:
 *   delta_{T-1} = g_{T-1} + dh_last,  delta_t = g_t + a_{t+1} delta_{t+1}
 *   dl_t   = delta_t (a_t h_{t-1} - (a_t^2 / beta_t) i_t x_t)
 *            (da/dl = a, dbeta/dl = -a^2/beta)
 *   dr_t   = -c s dl_t,          dLambda = sum c r_t sigma(-Lambda) dl_t
 *   di_t   = delta_t beta_t x_t, dx_t (direct) = delta_t beta_t i_t
 *   dz^a   = dr r (1 - r),       dz^x = di i (1 - i)
 *   db     = sum dz,             dW[h][o][j] = sum dz_t[hK+o] x_t[hK+j]
 *   dx_t[hK+j] += sum_o W_a[h][o][j] dz^a_t[hK+o] + W_x[h][o][j] dz^x_t[hK+o]
 *   dcb    = sum dx,             dcw[d][k] = sum_t dx_t u_{t-3+k}
 *   du_tau = sum_k cw[k] dx_{tau+3-k}  (terms past T-1 absent)
 *   dh0    = a_0 delta_0
 * Sums over (b, t) run in increasing b then t.  Every gradient is written,
 * not accumulated.  dh0 may be NULL. */
void oracle_bwd(int B, int T, int D, int H, double c, const double *u,
                const double *cw, const double *cb, const double *hist_in,
                const double *Wa, const double *ba, const double *Wx,
                const double *bx, const double *Lambda, const double *h0,
                const double *dy, const double *dh_last, double *du,
                double *dcw, double *dcb, double *dWa, double *dba,
                double *dWx, double *dbx, double *dLambda, double *dh0)
{
    const int K = D / H;
    const size_t n = (size_t)B * T * D;
    double *x = malloc(n * sizeof(double)), *r = malloc(n * sizeof(double));
    double *i = malloc(n * sizeof(double)), *a = malloc(n * sizeof(double));
    double *beta = malloc(n * sizeof(double)), *hprev = malloc(n * sizeof(double));
    double *dl = malloc(n * sizeof(double)), *dza = malloc(n * sizeof(double));
    double *dzx = malloc(n * sizeof(double)), *dx = malloc(n * sizeof(double));

    /* forward recompute: conv, gates, decay, states h_{t-1} */
    oracle_conv1d(B, T, D, u, cw, cb, hist_in, x, NULL);
    oracle_gates(B, T, D, H, x, Wa, ba, Wx, bx, r, i);
    oracle_decay((long)B * T, D, c, r, Lambda, a, beta);
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int d = 0; d < D; ++d) {
            double h = h0 ? h0[(size_t)b * D + d] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t e = IDX3(b, t, d, T, D);
                hprev[e] = h;
                h = a[e] * h + beta[e] * i[e] * x[e];
            }
        }

    /* reverse scan and local derivatives */
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int d = 0; d < D; ++d) {
            const double s = softplus(-Lambda[d]);
            double delta = 0.0;
            for (int t = T - 1; t >= 0; --t) {
                const size_t e = IDX3(b, t, d, T, D);
                delta = dy[e] + (t == T - 1 ? (dh_last ? dh_last[(size_t)b * D + d] : 0.0)
                                            : a[e + D] * delta);
                dl[e] = delta * (a[e] * hprev[e] - (a[e] * a[e] / beta[e]) * i[e] * x[e]);
                const double dr = -c * s * dl[e];
                const double di = delta * beta[e] * x[e];
                dx[e] = delta * beta[e] * i[e];
                dza[e] = dr * r[e] * (1.0 - r[e]);
                dzx[e] = di * i[e] * (1.0 - i[e]);
                if (t == 0 && dh0) dh0[(size_t)b * D + d] = a[e] * delta;
            }
        }

    /* parameter sums over (b, t): biases and Lambda */
    #pragma omp parallel for schedule(static)
    for (int d = 0; d < D; ++d) {
        double sa = 0.0, sx = 0.0, sl = 0.0;
        const double sg = sigmoid(-Lambda[d]);
        for (long row = 0; row < (long)B * T; ++row) {
            const size_t e = (size_t)row * D + d;
            sa += dza[e];
            sx += dzx[e];
            sl += c * r[e] * sg * dl[e];
        }
        dba[d] = sa; dbx[d] = sx; dLambda[d] = sl;
    }

    /* gate weights: dW[h][o][j] = sum_rows dz[hK+o] x[hK+j] */
    #pragma omp parallel for collapse(2) schedule(static)
    for (int h = 0; h < H; ++h)
        for (int o = 0; o < K; ++o)
            for (int j = 0; j < K; ++j) {
                double sa = 0.0, sx = 0.0;
                for (long row = 0; row < (long)B * T; ++row) {
                    const double xv = x[(size_t)row * D + h * K + j];
                    sa += dza[(size_t)row * D + h * K + o] * xv;
                    sx += dzx[(size_t)row * D + h * K + o] * xv;
                }
                dWa[((size_t)h * K + o) * K + j] = sa;
                dWx[((size_t)h * K + o) * K + j] = sx;
            }

    /* dx through the gates: dx[hK+j] += sum_o W[h][o][j] dz[hK+o] */
    #pragma omp parallel for schedule(static)
    for (long row = 0; row < (long)B * T; ++row)
        for (int h = 0; h < H; ++h)
            for (int j = 0; j < K; ++j) {
                double acc = 0.0;
                for (int o = 0; o < K; ++o)
                    acc += Wa[((size_t)h * K + o) * K + j] * dza[(size_t)row * D + h * K + o]
                         + Wx[((size_t)h * K + o) * K + j] * dzx[(size_t)row * D + h * K + o];
                dx[(size_t)row * D + h * K + j] += acc;
            }

    /* conv backward */
    #pragma omp parallel for schedule(static)
    for (int d = 0; d < D; ++d) {
        double sb = 0.0, sw[4] = {0.0, 0.0, 0.0, 0.0};
        for (int b = 0; b < B; ++b)
            for (int t = 0; t < T; ++t) {
                const double g = dx[IDX3(b, t, d, T, D)];
                sb += g;
                for (int k = 0; k < 4; ++k)
                    sw[k] += g * u_at(u, hist_in, T, D, b, t - 3 + k, d);
            }
        dcb[d] = sb;
        for (int k = 0; k < 4; ++k) dcw[(size_t)d * 4 + k] = sw[k];
    }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int tau = 0; tau < T; ++tau)
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int k = 0; k < 4; ++k) {
                    const int t = tau + 3 - k;
                    if (t < T) acc += cw[(size_t)d * 4 + k] * dx[IDX3(b, t, d, T, D)];
                }
                du[IDX3(b, tau, d, T, D)] = acc;
            }

    free(x); free(r); free(i); free(a); free(beta); free(hprev);
    free(dl); free(dza); free(dzx); free(dx);
}

/* ---------------------------------------------------------- recurrent block
 * [G] "Non-Linear Multiplicative Gating with GeLU" (R6). */

/* y[m][n] = sum_k x[m][k] W[n][k]  (a linear layer without bias, W [N][K]) */
void oracle_linear(long M, int K, int N, const double *x, const double *W, double *y)
{
    #pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += x[(size_t)m * K + k] * W[(size_t)n * K + k];
            y[(size_t)m * N + n] = acc;
        }
}

/* GeLU(v) = v Phi(v) = 0.5 v (1 + erf(v / sqrt 2)) */
void oracle_gelu(long n, const double *v, double *out)
{
    #pragma omp parallel for schedule(static)
    for (long e = 0; e < n; ++e) out[e] = 0.5 * v[e] * (1.0 + erf(v[e] / sqrt(2.0)));
}

/* z = y * GeLU(g), elementwise */
void oracle_merge(long n, const double *y, const double *g, double *z)
{
    #pragma omp parallel for schedule(static)
    for (long e = 0; e < n; ++e) z[e] = y[e] * (0.5 * g[e] * (1.0 + erf(g[e] / sqrt(2.0))));
}

/* ------------------------------------------------------------ local attention
 * [N] "Local Attention Path" and [G] "Local Sliding-Window Multi-Query
 * Attention (MQA)" (R7).  q [B][T][Hq][dh], k and v [B][T][dh] (one shared key
 * head and value head), o [B][T][Hq][dh]. */

/* softmax over the scores of one query row, then the weighted sum of values:
 * s_j = scale * (q . key_j) for the n keys given by row pointers, o = sum_j
 * p_j val_j with p = softmax(s) (the maximum is subtracted first, which leaves
 * softmax unchanged) */
static void attend_rows(int n, int dh, double scale, const double *q, const double *const *keys,
                        const double *const *vals, double *s, double *o)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int e = 0; e < dh; ++e) acc += q[e] * keys[j][e];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    double sum = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        sum += s[j];
    }
    for (int e = 0; e < dh; ++e) o[e] = 0.0;
    for (int j = 0; j < n; ++j) {
        const double p = s[j] / sum;
        for (int e = 0; e < dh; ++e) o[e] += p * vals[j][e];
    }
}

/* prefill: token t of stream b attends to positions t-W+1 .. t (those >= 0) */
void oracle_attn_fwd(int B, int T, int Hq, int dh, int W, double scale, const double *q,
                     const double *k, const double *v, double *o)
{
    #pragma omp parallel
    {
        const double **keys = malloc(sizeof(double *) * (size_t)W);
        const double **vals = malloc(sizeof(double *) * (size_t)W);
        double *s = malloc(sizeof(double) * (size_t)W);
        #pragma omp for schedule(dynamic) collapse(2)
        for (int b = 0; b < B; ++b)
            for (int t = 0; t < T; ++t) {
                const int lo = t - W + 1 < 0 ? 0 : t - W + 1;
                const int n = t - lo + 1;
                for (int j = 0; j < n; ++j) {
                    keys[j] = k + ((size_t)b * T + lo + j) * dh;
                    vals[j] = v + ((size_t)b * T + lo + j) * dh;
                }
                for (int h = 0; h < Hq; ++h) {
                    const size_t row = (((size_t)b * T + t) * Hq + h) * dh;
                    attend_rows(n, dh, scale, q + row, keys, vals, s, o + row);
                }
            }
        free(keys);
        free(vals);
        free(s);
    }
}

/* decode: the ring caches kc, vc [B][W][dh] hold the positions before pos[b]
 * (position p in slot p mod W); the new key and value (k_t, v_t [B][dh]) go to
 * slot pos[b] mod W, evicting position pos[b] - W, and q_t [B][Hq][dh]
 * attends to the positions max(0, pos[b]-W+1) .. pos[b]. */
void oracle_attn_step(int B, int Hq, int dh, int W, double scale, const double *q_t,
                      const double *k_t, const double *v_t, double *kc, double *vc,
                      const long *pos, double *o_t)
{
    const double **keys = malloc(sizeof(double *) * (size_t)W);
    const double **vals = malloc(sizeof(double *) * (size_t)W);
    double *s = malloc(sizeof(double) * (size_t)W);
    for (int b = 0; b < B; ++b) {
        const long p = pos[b];
        const size_t slot = (size_t)(p % W);
        for (int e = 0; e < dh; ++e) {
            kc[((size_t)b * W + slot) * dh + e] = k_t[(size_t)b * dh + e];
            vc[((size_t)b * W + slot) * dh + e] = v_t[(size_t)b * dh + e];
        }
        const long lo = p - W + 1 < 0 ? 0 : p - W + 1;
        const int n = (int)(p - lo + 1);
        for (int j = 0; j < n; ++j) {
            const size_t sl = (size_t)((lo + j) % W);
            keys[j] = kc + ((size_t)b * W + sl) * dh;
            vals[j] = vc + ((size_t)b * W + sl) * dh;
        }
        for (int h = 0; h < Hq; ++h) {
            const size_t row = ((size_t)b * Hq + h) * dh;
            attend_rows(n, dh, scale, q_t + row, keys, vals, s, o_t + row);
        }
    }
    free(keys);
    free(vals);
    free(s);
}

/* ------------------------------------------------------------ residual layer
 * [L] "Residual Block View" and the RecurrentGemma module page (R8). */

/* out[m][d] = x[m][d] / sqrt(mean_d x[m][d]^2 + eps) * (1 + w[d]) */
void oracle_rmsnorm(long M, int D, const double *x, const double *w, double eps, double *out)
{
    #pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int d = 0; d < D; ++d) ss += x[(size_t)m * D + d] * x[(size_t)m * D + d];
        const double r = 1.0 / sqrt(ss / D + eps);
        for (int d = 0; d < D; ++d) out[(size_t)m * D + d] = x[(size_t)m * D + d] * r * (1.0 + w[d]);
    }
}

/* GELU, tanh form: v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))) */
void oracle_gelu_tanh(long n, const double *v, double *out)
{
    const double k = sqrt(2.0 / 3.14159265358979323846);   /* sqrt(2 / pi) */
    for (long i = 0; i < n; ++i) out[i] = 0.5 * v[i] * (1.0 + tanh(k * (v[i] + 0.044715 * v[i] * v[i] * v[i])));
}

/* ------------------------------------------------------------ rotary embedding
 * (R9) x [M][H][dh] in place: row m has position pos[m]; pairs (j, j + rot/2)
 * for j < rot/2 turn by pos * base^(-2j/rot). */
void oracle_rope(long M, int H, int dh, int rot, double base, const long *pos, double *x)
{
    const int half = rot / 2;
    for (long m = 0; m < M; ++m)
        for (int h = 0; h < H; ++h) {
            double *v = x + ((size_t)m * H + h) * dh;
            for (int j = 0; j < half; ++j) {
                const double ang = (double)pos[m] * pow(base, -2.0 * j / rot);
                const double c = cos(ang), s = sin(ang);
                const double a = v[j], b = v[j + half];
                v[j] = a * c - b * s;
                v[j + half] = a * s + b * c;
            }
        }
}

/*
 * ttt_oracle.c -- plain, slow, fp64 CPU oracle for the forward scan of a
 * Test-Time-Training (TTT) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library; it does not include include/ttt.h.
 *
 * Sources (cited by page title and section; no other source is used):
 *   [KV]  "Test-Time Training Layers: How Inner-Loop Gradient Descent Replaces
 *         the Transformer KV Cache with Expressive Hidden Models"
 *         (news.premlal.in), section "The Core Mechanism: The Hidden State as a
 *         Machine Learning Model", steps 1-3 (loss with the 1/2 factor, one
 *         gradient step, readout with the updated weights); section "Hardware
 *         Parallelization: The Dual Form and Mini-Batch GPU Acceleration"
 *         (mini-batches of 16 or 32 tokens, dual form equivalent to mini-batch
 *         gradient descent).
 *   [SEQ] "Test-Time Training (TTT) Layers for Sequence Modeling"
 *         (dileepadev.github.io), sections "Mathematical Formulation" and
 *         "Variants: TTT-Linear vs. TTT-MLP" (linear inner model; two-layer MLP
 *         with a SiLU non-linearity).
 *   [MEM] the test-time-training essay on ren-xubin.github.io, paragraph on
 *         the dual form (gradients taken relative to the parameters at the
 *         start of a block, their effects accumulated in causal order) and the
 *         paragraph on fast weights being reset at the end of a sequence.
 *   [E2]  the E2-TTT write-up on zhichai.net, section "The Curse of
 *         Efficiency" (gradients computed at each chunk's start and applied to
 *         the whole chunk), section "E2-TTT's Breakthrough: A Closed-Form
 *         Solution" (gradient descent or momentum gradient descent on the
 *         squared loss, fast weights W and momentum M evolving token by token,
 *         the chunk-end W and M computed exactly) and section "Technical
 *         Details and Practical Implications", "Core Math (Simplified)"
 *         (learning rate alpha, momentum coefficient beta, W_k and M_k at each
 *         chunk's start).
 *
 * What is computed: mini-batch gradient descent in PRIMAL form, token by token,
 * every intermediate fast weight W_t materialised.  This is the plain
 * definition that the chunked dual form reaches exactly (up to rounding
 * order), so the oracle is that definition written out.
 *
 * Conventions (readings where the pages leave a step open):
 *   - row-vector form f(z;W) = z W, W[d_in][d_out] row-major.  The pages'
 *     listings use the column form W k; the two are the same map with
 *     W_row = W_col transposed.
 *   - loss l(W; k, v) = 1/2 || f(k; W) - v ||^2  ([KV] step 1).
 *   - within a mini-batch every gradient is taken at the chunk-start weights
 *     and the gradients are SUMMED (no 1/b) in causal order ([MEM], [E2]).
 *   - token t reads out with the weights after its own update ([KV] step 3).
 *   - a final partial mini-batch (T mod b != 0) follows the same rules.
 *   - eta is one value per head.
 *   - every sequence starts from the given initial weights ([MEM]).
 *
 * Layouts (all dense, row-major, fp64):
 *   Q, K, V, Y : [B][H][T][d]
 *   W0         : [H][d][d]   (w0_per_batch == 0)  or  [B][H][d][d]  (== 1)
 *   W_out      : [B][H][d][d]
 *   MLP: W1 [.][d][m], W2 [.][m][d] with the same leading dims.
 *
 * Parallelism: the (batch, head) chains are independent; they are spread
 * over OpenMP threads.  Inside a chain the loops are sequential and plain.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of OpenMP threads the next parallel region will use. */
int ttt_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear: inner model f(z; W) = z W ([SEQ] "TTT-Linear").               */
/* ------------------------------------------------------------------------ */

/* One (batch, head) chain of the linear scan.  q, k, v, y point at [T][d]. */
static void linear_chain(const double* q, const double* k, const double* v,
                         const double* w_init, double eta, long T, long d, long b,
                         double* y, double* w_final,
                         double* W, double* Wc, double* G, double* Wt, double* r)
{
    const long dd = d * d;
    memcpy(W, w_init, (size_t)dd * sizeof(double));
    for (long s = 0; s < T; s += b) {
        long e = s + b < T ? s + b : T;
        /* chunk-start weights; accumulated gradient starts at zero */
        memcpy(Wc, W, (size_t)dd * sizeof(double));
        memset(G, 0, (size_t)dd * sizeof(double));
        for (long t = s; t < e; ++t) {
            const double* kt = k + t * d;
            const double* vt = v + t * d;
            const double* qt = q + t * d;
            /* residual of the reconstruction at the chunk-start weights:
             * r = k Wc - v, so grad_W 1/2||k W - v||^2 = k^T r ([KV] step 1-2) */
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += kt[i] * Wc[i * d + j];
                r[j] = acc - vt[j];
            }
            /* G += k^T r  (sum over the tokens of the chunk so far) */
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    G[i * d + j] += kt[i] * r[j];
            /* W_t = Wc - eta G  ([KV] step 2, mini-batch reading) */
            for (long x = 0; x < dd; ++x)
                Wt[x] = Wc[x] - eta * G[x];
            /* y_t = q_t W_t  ([KV] step 3: readout after the update) */
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += qt[i] * Wt[i * d + j];
                y[t * d + j] = acc;
            }
        }
        /* the weights after the chunk are those after its last token */
        memcpy(W, Wt, (size_t)dd * sizeof(double));
    }
    memcpy(w_final, W, (size_t)dd * sizeof(double));
}

int ttt_oracle_linear_forward(const double* Q, const double* K, const double* V,
                              const double* W0, int w0_per_batch, const double* eta,
                              long B, long H, long T, long d, long b,
                              double* Y, double* W_out, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1)
        return ORACLE_EINVAL;
    if (!W0 || !eta || !W_out || (T > 0 && (!Q || !K || !V || !Y)))
        return ORACLE_EINVAL;
    const long dd = d * d;
    const long units = B * H;
    int status = ORACLE_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* ws = (double*)malloc((size_t)(4 * dd + d) * sizeof(double));
        if (!ws) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!ws)
                continue;
            long h = u % H;
            const double* w_init = W0 + (w0_per_batch ? u : h) * dd;
            const long off = u * T * d;
            linear_chain(Q + off, K + off, V + off, w_init, eta[h], T, d, b,
                         Y + off, W_out + u * dd,
                         ws, ws + dd, ws + 2 * dd, ws + 3 * dd, ws + 4 * dd);
        }
        free(ws);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear with a step size per token: token t's gradient term is scaled   */
/* by eta_t instead of the head's eta (the uTTT write-up on thelatestinai.com, */
/* Table D3: learning rates per token, head and matrix).  Same primal loops:  */
/*   r_t = k_t Wc - v_t,  G_t = G_{t-1} + eta_t k_t^T r_t,  W_t = Wc - G_t,   */
/*   y_t = q_t W_t.                                                           */
/* eta_tok: [B][H][T].  read_start != 0: every token of a mini-batch reads   */
/* out with the chunk-start weights instead, y_t = q_t Wc (the uTTT write-up, */
/* Figure 2(a): forward reads use the chunk-start state).                     */
/* ------------------------------------------------------------------------ */
static void linear_chain_tok(const double* q, const double* k, const double* v,
                             const double* w_init, const double* eta_t, int read_start,
                             long T, long d, long b, double* y, double* w_final,
                             double* W, double* Wc, double* G, double* Wt, double* r)
{
    const long dd = d * d;
    memcpy(W, w_init, (size_t)dd * sizeof(double));
    for (long s = 0; s < T; s += b) {
        long e = s + b < T ? s + b : T;
        memcpy(Wc, W, (size_t)dd * sizeof(double));
        memset(G, 0, (size_t)dd * sizeof(double));
        for (long t = s; t < e; ++t) {
            const double* kt = k + t * d;
            const double* vt = v + t * d;
            const double* qt = q + t * d;
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += kt[i] * Wc[i * d + j];
                r[j] = acc - vt[j];
            }
            /* G += eta_t k^T r: this token's step, at the chunk-start weights */
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    G[i * d + j] += eta_t[t] * kt[i] * r[j];
            for (long x = 0; x < dd; ++x)
                Wt[x] = Wc[x] - G[x];
            const double* Wr = read_start ? Wc : Wt;
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += qt[i] * Wr[i * d + j];
                y[t * d + j] = acc;
            }
        }
        memcpy(W, Wt, (size_t)dd * sizeof(double));
    }
    memcpy(w_final, W, (size_t)dd * sizeof(double));
}

int ttt_oracle_linear_forward_tok(const double* Q, const double* K, const double* V,
                                  const double* W0, int w0_per_batch, const double* eta_tok,
                                  int read_start, long B, long H, long T, long d, long b,
                                  double* Y, double* W_out, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1)
        return ORACLE_EINVAL;
    if (!W0 || !W_out || (T > 0 && (!Q || !K || !V || !Y || !eta_tok)))
        return ORACLE_EINVAL;
    const long dd = d * d;
    const long units = B * H;
    int status = ORACLE_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* ws = (double*)malloc((size_t)(4 * dd + d) * sizeof(double));
        if (!ws) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!ws)
                continue;
            long h = u % H;
            const double* w_init = W0 + (w0_per_batch ? u : h) * dd;
            const long off = u * T * d;
            linear_chain_tok(Q + off, K + off, V + off, w_init, eta_tok + u * T, read_start,
                             T, d, b, Y + off, W_out + u * dd,
                             ws, ws + dd, ws + 2 * dd, ws + 3 * dd, ws + 4 * dd);
        }
        free(ws);
    }
    return status;
}

/* LayerNorm over the last dimension of n rows of length d, in place:
 * x <- (x - mean) / sqrt(var + eps) * gamma + beta, with the biased variance
 * ([KV] listing: LayerNorm of the projected keys and queries).  gamma, beta
 * point at [H][d] each; row i belongs to head (i / T) % H. */
int ttt_oracle_layernorm_rows(double* X, long n, long T, long H, long d, const double* gamma,
                              const double* beta, double eps)
{
    if (n < 0 || T < 1 || H < 1 || d < 1 || !gamma || !beta || eps < 0.0 || (n > 0 && !X))
        return ORACLE_EINVAL;
    for (long i = 0; i < n; ++i) {
        double* x = X + i * d;
        const long h = (i / T) % H;
        double mean = 0.0;
        for (long j = 0; j < d; ++j)
            mean += x[j];
        mean /= (double)d;
        double var = 0.0;
        for (long j = 0; j < d; ++j)
            var += (x[j] - mean) * (x[j] - mean);
        var /= (double)d;
        const double inv = 1.0 / sqrt(var + eps);
        for (long j = 0; j < d; ++j)
            x[j] = (x[j] - mean) * inv * gamma[h * d + j] + beta[h * d + j];
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward of the TTT-Linear scan: the vector-Jacobian product of the map    */
/* (Q, K, V, W0, eta) -> (Y, W_out) computed above, for cotangents dY and     */
/* dW_out.  Outer-loop training differentiates the layer output through the   */
/* inner updates ([KV] section "Hardware Parallelization": the dual form      */
/* exists for training; the uTTT write-up on thelatestinai.com, Figure 2(b):  */
/* the read-output Jacobian runs backward through the earlier inner updates). */
/*                                                                            */
/* Written as reverse-mode differentiation of the primal loops of             */
/* linear_chain, token by token, with every intermediate quantity recomputed  */
/* from the chunk-start weights of the forward sweep:                         */
/*   r_t = k_t Wc - v_t,  G_t = G_{t-1} + k_t^T r_t,  W_t = Wc - eta G_t,     */
/*   y_t = q_t W_t,  and the weights after a chunk are W_{last token}.        */
/* Adjoints are written xb (x-bar).                                           */
/* ------------------------------------------------------------------------ */

struct lin_bwd_ws {
    double *Wcs;   /* [nchunks][d][d] chunk-start weights of the forward sweep */
    double *Gs;    /* [b][d][d]  G_t of the tokens of the current chunk       */
    double *R;     /* [b][d]     r_t of the tokens of the current chunk       */
    double *Wt;    /* [d][d]     W_t                                          */
    double *Wb;    /* [d][d]     adjoint of the weights after the chunk       */
    double *Wcb;   /* [d][d]     adjoint of the chunk-start weights           */
    double *Gb;    /* [d][d]     adjoint of G_t                               */
    double *Wtb;   /* [d][d]     adjoint of W_t                               */
    double *rb;    /* [d]        adjoint of r_t                               */
};

static void linear_chain_backward(const double* q, const double* k, const double* v,
                                  const double* w_init, double eta, long T, long d, long b,
                                  const double* dy, const double* dw_out,
                                  double* dq, double* dk, double* dv, double* dw0,
                                  double* deta, struct lin_bwd_ws* w)
{
    const long dd = d * d;
    const long nc = (T + b - 1) / b;

    /* forward sweep: chunk-start weights of every chunk */
    memcpy(w->Wcs, w_init, (size_t)dd * sizeof(double));
    for (long c = 0; c + 1 < nc; ++c) {
        const long s = c * b, e = s + b;
        const double* Wc = w->Wcs + c * dd;
        double* Wn = w->Wcs + (c + 1) * dd;
        memcpy(Wn, Wc, (size_t)dd * sizeof(double));
        for (long t = s; t < e; ++t) {
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += k[t * d + i] * Wc[i * d + j];
                w->rb[j] = acc - v[t * d + j];
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    Wn[i * d + j] -= eta * k[t * d + i] * w->rb[j];
        }
    }

    /* backward sweep */
    memcpy(w->Wb, dw_out, (size_t)dd * sizeof(double));
    double eb = 0.0;
    for (long c = nc - 1; c >= 0; --c) {
        const long s = c * b, e = s + b < T ? s + b : T;
        const double* Wc = w->Wcs + c * dd;
        /* recompute r_t and G_t of the chunk */
        for (long t = s; t < e; ++t) {
            double* r = w->R + (t - s) * d;
            double* G = w->Gs + (t - s) * dd;
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += k[t * d + i] * Wc[i * d + j];
                r[j] = acc - v[t * d + j];
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    G[i * d + j] = (t > s ? G[i * d + j - dd] : 0.0) + k[t * d + i] * r[j];
        }
        memset(w->Wcb, 0, (size_t)dd * sizeof(double));
        memset(w->Gb, 0, (size_t)dd * sizeof(double));
        for (long t = e - 1; t >= s; --t) {
            const double* r = w->R + (t - s) * d;
            const double* G = w->Gs + (t - s) * dd;
            /* W_t = Wc - eta G_t */
            for (long x = 0; x < dd; ++x)
                w->Wt[x] = Wc[x] - eta * G[x];
            /* y_t = q_t W_t:  qb_t = yb_t W_t^T,  Wtb = q_t^T yb_t; the last token's
             * W_t is also the weights after the chunk */
            for (long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += dy[t * d + j] * w->Wt[i * d + j];
                dq[t * d + i] = acc;
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    w->Wtb[i * d + j] = q[t * d + i] * dy[t * d + j]
                                        + (t == e - 1 ? w->Wb[i * d + j] : 0.0);
            /* W_t = Wc - eta G_t:  Wcb += Wtb,  Gb += -eta Wtb,  etab += -<Wtb, G_t> */
            for (long x = 0; x < dd; ++x) {
                w->Wcb[x] += w->Wtb[x];
                w->Gb[x] -= eta * w->Wtb[x];
                eb -= w->Wtb[x] * G[x];
            }
            /* G_t = G_{t-1} + k_t^T r_t:  kb_t = Gb r_t,  rb_t = k_t Gb
             * (Gb now holds the adjoint of G_t: every W_u with u >= t uses it) */
            for (long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += w->Gb[i * d + j] * r[j];
                dk[t * d + i] = acc;
            }
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += k[t * d + i] * w->Gb[i * d + j];
                w->rb[j] = acc;
            }
            /* r_t = k_t Wc - v_t:  kb_t += rb_t Wc^T,  Wcb += k_t^T rb_t,  vb_t = -rb_t */
            for (long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += w->rb[j] * Wc[i * d + j];
                dk[t * d + i] += acc;
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    w->Wcb[i * d + j] += k[t * d + i] * w->rb[j];
            for (long j = 0; j < d; ++j)
                dv[t * d + j] = -w->rb[j];
        }
        /* the chunk-start weights are the weights after the previous chunk */
        memcpy(w->Wb, w->Wcb, (size_t)dd * sizeof(double));
    }
    memcpy(dw0, w->Wb, (size_t)dd * sizeof(double));
    *deta = eb;
}

/* dQ, dK, dV: [B][H][T][d]; dW0 per chain: [B][H][d][d]; deta per chain:
 * [B][H] (summing over the batch where W0 or eta is shared is left to the
 * caller).  T = 0 gives dW0 = dW_out and deta = 0. */
int ttt_oracle_linear_backward(const double* Q, const double* K, const double* V,
                               const double* W0, int w0_per_batch, const double* eta,
                               long B, long H, long T, long d, long b,
                               const double* dY, const double* dW_out,
                               double* dQ, double* dK, double* dV,
                               double* dW0_chain, double* deta_chain, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1)
        return ORACLE_EINVAL;
    if (!W0 || !eta || !dW_out || !dW0_chain || !deta_chain ||
        (T > 0 && (!Q || !K || !V || !dY || !dQ || !dK || !dV)))
        return ORACLE_EINVAL;
    const long dd = d * d;
    const long units = B * H;
    const long nc = (T + b - 1) / b;
    const long bb = b < T ? b : (T > 0 ? T : 1);
    int status = ORACLE_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        const size_t n = (size_t)((nc > 0 ? nc : 1) * dd + bb * dd + bb * d + 5 * dd + d);
        double* buf = (double*)malloc(n * sizeof(double));
        struct lin_bwd_ws w = {0};
        if (!buf) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
        } else {
            w.Wcs = buf;
            w.Gs = w.Wcs + (nc > 0 ? nc : 1) * dd;
            w.R = w.Gs + bb * dd;
            w.Wt = w.R + bb * d;
            w.Wb = w.Wt + dd;
            w.Wcb = w.Wb + dd;
            w.Gb = w.Wcb + dd;
            w.Wtb = w.Gb + dd;
            w.rb = w.Wtb + dd;
        }
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!buf)
                continue;
            long h = u % H;
            const double* w_init = W0 + (w0_per_batch ? u : h) * dd;
            const long off = u * T * d;
            linear_chain_backward(Q + off, K + off, V + off, w_init, eta[h], T, d, b,
                                  dY + off, dW_out + u * dd, dQ + off, dK + off, dV + off,
                                  dW0_chain + u * dd, deta_chain + u, &w);
        }
        free(buf);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Backward of linear_chain_tok (per-token step sizes, optional chunk-start   */
/* read): reverse mode of its primal loops, token by token, as above:         */
/*   r_t = k_t Wc - v_t,  G_t = G_{t-1} + eta_t k_t^T r_t,  W_t = Wc - G_t,   */
/*   y_t = q_t (read_start ? Wc : W_t);  weights after a chunk = W_last.      */
/* deta_tok receives the gradient of every token's step size.                 */
/* ------------------------------------------------------------------------ */
static void linear_chain_tok_backward(const double* q, const double* k, const double* v,
                                      const double* w_init, const double* eta_t, int read_start,
                                      long T, long d, long b, const double* dy,
                                      const double* dw_out, double* dq, double* dk, double* dv,
                                      double* dw0, double* deta_tok, struct lin_bwd_ws* w)
{
    const long dd = d * d;
    const long nc = (T + b - 1) / b;

    /* forward sweep: chunk-start weights */
    memcpy(w->Wcs, w_init, (size_t)dd * sizeof(double));
    for (long c = 0; c + 1 < nc; ++c) {
        const long s = c * b, e = s + b;
        const double* Wc = w->Wcs + c * dd;
        double* Wn = w->Wcs + (c + 1) * dd;
        memcpy(Wn, Wc, (size_t)dd * sizeof(double));
        for (long t = s; t < e; ++t) {
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += k[t * d + i] * Wc[i * d + j];
                w->rb[j] = acc - v[t * d + j];
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    Wn[i * d + j] -= eta_t[t] * k[t * d + i] * w->rb[j];
        }
    }

    memcpy(w->Wb, dw_out, (size_t)dd * sizeof(double));
    for (long c = nc - 1; c >= 0; --c) {
        const long s = c * b, e = s + b < T ? s + b : T;
        const double* Wc = w->Wcs + c * dd;
        for (long t = s; t < e; ++t) {
            double* r = w->R + (t - s) * d;
            double* G = w->Gs + (t - s) * dd;
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += k[t * d + i] * Wc[i * d + j];
                r[j] = acc - v[t * d + j];
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    G[i * d + j] = (t > s ? G[i * d + j - dd] : 0.0) + eta_t[t] * k[t * d + i] * r[j];
        }
        memset(w->Wcb, 0, (size_t)dd * sizeof(double));
        memset(w->Gb, 0, (size_t)dd * sizeof(double));
        for (long t = e - 1; t >= s; --t) {
            const double* r = w->R + (t - s) * d;
            const double* G = w->Gs + (t - s) * dd;
            for (long x = 0; x < dd; ++x)
                w->Wt[x] = Wc[x] - G[x];
            /* readout: y_t = q_t Wr with Wr = Wc or W_t */
            const double* Wr = read_start ? Wc : w->Wt;
            for (long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += dy[t * d + j] * Wr[i * d + j];
                dq[t * d + i] = acc;
            }
            /* adjoint of W_t: the readout's share (when it reads W_t) and, for
             * the last token, the weights after the chunk */
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j) {
                    const double qy = q[t * d + i] * dy[t * d + j];
                    w->Wtb[i * d + j] = (read_start ? 0.0 : qy) + (t == e - 1 ? w->Wb[i * d + j] : 0.0);
                    if (read_start)
                        w->Wcb[i * d + j] += qy;
                }
            /* W_t = Wc - G_t */
            for (long x = 0; x < dd; ++x) {
                w->Wcb[x] += w->Wtb[x];
                w->Gb[x] -= w->Wtb[x];
            }
            /* G_t = G_{t-1} + eta_t k_t^T r_t:  etab_t = k_t Gb r_t^T,
             * kb_t = eta_t Gb r_t,  rb_t = eta_t k_t Gb */
            double et_b = 0.0;
            for (long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += w->Gb[i * d + j] * r[j];
                dk[t * d + i] = eta_t[t] * acc;
                et_b += k[t * d + i] * acc;
            }
            deta_tok[t] = et_b;
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += k[t * d + i] * w->Gb[i * d + j];
                w->rb[j] = eta_t[t] * acc;
            }
            /* r_t = k_t Wc - v_t */
            for (long i = 0; i < d; ++i) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += w->rb[j] * Wc[i * d + j];
                dk[t * d + i] += acc;
            }
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < d; ++j)
                    w->Wcb[i * d + j] += k[t * d + i] * w->rb[j];
            for (long j = 0; j < d; ++j)
                dv[t * d + j] = -w->rb[j];
        }
        memcpy(w->Wb, w->Wcb, (size_t)dd * sizeof(double));
    }
    memcpy(dw0, w->Wb, (size_t)dd * sizeof(double));
}

/* dQ, dK, dV: [B][H][T][d]; dW0 per chain [B][H][d][d]; deta_tok [B][H][T]. */
int ttt_oracle_linear_backward_tok(const double* Q, const double* K, const double* V,
                                   const double* W0, int w0_per_batch, const double* eta_tok,
                                   int read_start, long B, long H, long T, long d, long b,
                                   const double* dY, const double* dW_out,
                                   double* dQ, double* dK, double* dV,
                                   double* dW0_chain, double* deta_tok, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1)
        return ORACLE_EINVAL;
    if (!W0 || !dW_out || !dW0_chain ||
        (T > 0 && (!Q || !K || !V || !dY || !dQ || !dK || !dV || !eta_tok || !deta_tok)))
        return ORACLE_EINVAL;
    const long dd = d * d;
    const long units = B * H;
    const long nc = (T + b - 1) / b;
    const long bb = b < T ? b : (T > 0 ? T : 1);
    int status = ORACLE_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        const size_t n = (size_t)((nc > 0 ? nc : 1) * dd + bb * dd + bb * d + 5 * dd + d);
        double* buf = (double*)malloc(n * sizeof(double));
        struct lin_bwd_ws w = {0};
        if (!buf) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
        } else {
            w.Wcs = buf;
            w.Gs = w.Wcs + (nc > 0 ? nc : 1) * dd;
            w.R = w.Gs + bb * dd;
            w.Wt = w.R + bb * d;
            w.Wb = w.Wt + dd;
            w.Wcb = w.Wb + dd;
            w.Gb = w.Wcb + dd;
            w.Wtb = w.Gb + dd;
            w.rb = w.Wtb + dd;
        }
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!buf)
                continue;
            long h = u % H;
            const double* w_init = W0 + (w0_per_batch ? u : h) * dd;
            const long off = u * T * d;
            linear_chain_tok_backward(Q + off, K + off, V + off, w_init, eta_tok + u * T,
                                      read_start, T, d, b, dY + off, dW_out + u * dd, dQ + off,
                                      dK + off, dV + off, dW0_chain + u * dd, deta_tok + u * T, &w);
        }
        free(buf);
    }
    return status;
}

/* Backward of ttt_oracle_layernorm_rows: given X (the rows before the
 * normalisation) and dX holding the gradient of the normalised rows,
 * overwrite dX with the gradient of the raw rows and add the gradients of
 * gamma and beta into dgb ([H][2][d]: gamma row, then beta row).  With
 * xh = (x - mean) / sqrt(var + eps) and y = xh gamma + beta:
 *   dgamma += dy xh,  dbeta += dy,  dxh = dy gamma,
 *   dx = (dxh - mean(dxh) - xh mean(dxh xh)) / sqrt(var + eps). */
int ttt_oracle_layernorm_rows_backward(const double* X, double* dX, long n, long T, long H, long d,
                                       const double* gamma, double eps, double* dgb)
{
    if (n < 0 || T < 1 || H < 1 || d < 1 || !gamma || !dgb || eps < 0.0 || (n > 0 && (!X || !dX)))
        return ORACLE_EINVAL;
    double* xh = (double*)malloc((size_t)(2 * d) * sizeof(double));
    if (!xh)
        return ORACLE_ENOMEM;
    double* dxh = xh + d;
    for (long i = 0; i < n; ++i) {
        const double* x = X + i * d;
        double* g = dX + i * d;
        const long h = (i / T) % H;
        double mean = 0.0;
        for (long j = 0; j < d; ++j)
            mean += x[j];
        mean /= (double)d;
        double var = 0.0;
        for (long j = 0; j < d; ++j)
            var += (x[j] - mean) * (x[j] - mean);
        var /= (double)d;
        const double inv = 1.0 / sqrt(var + eps);
        double m1 = 0.0, m2 = 0.0;
        for (long j = 0; j < d; ++j) {
            xh[j] = (x[j] - mean) * inv;
            dgb[(2 * h) * d + j] += g[j] * xh[j];
            dgb[(2 * h + 1) * d + j] += g[j];
            dxh[j] = g[j] * gamma[h * d + j];
            m1 += dxh[j];
            m2 += dxh[j] * xh[j];
        }
        m1 /= (double)d;
        m2 /= (double)d;
        for (long j = 0; j < d; ++j)
            g[j] = (dxh[j] - m1 - xh[j] * m2) * inv;
    }
    free(xh);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* TTT-MLP: f(z; W1, W2) = SiLU(z W1) W2, d -> m -> d, no biases             */
/* ([SEQ] "TTT-MLP": two-layer MLP with a SiLU non-linearity).                */
/* ------------------------------------------------------------------------ */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * sigmoid(x); }
/* d/dx [x sigma(x)] = sigma(x) + x sigma(x) (1 - sigma(x)) */
static double silu_grad(double x)
{
    double s = sigmoid(x);
    return s * (1.0 + x * (1.0 - s));
}

struct mlp_ws {
    double *A1, *A2, *A1c, *A2c, *G1, *G2, *W1t, *W2t;
    double *h, *a, *e, *ga, *dh, *hq, *aq;
};

static void mlp_chain(const double* q, const double* k, const double* v,
                      const double* w1_init, const double* w2_init, double eta,
                      long T, long d, long m, long b,
                      double* y, double* w1_final, double* w2_final, struct mlp_ws* w)
{
    const long dm = d * m;
    memcpy(w->A1, w1_init, (size_t)dm * sizeof(double));
    memcpy(w->A2, w2_init, (size_t)dm * sizeof(double));
    for (long s = 0; s < T; s += b) {
        long e = s + b < T ? s + b : T;
        memcpy(w->A1c, w->A1, (size_t)dm * sizeof(double));
        memcpy(w->A2c, w->A2, (size_t)dm * sizeof(double));
        memset(w->G1, 0, (size_t)dm * sizeof(double));
        memset(w->G2, 0, (size_t)dm * sizeof(double));
        for (long t = s; t < e; ++t) {
            const double* kt = k + t * d;
            const double* vt = v + t * d;
            const double* qt = q + t * d;
            /* forward of the inner model on the key, at the chunk-start weights */
            for (long p = 0; p < m; ++p) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += kt[i] * w->A1c[i * m + p];
                w->h[p] = acc;
                w->a[p] = silu(acc);
            }
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long p = 0; p < m; ++p)
                    acc += w->a[p] * w->A2c[p * d + j];
                w->e[j] = acc - vt[j];                       /* dl/dz */
            }
            /* backward through the inner model (chain rule) */
            for (long p = 0; p < m; ++p) {
                double acc = 0.0;
                for (long j = 0; j < d; ++j)
                    acc += w->e[j] * w->A2c[p * d + j];
                w->ga[p] = acc;                              /* dl/da */
                w->dh[p] = acc * silu_grad(w->h[p]);         /* dl/dh */
            }
            for (long p = 0; p < m; ++p)
                for (long j = 0; j < d; ++j)
                    w->G2[p * d + j] += w->a[p] * w->e[j];   /* dl/dW2 = a^T e */
            for (long i = 0; i < d; ++i)
                for (long p = 0; p < m; ++p)
                    w->G1[i * m + p] += kt[i] * w->dh[p];    /* dl/dW1 = k^T dh */
            /* weights after token t, then the readout with them */
            for (long x = 0; x < dm; ++x) {
                w->W1t[x] = w->A1c[x] - eta * w->G1[x];
                w->W2t[x] = w->A2c[x] - eta * w->G2[x];
            }
            for (long p = 0; p < m; ++p) {
                double acc = 0.0;
                for (long i = 0; i < d; ++i)
                    acc += qt[i] * w->W1t[i * m + p];
                w->hq[p] = acc;
                w->aq[p] = silu(acc);
            }
            for (long j = 0; j < d; ++j) {
                double acc = 0.0;
                for (long p = 0; p < m; ++p)
                    acc += w->aq[p] * w->W2t[p * d + j];
                y[t * d + j] = acc;
            }
        }
        memcpy(w->A1, w->W1t, (size_t)dm * sizeof(double));
        memcpy(w->A2, w->W2t, (size_t)dm * sizeof(double));
    }
    memcpy(w1_final, w->A1, (size_t)dm * sizeof(double));
    memcpy(w2_final, w->A2, (size_t)dm * sizeof(double));
}

int ttt_oracle_mlp_forward(const double* Q, const double* K, const double* V,
                           const double* W1_0, const double* W2_0, int w0_per_batch,
                           const double* eta, long B, long H, long T, long d, long m, long b,
                           double* Y, double* W1_out, double* W2_out, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || d < 1 || m < 1 || b < 1)
        return ORACLE_EINVAL;
    if (!W1_0 || !W2_0 || !eta || !W1_out || !W2_out ||
        (T > 0 && (!Q || !K || !V || !Y)))
        return ORACLE_EINVAL;
    const long dm = d * m;
    const long units = B * H;
    int status = ORACLE_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* buf = (double*)malloc((size_t)(8 * dm + 6 * m + d) * sizeof(double));
        struct mlp_ws w;
        memset(&w, 0, sizeof w);
        if (!buf) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
        } else {
            w.A1 = buf;
            w.A2 = w.A1 + dm;
            w.A1c = w.A2 + dm;
            w.A2c = w.A1c + dm;
            w.G1 = w.A2c + dm;
            w.G2 = w.G1 + dm;
            w.W1t = w.G2 + dm;
            w.W2t = w.W1t + dm;
            w.h = w.W2t + dm;
            w.a = w.h + m;
            w.ga = w.a + m;
            w.dh = w.ga + m;
            w.hq = w.dh + m;
            w.aq = w.hq + m;
            w.e = w.aq + m;
        }
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!buf)
                continue;
            long h = u % H;
            long src = w0_per_batch ? u : h;
            const long off = u * T * d;
            mlp_chain(Q + off, K + off, V + off, W1_0 + src * dm, W2_0 + src * dm, eta[h],
                      T, d, m, b, Y + off, W1_out + u * dm, W2_out + u * dm, &w);
        }
        free(buf);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear single-token step (online gradient descent, the b = 1 case):    */
/* r = k W - v; W <- W - eta k^T r; y = q W  ([KV] steps 1-3; the section on  */
/* the dual form names online GD as the form used for token-by-token decode). */
/* q, k, v, y: [B][H][d]; W: [B][H][d][d] updated in place.                   */
/* ------------------------------------------------------------------------ */
int ttt_oracle_linear_decode(const double* q, const double* k, const double* v,
                             double* W, const double* eta, long B, long H, long d,
                             double* y)
{
    if (B < 0 || H < 0 || d < 1)
        return ORACLE_EINVAL;
    if (B * H > 0 && (!q || !k || !v || !W || !eta || !y))
        return ORACLE_EINVAL;
    double* r = (double*)malloc((size_t)d * sizeof(double));
    if (!r)
        return ORACLE_ENOMEM;
    for (long u = 0; u < B * H; ++u) {
        long h = u % H;
        const double* kt = k + u * d;
        const double* vt = v + u * d;
        const double* qt = q + u * d;
        double* Wu = W + u * d * d;
        for (long j = 0; j < d; ++j) {
            double acc = 0.0;
            for (long i = 0; i < d; ++i)
                acc += kt[i] * Wu[i * d + j];
            r[j] = acc - vt[j];
        }
        for (long i = 0; i < d; ++i)
            for (long j = 0; j < d; ++j) {
                double g = kt[i] * r[j];                     /* grad = k^T r */
                Wu[i * d + j] -= eta[h] * g;
            }
        for (long j = 0; j < d; ++j) {
            double acc = 0.0;
            for (long i = 0; i < d; ++i)
                acc += qt[i] * Wu[i * d + j];
            y[u * d + j] = acc;
        }
    }
    free(r);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* TTT-Linear with momentum gradient descent ([E2] "E2-TTT's Breakthrough"   */
/* and "Core Math"): fast weights W and a momentum M of the same shape, one   */
/* step per token on the squared loss 1/2 ||k W - v||^2:                      */
/*     r_t = k_t W_g - v_t                (residual; grad = k_t^T r_t)        */
/*     M_t = beta M_{t-1} + k_t^T r_t                                         */
/*     W_t = W_{t-1} - eta M_t                                                */
/*     y_t = q_t W_t                      (readout after the update, [KV])    */
/* The point W_g where the gradient is taken:                                 */
/*   grad_mode 0: W_g = W_{t-1}, the exact token-level step (online GD, and   */
/*                momentum GD, with no chunk approximation);                  */
/*   grad_mode 1: W_g = the weights at the start of the token's chunk of b    */
/*                tokens (the chunk-start gradients of "The Curse of          */
/*                Efficiency"); with beta = 0 this is the mini-batch scan of  */
/*                ttt_oracle_linear_forward.                                  */
/* b only matters in grad_mode 1.  beta is one value per head, like eta.      */
/* M0: null (every chain starts with M = 0) or [B][H][d][d].                  */
/* Outputs Y [B][H][T][d], W_out and M_out [B][H][d][d].                      */
/* ------------------------------------------------------------------------ */
static void momentum_chain(const double* q, const double* k, const double* v,
                           const double* w_init, const double* m_init, double eta, double beta,
                           int grad_mode, long T, long d, long b, double* y, double* w_final,
                           double* m_final, double* W, double* M, double* Wc, double* r)
{
    const long dd = d * d;
    memcpy(W, w_init, (size_t)dd * sizeof(double));
    if (m_init)
        memcpy(M, m_init, (size_t)dd * sizeof(double));
    else
        memset(M, 0, (size_t)dd * sizeof(double));
    for (long t = 0; t < T; ++t) {
        if (t % b == 0)
            memcpy(Wc, W, (size_t)dd * sizeof(double));   /* chunk start */
        const double* Wg = grad_mode ? Wc : W;
        const double* kt = k + t * d;
        const double* vt = v + t * d;
        const double* qt = q + t * d;
        for (long j = 0; j < d; ++j) {
            double acc = 0.0;
            for (long i = 0; i < d; ++i)
                acc += kt[i] * Wg[i * d + j];
            r[j] = acc - vt[j];
        }
        /* M <- beta M + k^T r, then W <- W - eta M */
        for (long i = 0; i < d; ++i)
            for (long j = 0; j < d; ++j) {
                M[i * d + j] = beta * M[i * d + j] + kt[i] * r[j];
                W[i * d + j] -= eta * M[i * d + j];
            }
        for (long j = 0; j < d; ++j) {
            double acc = 0.0;
            for (long i = 0; i < d; ++i)
                acc += qt[i] * W[i * d + j];
            y[t * d + j] = acc;
        }
    }
    memcpy(w_final, W, (size_t)dd * sizeof(double));
    memcpy(m_final, M, (size_t)dd * sizeof(double));
}

int ttt_oracle_linear_momentum(const double* Q, const double* K, const double* V,
                               const double* W0, int w0_per_batch, const double* M0,
                               const double* eta, const double* beta, int grad_mode,
                               long B, long H, long T, long d, long b,
                               double* Y, double* W_out, double* M_out, int nthreads)
{
    if (B < 0 || H < 0 || T < 0 || d < 1 || b < 1 || (grad_mode != 0 && grad_mode != 1))
        return ORACLE_EINVAL;
    if (!W0 || !eta || !beta || !W_out || !M_out || (T > 0 && (!Q || !K || !V || !Y)))
        return ORACLE_EINVAL;
    const long dd = d * d;
    const long units = B * H;
    int status = ORACLE_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double* ws = (double*)malloc((size_t)(3 * dd + d) * sizeof(double));
        if (!ws) {
#pragma omp atomic write
            status = ORACLE_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!ws)
                continue;
            long h = u % H;
            const long off = u * T * d;
            momentum_chain(Q + off, K + off, V + off, W0 + (w0_per_batch ? u : h) * dd,
                           M0 ? M0 + u * dd : NULL, eta[h], beta[h], grad_mode, T, d, b,
                           Y + off, W_out + u * dd, M_out + u * dd,
                           ws, ws + dd, ws + 2 * dd, ws + 3 * dd);
        }
        free(ws);
    }
    return status;
}

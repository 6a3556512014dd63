/*
 * Oracle for the Gated DeltaNet (GDN) recurrent decode step and its fused conv/gate prologue.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load or call this library. The GPU library shares no code, header,
 * table or helper with it, and neither side includes the other.
 *
 * Plain, slow, obviously correct: fp64 throughout, single-threaded, no blocking or fusion,
 * built with -ffp-contract=off so every product and sum is rounded as written. It reads the
 * exact values the device reads (bf16 and fp32 inputs are widened to fp64 by the caller, which
 * is exact) and never rounds to a narrower type.
 *
 * What is computed, and where it comes from:
 *  - "GDN tuning limits on Kunlun XPU" (buru.work), section 二 (背景): every linear-attention
 *    layer runs input projection -> short causal conv with kernel size 4 -> gating -> the
 *    recurrent update of a 128x128 state per head -> output projection; the recurrent update is
 *    a rank-1 change of the state plus a decay. The page prints no equation. The reading used
 *    here is the gated delta rule
 *        S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t,
 *    with S of shape dv x dk (rows indexed by v, columns by k). It is rank-1 plus decay:
 *    S_t - alpha_t S_{t-1} = beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T.
 *  - The conv/SiLU/L2-norm/gate prologue is the "short conv -> gating" part of the same chain;
 *    its exact forms are readings, listed at each function below.
 *
 * Layouts (row-major, last index fastest), all fp64:
 *    q, k   [B][T][H][dk]        v, o   [B][T][H][dv]
 *    alpha, beta, a_logit, b_logit   [B][T][H]
 *    state  [B][H][dv][dk]
 *    x (mixed q|k|v inputs)  [B][T][C],  C = H*dk + H*dk + H*dv, blocks ordered q, k, v,
 *                                       each block head-major with the head dim fastest
 *    conv_state [B][C][3] (oldest first),   conv_w [C][4],   conv_b [C] (optional)
 *
 * Every entry point returns 0 on success and -1 if a size is non-positive or a pointer is
 * missing; it never aborts.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One token of one head, in place on S (dv rows of dk entries).
 *
 * The matrix product S (I - beta k k^T) is written out elementwise: its (i, j) entry is
 * S_ij - beta (S k)_i k_j, because (S k k^T)_ij = (S k)_i k_j. */
static void gdn_one_token(int32_t dk, int32_t dv, double* S, double* Sk,
                          const double* q, const double* k, const double* v,
                          double alpha, double beta, double scale, double* o)
{
    /* (S k)_i = sum_j S_ij k_j, with the state before this token. */
    for (int32_t i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * k[j];
        Sk[i] = acc;
    }
    /* S_t = alpha * (S (I - beta k k^T)) + beta v k^T */
    for (int32_t i = 0; i < dv; ++i) {
        for (int32_t j = 0; j < dk; ++j) {
            double s_proj = S[(size_t)i * dk + j] - beta * Sk[i] * k[j];
            S[(size_t)i * dk + j] = alpha * s_proj + beta * v[i] * k[j];
        }
    }
    /* o_t = S_t (scale q): the readout uses the updated state. */
    for (int32_t i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (scale * q[j]);
        o[i] = acc;
    }
}

/* T sequential tokens for every (sequence, head). `state` is updated in place; `o` receives
 * one readout per token. alpha and beta are one scalar per (sequence, token, head). */
int oracle_gdn_decode(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                      const double* q, const double* k, const double* v,
                      const double* alpha, const double* beta,
                      double* state, double* o, double scale)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !alpha || !beta || !state || !o) return -1;
    double* Sk = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!Sk) return -1;
    for (int64_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < H; ++h) {
            double* S = state + ((size_t)b * H + h) * (size_t)dv * dk;
            for (int32_t t = 0; t < T; ++t) {
                size_t g = ((size_t)b * T + t) * H + h; /* (b, t, h) */
                gdn_one_token(dk, dv, S, Sk, q + g * dk, k + g * dk, v + g * dv,
                              alpha[g], beta[g], scale, o + g * dv);
            }
        }
    }
    free(Sk);
    return 0;
}

/* Logistic function sigma(x) = 1 / (1 + e^{-x}). */
static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^{-|x|}) (the same value,
 * without overflow for large x). */
static double softplus(double x)
{
    double m = x > 0.0 ? x : 0.0;
    return m + log1p(exp(-fabs(x)));
}

/* The fused prologue for T tokens of every (sequence, head):
 *
 *  1. Causal depthwise conv1d, kernel size 4, per channel c. The window for token t is the
 *     sequence u = (cs[c][0], cs[c][1], cs[c][2], x_0[c], x_1[c], ...) and
 *         y_t[c] = sum_{i=0..3} w[c][i] * u[t + i]  (+ bias[c]),
 *     so tap 3 multiplies the current input and tap 0 the input three tokens back.
 *     After the call the conv state holds the last three raw inputs, oldest first.
 *  2. SiLU on every channel: y <- y * sigma(y).
 *  3. Split the channels into q, k, v; L2-normalise q and k per head:
 *         q_hat = q / sqrt(sum_j q_j^2 + l2_eps), likewise k.
 *  4. Gates per (sequence, token, head): beta = sigma(b_logit), alpha = exp(-softplus(a_logit)).
 *
 * The outputs q, k, v, alpha, beta are the inputs of oracle_gdn_decode. */
int oracle_conv_gate(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                     const double* x, double* conv_state,
                     const double* conv_w, const double* conv_b,
                     const double* a_logit, const double* b_logit, double l2_eps,
                     double* q, double* k, double* v, double* alpha, double* beta)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!x || !conv_state || !conv_w || !a_logit || !b_logit) return -1;
    if (!q || !k || !v || !alpha || !beta) return -1;
    const size_t C = (size_t)H * dk * 2 + (size_t)H * dv;
    /* u holds, per channel, the three cached inputs followed by the T new inputs. */
    double* u = (double*)malloc(sizeof(double) * (size_t)(3 + T));
    double* y = (double*)malloc(sizeof(double) * C * (size_t)T); /* [T][C] */
    if (!u || !y) { free(u); free(y); return -1; }

    for (int64_t b = 0; b < B; ++b) {
        /* Steps 1-2: conv + SiLU per channel, and the new conv state. */
        for (size_t c = 0; c < C; ++c) {
            double* cs = conv_state + ((size_t)b * C + c) * 3;
            u[0] = cs[0]; u[1] = cs[1]; u[2] = cs[2];
            for (int32_t t = 0; t < T; ++t) u[3 + t] = x[((size_t)b * T + t) * C + c];
            const double* w = conv_w + c * 4;
            for (int32_t t = 0; t < T; ++t) {
                double acc = 0.0;
                for (int32_t i = 0; i < 4; ++i) acc += w[i] * u[t + i];
                if (conv_b) acc += conv_b[c];
                y[(size_t)t * C + c] = acc * logistic(acc);
            }
            cs[0] = u[T]; cs[1] = u[T + 1]; cs[2] = u[T + 2];
        }
        /* Steps 3-4 per token and head. */
        for (int32_t t = 0; t < T; ++t) {
            const double* yt = y + (size_t)t * C;
            for (int32_t h = 0; h < H; ++h) {
                size_t g = ((size_t)b * T + t) * H + h;
                const double* yq = yt + (size_t)h * dk;
                const double* yk = yt + (size_t)H * dk + (size_t)h * dk;
                const double* yv = yt + (size_t)H * dk * 2 + (size_t)h * dv;
                double sq = 0.0, sk = 0.0;
                for (int32_t j = 0; j < dk; ++j) { sq += yq[j] * yq[j]; sk += yk[j] * yk[j]; }
                double nq = sqrt(sq + l2_eps), nk = sqrt(sk + l2_eps);
                for (int32_t j = 0; j < dk; ++j) {
                    q[g * dk + j] = yq[j] / nq;
                    k[g * dk + j] = yk[j] / nk;
                }
                for (int32_t i = 0; i < dv; ++i) v[g * dv + i] = yv[i];
                beta[g] = logistic(b_logit[g]);
                alpha[g] = exp(-softplus(a_logit[g]));
            }
        }
    }
    free(u);
    free(y);
    return 0;
}

/* The whole fused layer step: oracle_conv_gate, then oracle_gdn_decode on its outputs. */
int oracle_gdn_conv_gate_decode(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                const double* x, double* conv_state,
                                const double* conv_w, const double* conv_b,
                                const double* a_logit, const double* b_logit,
                                double* state, double* o, double scale, double l2_eps)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    size_t n = (size_t)B * T * H;
    double* q = (double*)malloc(sizeof(double) * n * dk);
    double* k = (double*)malloc(sizeof(double) * n * dk);
    double* v = (double*)malloc(sizeof(double) * n * dv);
    double* al = (double*)malloc(sizeof(double) * n);
    double* be = (double*)malloc(sizeof(double) * n);
    int rc = -1;
    if (q && k && v && al && be) {
        rc = oracle_conv_gate(B, T, H, dk, dv, x, conv_state, conv_w, conv_b, a_logit, b_logit,
                              l2_eps, q, k, v, al, be);
        if (rc == 0) rc = oracle_gdn_decode(B, T, H, dk, dv, q, k, v, al, be, state, o, scale);
    }
    free(q); free(k); free(v); free(al); free(be);
    return rc;
}

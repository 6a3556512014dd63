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
 *  - The sliding-window low-rank state (same page, section 三.3) keeps only the last r rank-1
 *    writes of the same rule; its reading is stated at oracle_gdn_lowrank_decode.
 *
 * Layouts (row-major, last index fastest), all fp64:
 *    q, k   [B][T][H][dk]        v, o   [B][T][H][dv]
 *    alpha, beta, a_logit, b_logit   [B][T][H]
 *    state  [B][H][dv][dk]
 *    x (mixed q|k|v inputs)  [B][T][C],  C = H*dk + H*dk + H*dv, blocks ordered q, k, v,
 *                                       each block head-major with the head dim fastest
 *    conv_state [B][C][3] (oldest first),   conv_w [C][4],   conv_b [C] (optional)
 *    low-rank window  U [B][H][r][dv], K [B][H][r][dk], c [B][H][r], pos [B][H] (int32)
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

/* The sliding-window low-rank state of "GDN tuning limits on Kunlun XPU", section 三.3 (the
 * low-rank recurrent route, r = 16 or 32). The page states that its U/V state is a cache of the
 * most recent r rank-1 updates, not a low-rank factorisation of the state, and gives no
 * equations. The reading used here: the state a head stands for is the sum of the last r
 * update terms of the gated delta rule, each decayed by every gate since it was written,
 *     S_t = sum over the r most recent tokens i <= t of (alpha_{i+1} ... alpha_t) delta_i k_i^T,
 * where each token's write delta_t = beta_t (v_t - alpha_t S_{t-1} k_t) is the full rule's
 * write against that windowed S_{t-1}; a token older than the window is dropped whole. With a
 * window at least as long as the run and an empty start this is exactly the full recurrence.
 *
 * Storage, per (sequence, head): r slots, slot i holding a write vector U_i (dv values), its key
 * K_i (dk values) and a weight c_i (the decay it has collected since it was written), so that
 * S = sum_i c_i U_i K_i^T; pos is the slot the next token writes (the oldest one once the window
 * is full), taken modulo r as an unsigned 32-bit value. An all-zero state is the empty window.
 *
 * Per token, written out plainly (S is formed as an explicit dv x dk matrix every time):
 *   1. S = sum_i c_i U_i K_i^T                       (the state before the token)
 *   2. delta = beta (v - alpha S k)
 *   3. every weight is multiplied by alpha           (the decay reaches every stored update)
 *   4. slot pos becomes (delta, k, 1); pos <- (pos + 1) mod r   (the oldest update leaves)
 *   5. S = sum_i c_i U_i K_i^T again; o = S (scale q)  (the readout uses the updated state)
 *
 * Layouts: U [B][H][r][dv], K [B][H][r][dk], c [B][H][r] (fp64), pos [B][H] (int32); q, k, v, o,
 * alpha, beta as in oracle_gdn_decode. U, K, c and pos are updated in place. */
static void lowrank_form_state(int32_t r, int32_t dk, int32_t dv, const double* U,
                               const double* K, const double* c, double* S)
{
    for (int32_t i = 0; i < dv; ++i)
        for (int32_t j = 0; j < dk; ++j) S[(size_t)i * dk + j] = 0.0;
    for (int32_t s = 0; s < r; ++s)
        for (int32_t i = 0; i < dv; ++i)
            for (int32_t j = 0; j < dk; ++j)
                S[(size_t)i * dk + j] += c[s] * U[(size_t)s * dv + i] * K[(size_t)s * dk + j];
}

int oracle_gdn_lowrank_decode(int64_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t r,
                              const double* q, const double* k, const double* v,
                              const double* alpha, const double* beta,
                              double* U, double* K, double* c, int32_t* pos,
                              double* o, double scale)
{
    if (B <= 0 || T <= 0 || H <= 0 || dk <= 0 || dv <= 0 || r <= 0) return -1;
    if (!q || !k || !v || !alpha || !beta || !U || !K || !c || !pos || !o) return -1;
    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
    double* delta = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !delta) { free(S); free(delta); return -1; }
    for (int64_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < H; ++h) {
            size_t head = (size_t)b * H + h;
            double* Uh = U + head * (size_t)r * dv;
            double* Kh = K + head * (size_t)r * dk;
            double* ch = c + head * (size_t)r;
            int32_t p = (int32_t)((uint32_t)pos[head] % (uint32_t)r);
            for (int32_t t = 0; t < T; ++t) {
                size_t g = ((size_t)b * T + t) * H + h; /* (b, t, h) */
                const double* kt = k + g * dk;
                const double* qt = q + g * dk;
                const double* vt = v + g * dv;
                /* 1-2: the write against the state before the token */
                lowrank_form_state(r, dk, dv, Uh, Kh, ch, S);
                for (int32_t i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * kt[j];
                    delta[i] = beta[g] * (vt[i] - alpha[g] * acc);
                }
                /* 3: decay every stored update */
                for (int32_t s = 0; s < r; ++s) ch[s] = alpha[g] * ch[s];
                /* 4: the oldest slot takes the new update */
                for (int32_t i = 0; i < dv; ++i) Uh[(size_t)p * dv + i] = delta[i];
                for (int32_t j = 0; j < dk; ++j) Kh[(size_t)p * dk + j] = kt[j];
                ch[p] = 1.0;
                p = (p + 1) % r;
                /* 5: readout with the updated state */
                lowrank_form_state(r, dk, dv, Uh, Kh, ch, S);
                for (int32_t i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (scale * qt[j]);
                    o[g * dv + i] = acc;
                }
            }
            pos[head] = p;
        }
    }
    free(S);
    free(delta);
    return 0;
}

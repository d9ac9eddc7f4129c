/*
 * Exact scaled-dot-product attention forward, fp64, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU path is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it; the product library never links or calls it, and
 * it shares no code, header or constant with the GPU kernels.
 *
 * What it computes (the plain definition: no tiling, no recurrence):
 *
 *   For every batch b, query head h and query row i:
 *     kvh      = floor(h / (Hq / Hkv))                     GQA head mapping
 *                ("MiniPaged-Qwen: Qwen3 prefill FlashAttention", section 6:
 *                query head qh reads kv head floor(qh / group_size))
 *     s_ij     = scale * sum_c q[b,i,h,c] * k[b,j,kvh,c]   scores (same page,
 *                section 1: S = QK^T / sqrt(d) + M, with the scale passed in)
 *     visible  = { j < Sk : !causal or j <= i + (Sk - Sq) } bottom-right
 *                aligned causal mask (same page, section 13: query qi may see
 *                kv_len - q_len + qi + 1 keys)
 *     m_i      = max over visible j of s_ij
 *     p_ij     = exp(s_ij - m_i) / sum_{visible j'} exp(s_ij' - m_i)
 *                safe softmax ("FlashAttention personal implementation notes",
 *                section "Online Softmax", first formula)
 *     o[b,i,h,:] = sum_j p_ij * v[b,j,kvh,:]
 *     lse[b,h,i] = m_i + ln sum_{visible j} exp(s_ij - m_i)
 *
 *   Key range: oracle_attn_fwd_range restricts the visible set to keys j in
 *   [k_begin, k_end) (the causal rule still counts j against the full Sk).
 *   Its outputs are the partial state of the row over that key subset: the
 *   normalised output and the log-sum-exp of those keys alone.  These are the
 *   per-tile states (m, l, O~) of the online softmax ("FlashAttention
 *   personal implementation notes", section "Online Softmax": the state
 *   after the tiles of a subset, written as O = O~ / l and lse = m + ln l),
 *   which a merge combines.  oracle_attn_fwd is the range [0, Sk).
 *
 *   A row with no visible key (causal and i < Sq - Sk, or an empty key
 *   range) gets o = 0 and lse = -inf.  The pages do not define that case; this follows the CuTe DSL
 *   Ampere FlashAttention-2 example, whose normalisation leaves a zero
 *   accumulator unscaled when the row sum is zero.
 *
 * Layouts: q, o are (B, Sq, Hq, d); k, v are (B, Sk, Hkv, d), dense with d
 * contiguous (the (batch, seq, heads, d_head) layout of the personal-notes
 * page, opening section).  lse is (B, Hq, Sq).  Inputs arrive widened to fp64
 * (widening fp16/bf16 to fp64 is exact).
 *
 * Threads: rows are dealt to nthreads POSIX threads in a strided order
 * (thread t takes rows t, t+n, t+2n, ...), which spreads long and short causal
 * rows evenly.  Each row is computed on its own in a fixed order, so results do
 * not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    int64_t B, Sq, Sk, Hq, Hkv, d;
    double scale;
    int causal;
    int64_t k_begin, k_end; /* key range [k_begin, k_end) */
    const int64_t *rows; /* flat row ids (b*Hq + h)*Sq + i, or NULL = all rows */
    int64_t total;       /* number of rows to compute */
    int64_t first, stride;
} job_t;

/* One query row straight from the definition.  s and p are scratch rows of
 * Sk doubles each: the score row S and the probability row P. */
static void one_row(const job_t *J, int64_t b, int64_t h, int64_t i,
                    double *out_o, double *out_lse, double *s, double *p) {
    const int64_t d = J->d;
    const int64_t kvh = h / (J->Hq / J->Hkv);
    const double *qrow = J->q + ((b * J->Sq + i) * J->Hq + h) * d;

    /* the visible keys are j in [j0, nvis) */
    const int64_t j0 = J->k_begin;
    int64_t nvis = J->k_end;
    if (J->causal) {
        int64_t lim = i + (J->Sk - J->Sq) + 1;
        if (lim < 0) lim = 0;
        if (lim < nvis) nvis = lim;
    }
    if (nvis <= j0) {
        for (int64_t c = 0; c < d; ++c) out_o[c] = 0.0;
        *out_lse = -INFINITY;
        return;
    }

    /* first pass: scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = j0; j < nvis; ++j) {
        const double *krow = J->k + ((b * J->Sk + j) * J->Hkv + kvh) * d;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += qrow[c] * krow[c];
        s[j] = J->scale * acc;
        if (s[j] > m) m = s[j];
    }
    /* second pass: exp(s - m), the denominator, the probabilities */
    double sum = 0.0;
    for (int64_t j = j0; j < nvis; ++j) {
        p[j] = exp(s[j] - m);
        sum += p[j];
    }
    for (int64_t j = j0; j < nvis; ++j) p[j] /= sum;

    /* o = P V */
    for (int64_t c = 0; c < d; ++c) out_o[c] = 0.0;
    for (int64_t j = j0; j < nvis; ++j) {
        const double *vrow = J->v + ((b * J->Sk + j) * J->Hkv + kvh) * d;
        const double pj = p[j];
        for (int64_t c = 0; c < d; ++c) out_o[c] += pj * vrow[c];
    }
    *out_lse = m + log(sum);
}

static void *worker(void *arg) {
    const job_t *J = (const job_t *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)J->Sk);
    double *p = (double *)malloc(sizeof(double) * (size_t)J->Sk);
    if (!s || !p) {
        free(s);
        free(p);
        return (void *)1;
    }
    for (int64_t r = J->first; r < J->total; r += J->stride) {
        const int64_t flat = J->rows ? J->rows[r] : r;
        const int64_t i = flat % J->Sq;
        const int64_t h = (flat / J->Sq) % J->Hq;
        const int64_t b = flat / (J->Sq * J->Hq);
        double *o_dst, *lse_dst;
        if (J->rows) { /* compact output: request order */
            o_dst = J->o + r * J->d;
            lse_dst = J->lse + r;
        } else {       /* full (B,Sq,Hq,d) and (B,Hq,Sq) outputs */
            o_dst = J->o + ((b * J->Sq + i) * J->Hq + h) * J->d;
            lse_dst = J->lse + (b * J->Hq + h) * J->Sq + i;
        }
        one_row(J, b, h, i, o_dst, lse_dst, s, p);
    }
    free(s);
    free(p);
    return NULL;
}

/*
 * rows == NULL: compute every row; o is (B,Sq,Hq,d), lse is (B,Hq,Sq).
 * rows != NULL: compute only the nrows flat row ids (b*Hq + h)*Sq + i; o is
 *               (nrows, d) and lse is (nrows), in request order.
 * Keys are restricted to [k_begin, k_end), 0 <= k_begin <= k_end <= Sk.
 * Returns 0 on success, 1 on bad arguments, 2 if a thread could not start or
 * allocate its scratch rows.
 */
int oracle_attn_fwd_range(const double *q, const double *k, const double *v,
                          double *o, double *lse,
                          int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                          int64_t d, double scale, int causal,
                          int64_t k_begin, int64_t k_end,
                          const int64_t *rows, int64_t nrows, int nthreads) {
    if (!q || !k || !v || !o || !lse) return 1;
    if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || d < 1) return 1;
    if (k_begin < 0 || k_begin > k_end || k_end > Sk) return 1;
    if (Hq % Hkv != 0) return 1;
    if (causal != 0 && causal != 1) return 1;
    if (rows && nrows < 0) return 1;
    const int64_t total = rows ? nrows : B * Hq * Sq;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= B * Hq * Sq) return 1;
    if (total == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > total) nthreads = (int)total;

    job_t jobs[256];
    pthread_t tid[256];
    int started[256];
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        job_t *J = &jobs[t];
        J->q = q; J->k = k; J->v = v; J->o = o; J->lse = lse;
        J->B = B; J->Sq = Sq; J->Sk = Sk; J->Hq = Hq; J->Hkv = Hkv; J->d = d;
        J->scale = scale; J->causal = causal;
        J->k_begin = k_begin; J->k_end = k_end;
        J->rows = rows; J->total = total;
        J->first = t; J->stride = nthreads;
        started[t] = pthread_create(&tid[t], NULL, worker, J) == 0;
        if (!started[t]) rc = 2;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (!started[t]) continue;
        void *ret = NULL;
        pthread_join(tid[t], &ret);
        if (ret) rc = 2;
    }
    return rc;
}

/* Every key: the plain definition of the forward pass. */
int oracle_attn_fwd(const double *q, const double *k, const double *v,
                    double *o, double *lse,
                    int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                    int64_t d, double scale, int causal,
                    const int64_t *rows, int64_t nrows, int nthreads) {
    return oracle_attn_fwd_range(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, scale,
                                 causal, 0, Sk, rows, nrows, nthreads);
}

/*
 * Backward pass: the gradients of L = sum(dO * O) with respect to q, k and
 * v, from the plain definition, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY (see the top of this file).
 *
 * The pages return the LSE for training (the CuTe DSL example's docstring)
 * and name FlashAttention 1 and 2 as the algorithms; they print no backward
 * formula, so this is the chain rule through the forward definition above:
 *
 *   p_ij   = softmax_j(s_ij) over the visible keys   (forward definition)
 *   dv_j  += sum_i p_ij * do_i                       (O = P V)
 *   dp_ij  = do_i . v_j
 *   ds_ij  = p_ij * (dp_ij - sum_j' p_ij' dp_ij')    (Jacobian of softmax:
 *            d p_ij / d s_ij' = p_ij (delta_jj' - p_ij'))
 *   dq_i   = scale * sum_j ds_ij k_j                 (s = scale * q . k)
 *   dk_j  += scale * sum_i ds_ij q_i
 *
 * GQA: dk and dv of kv head kvh sum the contributions of every query head
 * that reads it.  Rows with no visible key contribute nothing and get dq = 0.
 * P is materialised per row (two passes, as in the forward); nothing is
 * tiled.  Work is dealt per (batch, kv head) so that each thread owns its
 * dk and dv rows; results do not depend on the thread count.
 */
typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    int64_t B, Sq, Sk, Hq, Hkv, d;
    double scale;
    int causal;
    int64_t first, stride; /* (b, kvh) pairs first, first + stride, ... */
} bjob_t;

static void *bwd_worker(void *arg) {
    const bjob_t *J = (const bjob_t *)arg;
    const int64_t d = J->d, g = J->Hq / J->Hkv;
    double *s = (double *)malloc(sizeof(double) * (size_t)J->Sk);
    double *p = (double *)malloc(sizeof(double) * (size_t)J->Sk);
    double *dp = (double *)malloc(sizeof(double) * (size_t)J->Sk);
    if (!s || !p || !dp) {
        free(s); free(p); free(dp);
        return (void *)1;
    }
    for (int64_t pair = J->first; pair < J->B * J->Hkv; pair += J->stride) {
        const int64_t b = pair / J->Hkv, kvh = pair % J->Hkv;
        for (int64_t j = 0; j < J->Sk; ++j)
            for (int64_t c = 0; c < d; ++c) {
                J->dk[((b * J->Sk + j) * J->Hkv + kvh) * d + c] = 0.0;
                J->dv[((b * J->Sk + j) * J->Hkv + kvh) * d + c] = 0.0;
            }
        for (int64_t h = kvh * g; h < (kvh + 1) * g; ++h) {
            for (int64_t i = 0; i < J->Sq; ++i) {
                const double *qrow = J->q + ((b * J->Sq + i) * J->Hq + h) * d;
                const double *dorow = J->dout + ((b * J->Sq + i) * J->Hq + h) * d;
                double *dqrow = J->dq + ((b * J->Sq + i) * J->Hq + h) * d;
                for (int64_t c = 0; c < d; ++c) dqrow[c] = 0.0;
                int64_t nvis = J->Sk;
                if (J->causal) {
                    int64_t lim = i + (J->Sk - J->Sq) + 1;
                    if (lim < 0) lim = 0;
                    if (lim < nvis) nvis = lim;
                }
                if (nvis == 0) continue;
                /* forward: scores, max, probabilities */
                double m = -INFINITY;
                for (int64_t j = 0; j < nvis; ++j) {
                    const double *krow = J->k + ((b * J->Sk + j) * J->Hkv + kvh) * d;
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc += qrow[c] * krow[c];
                    s[j] = J->scale * acc;
                    if (s[j] > m) m = s[j];
                }
                double sum = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    p[j] = exp(s[j] - m);
                    sum += p[j];
                }
                for (int64_t j = 0; j < nvis; ++j) p[j] /= sum;
                /* dp and the softmax Jacobian-vector product */
                double pdp = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    const double *vrow = J->v + ((b * J->Sk + j) * J->Hkv + kvh) * d;
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c) acc += dorow[c] * vrow[c];
                    dp[j] = acc;
                    pdp += p[j] * acc;
                }
                for (int64_t j = 0; j < nvis; ++j) {
                    const double ds = p[j] * (dp[j] - pdp);
                    const double *krow = J->k + ((b * J->Sk + j) * J->Hkv + kvh) * d;
                    double *dkrow = J->dk + ((b * J->Sk + j) * J->Hkv + kvh) * d;
                    double *dvrow = J->dv + ((b * J->Sk + j) * J->Hkv + kvh) * d;
                    for (int64_t c = 0; c < d; ++c) {
                        dqrow[c] += J->scale * ds * krow[c];
                        dkrow[c] += J->scale * ds * qrow[c];
                        dvrow[c] += p[j] * dorow[c];
                    }
                }
            }
        }
    }
    free(s); free(p); free(dp);
    return NULL;
}

/*
 * q, dout, dq: (B, Sq, Hq, d); k, v, dk, dv: (B, Sk, Hkv, d), all fp64.
 * Returns 0 on success, 1 on bad arguments, 2 if a thread failed.
 */
int oracle_attn_bwd(const double *q, const double *k, const double *v,
                    const double *dout, double *dq, double *dk, double *dv,
                    int64_t B, int64_t Sq, int64_t Sk, int64_t Hq, int64_t Hkv,
                    int64_t d, double scale, int causal, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
    if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || d < 1) return 1;
    if (Hq % Hkv != 0) return 1;
    if (causal != 0 && causal != 1) return 1;
    const int64_t pairs = B * Hkv;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > pairs) nthreads = (int)pairs;
    bjob_t jobs[256];
    pthread_t tid[256];
    int started[256];
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        bjob_t *J = &jobs[t];
        J->q = q; J->k = k; J->v = v; J->dout = dout;
        J->dq = dq; J->dk = dk; J->dv = dv;
        J->B = B; J->Sq = Sq; J->Sk = Sk; J->Hq = Hq; J->Hkv = Hkv; J->d = d;
        J->scale = scale; J->causal = causal;
        J->first = t; J->stride = nthreads;
        started[t] = pthread_create(&tid[t], NULL, bwd_worker, J) == 0;
        if (!started[t]) rc = 2;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (!started[t]) continue;
        void *ret = NULL;
        pthread_join(tid[t], &ret);
        if (ret) rc = 2;
    }
    return rc;
}

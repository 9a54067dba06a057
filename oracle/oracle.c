/*
 * Plain fp64 CPU oracle for row-wise softmax, its online (m, d) state and
 * the state merge.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * with the HIP library: it has its own dtype codes and its own bf16 widening.
 *
 * Everything here is deliberately slow and literal: one row at a time, one
 * element at a time, fp64 accumulation, libm exp/log, true division, no
 * blocking, no reordering beyond what each cited definition states.  Build
 * with -ffp-contract=off so that every expression rounds as written.
 *
 * Sources (the pages this implements):
 *  [P1] "5.2 CUDA Online Softmax 实现优化" (AIInfraGuide): §1.1 three-pass
 *       safe softmax; §2.1 the running-state recurrence and its derivation;
 *       §2.2 the two-pass pseudo-code; §2.3 stability; §4.1 the merge of two
 *       partial states.
 *  [P3] "从原始Softmax到在线Softmax": section on deriving the stable form, which
 *       defines log-sum-exp LSE = m + log sum e^(z-m).
 *  [P4] "Softmax 数值稳定性与 IO-Aware Attention：从在线归一化到 FlashAttention":
 *       §3 (three passes), §4 (running state), §4.1 (merge of two states,
 *       associativity, the random-chunking check).
 *       Also the log-softmax log p_j = z_j - LSE(z), and the cross-entropy of
 *       a labelled row, -log p_label, with its batch mean (section on the
 *       cross-entropy loss and the hand-worked loss example).
 *  [P5] "FlashAttention：为什么加速推理的同时还能节省显存": the 3-pass
 *       safe_softmax and the 2-pass online_safe_softmax listings (used as a
 *       description of what is computed, not copied); the attention
 *       o = softmax(q K^T / sqrt(d)) V per query and its tiled online form.
 *  [P1] §8.2 and [P3] FlashAttention section: attention with the running
 *       (m, l, o~) state per query, o~ rescaled by e^(m_old - m_new) when a
 *       key block raises the max; [P4] §7 the same loop per query tile.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - An element equal to -inf has weight e^(-inf) = 0; it changes neither
 *    the max of a row that has a larger element nor the sum.  A row whose
 *    elements are all -inf therefore has m = -inf, d = 0, LSE = -inf and
 *    y = 0/0 = NaN.  The state (-inf, 0) is the identity of the merge: the
 *    merge formula would produce 0 * e^(NaN) for two such states, so the
 *    merge returns the identity directly when both maxima are -inf.
 *  - The max ignores NaN (a NaN never compares greater); a NaN element makes
 *    its term e^(NaN - m) = NaN, so d, y and LSE of that row are NaN.
 *  - A +inf element makes m = +inf and its term e^(inf - inf) = NaN, so the
 *    row is NaN (as for a NaN element).
 *
 * Parity pins for every function are in the test suite; none is unpinned.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ---- ingest: read one stored element exactly ------------------------------
 * fp32 -> fp64 is exact.  A bf16 value is the upper 16 bits of the fp32 with
 * the same sign and exponent, so widening is a 16-bit left shift (exact). */
static double load_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32) {
        return (double)((const float *)x)[idx];
    } else {
        uint32_t bits = (uint32_t)((const uint16_t *)x)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

static int check_args(const void *x, int64_t ld, int64_t M, int64_t N, int dtype)
{
    if (M < 0 || N < 1) return ORACLE_EINVAL;
    if (ld < N) return ORACLE_EINVAL;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_EINVAL;
    if (M > 0 && x == NULL) return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* ---- the row's max and normaliser -------------------------------------------
 * [P1] §1.1 and [P4] §3, passes 1 and 2 over the first n elements of the
 * row at base: m = max_j x_j (NaN never compares greater, so it is
 * skipped), d = sum_j e^(x_j - m) (a -inf element has weight 0).
 * log d ([P3] stable-form section: LSE = m + log d) is evaluated as
 * log1p(s), s the sum of the terms other than one instance of the max: that
 * instance's term is exactly e^0 = 1, so d = 1 + s, and s summed apart from
 * the 1 keeps fp64 relative precision when d lies within rounding of 1 (a
 * row whose max dominates), where log of a rounded d would lose it.  A row
 * with no finite max has s = d - 1 taken as is (m = -inf: d = 0, log d =
 * -inf; m = +inf: its term is NaN). */
static void row_stats(const void *x, int dtype, int64_t base, int64_t n,
                      double *m_out, double *d_out, double *logd_out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double v = load_elem(x, dtype, base + j);
        if (v > m) m = v;
    }
    double d = 0.0, s = 0.0;
    int found = !isfinite(m);  /* no instance to leave out */
    for (int64_t j = 0; j < n; ++j) {
        double v = load_elem(x, dtype, base + j);
        double t = (v == -INFINITY) ? 0.0 : exp(v - m);
        d = d + t;
        if (!found && v == m) {
            found = 1;          /* the max's own 1, left out of s */
            continue;
        }
        s = s + t;
    }
    *m_out = m;
    *d_out = d;
    *logd_out = isfinite(m) ? log1p(s) : log(d);
}

/* ---- the definition: three-pass safe softmax ------------------------------
 * [P1] §1.1 and [P4] §3: m = max_j x_j, d = sum_j e^(x_j - m),
 * y_j = e^(x_j - m) / d.  [P3] stable-form section: LSE = m + log d.
 * Each pass is a separate loop over the row, in index order. */
int oracle_softmax(const void *x, int64_t ld, int64_t M, int64_t N, int dtype,
                   double *y, double *m_out, double *d_out, double *lse_out)
{
    int rc = check_args(x, ld, M, N, dtype);
    if (rc != ORACLE_OK) return rc;
    for (int64_t i = 0; i < M; ++i) {
        const int64_t base = i * ld;

        /* passes 1 and 2: the row max and the sum of e^(x - m) */
        double m, d, logd;
        row_stats(x, dtype, base, N, &m, &d, &logd);

        /* pass 3: normalise with a true division */
        if (y != NULL) {
            for (int64_t j = 0; j < N; ++j) {
                double v = load_elem(x, dtype, base + j);
                double t = (v == -INFINITY) ? 0.0 : exp(v - m);
                y[i * N + j] = t / d;
            }
        }
        if (m_out) m_out[i] = m;
        if (d_out) d_out[i] = d;
        if (lse_out) lse_out[i] = m + logd;
    }
    return ORACLE_OK;
}

/* ---- the merge of two partial states --------------------------------------
 * [P1] §4.1 and [P4] §4.1: m = max(m_a, m_b),
 * d = d_a e^(m_a - m) + d_b e^(m_b - m).  (-inf, 0) is the identity. */
void oracle_merge2(double ma, double da, double mb, double db,
                   double *m_out, double *d_out)
{
    double m = (mb > ma) ? mb : ma;
    if (m == -INFINITY) {
        /* both operands have max -inf: the sum of their weights is da + db
         * (0 for identities, NaN if a NaN was folded in) */
        *m_out = -INFINITY;
        *d_out = da + db;
        return;
    }
    *m_out = m;
    *d_out = da * exp(ma - m) + db * exp(mb - m);
}

/* ---- the method's running state: one element at a time ---------------------
 * [P1] §2.1/§2.2, [P4] §4, [P5] 2-pass listing: start from (-inf, 0); for
 * each element x: m' = max(m, x), d = d e^(m - m') + e^(x - m'), m = m'.
 * When the max does not change the correction factor is e^0 = 1 exactly
 * ([P1] §2.1 remark), which also keeps (-inf, 0) intact.  A -inf element
 * has zero weight and leaves the state unchanged. */
int oracle_state(const void *x, int64_t ld, int64_t M, int64_t N, int dtype,
                 double *m_out, double *d_out)
{
    int rc = check_args(x, ld, M, N, dtype);
    if (rc != ORACLE_OK) return rc;
    for (int64_t i = 0; i < M; ++i) {
        double m = -INFINITY, d = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double v = load_elem(x, dtype, i * ld + j);
            if (v == -INFINITY) continue;
            double m_new = (v > m) ? v : m;
            double corr = (m_new == m) ? 1.0 : exp(m - m_new);
            d = d * corr + exp(v - m_new);
            m = m_new;
        }
        if (m_out) m_out[i] = m;
        if (d_out) d_out[i] = d;
    }
    return ORACLE_OK;
}

/* ---- the merge of K states per row (left fold of oracle_merge2) -----------
 * Row i holds K states at m_in[i*ld + k], d_in[i*ld + k].  The fold starts
 * from the identity and merges k = 0, 1, ..., K-1 in order ([P4] §4.1:
 * merge repeatedly; the result does not depend on the grouping in exact
 * arithmetic).  LSE = m + log d as in [P3]. */
int oracle_merge(const double *m_in, const double *d_in, int64_t ld,
                 int64_t M, int64_t K, double *m_out, double *d_out,
                 double *lse_out)
{
    if (M < 0 || K < 1 || ld < K) return ORACLE_EINVAL;
    if (M > 0 && (m_in == NULL || d_in == NULL)) return ORACLE_EINVAL;
    for (int64_t i = 0; i < M; ++i) {
        double m = -INFINITY, d = 0.0;
        for (int64_t k = 0; k < K; ++k)
            oracle_merge2(m, d, m_in[i * ld + k], d_in[i * ld + k], &m, &d);
        if (m_out) m_out[i] = m;
        if (d_out) d_out[i] = d;
        if (lse_out) lse_out[i] = m + log(d);
    }
    return ORACLE_OK;
}

/* ---- log-softmax -----------------------------------------------------------
 * [P3] stable-form section: log p_j = z_j - LSE(z), LSE = m + log d, with m
 * and d from the definition above; written (z_j - m) - log d, the same
 * value with the common m subtracted first, so that a log-probability near
 * 0 is not the difference of two large numbers.  y is dense fp64 [M][N].
 * A row of only -inf gives -inf - (-inf) = NaN, as y = 0/0 does. */
int oracle_log_softmax(const void *x, int64_t ld, int64_t M, int64_t N,
                       int dtype, double *y)
{
    int rc = check_args(x, ld, M, N, dtype);
    if (rc != ORACLE_OK) return rc;
    if (M > 0 && y == NULL) return ORACLE_EINVAL;
    for (int64_t i = 0; i < M; ++i) {
        double m, d, logd;
        row_stats(x, dtype, i * ld, N, &m, &d, &logd);
        for (int64_t j = 0; j < N; ++j)
            y[i * N + j] = (load_elem(x, dtype, i * ld + j) - m) - logd;
    }
    return ORACLE_OK;
}

/* ---- pass 2 with a given state -----------------------------------------------
 * [P1] §2.2: the second pass writes y_j = e^(x_j - m) / d from the state
 * (m, d) the first pass left; [P3] stable-form section: its log form is
 * log p_j = (x_j - m) - log d.  Here the state is an input, (m_in[i*inc],
 * d_in[i*inc]) for row i, taken as given (fp64; an fp32 state widens
 * exactly): the exact value of the pass for that state, whatever rounding
 * the state carries.  log_form != 0 writes the log form.  y is dense fp64
 * [M][N].  The identity state (-inf, 0) gives NaN (0/0, -inf + inf). */
int oracle_normalize(const void *x, int64_t ld, int64_t M, int64_t N,
                     int dtype, const double *m_in, const double *d_in,
                     int64_t inc, int log_form, double *y)
{
    int rc = check_args(x, ld, M, N, dtype);
    if (rc != ORACLE_OK) return rc;
    if (M > 0 && (y == NULL || m_in == NULL || d_in == NULL)) return ORACLE_EINVAL;
    if (inc < 1) return ORACLE_EINVAL;
    for (int64_t i = 0; i < M; ++i) {
        const double m = m_in[i * inc];
        const double d = d_in[i * inc];
        for (int64_t j = 0; j < N; ++j) {
            const double v = load_elem(x, dtype, i * ld + j);
            y[i * N + j] = log_form ? (v - m) - log(d) : exp(v - m) / d;
        }
    }
    return ORACLE_OK;
}

/* ---- cross-entropy -----------------------------------------------------------
 * [P3] cross-entropy section: the loss of a row whose true class is c is
 * -log p_c = LSE(z) - z_c; the batch loss is the mean over rows.  Reading
 * for labels outside the row (the page has none): a negative label marks a
 * row to ignore (loss 0, left out of the mean), a label >= N gives NaN.
 * mean (nullable) is the mean over non-ignored rows, NaN when there are
 * none. */
int oracle_cross_entropy(const void *x, int64_t ld, int64_t M, int64_t N,
                         int dtype, const int64_t *labels, double *loss,
                         double *mean)
{
    int rc = check_args(x, ld, M, N, dtype);
    if (rc != ORACLE_OK) return rc;
    if (M > 0 && (labels == NULL || loss == NULL)) return ORACLE_EINVAL;
    double total = 0.0;
    int64_t count = 0;
    for (int64_t i = 0; i < M; ++i) {
        const int64_t c = labels[i];
        if (c < 0) {
            loss[i] = 0.0;
            continue;
        }
        if (c >= N) {
            loss[i] = NAN;
        } else {
            /* LSE - z_c = (m - z_c) + log d */
            double m, d, logd;
            row_stats(x, dtype, i * ld, N, &m, &d, &logd);
            loss[i] = (m - load_elem(x, dtype, i * ld + c)) + logd;
        }
        total = total + loss[i];
        count = count + 1;
    }
    if (mean) *mean = (count > 0) ? total / (double)count : NAN;
    return ORACLE_OK;
}

/* ---- masked rows ----------------------------------------------------------
 * Row i takes part in its softmax only through its first n_i columns:
 *   n_i = N, lowered to row_len[i] (clipped to [0, N]) when row_len is
 *   given, and to i + causal + 1 when causal >= 0 (a causal mask: row i sees
 *   columns 0..i+causal).
 * The other columns are masked: they are not read, and count as -inf
 * elements ([P4] §9.2 lists mask boundaries among the inputs to test; the
 * -inf reading above then fixes their output): y = 0 for softmax, -inf for
 * log-softmax.  A row with n_i = 0 has m = -inf, d = 0, lse = -inf and a NaN
 * y, as a row of only -inf.
 * The valid columns follow the definition of oracle_softmax over j < n_i.
 * log_y (nullable): (x - m) - log d on valid columns, as oracle_log_softmax. */
static int64_t valid_cols(int64_t i, int64_t N, const int32_t *row_len,
                          int64_t causal)
{
    int64_t n = N;
    if (row_len) {
        int64_t l = row_len[i];
        if (l < 0) l = 0;
        if (l < n) n = l;
    }
    if (causal >= 0 && i + causal + 1 < n) n = i + causal + 1;
    return n;
}

int oracle_softmax_masked(const void *x, int64_t ld, int64_t M, int64_t N,
                          int dtype, const int32_t *row_len, int64_t causal,
                          double *y, double *log_y, double *m_out,
                          double *d_out, double *lse_out)
{
    int rc = check_args(x, ld, M, N, dtype);
    if (rc != ORACLE_OK) return rc;
    for (int64_t i = 0; i < M; ++i) {
        const int64_t base = i * ld;
        const int64_t n = valid_cols(i, N, row_len, causal);
        double m, d, logd;
        row_stats(x, dtype, base, n, &m, &d, &logd);
        const double lse = m + logd;
        for (int64_t j = 0; j < N; ++j) {
            if (j < n) {
                double v = load_elem(x, dtype, base + j);
                double t = (v == -INFINITY) ? 0.0 : exp(v - m);
                if (y) y[i * N + j] = t / d;
                if (log_y) log_y[i * N + j] = (v - m) - logd;
            } else {
                if (y) y[i * N + j] = (n == 0) ? NAN : 0.0;
                if (log_y) log_y[i * N + j] = (n == 0) ? NAN : -INFINITY;
            }
        }
        if (m_out) m_out[i] = m;
        if (d_out) d_out[i] = d;
        if (lse_out) lse_out[i] = lse;
    }
    return ORACLE_OK;
}

/* ---- attention ------------------------------------------------------------
 * [P1] §8.2, [P3] FlashAttention section and worked attention example,
 * [P4] §7, [P5] attention listings: for query row i of one (batch, head)
 * slice, the scores against the admitted keys are s_j = scale * (q_i . k_j),
 * P = softmax(s) (three-pass safe form), o_i = sum_j P_j v_j, and
 * lse_i = m + log sum_j e^(s_j - m).  The pages use scale = 1/sqrt(d).
 *
 * Readings: key j is admitted for query i when j < Sk and, if causal >= 0,
 * j <= i + causal (a causal offset of Sk - Sq aligns the last query with the
 * last key; 0 is the square self-attention mask).  With causal >= 0 and
 * Sk >= 1 every query admits key 0, so no row is empty.  Non-finite scores
 * follow the softmax readings above (a NaN or +inf score gives a NaN row).
 *
 * rows (nullable): the query rows to evaluate, nrows of them, in that order
 * (all Sq rows when NULL, nrows ignored).  o: fp64 [nrows][D]; lse
 * (nullable): fp64 [nrows].  Q, K, V rows have strides ldq, ldk, ldv. */
static int attn_args(const void *q, int64_t ldq, const void *k, int64_t ldk,
                     const void *v, int64_t ldv, int dtype, int64_t Sq,
                     int64_t Sk, int64_t D, const int64_t *rows,
                     int64_t nrows)
{
    if (Sq < 0 || Sk < 1 || D < 1) return ORACLE_EINVAL;
    if (ldq < D || ldk < D || ldv < D) return ORACLE_EINVAL;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_EINVAL;
    if (!q || !k || !v) return ORACLE_EINVAL;
    if (rows) {
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= Sq) return ORACLE_EINVAL;
    }
    return ORACLE_OK;
}

static int64_t admitted_keys(int64_t i, int64_t Sk, int64_t causal)
{
    if (causal < 0) return Sk;
    const int64_t last = i + causal;            /* the last admitted key */
    return (last + 1 < Sk) ? last + 1 : Sk;
}

/* s_j = scale * sum_c q_ic k_jc, the dot product summed in index order. */
static double attn_score(const void *q, int64_t ldq, const void *k,
                         int64_t ldk, int dtype, int64_t i, int64_t j,
                         int64_t D, double scale)
{
    double dot = 0.0;
    for (int64_t c = 0; c < D; ++c)
        dot = dot + load_elem(q, dtype, i * ldq + c) *
                    load_elem(k, dtype, j * ldk + c);
    return scale * dot;
}

int oracle_attention(const void *q, int64_t ldq, const void *k, int64_t ldk,
                     const void *v, int64_t ldv, int dtype, int64_t Sq,
                     int64_t Sk, int64_t D, double scale, int64_t causal,
                     const int64_t *rows, int64_t nrows, double *o,
                     double *lse)
{
    int rc = attn_args(q, ldq, k, ldk, v, ldv, dtype, Sq, Sk, D, rows, nrows);
    if (rc != ORACLE_OK) return rc;
    if (!rows) nrows = Sq;
    if (nrows > 0 && !o) return ORACLE_EINVAL;
    double *s = (double *)malloc((size_t)Sk * sizeof(double));
    if (!s) return ORACLE_EINVAL;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        const int64_t n = admitted_keys(i, Sk, causal);
        /* pass 1: the scores and their max */
        double m = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            s[j] = attn_score(q, ldq, k, ldk, dtype, i, j, D, scale);
            if (s[j] > m) m = s[j];
        }
        /* pass 2: the normaliser */
        double l = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double t = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
            l = l + t;
        }
        /* pass 3: the probabilities, then the weighted sum of value rows */
        for (int64_t c = 0; c < D; ++c) o[r * D + c] = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double t = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
            double p = t / l;
            for (int64_t c = 0; c < D; ++c)
                o[r * D + c] = o[r * D + c] + p * load_elem(v, dtype, j * ldv + c);
        }
        if (lse) lse[r] = m + log(l);
    }
    free(s);
    return ORACLE_OK;
}

/* The tiled online form of the same attention, per query row ([P3] the
 * recurrence for m, l and the unnormalised output; [P4] §7 loop over K/V
 * tiles): keys are taken in blocks of Bc; a block with maximum m_blk moves
 * the running max to m_new = max(m, m_blk), the old l and o~ are scaled by
 * alpha = e^(m - m_new), the block adds sum e^(s_j - m_new) to l and
 * sum e^(s_j - m_new) v_j to o~, and o = o~ / l at the end.  The pages state
 * this equals the definition up to rounding; the pins check it. */
int oracle_attention_online(const void *q, int64_t ldq, const void *k,
                            int64_t ldk, const void *v, int64_t ldv, int dtype,
                            int64_t Sq, int64_t Sk, int64_t D, double scale,
                            int64_t causal, int64_t Bc, const int64_t *rows,
                            int64_t nrows, double *o, double *lse)
{
    int rc = attn_args(q, ldq, k, ldk, v, ldv, dtype, Sq, Sk, D, rows, nrows);
    if (rc != ORACLE_OK) return rc;
    if (Bc < 1) return ORACLE_EINVAL;
    if (!rows) nrows = Sq;
    if (nrows > 0 && !o) return ORACLE_EINVAL;
    double *s = (double *)malloc((size_t)Bc * sizeof(double));
    double *acc = (double *)malloc((size_t)D * sizeof(double));
    if (!s || !acc) { free(s); free(acc); return ORACLE_EINVAL; }
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        const int64_t n = admitted_keys(i, Sk, causal);
        double m = -INFINITY, l = 0.0;
        for (int64_t c = 0; c < D; ++c) acc[c] = 0.0;
        for (int64_t j0 = 0; j0 < n; j0 += Bc) {
            const int64_t nb = (n - j0 < Bc) ? n - j0 : Bc;
            double m_blk = -INFINITY;
            for (int64_t t = 0; t < nb; ++t) {
                s[t] = attn_score(q, ldq, k, ldk, dtype, i, j0 + t, D, scale);
                if (s[t] > m_blk) m_blk = s[t];
            }
            const double m_new = (m_blk > m) ? m_blk : m;
            if (m_new == -INFINITY) continue;          /* nothing admitted yet */
            const double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
            l = alpha * l;
            for (int64_t c = 0; c < D; ++c) acc[c] = alpha * acc[c];
            for (int64_t t = 0; t < nb; ++t) {
                double e = (s[t] == -INFINITY) ? 0.0 : exp(s[t] - m_new);
                l = l + e;
                for (int64_t c = 0; c < D; ++c)
                    acc[c] = acc[c] + e * load_elem(v, dtype, (j0 + t) * ldv + c);
            }
            m = m_new;
        }
        for (int64_t c = 0; c < D; ++c) o[r * D + c] = acc[c] / l;
        if (lse) lse[r] = m + log(l);
    }
    free(s);
    free(acc);
    return ORACLE_OK;
}

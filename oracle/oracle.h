/*
 * fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY (see oracle.c).
 * Own dtype codes and status codes; nothing here is shared with the library.
 */
#ifndef ROW_SOFTMAX_ORACLE_H
#define ROW_SOFTMAX_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_OK = 0, ORACLE_EINVAL = 1 };

/* Three-pass safe softmax of each of the M rows of x (row stride ld
 * elements, N columns).  y (nullable) is dense fp64 [M][N]; m, d, lse
 * (each nullable) are fp64 [M]. */
int oracle_softmax(const void *x, int64_t ld, int64_t M, int64_t N, int dtype,
                   double *y, double *m, double *d, double *lse);

/* The online recurrence, element by element, per row: (m, d) fp64 [M]. */
int oracle_state(const void *x, int64_t ld, int64_t M, int64_t N, int dtype,
                 double *m, double *d);

/* Merge of two states with the (-inf, 0) identity. */
void oracle_merge2(double ma, double da, double mb, double db,
                   double *m, double *d);

/* Left-fold merge of K states per row (row stride ld). */
int oracle_merge(const double *m_in, const double *d_in, int64_t ld,
                 int64_t M, int64_t K, double *m, double *d, double *lse);

/* log p = z - LSE(z) per row: y fp64 dense [M][N]. */
int oracle_log_softmax(const void *x, int64_t ld, int64_t M, int64_t N,
                       int dtype, double *y);

/* Cross-entropy per row from int64 labels; mean (nullable) over the rows
 * whose label is not negative. */
int oracle_normalize(const void *x, int64_t ld, int64_t M, int64_t N,
                     int dtype, const double *m_in, const double *d_in,
                     int64_t inc, int log_form, double *y);
int oracle_cross_entropy(const void *x, int64_t ld, int64_t M, int64_t N,
                         int dtype, const int64_t *labels, double *loss,
                         double *mean);

/* Softmax (y) and log-softmax (log_y) of each row over its first n_i
 * columns (row_len and/or a causal offset; see oracle.c); all nullable
 * except x. */
int oracle_softmax_masked(const void *x, int64_t ld, int64_t M, int64_t N,
                          int dtype, const int32_t *row_len, int64_t causal,
                          double *y, double *log_y, double *m, double *d,
                          double *lse);

/* Attention of one (batch, head) slice: o = softmax(scale q K^T) V and
 * lse per selected query row (rows nullable = all Sq rows); causal >= 0
 * admits key j for query i when j <= i + causal. */
int oracle_attention(const void *q, int64_t ldq, const void *k, int64_t ldk,
                     const void *v, int64_t ldv, int dtype, int64_t Sq,
                     int64_t Sk, int64_t D, double scale, int64_t causal,
                     const int64_t *rows, int64_t nrows, double *o,
                     double *lse);

/* The same by the tiled online recurrence over key blocks of Bc. */
int oracle_attention_online(const void *q, int64_t ldq, const void *k,
                            int64_t ldk, const void *v, int64_t ldv, int dtype,
                            int64_t Sq, int64_t Sk, int64_t D, double scale,
                            int64_t causal, int64_t Bc, const int64_t *rows,
                            int64_t nrows, double *o, double *lse);

#ifdef __cplusplus
}
#endif
#endif

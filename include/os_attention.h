/*
 * os_attention -- attention forward with the online softmax inside key
 * tiles, for AMD Instinct MI355X (gfx950).  Part of libos_softmax; shares
 * its status and dtype codes (os_softmax.h).
 *
 * What is computed, per batch b, head h and query row i:
 *   s_ij  = scale * (q_i . k_j)                 for the admitted keys j
 *   m_i   = max_j s_ij,  l_i = sum_j e^(s_ij - m_i)
 *   o_i   = sum_j (e^(s_ij - m_i) / l_i) v_j    (softmax(s_i) times V)
 *   lse_i = m_i + log l_i
 * This is attention as the consumer of the online softmax in
 * "5.2 CUDA Online Softmax 实现优化" (AIInfraGuide) §8.2, the FlashAttention
 * section of "从原始Softmax到在线Softmax" (its running m, l and unnormalised
 * output, rescaled by e^(m_old - m_new) when a key block raises the max),
 * and "Softmax 数值稳定性与 IO-Aware Attention：从在线归一化到
 * FlashAttention" §7 (the loop over K/V tiles that never writes the score
 * matrix to memory).  The score matrix is never stored: each workgroup
 * keeps 256 query rows in registers, streams K and V tiles of 64 keys
 * (128 at D = 32) through LDS, and carries (m, l, o~) per row.
 *
 * Arithmetic: Q, K, V are bfloat16; q.k and P.V are bf16 matrix-core
 * products with fp32 accumulation; the softmax state is fp32.  The
 * probabilities enter the P.V product rounded to bf16 (nearest even); l
 * sums them before that rounding.  lse is fp32.
 *
 * Layout: each of q, k, v, o is addressed as
 *   base + b * stride[0] + h * stride[1] + row * stride[2] + c
 * with strides in elements (host arrays of three int64) and the last axis
 * (c < D) contiguous, so dense [B][H][S][D] and [B][S][H][D] both work, and
 * stride 0 shares K/V across heads or batches.  lse (nullable) is dense
 * fp32 [B][H][Sq].  The output regions of different (b, h, row) must not
 * overlap each other or the inputs.
 *
 * Mask: causal_offset < 0 admits every key; causal_offset >= 0 admits key j
 * for query i when j <= i + causal_offset (0 is square self-attention;
 * Sk - Sq aligns the last query with the last key).  Every row then admits
 * key 0, so no row is empty.
 *
 * Special values: a NaN or +inf score makes its row's o and lse NaN (as in
 * the row-wise softmax); non-finite V entries propagate into o.
 */
#ifndef OS_ATTENTION_H
#define OS_ATTENTION_H

#include "os_softmax.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Attention forward.
 *  q          bf16 [B][H][Sq][D] under q_strides; device pointer.
 *  k, v       bf16 [B][H][Sk][D] under k_strides, v_strides; device.
 *  o          [B][H][Sq][D] under o_strides, dtype o_dtype (OS_BF16,
 *             rounded to nearest even, or OS_F32); device, written.
 *  lse        fp32 [B][H][Sq] dense, nullable; device, written.
 *  D          32, 64 or 128.
 *  *_strides  host arrays of 3 int64 (batch, head, row), in elements,
 *             each >= 0, the row stride >= D; read during the call only.
 *  scale      multiplies q.k; finite and > 0 (the pages use 1/sqrt(D)).
 *  stream     HIP stream the kernel is enqueued on (0: the null stream).
 * Returns OS_OK after enqueueing one kernel (nothing when B, H or Sq is 0;
 * beyond 2^22 workgroups, one launch per run of whole batches or of heads
 * of one batch, since a launch counts its threads in 32 bits), or, before
 * any HIP call:
 *  OS_ERR_NULL        a pointer the call needs is NULL;
 *  OS_ERR_SHAPE       B, H or Sq < 0, Sk < 1, Sq or Sk > 2^30, or more
 *                     than 2^31 - 1 workgroups (query blocks of 256 rows,
 *                     times B H);
 *  OS_ERR_STRIDE      a negative stride, a row stride < D, or a base or
 *                     stride not 16-byte aligned (all of q, k, v, o);
 *  OS_ERR_DTYPE       o_dtype is neither OS_F32 nor OS_BF16;
 *  OS_ERR_UNSUPPORTED D is not 32, 64 or 128, scale is not finite and > 0, or
 *                     a K or V row stride is 2^23 elements or more;
 * then, once the arguments are valid,
 *  OS_ERR_DEVICE      no device is current or it is not a gfx950 (read
 *                     with hipGetDevice, cached per device);
 *  OS_ERR_HIP         the launch failed.
 * Deterministic: the work partition depends on the shape only and no
 * atomics are used. */
os_status os_attention_fwd(const void *q, const void *k, const void *v,
                           void *o, float *lse, int64_t B, int64_t H,
                           int64_t Sq, int64_t Sk, int64_t D,
                           const int64_t *q_strides, const int64_t *k_strides,
                           const int64_t *v_strides, const int64_t *o_strides,
                           os_dtype o_dtype, float scale,
                           int64_t causal_offset, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif

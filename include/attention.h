/*
 * attention.h -- C ABI of the fused attention forward of libgemm (gfx950).
 *
 * Operation ("Modern GPU Programming For MLSys - 书籍总结", part IV,
 * sections 5.1-5.3: two matrix products with a softmax between them, the
 * running-max rescaling of section 5.2, causal masking and grouped-query
 * heads).  For batch b, query head h, query row i and dimension d:
 *
 *     s(i, j) = scale * sum_d Q[b][h][i][d] * K[b][g(h)][j][d]
 *     O[b][h][i][d] = sum_j softmax_j(s(i, j)) * V[b][g(h)][j][d]
 *     lse[b][h][i]  = log(sum_j exp(s(i, j)))
 *
 * over the keys j in [0, seq_k) visible to row i; g(h) = h / (heads_q /
 * heads_kv) is the key/value head of query head h.  With causal != 0 key j
 * is visible to row i when j <= i + (seq_k - seq_q) (the causal mask aligned
 * at the bottom-right corner, so the last query row sees every key).  A row
 * with no visible key gets O = 0 and lse = -inf.
 *
 * Layout.  Q is [batch][heads_q][seq_q][head_dim], K and V are
 * [batch][heads_kv][seq_k][head_dim], all bf16; O is the same shape as Q in
 * fp32; lse is dense fp32 [batch][heads_q][seq_q].  Each of Q, K, V and O is
 * addressed through three element strides (batch, head, sequence) read from a
 * host array of 3 int64_t, or dense when the pointer is NULL; the head
 * dimension is contiguous.  This covers both the [B][H][S][D] and the
 * [B][S][H][D] storage orders.
 *
 * Requirements (GEMM_ERR_INVALID_ARG otherwise, nothing written):
 *   - head_dim is 64 or 128; heads_q and heads_kv >= 1, heads_q a multiple of
 *     heads_kv; batch, seq_q, seq_k >= 0; scale finite and > 0;
 *   - Q, K, V 16-byte aligned with every stride a multiple of 8 elements;
 *     O (and lse) 16-byte (4-byte) aligned, O's strides multiples of 4;
 *   - within one head, (seq_q + 256) rows of Q and O and (seq_k + 64) rows of
 *     K and V span less than 2 GiB (32-bit buffer offsets);
 *   - non-NULL Q, K, V, O whenever the extents they cover are non-empty.
 * Returns GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED (not a gfx950
 * device) or GEMM_ERR_LAUNCH (the HIP runtime refused the launch).
 *
 * Numerics: both products take bf16 operands with fp32 accumulation; the
 * softmax runs in fp32, and its probabilities are rounded to bf16 (nearest
 * even) as the value product's operand, while the row sums that normalise O
 * add the unrounded fp32 values.  Elementwise,
 * |O - exact| <= 2^-8 (1 + 2^-6) * sum_j p(i, j) |V(j, d)| plus fp32
 * summation terms (stated with the tests).  O is the value sum times the
 * correctly rounded reciprocal of the row sum, refined by one fma residual
 * step (Markstein's correction); rows whose probabilities are exact (equal
 * scores, or one dominant key) with integer V give the IEEE quotient, as
 * the tests check bit for bit.
 *
 * Ownership and execution are those of every libgemm entry point: device
 * pointers owned by the caller, no allocation, copy or host synchronisation,
 * work enqueued on `stream` (a hipStream_t; NULL = default stream),
 * deterministic results, graph-capture safe, never aborts.  O and lse must
 * not alias Q, K or V.
 */
#ifndef LIBGEMM_ATTENTION_H
#define LIBGEMM_ATTENTION_H

#include <stdint.h>

#include "libgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

int attn_fwd_bf16(int64_t batch, int64_t heads_q, int64_t heads_kv,
                  int64_t seq_q, int64_t seq_k, int64_t head_dim,
                  const void* Q, const int64_t* q_strides,
                  const void* K, const int64_t* k_strides,
                  const void* V, const int64_t* v_strides,
                  float* O, const int64_t* o_strides,
                  float* lse, float scale, int causal, void* stream);

/* The same operation with the output type chosen by out_type (the constants
 * of libgemm.h): GEMM_OUT_F32 is attn_fwd_bf16 exactly; GEMM_OUT_BF16 stores
 * O as bf16, each element the fp32 result above rounded to nearest even
 * (NaN stays NaN), so the output has Q's type and half the bytes.  O is then
 * a 2-byte element array, 8-byte aligned, with strides (in its own elements)
 * that are multiples of 4; the 2 GiB span rule counts its 2-byte rows.  The
 * error bound adds that final rounding, 2^-8 |O| relative (bf16's unit
 * roundoff).  lse stays fp32.
 * Any other out_type, or any requirement above broken, returns
 * GEMM_ERR_INVALID_ARG with nothing written. */
int attn_fwd_bf16_out(int64_t batch, int64_t heads_q, int64_t heads_kv,
                      int64_t seq_q, int64_t seq_k, int64_t head_dim,
                      const void* Q, const int64_t* q_strides,
                      const void* K, const int64_t* k_strides,
                      const void* V, const int64_t* v_strides,
                      void* O, const int64_t* o_strides, int out_type,
                      float* lse, float scale, int causal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_ATTENTION_H */

/*
 * attention.h -- C ABI of the MI355X (gfx950) row softmax and attention
 * forward pass, the second workload of "TileLang simplifica la creación de
 * kernels GPU de alto rendimiento" (section "Softmax y FlashAttention sin
 * materializar matrices innecesarias"), built in the same library as the
 * GEMM (libgemm_relu.so) and returning the same status codes.
 *
 * Conventions shared with gemm_relu.h: device pointers to IEEE binary16
 * values, a stream passed as an opaque pointer (hipStream_t, or NULL), every
 * argument checked on the host before any HIP call, one kernel enqueued and
 * no wait. The caller owns every buffer.
 */
#ifndef ATTENTION_H
#define ATTENTION_H

#include <stdint.h>

#include "gemm_relu.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Row softmax: for each row i of X (rows x cols, row-major, leading dim cols),
 *     Y[i][j] = exp(X[i][j] - max_k X[i][k]) / sum_k exp(X[i][k] - max_k X[i][k])
 * computed in fp32 and rounded once to fp16 (nearest even). Y may be X (in
 * place) but must not otherwise overlap it. rows == 0 or cols == 0 is a no-op.
 * Rows of at most 8192 columns, a multiple of 8, with 16-byte aligned X and Y,
 * are held in registers and read once; other shapes are read twice.
 * Errors: EINVAL (negative size, NULL with data, partial overlap),
 * EUNSUPPORTED (size above INT32_MAX, odd address, device not gfx950), EHIP.
 */
int softmax_rows_f16(int64_t rows, int64_t cols, const void* X, void* Y, void* stream);

/*
 * Attention forward pass (the FlashAttention result): for each batch b < B
 * and head h < H, with Q[b][h] (Sq x D) and K[b][h], V[b][h] (Skv x D),
 *     O[b][h][i][:] = sum_j p_ij V[b][h][j][:],
 *     p_ij = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i),  s_ij = scale * Q[b][h][i][:] . K[b][h][j][:]
 * over the keys the query may see: all (causal = 0), or j <= i (causal = 1:
 * no position uses a later one, counted from the first key). Sums in fp32,
 * p rounded to fp16 before the product with V, O rounded once to fp16.
 *   Q, O      : [B][H][Sq][D] contiguous fp16
 *   K, V      : [B][H][Skv][D] contiguous fp16
 *   lse       : NULL, or [B][H][Sq] fp32 receiving m_i + ln(sum_j exp(s_ij - m_i))
 *               (-inf for a row with no keys)
 *   D         : 64 or 128
 * scale is a finite float with |scale| <= 2^64 (1/sqrt(D) is the usual
 * choice): the kernel scales scores in fp32, and with |Q.K| <= D * 65504^2
 * that bound keeps every scaled score and every difference of two finite.
 * Skv == 0 gives O = 0. Pointers must be 16-byte aligned (lse 4-byte); O must
 * not overlap Q, K, V or lse. Errors: EINVAL (negative size, NULL with data,
 * causal not 0/1, scale not finite, overlap), EUNSUPPORTED (D not 64/128,
 * |scale| > 2^64, a size above the kernel's 32-bit offsets (B*H, Sq,
 * Skv < 2^31, S * D < 2^30), misaligned pointer, device not gfx950), EHIP.
 */
int flash_attn_fwd_f16(int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D, const void* Q, const void* K,
                       const void* V, void* O, void* lse, float scale, int causal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTENTION_H */

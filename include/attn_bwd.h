/*
 * attn_bwd.h -- C ABI of the MI355X (gfx950) attention backward (gradients of attn_fwd).
 *
 * Operation.  For the forward of attn_fwd.h (same masks: key padding and the top-left causal
 * mask), a loss whose gradient with respect to O is dO and with respect to LSE is dLSE, and
 * P[i,j] = exp(scale q_i . k_j - LSE_i) on the valid keys (0 elsewhere):
 *     dV[j] = sum_i P[i,j] dO[i]
 *     dS[i,j] = P[i,j] ( dO[i] . V[j] - (dO[i] . O[i] - dLSE[i]) )
 *     dQ[i] = scale sum_j dS[i,j] K[j],     dK[j] = scale sum_i dS[i,j] Q[i]
 * Sources: the backward needs the softmax output of the forward (aicoding.csdn.net page,
 * ch.1); FlashAttention-2 rebuilds it in the backward from what the forward kept instead of
 * storing the N x N matrix (hotelren.com page on attention, sec.4.2).  Here P is rebuilt from
 * the forward's LSE, so the forward's O and LSE (from attn_fwd on the same inputs) are inputs.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include "attn_fwd.h"

/* The entry points are the only symbols the library exports (it is built with hidden
 * visibility); ATTN_API marks them. */
#ifndef ATTN_API
#if defined(__GNUC__) || defined(__clang__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif
#endif

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_bwd -- enqueue the attention backward on `stream` and return.
 *
 *   q, o, dout  device, [B, H, Nq, D] row-major contiguous, `dtype`: the forward's Q, its output
 *               O and the gradient dO.
 *   k, v        device, [B, H, Nk, D] row-major contiguous, `dtype`.
 *   lse         device, fp32 [B, H, Nq]: the forward's LSE (-inf for a row with no valid key).
 *   dlse        device, fp32 [B, H, Nq] gradient with respect to LSE, or NULL for zero.
 *   dq          device, [B, H, Nq, D], `dtype` (written).
 *   dk, dv      device, [B, H, Nk, D], `dtype` (written; keys no row sees get 0).
 *   B, H, Nq, Nk, D, scale, key_lens  as attn_fwd; causal 0 or 1 (top-left).
 *   dtype       ATTN_BF16 or ATTN_F16 (fp32 accumulation; outputs rounded to nearest even), or
 *               ATTN_F32 (fp32 throughout, on the vector ALUs: meant for small problems).
 *   workspace   device memory of at least attn_bwd_workspace_size(B, H, Nq) bytes, 16-byte
 *               aligned, owned by the caller; contents on entry do not matter (overwritten).
 *   stream      hipStream_t as void*, NULL for the default stream.
 *
 * Two kernels run in order on the stream: the first forms dQ and the per-row statistics
 * (LSE in base 2, dO . O - dLSE) in the workspace, the second dK and dV.  Calls that share a
 * workspace must not overlap in time.  Alignment: every tensor pointer 16-byte aligned,
 * key_lens 4-byte.  Errors as attn_fwd (checked on the host, nothing enqueued on error), plus
 * ATTN_ERR_NULL / ATTN_ERR_ALIGN / ATTN_ERR_WORKSPACE for a missing, misaligned or short
 * workspace.  Outputs must not alias inputs.
 */
ATTN_API int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, const float* dlse, void* dq, void* dk, void* dv, int B, int H,
                      int Nq, int Nk, int D, float scale, int causal, const int32_t* key_lens, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_window -- attn_bwd for the forward of attn_fwd_window: the gradients of attention
 * restricted to the local band |i - j| <= window (on top of the causal and padding rules).
 * window -1 is no band (identical to attn_bwd); a band at least max(Nq, Nk) wide is no band;
 * window < -1 returns ATTN_ERR_WINDOW and writes nothing.  o and lse must come from
 * attn_fwd_window with the same window.  Key and query tiles outside every band are skipped.
 * Other arguments, layout, workspace, ownership and errors as attn_bwd.
 */
ATTN_API int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, const float* dlse, void* dq, void* dk, void* dv, int B, int H,
                             int Nq, int Nk, int D, float scale, int causal, int window,
                             const int32_t* key_lens, int dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes attn_bwd needs: 2 * B * H * round_up(Nq, 64) * 4; 0 for B, H or Nq < 1.
 * attn_bwd returns ATTN_ERR_SHAPE when this exceeds 2^31 - 1 bytes. */
ATTN_API size_t attn_bwd_workspace_size(int B, int H, int Nq);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */

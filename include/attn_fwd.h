/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused attention forward.
 *
 * Operation (multi-head scaled-dot-product attention, forward only).  For every batch b,
 * head h and query row i:
 *     O[b,h,i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:]  over the valid keys j ) V[b,h,:,:]
 *     LSE[b,h,i] = ln sum_j exp( scale * Q[b,h,i,:] . K[b,h,j,:] )   over the same keys
 * Sources: the definition softmax(Q K^T / sqrt(d_k)) V with an optional mask filled before the
 * softmax (hotelren.com page on attention, ch.1 code and sec.2.1); the causal mask that lets a
 * position see only itself and earlier positions (same page, sec.2.1; lshu.cn page, sec.3.1);
 * the boolean padding mask where true means "may attend" (lshu.cn page, sec.5.2); the
 * max-shifted log-sum-exp (aicoding.csdn.net page, sec.2.2); the fused tiled loop that never
 * stores the score matrix (hotelren.com page, sec.4.1) and skips inactive key tiles (same
 * page, ch.5); the fused-library call taking q, k, v in [b, h, s, d] with a causal flag and a
 * softmax scale (aicoding.csdn.net page, ch.5).
 *
 * Valid keys of row i in batch b: j < L_b, and j <= i when causal (top-left aligned), with
 * L_b = key_lens ? clamp(key_lens[b], 0, Nk) : Nk.  A row with no valid key gets O = 0 and
 * LSE = -inf.  Masked keys are left out of the softmax (equal to filling with -inf, -1e9 or
 * adding -10000 on every row that keeps a key).
 *
 * The library allocates nothing, keeps no pointer after returning, holds no mutable global
 * state and is re-entrant.  No HIP header is needed to call it: the stream is passed as
 * void* (a hipStream_t; NULL is the default stream).
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stddef.h>
#include <stdint.h>

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

/* Storage type of q, k, v and o.  Scores, softmax state and accumulation are fp32 for all. */
typedef enum {
    ATTN_F32 = 0,  /* IEEE binary32 */
    ATTN_F16 = 1,  /* IEEE binary16 */
    ATTN_BF16 = 2  /* bfloat16 (top half of binary32) */
} attn_dtype;

typedef enum {
    /* The first seven codes and their values are the interface's original set. */
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,      /* q, k, v, o or lse is NULL (attn_decode, attn_bwd: also a needed workspace) */
    ATTN_ERR_SHAPE = -2,     /* B, H, Nq or Nk < 1, or a size beyond the 32-bit limits below */
    ATTN_ERR_HEAD_DIM = -3,  /* D is not 64 or 128 */
    ATTN_ERR_DTYPE = -4,     /* dtype is not an attn_dtype */
    ATTN_ERR_SCALE = -5,     /* scale is not finite */
    ATTN_ERR_LAUNCH = -6,    /* the HIP runtime rejected the kernel launch */
    /* Added after the original set, which had no code for these argument errors. */
    ATTN_ERR_FLAG = -7,      /* causal is not 0 or 1 */
    ATTN_ERR_ALIGN = -8,     /* q, k, v, o or lse is not 16-byte aligned (key_lens: 4-byte) */
    ATTN_ERR_WINDOW = -9,    /* window is below -1 (attn_fwd_window, attn_bwd_window) */
    ATTN_ERR_WORKSPACE = -10, /* workspace smaller than the *_workspace_size() query (attn_decode, attn_bwd) */
    ATTN_ERR_SCRATCH = -11    /* attn_decode_noalloc: the call needs more than ATTN_DECODE_SCRATCH_BYTES */
} attn_status;

/*
 * attn_fwd -- enqueue the fused attention forward on `stream` and return.
 *
 *   q        device, [B, H, Nq, D] row-major contiguous, `dtype`.
 *   k, v     device, [B, H, Nk, D] row-major contiguous, `dtype`.
 *   o        device, [B, H, Nq, D] row-major contiguous, `dtype` (written; rounded to nearest
 *            even from the fp32 result).
 *   lse      device, fp32 [B, H, Nq] (written): natural-log log-sum-exp of the scaled logits over
 *            the valid keys.
 *   B, H     batch and heads, >= 1.
 *   Nq, Nk   query and key lengths, >= 1.  Any length is accepted (tails are masked inside the
 *            kernel); Nk * D and Nq * D must stay below 2^29 elements per (b, h).
 *   D        head dimension shared by q, k and v: 64 or 128.
 *   scale    finite fp32 multiplier of the raw dot products (normally 1/sqrt(D)); it may be 0 or
 *            negative.
 *   causal   0 or 1.
 *   key_lens NULL (all Nk keys valid) or device int32[B]; values outside [0, Nk] are clamped.
 *   dtype    an attn_dtype.
 *   stream   hipStream_t as void*, NULL for the default stream.
 *
 * Alignment: q, k, v, o and lse must be 16-byte aligned, key_lens 4-byte aligned.
 * Ownership: every buffer belongs to the caller and must stay valid until the enqueued work
 * has finished; outputs must not alias inputs.
 * Errors: arguments are checked on the host before anything is enqueued; on any error the
 * function returns a negative attn_status and writes nothing.  A launch failure reported by
 * the runtime returns ATTN_ERR_LAUNCH.  Faults inside the kernel (e.g. a pointer that is not
 * device memory of the stated size) surface on the stream, not here.
 */
ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int Nq, int Nk, int D, float scale, int causal, const int32_t* key_lens, int dtype,
                      void* stream);

/*
 * attn_fwd_window -- attn_fwd restricted to a local band (sliding-window attention): row i
 * attends only to keys j with |i - j| <= window, on top of the causal and padding rules above.
 * Source: the local-window method in which each position attends to the positions within a
 * window before and after it and every other weight is zero (lshu.cn page, sec.2,
 * "localization", Longformer / BigBird windows; aicoding.csdn.net page, sec.4.3, w = 512).
 * With causal = 1 the band keeps i - window <= j <= i.
 *
 *   window   -1 for no band (then identical to attn_fwd), or >= 0.  A band at least as wide as
 *            max(Nq, Nk) is no band.  Key tiles outside every row's band are never read, so
 *            the work falls with the band.
 *   other arguments, layout, ownership and errors as attn_fwd; window < -1 returns
 *   ATTN_ERR_WINDOW and writes nothing.  A row whose band holds no valid key gets O = 0 and
 *   LSE = -inf.
 */
ATTN_API int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                             int H, int Nq, int Nk, int D, float scale, int causal, int window,
                             const int32_t* key_lens, int dtype, void* stream);

/*
 * attn_decode -- attention of Nq new queries against a KV cache: the queries are the last Nq
 * positions of each cached sequence (the cache already holds their own keys and values), so
 * with causal = 1 query i keeps keys j <= i + L_b - Nq (bottom-right aligned), and with one
 * query every valid key.  Source: the KV cache that keeps every token's key and value and lets
 * each new token reuse them instead of recomputing the sequence (hotelren.com page, sec.3.1).
 *
 * Made for small Nq and long Nk: the keys of each (query tile, b, h) are split over several
 * workgroups so that even B*H = 32 fills the chip; each split writes an fp32 partial result (O
 * over its keys, its log-sum-exp) to `workspace`, and a second kernel on the same stream merges
 * them: LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.  When one split is enough no
 * workspace is used.  Otherwise identical to attn_fwd (layouts, key_lens, dtypes, scale, O
 * rounding, empty rows give O = 0 and LSE = -inf).
 *
 *   causal           0: every valid key; 1: bottom-right causal mask as above.
 *   workspace        device memory of at least attn_decode_workspace_size(B, H, Nq, Nk, D, dtype)
 *                    bytes, 16-byte aligned, owned by the caller (may be NULL when that size is
 *                    0); its contents on entry do not matter, and it is overwritten.
 *   workspace_bytes  its size.
 * Errors as attn_fwd, plus ATTN_ERR_NULL / ATTN_ERR_ALIGN for a missing or misaligned
 * workspace and ATTN_ERR_WORKSPACE when it is too small; nothing is enqueued on any error.
 * Calls that share a workspace must not overlap in time.
 */
ATTN_API int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                         int Nq, int Nk, int D, float scale, int causal, const int32_t* key_lens, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_workspace_size -- bytes of workspace attn_decode needs for these sizes (0 when it
 * needs none, or when the sizes are invalid).  A pure function of its arguments.
 */
ATTN_API size_t attn_decode_workspace_size(int B, int H, int Nq, int Nk, int D, int dtype);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the split partials
 * go to a scratch buffer the library holds itself, a static device array of
 * ATTN_DECODE_SCRATCH_BYTES per GPU (reserved on each GPU the library runs on, until the process
 * ends).  Nothing is allocated, here or in the call: no hipMalloc, no hipFree, no allocating
 * library routine.  The first call on a device looks up that device's copy of the array.
 *
 *   arguments   as attn_decode without the workspace; results are bitwise those of
 *               attn_decode for the same inputs.
 *   limit       the call needs attn_decode_workspace_size(B, H, Nq, Nk, D, dtype) bytes of
 *               scratch; above ATTN_DECODE_SCRATCH_BYTES it returns ATTN_ERR_SCRATCH and enqueues
 *               nothing (use attn_decode with a workspace then).  With one query per sequence
 *               the need is about 0.5 MiB for any batch; it grows with Nq (about 16 MiB at
 *               Nq = 31, D = 128).
 *   concurrency every call on one GPU shares that GPU's scratch: calls that overlap in time on
 *               one GPU (different streams, different host threads) race and must not be made.
 *               Nothing in the scratch needs clearing between calls (each call overwrites what
 *               it reads).
 * Errors as attn_decode, plus ATTN_ERR_SCRATCH; ATTN_ERR_LAUNCH if the scratch's device address
 * cannot be obtained on the current device.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
ATTN_API int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                 int H, int Nq, int Nk, int D, float scale, int causal,
                                 const int32_t* key_lens, int dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
ATTN_API const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */

// attn_bwd.h -- parameters shared by the backward kernels and their launcher (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct BwdParams {
    const void* q;       // [B, H, Nq, D]
    const void* k;       // [B, H, Nk, D]
    const void* v;       // [B, H, Nk, D]
    const void* o;       // [B, H, Nq, D], the forward's output
    const void* dout;    // [B, H, Nq, D], gradient of the loss with respect to O
    const float* lse;    // [B, H, Nq], the forward's natural-log LSE
    const float* dlse;   // [B, H, Nq] gradient with respect to the LSE, or nullptr (zero)
    void* dq;            // [B, H, Nq, D]
    void* dk;            // [B, H, Nk, D]
    void* dv;            // [B, H, Nk, D]
    // Workspace written by the dQ kernel and read by the dK/dV kernel: two planes of
    // [B, H, nq_pad] fp32 (rows padded to a multiple of 64): LSE * log2(e) (+inf for a row that
    // sees no key and for padding rows), then Dr = rowsum(dO * O) - dLSE (0 on padding rows).
    float* stats;
    int nq_pad;
    const int32_t* key_lens;
    int B, H, Nq, Nk;
    int n_qtiles, n_ktiles;  // Q tiles of the dQ kernel, key tiles of the dK/dV kernel
    int n_blocks_q, n_blocks_k;
    float scale;         // the caller's scale (signed)
    float scale_log2;    // max(|scale| * log2(e), 1e-30)
    int negate;          // scale < 0: the sign is moved onto Q (dQ kernel) or K (dK/dV kernel)
    int causal;
    int window;          // half-width w of the local band |i - j| <= w, or -1 for none
};

// Keys [lo, hi) row i may attend to within the valid length kv_valid: the top-left causal rule
// keeps j <= i, the local band (WIN) keeps |i - j| <= w.
template <bool WIN>
__device__ __forceinline__ int bwd_key_lo(const BwdParams& p, int i) { return WIN ? i - p.window : 0; }
template <bool WIN>
__device__ __forceinline__ int bwd_key_hi(const BwdParams& p, int i, int kv_valid) {
    int hi = kv_valid;
    if (p.causal) hi = min(hi, i + 1);
    if (WIN) hi = min(hi, i + p.window + 1);
    return hi;
}
// Rows [lo, hi) that may see key j (before the query length): the inverse of the rules above.
template <bool WIN>
__device__ __forceinline__ int bwd_row_lo(const BwdParams& p, int j) {
    int lo = p.causal ? j : 0;
    if (WIN) lo = max(lo, j - p.window);
    return max(lo, 0);
}
template <bool WIN>
__device__ __forceinline__ int bwd_row_hi(const BwdParams& p, int j) {
    return WIN ? min(p.Nq, j + p.window + 1) : p.Nq;
}

}  // namespace attn

hipError_t attn_launch_bwd_mfma(const attn::BwdParams& p, int dtype, int D, hipStream_t stream);
int attn_bwd_q_block();   // query rows per dQ workgroup
int attn_bwd_k_block();   // keys per dK/dV workgroup
// fp32 storage: the vector-ALU kernels of attn_bwd_f32.hip
hipError_t attn_launch_bwd_f32(const attn::BwdParams& p, int D, hipStream_t stream);
int attn_bwd_f32_q_block();
int attn_bwd_f32_k_block();

// attn_bwd_api.hip -- the C ABI of the backward: argument checks and the two launches.
#include <math.h>
#include <stdint.h>

#include <attn_bwd.h>
#include "attn_bwd.h"

namespace {

// Statistics rows are padded to whole 64-row tiles so the dK/dV kernel's tile reads stay
// inside each (b, h) slice.
int64_t nq_padded(int Nq) { return ((int64_t)Nq + 63) / 64 * 64; }

}  // namespace

extern "C" size_t attn_bwd_workspace_size(int B, int H, int Nq) {
    if (B < 1 || H < 1 || Nq < 1) return 0;
    return (size_t)2 * B * H * (size_t)nq_padded(Nq) * sizeof(float);
}

extern "C" int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, const float* dlse, void* dq, void* dk, void* dv, int B,
                               int H, int Nq, int Nk, int D, float scale, int causal, int window,
                               const int32_t* key_lens, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
    if (window < -1) return ATTN_ERR_WINDOW;
    const uintptr_t ptrs = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
                           (uintptr_t)lse | (uintptr_t)dlse | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
    if ((ptrs & 15) != 0 || ((uintptr_t)key_lens & 3) != 0) return ATTN_ERR_ALIGN;
    if ((int64_t)Nq * D >= ((int64_t)1 << 29) || (int64_t)Nk * D >= ((int64_t)1 << 29)) return ATTN_ERR_SHAPE;

    const bool f32 = dtype == ATTN_F32;
    const int64_t bm = f32 ? attn_bwd_f32_q_block() : attn_bwd_q_block();
    const int64_t bn = f32 ? attn_bwd_f32_k_block() : attn_bwd_k_block();
    const int64_t n_qtiles = ((int64_t)Nq + bm - 1) / bm, n_ktiles = ((int64_t)Nk + bn - 1) / bn;
    const int64_t nbq = n_qtiles * H * B, nbk = n_ktiles * H * B;
    const int64_t pad = nq_padded(Nq);
    // the statistics planes are addressed with 32-bit byte offsets
    if (nbq > INT32_MAX || nbk > INT32_MAX || 2 * (int64_t)B * H * pad * 4 > INT32_MAX) return ATTN_ERR_SHAPE;

    if (!workspace) return ATTN_ERR_NULL;
    if (((uintptr_t)workspace & 15) != 0) return ATTN_ERR_ALIGN;
    if (workspace_bytes < attn_bwd_workspace_size(B, H, Nq)) return ATTN_ERR_WORKSPACE;

    attn::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dlse = dlse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.stats = (float*)workspace;
    p.nq_pad = (int)pad;
    p.key_lens = key_lens;
    p.B = B;
    p.H = H;
    p.Nq = Nq;
    p.Nk = Nk;
    p.n_qtiles = (int)n_qtiles;
    p.n_ktiles = (int)n_ktiles;
    p.n_blocks_q = (int)nbq;
    p.n_blocks_k = (int)nbk;
    p.scale = scale;
    // As in the forward: base-2 logits with a strictly positive multiplier; the sign of a
    // negative scale moves onto Q (dQ kernel) or K (dK/dV kernel), and the gradients take the
    // signed scale.
    p.scale_log2 = (float)fmax(fabs((double)scale) * 1.4426950408889634074, 1e-30);
    p.negate = scale < 0.f;
    p.causal = causal;
    // |i - j| < max(Nq, Nk) always holds: a band at least that wide is no band
    p.window = window >= (Nq > Nk ? Nq : Nk) ? -1 : window;
    const hipError_t e = f32 ? attn_launch_bwd_f32(p, D, (hipStream_t)stream)
                             : attn_launch_bwd_mfma(p, dtype, D, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const float* dlse, void* dq, void* dk, void* dv, int B, int H,
                        int Nq, int Nk, int D, float scale, int causal, const int32_t* key_lens, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return attn_bwd_window(q, k, v, o, dout, lse, dlse, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, -1,
                           key_lens, dtype, workspace, workspace_bytes, stream);
}

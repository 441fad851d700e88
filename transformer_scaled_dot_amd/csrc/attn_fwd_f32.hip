// attn_fwd_f32.hip -- fused attention forward for fp32 storage, full fp32 arithmetic.
//
// Same tiled loop as the matrix-core kernel (per Q tile, stream K/V tiles through LDS, online
// softmax, never store S), but on the vector ALUs: fp32 MFMA would change nothing in the
// precision and this path serves small fp32 problems.  One wave per workgroup, one query row
// per lane; K and V rows are read from LDS as broadcasts, the Q tile sits in LDS with a padded
// row stride so that the 64 lanes reading one column hit 64 different banks.  The same key
// splits as the matrix-core kernel apply (partial results for the merge kernel).
#include "attn_common.h"

namespace {

constexpr int BMF = 64;  // query rows per workgroup (one per lane)

template <int D>
__global__ void __launch_bounds__(BMF) attn_fwd_f32_kernel(attn::Params p) {
    constexpr int BNF = D == 128 ? 16 : 32;  // keys per K/V tile (keeps LDS under 64 KiB)
    __shared__ float qs[BMF][D + 1];
    __shared__ float ks[BNF][D];
    __shared__ float vs[BNF][D];

    const int tid = threadIdx.x;
    const attn::BlockWork bw = attn::block_work(p, attn::xcd_remap(blockIdx.x, p.n_blocks));
    const int bh = bw.bh;
    int qt = bw.qt;
    if (p.causal && !p.causal_br) qt = p.n_qtiles - 1 - qt;
    const int b = bh / p.H;
    const int q0 = qt * BMF;
    const int qi = q0 + tid;

    const float* qg = (const float*)p.q + (size_t)bh * p.Nq * D;
    const float* kg = (const float*)p.k + (size_t)bh * p.Nk * D;
    const float* vg = (const float*)p.v + (size_t)bh * p.Nk * D;
    const float qsign = p.negate_q ? -1.f : 1.f;

    for (int idx = tid; idx < BMF * D; idx += BMF) {
        const int row = idx / D, d = idx % D;
        qs[row][d] = (q0 + row < p.Nq) ? qsign * qg[(size_t)(q0 + row) * D + d] : 0.f;
    }

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const int q_last = min(p.Nq, q0 + BMF) - 1;
    int kv_end = min(kv_valid, attn::row_key_hi(p, q_last, kv_valid));
    int kv_begin = max(0, attn::row_key_lo(p, q0)) / BNF * BNF;
    if (p.n_splits > 1) {  // this workgroup's share of the keys (split_len is a multiple of BNF)
        kv_begin = max(kv_begin, bw.split * p.split_len);
        kv_end = min(kv_end, (bw.split + 1) * p.split_len);
    }
    const int lo = attn::row_key_lo(p, qi), hi = attn::row_key_hi(p, qi, kv_valid);
    const float c2 = p.scale_log2;

    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int j0 = kv_begin; j0 < kv_end; j0 += BNF) {
        __syncthreads();
        for (int idx = tid; idx < BNF * D; idx += BMF) {
            const int row = idx / D, d = idx % D;
            const bool ok = j0 + row < kv_valid;
            ks[row][d] = ok ? kg[(size_t)(j0 + row) * D + d] : 0.f;
            vs[row][d] = ok ? vg[(size_t)(j0 + row) * D + d] : 0.f;
        }
        __syncthreads();

        float s[BNF];
        float mt = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < BNF; ++jj) {
            float acc = 0.f;
#pragma unroll 16
            for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qs[tid][d], ks[jj][d], acc);
            const float t = (j0 + jj >= lo && j0 + jj < hi) ? acc * c2 : -INFINITY;
            s[jj] = t;
            mt = fmaxf(mt, t);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float ls = 0.f;
#pragma unroll
        for (int jj = 0; jj < BNF; ++jj) {
            s[jj] = __builtin_amdgcn_exp2f(s[jj] - m_use);
            ls += s[jj];
        }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float acc = o[d] * alpha;
#pragma unroll
            for (int jj = 0; jj < BNF; ++jj) acc = __builtin_fmaf(s[jj], vs[jj][d], acc);
            o[d] = acc;
        }
    }

    if (qi < p.Nq) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        const size_t row = p.n_splits > 1 ? ((size_t)bw.split * p.B * p.H + bh) * p.Nq + qi
                                          : (size_t)bh * p.Nq + qi;
        float* og = (p.n_splits > 1 ? p.o_part : (float*)p.o) + row * D;
        float* lg = p.n_splits > 1 ? p.lse_part : p.lse;
#pragma unroll
        for (int d = 0; d < D; d += 4)
            *(float4*)(og + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
        lg[row] = l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * attn::kLn2 : -INFINITY;
    }
}

template <int D>
hipError_t launch_one(const attn::Params& p, hipStream_t stream) {
    attn::Params pc = p;
    void* args[] = {&pc};
    return hipLaunchKernel((const void*)attn_fwd_f32_kernel<D>, dim3(p.n_blocks), dim3(BMF), args,
                           0, stream);
}

}  // namespace

int attn_f32_block_m() { return BMF; }

hipError_t attn_launch_f32(const attn::Params& p, int D, hipStream_t stream) {
    return D == 128 ? launch_one<128>(p, stream) : launch_one<64>(p, stream);
}

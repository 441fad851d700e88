// attn_fwd_f32.hip -- fused attention forward for fp32 storage, full fp32 arithmetic.
//
// Same tiled loop as the matrix-core kernel (per Q tile, stream K/V tiles through LDS, online
// softmax, never store S), but on the vector ALUs: fp32 MFMA would change nothing in the
// precision and this path serves small fp32 problems.  Four lanes per query row, each owning a
// quarter of the head dimension; the NW waves of a workgroup (eight for D = 64, four for D = 128)
// share the 16-row Q tile (in LDS, with a padded row stride so that the 64 lanes reading one
// column slice hit 64 different banks) and split its keys, wave w taking key tiles w, w + NW, ...  Each
// wave keeps its own running max, sum and output; at the end the waves' partial states of a row
// are combined by the log-sum-exp rule (rescale each to the common max, add the sums and the
// outputs), the same rule the split-K merge applies across workgroups (here in a tree, log2 of
// the wave count rounds).  K and V rows are read from LDS as broadcasts.  The key splits of the
// matrix-core kernel apply here too (partial results for the merge kernel).
#include "attn_common.h"

namespace {

constexpr int LPR = 4;        // lanes per query row (2 or 4)
constexpr int BMF = 64 / LPR; // query rows per workgroup
constexpr int BNF = 16;       // keys per K/V tile
// waves per workgroup, each on every NW-th key tile (LDS: the Q tile plus one K and V tile per wave)
template <int D>
constexpr int waves_f32() { return D == 64 ? 8 : 4; }
constexpr unsigned kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data, gfx9-family layout
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// LPR lanes per query row: lane (r, h) = (lane % BMF, lane / BMF) owns row q0 + r and the columns
// [h D/LPR, (h + 1) D/LPR) of Q and O.  A score is the sum of the lanes' partial dot products
// (lanes 16 apart by v_permlane16_swap, then 32 apart by v_permlane32_swap, each swap followed by
// one add, in the same order in every lane), after which all lanes of the row hold it and run the
// same softmax; each then accumulates its share of the output.  Against one lane per row this cuts
// the vector work per lane by LPR and spreads a row tile over LPR times as many workgroups
// (16 rows per workgroup at LPR = 4); the tiny fp32 case (2 heads of 128 rows) went from 18.8 us
// per call to 12.0 (LPR = 2) and 9.5 (LPR = 4).
template <int D>
__global__ void __launch_bounds__(64 * waves_f32<D>()) attn_fwd_f32_kernel(attn::Params p) {
    constexpr int NWF = waves_f32<D>();
    constexpr int DH = D / LPR;  // columns per lane
    __shared__ float qs[BMF][D + 1];
    __shared__ float kv[NWF][2][BNF][D];  // each wave's K and V tile; the combine reuses it
    __shared__ float part_m[NWF][BMF], part_l[NWF][BMF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int r = lane % BMF, h = lane / BMF;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const attn::BlockWork bw = attn::block_work(p, attn::xcd_remap(blockIdx.x, p.n_blocks, p.n_qtiles * p.n_splits, p.xcd_interleave));
    const int bh = bw.bh;
    int qt = bw.qt;
    if (p.causal && !p.causal_br) qt = p.n_qtiles - 1 - qt;
    const int b = bh / p.H;
    const int q0 = qt * BMF;
    const int qi = q0 + r;

    const float* qg = (const float*)p.q + (size_t)bh * p.Nq * D;
    const float* kg = (const float*)p.k + (size_t)bh * p.Nk * D;
    const float* vg = (const float*)p.v + (size_t)bh * p.Nk * D;
    const float qsign = p.negate_q ? -1.f : 1.f;

    {
        // 16-byte loads, all in flight together; rows past Nq fall outside the buffer and read as 0
        constexpr int QV = BMF * D / 4;                  // float4s in the Q tile
        constexpr int L4 = (QV + 64 * NWF - 1) / (64 * NWF);
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(qg + (size_t)q0 * D), 0, (p.Nq - q0) * D * 4, kBufferWord3);
        f32x4_t qx[L4];
#pragma unroll
        for (int i = 0; i < L4; ++i)
            if (QV % (64 * NWF) == 0 || i * 64 * NWF + tid < QV)
                qx[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(qrs, (i * 64 * NWF + tid) * 16, 0, 0));
#pragma unroll
        for (int i = 0; i < L4; ++i) {
            if (QV % (64 * NWF) != 0 && i * 64 * NWF + tid >= QV) continue;
            const int e = (i * 64 * NWF + tid) * 4, row = e / D, d = e % D;
#pragma unroll
            for (int c = 0; c < 4; ++c) qs[row][d + c] = qsign * qx[i][c];
        }
    }

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const int q_last = min(p.Nq, q0 + BMF) - 1;
    int kv_end = min(kv_valid, attn::row_key_hi(p, q_last, kv_valid));
    int kv_begin = max(0, attn::row_key_lo(p, q0)) / BNF * BNF;
    if (p.n_splits > 1) {  // this workgroup's share of the keys (split_len is a multiple of BNF)
        kv_begin = max(kv_begin, bw.split * p.split_len);
        kv_end = min(kv_end, (bw.split + 1) * p.split_len);
    }
    const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + BNF - 1) / BNF : 0;
    const int lo = attn::row_key_lo(p, qi), hi = attn::row_key_hi(p, qi, kv_valid);
    const float c2 = p.scale_log2;
    float (*const ks)[D] = kv[wave][0];
    float (*const vs)[D] = kv[wave][1];
    const int c0 = h * DH;  // this lane's first column

    float o[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Round r: wave w takes tile r * NWF + w.  The barriers keep the waves in rounds, so a wave's
    // tile loads never overtake another wave's reads of the Q tile or of its own previous tile.
    for (int t0 = 0; t0 < n_tiles; t0 += NWF) {
        const int t = t0 + wave;
        const int j0 = kv_begin + t * BNF;
        __syncthreads();
        if (t < n_tiles) {
            // 16-byte loads, all in flight together; rows at or past the valid length fall
            // outside the buffer and read as zeros
            constexpr int L4 = BNF * D / 4 / 64;  // float4s per lane per tile
            const int bytes = (kv_valid - j0) * D * 4;
            const __amdgpu_buffer_rsrc_t krs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(kg + (size_t)j0 * D), 0, bytes, kBufferWord3);
            const __amdgpu_buffer_rsrc_t vrs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(vg + (size_t)j0 * D), 0, bytes, kBufferWord3);
            f32x4_t kx[L4], vx[L4];
#pragma unroll
            for (int i = 0; i < L4; ++i) {
                kx[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, (i * 64 + lane) * 16, 0, 0));
                vx[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, (i * 64 + lane) * 16, 0, 0));
            }
#pragma unroll
            for (int i = 0; i < L4; ++i) {
                *(f32x4_t*)(&ks[0][0] + (i * 64 + lane) * 4) = kx[i];
                *(f32x4_t*)(&vs[0][0] + (i * 64 + lane) * 4) = vx[i];
            }
        }
        __syncthreads();
        if (t >= n_tiles) continue;

        // partial dot products for the tile's 16 keys: 16 independent accumulators, K read as
        // 4-wide broadcasts (the LPR lane groups of the wave read LPR addresses)
        float s[BNF];
#pragma unroll
        for (int jj = 0; jj < BNF; ++jj) s[jj] = 0.f;
#pragma unroll 2
        for (int d = 0; d < DH; d += 4) {
            // all 16 broadcasts of this 4-column slice are requested before the first FMA, so one
            // wave per SIMD pays the LDS latency once per slice, not once per key
            f32x4_t kq[BNF];
#pragma unroll
            for (int jj = 0; jj < BNF; ++jj) kq[jj] = *(const f32x4_t*)&ks[jj][c0 + d];
            const float q0v = qs[r][c0 + d], q1v = qs[r][c0 + d + 1], q2v = qs[r][c0 + d + 2], q3v = qs[r][c0 + d + 3];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < BNF; ++jj) {
                s[jj] = __builtin_fmaf(q0v, kq[jj][0], s[jj]);
                s[jj] = __builtin_fmaf(q1v, kq[jj][1], s[jj]);
                s[jj] = __builtin_fmaf(q2v, kq[jj][2], s[jj]);
                s[jj] = __builtin_fmaf(q3v, kq[jj][3], s[jj]);
            }
        }
        // whole scores: the parts summed in the same order in every lane of the row
#pragma unroll
        for (int jj = 0; jj < BNF; ++jj) {
            if constexpr (LPR == 4) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, s[jj]),
                                                                 __builtin_bit_cast(unsigned, s[jj]), false, false);
                s[jj] = __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
            }
            const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, s[jj]),
                                                             __builtin_bit_cast(unsigned, s[jj]), false, false);
            s[jj] = __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
        }
        float mt = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < BNF; ++jj) {
            const float tv = (j0 + jj >= lo && j0 + jj < hi) ? s[jj] * c2 : -INFINITY;
            s[jj] = tv;
            mt = fmaxf(mt, tv);
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
        for (int d = 0; d < DH; d += 4) {
            float a0 = o[d] * alpha, a1 = o[d + 1] * alpha, a2 = o[d + 2] * alpha, a3 = o[d + 3] * alpha;
            f32x4_t vv[BNF];  // as for K: the slice's 16 broadcasts first
#pragma unroll
            for (int jj = 0; jj < BNF; ++jj) vv[jj] = *(const f32x4_t*)&vs[jj][c0 + d];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < BNF; ++jj) {
                const f32x4_t vq = vv[jj];
                a0 = __builtin_fmaf(s[jj], vq[0], a0);
                a1 = __builtin_fmaf(s[jj], vq[1], a1);
                a2 = __builtin_fmaf(s[jj], vq[2], a2);
                a3 = __builtin_fmaf(s[jj], vq[3], a3);
            }
            o[d] = a0;
            o[d + 1] = a1;
            o[d + 2] = a2;
            o[d + 3] = a3;
        }
    }

    // Combine the waves' partial states of each row (base 2): M = max_w m_w, l = sum_w 2^(m_w - M) l_w,
    // O = sum_w 2^(m_w - M) O_w.  A wave that saw no key of the row has m = -inf and weight 0.  All
    // lanes of a row hold the same m and l; the first one publishes them.
    __syncthreads();
    if (h == 0) {
        part_m[wave][r] = m_run;
        part_l[wave][r] = l_run;
    }
    __syncthreads();
    float m_all = part_m[0][r];
#pragma unroll
    for (int w = 1; w < NWF; ++w) m_all = fmaxf(m_all, part_m[w][r]);
    const float m_ref = m_all == -INFINITY ? 0.f : m_all;
    float l_all = 0.f;
#pragma unroll
    for (int w = 0; w < NWF; ++w) l_all += part_l[w][r] * __builtin_amdgcn_exp2f(part_m[w][r] - m_ref);
    const float wgt = __builtin_amdgcn_exp2f(m_run - m_ref);
    // Tree combine of the weighted outputs: in each round the upper half of the remaining waves
    // writes its output to a slot of the LDS the key loop no longer reads (the K/V tiles, then
    // the Q tile) and the lower half adds it in: log2(NWF) rounds instead of NWF - 1 in turn.
    // The order of the additions is fixed, so results are the same on every run.
    constexpr int SLOT = BMF * (D + 1);                                    // floats per slot
    constexpr int KV_SLOTS = (int)(sizeof(kv) / sizeof(float)) / SLOT;
    constexpr int Q_SLOTS = (int)(sizeof(qs) / sizeof(float)) / SLOT;
    static_assert(KV_SLOTS + Q_SLOTS >= NWF / 2, "not enough LDS for the tree combine");
    auto slot = [&](const int i) -> float* {
        return i < KV_SLOTS ? &kv[0][0][0][0] + i * SLOT : &qs[0][0] + (i - KV_SLOTS) * SLOT;
    };
#pragma unroll
    for (int d = 0; d < DH; ++d) o[d] *= wgt;
    for (int half = NWF / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
            float* dst = slot(wave - half) + r * (D + 1) + c0;
#pragma unroll
            for (int d = 0; d < DH; ++d) dst[d] = o[d];
        }
        __syncthreads();
        if (wave < half) {
            const float* src = slot(wave) + r * (D + 1) + c0;
#pragma unroll
            for (int d = 0; d < DH; ++d) o[d] += src[d];
        }
        __syncthreads();
    }

    if (wave == 0 && qi < p.Nq) {
        const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
        const size_t row = p.n_splits > 1 ? ((size_t)bw.split * p.B * p.H + bh) * p.Nq + qi
                                          : (size_t)bh * p.Nq + qi;
        float* og = (p.n_splits > 1 ? p.o_part : (float*)p.o) + row * D + c0;
        float* lg = p.n_splits > 1 ? p.lse_part : p.lse;
#pragma unroll
        for (int d = 0; d < DH; d += 4)
            *(float4*)(og + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
        if (h == 0) lg[row] = l_all > 0.f ? (m_all + __builtin_amdgcn_logf(l_all)) * attn::kLn2 : -INFINITY;
    }
}

template <int D>
hipError_t launch_one(const attn::Params& p, hipStream_t stream) {
    attn::Params pc = p;
    void* args[] = {&pc};
    return hipLaunchKernel((const void*)attn_fwd_f32_kernel<D>, dim3(p.n_blocks), dim3(64 * waves_f32<D>()), args,
                           0, stream);
}

}  // namespace

int attn_f32_block_m() { return BMF; }

hipError_t attn_launch_f32(const attn::Params& p, int D, hipStream_t stream) {
    return D == 128 ? launch_one<128>(p, stream) : launch_one<64>(p, stream);
}

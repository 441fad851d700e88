// attn_bwd_f32.hip -- attention backward (dQ, dK, dV) for fp32 storage, full fp32 arithmetic.
//
// The same gradients as the matrix-core backward (hotelren.com page on attention, sec.4.2:
// P is rebuilt from the forward's LSE, never stored):
//   P = exp(scale Q K^T - LSE),  dP = dO V^T,  Dr_i = rowsum(dO * O)_i - dLSE_i,
//   dS = P (dP - Dr),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// on the vector ALUs, for the small fp32 problems the fp32 forward serves.  Two kernels, no
// atomics, in order on the caller's stream:
//
//   attn_bwd_f32_dq_kernel    64 query rows per workgroup, one per lane; the workgroup's waves
//                             split the row tile's keys (16-key tiles w, w + NW, ...) and add
//                             their partial dQ through LDS at the end.  Wave 0 also writes the
//                             rows' LSE * log2(e) and Dr to the workspace.
//   attn_bwd_f32_dkdv_kernel  16 keys per workgroup, four lanes per key, each holding a quarter
//                             of the key's K, V, dK and dV columns; the partial dot products of
//                             a (row, key) pair meet by two lane exchanges.  The waves split the
//                             rows (16-row tiles w, w + NW, ...) and add their partial dK and dV
//                             through LDS at the end.
#include "attn_bwd.h"
#include "attn_common.h"

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.44269504088896340736f;
constexpr unsigned kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data, gfx9-family layout
constexpr int BQF = 64;  // dQ kernel: query rows per workgroup (one per lane)
constexpr int BKF = 16;  // dK/dV kernel: keys per workgroup (four lanes each)
constexpr int TF = 16;   // keys (dQ kernel) or rows (dK/dV kernel) per streamed tile
constexpr int NWB = 4;   // waves per workgroup in both kernels

// One 16-row slice [row0, row0 + TF) of a [rows, D] fp32 array into LDS (row-major, D floats per
// row) by the 64 lanes of one wave, 16-byte loads; rows at or past `valid` read as zeros.
template <int D>
__device__ __forceinline__ void load_rows(float* dst, const float* src, int row0, int valid, int lane) {
    constexpr int L4 = TF * D / 4 / 64;
    const int bytes = (valid - row0) * D * 4;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + (size_t)row0 * D), 0, bytes > 0 ? bytes : 0, kBufferWord3);
    f32x4_t x[L4];
#pragma unroll
    for (int i = 0; i < L4; ++i)
        x[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (i * 64 + lane) * 16, 0, 0));
#pragma unroll
    for (int i = 0; i < L4; ++i) *(f32x4_t*)(dst + (i * 64 + lane) * 4) = x[i];
}

// ------------------------------------------------------------------------------------ dQ
template <int D, bool WIN>
__global__ void __launch_bounds__(64 * NWB) attn_bwd_f32_dq_kernel(attn::BwdParams p) {
    __shared__ float qs[BQF][D + 1];
    __shared__ float dos[BQF][D + 1];
    __shared__ float kv[NWB][2][TF][D];  // each wave's K and V tile; the final sum reuses it
    __shared__ float row_l2[BQF], row_dr[BQF];
    static_assert(NWB * 2 * TF * D >= BQF * (D + 1), "reduction buffer does not fit");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = attn::xcd_remap(blockIdx.x, p.n_blocks_q, p.n_qtiles);
    const int bh = blk / p.n_qtiles;
    int qt = blk - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest rows first
    const int b = bh / p.H;
    const int q0 = qt * BQF;
    const int qi = q0 + lane;

    const size_t qbase = (size_t)bh * p.Nq * D;
    const float* qg = (const float*)p.q + qbase;
    const float* dog = (const float*)p.dout + qbase;
    const float* og = (const float*)p.o + qbase;
    const float* kg = (const float*)p.k + (size_t)bh * p.Nk * D;
    const float* vg = (const float*)p.v + (size_t)bh * p.Nk * D;
    const float qsign = p.negate ? -1.f : 1.f;  // a negative scale moves onto Q

    // Q and dO rows of the tile into LDS by 16-byte loads, all in flight together (rows past Nq
    // fall outside the buffers and read as zeros): thread t takes float4 t, t + 256, ...
    {
        constexpr int L4 = BQF * D / 4 / (64 * NWB);
        const int bytes = (p.Nq - q0) * D * 4;
        const __amdgpu_buffer_rsrc_t qrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(qg + (size_t)q0 * D), 0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t drs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(dog + (size_t)q0 * D), 0, bytes, kBufferWord3);
        f32x4_t xq[L4], xd[L4];
#pragma unroll
        for (int i = 0; i < L4; ++i) {
            xq[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(qrs, (i * 64 * NWB + tid) * 16, 0, 0));
            xd[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(drs, (i * 64 * NWB + tid) * 16, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < L4; ++i) {
            const int e = (i * 64 * NWB + tid) * 4, row = e / D, d = e % D;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                qs[row][d + c] = qsign * xq[i][c];
                dos[row][d + c] = xd[i][c];
            }
        }
    }
    __syncthreads();
    // Row statistics (wave 0): Dr = dO . O - dLSE, LSE in base 2 (+inf: the row sees no key or
    // is past Nq, so all its weights are 0).
    if (wave == 0) {
        float dr = 0.f, l2 = INFINITY;
        if (qi < p.Nq) {
            const f32x4_t* orow = (const f32x4_t*)(og + (size_t)qi * D);
#pragma unroll
            for (int d = 0; d < D; d += 4) {
                const f32x4_t ov = orow[d / 4];
#pragma unroll
                for (int c = 0; c < 4; ++c) dr = __builtin_fmaf(dos[lane][d + c], ov[c], dr);
            }
            const size_t ri = (size_t)bh * p.Nq + qi;
            if (p.dlse) dr -= p.dlse[ri];
            const float l = p.lse[ri];
            if (l != -INFINITY) l2 = l * kLog2e;
        }
        row_l2[lane] = l2;
        row_dr[lane] = dr;
        if (qi < p.nq_pad) {
            const size_t si = (size_t)bh * p.nq_pad + qi;
            p.stats[si] = l2;
            p.stats[(size_t)p.B * p.H * p.nq_pad + si] = dr;
        }
    }
    __syncthreads();

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const int q_last = min(p.Nq, q0 + BQF) - 1;
    const int kv_end = min(kv_valid, attn::bwd_key_hi<WIN>(p, q_last, kv_valid));
    const int kv_begin = max(0, attn::bwd_key_lo<WIN>(p, q0)) / TF * TF;
    const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + TF - 1) / TF : 0;
    const int lo = attn::bwd_key_lo<WIN>(p, qi), hi = attn::bwd_key_hi<WIN>(p, qi, kv_valid);
    const float c2 = p.scale_log2;
    const float l2 = row_l2[lane], dr = row_dr[lane];
    float* const ks = &kv[wave][0][0][0];
    float* const vs = &kv[wave][1][0][0];

    float dq[D];
#pragma unroll
    for (int d = 0; d < D; ++d) dq[d] = 0.f;

    // Round r: wave w takes key tile r * NWB + w; the barriers keep the waves in rounds.
    for (int t0 = 0; t0 < n_tiles; t0 += NWB) {
        const int t = t0 + wave;
        const int j0 = kv_begin + t * TF;
        __syncthreads();
        if (t < n_tiles) {
            load_rows<D>(ks, kg, j0, kv_valid, lane);
            load_rows<D>(vs, vg, j0, kv_valid, lane);
        }
        __syncthreads();
        if (t >= n_tiles) continue;

        // S and dP for the tile's 16 keys: 32 independent accumulators, K and V as broadcasts
        float s[TF], dp[TF];
#pragma unroll
        for (int jj = 0; jj < TF; ++jj) s[jj] = dp[jj] = 0.f;
#pragma unroll 2
        for (int d = 0; d < D; d += 4) {
            f32x4_t kq[TF], vq[TF];
#pragma unroll
            for (int jj = 0; jj < TF; ++jj) {
                kq[jj] = *(const f32x4_t*)(ks + jj * D + d);
                vq[jj] = *(const f32x4_t*)(vs + jj * D + d);
            }
            const float q0v = qs[lane][d], q1v = qs[lane][d + 1], q2v = qs[lane][d + 2], q3v = qs[lane][d + 3];
            const float g0 = dos[lane][d], g1 = dos[lane][d + 1], g2 = dos[lane][d + 2], g3 = dos[lane][d + 3];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < TF; ++jj) {
                s[jj] = __builtin_fmaf(q0v, kq[jj][0], s[jj]);
                s[jj] = __builtin_fmaf(q1v, kq[jj][1], s[jj]);
                s[jj] = __builtin_fmaf(q2v, kq[jj][2], s[jj]);
                s[jj] = __builtin_fmaf(q3v, kq[jj][3], s[jj]);
                dp[jj] = __builtin_fmaf(g0, vq[jj][0], dp[jj]);
                dp[jj] = __builtin_fmaf(g1, vq[jj][1], dp[jj]);
                dp[jj] = __builtin_fmaf(g2, vq[jj][2], dp[jj]);
                dp[jj] = __builtin_fmaf(g3, vq[jj][3], dp[jj]);
            }
        }
        // dS = P (dP - Dr); keys the row cannot see get P = 0
        float ds[TF];
#pragma unroll
        for (int jj = 0; jj < TF; ++jj) {
            const int j = j0 + jj;
            const float pv = (j >= lo && j < hi) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[jj], c2, -l2)) : 0.f;
            ds[jj] = pv * (dp[jj] - dr);
        }
        // dQ += dS K
#pragma unroll
        for (int d = 0; d < D; d += 4) {
            f32x4_t kq[TF];
#pragma unroll
            for (int jj = 0; jj < TF; ++jj) kq[jj] = *(const f32x4_t*)(ks + jj * D + d);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < TF; ++jj) {
                dq[d] = __builtin_fmaf(ds[jj], kq[jj][0], dq[d]);
                dq[d + 1] = __builtin_fmaf(ds[jj], kq[jj][1], dq[d + 1]);
                dq[d + 2] = __builtin_fmaf(ds[jj], kq[jj][2], dq[d + 2]);
                dq[d + 3] = __builtin_fmaf(ds[jj], kq[jj][3], dq[d + 3]);
            }
        }
    }

    // dQ = scale * (sum over the waves): waves NWB-1 .. 1 add into LDS in turn, wave 0 stores.
    __syncthreads();
    float (*const acc)[D + 1] = reinterpret_cast<float (*)[D + 1]>(&kv[0][0][0][0]);
    for (int w = NWB - 1; w >= 1; --w) {
        if (wave == w) {
#pragma unroll
            for (int d = 0; d < D; ++d) acc[lane][d] = (w == NWB - 1 ? 0.f : acc[lane][d]) + dq[d];
        }
        __syncthreads();
    }
    if (wave == 0 && qi < p.Nq) {
        float* dqg = (float*)p.dq + qbase + (size_t)qi * D;
#pragma unroll
        for (int d = 0; d < D; d += 4)
            *(float4*)(dqg + d) = make_float4(p.scale * (acc[lane][d] + dq[d]), p.scale * (acc[lane][d + 1] + dq[d + 1]),
                                              p.scale * (acc[lane][d + 2] + dq[d + 2]), p.scale * (acc[lane][d + 3] + dq[d + 3]));
    }
}

// ------------------------------------------------------------------------------------ dK, dV
template <int D, bool WIN>
__global__ void __launch_bounds__(64 * NWB) attn_bwd_f32_dkdv_kernel(attn::BwdParams p) {
    constexpr int DQ = D / 4;  // columns per lane
    __shared__ float rows[NWB][2][TF][D];  // each wave's Q and dO tile; the final sums reuse it
    __shared__ float stl2[NWB][TF], stdr[NWB][TF];
    static_assert(NWB * 2 * TF * D >= 2 * 64 * (DQ + 1), "reduction buffer does not fit");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kk = lane >> 2, part = lane & 3;  // key within the tile, quarter of the columns
    const int blk = attn::xcd_remap(blockIdx.x, p.n_blocks_k, p.n_ktiles);
    const int bh = blk / p.n_ktiles;
    const int kt_idx = blk - bh * p.n_ktiles;
    const int b = bh / p.H;
    const int k0 = kt_idx * BKF;
    const int kj = k0 + kk;

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const size_t kbase = (size_t)bh * p.Nk * D;
    const size_t qbase = (size_t)bh * p.Nq * D;
    const float ksign = p.negate ? -1.f : 1.f;  // a negative scale moves onto K

    float kr[DQ], vr[DQ], dk[DQ], dv[DQ];
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        f32x4_t a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
        if (kj < p.Nk) {
            a = *(const f32x4_t*)((const float*)p.k + kbase + (size_t)kj * D + part * DQ + d);
            c = *(const f32x4_t*)((const float*)p.v + kbase + (size_t)kj * D + part * DQ + d);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kr[d + e] = ksign * a[e];
            vr[d + e] = c[e];
            dk[d + e] = 0.f;
            dv[d + e] = 0.f;
        }
    }

    // Row tiles [t_begin, t_end) hold every row that may see a key of this workgroup.
    const int k_last = min(kv_valid, k0 + BKF) - 1;
    const int r_begin = k0 < kv_valid ? min(attn::bwd_row_lo<WIN>(p, k0), p.Nq) / TF * TF : 0;
    const int r_end = k0 < kv_valid ? attn::bwd_row_hi<WIN>(p, k_last) : 0;
    const int n_tiles = r_end > r_begin ? (r_end - r_begin + TF - 1) / TF : 0;
    const float c2 = p.scale_log2;
    const float* const plane_l2 = p.stats + (size_t)bh * p.nq_pad;
    const float* const plane_dr = p.stats + (size_t)p.B * p.H * p.nq_pad + (size_t)bh * p.nq_pad;
    float* const qt = &rows[wave][0][0][0];
    float* const dt = &rows[wave][1][0][0];

    for (int t0 = 0; t0 < n_tiles; t0 += NWB) {
        const int t = t0 + wave;
        const int i0 = r_begin + t * TF;
        __syncthreads();
        if (t < n_tiles) {
            load_rows<D>(qt, (const float*)p.q + qbase, i0, p.Nq, lane);
            load_rows<D>(dt, (const float*)p.dout + qbase, i0, p.Nq, lane);
            if (lane < TF) {
                const int i = i0 + lane;
                stl2[wave][lane] = i < p.Nq ? plane_l2[i] : INFINITY;
                stdr[wave][lane] = i < p.Nq ? plane_dr[i] : 0.f;
            }
        }
        __syncthreads();
        if (t >= n_tiles) continue;

        // partial S and dP of this lane's quarter for the tile's 16 rows, then the four quarters meet
        float s[TF], dp[TF];
#pragma unroll
        for (int r = 0; r < TF; ++r) {
            float a = 0.f, c = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; d += 4) {
                const f32x4_t qv = *(const f32x4_t*)(qt + r * D + part * DQ + d);
                const f32x4_t gv = *(const f32x4_t*)(dt + r * D + part * DQ + d);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a = __builtin_fmaf(qv[e], kr[d + e], a);
                    c = __builtin_fmaf(gv[e], vr[d + e], c);
                }
            }
            s[r] = a;
            dp[r] = c;
        }
#pragma unroll
        for (int r = 0; r < TF; ++r) {
            s[r] += __shfl_xor(s[r], 1);
            dp[r] += __shfl_xor(dp[r], 1);
            s[r] += __shfl_xor(s[r], 2);
            dp[r] += __shfl_xor(dp[r], 2);
        }
        // P and dS; the rows that cannot see the key get P = 0
        float pr[TF], dsr[TF];
#pragma unroll
        for (int r = 0; r < TF; ++r) {
            const int i = i0 + r;
            const bool vis = kj < kv_valid && kj >= attn::bwd_key_lo<WIN>(p, i) &&
                             kj < attn::bwd_key_hi<WIN>(p, i, kv_valid);
            const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -stl2[wave][r])) : 0.f;
            pr[r] = pv;
            dsr[r] = pv * (dp[r] - stdr[wave][r]);
        }
        // dK += dS Q, dV += P dO over this lane's quarter of the columns
#pragma unroll
        for (int r = 0; r < TF; ++r) {
#pragma unroll
            for (int d = 0; d < DQ; d += 4) {
                const f32x4_t qv = *(const f32x4_t*)(qt + r * D + part * DQ + d);
                const f32x4_t gv = *(const f32x4_t*)(dt + r * D + part * DQ + d);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dk[d + e] = __builtin_fmaf(dsr[r], qv[e], dk[d + e]);
                    dv[d + e] = __builtin_fmaf(pr[r], gv[e], dv[d + e]);
                }
            }
        }
    }

    // dK = scale * (sum over the waves), dV = sum: waves NWB-1 .. 1 add into LDS in turn, wave 0 stores.
    __syncthreads();
    float (*const ak)[DQ + 1] = reinterpret_cast<float (*)[DQ + 1]>(&rows[0][0][0][0]);
    float (*const av)[DQ + 1] = ak + 64;
    for (int w = NWB - 1; w >= 1; --w) {
        if (wave == w) {
#pragma unroll
            for (int d = 0; d < DQ; ++d) {
                ak[lane][d] = (w == NWB - 1 ? 0.f : ak[lane][d]) + dk[d];
                av[lane][d] = (w == NWB - 1 ? 0.f : av[lane][d]) + dv[d];
            }
        }
        __syncthreads();
    }
    if (wave == 0 && kj < p.Nk) {
        float* dkg = (float*)p.dk + kbase + (size_t)kj * D + part * DQ;
        float* dvg = (float*)p.dv + kbase + (size_t)kj * D + part * DQ;
#pragma unroll
        for (int d = 0; d < DQ; d += 4) {
            *(float4*)(dkg + d) = make_float4(p.scale * (ak[lane][d] + dk[d]), p.scale * (ak[lane][d + 1] + dk[d + 1]),
                                              p.scale * (ak[lane][d + 2] + dk[d + 2]), p.scale * (ak[lane][d + 3] + dk[d + 3]));
            *(float4*)(dvg + d) = make_float4(av[lane][d] + dv[d], av[lane][d + 1] + dv[d + 1],
                                              av[lane][d + 2] + dv[d + 2], av[lane][d + 3] + dv[d + 3]);
        }
    }
}

template <int D, bool WIN>
hipError_t launch_two(const attn::BwdParams& p, hipStream_t stream) {
    attn::BwdParams pc = p;
    void* args[] = {&pc};
    hipError_t e = hipLaunchKernel((const void*)attn_bwd_f32_dq_kernel<D, WIN>, dim3(p.n_blocks_q),
                                   dim3(64 * NWB), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel((const void*)attn_bwd_f32_dkdv_kernel<D, WIN>, dim3(p.n_blocks_k), dim3(64 * NWB),
                           args, 0, stream);
}

template <int D>
hipError_t launch_one(const attn::BwdParams& p, hipStream_t stream) {
    return p.window >= 0 ? launch_two<D, true>(p, stream) : launch_two<D, false>(p, stream);
}

}  // namespace

int attn_bwd_f32_q_block() { return BQF; }
int attn_bwd_f32_k_block() { return BKF; }

hipError_t attn_launch_bwd_f32(const attn::BwdParams& p, int D, hipStream_t stream) {
    return D == 128 ? launch_one<128>(p, stream) : launch_one<64>(p, stream);
}

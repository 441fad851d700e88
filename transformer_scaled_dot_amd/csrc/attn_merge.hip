// attn_merge.hip -- combine the partial results of a key-split launch.
//
// Split s of a query row holds O_s (normalised over the split's keys) and LSE_s (natural log of
// the split's sum of exponentials).  The row's result over all keys is
//     LSE = ln sum_s e^{LSE_s},   O = sum_s e^{LSE_s - LSE} O_s
// -- the log-sum-exp merge of partial softmax results (the row-wise max shift and
// log-sum-exp of the aicoding.csdn.net page, sec.2.2, applied to per-split sums).  A split that
// saw no valid key has LSE_s = -inf and weight 0; a row with no valid key at all gets O = 0 and
// LSE = -inf, as in the unsplit kernels.
#include "attn_common.h"

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int NT = 256;  // threads per row

// One workgroup per query row.  Every thread owns one float4 column of O and every
// (NT / (D/4))-th split, and requests its partial-O values first, so that all of a row's loads
// are in flight while wave 0 turns the splits' LSEs (one per lane, S <= 64) into normalised
// weights w_s = e^{LSE_s - LSE}; the per-group weighted sums then meet in LDS.
template <typename T, int D>
__global__ void __launch_bounds__(NT) attn_merge_kernel(attn::Params p) {
    constexpr int C4 = D / 4;     // float4 columns per row
    constexpr int NG = NT / C4;   // split groups
    __shared__ float wsh[64];
    __shared__ float4 red[NG][C4];

    const int tid = threadIdx.x;
    const size_t row = blockIdx.x;  // (b * H + h) * Nq + i
    const size_t plane = (size_t)p.B * p.H * p.Nq;
    const int S = p.n_splits;

    constexpr int KS = 64 / NG;  // splits per thread
    const int g = tid / C4, c = tid - g * C4;
    float4 v[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int sp = g + k * NG;
        v[k] = sp < S ? *((const float4*)(p.o_part + (sp * plane + row) * D) + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    if (tid < 64) {
        const float ls = tid < S ? p.lse_part[tid * plane + row] : -INFINITY;
        float m = ls;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        const float e = (tid < S && m != -INFINITY) ? __builtin_amdgcn_exp2f((ls - m) * kLog2e) : 0.f;
        float l = e;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
        wsh[tid] = l > 0.f ? e / l : 0.f;
        if (tid == 0) p.lse[row] = l > 0.f ? m + __builtin_amdgcn_logf(l) * attn::kLn2 : -INFINITY;
    }
    __syncthreads();

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int sp = g + k * NG;
        if (sp < S) {
            const float w = wsh[sp];
            acc.x = __builtin_fmaf(w, v[k].x, acc.x);
            acc.y = __builtin_fmaf(w, v[k].y, acc.y);
            acc.z = __builtin_fmaf(w, v[k].z, acc.z);
            acc.w = __builtin_fmaf(w, v[k].w, acc.w);
        }
    }
    red[g][c] = acc;
    __syncthreads();
    if (tid < D) {
        const float* rf = (const float*)&red[0][0];
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k) o += rf[k * D + tid];
        ((T*)p.o)[row * D + tid] = (T)o;
    }
}

template <typename T, int D>
hipError_t launch_one(const attn::Params& p, hipStream_t stream) {
    attn::Params pc = p;
    void* args[] = {&pc};
    return hipLaunchKernel((const void*)attn_merge_kernel<T, D>,
                           dim3((unsigned)((size_t)p.B * p.H * p.Nq)), dim3(NT), args, 0, stream);
}

}  // namespace

hipError_t attn_launch_merge(const attn::Params& p, int dtype, int D, hipStream_t stream) {
    if (dtype == 2) return D == 128 ? launch_one<__bf16, 128>(p, stream) : launch_one<__bf16, 64>(p, stream);
    if (dtype == 1) return D == 128 ? launch_one<_Float16, 128>(p, stream) : launch_one<_Float16, 64>(p, stream);
    return D == 128 ? launch_one<float, 128>(p, stream) : launch_one<float, 64>(p, stream);
}

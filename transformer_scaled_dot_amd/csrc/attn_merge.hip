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

template <typename T, int D>
__global__ void __launch_bounds__(64) attn_merge_kernel(attn::Params p) {
    constexpr int PER = D / 64;  // output elements per lane
    const int lane = threadIdx.x;
    const size_t row = blockIdx.x;  // (b * H + h) * Nq + i
    const size_t plane = (size_t)p.B * p.H * p.Nq;
    const int S = p.n_splits;  // <= 64: one split per lane

    const float ls = lane < S ? p.lse_part[lane * plane + row] : -INFINITY;
    float m = ls;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float w = (lane < S && m != -INFINITY) ? __builtin_amdgcn_exp2f((ls - m) * kLog2e) : 0.f;
    float l = w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);

    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s = 0; s < S; ++s) {
        const float ws = __shfl(w, s);
        if (ws == 0.f) continue;  // the same on every lane
        const float* op = p.o_part + (s * plane + row) * D;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(ws, op[lane + 64 * e], acc[e]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T* og = (T*)p.o + row * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) og[lane + 64 * e] = (T)(acc[e] * inv);
    if (lane == 0) p.lse[row] = l > 0.f ? m + __builtin_amdgcn_logf(l) * attn::kLn2 : -INFINITY;
}

template <typename T, int D>
hipError_t launch_one(const attn::Params& p, hipStream_t stream) {
    attn::Params pc = p;
    void* args[] = {&pc};
    return hipLaunchKernel((const void*)attn_merge_kernel<T, D>,
                           dim3((unsigned)((size_t)p.B * p.H * p.Nq)), dim3(64), args, 0, stream);
}

}  // namespace

hipError_t attn_launch_merge(const attn::Params& p, int dtype, int D, hipStream_t stream) {
    if (dtype == 2) return D == 128 ? launch_one<__bf16, 128>(p, stream) : launch_one<__bf16, 64>(p, stream);
    if (dtype == 1) return D == 128 ? launch_one<_Float16, 128>(p, stream) : launch_one<_Float16, 64>(p, stream);
    return D == 128 ? launch_one<float, 128>(p, stream) : launch_one<float, 64>(p, stream);
}

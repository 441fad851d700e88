// attn_common.h -- types shared by the HIP kernels and their host launcher (HIP path only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Everything a kernel needs about one call.  Sizes are validated on the host.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* key_lens;  // device int32[B] or nullptr
    int B, H, Nq, Nk;
    int n_qtiles;      // ceil(Nq / BM) for the kernel's BM
    int n_blocks;      // n_qtiles * H * B
    float scale_log2;  // max(|scale| * log2(e), 1e-30): logits are handled in base-2 units
    int negate_q;      // scale < 0: the sign is moved onto Q (an exact bit flip)
    int causal;
    int causal_br;     // causal mask aligned bottom-right: query i keeps keys j <= i + L_b - Nq
    int window;        // half-width w of the local band |i - j| <= w, or -1 for none
    int xcd_interleave;  // groups each XCD alternates between (xcd_remap); 1 = one at a time
    // Key-range split: each (Q tile, b, h) is spread over n_splits workgroups, split s taking
    // keys [s * split_len, (s + 1) * split_len).  With n_splits > 1 the workgroups write fp32
    // partial results (O normalised over the split's keys, LSE of the split) to o_part
    // [n_splits, B, H, Nq, D] and lse_part [n_splits, B, H, Nq]; a merge kernel combines them.
    int n_splits;
    int split_len;
    float* o_part;
    float* lse_part;
};

// Which (split, b*H + h, Q tile) a workgroup owns; splits of one Q tile are adjacent in the
// logical order.
struct BlockWork {
    int split, bh, qt;
};
__host__ __device__ __forceinline__ BlockWork block_work(const Params& p, int blk) {
    BlockWork w;
    w.split = blk % p.n_splits;
    const int rest = blk / p.n_splits;
    w.bh = rest / p.n_qtiles;
    w.qt = rest - w.bh * p.n_qtiles;
    return w;
}

// Keys [lo, hi) that row i may attend to, within the valid length: the causal rule keeps
// j <= i (top-left), or j <= i + L_b - Nq when the queries are the last Nq positions of a
// cached sequence of length L_b (bottom-right); the local band keeps |i - j| <= w.
__device__ __forceinline__ int row_key_lo(const Params& p, int i) {
    return p.window >= 0 ? i - p.window : 0;
}
__device__ __forceinline__ int row_key_hi(const Params& p, int i, int kv_valid) {
    int hi = kv_valid;
    if (p.causal) hi = min(hi, i + 1 + (p.causal_br ? kv_valid - p.Nq : 0));
    if (p.window >= 0) hi = min(hi, i + p.window + 1);
    return hi;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD i % 8).  In the
// logical order every `group` consecutive items share one (b, h), and with it the stream of K/V
// (or Q/dO) tiles.  Whole groups are dealt round-robin over the XCDs: XCD x walks groups x, x + 8,
// x + 16, ... in turn, so that a group runs on one XCD at about the same time and shares that
// XCD's L2, while groups of unequal work (padded or ragged sequence lengths, which vary with b)
// spread evenly over the XCDs instead of one XCD taking a run of whole batches.  With
// `interleave` = P > 1 (P dividing the XCD's group count), the XCD walks its groups P at a time
// and alternates between them item by item: with causal Q tiles ordered longest first inside a
// group, the XCD then starts the P longest tiles of P heads before any shorter one, and the
// shortest tiles of the last heads fill the end instead of a few long ones running alone.  With a
// group count that is not a multiple of 8, each XCD walks one contiguous range of the logical
// order (or the identity order when n itself is not a multiple of 8).  n must be a multiple of
// group.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int n, int group, int interleave = 1) {
    if (((n / group) & 7) == 0) {
        const int x = bid & 7, k = bid >> 3;
        const int P = interleave;
        if (P > 1 && ((n / group / 8) % P) == 0) {
            const int chunk = k / (P * group), w = k - chunk * P * group;
            const int item = w / P, sub = w - item * P;
            return (((chunk * P + sub) << 3) + x) * group + item;
        }
        const int gi = k / group, within = k - gi * group;
        return ((gi << 3) + x) * group + within;
    }
    if ((n & 7) != 0) return bid;
    return (bid & 7) * (n >> 3) + (bid >> 3);
}

__device__ __forceinline__ int clamp_len(const int32_t* key_lens, int b, int Nk) {
    if (!key_lens) return Nk;
    int L = key_lens[b];
    return L < 0 ? 0 : (L > Nk ? Nk : L);
}

constexpr float kLn2 = 0.693147180559945309417f;

}  // namespace attn

// Launchers, one per kernel family (defined in their .hip files).
hipError_t attn_launch_mfma(const attn::Params& p, int dtype, int D, hipStream_t stream);
hipError_t attn_launch_f32(const attn::Params& p, int D, hipStream_t stream);
hipError_t attn_launch_merge(const attn::Params& p, int dtype, int D, hipStream_t stream);
int attn_mfma_block_m();
int attn_f32_block_m();

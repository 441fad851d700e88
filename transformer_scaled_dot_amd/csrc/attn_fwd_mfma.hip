// attn_fwd_mfma.hip -- fused attention forward for bf16 / fp16 on gfx950 matrix cores.
//
// The tiled loop of the pages (hotelren.com page on attention, sec.4.1: per Q tile, stream the
// K/V tiles, form the scores on chip, normalise online, accumulate P V, never store S; ch.5:
// load only the K/V tiles a Q tile can see) laid out for CDNA4:
//
//   * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32 rows;
//   * K/V tiles of 64 keys go HBM -> registers -> LDS (double buffered, one barrier per tile);
//   * both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation, arranged so
//     that a lane always holds one query row:
//        S^T = K Q^T   (A = K tile from LDS, B = Q^T kept in registers for the whole loop)
//        O^T = V^T P^T (A = V^T tile from LDS, B = P^T taken straight from the S^T accumulator)
//     The 32x32 accumulator gives lane l the column l%32 (the query) and 16 rows (keys); the K
//     rows are fed to the MFMA with bits 2 and 3 of the row index swapped, which makes each
//     lane's 8-register halves hold 8 consecutive keys -- exactly the B-operand layout of the
//     next MFMA, so P never moves between lanes;
//   * the softmax runs per lane in base-2 units (logit * scale * log2 e) with fp32 running
//     max and sum; the two lanes that share a query row swap maxima once per tile and sums
//     once at the end;
//   * tiles beyond a row's last valid key are never loaded (causal and key padding); masks
//     are evaluated only on the tiles that straddle a boundary.
#include "attn_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
    using vec8 = bf16x8_t;
    static __device__ __forceinline__ f32x16_t mma(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<_Float16> {
    using vec8 = f16x8_t;
    static __device__ __forceinline__ f32x16_t mma(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per K/V tile
constexpr unsigned kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data, gfx9-family layout

// Row permutation of the K operand: swap bits 2 and 3 of a 0..31 row index (an involution).
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// XOR swizzles of the 16-byte chunk index, chosen so that the 32 lanes of a half-wave that
// read one MFMA operand (one chunk column, 32 different rows) hit distinct LDS banks whether
// the LDS serves 8 or 16 lanes of a 128-bit read per clock.
template <int D>
__device__ __forceinline__ int kswz(int r) {  // r: lane row 0..31 of the A operand
    return D == 128 ? (r & 15) : (((r >> 1) & 7) ^ ((r & 1) << 2));
}
__device__ __forceinline__ int vswz(int d) { return ((d >> 1) & 7) ^ ((d & 1) << 2); }

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::vec8 to_vec8(u32x4_t x) {
    return __builtin_bit_cast(typename Mfma<T>::vec8, x);
}

// 8 fp32 values -> 8 x T, round to nearest even.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::vec8 cvt8(const f32x16_t& s, int base) {
    typename Mfma<T>::vec8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (T)s[base + i];
    return r;
}

template <typename T>
__device__ __forceinline__ unsigned short bits16(T x) {
    return __builtin_bit_cast(unsigned short, x);
}

template <typename T, int D>
__global__ void __launch_bounds__(NT, 2) attn_fwd_mfma_kernel(attn::Params p) {
    using M = Mfma<T>;
    constexpr int NCH = D / 8;             // 16-byte chunks per K/V row
    constexpr int KSTEPS = D / 16;         // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;             // 32-row tiles of O^T
    constexpr int KT = BN / 32;            // 32-key tiles of S^T
    constexpr int K_LOADS = BN * NCH / NT; // 16-byte K chunks per thread per tile
    constexpr int V_ITEMS = (BN / 2) * NCH / NT;  // (key pair, chunk) items per thread per tile
    constexpr int TILE_BYTES = BN * D * 2;
    static_assert(K_LOADS >= 1 && V_ITEMS >= 1, "tile too small for the workgroup");

    __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TILE_BYTES];  // K[2], V^T[2]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, g = lane >> 5;

    const int blk = attn::xcd_remap(blockIdx.x, p.n_blocks);
    const int bh = blk / p.n_qtiles;
    int qt = blk - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest rows first
    const int b = bh / p.H;
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + r;

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    int kv_end = kv_valid;
    if (p.causal) kv_end = min(kv_end, min(p.Nq, q0 + BM));
    const int n_tiles = (kv_end + BN - 1) / BN;

    const T* qg = (const T*)p.q + (size_t)bh * p.Nq * D;
    const T* kg = (const T*)p.k + (size_t)bh * p.Nk * D;
    const T* vg = (const T*)p.v + (size_t)bh * p.Nk * D;
    // Out-of-range buffer reads return 0: rows past Nq, and keys past the valid length.
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)qg, 0, p.Nq * D * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, kv_valid * D * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, kv_valid * D * 2, kBufferWord3);

    // Q^T operand: lane (r, g) holds Q[qi][16 ks + 8 g .. +7] for every k-step.
    typename M::vec8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4_t x = buf_load16(qrs, (qi * D + 16 * ks + 8 * g) * 2);
        if (p.negate_q) x ^= 0x80008000u;
        qf[ks] = to_vec8<T>(x);
    }

    u32x4_t kreg[K_LOADS];
    u32x4_t vreg[2 * V_ITEMS];

    auto load_tile = [&](int j0) {
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int c = tid + NT * i;
            const int row = c / NCH, ch = c % NCH;
            kreg[i] = buf_load16(krs, ((j0 + row) * D + ch * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < V_ITEMS; ++i) {
            const int c = tid + NT * i;
            const int pr = c % 32, dc = c / 32;
            vreg[2 * i] = buf_load16(vrs, ((j0 + 2 * pr) * D + dc * 8) * 2);
            vreg[2 * i + 1] = buf_load16(vrs, ((j0 + 2 * pr + 1) * D + dc * 8) * 2);
        }
    };

    auto store_tile = [&](int buf) {
        unsigned char* kl = smem + buf * TILE_BYTES;
        unsigned char* vl = smem + (2 + buf) * TILE_BYTES;
#pragma unroll
        for (int i = 0; i < K_LOADS; ++i) {
            const int c = tid + NT * i;
            const int row = c / NCH, ch = c % NCH;
            const int phys = ch ^ kswz<D>(swap23(row & 31));
            *(u32x4_t*)(kl + row * (D * 2) + phys * 16) = kreg[i];
        }
        // V is stored transposed, V^T[d][key], so the O^T operand reads 8 consecutive keys.
#pragma unroll
        for (int i = 0; i < V_ITEMS; ++i) {
            const int c = tid + NT * i;
            const int pr = c % 32, dc = c / 32;
            const u32x4_t x0 = vreg[2 * i], x1 = vreg[2 * i + 1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned a = x0[e >> 1], bb = x1[e >> 1];
                const unsigned w = (e & 1) ? ((a >> 16) | (bb & 0xffff0000u))
                                           : ((a & 0xffffu) | (bb << 16));
                const int d = dc * 8 + e;
                const int phys = (pr >> 2) ^ vswz(d);
                *(unsigned*)(vl + d * (BN * 2) + phys * 16 + (pr & 3) * 4) = w;
            }
        }
    };

    f32x16_t oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16_t{};
    float m_run = -INFINITY;  // running max of this row, base-2 units
    float l_run = 0.f;        // this lane's share of the running sum

    const float c2 = p.scale_log2;
    const int kswz_r = kswz<D>(r);
    const int vswz_r = vswz(r);
    const bool wave_has_rows = qw0 < p.Nq;

    if (n_tiles > 0) load_tile(0);
    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        store_tile(buf);
        __syncthreads();
        if (it + 1 < n_tiles) load_tile((it + 1) * BN);

        const int j0 = it * BN;
        const bool active = wave_has_rows && !(p.causal && j0 > qw0 + 31);
        if (!active) continue;

        const unsigned char* kl = smem + buf * TILE_BYTES;
        const unsigned char* vl = smem + (2 + buf) * TILE_BYTES;

        // ---- S^T = K Q^T: 32 keys x 32 queries per accumulator
        f32x16_t s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16_t{};
            const unsigned char* krow = kl + (swap23(r) + 32 * kt) * (D * 2);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const u32x4_t a = *(const u32x4_t*)(krow + (((2 * ks + g) ^ kswz_r) * 16));
                s[kt] = M::mma(to_vec8<T>(a), qf[ks], s[kt]);
            }
        }

        // ---- online softmax.  Register i of s[kt] holds key j0 + 32 kt + 16 (i/8) + 8 g + i%8.
        const bool need_mask = (j0 + BN > kv_valid) || (p.causal && j0 + BN - 1 > qw0);
        float mt = -INFINITY;
        if (need_mask) {
            const int lim = p.causal ? min(kv_valid, qi + 1) : kv_valid;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = j0 + 32 * kt + 16 * (i >> 3) + 8 * g + (i & 7);
                    const float t = j < lim ? s[kt][i] * c2 : -INFINITY;
                    s[kt][i] = t;
                    mt = fmaxf(mt, t);
                }
        } else {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
            mt = mx * c2;
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float ls = 0.f;
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = __builtin_amdgcn_exp2f(s[kt][i] - m_use);
                    s[kt][i] = e;
                    ls += e;
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c2, -m_use));
                    s[kt][i] = e;
                    ls += e;
                }
        }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[t] *= alpha;

        // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
        for (int h16 = 0; h16 < BN / 16; ++h16) {
            const typename M::vec8 pb = cvt8<T>(s[h16 >> 1], 8 * (h16 & 1));
            const int vch = (2 * h16 + g) ^ vswz_r;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const u32x4_t a = *(const u32x4_t*)(vl + (32 * t + r) * (BN * 2) + vch * 16);
                oacc[t] = M::mma(to_vec8<T>(a), pb, oacc[t]);
            }
        }
    }

    // ---- epilogue: O = O / l (rounded to T), LSE = ln 2 * (m + log2 l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi < p.Nq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        T* og = (T*)p.o + ((size_t)bh * p.Nq + qi) * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // accumulator registers 4a..4a+3 hold O[qi][32 t + 8 a + 4 g + 0..3]
                const unsigned w0 = bits16((T)(oacc[t][4 * a + 0] * inv)) |
                                    ((unsigned)bits16((T)(oacc[t][4 * a + 1] * inv)) << 16);
                const unsigned w1 = bits16((T)(oacc[t][4 * a + 2] * inv)) |
                                    ((unsigned)bits16((T)(oacc[t][4 * a + 3] * inv)) << 16);
                uint2* dst = (uint2*)(og + 32 * t + 8 * a + 4 * g);
                *dst = make_uint2(w0, w1);
            }
        if (g == 0)
            p.lse[(size_t)bh * p.Nq + qi] =
                l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * attn::kLn2 : -INFINITY;
    }
}

template <typename T, int D>
hipError_t launch_one(const attn::Params& p, hipStream_t stream) {
    attn::Params pc = p;
    void* args[] = {&pc};
    return hipLaunchKernel((const void*)attn_fwd_mfma_kernel<T, D>, dim3(p.n_blocks), dim3(NT),
                           args, 0, stream);
}

}  // namespace

int attn_mfma_block_m() { return BM; }

hipError_t attn_launch_mfma(const attn::Params& p, int dtype, int D, hipStream_t stream) {
    if (dtype == 2) return D == 128 ? launch_one<__bf16, 128>(p, stream) : launch_one<__bf16, 64>(p, stream);
    return D == 128 ? launch_one<_Float16, 128>(p, stream) : launch_one<_Float16, 64>(p, stream);
}

// attn_bwd_mfma.hip -- attention backward (dQ, dK, dV) for bf16 / fp16 on gfx950 matrix cores.
//
// The gradients of O = softmax(scale Q K^T + mask) V and LSE, given dO and dLSE, are
//   P  = exp(scale Q K^T - LSE)          (rebuilt from the forward's LSE, never stored)
//   dV = P^T dO,  dP = dO V^T,  Dr_i = rowsum(dO * O)_i - dLSE_i,  dS = P * (dP - Dr)
//   dQ = scale dS K,  dK = scale dS^T Q
// -- the backward that rebuilds the softmax output from the forward's statistics instead of
// keeping the N x N matrix (hotelren.com page on attention, sec.4.2; aicoding.csdn.net page,
// ch.1: the backward needs the softmax output).  Two kernels, no atomics:
//
//   attn_bwd_dq_kernel   one workgroup per 128-row Q tile (lane = query, as in the forward):
//                        Dr for its rows (written to the workspace), then for every visible
//                        64-key K/V tile  S^T = K Q^T,  dP^T = V dO^T,  dQ^T += K^T dS^T.
//   attn_bwd_dkdv_kernel one workgroup per 128-key tile (lane = key): K and V stay in registers,
//                        32-row Q/dO tiles stream through LDS;  S = Q K^T,  dP = dO V^T,
//                        dV^T += dO^T P,  dK^T += Q^T dS.
//
// Each streamed tile is read both by rows (A operand of the score-like products) and
// transposed (A operand of the gradient products, LDS transpose read), so its 16-byte chunks are
// XOR-swizzled with one function of the row that keeps both access patterns free of bank
// conflicts.  Every product runs on v_mfma_f32_32x32x16 with fp32 accumulation; the rows of the
// streamed A operand are fed with bits 2 and 3 of the row index swapped, so the accumulator of
// S (or dP) already has the B-operand layout of the next product, as in the forward kernel.
#include "attn_bwd.h"
#include "attn_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
    using vec8 = bf16x8_t;
    static __device__ __forceinline__ f32x16_t mma(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mma<_Float16> {
    using vec8 = f16x8_t;
    static __device__ __forceinline__ f32x16_t mma(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int NT = 256;    // threads per workgroup (4 waves)
constexpr int BMQ = 128;   // dQ kernel: query rows per workgroup
constexpr int BNQ = 64;    // dQ kernel: keys per K/V tile
constexpr int BNK = 128;   // dK/dV kernel: keys per workgroup
constexpr int BMK = 64;    // dK/dV kernel: query rows per Q/dO tile
constexpr float kLog2e = 1.44269504088896340736f;
constexpr unsigned kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data, gfx9-family layout

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Chunk swizzle of a tile row that serves both the row read (32 rows, one chunk column per
// half-wave) and the transpose read (4 consecutive rows x 2 chunks per 16 lanes): for D = 128
// the two 2-bit halves of (row mod 16) are swapped into the chunk index; for D = 64 (8 chunks)
// bit 1 of the row flips chunk bit 2 and bits 2-3 of the row flip chunk bits 0-1.
template <int D>
__device__ __forceinline__ int dswz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) ^ ((row >> 2) & 3));
}

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

// One lane's 8 elements of a [rows, D] slice: row `row`, columns c0 .. c0+7 (zeros past `bytes`).
__device__ __forceinline__ u32x4_t load8(const void* base, int bytes, int off_bytes) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off_bytes, 0, 0);
}

// ------------------------------------------------------------------------------------ dQ
template <typename T, int D, bool WIN>
__global__ void __launch_bounds__(NT, 2) attn_bwd_dq_kernel(attn::BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    using M = Mma<T>;
    using vec8 = typename M::vec8;
    constexpr int BN = BNQ;
    constexpr int NCH = D / 8;              // 16-byte chunks per row
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int KT = BN / 32;
    constexpr int RB = D * 2;               // bytes per row
    constexpr int CPT = BN * NCH / NT;      // chunks per thread per tile
    constexpr int TILE = BN * RB;
    constexpr int STAGE = 2 * TILE;         // K tile then V tile
    static_assert(CPT >= 1, "tile too small for the workgroup");

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * STAGE];
    lds_u8* const smem = (lds_u8*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, g = lane >> 5;

    const int blk = attn::xcd_remap(blockIdx.x, p.n_blocks_q, p.n_qtiles);
    const int bh = blk / p.n_qtiles;
    int qt = blk - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest rows first
    const int b = bh / p.H;
    const int q0 = qt * BMQ;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + r;
    const bool row_ok = qi < p.Nq;
    const bool wave_has_rows = qw0 < p.Nq;

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const int q_last = min(p.Nq, q0 + BMQ) - 1;
    // key tiles [t_begin, n_tiles) hold every key some row of this workgroup may see
    const int kv_end = min(kv_valid, attn::bwd_key_hi<WIN>(p, q_last, kv_valid));
    const int t_begin = max(0, attn::bwd_key_lo<WIN>(p, q0)) / BN;
    const int n_tiles = (kv_end + BN - 1) / BN;

    const size_t qbase = (size_t)bh * p.Nq * D;
    const T* kg = (const T*)p.k + (size_t)bh * p.Nk * D;
    const T* vg = (const T*)p.v + (size_t)bh * p.Nk * D;
    const int qbytes = p.Nq * D * 2;

    // Q^T and dO^T operands: lane (r, g) holds row qi, columns 16 ks + 8 g .. +7; Dr from O.
    vec8 qf[KSTEPS], df[KSTEPS];
    float dr_part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int off = (qi * D + 16 * ks + 8 * g) * 2;
        u32x4_t xq = load8((const T*)p.q + qbase, qbytes, off);
        if (p.negate) xq ^= 0x80008000u;
        qf[ks] = __builtin_bit_cast(vec8, xq);
        df[ks] = __builtin_bit_cast(vec8, load8((const T*)p.dout + qbase, qbytes, off));
        const vec8 of = __builtin_bit_cast(vec8, load8((const T*)p.o + qbase, qbytes, off));
#pragma unroll
        for (int e = 0; e < 8; ++e) dr_part = __builtin_fmaf(to_f(df[ks][e]), to_f(of[e]), dr_part);
    }
    float dr = dr_part + __shfl_xor(dr_part, 32);
    float lse2 = INFINITY;  // rows past Nq (and rows that see no key) get P = 0
    if (row_ok) {
        const size_t ri = (size_t)bh * p.Nq + qi;
        if (p.dlse) dr -= p.dlse[ri];
        const float l = p.lse[ri];
        if (l != -INFINITY) lse2 = l * kLog2e;
    }
    if (g == 0 && qi < p.nq_pad) {
        const size_t si = (size_t)bh * p.nq_pad + qi;
        p.stats[si] = lse2;
        p.stats[(size_t)p.B * p.H * p.nq_pad + si] = dr;
    }

    // DMA offsets: slot (i*NT + tid) of a tile holds global chunk (row, chunk ^ dswz(row)).
    int toff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int s = i * NT + tid;
        const int row = s / NCH, phys = s % NCH;
        toff[i] = (row * D + (phys ^ dswz<D>(row)) * 8) * 2;
    }
    auto issue_tile = [&](const int tile, const int stage) {
        const int j0 = tile * BN;
        const int bytes = (kv_valid - j0) * D * 2;  // keys past the valid length arrive as zeros
        const __amdgpu_buffer_rsrc_t krs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kg + (size_t)j0 * D), 0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vg + (size_t)j0 * D), 0, bytes, kBufferWord3);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            lds_u8* kd = smem + stage * STAGE + (i * NT + wave * 64) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kd, 16, toff[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            lds_u8* vd = smem + stage * STAGE + TILE + (i * NT + wave * 64) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vd, 16, toff[i], 0, 0, 0);
        }
    };

    // Row reads (A of S^T and dP^T): row swap23(r) (+32 kt), chunk (2 ks + g) ^ dswz.
    int raddr[KSTEPS];
    {
        const int row = swap23(r);
        const int sw = dswz<D>(row);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) raddr[ks] = row * RB + (((2 * ks + g) ^ sw) * 16);
    }
    // Transpose reads (A of dQ^T = K^T dS^T): lane s of a 16-lane group names 8 bytes of row
    // 8 g + s/4 (+4 for the upper half, +16 h16) at columns 32 dt + 16 G + 4 (s & 3).
    int taddr_lo[DT], taddr_hi[DT];
    {
        const int s = lane & 15, G1 = (lane >> 4) & 1;
        const int rlo = 8 * g + (s >> 2), rhi = rlo + 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int c = 4 * dt + 2 * G1 + ((s & 3) >> 1);
            taddr_lo[dt] = rlo * RB + ((c ^ dswz<D>(rlo)) * 16) + 8 * (s & 1);
            taddr_hi[dt] = rhi * RB + ((c ^ dswz<D>(rhi)) * 16) + 8 * (s & 1);
        }
    }

    f32x16_t acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = f32x16_t{};
    const float c2 = p.scale_log2;

    auto do_tile = [&](const int it, const int stage) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (it + 1 < n_tiles) issue_tile(it + 1, stage ^ 1);

        const int j0 = it * BN;
        if (!wave_has_rows || j0 >= attn::bwd_key_hi<WIN>(p, qw0 + 31, kv_valid) || j0 + BN <= attn::bwd_key_lo<WIN>(p, qw0))
            return;
        const lds_u8* kb = smem + stage * STAGE;
        const lds_u8* vb = kb + TILE;

        f32x16_t s[KT], dp[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16_t{};
            dp[kt] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const u32x4_t a = *(const lds_u32x4*)(kb + raddr[ks] + kt * 32 * RB);
                s[kt] = M::mma(__builtin_bit_cast(vec8, a), qf[ks], s[kt]);
            }
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const u32x4_t a = *(const lds_u32x4*)(vb + raddr[ks] + kt * 32 * RB);
                dp[kt] = M::mma(__builtin_bit_cast(vec8, a), df[ks], dp[kt]);
            }
        }

        // Register i of s[kt] / dp[kt] holds key j0 + 32 kt + 16 (i/8) + 8 g + i%8.  The mask
        // matters only on tiles that reach past the valid keys or the wave's first row.
        const bool need_mask = j0 + BN > attn::bwd_key_hi<WIN>(p, qw0, kv_valid) || j0 < attn::bwd_key_lo<WIN>(p, qw0 + 31);
        if (need_mask) {
            const int lo = attn::bwd_key_lo<WIN>(p, qi), hi = attn::bwd_key_hi<WIN>(p, qi, kv_valid);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = j0 + 32 * kt + 16 * (i >> 3) + 8 * g + (i & 7);
                    const bool off = j < lo || j >= hi;
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c2, -lse2));
                    s[kt][i] = off ? 0.f : pv;
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c2, -lse2));
        }
        vec8 dsb[BN / 16];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) dsb[2 * kt + (i >> 3)][i & 7] = (T)(s[kt][i] * (dp[kt][i] - dr));

        // dQ^T += K^T dS^T, 16 keys per MFMA
#pragma unroll
        for (int h16 = 0; h16 < BN / 16; ++h16) {
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + taddr_lo[t] + 16 * h16 * RB));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + taddr_hi[t] + 16 * h16 * RB));
                const vec8 a = __builtin_bit_cast(vec8, u32x4_t{__builtin_bit_cast(u32x2_t, lo)[0],
                                                                 __builtin_bit_cast(u32x2_t, lo)[1],
                                                                 __builtin_bit_cast(u32x2_t, hi)[0],
                                                                 __builtin_bit_cast(u32x2_t, hi)[1]});
                acc[t] = M::mma(a, dsb[h16], acc[t]);
            }
        }
    };

    if (t_begin < n_tiles) issue_tile(t_begin, 0);
    for (int it = t_begin; it < n_tiles; it += 2) {
        do_tile(it, 0);
        if (it + 1 < n_tiles) do_tile(it + 1, 1);
    }

    // dQ = scale * acc; accumulator registers 4a..4a+3 of acc[t] hold dQ[qi][32 t + 8 a + 4 g + 0..3]
    if (row_ok) {
        T* dqg = (T*)p.dq + qbase + (size_t)qi * D;
        const float sc = p.scale;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u32x2_t w;
                w[0] = (unsigned)__builtin_bit_cast(unsigned short, (T)(acc[t][4 * a + 0] * sc)) |
                       ((unsigned)__builtin_bit_cast(unsigned short, (T)(acc[t][4 * a + 1] * sc)) << 16);
                w[1] = (unsigned)__builtin_bit_cast(unsigned short, (T)(acc[t][4 * a + 2] * sc)) |
                       ((unsigned)__builtin_bit_cast(unsigned short, (T)(acc[t][4 * a + 3] * sc)) << 16);
                *(u32x2_t*)(dqg + 32 * t + 8 * a + 4 * g) = w;
            }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------- dK, dV
template <typename T, int D, bool WIN>
__global__ void __launch_bounds__(NT, 1) attn_bwd_dkdv_kernel(attn::BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    using M = Mma<T>;
    using vec8 = typename M::vec8;
    constexpr int BM = BMK;                 // query rows per streamed tile
    constexpr int QB = BM / 32;             // 32-row blocks per tile
    constexpr int NCH = D / 8;
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int RB = D * 2;
    constexpr int CPT = BM * NCH / NT;
    constexpr int TILE = BM * RB;
    constexpr int SBYTES = 1024;            // row statistics: one 64-lane DMA of 16 bytes each
    constexpr int STAGE = 2 * TILE + SBYTES;  // Q tile, dO tile, LSE * log2(e) and Dr of its rows
    static_assert(CPT >= 1, "tile too small for the workgroup");
    static_assert(BM / 2 <= 64, "statistics DMA covers at most 64 chunks");

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * STAGE];
    lds_u8* const smem = (lds_u8*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, g = lane >> 5;

    const int blk = attn::xcd_remap(blockIdx.x, p.n_blocks_k, p.n_ktiles);
    const int bh = blk / p.n_ktiles;
    const int kt_idx = blk - bh * p.n_ktiles;
    const int b = bh / p.H;
    const int k0 = kt_idx * BNK;
    const int kw0 = k0 + wave * 32;
    const int kj = kw0 + r;  // this lane's key

    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const size_t kbase = (size_t)bh * p.Nk * D;
    const int kbytes = p.Nk * D * 2;
    const size_t qbase = (size_t)bh * p.Nq * D;
    const T* qg = (const T*)p.q + qbase;
    const T* dog = (const T*)p.dout + qbase;

    // Query tiles [t_begin, n_tiles) hold every row that may see a key of this workgroup.
    const int k_last = min(kv_valid, k0 + BNK) - 1;
    const int n_tiles = k0 < kv_valid ? (attn::bwd_row_hi<WIN>(p, k_last) + BM - 1) / BM : 0;
    const int t_begin = min(attn::bwd_row_lo<WIN>(p, k0), p.Nq) / BM;
    const bool wave_has_keys = kw0 < kv_valid;
    const int wave_row_lo = attn::bwd_row_lo<WIN>(p, kw0);
    const int wave_row_hi = attn::bwd_row_hi<WIN>(p, min(kw0 + 31, kv_valid - 1));

    // K^T and V^T operands: lane (r, g) holds key kj, columns 16 ks + 8 g .. +7.
    vec8 kf[KSTEPS], vf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int off = (kj * D + 16 * ks + 8 * g) * 2;
        u32x4_t xk = load8((const T*)p.k + kbase, kbytes, off);
        if (p.negate) xk ^= 0x80008000u;
        kf[ks] = __builtin_bit_cast(vec8, xk);
        vf[ks] = __builtin_bit_cast(vec8, load8((const T*)p.v + kbase, kbytes, off));
    }

    int toff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int s = i * NT + tid;
        const int row = s / NCH, phys = s % NCH;
        toff[i] = (row * D + (phys ^ dswz<D>(row)) * 8) * 2;
    }
    // Statistics DMA (wave 0): lanes 0 .. BM/4-1 fetch the tile's LSE * log2(e) in 4-row chunks,
    // lanes BM/4 .. BM/2-1 its Dr; the other lanes point past the buffer and write zeros.
    const int plane = p.B * p.H * p.nq_pad;
    const int stat_total = 2 * plane * 4;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)p.stats, 0, stat_total, kBufferWord3);
    const int soff = lane < BM / 4 ? (bh * p.nq_pad + 4 * lane) * 4
                     : lane < BM / 2 ? (plane + bh * p.nq_pad + 4 * (lane - BM / 4)) * 4
                                     : stat_total;
    auto issue_tile = [&](const int tile, const int stage) {
        const int i0 = tile * BM;
        const int bytes = (p.Nq - i0) * D * 2;  // rows past Nq arrive as zeros
        const __amdgpu_buffer_rsrc_t qrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(qg + (size_t)i0 * D), 0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t drs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(dog + (size_t)i0 * D), 0, bytes, kBufferWord3);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            lds_u8* qd = smem + stage * STAGE + (i * NT + wave * 64) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (__attribute__((address_space(3))) void*)qd, 16, toff[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            lds_u8* dd = smem + stage * STAGE + TILE + (i * NT + wave * 64) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)dd, 16, toff[i], 0, 0, 0);
        }
        if (wave == 0) {
            lds_u8* sd = smem + stage * STAGE + 2 * TILE;
            const int off = soff < stat_total ? soff + i0 * 4 : stat_total;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (__attribute__((address_space(3))) void*)sd, 16, off, 0, 0, 0);
        }
    };

    int raddr[KSTEPS];
    {
        const int row = swap23(r);
        const int sw = dswz<D>(row);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) raddr[ks] = row * RB + (((2 * ks + g) ^ sw) * 16);
    }
    int taddr_lo[DT], taddr_hi[DT];
    {
        const int s = lane & 15, G1 = (lane >> 4) & 1;
        const int rlo = 8 * g + (s >> 2), rhi = rlo + 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int c = 4 * dt + 2 * G1 + ((s & 3) >> 1);
            taddr_lo[dt] = rlo * RB + ((c ^ dswz<D>(rlo)) * 16) + 8 * (s & 1);
            taddr_hi[dt] = rhi * RB + ((c ^ dswz<D>(rhi)) * 16) + 8 * (s & 1);
        }
    }

    f32x16_t dka[DT], dva[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
        dka[t] = f32x16_t{};
        dva[t] = f32x16_t{};
    }
    const float c2 = p.scale_log2;

    auto do_tile = [&](const int it, const int stage) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (it + 1 < n_tiles) issue_tile(it + 1, stage ^ 1);

        const int i0 = it * BM;
        // nothing of this tile reaches the wave's keys
        if (!wave_has_keys || i0 + BM <= wave_row_lo || i0 >= wave_row_hi) return;
        const lds_u8* qb = smem + stage * STAGE;
        const lds_u8* db = qb + TILE;
        const lds_u8* sb = qb + 2 * TILE;

        // The tile is processed in 32-row blocks; a block none of whose rows reaches the wave's
        // keys is skipped (a wave-uniform branch).
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2) {
            const int ib = i0 + 32 * qb2;  // first row of the block
            if (ib + 32 <= wave_row_lo || ib >= wave_row_hi) continue;
            const lds_u8* qr = qb + qb2 * 32 * RB;
            const lds_u8* dr = db + qb2 * 32 * RB;

            // S = Q K^T, 32 queries x 32 keys.  Every row operand of S and dP is requested before
            // the first product, so one wave per SIMD does not wait out the LDS latency per step.
            u32x4_t qa[KSTEPS], da[KSTEPS];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qa[ks] = *(const lds_u32x4*)(qr + raddr[ks]);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) da[ks] = *(const lds_u32x4*)(dr + raddr[ks]);
            __builtin_amdgcn_sched_barrier(0);
            f32x16_t s = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) s = M::mma(__builtin_bit_cast(vec8, qa[ks]), kf[ks], s);

            // Exponent of P in base 2: scale S log2(e) - LSE log2(e), or -inf where a row cannot
            // see the key.  Register i of s holds query ib + 16 (i/8) + 8 g + i%8; rows past Nq
            // carry an LSE of +inf, so their weights are already 0.  The statistics of block rows
            // 16 (v4/2) + 8 g + 4 (v4%2) + 0..3 sit in one 16-byte LDS read each.
            f32x4_t rs[4];
            float x[16];
            // the mask matters only if some key of the wave is padding or lies outside some row's range
            const bool need_mask = kw0 + 31 >= kv_valid || (p.causal && kw0 + 31 > ib) ||
                                   (WIN && (ib + 31 - kw0 > p.window || kw0 + 31 - ib > p.window));
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int rl = 32 * qb2 + 16 * (v4 >> 1) + 8 * g + 4 * (v4 & 1);
                const f32x4_t ls = *(const __attribute__((address_space(3))) f32x4_t*)(sb + rl * 4);
                rs[v4] = *(const __attribute__((address_space(3))) f32x4_t*)(sb + BM * 4 + rl * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * v4 + e] = __builtin_fmaf(s[4 * v4 + e], c2, -ls[e]);
            }
            if (need_mask) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int qrow = ib + 16 * (i >> 3) + 8 * g + (i & 7);
                    const bool off = kj >= kv_valid || kj < attn::bwd_key_lo<WIN>(p, qrow) ||
                                     kj >= attn::bwd_key_hi<WIN>(p, qrow, kv_valid);
                    x[i] = off ? -INFINITY : x[i];
                }
            }

            // From here on one straight-line block (the mask above only edits x): dP = dO V^T runs
            // on the matrix cores while the exponentials form P, and dS of the second 16 rows forms
            // under the dV / dK products of the first 16.
            f32x16_t dp = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) dp = M::mma(__builtin_bit_cast(vec8, da[ks]), vf[ks], dp);
            // P = 2^x and dS = P (dP - Dr), rounded to T for the MFMAs
            vec8 pb[2], dsb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = __builtin_amdgcn_exp2f(x[i]);
                pb[i >> 3][i & 7] = (T)pv;
                dsb[i >> 3][i & 7] = (T)(pv * (dp[i] - rs[i >> 2][i & 3]));
            }

            // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per MFMA
#pragma unroll
            for (int h16 = 0; h16 < 2; ++h16) {
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const int ro = (32 * qb2 + 16 * h16) * RB;
                    const s16x4_t dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(db + taddr_lo[t] + ro));
                    const s16x4_t dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(db + taddr_hi[t] + ro));
                    const vec8 ad = __builtin_bit_cast(vec8, u32x4_t{__builtin_bit_cast(u32x2_t, dlo)[0],
                                                                      __builtin_bit_cast(u32x2_t, dlo)[1],
                                                                      __builtin_bit_cast(u32x2_t, dhi)[0],
                                                                      __builtin_bit_cast(u32x2_t, dhi)[1]});
                    dva[t] = M::mma(ad, pb[h16], dva[t]);
                    const s16x4_t qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + taddr_lo[t] + ro));
                    const s16x4_t qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(qb + taddr_hi[t] + ro));
                    const vec8 aq = __builtin_bit_cast(vec8, u32x4_t{__builtin_bit_cast(u32x2_t, qlo)[0],
                                                                      __builtin_bit_cast(u32x2_t, qlo)[1],
                                                                      __builtin_bit_cast(u32x2_t, qhi)[0],
                                                                      __builtin_bit_cast(u32x2_t, qhi)[1]});
                    dka[t] = M::mma(aq, dsb[h16], dka[t]);
                }
            }
        }
    };

    if (t_begin < n_tiles) issue_tile(t_begin, 0);
    for (int it = t_begin; it < n_tiles; it += 2) {
        do_tile(it, 0);
        if (it + 1 < n_tiles) do_tile(it + 1, 1);
    }

    // dK = scale * dka, dV = dva; registers 4a..4a+3 of [t] hold column 32 t + 8 a + 4 g + 0..3
    if (kj < p.Nk) {
        T* dkg = (T*)p.dk + kbase + (size_t)kj * D;
        T* dvg = (T*)p.dv + kbase + (size_t)kj * D;
        const float sc = p.scale;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u32x2_t wk, wv;
                wk[0] = (unsigned)__builtin_bit_cast(unsigned short, (T)(dka[t][4 * a + 0] * sc)) |
                        ((unsigned)__builtin_bit_cast(unsigned short, (T)(dka[t][4 * a + 1] * sc)) << 16);
                wk[1] = (unsigned)__builtin_bit_cast(unsigned short, (T)(dka[t][4 * a + 2] * sc)) |
                        ((unsigned)__builtin_bit_cast(unsigned short, (T)(dka[t][4 * a + 3] * sc)) << 16);
                wv[0] = (unsigned)__builtin_bit_cast(unsigned short, (T)dva[t][4 * a + 0]) |
                        ((unsigned)__builtin_bit_cast(unsigned short, (T)dva[t][4 * a + 1]) << 16);
                wv[1] = (unsigned)__builtin_bit_cast(unsigned short, (T)dva[t][4 * a + 2]) |
                        ((unsigned)__builtin_bit_cast(unsigned short, (T)dva[t][4 * a + 3]) << 16);
                *(u32x2_t*)(dkg + 32 * t + 8 * a + 4 * g) = wk;
                *(u32x2_t*)(dvg + 32 * t + 8 * a + 4 * g) = wv;
            }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int D, bool WIN>
hipError_t launch_two(const attn::BwdParams& p, hipStream_t stream) {
    attn::BwdParams pc = p;
    void* args[] = {&pc};
    hipError_t e = hipLaunchKernel((const void*)attn_bwd_dq_kernel<T, D, WIN>, dim3(p.n_blocks_q), dim3(NT),
                                   args, 0, stream);
    if (e != hipSuccess) return e;
    return hipLaunchKernel((const void*)attn_bwd_dkdv_kernel<T, D, WIN>, dim3(p.n_blocks_k), dim3(NT), args,
                           0, stream);
}

// The band logic is compiled only into the windowed kernels.
template <typename T, int D>
hipError_t launch_one(const attn::BwdParams& p, hipStream_t stream) {
    return p.window >= 0 ? launch_two<T, D, true>(p, stream) : launch_two<T, D, false>(p, stream);
}

}  // namespace

int attn_bwd_q_block() { return BMQ; }
int attn_bwd_k_block() { return BNK; }

hipError_t attn_launch_bwd_mfma(const attn::BwdParams& p, int dtype, int D, hipStream_t stream) {
    if (dtype == 2) return D == 128 ? launch_one<__bf16, 128>(p, stream) : launch_one<__bf16, 64>(p, stream);
    return D == 128 ? launch_one<_Float16, 128>(p, stream) : launch_one<_Float16, 64>(p, stream);
}

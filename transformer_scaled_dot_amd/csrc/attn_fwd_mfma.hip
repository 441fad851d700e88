// attn_fwd_mfma.hip -- fused attention forward for bf16 / fp16 on gfx950 matrix cores.
//
// The tiled loop of the pages (hotelren.com page on attention, sec.4.1: per Q tile, stream the
// K/V tiles, form the scores on chip, normalise online, accumulate P V, never store S; ch.5:
// load only the K/V tiles a Q tile can see) laid out for CDNA4:
//
//   * one workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32 rows.  Long
//     sequences (more than 8K rows, D = 128, no band, no key split) run 8 waves = 256 rows per
//     workgroup instead: each K/V tile copied to LDS then serves twice the rows;
//   * K/V tiles of 64 keys go HBM -> LDS by the buffer-load-to-LDS path (no registers, no LDS
//     store instructions), double buffered, one barrier per tile; the next tile's loads are in
//     flight while the current one is computed.  The copies are issued as assembly and waited
//     for explicitly, so that no LDS read of the current tile waits for the next tile's copy;
//   * both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation, arranged so
//     that a lane always holds one query row:
//        S^T = K Q^T   (A = K tile read from LDS, B = Q^T kept in registers for the whole loop)
//        O^T = V^T P^T (A = V^T read from the row-major V tile with the LDS transpose read,
//                       B = P^T taken straight from the S^T accumulator)
//     The 32x32 accumulator gives lane l the column l%32 (the query) and 16 rows (keys); the K
//     rows are fed to the MFMA with bits 2 and 3 of the row index swapped, which makes each
//     lane's 8-register halves hold 8 consecutive keys -- exactly the B-operand layout of the
//     next MFMA, so P never moves between lanes;
//   * the softmax runs per lane in base-2 units (logit * scale * log2 e) with an fp32 running
//     max and sum.  The two lanes that share a query row swap maxima once per tile.  The
//     reference max is raised (and O, l rescaled) only when a row's tile max exceeds it by more
//     than 2^8; otherwise P is formed against the stale reference, which leaves O / l and
//     ln 2 (m + log2 l) unchanged;
//   * tiles outside every row's visible keys are never loaded (causal, key padding and the
//     local band |i - j| <= w of sliding-window attention, lshu.cn page sec.2); masks are
//     evaluated only on the tiles that straddle a boundary;
//   * for queries at the end of a KV cache the keys of a Q tile may be split over several
//     workgroups (hotelren.com page sec.3.1); each then writes its fp32 partial O and LSE for the
//     log-sum-exp merge instead of the final output.
#include "attn_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

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
constexpr float kRescaleGap = 8.0f;             // base-2 units: P stays below 2^8
constexpr unsigned kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data, gfx9-family layout

// Row permutation of the K operand: swap bits 2 and 3 of a 0..31 row index (an involution).
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// K tile in LDS: row-major [BN][D], 16-byte chunk c of row `row` stored at chunk c ^ kswz(...).
// The 32 lanes of a half-wave read one chunk column of 32 rows (rows swap23(r)); the XOR puts
// them on distinct banks whether the LDS serves 8 or 16 lanes of a 128-bit read per clock.
template <int D>
__device__ __forceinline__ int kswz_lane(int r) {  // r: lane row 0..31 of the A operand
    return D == 128 ? (r & 15) : (((r >> 1) & 7) ^ ((r & 1) << 2));
}
template <int D>
__device__ __forceinline__ int kswz_row(int row) { return kswz_lane<D>(swap23(row & 31)); }

// V tile in LDS: row-major [BN][D].  The transpose read takes 4 consecutive rows x 32 bytes
// per 16 lanes; XOR-ing the chunk index with a function of (row mod 4) spreads the 32 lanes of
// a half-wave over all banks.
template <int D>
__device__ __forceinline__ int vswz_row(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// One 16-byte-per-lane copy HBM -> LDS (buffer load to LDS): lane l's 16 bytes from byte offset
// voff + soff of the buffer land at LDS byte address lds_base + 16 l.  The compiler cannot tell
// which LDS bytes such a copy writes; issued through its builtin, every later LDS read (the V^T
// transpose reads of the current tile in particular) would wait for all copies in flight,
// including the next tile's.  Issued as assembly it is invisible to that bookkeeping, and the
// kernel waits for its own copies (vmcnt) before the barrier that publishes a tile.  The
// instruction writes no registers; m0 carries the LDS address.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, unsigned lds_base, int voff,
                                            int soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_base)
                 : "memory");
}

// The lane id (0..63), computed where it is used: the volatile assembly has no inputs, so the
// compiler cannot hoist it and keep it in a register for the length of the loop.
__device__ __forceinline__ int lane_id_here() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// NW waves per workgroup (4 or 8), 32 query rows each.
template <typename T, int D, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) attn_fwd_mfma_kernel(attn::Params p) {
    // The body is device code only: its LDS address-space casts mean nothing to the host pass,
    // which needs just the kernel's signature to emit the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using M = Mfma<T>;
    using vec8 = typename M::vec8;
    constexpr int NCH = D / 8;              // 16-byte chunks per K/V row
    constexpr int KSTEPS = D / 16;          // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;              // 32-row tiles of O^T
    constexpr int KT = BN / 32;             // 32-key tiles of S^T
    constexpr int NTW = 64 * NW;            // threads of the workgroup
    constexpr int BMW = 32 * NW;            // query rows of the workgroup
    constexpr int CPT = BN * NCH / NTW;     // 16-byte chunks per thread per tile (K or V)
    constexpr int TILE = BN * D * 2;        // bytes of one K or V tile
    constexpr int STAGE = 2 * TILE;         // K tile then V tile
    static_assert(CPT >= 1, "tile too small for the workgroup");

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * STAGE];
    lds_u8* const smem = (lds_u8*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is the same on every lane: keep it (and all per-wave decisions) scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, g = lane >> 5;

    const attn::BlockWork bw = attn::block_work(p, attn::xcd_remap(blockIdx.x, p.n_blocks, p.n_qtiles * p.n_splits, p.xcd_interleave));
    const int bh = bw.bh;
    int qt = bw.qt;
    if (p.causal && !p.causal_br) qt = p.n_qtiles - 1 - qt;  // longest rows first
    const int b = bh / p.H;
    const int q0 = qt * BMW;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + r;

    const T* qg = (const T*)p.q + (size_t)bh * p.Nq * D;
    const T* kg = (const T*)p.k + (size_t)bh * p.Nk * D;
    const T* vg = (const T*)p.v + (size_t)bh * p.Nk * D;

    // Q^T operand: lane (r, g) holds Q[qi][16 ks + 8 g .. +7]; rows past Nq read as 0.  Requested
    // first, so that the key-length load and the first K/V tile overlap it (its sign flip, when
    // asked for, waits until both are issued).
    u32x4_t qraw[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t qrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)qg, 0, p.Nq * D * 2, kBufferWord3);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qraw[ks] = __builtin_amdgcn_raw_buffer_load_b128(qrs, (qi * D + 16 * ks + 8 * g) * 2, 0, 0);
    }
    vec8 qf[KSTEPS];  // qraw with the sign flip applied, set once the first tile is requested

    // Key tiles [t_begin, n_tiles) hold every key some row of this workgroup may see.
    const int kv_valid = attn::clamp_len(p.key_lens, b, p.Nk);
    const int q_last = min(p.Nq, q0 + BMW) - 1;
    int kv_end = min(kv_valid, attn::row_key_hi(p, q_last, kv_valid));
    int k_begin = max(0, attn::row_key_lo(p, q0));
    if (p.n_splits > 1) {  // this workgroup's share of the keys (split_len is a multiple of BN)
        k_begin = max(k_begin, bw.split * p.split_len);
        kv_end = min(kv_end, (bw.split + 1) * p.split_len);
    }
    const int n_tiles = (kv_end + BN - 1) / BN;
    const int t_begin = k_begin / BN;

    // This thread's 16-byte copy slots of a tile are i NTW + tid (i < CPT): row (i NTW + tid) /
    // NCH, chunk (tid % NCH) ^ swizzle(row).  The swizzles depend on the row only modulo 16 (K,
    // D = 128), 32 (K, D = 64) and 4 (V), and NTW / NCH (16 or 32) rows separate consecutive
    // slots, so slot i sits i NTW 16 bytes after slot 0 (a scalar offset) with the same chunk order.
    static_assert(NTW / NCH == 16 || NTW / NCH == 32, "copy slots must share their swizzle");
    int koff0, voff0;
    {
        const unsigned row = (unsigned)tid / NCH, phys = (unsigned)tid % NCH;
        koff0 = (int)((row * D + (phys ^ kswz_row<D>(row)) * 8) * 2);
        voff0 = (int)((row * D + (phys ^ vswz_row<D>(row)) * 8) * 2);
    }
    auto issue_tile = [&](const int tile, const int stage) {
        const int j0 = tile * BN;
        // Keys at or past the valid length fall outside the buffer and arrive as zeros.
        const int bytes = (kv_valid - j0) * D * 2;
        const __amdgpu_buffer_rsrc_t krs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kg + (size_t)j0 * D), 0, bytes, kBufferWord3);
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vg + (size_t)j0 * D), 0, bytes, kBufferWord3);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const unsigned kd = __builtin_amdgcn_readfirstlane(
                (unsigned)(uintptr_t)(smem + stage * STAGE + (i * NTW + wave * 64) * 16));
            copy_to_lds(krs, kd, koff0, i * NTW * 16);
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const unsigned vd = __builtin_amdgcn_readfirstlane(
                (unsigned)(uintptr_t)(smem + stage * STAGE + TILE + (i * NTW + wave * 64) * 16));
            copy_to_lds(vrs, vd, voff0, i * NTW * 16);
        }
    };

    // Per-lane LDS read offsets.
    // K (A operand of S^T) at k-step ks: row swap23(r) (+32 kt), chunk (2 ks + g) ^ kswz.  Chunk
    // bit 0 is g ^ (kswz & 1) and the upper chunk bits are ks ^ (kswz >> 1), so k-step ks reads at
    // kbase ^ (32 ks): one register and one XOR per read instead of a register per k-step.
    const int kbase = swap23(r) * (D * 2) + ((g ^ (kswz_lane<D>(r) & 1)) * 16) + (kswz_lane<D>(r) >> 1) * 32;
    // V^T (A operand of O^T) by transpose reads: within each 16-lane group (s = lane & 15), lane
    // s names 8 bytes of V row (16 h16 + 8 g + 4 u + s/4) at columns 32 dt + 16 G + 4 (s & 3);
    // lane s then receives column 32 dt + 16 G + s of those 4 rows.  Column tile dt sits at
    // vbase ^ (64 dt).
    int vbase;
    {
        const int s = lane & 15, G1 = (lane >> 4) & 1;
        const int fl = vswz_row<D>(s >> 2) >> 2;  // rows of one read differ only in their low 2 bits
        vbase = (8 * g + (s >> 2)) * (D * 2) + (2 * G1 + ((s & 3) >> 1)) * 16 + 8 * (s & 1) + 64 * fl;
    }

    f32x16_t oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16_t{};
    float m_ref = -INFINITY;  // reference max of this row (base-2 units)
    float l_run = 0.f;        // this lane's share of the running sum
    const float c2 = p.scale_log2;
    const bool wave_has_rows = qw0 < p.Nq;

    auto do_tile = [&](const int it, const int stage) {
        // Tile `it` is in LDS once every wave's loads have landed; the barrier also retires all
        // reads of the other stage, which the next loads overwrite.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (it + 1 < n_tiles) issue_tile(it + 1, stage ^ 1);

        const int j0 = it * BN;
        // nothing visible to this wave's rows qw0 .. qw0+31 in keys j0 .. j0+BN-1
        if (!wave_has_rows || j0 >= attn::row_key_hi(p, qw0 + 31, kv_valid) ||
            j0 + BN <= attn::row_key_lo(p, qw0))
            return;
        const lds_u8* kb = smem + stage * STAGE;
        const lds_u8* vb = kb + TILE;

        // ---- S^T = K Q^T: 32 keys x 32 queries per accumulator
        f32x16_t s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const u32x4_t a = *(const lds_u32x4*)(kb + (kbase ^ (32 * ks)) + kt * 32 * D * 2);
                s[kt] = M::mma(__builtin_bit_cast(vec8, a), qf[ks], s[kt]);
            }
        }

        // ---- online softmax.  Register i of s[kt] holds key j0 + 32 kt + 16 (i/8) + 8 g + i%8.
        // a mask applies unless every key of the tile is visible to every row of the wave
        const bool need_mask = j0 + BN > attn::row_key_hi(p, qw0, kv_valid) ||
                               j0 < attn::row_key_lo(p, qw0 + 31);
        float mt;
        if (need_mask) {
            // Register i holds key j0 + 8 g + kk with kk = 32 kt + 16 (i / 8) + i % 8 a constant;
            // it is visible iff kk - lo' lies in [0, hi - lo), lo' = lo - j0 - 8 g: one unsigned
            // compare per element.  The lane id is recomputed here rather than kept live.
            const int l = lane_id_here();
            const int row = qw0 + (l & 31);
            const int lo = attn::row_key_lo(p, row), hi = attn::row_key_hi(p, row, kv_valid);
            const int lo_rel = lo - j0 - 8 * (l >> 5);
            const unsigned span = hi > lo ? (unsigned)(hi - lo) : 0u;
            mt = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = 32 * kt + 16 * (i >> 3) + (i & 7);
                    const float t = (unsigned)(kk - lo_rel) < span ? s[kt][i] * c2 : -INFINITY;
                    s[kt][i] = t;
                    mt = fmaxf(mt, t);
                }
        } else {
            float mx = s[0][0];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = (kt == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
            mt = mx * c2;
        }
        {
            // both halves of the wave hold one row: take the max across lanes l and l ^ 32
            const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mt),
                                                             __builtin_bit_cast(unsigned, mt), false, false);
            mt = fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
        }
        if (__any(mt > m_ref + kRescaleGap)) {
            const float m_new = fmaxf(m_ref, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_ref - (m_new == -INFINITY ? 0.f : m_new));
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;

        // ---- P = 2^(t - m): fp32 row sum, rounded to T for the MFMA
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kt][i] = __builtin_amdgcn_exp2f(s[kt][i] - m_use);
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[kt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c2, -m_use));
        }
        vec8 pb[BN / 16];
#pragma unroll
        for (int h16 = 0; h16 < BN / 16; ++h16) {
            const int kt = h16 >> 1, base = 8 * (h16 & 1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pb[h16][e] = (T)s[kt][base + e];
                l_run += s[kt][base + e];
            }
        }

        // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
        for (int h16 = 0; h16 < BN / 16; ++h16) {
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const lds_u8* a0 = vb + (vbase ^ (64 * t)) + (16 * h16) * (D * 2);
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a0);
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 4 * D * 2));
                const vec8 a = __builtin_bit_cast(vec8, u32x4_t{__builtin_bit_cast(u32x2_t, lo)[0],
                                                                 __builtin_bit_cast(u32x2_t, lo)[1],
                                                                 __builtin_bit_cast(u32x2_t, hi)[0],
                                                                 __builtin_bit_cast(u32x2_t, hi)[1]});
                oacc[t] = M::mma(a, pb[h16], oacc[t]);
            }
        }
    };

    if (t_begin < n_tiles) issue_tile(t_begin, 0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
        qf[ks] = __builtin_bit_cast(vec8, p.negate_q ? qraw[ks] ^ 0x80008000u : qraw[ks]);
    for (int it = t_begin; it < n_tiles; it += 2) {
        do_tile(it, 0);
        if (it + 1 < n_tiles) do_tile(it + 1, 1);
    }

    // ---- epilogue: O = O / l (rounded to T), LSE = ln 2 * (m + log2 l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (p.n_splits > 1) {  // fp32 partial result of this split, merged by attn_merge_kernel
        if (qi < p.Nq) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const size_t row = ((size_t)bw.split * p.B * p.H + bh) * p.Nq + qi;
            float* og = p.o_part + row * D;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *(float4*)(og + 32 * t + 8 * a + 4 * g) =
                        make_float4(oacc[t][4 * a + 0] * inv, oacc[t][4 * a + 1] * inv,
                                    oacc[t][4 * a + 2] * inv, oacc[t][4 * a + 3] * inv);
            if (g == 0)
                p.lse_part[row] = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * attn::kLn2 : -INFINITY;
        }
    } else if (qi < p.Nq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        T* og = (T*)p.o + ((size_t)bh * p.Nq + qi) * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // accumulator registers 4a..4a+3 hold O[qi][32 t + 8 a + 4 g + 0..3]; a vector of
                // T converts two values per instruction (scalar casts joined by shifts took three)
                using T4 = T __attribute__((ext_vector_type(4)));
                const T4 w = {(T)(oacc[t][4 * a + 0] * inv), (T)(oacc[t][4 * a + 1] * inv),
                              (T)(oacc[t][4 * a + 2] * inv), (T)(oacc[t][4 * a + 3] * inv)};
                *(T4*)(og + 32 * t + 8 * a + 4 * g) = w;
            }
        if (g == 0)
            p.lse[(size_t)bh * p.Nq + qi] =
                l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * attn::kLn2 : -INFINITY;
    }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int D>
hipError_t launch_one(const attn::Params& p, hipStream_t stream) {
    attn::Params pc = p;
    void* args[] = {&pc};
    if constexpr (D == 128) {
        // Long sequences: 256-row workgroups of 8 waves (one per CU at two waves per SIMD).  Each
        // K/V tile copied to LDS serves twice the rows; at 16K causal this measured 0.6-2.2 %
        // faster (same bits), at 4K 1-2 % slower and on the band 13 % slower.
        if (p.n_splits == 1 && p.window < 0 && p.Nq > 8192) {
            pc.n_qtiles = (p.Nq + 2 * BM - 1) / (2 * BM);
            pc.n_blocks = pc.n_qtiles * p.H * p.B;
            return hipLaunchKernel((const void*)attn_fwd_mfma_kernel<T, D, 8>, dim3(pc.n_blocks),
                                   dim3(2 * NT), args, 0, stream);
        }
    }
    return hipLaunchKernel((const void*)attn_fwd_mfma_kernel<T, D, 4>, dim3(p.n_blocks), dim3(NT),
                           args, 0, stream);
}

}  // namespace

int attn_mfma_block_m() { return BM; }

hipError_t attn_launch_mfma(const attn::Params& p, int dtype, int D, hipStream_t stream) {
    if (dtype == 2) return D == 128 ? launch_one<__bf16, 128>(p, stream) : launch_one<__bf16, 64>(p, stream);
    return D == 128 ? launch_one<_Float16, 128>(p, stream) : launch_one<_Float16, 64>(p, stream);
}

// attn_fwd_api.hip -- the C ABI: argument checks, kernel choice, launch on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include <attn_fwd.h>
#include "attn_common.h"

namespace {

// Checks shared by every entry point and the parameters they have in common.  Returns
// ATTN_OK and fills p, or the first error found (nothing is enqueued then).
int prepare(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
            int Nk, int D, float scale, int causal, const int32_t* key_lens, int dtype,
            attn::Params& p) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
    if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15) != 0 ||
        ((uintptr_t)key_lens & 3) != 0)
        return ATTN_ERR_ALIGN;
    // Per-(b, h) slices are addressed with 32-bit byte offsets (4-byte elements at most).
    if ((int64_t)Nq * D >= ((int64_t)1 << 29) || (int64_t)Nk * D >= ((int64_t)1 << 29))
        return ATTN_ERR_SHAPE;

    const int bm = dtype == ATTN_F32 ? attn_f32_block_m() : attn_mfma_block_m();
    const int64_t n_qtiles = ((int64_t)Nq + bm - 1) / bm;
    const int64_t n_blocks = n_qtiles * H * B;
    if (n_blocks > INT32_MAX) return ATTN_ERR_SHAPE;

    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.key_lens = key_lens;
    p.B = B;
    p.H = H;
    p.Nq = Nq;
    p.Nk = Nk;
    p.n_qtiles = (int)n_qtiles;
    p.n_blocks = (int)n_blocks;
    // Logits are handled in base-2 units.  The kernels need a strictly positive multiplier (a
    // masked logit is -inf and must stay -inf after scaling): a zero scale runs as 1e-30, which
    // still gives every weight exactly 1 for raw dot products below 2^70 in magnitude
    // (2^(1e-30 x) rounds to 1 in fp32 there).
    p.scale_log2 = (float)fmax(fabs((double)scale) * 1.4426950408889634074, 1e-30);
    p.negate_q = scale < 0.f;
    p.causal = causal;
    p.causal_br = 0;
    p.window = -1;
    p.xcd_interleave = 1;
    p.n_splits = 1;
    p.split_len = 0;
    p.o_part = nullptr;
    p.lse_part = nullptr;
    return ATTN_OK;
}

hipError_t launch(const attn::Params& p, int dtype, int D, hipStream_t s) {
    return dtype == ATTN_F32 ? attn_launch_f32(p, D, s) : attn_launch_mfma(p, dtype, D, s);
}

// How a decode call spreads the keys over workgroups: enough splits to give the chip about
// 1024 workgroups (four per CU; 512 to 2048 measure within a few percent), at most 64, each
// split at least four 64-key tiles long.  A pure function of the sizes, so the workspace query
// and the call always agree.
struct DecodePlan {
    int n_splits;
    int split_len;
    size_t workspace_bytes;
};

DecodePlan decode_plan(int B, int H, int Nq, int Nk, int D, int dtype) {
    const int bm = dtype == ATTN_F32 ? attn_f32_block_m() : attn_mfma_block_m();
    const int64_t base = (int64_t)B * H * (((int64_t)Nq + bm - 1) / bm);
    int64_t S = (1024 + base - 1) / base;
    S = S < 64 ? S : 64;
    const int64_t by_len = Nk / 256;
    S = S < by_len ? S : by_len;
    if (S < 1) S = 1;
    DecodePlan plan{1, 0, 0};
    if (S == 1) return plan;
    const int64_t len = ((Nk + S - 1) / S + 63) / 64 * 64;
    plan.split_len = (int)len;
    plan.n_splits = (int)((Nk + len - 1) / len);
    if (plan.n_splits > 1)
        plan.workspace_bytes = (size_t)plan.n_splits * B * H * Nq * (size_t)(D + 1) * sizeof(float);
    else
        plan.split_len = 0;
    return plan;
}

}  // namespace

extern "C" int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Nq, int Nk, int D, float scale, int causal,
                               int window, const int32_t* key_lens, int dtype, void* stream) {
    attn::Params p;
    const int rc = prepare(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens, dtype, p);
    if (rc != ATTN_OK) return rc;
    if (window < -1) return ATTN_ERR_WINDOW;
    // |i - j| < max(Nq, Nk) always holds: a band at least that wide is no band.
    p.window = window >= (Nq > Nk ? Nq : Nk) ? -1 : window;
    // Causal Q tiles differ in length (longest first within a head): with up to 8K rows each XCD
    // alternates between four heads so that the long tiles of all its heads start before the
    // short ones (the last XCD slots would otherwise run a few long tiles alone; 4K causal: +4 to
    // 8 %).  Longer heads already fill an XCD's slots with tiles of every length, and four heads'
    // K/V streams at once no longer share its L2: at 16K the interleave was no faster and fetched
    // 3.8x the bytes from beyond the L2.  Banded and unmasked tiles are of equal length and read
    // overlapping K/V, which one head at a time keeps in the XCD's L2.
    if (causal && p.window < 0 && Nq <= 8192) p.xcd_interleave = 4;
    return launch(p, dtype, D, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" size_t attn_decode_workspace_size(int B, int H, int Nq, int Nk, int D, int dtype) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (D != 64 && D != 128) ||
        (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16))
        return 0;
    return decode_plan(B, H, Nq, Nk, D, dtype).workspace_bytes;
}

namespace {

// attn_decode's work after its argument checks, with the split partials in `workspace`.
int decode_run(attn::Params& p, const DecodePlan& plan, int B, int H, int Nq, int D, int dtype,
               void* workspace, size_t workspace_bytes, hipStream_t s) {
    if (plan.n_splits == 1) return launch(p, dtype, D, s) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    if (!workspace) return ATTN_ERR_NULL;
    if (((uintptr_t)workspace & 15) != 0) return ATTN_ERR_ALIGN;
    if (workspace_bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE;
    const int64_t n_blocks = (int64_t)p.n_blocks * plan.n_splits;
    if (n_blocks > INT32_MAX || (int64_t)B * H * Nq > INT32_MAX) return ATTN_ERR_SHAPE;
    p.n_blocks = (int)n_blocks;
    p.n_splits = plan.n_splits;
    p.split_len = plan.split_len;
    p.o_part = (float*)workspace;
    p.lse_part = p.o_part + (size_t)plan.n_splits * B * H * Nq * D;
    if (launch(p, dtype, D, s) != hipSuccess) return ATTN_ERR_LAUNCH;
    return attn_launch_merge(p, dtype, D, s) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int Nq, int Nk, int D, float scale, int causal,
                           const int32_t* key_lens, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
    attn::Params p;
    const int rc = prepare(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens, dtype, p);
    if (rc != ATTN_OK) return rc;
    p.causal_br = 1;  // the queries are the last Nq positions of each cached sequence
    const DecodePlan plan = decode_plan(B, H, Nq, Nk, D, dtype);
    return decode_run(p, plan, B, H, Nq, D, dtype, workspace, workspace_bytes, (hipStream_t)stream);
}

// ---- attn_decode without a caller workspace: the split partials live in `scratch`, a
// file-scope device array of ATTN_DECODE_SCRATCH_BYTES.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device id, once looked up

// The current device's copy of `scratch`, looked up on the first call on that device.
// Returns nullptr if the device id is out of range or the lookup fails.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int H, int Nq, int Nk, int D, float scale, int causal,
                                   const int32_t* key_lens, int dtype, void* stream) {
    attn::Params p;
    const int rc = prepare(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, key_lens, dtype, p);
    if (rc != ATTN_OK) return rc;
    p.causal_br = 1;
    const DecodePlan plan = decode_plan(B, H, Nq, Nk, D, dtype);
    if (plan.workspace_bytes > ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    void* ws = nullptr;
    if (plan.n_splits > 1 && !(ws = scratch_on_current_device())) return ATTN_ERR_LAUNCH;
    // every split writes all of its rows' partials (O = 0, LSE = -inf where it sees no key)
    // before the merge reads them, so nothing left by an earlier call needs clearing
    return decode_run(p, plan, B, H, Nq, D, dtype, ws, ATTN_DECODE_SCRATCH_BYTES, (hipStream_t)stream);
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Nq, int Nk, int D, float scale, int causal,
                        const int32_t* key_lens, int dtype, void* stream) {
    return attn_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, -1, key_lens, dtype,
                           stream);
}

extern "C" const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer (q, k, v, o, lse) is NULL";
        case ATTN_ERR_SHAPE: return "B, H, Nq, Nk must be >= 1 and each (b, h) slice below 2^29 elements";
        case ATTN_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
        case ATTN_ERR_DTYPE: return "dtype must be ATTN_F32, ATTN_F16 or ATTN_BF16";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_FLAG: return "causal must be 0 or 1";
        case ATTN_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
        case ATTN_ERR_ALIGN: return "q, k, v, o and lse must be 16-byte aligned, key_lens 4-byte aligned";
        case ATTN_ERR_WINDOW: return "window must be -1 (no band) or >= 0";
        case ATTN_ERR_WORKSPACE: return "workspace_bytes is below the *_workspace_size() query";
        case ATTN_ERR_SCRATCH:
            return "attn_decode_noalloc: the call needs more than the library's static scratch "
                   "(ATTN_DECODE_SCRATCH_BYTES); use attn_decode with a workspace";
        default: return "unknown status";
    }
}

/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU reference for the forward pass of
 * multi-head scaled-dot-product attention and for its gradients (oracle_attn_bwd, below).
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load this
 * library; the product path never does.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes (the textbook definition, not the tiled algorithm):
 *   For each batch b, head h and query row i,
 *     J(i)   = { j : 0 <= j < L_b and (not causal or j <= i + c_b)
 *                    and (w < 0 or i - w <= j <= i + w) }          (masked keys excluded)
 *   with c_b = 0 for the top-left causal mask (causal = 1) and c_b = L_b - Nq for the
 *   bottom-right one (causal = 2: the Nq queries are the last Nq positions of a key sequence
 *   of length L_b, as when new tokens attend to a KV cache that already holds them),
 *     s_j    = scale * sum_d q[i,d] k[j,d]                          for j in J(i)
 *     m      = max_j s_j                                            (two-pass max shift)
 *     e_j    = exp(s_j - m),  l = sum_j e_j
 *     O[i,:] = sum_j e_j v[j,:] / l
 *     lse[i] = m + ln l                                             (natural log)
 *   and for an empty J(i):  O[i,:] = 0,  lse[i] = -inf.
 *
 * Sources (the pages on scaled dot-product attention):
 *   - definition softmax(Q K^T / sqrt(d_k)) V and the masked_fill(mask == 0, -inf) step:
 *     the hotelren.com page, ch.1 code and sec.2.1 formula and "PyTorch hand-written
 *     implementation"; the qqiyuan.cn page, "original implementation" (fill -1e9) and
 *     its pitfalls list (additive -10000 mask).  Excluding masked keys equals all three
 *     fill conventions on every row that keeps at least one key.
 *   - causal mask = attend only to the current and earlier positions: hotelren.com
 *     sec.2.1 note 2; lshu.cn sec.3.1.  Read here as j <= i (top-left aligned); for queries
 *     that extend a KV cache (hotelren.com sec.3.1: each new token appends its own key and
 *     value and reuses the cached ones), query i sits at position L_b - Nq + i.
 *   - local (sliding-window) attention: each position attends only to the w positions before
 *     and after it, every other weight is zero: lshu.cn sec.2 ("localization", Longformer /
 *     BigBird windows); aicoding.csdn.net sec.4.3 (window w = 512).  Read here as the band
 *     |i - j| <= w, combined with the causal and padding masks; w < 0 means no window.
 *   - max-shifted softmax and log-sum-exp = max + log(sum exp(x - max)):
 *     aicoding.csdn.net sec.2.2 ("numerical stability of softmax", chunked logsumexp).
 *   - the fused method is numerically the same as the plain one: aicoding.csdn.net ch.1
 *     table; lshu.cn sec.2.2.  So the oracle is the plain definition.
 *
 * Inputs are the stored bytes (fp32, fp16 or bf16); each is widened exactly to fp64 by
 * the decoders below.  `scale` is the same value the GPU path receives (already rounded
 * to float32 by the caller), widened.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* bfloat16 is the top half of an IEEE binary32 pattern. */
static double dec_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double dec(const void* base, int dtype, int64_t idx) {
    if (dtype == OR_F32) {
        float f;
        memcpy(&f, (const char*)base + 4 * idx, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char*)base + 2 * idx, 2);
    return dtype == OR_F16 ? dec_f16(h) : dec_bf16(h);
}

static void decode_row(const void* base, int dtype, int64_t off, int D, double* out) {
    for (int d = 0; d < D; ++d) out[d] = dec(base, dtype, off + d);
}

/* One query row (b, h, i).  Scratch: qrow[D], s[Nk]. */
static void one_row(const void* q, const void* k, const void* v, int dtype, int H, int Nq,
                    int Nk, int D, double scale, int causal, int window, const int32_t* key_lens,
                    int64_t row, double* o, double* lse, double* qrow, double* s, double* krow) {
    int64_t bh = row / Nq;
    int i = (int)(row % Nq);
    int b = (int)(bh / H);
    int64_t L = Nk;
    if (key_lens) {
        L = key_lens[b];
        if (L < 0) L = 0;
        if (L > Nk) L = Nk;
    }
    int64_t jbeg = 0, jend = L; /* J(i) = [jbeg, jend) */
    int64_t cb = causal == 2 ? L - Nq : 0;
    if (causal && jend > (int64_t)i + cb + 1) jend = (int64_t)i + cb + 1;
    if (window >= 0) {
        if (jbeg < (int64_t)i - window) jbeg = (int64_t)i - window;
        if (jend > (int64_t)i + window + 1) jend = (int64_t)i + window + 1;
    }

    if (jend <= jbeg) {
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    decode_row(q, dtype, row * D, D, qrow);
    int64_t kbase = bh * (int64_t)Nk * D;

    /* logits; s[j - jbeg] holds key j */
    for (int64_t j = jbeg; j < jend; ++j) {
        decode_row(k, dtype, kbase + j * D, D, krow);
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * krow[d];
        s[j - jbeg] = scale * acc;
    }
    const int64_t n = jend - jbeg;
    /* pass 1: max */
    double m = s[0];
    for (int64_t j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    /* pass 2: shifted exponentials and their sum */
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* weighted sum of values */
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        decode_row(v, dtype, kbase + (jbeg + j) * D, D, krow);
        for (int d = 0; d < D; ++d) o[d] += s[j] * krow[d];
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
    *lse = m + log(l);
}

/*
 * oracle_attn_rows_window -- reference attention on selected query rows.
 *   q: [B,H,Nq,D], k, v: [B,H,Nk,D], contiguous, stored as `dtype` (0 fp32, 1 fp16, 2 bf16).
 *   causal: 0 none, 1 top-left (j <= i), 2 bottom-right (j <= i + L_b - Nq).
 *   window: half-width w of the local band |i - j| <= w, or any negative value for none.
 *   key_lens: int32[B] or NULL (every key valid); values are clamped to [0, Nk].
 *   rows: flat row ids ((b*H + h)*Nq + i), or NULL for all B*H*Nq rows in order.
 *   o: fp64 [nrows, D]; lse: fp64 [nrows].
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, -1 on a bad argument, -2 if scratch memory cannot be allocated.
 */
int oracle_attn_rows_window(const void* q, const void* k, const void* v, int dtype, int B, int H,
                            int Nq, int Nk, int D, double scale, int causal, int window,
                            const int32_t* key_lens, const int64_t* rows, int64_t nrows, double* o,
                            double* lse, int nthreads) {
    if (!q || !k || !v || !o || !lse) return -1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1) return -1;
    if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return -1;
    if (causal < 0 || causal > 2) return -1;
    int64_t total = (int64_t)B * H * Nq;
    if (!rows) nrows = total;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return -1;
    int nt = 1;
#ifdef _OPENMP
    nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    (void)nthreads;
    /* per-thread scratch: qrow[D], krow[D], s[Nk] */
    size_t per = (size_t)2 * D + (size_t)Nk;
    double* scratch = (double*)malloc(sizeof(double) * per * (size_t)nt);
    if (!scratch) return -2;
#pragma omp parallel num_threads(nt)
    {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
        double* qrow = scratch + per * (size_t)t;
        double* krow = qrow + D;
        double* s = krow + D;
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows ? rows[r] : r;
            one_row(q, k, v, dtype, H, Nq, Nk, D, scale, causal, window, key_lens, row, o + r * D,
                    lse + r, qrow, s, krow);
        }
    }
    free(scratch);
    return 0;
}

/* oracle_attn_rows -- the same without a window. */
int oracle_attn_rows(const void* q, const void* k, const void* v, int dtype, int B, int H, int Nq,
                     int Nk, int D, double scale, int causal, const int32_t* key_lens,
                     const int64_t* rows, int64_t nrows, double* o, double* lse, int nthreads) {
    return oracle_attn_rows_window(q, k, v, dtype, B, H, Nq, Nk, D, scale, causal, -1, key_lens,
                                   rows, nrows, o, lse, nthreads);
}

/*
 * Backward pass (gradients of the forward above, for causal in {0, 1}, with or without a
 * local band).
 *
 * With the row probabilities P[i,j] = e_j / l over J(i) (0 outside it) and a scalar loss whose
 * gradients with respect to the outputs are dO (same shape as O) and dlse (same shape as lse,
 * zero when not given), the chain rule through O[i,:] = sum_j P[i,j] v[j,:] and
 * lse[i] = ln sum_{j in J(i)} exp(s[i,j]) gives
 *   dv[j,:]  = sum_i P[i,j] dO[i,:]
 *   dP[i,j]  = dO[i,:] . v[j,:]
 *   Dr[i]    = sum_j P[i,j] dP[i,j]
 *   dS[i,j]  = P[i,j] (dP[i,j] - Dr[i] + dlse[i])      (the softmax Jacobian, plus d lse / d s = P)
 *   dq[i,:]  = scale sum_j dS[i,j] k[j,:]
 *   dk[j,:]  = scale sum_i dS[i,j] q[i,:]
 * Source: the pages say training must keep or rebuild the softmax output for the backward pass
 * (aicoding.csdn.net ch.1 list) and that FlashAttention-2's backward rebuilds the products from
 * the forward's softmax instead of storing the N x N matrix (hotelren.com sec.4.2, "gradient
 * back-propagation reconstruction"; its printed helper is garbled, so the gradient itself is
 * taken from the calculus above).
 *
 * Pass 1 (over query rows): P from the definition (two-pass max), Dr[i], lse[i] and dq[i,:].
 * Pass 2 (over keys): P[i,j] = exp(s[i,j] - lse[i]) for every row i that sees key j, then dk and
 * dv.  Both passes are plain sums in fp64; the second re-derives P from lse only so that each
 * key's sums can be formed independently.
 */
typedef struct {
    int dtype, Nq, Nk, D, causal, window;
    double scale;
} bwd_shape;

/* keys [bwd_jbeg, bwd_jend) visible to row i of a batch with L valid keys: causal 0 / 1, and
 * the band |i - j| <= window when window >= 0 */
static int64_t bwd_jbeg(const bwd_shape* sh, int i) {
    return sh->window >= 0 && (int64_t)i - sh->window > 0 ? (int64_t)i - sh->window : 0;
}
static int64_t bwd_jend(const bwd_shape* sh, int64_t L, int i) {
    int64_t jend = L;
    if (sh->causal && jend > (int64_t)i + 1) jend = (int64_t)i + 1;
    if (sh->window >= 0 && jend > (int64_t)i + sh->window + 1) jend = (int64_t)i + sh->window + 1;
    return jend;
}

/*
 * oracle_attn_bwd -- reference gradients for selected (b, h) slices.
 *   q, dO: [B,H,Nq,D]; k, v: [B,H,Nk,D]; contiguous, stored as `dtype`.
 *   dlse: fp32 [B,H,Nq] or NULL (zero).  causal: 0 or 1.  window: half-width of the local band
 *   |i - j| <= window, or any negative value for none.  key_lens: int32[B] or NULL.
 *   bh: slice ids b*H + h (n_bh of them), or NULL for all B*H in order.
 *   dq: fp64 [n_bh, Nq, D]; dk, dv: fp64 [n_bh, Nk, D].
 * Returns 0, -1 on a bad argument, -2 if memory cannot be allocated.
 */
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dO,
                    const float* dlse, int dtype, int B, int H, int Nq, int Nk, int D,
                    double scale, int causal, int window, const int32_t* key_lens,
                    const int64_t* bh, int64_t n_bh, double* dq, double* dk, double* dv,
                    int nthreads) {
    if (!q || !k || !v || !dO || !dq || !dk || !dv) return -1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1) return -1;
    if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return -1;
    if (causal != 0 && causal != 1) return -1;
    if (!bh) n_bh = (int64_t)B * H;
    for (int64_t t = 0; bh && t < n_bh; ++t)
        if (bh[t] < 0 || bh[t] >= (int64_t)B * H) return -1;
    int nt = 1;
#ifdef _OPENMP
    nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    (void)nthreads;
    const bwd_shape sh = {dtype, Nq, Nk, D, causal, window < 0 ? -1 : window, scale};
    /* one slice at a time: its inputs widened to fp64, lse and Dr per row */
    const size_t nq = (size_t)Nq * D, nk = (size_t)Nk * D;
    double* buf = (double*)malloc(sizeof(double) * (2 * nq + 2 * nk + 2 * (size_t)Nq));
    const size_t per = 2 * (size_t)Nk; /* per thread: P[Nk], dP[Nk] of one row */
    double* sc = (double*)malloc(sizeof(double) * (size_t)nt * per);
    if (!buf || !sc) {
        free(buf);
        free(sc);
        return -2;
    }
    double *Qd = buf, *dOd = Qd + nq, *Kd = dOd + nq, *Vd = Kd + nk, *lse = Vd + nk, *Dr = lse + Nq;
    for (int64_t t = 0; t < n_bh; ++t) {
        const int64_t s_bh = bh ? bh[t] : t;
        const int b = (int)(s_bh / H);
        int64_t L = Nk;
        if (key_lens) {
            L = key_lens[b];
            if (L < 0) L = 0;
            if (L > Nk) L = Nk;
        }
        for (size_t x = 0; x < nq; ++x) {
            Qd[x] = dec(q, dtype, (int64_t)(s_bh * nq + x));
            dOd[x] = dec(dO, dtype, (int64_t)(s_bh * nq + x));
        }
        for (size_t x = 0; x < nk; ++x) {
            Kd[x] = dec(k, dtype, (int64_t)(s_bh * nk + x));
            Vd[x] = dec(v, dtype, (int64_t)(s_bh * nk + x));
        }
        double* dqs = dq + t * nq;
        double* dks = dk + t * nk;
        double* dvs = dv + t * nk;

        /* pass 1: rows */
#pragma omp parallel for num_threads(nt) schedule(dynamic, 8)
        for (int i = 0; i < Nq; ++i) {
            int tid = 0;
#ifdef _OPENMP
            tid = omp_get_thread_num();
#endif
            double* P = sc + (size_t)tid * per;
            double* dP = P + Nk;
            const double* qi = Qd + (size_t)i * D;
            const double* gi = dOd + (size_t)i * D;
            double* dqi = dqs + (size_t)i * D;
            for (int d = 0; d < D; ++d) dqi[d] = 0.0;
            const int64_t jb = bwd_jbeg(&sh, i), n = bwd_jend(&sh, L, i);
            if (n <= jb) {
                lse[i] = -INFINITY;
                Dr[i] = 0.0;
                continue;
            }
            /* logits, max, sum, probabilities (P[j], dP[j] hold key j) */
            double m = -INFINITY;
            for (int64_t j = jb; j < n; ++j) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += qi[d] * Kd[j * D + d];
                P[j] = sh.scale * acc;
                if (P[j] > m) m = P[j];
            }
            double l = 0.0;
            for (int64_t j = jb; j < n; ++j) l += exp(P[j] - m);
            lse[i] = m + log(l);
            for (int64_t j = jb; j < n; ++j) P[j] = exp(P[j] - m) / l;
            /* dP and Dr = sum_j P dP */
            double Dsum = 0.0;
            for (int64_t j = jb; j < n; ++j) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += gi[d] * Vd[j * D + d];
                dP[j] = acc;
                Dsum += P[j] * acc;
            }
            Dr[i] = Dsum;
            /* dq = scale sum_j P (dP - Dr + g) k_j */
            const double g = dlse ? (double)dlse[s_bh * Nq + i] : 0.0;
            for (int64_t j = jb; j < n; ++j) {
                const double ds = P[j] * (dP[j] - Dsum + g);
                for (int d = 0; d < D; ++d) dqi[d] += sh.scale * ds * Kd[j * D + d];
            }
        }

        /* pass 2: keys */
#pragma omp parallel for num_threads(nt) schedule(dynamic, 8)
        for (int j = 0; j < Nk; ++j) {
            double* dkj = dks + (size_t)j * D;
            double* dvj = dvs + (size_t)j * D;
            for (int d = 0; d < D; ++d) dkj[d] = dvj[d] = 0.0;
            if (j >= L) continue; /* padding keys are never seen */
            for (int i = 0; i < Nq; ++i) {
                if ((int64_t)j < bwd_jbeg(&sh, i) || (int64_t)j >= bwd_jend(&sh, L, i)) continue;
                const double* qi = Qd + (size_t)i * D;
                const double* gi = dOd + (size_t)i * D;
                double acc = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) {
                    acc += qi[d] * Kd[(size_t)j * D + d];
                    dp += gi[d] * Vd[(size_t)j * D + d];
                }
                const double pij = exp(sh.scale * acc - lse[i]);
                const double g = dlse ? (double)dlse[s_bh * Nq + i] : 0.0;
                const double ds = pij * (dp - Dr[i] + g);
                for (int d = 0; d < D; ++d) {
                    dkj[d] += sh.scale * ds * qi[d];
                    dvj[d] += pij * gi[d];
                }
            }
        }
    }
    free(buf);
    free(sc);
    return 0;
}

/* Decoders exposed for the tests' checks of the widening itself. */
double oracle_decode(const void* base, int dtype, int64_t idx) { return dec(base, dtype, idx); }

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

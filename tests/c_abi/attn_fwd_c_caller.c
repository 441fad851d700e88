/*
 * attn_fwd_c_caller.c -- a C program that calls the attention library through its C header
 * alone (test infrastructure: the GPU test feeds it inputs and checks its outputs).
 *
 * usage: attn_fwd_c_caller B H Nq Nk D causal dtype in.bin out.bin
 *   in.bin   q, k, v back to back, raw storage bytes of `dtype` (0 fp32, 1 fp16, 2 bf16),
 *            [B, H, Nq, D] then [B, H, Nk, D] twice, row-major
 *   out.bin  o ([B, H, Nq, D], storage bytes of `dtype`) then lse (fp32 [B, H, Nq])
 * The scale is 1/sqrt(D).  Device memory comes from the HIP runtime (the library allocates
 * nothing); the call runs on a stream the program creates.  It also makes calls that must be
 * refused on the host, one from each group of status codes: an unsupported head dimension
 * (ATTN_ERR_HEAD_DIM, of the original set) and a causal flag of 2 (ATTN_ERR_FLAG, added later),
 * and checks the codes by their names and values.
 * Exit status 0 on success.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "attn_fwd.h"

static int fail(const char* what) {
    fprintf(stderr, "attn_fwd_c_caller: %s\n", what);
    return 1;
}

int main(int argc, char** argv) {
    if (argc != 10) return fail("usage: B H Nq Nk D causal dtype in.bin out.bin");
    const int B = atoi(argv[1]), H = atoi(argv[2]), Nq = atoi(argv[3]), Nk = atoi(argv[4]), D = atoi(argv[5]);
    const int causal = atoi(argv[6]), dtype = atoi(argv[7]);
    const size_t es = dtype == ATTN_F32 ? 4 : 2;
    const size_t nq = (size_t)B * H * Nq * D, nk = (size_t)B * H * Nk * D, nl = (size_t)B * H * Nq;

    unsigned char* host = malloc((nq + 2 * nk) * es);
    unsigned char* outh = malloc(nq * es + nl * 4);
    if (!host || !outh) return fail("host allocation");
    FILE* f = fopen(argv[8], "rb");
    if (!f || fread(host, es, nq + 2 * nk, f) != nq + 2 * nk) return fail("cannot read the inputs");
    fclose(f);

    void *q, *k, *v, *o;
    float* lse;
    hipStream_t stream;
    if (hipMalloc(&q, nq * es) || hipMalloc(&k, nk * es) || hipMalloc(&v, nk * es) || hipMalloc(&o, nq * es) ||
        hipMalloc((void**)&lse, nl * 4) || hipStreamCreate(&stream))
        return fail("device allocation");
    if (hipMemcpy(q, host, nq * es, hipMemcpyHostToDevice) ||
        hipMemcpy(k, host + nq * es, nk * es, hipMemcpyHostToDevice) ||
        hipMemcpy(v, host + (nq + nk) * es, nk * es, hipMemcpyHostToDevice))
        return fail("copy to the device");

    /* bad arguments are refused on the host, before anything is enqueued */
    const int bad = attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, 96, 0.1f, causal, NULL, dtype, stream);
    if (bad != ATTN_ERR_HEAD_DIM || ATTN_ERR_HEAD_DIM != -3) return fail("D = 96 was not refused with -3");
    printf("D=96: %s\n", attn_status_str(bad));
    const int bad_flag = attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, 0.1f, 2, NULL, dtype, stream);
    if (bad_flag != ATTN_ERR_FLAG || ATTN_ERR_FLAG != -7) return fail("causal = 2 was not refused with -7");
    printf("causal=2: %s\n", attn_status_str(bad_flag));
    if (ATTN_ERR_LAUNCH != -6) return fail("ATTN_ERR_LAUNCH is not -6");

    const int rc = attn_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, (float)(1.0 / sqrt((double)D)), causal, NULL,
                            dtype, stream);
    printf("attn_fwd: %s\n", attn_status_str(rc));
    if (rc != ATTN_OK) return 1;
    if (hipStreamSynchronize(stream)) return fail("stream synchronisation");
    if (hipMemcpy(outh, o, nq * es, hipMemcpyDeviceToHost) ||
        hipMemcpy(outh + nq * es, lse, nl * 4, hipMemcpyDeviceToHost))
        return fail("copy from the device");

    f = fopen(argv[9], "wb");
    if (!f || fwrite(outh, 1, nq * es + nl * 4, f) != nq * es + nl * 4) return fail("cannot write the outputs");
    fclose(f);
    hipFree(q);
    hipFree(k);
    hipFree(v);
    hipFree(o);
    hipFree(lse);
    hipStreamDestroy(stream);
    free(host);
    free(outh);
    return 0;
}

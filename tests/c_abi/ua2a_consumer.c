/*
 * A plain C program using only include/ua2a.h, libua2a.so and the HIP
 * runtime API: the C ABI needs no Python or torch.  Test infrastructure.
 *
 *   ua2a_consumer OUT_DIR
 *
 * For two shapes (one taking the direct path, one the LDS path) it fills a
 * device buffer with each element's own flat index (uint32), runs mode 0
 * unchunked, writes the result to OUT_DIR/case<k>_mode0.bin for the test to
 * compare with the oracle, runs mode 1 chunked on that result and checks the
 * round trip returns the input.  The same mode-0 exchange then runs between
 * per-rank allocations (every sender in one call, then one call per sender)
 * and as a publishing exchange whose readiness credits a second stream waits
 * for before copying the output; each must equal the stacked result.  It
 * also checks a few error paths.  Exit 0 and "c-abi ok" on success.
 */
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ua2a.h"

#define HIP_OK(x)                                                                 \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "HIP %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                             \
        }                                                                         \
    } while (0)

#define UA_OK(x)                                                                          \
    do {                                                                                  \
        int s_ = (x);                                                                     \
        if (s_ != UA2A_OK) {                                                              \
            fprintf(stderr, "ua2a %d (%s) at line %d\n", s_, ua2a_status_string(s_), __LINE__); \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

static int ranks_and_credits(ua2a_plan_t plan, int32_t w, const ua2a_layout_t* lay,
                             const void* in, const void* out_ref, hipStream_t stream)
{
    const size_t bytes = (size_t)lay->tensor_bytes, rank = bytes / (size_t)w;
    void* ins[64];
    void* outs[64];
    char* ref = (char*)malloc(bytes);
    char* got = (char*)malloc(bytes);
    if (!ref || !got || w > 64) return 1;
    HIP_OK(hipMemcpy(ref, out_ref, bytes, hipMemcpyDeviceToHost));
    for (int r = 0; r < w; ++r) {
        HIP_OK(hipMalloc(&ins[r], rank));
        HIP_OK(hipMalloc(&outs[r], rank));
        HIP_OK(hipMemcpy(ins[r], (const char*)in + (size_t)r * rank, rank, hipMemcpyDeviceToDevice));
    }
    for (int pass = 0; pass < 2; ++pass) {
        for (int r = 0; r < w; ++r) HIP_OK(hipMemset(outs[r], 0xFF, rank));
        if (pass == 0) {
            UA_OK(ua2a_exchange_ranks(plan, 0, (const void* const*)ins, outs, 0, w, stream));
        } else {
            for (int j = 0; j < w; ++j)
                UA_OK(ua2a_exchange_ranks(plan, 0, (const void* const*)ins, outs, j, 1, stream));
        }
        HIP_OK(hipStreamSynchronize(stream));
        for (int r = 0; r < w; ++r)
            HIP_OK(hipMemcpy(got + (size_t)r * rank, outs[r], rank, hipMemcpyDeviceToHost));
        if (memcmp(got, ref, bytes) != 0) {
            fprintf(stderr, "per-rank exchange (pass %d) differs\n", pass);
            return 1;
        }
    }
    /* publishing exchange: a second stream waits for every receiver's credit, then copies */
    void *pub, *copy;
    uint32_t* credits;
    int32_t* status;
    hipStream_t side;
    uint32_t cr[64];
    int32_t st = -1;
    HIP_OK(hipMalloc(&pub, bytes));
    HIP_OK(hipMalloc(&copy, bytes));
    HIP_OK(hipMalloc((void**)&credits, (size_t)w * sizeof(uint32_t)));
    HIP_OK(hipMalloc((void**)&status, sizeof(int32_t)));
    HIP_OK(hipMemset(credits, 0, (size_t)w * sizeof(uint32_t)));
    HIP_OK(hipMemset(status, 0, sizeof(int32_t)));
    HIP_OK(hipStreamCreate(&side));
    HIP_OK(hipDeviceSynchronize());
    UA_OK(ua2a_exchange_publish(plan, 0, in, pub, credits, w, stream));
    UA_OK(ua2a_wait_credits(credits, 0, w, 1, 1u << 22, status, side));
    HIP_OK(hipMemcpyAsync(copy, pub, bytes, hipMemcpyDeviceToDevice, side));
    HIP_OK(hipStreamSynchronize(side));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(cr, credits, (size_t)w * sizeof(uint32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&st, status, sizeof(int32_t), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(got, copy, bytes, hipMemcpyDeviceToHost));
    if (st != 0 || memcmp(got, ref, bytes) != 0) {
        fprintf(stderr, "publishing exchange differs (wait status %d)\n", st);
        return 1;
    }
    for (int r = 0; r < w; ++r)
        if (cr[r] != 1) {
            fprintf(stderr, "receiver %d holds credit %u, want 1\n", r, cr[r]);
            return 1;
        }
    HIP_OK(hipStreamDestroy(side));
    HIP_OK(hipFree(pub));
    HIP_OK(hipFree(copy));
    HIP_OK(hipFree(credits));
    HIP_OK(hipFree(status));
    for (int r = 0; r < w; ++r) {
        HIP_OK(hipFree(ins[r]));
        HIP_OK(hipFree(outs[r]));
    }
    free(ref);
    free(got);
    return 0;
}

static int run_case(int k, int32_t w, int64_t B, int64_t S, int64_t H, int64_t D, const char* dir)
{
    ua2a_layout_t lay;
    UA_OK(ua2a_layout(w, B, S, H, D, 4, &lay));
    const size_t n = (size_t)lay.tensor_elems, bytes = (size_t)lay.tensor_bytes;
    uint32_t* host = (uint32_t*)malloc(bytes);
    uint32_t* back = (uint32_t*)malloc(bytes);
    if (!host || !back) return 1;
    for (size_t i = 0; i < n; ++i) host[i] = (uint32_t)i;
    void *in, *out, *rt, *win;
    HIP_OK(hipMalloc(&in, bytes));
    HIP_OK(hipMalloc(&out, bytes));
    HIP_OK(hipMalloc(&rt, bytes));
    HIP_OK(hipMalloc(&win, (size_t)lay.window_bytes));
    HIP_OK(hipMemcpy(in, host, bytes, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    ua2a_plan_t plan;
    UA_OK(ua2a_plan(&plan, w, B, S, H, D, 4, 0, win, lay.window_bytes, 0));
    ua2a_launch_info_t info;
    UA_OK(ua2a_describe(plan, 0, 0, in, out, &info));
    UA_OK(ua2a_exchange(plan, 0, 0, in, out, stream));
    UA_OK(ua2a_exchange(plan, 1, 1, out, rt, stream));      /* chunked inverse */
    HIP_OK(hipStreamSynchronize(stream));

    /* mode 0 result for the oracle comparison */
    HIP_OK(hipMemcpy(back, out, bytes, hipMemcpyDeviceToHost));
    char path[4096];
    snprintf(path, sizeof path, "%s/case%d_mode0.bin", dir, k);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(back, 1, bytes, f) != bytes) return 1;
    fclose(f);
    /* round trip */
    HIP_OK(hipMemcpy(back, rt, bytes, hipMemcpyDeviceToHost));
    if (memcmp(back, host, bytes) != 0) {
        fprintf(stderr, "case %d: round trip differs\n", k);
        return 1;
    }
    if (ranks_and_credits(plan, w, &lay, in, out, stream)) return 1;
    /* error paths leave the plan usable */
    if (ua2a_exchange(plan, 0, 0, in, in, stream) != UA2A_ERR_ALIAS) return 1;
    if (ua2a_exchange(plan, 2, 0, in, out, stream) != UA2A_ERR_INVALID_ARG) return 1;
    if (ua2a_exchange(plan, 0, 0, (const char*)in + 2, out, stream) != UA2A_ERR_ALIGN) return 1;
    if (ua2a_plan_last_error(plan)[0] != '\0') return 1;
    UA_OK(ua2a_exchange(plan, 0, 1, in, out, stream));
    HIP_OK(hipStreamSynchronize(stream));
    printf("case %d: w=%d B=%lld S=%lld H=%lld D=%lld path=%d vector=%d grid=%lld -> ok\n", k, w,
           (long long)B, (long long)S, (long long)H, (long long)D, info.path, info.vector_bytes,
           (long long)info.grid);
    UA_OK(ua2a_destroy(plan));
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(in));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(rt));
    HIP_OK(hipFree(win));
    free(host);
    free(back);
    return 0;
}

int main(int argc, char** argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT_DIR\n", argv[0]);
        return 2;
    }
    if (run_case(0, 4, 1, 300, 8, 64, argv[1])) return 1;     /* run 256 B: direct path */
    if (run_case(1, 3, 2, 37, 6, 5, argv[1])) return 1;       /* run 40 B: LDS path */
    printf("c-abi ok\n");
    return 0;
}

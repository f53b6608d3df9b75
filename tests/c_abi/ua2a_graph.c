/*
 * HIP-graph capture of the exchange through the C ABI alone (no Python or
 * torch in the process).  Test infrastructure.
 *
 *   ua2a_graph OUT_DIR
 *
 * For each case (the tiny and mid workloads' shapes, 2-byte elements filled
 * with their flat index modulo 2^16) it captures `pairs` exchange pairs
 * (mode 0, then mode 1 on its output) on one stream with
 * hipStreamBeginCapture / hipStreamEndCapture, instantiates the graph, and
 *   - replays it 3 times with the outputs poisoned in between, checking that
 *     every replay returns the input and writing the first replay's mode-0
 *     output to OUT_DIR/graph<k>_mode0.bin for the test to compare with the
 *     oracle;
 *   - times K back-to-back replays (hipGraphLaunch) against K back-to-back
 *     eager calls of the same exchanges, with events on the stream, and the
 *     host time each takes to enqueue;
 *   - times one replay and one eager step each followed by a stream
 *     synchronisation (the latency a decode loop sees).
 * One JSON line per case and pair count; "graph ok" at the end on success.
 */
#define _POSIX_C_SOURCE 199309L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include <hip/hip_runtime_api.h>

#include "ua2a.h"

#define HIP_OK(x)                                                                      \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP %s at line %d\n", hipGetErrorString(e_), __LINE__);   \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

#define UA_OK(x)                                                                               \
    do {                                                                                       \
        int s_ = (x);                                                                          \
        if (s_ != UA2A_OK) {                                                                   \
            fprintf(stderr, "ua2a %d (%s) at line %d\n", s_, ua2a_status_string(s_), __LINE__); \
            return 1;                                                                          \
        }                                                                                      \
    } while (0)

enum { K = 200, MAX_PAIRS = 8 };

static double now_us(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return ts.tv_sec * 1e6 + ts.tv_nsec * 1e-3;
}

/* `pairs` exchange pairs, each from its own buffer set: in[i] -> out[i] -> rt[i] */
static int enqueue_pairs(ua2a_plan_t plan, int pairs, void** in, void** out, void** rt, hipStream_t s)
{
    for (int i = 0; i < pairs; ++i) {
        UA_OK(ua2a_exchange(plan, 0, 0, in[i], out[i], s));
        UA_OK(ua2a_exchange(plan, 1, 0, out[i], rt[i], s));
    }
    return 0;
}

static int run_case(int k, const char* name, int32_t w, int64_t B, int64_t S, int64_t H, int64_t D,
                    int pairs, const char* dir)
{
    ua2a_layout_t lay;
    UA_OK(ua2a_layout(w, B, S, H, D, 2, &lay));
    const size_t n = (size_t)lay.tensor_elems, bytes = (size_t)lay.tensor_bytes;
    uint16_t* host = (uint16_t*)malloc(bytes);
    uint16_t* back = (uint16_t*)malloc(bytes);
    if (!host || !back) return 1;
    for (size_t i = 0; i < n; ++i) host[i] = (uint16_t)(i & 0xFFFF);
    void *in[MAX_PAIRS], *out[MAX_PAIRS], *rt[MAX_PAIRS];
    for (int i = 0; i < pairs; ++i) {
        HIP_OK(hipMalloc(&in[i], bytes));
        HIP_OK(hipMalloc(&out[i], bytes));
        HIP_OK(hipMalloc(&rt[i], bytes));
        HIP_OK(hipMemcpy(in[i], host, bytes, hipMemcpyHostToDevice));
    }
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    ua2a_plan_t plan;
    UA_OK(ua2a_plan(&plan, w, B, S, H, D, 2, 0, NULL, 0, 0));

    /* capture */
    hipGraph_t graph;
    hipGraphExec_t exec;
    HIP_OK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    if (enqueue_pairs(plan, pairs, in, out, rt, s)) return 1;
    HIP_OK(hipStreamEndCapture(s, &graph));
    size_t nodes = 0;
    HIP_OK(hipGraphGetNodes(graph, NULL, &nodes));
    HIP_OK(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));

    /* replays, each checked; outputs poisoned in between (outside the graph) */
    for (int rep = 0; rep < 3; ++rep) {
        for (int i = 0; i < pairs; ++i) {
            HIP_OK(hipMemset(out[i], 0xFF, bytes));
            HIP_OK(hipMemset(rt[i], 0xFF, bytes));
        }
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipGraphLaunch(exec, s));
        HIP_OK(hipStreamSynchronize(s));
        for (int i = 0; i < pairs; ++i) {
            HIP_OK(hipMemcpy(back, rt[i], bytes, hipMemcpyDeviceToHost));
            if (memcmp(back, host, bytes) != 0) {
                fprintf(stderr, "%s: replay %d, pair %d did not return the input\n", name, rep, i);
                return 1;
            }
        }
        if (rep == 0 && pairs == 1) {
            HIP_OK(hipMemcpy(back, out[0], bytes, hipMemcpyDeviceToHost));
            char path[4096];
            snprintf(path, sizeof path, "%s/graph%d_mode0.bin", dir, k);
            FILE* f = fopen(path, "wb");
            if (!f || fwrite(back, 1, bytes, f) != bytes) return 1;
            fclose(f);
        }
    }

    /* K back-to-back: device time between events, host time to enqueue */
    hipEvent_t a, b;
    HIP_OK(hipEventCreate(&a));
    HIP_OK(hipEventCreate(&b));
    float ms_eager = 0, ms_graph = 0;
    for (int i = 0; i < 10; ++i) {
        if (enqueue_pairs(plan, pairs, in, out, rt, s)) return 1;
        HIP_OK(hipGraphLaunch(exec, s));
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipEventRecord(a, s));
    double h0 = now_us();
    for (int i = 0; i < K; ++i)
        if (enqueue_pairs(plan, pairs, in, out, rt, s)) return 1;
    double host_eager = (now_us() - h0) / K;
    HIP_OK(hipEventRecord(b, s));
    HIP_OK(hipEventSynchronize(b));
    HIP_OK(hipEventElapsedTime(&ms_eager, a, b));
    HIP_OK(hipEventRecord(a, s));
    h0 = now_us();
    for (int i = 0; i < K; ++i) HIP_OK(hipGraphLaunch(exec, s));
    double host_graph = (now_us() - h0) / K;
    HIP_OK(hipEventRecord(b, s));
    HIP_OK(hipEventSynchronize(b));
    HIP_OK(hipEventElapsedTime(&ms_graph, a, b));

    /* one step, then wait for it: what a loop that needs each result sees */
    double lat_eager = 0, lat_graph = 0;
    for (int i = 0; i < K; ++i) {
        h0 = now_us();
        if (enqueue_pairs(plan, pairs, in, out, rt, s)) return 1;
        HIP_OK(hipStreamSynchronize(s));
        lat_eager += now_us() - h0;
        h0 = now_us();
        HIP_OK(hipGraphLaunch(exec, s));
        HIP_OK(hipStreamSynchronize(s));
        lat_graph += now_us() - h0;
    }
    printf("{\"case\": \"%s\", \"pairs\": %d, \"kernels\": %d, \"graph_nodes\": %zu, "
           "\"eager_us\": %.2f, \"graph_us\": %.2f, \"eager_host_enqueue_us\": %.2f, "
           "\"graph_host_enqueue_us\": %.2f, \"eager_sync_us\": %.2f, \"graph_sync_us\": %.2f}\n",
           name, pairs, 2 * pairs, nodes, ms_eager * 1e3 / K, ms_graph * 1e3 / K, host_eager, host_graph,
           lat_eager / K, lat_graph / K);
    fflush(stdout);

    HIP_OK(hipGraphExecDestroy(exec));
    HIP_OK(hipGraphDestroy(graph));
    HIP_OK(hipEventDestroy(a));
    HIP_OK(hipEventDestroy(b));
    UA_OK(ua2a_destroy(plan));
    HIP_OK(hipStreamDestroy(s));
    for (int i = 0; i < pairs; ++i) {
        HIP_OK(hipFree(in[i]));
        HIP_OK(hipFree(out[i]));
        HIP_OK(hipFree(rt[i]));
    }
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
    HIP_OK(hipSetDevice(0));
    static const int pair_counts[] = {1, 4};
    for (int p = 0; p < 2; ++p) {
        if (run_case(0, "tiny", 2, 1, 8, 4, 16, pair_counts[p], argv[1])) return 1;
        if (run_case(1, "mid", 4, 1, 1024, 24, 128, pair_counts[p], argv[1])) return 1;
    }
    printf("graph ok\n");
    return 0;
}

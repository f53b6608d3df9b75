/*
 * Plain CPU oracle of the Ulysses all_to_all_4D head/sequence exchange.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no header, helper or constant
 * with the HIP library; it takes its own shape arguments.
 *
 * What it computes (FastVideo "ulysses_a2a" API page, method run_armed):
 *   - mode 0 ("scatter heads, gather sequence"): each of the w ranks holds
 *     x[B, S_local, H, D]; afterwards each rank holds [B, S_local*w, H/w, D].
 *   - mode 1 (the inverse): each rank holds [B, S_global, H_local, D] with
 *     S_global = S_local*w, H_local = H/w; afterwards [B, S_local, H, D].
 *   - chunked: the same exchange issued once per batch plane on the slices
 *     x[plane:plane+1] / out[plane:plane+1] (same method, chunked branch),
 *     each plane passing through a window sized for one plane.
 *
 * Readings of the page (it prints only shapes):
 *   - rank r receives the contiguous head block [r*H/w, (r+1)*H/w);
 *   - the gathered sequence is rank-major: token s of source rank j lands at
 *     global position j*S_local + s (the order an all-to-all concatenation
 *     of the per-rank chunks gives, which the fused path must reproduce since
 *     the same page falls back to the framework's all-to-all on decline);
 *   - H must be a multiple of w (the page floors H // w silently; we reject).
 *
 * The w rank tensors are stacked rank-major in one buffer:
 *   mode-0 side  [w][B][S_local][H][D]
 *   mode-1 side  [w][B][S_local*w][H/w][D]
 * Elements are copied as raw elem_bytes-byte patterns; no value is ever
 * interpreted, so NaN payloads, signed zeros and denormals pass unchanged.
 *
 * Return codes: 0 ok, -1 bad argument (null pointer, elem_bytes not in
 * {1,2,4,8}, mode not in {0,1}), -2 bad shape (a dimension < 1 or H % w != 0),
 * -9 out of host memory (chunked scratch).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int check_args(int32_t w, int64_t B, int64_t S_local, int64_t H,
                      int64_t D, int32_t elem_bytes, const void* in,
                      const void* out)
{
    if (in == NULL || out == NULL) return -1;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
        return -1;
    if (w < 1 || B < 1 || S_local < 1 || H < 1 || D < 1) return -2;
    if (H % w != 0) return -2;
    return 0;
}

/* Mode 0, destination order: out[r][b][j*S_local+s][h][d] = in[j][b][s][r*Hl+h][d]. */
int ua2a_oracle_mode0(int32_t w, int64_t B, int64_t S_local, int64_t H,
                      int64_t D, int32_t elem_bytes, const void* in, void* out)
{
    int rc = check_args(w, B, S_local, H, D, elem_bytes, in, out);
    if (rc != 0) return rc;
    const int64_t Hl = H / w;
    const int64_t S_global = S_local * w;
    const size_t e = (size_t)elem_bytes;
    const unsigned char* src = (const unsigned char*)in;
    unsigned char* dst = (unsigned char*)out;

    for (int64_t r = 0; r < w; ++r)                   /* receiving rank */
        for (int64_t b = 0; b < B; ++b)               /* batch plane */
            for (int64_t j = 0; j < w; ++j)           /* sending rank */
                for (int64_t s = 0; s < S_local; ++s) /* sender's token */
                    for (int64_t h = 0; h < Hl; ++h)  /* head within r's block */
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t si = (((j * B + b) * S_local + s) * H + (r * Hl + h)) * D + d;
                            int64_t di = (((r * B + b) * S_global + (j * S_local + s)) * Hl + h) * D + d;
                            memcpy(dst + (size_t)di * e, src + (size_t)si * e, e);
                        }
    return 0;
}

/* Mode 1, destination order: out[j][b][s][r*Hl+h][d] = in[r][b][j*S_local+s][h][d].
 * Shape arguments are the mode-0-side (local) ones, as the page derives
 * S_local = S_global // w and H = H_local * w before the native call. */
int ua2a_oracle_mode1(int32_t w, int64_t B, int64_t S_local, int64_t H,
                      int64_t D, int32_t elem_bytes, const void* in, void* out)
{
    int rc = check_args(w, B, S_local, H, D, elem_bytes, in, out);
    if (rc != 0) return rc;
    const int64_t Hl = H / w;
    const int64_t S_global = S_local * w;
    const size_t e = (size_t)elem_bytes;
    const unsigned char* src = (const unsigned char*)in;
    unsigned char* dst = (unsigned char*)out;

    for (int64_t j = 0; j < w; ++j)                   /* receiving rank (owner of tokens) */
        for (int64_t b = 0; b < B; ++b)
            for (int64_t s = 0; s < S_local; ++s)
                for (int64_t r = 0; r < w; ++r)       /* sending rank (owner of heads) */
                    for (int64_t h = 0; h < Hl; ++h)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t si = (((r * B + b) * S_global + (j * S_local + s)) * Hl + h) * D + d;
                            int64_t di = (((j * B + b) * S_local + s) * H + (r * Hl + h)) * D + d;
                            memcpy(dst + (size_t)di * e, src + (size_t)si * e, e);
                        }
    return 0;
}

/* Chunked variant: for every batch plane, gather plane p of each rank into a
 * one-plane send buffer, run the exchange with B = 1 into a one-plane
 * receive window, then copy the window into plane p of each rank's output. */
int ua2a_oracle_chunked(int32_t mode, int32_t w, int64_t B, int64_t S_local,
                        int64_t H, int64_t D, int32_t elem_bytes,
                        const void* in, void* out)
{
    int rc = check_args(w, B, S_local, H, D, elem_bytes, in, out);
    if (rc != 0) return rc;
    if (mode != 0 && mode != 1) return -1;
    /* one plane of one rank has the same element count on both sides */
    const size_t plane_bytes = (size_t)(S_local * H * D) * (size_t)elem_bytes;
    unsigned char* send = (unsigned char*)malloc(plane_bytes * (size_t)w);
    unsigned char* window = (unsigned char*)malloc(plane_bytes * (size_t)w);
    if (send == NULL || window == NULL) {
        free(send);
        free(window);
        return -9;
    }
    const unsigned char* src = (const unsigned char*)in;
    unsigned char* dst = (unsigned char*)out;
    for (int64_t p = 0; p < B; ++p) {
        for (int64_t k = 0; k < w; ++k)
            memcpy(send + (size_t)k * plane_bytes,
                   src + ((size_t)(k * B + p)) * plane_bytes, plane_bytes);
        rc = (mode == 0)
                 ? ua2a_oracle_mode0(w, 1, S_local, H, D, elem_bytes, send, window)
                 : ua2a_oracle_mode1(w, 1, S_local, H, D, elem_bytes, send, window);
        if (rc != 0) break;
        for (int64_t k = 0; k < w; ++k)
            memcpy(dst + ((size_t)(k * B + p)) * plane_bytes,
                   window + (size_t)k * plane_bytes, plane_bytes);
    }
    free(send);
    free(window);
    return rc;
}

/* Per-rank allocations, restricted to the runs that ranks [first,
 * first+count) send.  in[k] and out[k] are the separate tensors of rank k
 * (the rank-stacked layouts above without the leading w); in[] is indexed by
 * the sending rank (mode 0: token owner j, mode 1: head-block owner r), out[]
 * by the receiving rank.  Only senders' inputs are read (other entries may be
 * NULL); output elements whose source rank lies outside the range are left
 * untouched.  Same page and method as the unrestricted exchange, read for a
 * device communicator whose ranks each own their buffers; (0, w) is the
 * whole exchange. */
int ua2a_oracle_ranks(int32_t mode, int32_t w, int64_t B, int64_t S_local, int64_t H,
                      int64_t D, int32_t elem_bytes, const void* const* in, void* const* out,
                      int32_t first, int32_t count)
{
    if (in == NULL || out == NULL) return -1;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return -1;
    if (mode != 0 && mode != 1) return -1;
    if (w < 1 || B < 1 || S_local < 1 || H < 1 || D < 1 || H % w != 0) return -2;
    if (first < 0 || count < 1 || first + count > w) return -1;
    for (int32_t k = first; k < first + count; ++k)
        if (in[k] == NULL) return -1;
    for (int32_t k = 0; k < w; ++k)
        if (out[k] == NULL) return -1;
    const int64_t Hl = H / w;
    const int64_t S_global = S_local * w;
    const size_t e = (size_t)elem_bytes;

    if (mode == 0) {
        for (int64_t r = 0; r < w; ++r)                          /* receiving rank */
            for (int64_t b = 0; b < B; ++b)
                for (int64_t j = first; j < first + count; ++j)  /* sending rank */
                    for (int64_t s = 0; s < S_local; ++s)
                        for (int64_t h = 0; h < Hl; ++h)
                            for (int64_t d = 0; d < D; ++d) {
                                int64_t si = ((b * S_local + s) * H + (r * Hl + h)) * D + d;
                                int64_t di = ((b * S_global + (j * S_local + s)) * Hl + h) * D + d;
                                memcpy((unsigned char*)out[r] + (size_t)di * e,
                                       (const unsigned char*)in[j] + (size_t)si * e, e);
                            }
    } else {
        for (int64_t j = 0; j < w; ++j)                          /* receiving rank */
            for (int64_t b = 0; b < B; ++b)
                for (int64_t s = 0; s < S_local; ++s)
                    for (int64_t r = first; r < first + count; ++r)   /* sending rank */
                        for (int64_t h = 0; h < Hl; ++h)
                            for (int64_t d = 0; d < D; ++d) {
                                int64_t si = ((b * S_global + (j * S_local + s)) * Hl + h) * D + d;
                                int64_t di = ((b * S_local + s) * H + (r * Hl + h)) * D + d;
                                memcpy((unsigned char*)out[j] + (size_t)di * e,
                                       (const unsigned char*)in[r] + (size_t)si * e, e);
                            }
    }
    return 0;
}

/* The exchange between per-rank allocations in two steps, pack then unpack,
 * through one receive window per receiving rank.  In a multi-device exchange
 * each sender pushes its share into every receiver's registered window and
 * each receiver then moves its window into its own output, which never
 * aliases the window (same page, method run_armed: saved activations never
 * alias the reusable window).  Reading: the window of receiver q has the
 * layout of one rank's sequence-gathered tensor, [B][w*S_local][H/w][D], and
 * its token block k of plane b, [k*S_local, (k+1)*S_local), holds what
 * sender k sends q, so every sender's share is one contiguous block per
 * plane.
 *
 * Pack, senders [first, first+count): win[q][b][k*S_local+s][h][d] =
 *   mode 0: in[k][b][s][q*Hl+h][d]       (in[k]: [B][S_local][H][D])
 *   mode 1: in[k][b][q*S_local+s][h][d]  (in[k]: [B][S_local*w][Hl][D])
 * for every receiver q; other window elements are left untouched.
 * Unpack, receivers [first, first+count): out[q] from win[q] =
 *   mode 0: out[q][b][t][h][d] = win[q][b][t][h][d]  (out[q]: [B][S_local*w][Hl][D])
 *   mode 1: out[q][b][s][k*Hl+h][d] = win[q][b][k*S_local+s][h][d]  (out[q]: [B][S_local][H][D])
 * Pack by every sender followed by unpack of every receiver is the exchange
 * of ua2a_oracle_ranks with every rank sending. */
static int check_ranks_args(int32_t mode, int32_t w, int64_t B, int64_t S_local, int64_t H, int64_t D,
                            int32_t elem_bytes, const void* const* in, void* const* out,
                            int32_t first, int32_t count)
{
    if (in == NULL || out == NULL) return -1;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return -1;
    if (mode != 0 && mode != 1) return -1;
    if (w < 1 || B < 1 || S_local < 1 || H < 1 || D < 1 || H % w != 0) return -2;
    if (first < 0 || count < 1 || first + count > w) return -1;
    return 0;
}

int ua2a_oracle_pack_ranks(int32_t mode, int32_t w, int64_t B, int64_t S_local, int64_t H,
                           int64_t D, int32_t elem_bytes, const void* const* in, void* const* win,
                           int32_t first, int32_t count)
{
    int rc = check_ranks_args(mode, w, B, S_local, H, D, elem_bytes, in, win, first, count);
    if (rc != 0) return rc;
    for (int32_t k = first; k < first + count; ++k)
        if (in[k] == NULL) return -1;
    for (int32_t q = 0; q < w; ++q)
        if (win[q] == NULL) return -1;
    const int64_t Hl = H / w;
    const int64_t S_global = S_local * w;
    const size_t e = (size_t)elem_bytes;
    for (int64_t q = 0; q < w; ++q)                              /* receiving rank */
        for (int64_t b = 0; b < B; ++b)
            for (int64_t k = first; k < first + count; ++k)      /* sending rank */
                for (int64_t s = 0; s < S_local; ++s)
                    for (int64_t h = 0; h < Hl; ++h)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t si = mode == 0 ? ((b * S_local + s) * H + (q * Hl + h)) * D + d
                                                   : ((b * S_global + (q * S_local + s)) * Hl + h) * D + d;
                            int64_t wi = ((b * S_global + (k * S_local + s)) * Hl + h) * D + d;
                            memcpy((unsigned char*)win[q] + (size_t)wi * e,
                                   (const unsigned char*)in[k] + (size_t)si * e, e);
                        }
    return 0;
}

int ua2a_oracle_unpack_ranks(int32_t mode, int32_t w, int64_t B, int64_t S_local, int64_t H,
                             int64_t D, int32_t elem_bytes, const void* const* win, void* const* out,
                             int32_t first, int32_t count)
{
    int rc = check_ranks_args(mode, w, B, S_local, H, D, elem_bytes, win, out, first, count);
    if (rc != 0) return rc;
    for (int32_t q = first; q < first + count; ++q)
        if (win[q] == NULL || out[q] == NULL) return -1;
    const int64_t Hl = H / w;
    const int64_t S_global = S_local * w;
    const size_t e = (size_t)elem_bytes;
    for (int64_t q = first; q < first + count; ++q)              /* receiving rank */
        for (int64_t b = 0; b < B; ++b)
            for (int64_t k = 0; k < w; ++k)                      /* sending rank */
                for (int64_t s = 0; s < S_local; ++s)
                    for (int64_t h = 0; h < Hl; ++h)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t wi = ((b * S_global + (k * S_local + s)) * Hl + h) * D + d;
                            int64_t di = mode == 0 ? wi : ((b * S_local + s) * H + (k * Hl + h)) * D + d;
                            memcpy((unsigned char*)out[q] + (size_t)di * e,
                                   (const unsigned char*)win[q] + (size_t)wi * e, e);
                        }
    return 0;
}

/* Flat position in the rank-stacked input of the element that the exchange
 * (mode 0 or 1) writes at flat position out_index of the output: the
 * definitions above, for one element at a time (used to check outputs too
 * large for a whole CPU copy).  -1 on a bad argument or an index out of
 * range. */
int64_t ua2a_oracle_source_index(int32_t mode, int32_t w, int64_t B, int64_t S_local,
                                 int64_t H, int64_t D, int64_t out_index)
{
    if (w < 1 || B < 1 || S_local < 1 || H < 1 || D < 1 || H % w != 0) return -1;
    if (mode != 0 && mode != 1) return -1;
    const int64_t Hl = H / w;
    const int64_t S_global = S_local * w;
    if (out_index < 0 || out_index >= (int64_t)w * B * S_local * H * D) return -1;
    int64_t i = out_index;
    const int64_t d = i % D;
    i /= D;
    if (mode == 0) {                       /* out[r][b][t][h][d], t = j*S_local + s */
        const int64_t h = i % Hl;
        i /= Hl;
        const int64_t t = i % S_global;
        i /= S_global;
        const int64_t b = i % B;
        const int64_t r = i / B;
        const int64_t j = t / S_local, s = t % S_local;
        return (((j * B + b) * S_local + s) * H + (r * Hl + h)) * D + d;
    }
    /* mode 1: out[j][b][s][hh][d], hh = r*Hl + h */
    const int64_t hh = i % H;
    i /= H;
    const int64_t s = i % S_local;
    i /= S_local;
    const int64_t b = i % B;
    const int64_t j = i / B;
    const int64_t r = hh / Hl, h = hh % Hl;
    return (((r * B + b) * S_global + (j * S_local + s)) * Hl + h) * D + d;
}

/* ua2a_oracle_source_index for n output positions. Returns 0, or -1 if any
 * argument or index is out of range. */
int ua2a_oracle_source_indices(int32_t mode, int32_t w, int64_t B, int64_t S_local, int64_t H,
                               int64_t D, const int64_t* out_index, int64_t n, int64_t* src)
{
    if (out_index == NULL || src == NULL || n < 0) return -1;
    for (int64_t k = 0; k < n; ++k) {
        src[k] = ua2a_oracle_source_index(mode, w, B, S_local, H, D, out_index[k]);
        if (src[k] < 0) return -1;
    }
    return 0;
}

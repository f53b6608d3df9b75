/*
 * ua2a.h -- C ABI of the MI355X (gfx950) Ulysses all_to_all_4D exchange.
 *
 * The operation (FastVideo "ulysses_a2a" API page, method run_armed):
 *   w ranks each hold x[B, S_local, H, D].
 *   mode 0 ("scatter heads, gather sequence"): rank r ends with
 *       out_r[b][j*S_local + s][h][d] = x_j[b][s][r*(H/w) + h][d]
 *     i.e. [B, S_local*w, H/w, D]: the full sequence, gathered from all
 *     ranks in rank order, for its own contiguous block of H/w heads.
 *   mode 1 (the inverse, same page): rank j holds y_j[B, S_global, H/w, D]
 *     with S_global = S_local*w and ends with [B, S_local, H, D]:
 *       out_j[b][s][r*(H/w) + h][d] = y_r[b][j*S_local + s][h][d].
 *   chunked (same method, chunked branch): the exchange is issued once per
 *     batch plane, each plane passing through a window sized for one plane;
 *     the result is identical to the unchunked call.
 *
 * All w "virtual ranks" live on ONE device, stacked rank-major in one
 * allocation per tensor:
 *   mode-0 side ("head-complete")     [w][B][S_local][H][D]
 *   mode-1 side ("sequence-gathered") [w][B][S_local*w][H/w][D]
 * Both are dense, row-major, no padding.  Elements are moved as raw
 * elem_bytes-byte patterns (bf16/fp16 = 2, fp32 = 4, ...): the result is a
 * bit-exact permutation of the input for every dtype.
 *
 * Conventions for every function below:
 *   - return 0 (UA2A_OK) or a negative UA2A_ERR_* code; nothing throws;
 *   - no function synchronises the host with the device;
 *   - no function allocates device memory; the ones that launch work
 *     (ua2a_exchange, ua2a_exchange_chunked_noalloc, ua2a_exchange_ranks,
 *     ua2a_pack_ranks, ua2a_unpack_ranks, ua2a_exchange_publish,
 *     ua2a_wait_credits) launch only on the given stream;
 *   - pointers named in/out/window are device pointers on the plan's
 *     device, owned by the caller, and are only borrowed by the library;
 *   - kernels write only the bytes of out (and of the window and counters
 *     where a call names them); they may read an input's first or last
 *     aligned 16-byte chunk whole when the input starts or ends inside it,
 *     and never use the bytes outside the input (an aligned 16-byte chunk
 *     lies within one page, so such a read cannot fault).
 */
#ifndef UA2A_H
#define UA2A_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
#define UA2A_OK                0
#define UA2A_ERR_INVALID_ARG  (-1) /* null pointer, mode/chunked not 0/1, bad elem_bytes, bad path */
#define UA2A_ERR_SHAPE        (-2) /* a dimension < 1, H % w != 0, or a size beyond the limits below */
#define UA2A_ERR_ALIGN        (-3) /* a tensor or window pointer not aligned to elem_bytes */
#define UA2A_ERR_ALIAS        (-4) /* byte ranges of inputs, outputs, window or counters overlap */
#define UA2A_ERR_CAPACITY     (-5) /* chunked call with no window or one smaller than one plane */
#define UA2A_ERR_DEVICE       (-6) /* the calling thread's current device is not the plan's */
#define UA2A_ERR_HIP          (-7) /* a HIP runtime or launch call failed: the plan is now disabled */
#define UA2A_ERR_DISABLED     (-8) /* the plan was disabled by an earlier UA2A_ERR_HIP */
#define UA2A_ERR_NOMEM        (-9) /* host allocation of the plan object failed */

/* Limits (UA2A_ERR_SHAPE beyond them): w <= 65536; each of B, S_local, H,
 * D <= 2^31 - 1; one token of all heads (H*D*elem_bytes) <= 2^31 bytes; one
 * batch plane of one rank (S_local*H*D*elem_bytes) < 2^32 bytes;
 * w*w*B*S_local < 2^32; one rank-stacked tensor <= 2^38 bytes (256 GiB). */

typedef struct ua2a_plan_s* ua2a_plan_t;

/* Sizes derived from a shape (host only; see ua2a_layout). */
typedef struct ua2a_layout_s {
    int64_t H_local;       /* H / w: heads each rank keeps in mode 0 */
    int64_t S_global;      /* S_local * w */
    int64_t run_bytes;     /* H_local * D * elem_bytes: one token's slice of one head block,
                              the unit that stays contiguous on both sides */
    int64_t tensor_elems;  /* w * B * S_local * H * D (input and output alike) */
    int64_t tensor_bytes;  /* tensor_elems * elem_bytes */
    int64_t window_bytes;  /* w * S_local * H * D * elem_bytes: one batch plane of every rank,
                              the least window a chunked call accepts */
    int64_t moved_bytes;   /* 2 * tensor_bytes: every element read once and written once */
} ua2a_layout_t;

/* Which kernel family runs an exchange (ua2a_plan_set_path, ua2a_describe). */
/* UA2A_PATH_AUTO (default) takes the direct path when runs are whole 128-byte
 * lines and the bases are 16-byte aligned (mode 1: when each 1 KiB tile reads at
 * least 256 contiguous bytes per head block, or, for runs that are multiples of
 * 16 bytes, when an unchunked launch moves under 80 MiB a side), the LDS path
 * otherwise; ua2a_describe reports the choice. */
#define UA2A_PATH_AUTO    0  /* the library chooses (default) */
#define UA2A_PATH_DIRECT  1  /* one pass, each lane moves whole vectors of a run */
#define UA2A_PATH_LDS     2  /* rows staged through LDS, both sides moved as contiguous spans */

/* How a chunked exchange is launched (ua2a_launch_info_t.chunked_form): one
 * launch of the chunked kernel (direct path) or of the chunked LDS kernel. */
#define UA2A_CHUNKED_ONE_LAUNCH  1

/* What an exchange would launch (ua2a_describe). */
typedef struct ua2a_launch_info_s {
    int32_t path;          /* UA2A_PATH_DIRECT or UA2A_PATH_LDS */
    int32_t vector_bytes;  /* bytes per lane access of the permutation kernel (1..16) */
    int32_t block;         /* threads per workgroup */
    int32_t launches;      /* kernel launches per exchange: 1, chunked or not */
    int64_t grid;          /* workgroups of the permutation kernel per launch (all dimensions) */
    int64_t tiles;         /* work tiles per launch */
    int32_t lds_rows;      /* rows per LDS tile (LDS path), else 0 */
    int32_t grid_dims;     /* 3: a 3-D grid (direct path by default, every per-rank launch); else 1 */
    int32_t chunked_form;  /* 0: not chunked; else UA2A_CHUNKED_ONE_LAUNCH */
    int32_t lds_bytes;     /* dynamic LDS per workgroup (LDS path), else 0 */
    int32_t lds_planes;    /* chunked LDS path: batch planes held in LDS at once (1..B), else 0 */
} ua2a_launch_info_t;

/*
 * ua2a_layout: validate a shape and fill *layout.  Host only, no device call.
 *   w           virtual ranks (>= 1)
 *   B, S_local, H, D   the mode-0-side (local) shape, as the page passes it to
 *               the native call in both modes (mode 1 derives S_local and H
 *               from [B, S_global, H_local, D] first)
 *   elem_bytes  1, 2, 4 or 8
 * Errors: INVALID_ARG (layout NULL, elem_bytes), SHAPE.
 */
int ua2a_layout(int32_t w, int64_t B, int64_t S_local, int64_t H, int64_t D,
                int32_t elem_bytes, ua2a_layout_t* layout);

/*
 * ua2a_plan: create a plan for one shape on one device.  Host only: it makes
 * no HIP call and allocates only the small host-side plan object.
 *   blocks      grid-size cap for the permutation kernel (the page passes
 *               `blocks` to the native op); 0 = one workgroup per work tile
 *               (the fastest shape on MI355X).  With a smaller cap each
 *               workgroup loops over several tiles.  The result never
 *               depends on it.
 *   window, window_bytes  caller-owned device buffer used by chunked calls
 *               as the one-plane receive window of all w ranks; it may be
 *               NULL/0 if chunked is never requested.  The plan borrows it:
 *               the caller keeps it alive and unchanged until ua2a_destroy.
 *               A bigger window needs a new plan (windows never shrink or
 *               grow in place, as on the page, where growth re-builds).
 *   device      HIP device ordinal the plan launches on.
 * Errors: INVALID_ARG (plan_out NULL, device < 0, blocks < 0, window_bytes
 * < 0, window NULL with window_bytes > 0), SHAPE, ALIGN (window not
 * elem_bytes-aligned), NOMEM.  *plan_out is NULL on error.
 */
int ua2a_plan(ua2a_plan_t* plan_out, int32_t w, int64_t B, int64_t S_local,
              int64_t H, int64_t D, int32_t elem_bytes, int32_t blocks,
              void* window, int64_t window_bytes, int32_t device);

/*
 * ua2a_exchange: enqueue one exchange on `stream` (a hipStream_t; NULL = the
 * device's null stream) and return without waiting.
 *   mode     0 or 1 (see the top of this file)
 *   chunked  0: one permutation launch over all B planes;
 *            1: per plane p, a permutation of plane p of every rank into the
 *               window, then a copy of the window into plane p of `out`;
 *               plane p+1 overwrites a window byte only after plane p's copy
 *               has read it, and every byte of `out` is read from the
 *               window.  The whole exchange is ONE launch
 *               (UA2A_CHUNKED_ONE_LAUNCH).  On the direct path each
 *               workgroup owns one tile of the window (or, under a `blocks`
 *               cap, several in turn) and, plane after plane, writes the
 *               tile, reads it back and stores it to `out`.  On the LDS path
 *               each workgroup stages its tile of every plane in LDS (two
 *               planes at a time when a plane of one rank is a multiple of
 *               16 bytes), and each lane writes its chunks of the tile to
 *               the window, reads them back and stores them to `out`.
 *               After the call the window holds plane B-1 of every rank, in
 *               `out`'s layout.  Needs window_bytes >= layout.window_bytes.
 *   in       mode 0: [w][B][S_local][H][D]; mode 1: [w][B][S_local*w][H/w][D]
 *   out      the other layout; must not overlap `in` or the window.
 * Both tensors must be elem_bytes-aligned; 16-byte alignment (and run_bytes
 * a multiple of 16) selects the widest vectors.  The calling thread's current
 * device must be the plan's device.  One plan serves one stream at a time:
 * calls on one plan must not run concurrently from several threads.
 * Errors: INVALID_ARG, ALIGN, ALIAS, CAPACITY, DEVICE (no state change);
 * HIP (the launch failed; the plan becomes disabled, see
 * ua2a_plan_last_error); DISABLED (an earlier HIP error).
 */
int ua2a_exchange(ua2a_plan_t plan, int32_t mode, int32_t chunked,
                  const void* in, void* out, void* stream);

/* Bytes of the library's own window (64 MiB), the largest one-plane window
 * (layout.window_bytes) that ua2a_exchange_chunked_noalloc accepts. */
#define UA2A_NOALLOC_WINDOW_BYTES (64 * 1024 * 1024)

/*
 * ua2a_exchange_chunked_noalloc: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It is ua2a_exchange(plan, mode, 1, in, out, stream)
 * with the library's own window in place of the plan's, so the plan needs no
 * window (one it has is not used).  That window is a static device array of
 * UA2A_NOALLOC_WINDOW_BYTES that every device the library runs on holds for
 * the life of the process; the first call on a device looks up its address
 * there, and no call allocates or frees anything.
 *   All calls on one device share its window, which keeps the last call's
 *   contents (plane B-1 of every rank, as ua2a_exchange leaves its window).
 *   Calls that can overlap on one device -- on different streams, or from
 *   different threads without ordering -- race on the window: order them on
 *   one stream, or with events between streams.
 * Errors: those of ua2a_exchange with chunked = 1, with CAPACITY meaning
 * layout.window_bytes > UA2A_NOALLOC_WINDOW_BYTES; HIP also when the window's
 * address cannot be looked up (the plan becomes disabled).
 */
int ua2a_exchange_chunked_noalloc(ua2a_plan_t plan, int32_t mode, const void* in, void* out,
                                  void* stream);

/*
 * ua2a_exchange_ranks: the same exchange when each rank's tensors are
 * allocations of their own, as when every rank of the page's device
 * communicator owns its buffers and its registered window (FastVideo
 * "ulysses_a2a" API page: run_armed, and close for the per-rank windows),
 * optionally restricted to the runs that a range of ranks SENDS.
 *   in_ptrs   host array of w device pointers, indexed by sending rank:
 *             mode 0: in_ptrs[j] -> x_j [B][S_local][H][D];
 *             mode 1: in_ptrs[r] -> y_r [B][S_local*w][H/w][D].
 *             Only entries first .. first+count-1 are read (others may be NULL).
 *   out_ptrs  host array of w device pointers, indexed by receiving rank,
 *             all used: mode 0: out_ptrs[r] -> [B][S_local*w][H/w][D];
 *             mode 1: out_ptrs[j] -> [B][S_local][H][D].
 *   first, count  sending ranks [first, first + count), 0 <= first,
 *             1 <= count, first + count <= w.  Only runs from those senders
 *             are written: mode 0, the token block [j*S_local, (j+1)*S_local)
 *             of every out_ptrs[r] for each sender j; mode 1, the head block
 *             [r*H/w, (r+1)*H/w) of every token of every out_ptrs[j] for each
 *             sender r.  Every other output byte is left as it was.  (0, w)
 *             is the whole exchange; (j, 1) is the part that rank j pushes
 *             to its peers in a multi-device exchange.
 * The tables are read during the call only (copied into the launch); the
 * tensors are borrowed as in ua2a_exchange.  Each used pointer must be
 * elem_bytes-aligned; outputs may overlap neither each other nor a used
 * input.  One launch: the kernel family is chosen as for ua2a_exchange (and
 * ua2a_plan_set_path applies), except that mode 1 with part of the senders
 * always takes the direct family, whose writes need not cover whole rows.
 * The plan's window and chunked mode do not apply.  w <= 64 (the tables
 * travel in the kernel argument).
 * Errors: INVALID_ARG (NULL table or used entry, mode, first/count out of
 * range), SHAPE (w > 64), ALIGN, ALIAS, DEVICE (no state change); HIP
 * (the plan becomes disabled); DISABLED.
 */
int ua2a_exchange_ranks(ua2a_plan_t plan, int32_t mode, const void* const* in_ptrs,
                        void* const* out_ptrs, int32_t first, int32_t count, void* stream);

/*
 * ua2a_pack_ranks / ua2a_unpack_ranks: the per-rank exchange in two steps
 * through one receive window per receiving rank, as a multi-device exchange
 * runs it: every sender pushes its share into each receiver's registered
 * window, then each receiver moves its window into its own output, which never
 * aliases the window (FastVideo "ulysses_a2a" API page, run_armed: saved
 * activations never alias the reusable window).
 *   Window of receiver q (win_ptrs[q]): one rank's sequence-gathered layout,
 *   [B][S_local*w][H/w][D] (layout.tensor_bytes / w bytes); token block k of
 *   plane b, [k*S_local, (k+1)*S_local), holds what sender k sends q:
 *     mode 0: win_q[b][k*S_local+s][h][d] = x_k[b][s][q*(H/w)+h][d]
 *     mode 1: win_q[b][k*S_local+s][h][d] = y_k[b][q*S_local+s][h][d]
 *   so each sender's share is one contiguous block per plane and receiver
 *   (in mode 1 a plain copy of S_local runs, whatever the run length).
 * ua2a_pack_ranks: senders [first, first+count) write their blocks into
 *   every window (in_ptrs as for ua2a_exchange_ranks; all w windows must
 *   exist; other blocks are left as they were).  Mode 0 is exactly
 *   ua2a_exchange_ranks with the windows as outputs.  One launch.
 * ua2a_unpack_ranks: receivers [first, first+count) move their windows to
 *   their outputs (out_ptrs[q] as ua2a_exchange_ranks' outputs):
 *     mode 0: out_q = win_q (the same layout);
 *     mode 1: out_q[b][s][k*(H/w)+h][d] = win_q[b][k*S_local+s][h][d].
 *   One launch per receiver; entries outside the range are not read.
 * Packing every sender and then unpacking every receiver gives
 * ua2a_exchange_ranks(plan, mode, in, out, 0, w).  Tables are read during
 * the call only; tensors and windows are borrowed.  Each used pointer must be
 * elem_bytes-aligned.  Pack: windows may overlap neither each other nor a
 * used input, and w <= 64 (the tables travel in the kernel argument).
 * Unpack: a used output may overlap no other used output and no used window.
 * Errors: INVALID_ARG (NULL table or used entry, mode, first/count out of
 * range), SHAPE (pack with w > 64), ALIGN, ALIAS, DEVICE (no state change);
 * HIP (the plan becomes disabled); DISABLED.
 */
int ua2a_pack_ranks(ua2a_plan_t plan, int32_t mode, const void* const* in_ptrs,
                    void* const* win_ptrs, int32_t first, int32_t count, void* stream);
int ua2a_unpack_ranks(ua2a_plan_t plan, int32_t mode, const void* const* win_ptrs,
                      void* const* out_ptrs, int32_t first, int32_t count, void* stream);

/* ------------------------------------------------------ readiness credits */
/*
 * A consumer of the exchange (attention on a rank's gathered sequence, a
 * projection on a rank's restored tokens) can start on the receiving ranks
 * whose output is complete while the rest is still moving.  This is the
 * pipelining of the pypto-lib pull request "Perf: pipeline HCA AllToAll into
 * O-A" (its summary: the exchange marks parts ready, the consumer starts on
 * them, and readiness is handed back when consumed), with one counter per
 * RECEIVING rank (mode 0: rank r's [B, S_local*w, H/w, D]; mode 1: rank j's
 * [B, S_local, H, D]).
 *
 * Credits are a caller-owned device array of w uint32_t, zeroed by the
 * caller once before first use; the library only ever adds to them.  Each
 * publishing exchange adds 1 to every receiver's counter once that
 * receiver's output is complete and visible device-wide, so after the n-th
 * call on the same counters receiver k is ready when credits[k] reaches n
 * (modulo 2^32).  A credits array belongs to one plan and mode.
 */

/*
 * ua2a_exchange_publish: ua2a_exchange(plan, mode, 0, in, out, stream) in
 * `parts` launches (1 <= parts <= w), part k covering receiving ranks
 * [w*k/parts, w*(k+1)/parts); once part k has completed, 1 is added to
 * those receivers' credits (w counters, 4-byte aligned, not overlapping in or
 * out) -- by part k+1's launch, or after the last part by one more small
 * launch on the same stream.  parts = w publishes each receiver as soon as
 * its own part is done.  Always the direct kernel family, never chunked.
 * Errors: those of ua2a_exchange, plus INVALID_ARG (credits NULL, parts out
 * of range), ALIGN, ALIAS.
 */
int ua2a_exchange_publish(ua2a_plan_t plan, int32_t mode, const void* in, void* out,
                          uint32_t* credits, int32_t parts, void* stream);

/*
 * ua2a_wait_credits: enqueue on `stream` one small kernel that returns once
 * credits[first .. first+count) have all reached `target` (modulo 2^32), so
 * that work enqueued after it on that stream sees those receivers' bytes.
 * Run it on a stream other than the exchange's, enqueued after the exchange.
 * It polls each counter at most spin_limit times (with a short sleep between
 * polls); if one never gets there it stores 1 into *status (a caller-owned,
 * caller-zeroed device int32) and returns anyway, so it always ends: check
 * *status after synchronising before trusting what followed it.  No plan is
 * needed.  Errors: INVALID_ARG (NULL pointer, count < 1, first < 0, range
 * past 2^32, spin_limit 0), ALIGN, ALIAS (status inside the range), HIP.
 */
int ua2a_wait_credits(const uint32_t* credits, int64_t first, int64_t count, uint32_t target,
                      uint32_t spin_limit, int32_t* status, void* stream);

/*
 * ua2a_destroy: release the plan object.  It always consumes the plan, also
 * a disabled one, and never touches the window or device memory (the page's
 * disposer likewise consumes its handle even when cleanup reports an error).
 * NULL is accepted and ignored.  Returns UA2A_OK.
 */
int ua2a_destroy(ua2a_plan_t plan);

/* ua2a_status_string: static English text for a status code (never NULL). */
const char* ua2a_status_string(int32_t status);

/* ua2a_plan_last_error: why the plan is disabled, or "" if it is not (or
 * plan is NULL).  The string lives as long as the plan. */
const char* ua2a_plan_last_error(ua2a_plan_t plan);

/*
 * ua2a_plan_set_path: force a kernel family for later exchanges (for
 * measurement); UA2A_PATH_AUTO restores the default choice.  Forcing
 * UA2A_PATH_LDS on a shape whose rows do not fit the LDS tile makes
 * exchanges fall back to UA2A_PATH_DIRECT (ua2a_describe reports which).
 * Errors: INVALID_ARG.
 */
int ua2a_plan_set_path(ua2a_plan_t plan, int32_t path);

/*
 * ua2a_describe: report in *info what ua2a_exchange(plan, mode, chunked,
 * in, out, ...) would launch, after the same argument checks (same error
 * codes, minus DEVICE and HIP).  Host only; the pointers are only inspected
 * for alignment and overlap, never dereferenced.
 */
int ua2a_describe(ua2a_plan_t plan, int32_t mode, int32_t chunked,
                  const void* in, const void* out, ua2a_launch_info_t* info);

/*
 * ua2a_describe_ranks: as ua2a_describe, for ua2a_exchange_ranks with the
 * same arguments (same checks; host only, pointers never dereferenced).
 * info->tiles counts the launch's work tiles, grid its workgroups.
 */
int ua2a_describe_ranks(ua2a_plan_t plan, int32_t mode, const void* const* in_ptrs,
                        void* const* out_ptrs, int32_t first, int32_t count,
                        ua2a_launch_info_t* info);

#ifdef __cplusplus
}
#endif

#endif /* UA2A_H */

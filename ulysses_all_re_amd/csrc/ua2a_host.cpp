// Host side of the ua2a C ABI: shape validation, plans, per-call argument
// checks, kernel-path choice and launch geometry.  It calls the device only
// through the backend hooks of ua2a_internal.h.
//
// Semantics follow the FastVideo "ulysses_a2a" API page, method run_armed
// (shapes of mode 0 / mode 1, per-plane chunked loop, one window sized for a
// plane); the argument checks follow the launch-validation practice of the
// b12x PCIe two-shot collectives page (validate every input and caller-owned
// output before launching; reject overlapping storage by byte range, not by
// pointer equality).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ua2a_internal.h"

using namespace ua2a;

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxRowBytes = int64_t(1) << 31;      // H * D * elem_bytes
constexpr int64_t kMaxRuns = (int64_t(1) << 32) - 1;     // w * w * B * S_local
constexpr int64_t kMaxPlaneBytes = (int64_t(1) << 32) - 1;   // S_local * H * D * elem_bytes
constexpr int64_t kMaxTensorBytes = int64_t(1) << 38;    // 256 GiB

// Largest power of two <= 16 that divides x (16 for x == 0).
uint32_t pow2_align(uint64_t x)
{
    uint32_t a = 16;
    while (a > 1 && (x % a) != 0) a >>= 1;
    return a;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && pa < pb + static_cast<uintptr_t>(nb) &&
           pb < pa + static_cast<uintptr_t>(na);
}

// Multiply with an overflow check against `limit` (all operands >= 0).
bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t* out)
{
    if (a != 0 && b > limit / a) return false;
    *out = a * b;
    return *out <= limit;
}

// One tile per workgroup unless the caller's hint caps the grid, and never
// more work-items along x than a dispatch packet counts (32 bits); a capped
// grid's kernels loop over their tiles grid-stride.
uint32_t grid_for(uint32_t tiles, int32_t hint, uint32_t block)
{
    uint64_t g = tiles;
    if (hint > 0 && static_cast<uint64_t>(hint) < g) g = static_cast<uint64_t>(hint);
    const uint64_t cap = kMaxGridWorkItems / block;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return static_cast<uint32_t>(g);
}

// The one launch of an exchange: the permutation kernel, or for a chunked
// exchange the chunked kernel (direct path: on the 3-D grid, or on a flat
// grid under a `blocks` cap) or the chunked LDS kernel.
struct Prepared {
    int32_t path;            // UA2A_PATH_DIRECT or UA2A_PATH_LDS
    Launch perm;
};

// `recv` receiving ranks from the ones at the given bases (w for a whole
// exchange; fewer for a part of a publishing one, which may not use the
// grouped order since that order cycles through all w head blocks).
DirectGeom make_direct(const ua2a_plan_s* p, uint32_t vb, uint8_t* p_ptr, uint8_t* a_ptr,
                       int mode, int64_t p_rank, int64_t p_plane, int64_t a_rank,
                       int64_t a_plane, uint32_t nb, uint32_t recv, bool allow_group)
{
    DirectGeom g;
    memset(&g, 0, sizeof g);
    const int64_t run = p->layout.run_bytes;
    g.src = mode == 0 ? p_ptr : a_ptr;
    g.dst = mode == 0 ? a_ptr : p_ptr;
    g.a_rank = a_rank / vb;
    g.a_plane = a_plane / vb;
    g.p_rank = p_rank / vb;
    g.p_plane = p_plane / vb;
    g.vr = static_cast<uint32_t>(run / vb);
    g.p_row = static_cast<uint32_t>(p->w) * g.vr;
    g.s_local = static_cast<uint32_t>(p->S_local);
    g.w = static_cast<uint32_t>(p->w);
    g.nb = nb;
    // slabs are cut along the written side: (r, b, j) runs in mode 0, (j, b) rows in mode 1
    const uint64_t slab_vecs = static_cast<uint64_t>(g.s_local) * (mode == 0 ? g.vr : g.p_row);
    const uint64_t slabs = static_cast<uint64_t>(recv) * nb * (mode == 0 ? g.w : 1u);
    g.slab_vecs = static_cast<uint32_t>(slab_vecs);   // < 2^32 by the plane-size limit
    g.tile_vecs = kTileBytes / vb;      // 1 KiB of data whatever the vector width
    g.tiles_per_slab = static_cast<uint32_t>((slab_vecs + g.tile_vecs - 1) / g.tile_vecs);
    // mode 0 reads one head-block column of P rows per slab: when the row
    // stride is a multiple of 4 KiB, cycle head blocks fastest (measured:
    // slab after slab is up to 20 % slower there)
    // (the grouped order pads each slab to whole groups; it is skipped when
    // the padded tile count would not fit the kernel's 32-bit tile index)
    const int64_t row_bytes = run * p->w;
    if (allow_group && mode == 0 && p->w > 1 && row_bytes % kDirectGroupRowAlign == 0) {
        const uint64_t groups = (g.tiles_per_slab + kDirectGroup - 1) / kDirectGroup;
        if (groups * kDirectGroup * slabs <= UINT32_MAX) {
            g.group = kDirectGroup;
            g.groups = static_cast<uint32_t>(groups);
            g.num_tiles = static_cast<uint32_t>(groups * kDirectGroup * slabs);
        }
    }
    if (!g.group)   // < 2^32: one tile per slab needs slabs < 2^32 runs, more needs >= 1 KiB per slab
        g.num_tiles = static_cast<uint32_t>(slabs * g.tiles_per_slab);
    g.d_vr = make_div32(g.vr);
    g.d_prow = make_div32(g.p_row);
    g.d_tps = make_div32(g.tiles_per_slab);
    g.d_w = make_div32(g.w);
    g.d_nb = make_div32(nb);
    g.d_group = make_div32(g.group ? g.group : 1);
    g.d_groups = make_div32(g.groups ? g.groups : 1);
    return g;
}

// Whether the direct path's reads cover whole, aligned 128-byte lines, so
// that staging through LDS cannot save traffic (measured rule, 16-byte
// vectors).  Mode 0 reads one run per token: whole lines when the run is a
// multiple of 128 bytes, or when w = 1 (the runs are then adjacent).  Mode 1
// reads, per 1 KiB tile, one contiguous stretch per head block: a whole run
// when a token row exceeds the tile, else 1024 / w bytes of consecutive
// runs; it wants at least 256 line-aligned bytes per stretch.
bool direct_reads_whole_lines(int mode, int64_t w, int64_t run)
{
    if (w == 1) return run % 16 == 0;
    if (mode == 0) return run % 128 == 0;
    const int64_t row = w * run;
    if (row > kTileBytes) return run % 128 == 0 && run >= kDirectMinRun;
    return kTileBytes % row == 0 && kTileBytes / w >= kDirectMinRun;
}

// Whether a mode-1 launch of short 16-byte-multiple runs is small enough that
// the direct kernel beats the LDS kernel (measured rule): a launch moving
// under kDirectMode1Bytes per side runs few rounds of LDS workgroups, so the
// round at each end (fill, barrier, drain) costs more than the direct
// kernel's half-line reads.  Measured with runs of 32, 64 and 96 bytes and w
// of 4 and 8: direct ahead by 25 % at 17 MB per side, 10 % at 34 MB and 4 %
// at 67 MB; LDS ahead by 2-9 % from 100 MB up.
bool direct_for_small_mode1(int mode, uint32_t g, int64_t bytes_per_side)
{
    return mode == 1 && g == 16 && bytes_per_side < kDirectMode1Bytes;
}

// LDS padding per row for piece size G: with G = 16 every span is 16-aligned
// and a row may be padded so that its LDS stride equals run modulo 256 bytes
// (consecutive rows' runs on disjoint banks); otherwise rows stay packed.
uint32_t lds_pad(const ua2a_plan_s* p, uint32_t G)
{
    if (G != 16) return 0;
    const int64_t run = p->layout.run_bytes, row = run * p->w;
    return static_cast<uint32_t>((256 - (row - run) % 256) % 256);
}

// Rows of one (j, b) per LDS tile: about the mode's target size, rounded to
// the nearest multiple of 128 / gcd(run, 128) rows so that every tile's A
// spans (rows * run bytes) are whole 128-byte lines -- otherwise neighbouring
// tiles share a line at every span boundary, read twice in mode 1 and
// written in parts in mode 0 -- at least one row and within the largest tile
// a workgroup may hold; 0 (no LDS path) if one row plus padding and the
// alignment slack does not fit.
uint32_t lds_rows(const ua2a_plan_s* p, int mode, uint32_t G, bool chunked = false)
{
    const int64_t row = p->layout.run_bytes * p->w + lds_pad(p, G);
    if (row + 16 > kLdsTileMax) return 0;
    const int64_t target = chunked ? (mode == 0 ? kLdsChunkTileMode0 : kLdsChunkTileMode1)
                                   : (mode == 0 ? kLdsTileMode0 : kLdsTileMode1);
    int64_t rows = (target - 16) / row;
    int64_t g = p->layout.run_bytes, m = kLineBytes;
    while (m != 0) {
        const int64_t t = g % m;
        g = m;
        m = t;
    }
    const int64_t unit = kLineBytes / g;            // rows per whole number of lines
    const int64_t fit = (kLdsTileMax - 16) / row;   // most rows a tile may hold
    const int64_t aligned = (rows + unit / 2) / unit * unit;
    if (aligned >= unit && aligned <= fit) rows = aligned;
    else if (rows < unit && unit <= fit) rows = unit;
    if (rows < 1) rows = 1;
    if (rows > p->S_local) rows = p->S_local;
    return static_cast<uint32_t>(rows);
}

// Launch slots of an LDS launch: num_tiles rounded up to whole XCD turns of
// consecutive tiles (plain order if that would not fit 32 bits).
void set_lds_slots(LdsGeom* g)
{
    g->xlog = kLdsXcdLog;
    const uint64_t span = uint64_t(kXcds) << g->xlog;
    const uint64_t slots = (uint64_t(g->num_tiles) + span - 1) / span * span;
    if (slots > UINT32_MAX) {
        g->xlog = 0;
        g->num_slots = g->num_tiles;
    } else {
        g->num_slots = static_cast<uint32_t>(slots);
    }
}

LdsGeom make_lds(const ua2a_plan_s* p, int mode, uint32_t G, uint8_t* p_ptr, uint8_t* a_ptr,
                 int64_t p_rank, int64_t p_plane, int64_t a_rank, int64_t a_plane, uint32_t nb,
                 bool chunked = false)
{
    LdsGeom g;
    memset(&g, 0, sizeof g);
    g.p_ptr = p_ptr;
    g.a_ptr = a_ptr;
    g.a_rank = a_rank;
    g.a_plane = a_plane;
    g.p_rank = p_rank;
    g.p_plane = p_plane;
    g.run = static_cast<uint32_t>(p->layout.run_bytes);
    g.row = g.run * static_cast<uint32_t>(p->w);
    g.pad = lds_pad(p, G);
    g.lrow = g.row + g.pad;
    g.s_local = static_cast<uint32_t>(p->S_local);
    g.rows_per_tile = lds_rows(p, mode, G, chunked);
    g.tiles_per_plane = (g.s_local + g.rows_per_tile - 1) / g.rows_per_tile;
    g.w = static_cast<uint32_t>(p->w);
    g.nb = nb;
    g.num_tiles = g.w * nb * g.tiles_per_plane;
    set_lds_slots(&g);
    g.lds_bytes = (16 + g.rows_per_tile * g.lrow + 15) & ~15u;
    // every A span of a stacked tensor lies in [a_ptr, a_ptr + w * a_rank)
    g.a_window = (a_ptr != nullptr && static_cast<uint64_t>(g.w) * static_cast<uint64_t>(a_rank) + 64 <=
                  UINT32_MAX) ? 1u : 0u;
    g.a_whole16 = (a_ptr != nullptr && reinterpret_cast<uintptr_t>(a_ptr) % 16 == 0 && a_rank % 16 == 0) ? 1u : 0u;
    // chunk slots per A span: its chunks when spans are 16-aligned, else room
    // for an unaligned start (the longest a span can touch), rounded up to
    // whole 128-byte lines.  Consecutive lanes take consecutive slots, so a
    // line-aligned span's lines then fall on 8 consecutive lanes of one wave
    // and each line is written (mode 0) or read (mode 1) by one instruction.
    // With 14-byte runs the unrounded 113 slots per span split some lines
    // over two waves; their halves reached memory separately (PMC: 1 % more
    // write requests, 32-byte ones among them, in mode 0 and 0.7 % more read
    // requests in mode 1).
    const uint32_t rows_last = g.s_local - (g.tiles_per_plane - 1) * g.rows_per_tile;
    const auto slots = [&](uint32_t rows) {
        const uint32_t n = G == 16 ? rows * g.run / 16 : span_chunks(15, rows * g.run);
        return (n + 7) & ~7u;
    };
    g.stride_full = slots(g.rows_per_tile);
    g.stride_last = slots(rows_last);
    g.d_tpp = make_div32(g.tiles_per_plane);
    g.d_nb = make_div32(nb);
    g.d_run = make_div32(g.run);
    g.d_row = make_div32(g.row);
    g.d_stride_full = make_div32(g.stride_full);
    g.d_stride_last = make_div32(g.stride_last);
    return g;
}

CopyGeom make_copy(uint32_t vb, const uint8_t* src, uint8_t* dst, int64_t src_stride,
                   int64_t dst_stride, int64_t span_bytes, uint32_t count)
{
    CopyGeom g;
    memset(&g, 0, sizeof g);
    g.src = src;
    g.dst = dst;
    g.src_stride = src_stride / vb;
    g.dst_stride = dst_stride / vb;
    g.span = span_bytes / vb;
    g.tile_vecs = kTileBytes / vb;
    g.tiles_per_span = static_cast<uint32_t>((g.span + g.tile_vecs - 1) / g.tile_vecs);
    g.num_tiles = count * g.tiles_per_span;
    g.d_tps = make_div32(g.tiles_per_span);
    return g;
}

// The direct kernel's launch for receiving ranks [0, recv) of the given bases.
// Default order, no grid cap: one tile per workgroup on a 3-D grid whose
// coordinates are the tile's (x = tile in slab; mode 0: y = j, z = r*nb + b;
// mode 1: y = b, z = j), sparing each workgroup the scalar division of a flat
// tile index.
void direct_launch(const ua2a_plan_s* p, int mode, uint32_t vb, uint8_t* p_ptr, uint8_t* a_ptr,
                   int64_t p_rank, int64_t p_plane, int64_t a_rank, int64_t a_plane, uint32_t nb,
                   uint32_t recv, bool allow_group, Launch* L)
{
    L->kernel = Kernel::Direct;
    L->block = kDirectBlock;
    L->width = static_cast<int32_t>(vb);
    L->mode = mode;
    L->grid_y = L->grid_z = 1;
    L->grid3d = 0;
    L->direct = make_direct(p, vb, p_ptr, a_ptr, mode, p_rank, p_plane, a_rank, a_plane, nb, recv,
                            allow_group);
    L->grid = grid_for(L->direct.num_tiles, p->blocks, kDirectBlock);
    // A grid capped below the tiles it covers loops over them.  Measured on
    // the video-DiT exchange: one tile per iteration loses 25 % at a 2048
    // cap (358 against 271 us with four tiles loaded before any is stored),
    // while from 4096 workgroups on, four tiles per iteration is no faster
    // (4096: 292 against 279 us; 16,384: 305-342 against 292-299).  So four
    // only while the grid holds at most kCapInFlight tiles in flight with them.
    L->direct.cap_tiles = (L->grid < L->direct.num_tiles &&
                           static_cast<uint64_t>(L->grid) * kCapTiles <= kCapInFlight) ? kCapTiles : 1u;
    const uint32_t ny = mode == 0 ? static_cast<uint32_t>(p->w) : nb;
    const uint32_t nz = mode == 0 ? recv * nb : recv;
    if (p->blocks == 0 && L->direct.group == 0 && ny <= kMaxGridYZ && nz <= kMaxGridYZ) {
        L->grid3d = 1;
        L->grid = L->direct.tiles_per_slab;
        L->grid_y = ny;
        L->grid_z = nz;
    }
}

// Checks of one exchange call against a window of window_bytes at `window`
// (the plan's, or the library's own for the no-allocation entry point).
int check_call_window(const ua2a_plan_s* p, int32_t mode, int32_t chunked, const void* in,
                      const void* out, const void* window, int64_t window_bytes)
{
    if (p == nullptr) return UA2A_ERR_INVALID_ARG;
    if (p->disabled) return UA2A_ERR_DISABLED;
    if ((mode != 0 && mode != 1) || (chunked != 0 && chunked != 1)) return UA2A_ERR_INVALID_ARG;
    if (in == nullptr || out == nullptr) return UA2A_ERR_INVALID_ARG;
    const uintptr_t e = static_cast<uintptr_t>(p->elem_bytes);
    if (reinterpret_cast<uintptr_t>(in) % e || reinterpret_cast<uintptr_t>(out) % e)
        return UA2A_ERR_ALIGN;
    const int64_t n = p->layout.tensor_bytes;
    if (overlaps(in, n, out, n)) return UA2A_ERR_ALIAS;
    if (chunked) {
        if (window == nullptr || window_bytes < p->layout.window_bytes) return UA2A_ERR_CAPACITY;
        const int64_t wn = p->layout.window_bytes;
        if (overlaps(window, wn, in, n) || overlaps(window, wn, out, n)) return UA2A_ERR_ALIAS;
    }
    return UA2A_OK;
}

int check_call(const ua2a_plan_s* p, int32_t mode, int32_t chunked, const void* in,
               const void* out)
{
    if (p == nullptr) return UA2A_ERR_INVALID_ARG;
    return check_call_window(p, mode, chunked, in, out, p->window, p->window_bytes);
}

// The launches of one exchange; a chunked one goes through `window` (the
// plan's own unless given).
void prepare(const ua2a_plan_s* p, int32_t mode, int32_t chunked, const void* in, void* out,
             Prepared* pr, int32_t force_path = UA2A_PATH_AUTO, uint8_t* window = nullptr)
{
    if (window == nullptr) window = p->window;
    memset(pr, 0, sizeof *pr);
    const int64_t run = p->layout.run_bytes;
    const int64_t plane = p->S_local * p->H * p->D * p->elem_bytes;   // one plane of one rank
    const int64_t rank_bytes = plane * p->B;
    uint8_t* inb = const_cast<uint8_t*>(static_cast<const uint8_t*>(in));
    uint8_t* outb = static_cast<uint8_t*>(out);

    uint32_t g = pow2_align(static_cast<uint64_t>(run));
    g = umin32(g, pow2_align(reinterpret_cast<uintptr_t>(in)));
    g = umin32(g, pow2_align(reinterpret_cast<uintptr_t>(out)));
    if (chunked) g = umin32(g, pow2_align(reinterpret_cast<uintptr_t>(window)));

    const uint32_t rows = lds_rows(p, mode, g);
    const int32_t want = force_path != UA2A_PATH_AUTO ? force_path : p->path;
    int32_t path;
    if (want == UA2A_PATH_DIRECT)
        path = UA2A_PATH_DIRECT;
    else if (want == UA2A_PATH_LDS)
        path = rows > 0 ? UA2A_PATH_LDS : UA2A_PATH_DIRECT;
    else if (g == 16 && direct_reads_whole_lines(mode, p->w, run))
        path = UA2A_PATH_DIRECT;
    else if (!chunked && direct_for_small_mode1(mode, g, rank_bytes * p->w))
        path = UA2A_PATH_DIRECT;
    else
        path = rows > 0 ? UA2A_PATH_LDS : UA2A_PATH_DIRECT;

    // Which tensor is the P side ([j][b][s][H][D]) and which the A side
    // ([r][b][S_global][H/w][D]); strides in bytes.
    uint8_t *p_ptr, *a_ptr;
    int64_t p_rank, p_plane, a_rank, a_plane;
    uint32_t nb;
    if (!chunked) {
        p_ptr = mode == 0 ? inb : outb;
        a_ptr = mode == 0 ? outb : inb;
        p_rank = a_rank = rank_bytes;
        p_plane = a_plane = plane;
        nb = static_cast<uint32_t>(p->B);
    } else {
        // plane 0 of every rank <-> the window ([w][one plane] in the layout
        // of the exchange's output side)
        nb = 1;
        if (mode == 0) {
            p_ptr = inb;       p_rank = rank_bytes;
            a_ptr = window;    a_rank = plane;
        } else {
            a_ptr = inb;       a_rank = rank_bytes;
            p_ptr = window;    p_rank = plane;
        }
        p_plane = a_plane = 0;
    }

    pr->path = path;
    Launch& L = pr->perm;
    L.mode = mode;
    L.grid_y = L.grid_z = 1;
    if (path == UA2A_PATH_DIRECT) {
        direct_launch(p, mode, g, p_ptr, a_ptr, p_rank, p_plane, a_rank, a_plane, nb,
                      static_cast<uint32_t>(p->w), true, &L);
    } else {
        L.kernel = Kernel::Lds;
        L.block = kLdsBlock;
        L.width = static_cast<int32_t>(g);
        L.lds = make_lds(p, mode, g, p_ptr, a_ptr, p_rank, p_plane, a_rank, a_plane, nb);
        L.lds_bytes = L.lds.lds_bytes;
        L.grid = grid_for(L.lds.num_slots, p->blocks, kLdsBlock);
    }
    if (chunked) {
        // the LDS path: one launch of the chunked LDS kernel
        if (L.kernel == Kernel::Lds) {
            L.kernel = Kernel::LdsChunked;
            L.lds = make_lds(p, mode, g, p_ptr, a_ptr, p_rank, p_plane, a_rank, a_plane, nb, true);
            L.lds_bytes = L.lds.lds_bytes;
            L.grid = grid_for(L.lds.num_slots, p->blocks, kLdsBlock);
            L.lds_chunk.out = outb;
            L.lds_chunk.rank_step = rank_bytes - plane;
            L.lds_chunk.plane = plane;
            L.lds_chunk.planes = static_cast<uint32_t>(p->B);
            // planes staged per fill: up to kLdsChunkStage, as many images as
            // fit kLdsChunkLds, at least one (an image alone is within the tile
            // limit); several only when a plane is a multiple of 16 bytes, so
            // that every plane's image is laid out alike
            L.lds_chunk.image = L.lds.lds_bytes;            // a multiple of 16
            uint32_t stage = plane % 16 == 0 ? kLdsChunkLds / L.lds.lds_bytes : 1u;
            if (stage > kLdsChunkStage) stage = kLdsChunkStage;
            if (stage > L.lds_chunk.planes) stage = L.lds_chunk.planes;
            L.lds_chunk.stage = stage < 1 ? 1 : stage;
            L.lds_bytes = L.lds_chunk.stage * L.lds_chunk.image;
            return;
        }
        // mode 0 with the grouped tile order (4 KiB-multiple rows): the chunked
        // kernel takes it on a 3-D grid too, x running over (tile group, head
        // block r, tile within the group) and y over the sending rank j
        const DirectGeom& dg = L.direct;
        if (!L.grid3d && dg.group != 0 && p->blocks == 0 &&
            p->w <= static_cast<int32_t>(kMaxGridYZ)) {
            L.grid3d = 1;
            L.grid = dg.groups * dg.group * dg.w;      // <= num_tiles (nb = 1), < 2^32
            L.grid_y = dg.w;
            L.grid_z = 1;
        }
        // the direct path: one launch of the chunked kernel, each tile of the
        // one-plane window moved through all B planes (the window block is
        // the head block r in mode 0, the receiving rank j in mode 1); on the
        // 3-D grid, or on a flat grid whose workgroups loop over the tiles
        L.kernel = Kernel::Chunked;
        L.chunk.out = outb;
        L.chunk.step = (rank_bytes - plane) / L.width;
        L.chunk.plane = plane / L.width;
        L.chunk.planes = static_cast<uint32_t>(p->B);
    }
}

// Per-rank tables: only the entries a call uses are looked at -- the inputs
// of the sending ranks and every output (each receives runs from every
// sender).  Outputs may overlap neither each other nor a used input.
int check_ranks_call(const ua2a_plan_s* p, int32_t mode, const void* const* in,
                     void* const* out, int32_t first, int32_t count)
{
    if (p == nullptr) return UA2A_ERR_INVALID_ARG;
    if (p->disabled) return UA2A_ERR_DISABLED;
    if (mode != 0 && mode != 1) return UA2A_ERR_INVALID_ARG;
    if (in == nullptr || out == nullptr) return UA2A_ERR_INVALID_ARG;
    if (p->w > static_cast<int32_t>(kMaxRankTable)) return UA2A_ERR_SHAPE;
    if (first < 0 || count < 1 || first > p->w - count) return UA2A_ERR_INVALID_ARG;
    const int32_t last = first + count;
    for (int32_t k = first; k < last; ++k)
        if (in[k] == nullptr) return UA2A_ERR_INVALID_ARG;
    for (int32_t k = 0; k < p->w; ++k)
        if (out[k] == nullptr) return UA2A_ERR_INVALID_ARG;
    const uintptr_t e = static_cast<uintptr_t>(p->elem_bytes);
    for (int32_t k = first; k < last; ++k)
        if (reinterpret_cast<uintptr_t>(in[k]) % e) return UA2A_ERR_ALIGN;
    for (int32_t k = 0; k < p->w; ++k)
        if (reinterpret_cast<uintptr_t>(out[k]) % e) return UA2A_ERR_ALIGN;
    const int64_t n = p->layout.tensor_bytes / p->w;     // one rank's tensor
    for (int32_t k = 0; k < p->w; ++k) {
        for (int32_t k2 = k + 1; k2 < p->w; ++k2)
            if (overlaps(out[k], n, out[k2], n)) return UA2A_ERR_ALIAS;
        for (int32_t k2 = first; k2 < last; ++k2)
            if (overlaps(out[k], n, in[k2], n)) return UA2A_ERR_ALIAS;
    }
    return UA2A_OK;
}

// The one launch of a per-rank exchange.  Default grid: one tile per
// workgroup over (tile, y, z), y and z capped at the hardware extent (the
// kernel loops past a cap); a `blocks` hint caps the total.
void prepare_ranks(const ua2a_plan_s* p, int32_t mode, const void* const* in, void* const* out,
                   int32_t first, int32_t count, Launch* L)
{
    memset(L, 0, sizeof *L);
    const int64_t run = p->layout.run_bytes;
    const int64_t plane = p->S_local * p->H * p->D * p->elem_bytes;
    const int32_t last = first + count;
    uint32_t vb = pow2_align(static_cast<uint64_t>(run));
    for (int32_t k = first; k < last; ++k)
        vb = umin32(vb, pow2_align(reinterpret_cast<uintptr_t>(in[k])));
    for (int32_t k = 0; k < p->w; ++k)
        vb = umin32(vb, pow2_align(reinterpret_cast<uintptr_t>(out[k])));

    // The LDS kernel moves whole P rows, so it serves mode 0 (every sender's
    // rows are its own) and mode 1 only when every rank sends (each written
    // row is then complete); the choice between the two follows ua2a_exchange.
    const uint32_t rows = (mode == 0 || count == p->w) ? lds_rows(p, mode, vb) : 0;
    bool use_lds;
    if (p->path == UA2A_PATH_DIRECT || rows == 0)
        use_lds = false;
    else if (p->path == UA2A_PATH_LDS)
        use_lds = true;
    else
        use_lds = !(vb == 16 && direct_reads_whole_lines(mode, p->w, run));
    if (use_lds) {
        L->kernel = Kernel::LdsRanks;
        L->block = kLdsBlock;
        L->width = static_cast<int32_t>(vb);
        L->mode = mode;
        L->grid_y = L->grid_z = 1;
        // bases come from the tables: rank strides 0, plane strides within a rank
        L->lds = make_lds(p, mode, vb, nullptr, nullptr, 0, plane, 0, plane,
                          static_cast<uint32_t>(p->B));
        L->lds.j0 = mode == 0 ? static_cast<uint32_t>(first) : 0u;
        const uint32_t nj = mode == 0 ? static_cast<uint32_t>(count) : static_cast<uint32_t>(p->w);
        L->lds.num_tiles = nj * L->lds.nb * L->lds.tiles_per_plane;
        set_lds_slots(&L->lds);
        L->lds_bytes = L->lds.lds_bytes;
        for (int32_t k = 0; k < p->w; ++k) {
            uint8_t* inb = const_cast<uint8_t*>(static_cast<const uint8_t*>(
                (k >= first && k < last) ? in[k] : nullptr));
            uint8_t* outb = static_cast<uint8_t*>(out[k]);
            L->lds_tab.p[k] = mode == 0 ? inb : outb;
            L->lds_tab.a[k] = mode == 0 ? outb : inb;
        }
        L->grid = grid_for(L->lds.num_slots, p->blocks, kLdsBlock);
        return;
    }

    RanksGeom& g = L->ranks;
    for (int32_t k = 0; k < p->w; ++k) {
        g.dst[k] = static_cast<uint8_t*>(out[k]);
        g.src[k] = (k >= first && k < last) ? static_cast<const uint8_t*>(in[k]) : nullptr;
    }
    g.a_plane = plane / vb;     // S_global * run bytes == S_local * H * D * e
    g.p_plane = plane / vb;
    g.vr = static_cast<uint32_t>(run / vb);
    g.p_row = static_cast<uint32_t>(p->w) * g.vr;
    g.seg = static_cast<uint32_t>(count) * g.vr;
    g.s_local = static_cast<uint32_t>(p->S_local);
    g.w = static_cast<uint32_t>(p->w);
    g.nb = static_cast<uint32_t>(p->B);
    g.first = static_cast<uint32_t>(first);
    g.count = static_cast<uint32_t>(count);
    g.slab_vecs = g.s_local * (mode == 0 ? g.vr : g.seg);   // < 2^32 by the plane-size limit
    g.tile_vecs = kTileBytes / vb;
    g.tiles_per_slab = (g.slab_vecs + g.tile_vecs - 1) / g.tile_vecs;
    // a tile of tile_vecs consecutive vectors lies in at most two runs when
    // runs are at least that long; with one sender all its runs share a tensor
    g.two_runs = (g.count == 1 || g.vr >= g.tile_vecs) ? 1u : 0u;
    g.ny = mode == 0 ? g.count : g.nb;
    g.nz = mode == 0 ? g.w * g.nb : g.w;     // w * B < 2^32 by the run-count limit
    g.d_vr = make_div32(g.vr);
    g.d_seg = make_div32(g.seg);
    g.d_nb = make_div32(g.nb);
    g.d_count = make_div32(g.count);

    L->kernel = Kernel::Ranks;
    L->block = kDirectBlock;
    L->width = static_cast<int32_t>(vb);
    L->mode = mode;
    L->grid = grid_for(g.tiles_per_slab, p->blocks, kDirectBlock);
    uint64_t room = p->blocks > 0 ? static_cast<uint64_t>(p->blocks) / L->grid : kMaxGridYZ;
    if (room < 1) room = 1;
    L->grid_y = static_cast<uint32_t>(g.ny < room ? g.ny : room);
    if (L->grid_y > kMaxGridYZ) L->grid_y = kMaxGridYZ;
    room = p->blocks > 0 ? room / L->grid_y : kMaxGridYZ;
    if (room < 1) room = 1;
    L->grid_z = static_cast<uint32_t>(g.nz < room ? g.nz : room);
    if (L->grid_z > kMaxGridYZ) L->grid_z = kMaxGridYZ;
}

// Pack, mode 1: for every sender k in [first, first + count), receiver q and
// plane b, the contiguous block of q's tokens (S_local runs) goes to block k
// of plane b of q's window.  Every offset is a multiple of the block, so the
// vector width follows the block and the bases, not the run: 14-byte runs
// still move as 16-byte vectors when S_local * run allows.  (Mode 0's pack
// is the per-rank exchange into the windows, prepare_ranks.)
void prepare_pack1(const ua2a_plan_s* p, const void* const* in, void* const* win, int32_t first,
                   int32_t count, Launch* L)
{
    memset(L, 0, sizeof *L);
    const int64_t run = p->layout.run_bytes;
    const int64_t block = p->S_local * run;                 // one token block of one plane
    const int64_t plane = block * p->w;                     // one plane of a sequence-gathered tensor
    uint32_t vb = pow2_align(static_cast<uint64_t>(block));
    for (int32_t k = first; k < first + count; ++k)
        vb = umin32(vb, pow2_align(reinterpret_cast<uintptr_t>(in[k])));
    for (int32_t q = 0; q < p->w; ++q) vb = umin32(vb, pow2_align(reinterpret_cast<uintptr_t>(win[q])));
    PackGeom& g = L->pack;
    for (int32_t k = 0; k < p->w; ++k) {
        g.src[k] = (k >= first && k < first + count) ? static_cast<const uint8_t*>(in[k]) : nullptr;
        g.dst[k] = static_cast<uint8_t*>(win[k]);
    }
    g.src_b = g.dst_b = plane / vb;
    g.src_q = g.dst_k = block / vb;
    g.block_vecs = static_cast<uint32_t>(block / vb);      // < 2^32 by the plane-size limit
    g.tile_vecs = kTileBytes / vb;
    g.tiles_per_block = (g.block_vecs + g.tile_vecs - 1) / g.tile_vecs;
    g.first = static_cast<uint32_t>(first);
    g.ny = static_cast<uint32_t>(count);
    g.nz = static_cast<uint32_t>(p->w) * static_cast<uint32_t>(p->B);   // < 2^32 by the run-count limit
    g.d_nb = make_div32(static_cast<uint32_t>(p->B));
    L->kernel = Kernel::Pack;
    L->block = kDirectBlock;
    L->width = static_cast<int32_t>(vb);
    L->mode = 1;
    L->grid = grid_for(g.tiles_per_block, p->blocks, kDirectBlock);
    uint64_t room = p->blocks > 0 ? static_cast<uint64_t>(p->blocks) / L->grid : kMaxGridYZ;
    if (room < 1) room = 1;
    L->grid_y = static_cast<uint32_t>(g.ny < room ? g.ny : room);
    room = p->blocks > 0 ? room / L->grid_y : kMaxGridYZ;
    if (room < 1) room = 1;
    L->grid_z = static_cast<uint32_t>(g.nz < room ? g.nz : room);
    if (L->grid_z > kMaxGridYZ) L->grid_z = kMaxGridYZ;
}

// Unpack of one receiver: mode 0's window already has the output's layout
// (one copy); mode 1 is the mode-1 exchange restricted to this receiver's
// rows, reading sender k's runs from token block k of the window (A-side
// rank stride S_local * run, plane stride S_local * w * run), by the same
// path choice as ua2a_exchange.
void prepare_unpack(const ua2a_plan_s* p, int32_t mode, const void* win, void* out, Launch* L)
{
    memset(L, 0, sizeof *L);
    uint8_t* winb = const_cast<uint8_t*>(static_cast<const uint8_t*>(win));
    uint8_t* outb = static_cast<uint8_t*>(out);
    const int64_t run = p->layout.run_bytes;
    const int64_t rank_bytes = p->layout.tensor_bytes / p->w;
    L->grid_y = L->grid_z = 1;
    L->mode = mode;
    if (mode == 0) {
        uint32_t vb = pow2_align(static_cast<uint64_t>(rank_bytes));
        vb = umin32(vb, pow2_align(reinterpret_cast<uintptr_t>(win)));
        vb = umin32(vb, pow2_align(reinterpret_cast<uintptr_t>(out)));
        L->kernel = Kernel::Copy;
        L->block = kCopyBlock;
        L->width = static_cast<int32_t>(vb);
        L->copy = make_copy(vb, winb, outb, 0, 0, rank_bytes, 1);
        L->grid = grid_for(L->copy.num_tiles, 0, kCopyBlock);
        return;
    }
    const int64_t block = p->S_local * run;
    const int64_t a_plane = block * p->w;
    const int64_t p_plane = p->S_local * p->H * p->D * p->elem_bytes;
    uint32_t g = pow2_align(static_cast<uint64_t>(run));
    g = umin32(g, pow2_align(reinterpret_cast<uintptr_t>(win)));
    g = umin32(g, pow2_align(reinterpret_cast<uintptr_t>(out)));
    const uint32_t rows = lds_rows(p, 1, g);
    bool lds;
    if (p->path == UA2A_PATH_DIRECT || rows == 0)
        lds = false;
    else if (p->path == UA2A_PATH_LDS)
        lds = true;
    else
        lds = !(g == 16 && direct_reads_whole_lines(1, p->w, run)) && !direct_for_small_mode1(1, g, rank_bytes);
    if (!lds) {
        direct_launch(p, 1, g, outb, winb, 0, p_plane, block, a_plane, static_cast<uint32_t>(p->B), 1, false, L);
        return;
    }
    L->kernel = Kernel::Lds;
    L->block = kLdsBlock;
    L->width = static_cast<int32_t>(g);
    L->lds = make_lds(p, 1, g, outb, winb, 0, p_plane, block, a_plane, static_cast<uint32_t>(p->B));
    L->lds.num_tiles = L->lds.nb * L->lds.tiles_per_plane;     // the receiver's rows only
    set_lds_slots(&L->lds);
    L->lds_bytes = L->lds.lds_bytes;
    L->grid = grid_for(L->lds.num_slots, p->blocks, kLdsBlock);
}

// Unpack arguments: receivers [first, first + count) need their windows and
// outputs; an output may overlap no other used output and no used window.
int check_unpack_call(const ua2a_plan_s* p, int32_t mode, const void* const* win, void* const* out,
                      int32_t first, int32_t count)
{
    if (p == nullptr) return UA2A_ERR_INVALID_ARG;
    if (p->disabled) return UA2A_ERR_DISABLED;
    if (mode != 0 && mode != 1) return UA2A_ERR_INVALID_ARG;
    if (win == nullptr || out == nullptr) return UA2A_ERR_INVALID_ARG;
    if (first < 0 || count < 1 || first > p->w - count) return UA2A_ERR_INVALID_ARG;
    const int32_t last = first + count;
    const uintptr_t e = static_cast<uintptr_t>(p->elem_bytes);
    for (int32_t q = first; q < last; ++q) {
        if (win[q] == nullptr || out[q] == nullptr) return UA2A_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(win[q]) % e || reinterpret_cast<uintptr_t>(out[q]) % e)
            return UA2A_ERR_ALIGN;
    }
    const int64_t n = p->layout.tensor_bytes / p->w;       // one rank's tensor, and one window
    for (int32_t q = first; q < last; ++q)
        for (int32_t q2 = first; q2 < last; ++q2)
            if ((q2 > q && overlaps(out[q], n, out[q2], n)) || overlaps(out[q], n, win[q2], n))
                return UA2A_ERR_ALIAS;
    return UA2A_OK;
}

void disable(ua2a_plan_s* p, const char* what, int err)
{
    p->disabled = 1;
    snprintf(p->reason, sizeof p->reason, "%s failed: %s (%d)", what, backend_error_name(err), err);
}

// Enqueue one validated exchange (the current device is the plan's).
int launch_exchange(ua2a_plan_s* plan, int32_t mode, int32_t chunked, const void* in, void* out,
                    uint8_t* window, void* stream)
{
    Prepared pr;
    prepare(plan, mode, chunked, in, out, &pr, UA2A_PATH_AUTO, window);
    const int err = backend_launch(pr.perm, stream);
    if (err != 0) {
        disable(plan, chunked ? "launching the chunked exchange kernel" : "launching the exchange kernel", err);
        return UA2A_ERR_HIP;
    }
    return UA2A_OK;
}

// The calling thread's current device is the plan's (UA2A_OK), is another
// (UA2A_ERR_DEVICE), or cannot be queried (UA2A_ERR_HIP, plan disabled).
int check_device(ua2a_plan_s* plan)
{
    int32_t dev = -1;
    const int err = backend_current_device(&dev);
    if (err != 0) {
        disable(plan, "querying the current device", err);
        return UA2A_ERR_HIP;
    }
    return dev == plan->device ? UA2A_OK : UA2A_ERR_DEVICE;
}

}  // namespace

extern "C" {

int ua2a_layout(int32_t w, int64_t B, int64_t S_local, int64_t H, int64_t D,
                int32_t elem_bytes, ua2a_layout_t* layout)
{
    if (layout == nullptr) return UA2A_ERR_INVALID_ARG;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
        return UA2A_ERR_INVALID_ARG;
    if (w < 1 || w > 65536 || B < 1 || S_local < 1 || H < 1 || D < 1) return UA2A_ERR_SHAPE;
    if (B > kMaxDim || S_local > kMaxDim || H > kMaxDim || D > kMaxDim) return UA2A_ERR_SHAPE;
    if (H % w != 0) return UA2A_ERR_SHAPE;
    int64_t row, runs, elems, bytes, t;
    if (!mul_ok(H, D, kMaxRowBytes, &t) || !mul_ok(t, elem_bytes, kMaxRowBytes, &row))
        return UA2A_ERR_SHAPE;
    if (!mul_ok(int64_t(w) * w, B, kMaxRuns, &t) || !mul_ok(t, S_local, kMaxRuns, &runs))
        return UA2A_ERR_SHAPE;
    if (!mul_ok(runs / w, row / elem_bytes, kMaxTensorBytes, &elems) ||
        !mul_ok(elems, elem_bytes, kMaxTensorBytes, &bytes))
        return UA2A_ERR_SHAPE;
    int64_t plane;
    if (!mul_ok(S_local, row, kMaxPlaneBytes, &plane)) return UA2A_ERR_SHAPE;
    layout->H_local = H / w;
    layout->S_global = S_local * w;
    layout->run_bytes = (H / w) * D * elem_bytes;
    layout->tensor_elems = elems;
    layout->tensor_bytes = bytes;
    layout->window_bytes = int64_t(w) * S_local * row;
    layout->moved_bytes = 2 * bytes;
    return UA2A_OK;
}

int ua2a_plan(ua2a_plan_t* plan_out, int32_t w, int64_t B, int64_t S_local, int64_t H,
              int64_t D, int32_t elem_bytes, int32_t blocks, void* window,
              int64_t window_bytes, int32_t device)
{
    if (plan_out == nullptr) return UA2A_ERR_INVALID_ARG;
    *plan_out = nullptr;
    ua2a_layout_t lay;
    const int rc = ua2a_layout(w, B, S_local, H, D, elem_bytes, &lay);
    if (rc != UA2A_OK) return rc;
    if (device < 0 || blocks < 0 || window_bytes < 0) return UA2A_ERR_INVALID_ARG;
    if (window == nullptr && window_bytes > 0) return UA2A_ERR_INVALID_ARG;
    if (window != nullptr && reinterpret_cast<uintptr_t>(window) % elem_bytes)
        return UA2A_ERR_ALIGN;
    ua2a_plan_s* p = static_cast<ua2a_plan_s*>(calloc(1, sizeof(ua2a_plan_s)));
    if (p == nullptr) return UA2A_ERR_NOMEM;
    p->w = w;
    p->B = B;
    p->S_local = S_local;
    p->H = H;
    p->D = D;
    p->elem_bytes = elem_bytes;
    p->layout = lay;
    p->blocks = blocks;
    p->window = static_cast<uint8_t*>(window);
    p->window_bytes = window == nullptr ? 0 : window_bytes;
    p->device = device;
    p->path = UA2A_PATH_AUTO;
    *plan_out = p;
    return UA2A_OK;
}

int ua2a_exchange(ua2a_plan_t plan, int32_t mode, int32_t chunked, const void* in, void* out,
                  void* stream)
{
    int rc = check_call(plan, mode, chunked, in, out);
    if (rc == UA2A_OK) rc = check_device(plan);
    if (rc != UA2A_OK) return rc;
    return launch_exchange(plan, mode, chunked, in, out, plan->window, stream);
}

int ua2a_exchange_chunked_noalloc(ua2a_plan_t plan, int32_t mode, const void* in, void* out,
                                  void* stream)
{
    // everything but the window first, as for ua2a_exchange: the window's
    // address is known only once the device is
    int rc = check_call_window(plan, mode, 0, in, out, nullptr, 0);
    if (rc != UA2A_OK) return rc;
    if (plan->layout.window_bytes > UA2A_NOALLOC_WINDOW_BYTES) return UA2A_ERR_CAPACITY;
    rc = check_device(plan);
    if (rc != UA2A_OK) return rc;
    uint8_t* window = nullptr;
    const int err = backend_scratch_window(plan->device, &window);
    if (err != 0) {
        disable(plan, "looking up the library's window", err);
        return UA2A_ERR_HIP;
    }
    rc = check_call_window(plan, mode, 1, in, out, window, UA2A_NOALLOC_WINDOW_BYTES);
    if (rc != UA2A_OK) return rc;
    return launch_exchange(plan, mode, 1, in, out, window, stream);
}

int ua2a_exchange_ranks(ua2a_plan_t plan, int32_t mode, const void* const* in_ptrs,
                        void* const* out_ptrs, int32_t first, int32_t count, void* stream)
{
    int rc = check_ranks_call(plan, mode, in_ptrs, out_ptrs, first, count);
    if (rc == UA2A_OK) rc = check_device(plan);
    if (rc != UA2A_OK) return rc;
    Launch L;
    prepare_ranks(plan, mode, in_ptrs, out_ptrs, first, count, &L);
    const int err = backend_launch(L, stream);
    if (err != 0) {
        disable(plan, "launching the per-rank exchange kernel", err);
        return UA2A_ERR_HIP;
    }
    return UA2A_OK;
}

int ua2a_pack_ranks(ua2a_plan_t plan, int32_t mode, const void* const* in_ptrs, void* const* win_ptrs,
                    int32_t first, int32_t count, void* stream)
{
    // the windows are checked as the per-rank exchange checks its outputs
    int rc = check_ranks_call(plan, mode, in_ptrs, win_ptrs, first, count);
    if (rc == UA2A_OK) rc = check_device(plan);
    if (rc != UA2A_OK) return rc;
    Launch L;
    if (mode == 0)
        prepare_ranks(plan, 0, in_ptrs, win_ptrs, first, count, &L);
    else
        prepare_pack1(plan, in_ptrs, win_ptrs, first, count, &L);
    const int err = backend_launch(L, stream);
    if (err != 0) {
        disable(plan, "launching the pack kernel", err);
        return UA2A_ERR_HIP;
    }
    return UA2A_OK;
}

int ua2a_unpack_ranks(ua2a_plan_t plan, int32_t mode, const void* const* win_ptrs, void* const* out_ptrs,
                      int32_t first, int32_t count, void* stream)
{
    int rc = check_unpack_call(plan, mode, win_ptrs, out_ptrs, first, count);
    if (rc == UA2A_OK) rc = check_device(plan);
    if (rc != UA2A_OK) return rc;
    for (int32_t q = first; q < first + count; ++q) {
        Launch L;
        prepare_unpack(plan, mode, win_ptrs[q], out_ptrs[q], &L);
        const int err = backend_launch(L, stream);
        if (err != 0) {
            disable(plan, "launching the unpack kernel", err);
            return UA2A_ERR_HIP;
        }
    }
    return UA2A_OK;
}

int ua2a_exchange_publish(ua2a_plan_t plan, int32_t mode, const void* in, void* out,
                          uint32_t* credits, int32_t parts, void* stream)
{
    int rc = check_call(plan, mode, 0, in, out);
    if (rc != UA2A_OK) return rc;
    if (credits == nullptr || parts < 1 || parts > plan->w) return UA2A_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(credits) % sizeof(uint32_t)) return UA2A_ERR_ALIGN;
    const int64_t cbytes = int64_t(plan->w) * static_cast<int64_t>(sizeof(uint32_t));
    const int64_t n = plan->layout.tensor_bytes;
    if (overlaps(credits, cbytes, in, n) || overlaps(credits, cbytes, out, n)) return UA2A_ERR_ALIAS;
    rc = check_device(plan);
    if (rc != UA2A_OK) return rc;
    int err;
    // Part k covers receiving ranks [w*k/parts, w*(k+1)/parts): the direct
    // kernel on bases moved to its first receiver (mode 0: A rank r0 and head
    // block r0 of the P rows; mode 1: P rank j0 and token block j0 of the A
    // side).  Part k's credits are added by part k+1's first workgroup, which
    // starts only after part k has completed; the last part's by a signal
    // launch.
    Prepared pr;
    prepare(plan, mode, 0, in, out, &pr, UA2A_PATH_DIRECT);
    const DirectGeom& g0 = pr.perm.direct;
    const int64_t vb = pr.perm.width;
    const int64_t plane = plan->S_local * plan->H * plan->D * plan->elem_bytes;
    const int64_t rank_bytes = plane * plan->B;
    uint8_t* p_base = const_cast<uint8_t*>(mode == 0 ? g0.src : g0.dst);
    uint8_t* a_base = const_cast<uint8_t*>(mode == 0 ? g0.dst : g0.src);
    for (int32_t k = 0; k < parts; ++k) {
        const int64_t r0 = int64_t(plan->w) * k / parts;
        const int64_t r1 = int64_t(plan->w) * (k + 1) / parts;
        uint8_t* pp = p_base + (mode == 0 ? r0 * g0.vr * vb : r0 * rank_bytes);
        uint8_t* ap = a_base + (mode == 0 ? r0 * rank_bytes : r0 * int64_t(g0.s_local) * g0.vr * vb);
        Launch L;
        memset(&L, 0, sizeof L);
        direct_launch(plan, mode, static_cast<uint32_t>(vb), pp, ap, rank_bytes, plane, rank_bytes,
                      plane, static_cast<uint32_t>(plan->B), static_cast<uint32_t>(r1 - r0), false, &L);
        if (k > 0) {
            L.direct.sig_credits = credits;
            L.direct.sig_first = static_cast<uint32_t>(int64_t(plan->w) * (k - 1) / parts);
            L.direct.sig_count = static_cast<uint32_t>(r0) - L.direct.sig_first;
        }
        err = backend_launch(L, stream);
        if (err != 0) {
            disable(plan, "launching a part of a publishing exchange", err);
            return UA2A_ERR_HIP;
        }
    }
    Launch S;
    memset(&S, 0, sizeof S);
    S.kernel = Kernel::Signal;
    S.block = kWaitBlock;
    S.grid = S.grid_y = S.grid_z = 1;
    S.signal.credits = credits;
    S.signal.first = static_cast<uint32_t>(int64_t(plan->w) * (parts - 1) / parts);
    S.signal.count = static_cast<uint32_t>(plan->w) - S.signal.first;
    err = backend_launch(S, stream);
    if (err != 0) {
        disable(plan, "launching a part of a publishing exchange", err);
        return UA2A_ERR_HIP;
    }
    return UA2A_OK;
}

int ua2a_wait_credits(const uint32_t* credits, int64_t first, int64_t count, uint32_t target,
                      uint32_t spin_limit, int32_t* status, void* stream)
{
    if (credits == nullptr || status == nullptr) return UA2A_ERR_INVALID_ARG;
    if (first < 0 || count < 1 || count > int64_t(UINT32_MAX) ||
        first > int64_t(UINT32_MAX) - count || spin_limit < 1)
        return UA2A_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(credits) % sizeof(uint32_t) ||
        reinterpret_cast<uintptr_t>(status) % sizeof(int32_t))
        return UA2A_ERR_ALIGN;
    if (overlaps(credits + first, count * static_cast<int64_t>(sizeof(uint32_t)), status,
                 sizeof(int32_t)))
        return UA2A_ERR_ALIAS;
    Launch L;
    memset(&L, 0, sizeof L);
    L.kernel = Kernel::Wait;
    L.block = kWaitBlock;
    L.grid = L.grid_y = L.grid_z = 1;
    L.wait.credits = credits;
    L.wait.first = static_cast<uint32_t>(first);
    L.wait.count = static_cast<uint32_t>(count);
    L.wait.target = target;
    L.wait.spin_limit = spin_limit;
    L.wait.status = status;
    return backend_launch(L, stream) == 0 ? UA2A_OK : UA2A_ERR_HIP;
}

int ua2a_destroy(ua2a_plan_t plan)
{
    free(plan);
    return UA2A_OK;
}

const char* ua2a_status_string(int32_t status)
{
    switch (status) {
    case UA2A_OK: return "ok";
    case UA2A_ERR_INVALID_ARG: return "invalid argument";
    case UA2A_ERR_SHAPE: return "unsupported shape (dimension < 1, H not divisible by w, or beyond the size limits)";
    case UA2A_ERR_ALIGN: return "pointer not aligned to the element size";
    case UA2A_ERR_ALIAS: return "input, output and window byte ranges overlap";
    case UA2A_ERR_CAPACITY: return "chunked exchange needs a window of at least one batch plane of every rank";
    case UA2A_ERR_DEVICE: return "current device is not the plan's device";
    case UA2A_ERR_HIP: return "HIP runtime or launch failure; the plan is disabled";
    case UA2A_ERR_DISABLED: return "plan disabled by an earlier HIP failure";
    case UA2A_ERR_NOMEM: return "out of host memory";
    default: return "unknown status";
    }
}

const char* ua2a_plan_last_error(ua2a_plan_t plan)
{
    if (plan == nullptr || !plan->disabled) return "";
    return plan->reason;
}

int ua2a_plan_set_path(ua2a_plan_t plan, int32_t path)
{
    if (plan == nullptr) return UA2A_ERR_INVALID_ARG;
    if (path != UA2A_PATH_AUTO && path != UA2A_PATH_DIRECT && path != UA2A_PATH_LDS)
        return UA2A_ERR_INVALID_ARG;
    plan->path = path;
    return UA2A_OK;
}

int ua2a_describe(ua2a_plan_t plan, int32_t mode, int32_t chunked, const void* in,
                  const void* out, ua2a_launch_info_t* info)
{
    if (info == nullptr) return UA2A_ERR_INVALID_ARG;
    const int rc = check_call(plan, mode, chunked, in, out);
    if (rc != UA2A_OK) return rc;
    Prepared pr;
    prepare(plan, mode, chunked, in, const_cast<void*>(out), &pr);
    memset(info, 0, sizeof *info);
    info->path = pr.path;
    info->vector_bytes = pr.perm.width;
    info->grid = static_cast<int64_t>(static_cast<uint64_t>(pr.perm.grid) * pr.perm.grid_y *
                                      pr.perm.grid_z);
    info->block = static_cast<int32_t>(pr.perm.block);
    const bool lds = pr.perm.kernel == Kernel::Lds || pr.perm.kernel == Kernel::LdsChunked;
    info->tiles = lds ? pr.perm.lds.num_tiles : pr.perm.direct.num_tiles;
    info->launches = 1;
    info->lds_rows = lds ? static_cast<int32_t>(pr.perm.lds.rows_per_tile) : 0;
    info->grid_dims = pr.perm.grid3d ? 3 : 1;
    info->chunked_form = chunked ? UA2A_CHUNKED_ONE_LAUNCH : 0;
    info->lds_bytes = lds ? static_cast<int32_t>(pr.perm.lds_bytes) : 0;
    info->lds_planes = pr.perm.kernel == Kernel::LdsChunked ? static_cast<int32_t>(pr.perm.lds_chunk.stage) : 0;
    return UA2A_OK;
}

int ua2a_describe_ranks(ua2a_plan_t plan, int32_t mode, const void* const* in_ptrs,
                        void* const* out_ptrs, int32_t first, int32_t count,
                        ua2a_launch_info_t* info)
{
    if (info == nullptr) return UA2A_ERR_INVALID_ARG;
    const int rc = check_ranks_call(plan, mode, in_ptrs, out_ptrs, first, count);
    if (rc != UA2A_OK) return rc;
    Launch L;
    prepare_ranks(plan, mode, in_ptrs, out_ptrs, first, count, &L);
    memset(info, 0, sizeof *info);
    const bool lds = L.kernel == Kernel::LdsRanks;
    info->path = lds ? UA2A_PATH_LDS : UA2A_PATH_DIRECT;
    info->vector_bytes = L.width;
    info->grid = static_cast<int64_t>(static_cast<uint64_t>(L.grid) * L.grid_y * L.grid_z);
    info->block = static_cast<int32_t>(L.block);
    info->tiles = lds ? static_cast<int64_t>(L.lds.num_tiles)
                      : static_cast<int64_t>(L.ranks.tiles_per_slab) * L.ranks.ny * L.ranks.nz;
    info->launches = 1;
    info->lds_rows = lds ? static_cast<int32_t>(L.lds.rows_per_tile) : 0;
    info->grid_dims = lds ? 1 : 3;
    info->lds_bytes = lds ? static_cast<int32_t>(L.lds_bytes) : 0;
    return UA2A_OK;
}

}  // extern "C"

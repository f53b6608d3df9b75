// Host emulation of the ua2a device backend -- TEST ONLY.
//
// Linked with the library's own host logic (ua2a_host.cpp) into
// tests/emu/libua2a_emu.so, it replaces the HIP launches by running the
// kernels' per-thread bodies (ua2a_bodies.h) on the CPU: every tile, every
// thread of the workgroup, the LDS kernel's fill phase for all threads
// before its drain phase (what the workgroup barrier guarantees on the GPU).
// Buffers are ordinary host memory, so the same C ABI can be exercised on a
// machine with no GPU, under AddressSanitizer, and compared with the oracle.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "ua2a_bodies.h"
#include "ua2a_internal.h"

namespace ua2a {

// The window of a one-launch chunked exchange: which lane (of which tile)
// last stored each byte.  A lane may read back only window bytes that it
// stored itself, so no lane depends on another's window accesses, and the
// order in which the emulation runs lanes (one lane's planes after another's)
// cannot hide a race that the device could hit.
namespace {
const uint8_t* g_win = nullptr;
size_t g_win_bytes = 0;
std::vector<int64_t> g_win_owner;     // -1: never stored
int64_t g_lane_id = 0;                // tile * 64 + lane of the running body
// LDS chunked kernel: the running lane's tile and lane; CheckedMem::win_plane
// makes its writer id (tile, plane, lane)
uint32_t g_lane_tile = 0, g_lane_tid = 0, g_lane_planes = 0;
}  // namespace

// PlainMem, with every tile store checked against the tile's written range
// (the kernels store through a buffer resource over exactly that range).
struct CheckedMem : PlainMem {
    template <class T>
    static size_t win_index(const T* p)
    {
        const uint8_t* b = reinterpret_cast<const uint8_t*>(p);
        if (g_win == nullptr || b < g_win || b + sizeof(T) > g_win + g_win_bytes) {
            fprintf(stderr, "emu: window access outside the window\n");
            abort();
        }
        if (g_lane_id == -2) {
            fprintf(stderr, "emu: window access before the lane named its plane\n");
            abort();
        }
        return static_cast<size_t>(b - g_win);
    }
    static void win_plane(uint32_t p)
    {
        if (p >= g_lane_planes) {
            fprintf(stderr, "emu: window plane %u of %u\n", p, g_lane_planes);
            abort();
        }
        g_lane_id = (static_cast<int64_t>(g_lane_tile) * g_lane_planes + p) * kLdsBlock + g_lane_tid;
    }
    template <class T>
    static void st_win(T* p, T v)
    {
        const size_t i = win_index(p);
        for (size_t k = 0; k < sizeof(T); ++k) g_win_owner[i + k] = g_lane_id;
        *p = v;
    }
    template <class T>
    static T ld_win(const T* p)
    {
        const size_t i = win_index(p);
        for (size_t k = 0; k < sizeof(T); ++k)
            if (g_win_owner[i + k] != g_lane_id) {
                fprintf(stderr, "emu: window byte %zu read by a lane that did not store it\n", i + k);
                abort();
            }
        return *p;
    }
    template <class T>
    static void st_tile(uint8_t* base, uint32_t nbytes, uint32_t off, T v)
    {
        if (off % sizeof(T) != 0 || static_cast<uint64_t>(off) + sizeof(T) > nbytes) {
            fprintf(stderr, "emu: tile store at %u (+%zu) outside its %u bytes\n", off, sizeof(T), nbytes);
            abort();
        }
        *reinterpret_cast<T*>(base + off) = v;
    }
};

namespace {
int g_fail_next = 0;          // test hook: fail the next launch with this code
int g_device = 0;             // device the emulation reports as current
int g_launches = 0;           // launches since the last reset
int g_kernel_counts[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
uint32_t g_last_grid = 0;
long long g_tile_budget = -1;  // test hook: direct tiles left to run (< 0: all)
bool g_stalled = false;        // a launch was cut short: later launches on the stream wait

// Whether the next direct tile runs.  When the budget runs out the launch
// stops part-way, as a kernel still in flight would look to a consumer, and
// nothing later on the stream starts (stream order).
bool take_tile()
{
    if (g_tile_budget < 0) return true;
    if (g_tile_budget == 0) {
        g_stalled = true;
        return false;
    }
    --g_tile_budget;
    return true;
}

template <int VB, bool M1>
void run_direct(const Launch& L)
{
    const DirectGeom& g = L.direct;
    // a later part of a publishing exchange: its first workgroup adds the
    // previous part's credits (that part has completed: stream order)
    for (uint32_t i = 0; i < g.sig_count; ++i) ++g.sig_credits[g.sig_first + i];
    if (L.grid3d) {
        for (uint32_t z = 0; z < L.grid_z; ++z)
            for (uint32_t y = 0; y < L.grid_y; ++y)
                for (uint32_t x = 0; x < L.grid; ++x) {
                    if (!take_tile()) return;
                    const DirectTile d = direct_tile_3d<M1>(g, x, y, z);
                    for (uint32_t tid = 0; tid < kDirectBlock; ++tid)
                        direct_tile_body<CheckedMem, VB, M1, kDirectBlock, kDirectUnroll>(g, d, tid);
                }
        return;
    }
    // every workgroup runs the kernel's loop: with cap_tiles > 1, groups of
    // kCapTiles grid-strided tiles (all loaded before any is stored when all
    // are full), then the rest one at a time; each tile visited exactly once
    std::vector<uint8_t> seen(g.num_tiles, 0);
    const uint64_t step = L.grid;
    for (uint32_t bx = 0; bx < L.grid; ++bx) {
        uint64_t t = bx;
        for (; g.cap_tiles > 1 && t + (kCapTiles - 1) * step < g.num_tiles; t += kCapTiles * step) {
            DirectTile d[kCapTiles];
            bool full = true;
            for (uint32_t i = 0; i < kCapTiles; ++i) {
                if (!take_tile()) return;
                if (seen[t + i * step]++) abort();
                d[i] = direct_tile<M1>(g, static_cast<uint32_t>(t + i * step));
                full = full && d[i].nvec == g.tile_vecs;
            }
            for (uint32_t tid = 0; tid < kDirectBlock; ++tid) {
                if (full)
                    direct_full_tiles_body<CheckedMem, VB, M1, kDirectBlock, kCapTiles>(g, d, tid);
                else
                    for (uint32_t i = 0; i < kCapTiles; ++i)
                        direct_tile_body<CheckedMem, VB, M1, kDirectBlock, kDirectUnroll>(g, d[i], tid);
            }
        }
        for (; t < g.num_tiles; t += step) {
            if (!take_tile()) return;
            if (seen[t]++) abort();
            const DirectTile d = direct_tile<M1>(g, static_cast<uint32_t>(t));
            for (uint32_t tid = 0; tid < kDirectBlock; ++tid)
                direct_tile_body<CheckedMem, VB, M1, kDirectBlock, kDirectUnroll>(g, d, tid);
        }
    }
    for (uint32_t t = 0; t < g.num_tiles; ++t)
        if (!seen[t]) abort();
}

// The one-launch chunked exchange: every workgroup of the 3-D grid, every
// lane, with the window's byte owners tracked (see CheckedMem).
template <int VB, bool M1>
void run_chunked(const Launch& L)
{
    const DirectGeom& g = L.direct;
    g_win = g.dst;
    g_win_bytes = static_cast<size_t>(g.w) * static_cast<size_t>(L.chunk.plane) * VB;
    g_win_owner.assign(g_win_bytes, -1);
    if (!L.grid3d) {
        // the flat kernel's loop: workgroup bx takes tiles bx, bx + grid, ...
        std::vector<uint8_t> seen(g.num_tiles, 0);
        for (uint32_t bx = 0; bx < L.grid; ++bx)
            for (uint64_t t = bx; t < g.num_tiles; t += L.grid) {
                if (seen[t]++) abort();
                uint32_t slab;
                const DirectTile d = direct_tile<M1>(g, static_cast<uint32_t>(t), &slab);
                if (d.nvec == 0) continue;
                const uint32_t block = chunked_block<M1>(g, slab);
                const bool full = d.nvec == ChunkedLane<VB>::kVecs * kDirectBlock;
                for (uint32_t tid = 0; tid < kDirectBlock; ++tid) {
                    g_lane_id = static_cast<int64_t>(t) * kDirectBlock + tid;
                    if (full)
                        chunked_tile_body<CheckedMem, VB, M1, kDirectBlock, true>(g, d, L.chunk, block, tid);
                    else
                        chunked_tile_body<CheckedMem, VB, M1, kDirectBlock, false>(g, d, L.chunk, block, tid);
                }
            }
        for (uint32_t t = 0; t < g.num_tiles; ++t)
            if (!seen[t]) abort();
    }
    int64_t tile = 0;
    for (uint32_t z = 0; L.grid3d && z < L.grid_z; ++z)
        for (uint32_t y = 0; y < L.grid_y; ++y)
            for (uint32_t x = 0; x < L.grid; ++x, ++tile) {
                uint32_t block;
                const DirectTile d = chunked_tile<M1>(g, x, y, z, block);
                if (d.nvec == 0) continue;          // padding tile of the grouped order
                const bool full = d.nvec == ChunkedLane<VB>::kVecs * kDirectBlock;
                for (uint32_t tid = 0; tid < kDirectBlock; ++tid) {
                    g_lane_id = tile * kDirectBlock + tid;
                    if (full)
                        chunked_tile_body<CheckedMem, VB, M1, kDirectBlock, true>(g, d, L.chunk, block, tid);
                    else
                        chunked_tile_body<CheckedMem, VB, M1, kDirectBlock, false>(g, d, L.chunk, block, tid);
                }
            }
    // every window byte belongs to exactly one lane and was written
    for (size_t i = 0; i < g_win_bytes; ++i)
        if (g_win_owner[i] < 0) {
            fprintf(stderr, "emu: window byte %zu never written\n", i);
            abort();
        }
    g_win = nullptr;
    g_win_bytes = 0;
}

// The wait kernel with nothing running beside it: a counter short of its
// target can never move, so the time-out is immediate.
void run_wait(const WaitGeom& g)
{
    for (uint32_t i = 0; i < g.count; ++i)
        if (!credit_reached(g.credits[g.first + i], g.target)) {
            *g.status = 1;
            return;
        }
}

template <int G, bool M1, class Bases>
void run_lds(const LdsGeom& g, const Bases& bases)
{
    // exactly lds_bytes, so any access past the reserved LDS is a heap
    // overflow that AddressSanitizer reports
    std::vector<uint8_t> lds(g.lds_bytes);
    std::vector<uint8_t> seen(g.num_tiles, 0);
    for (uint32_t slot = 0; slot < g.num_slots; ++slot) {
        const uint32_t t = lds_slot_tile(g, slot);
        if (t >= g.num_tiles) continue;
        if (seen[t]++) {                 // the slot order must visit each tile once
            fprintf(stderr, "emu: LDS tile %u visited twice\n", t);
            abort();
        }
        memset(lds.data(), 0xA5, lds.size());
        const LdsTile d = lds_tile(g, bases, t);
        for (uint32_t tid = 0; tid < kLdsBlock; ++tid)
            lds_fill<CheckedMem, G, M1, kLdsBlock, (G == 16 ? kLdsUnroll : 1)>(g, bases, d, tid, lds.data());
        for (uint32_t tid = 0; tid < kLdsBlock; ++tid)
            lds_drain<CheckedMem, G, M1, kLdsBlock>(g, bases, d, tid, lds.data());
    }
    for (uint32_t t = 0; t < g.num_tiles; ++t)
        if (!seen[t]) {                  // ... and miss none
            fprintf(stderr, "emu: LDS tile %u never visited\n", t);
            abort();
        }
}

// The LDS path's one-launch chunked exchange: every launch slot's tile
// through all planes -- fill for all lanes (the workgroup barrier), then
// each lane's drain through the window, with the window bytes' writers
// tracked per (tile, plane, lane): a lane may read back only what it stored
// in the same plane.
template <int G, bool M1>
void run_lds_chunked(const Launch& L)
{
    const LdsGeom& g = L.lds;
    const LdsChunkGeom& c = L.lds_chunk;
    g_win = M1 ? g.p_ptr : g.a_ptr;
    g_win_bytes = static_cast<size_t>(g.w) * static_cast<size_t>(c.plane);
    g_win_owner.assign(g_win_bytes, -1);
    // exactly the launch's LDS (stage images), so an access past it is a heap
    // overflow under the sanitizer build
    std::vector<uint8_t> lds(L.lds_bytes);
    std::vector<uint8_t> seen(g.num_tiles, 0);
    for (uint32_t slot = 0; slot < g.num_slots; ++slot) {
        const uint32_t t = lds_slot_tile(g, slot);
        if (t >= g.num_tiles) continue;
        if (seen[t]++) {
            fprintf(stderr, "emu: LDS tile %u visited twice\n", t);
            abort();
        }
        // as the kernel: `stage` planes filled (one image each), a barrier,
        // then each lane drains them plane after plane, then a barrier
        const uint32_t per = c.stage == 0 ? 1u : std::min(c.stage, kLdsChunkStage);
        for (uint32_t p0 = 0, n = 0; p0 < c.planes; p0 += n) {
            n = std::min(per, c.planes - p0);
            memset(lds.data(), 0xA5, lds.size());
            for (uint32_t tid = 0; tid < kLdsBlock; ++tid)
                lds_chunked_fill<CheckedMem, G, M1, kLdsBlock, (G == 16 ? kLdsUnroll : 1), kLdsChunkStage>(
                    g, c, t, p0, n, tid, lds.data());
            for (uint32_t tid = 0; tid < kLdsBlock; ++tid) {
                g_lane_tile = t;
                g_lane_tid = tid;
                g_lane_planes = c.planes;
                g_lane_id = -2;      // win_plane() must name the plane before any window access
                lds_chunked_drain<CheckedMem, G, M1, kLdsBlock, kLdsReadback, kLdsChunkStage>(g, c, t, p0, n, tid,
                                                                                          lds.data());
            }
        }
    }
    for (uint32_t t = 0; t < g.num_tiles; ++t)
        if (!seen[t]) {
            fprintf(stderr, "emu: LDS tile %u never visited\n", t);
            abort();
        }
    for (size_t i = 0; i < g_win_bytes; ++i)
        if (g_win_owner[i] < 0) {
            fprintf(stderr, "emu: window byte %zu never written\n", i);
            abort();
        }
    g_win = nullptr;
    g_win_bytes = 0;
}

template <bool M1>
int dispatch_lds_chunked(const Launch& L)
{
    switch (L.width) {
    case 16: run_lds_chunked<16, M1>(L); return 0;
    case 8: run_lds_chunked<8, M1>(L); return 0;
    case 4: run_lds_chunked<4, M1>(L); return 0;
    case 2: run_lds_chunked<2, M1>(L); return 0;
    case 1: run_lds_chunked<1, M1>(L); return 0;
    default: return 1;
    }
}

template <int VB>
void run_copy(const CopyGeom& g)
{
    for (uint32_t t = 0; t < g.num_tiles; ++t)
        for (uint32_t tid = 0; tid < kCopyBlock; ++tid)
            copy_tile_body<CheckedMem, VB, kCopyBlock, kDirectUnroll>(g, t, tid);
}

// Every workgroup of the launch's grid runs the kernel's loops over the
// slab grid exactly as on the device.
template <int VB, bool M1, bool TWO, bool PART>
void run_ranks(const Launch& L)
{
    const RanksGeom& g = L.ranks;
    for (uint32_t bz = 0; bz < L.grid_z; ++bz)
        for (uint32_t by = 0; by < L.grid_y; ++by)
            for (uint32_t bx = 0; bx < L.grid; ++bx)
                for (uint32_t z = bz; z < g.nz; z += L.grid_z)
                    for (uint32_t y = by; y < g.ny; y += L.grid_y)
                        for (uint32_t x = bx; x < g.tiles_per_slab; x += L.grid) {
                            const RanksTile d = ranks_tile<M1, TWO>(g, x, y, z);
                            for (uint32_t tid = 0; tid < kDirectBlock; ++tid)
                                ranks_tile_body<CheckedMem, VB, M1, TWO, PART, kDirectBlock>(g, d, tid);
                        }
}

// Every workgroup of the pack launch's grid runs the kernel's loops.
template <int VB>
void run_pack(const Launch& L)
{
    const PackGeom& g = L.pack;
    for (uint32_t bz = 0; bz < L.grid_z; ++bz)
        for (uint32_t by = 0; by < L.grid_y; ++by)
            for (uint32_t bx = 0; bx < L.grid; ++bx)
                for (uint32_t z = bz; z < g.nz; z += L.grid_z)
                    for (uint32_t y = by; y < g.ny; y += L.grid_y)
                        for (uint32_t x = bx; x < g.tiles_per_block; x += L.grid) {
                            const PackTile t = pack_tile<VB>(g, x, y, z);
                            for (uint32_t tid = 0; tid < kDirectBlock; ++tid)
                                pack_tile_body<CheckedMem, VB, kDirectBlock>(t, tid);
                        }
}

int dispatch_pack(const Launch& L, int vb)
{
    switch (vb) {
    case 16: run_pack<16>(L); return 0;
    case 8: run_pack<8>(L); return 0;
    case 4: run_pack<4>(L); return 0;
    case 2: run_pack<2>(L); return 0;
    case 1: run_pack<1>(L); return 0;
    default: return 1;
    }
}

template <bool M1, bool TWO, bool PART>
int dispatch_ranks(const Launch& L, int vb)
{
    switch (vb) {
    case 16: run_ranks<16, M1, TWO, PART>(L); return 0;
    case 8: run_ranks<8, M1, TWO, PART>(L); return 0;
    case 4: run_ranks<4, M1, TWO, PART>(L); return 0;
    case 2: run_ranks<2, M1, TWO, PART>(L); return 0;
    case 1: run_ranks<1, M1, TWO, PART>(L); return 0;
    default: return 1;
    }
}

template <bool M1>
int dispatch_direct(const Launch& L, int vb)
{
    switch (vb) {
    case 16: run_direct<16, M1>(L); return 0;
    case 8: run_direct<8, M1>(L); return 0;
    case 4: run_direct<4, M1>(L); return 0;
    case 2: run_direct<2, M1>(L); return 0;
    case 1: run_direct<1, M1>(L); return 0;
    default: return 1;
    }
}

template <bool M1>
int dispatch_chunked(const Launch& L, int vb)
{
    switch (vb) {
    case 16: run_chunked<16, M1>(L); return 0;
    case 8: run_chunked<8, M1>(L); return 0;
    case 4: run_chunked<4, M1>(L); return 0;
    case 2: run_chunked<2, M1>(L); return 0;
    case 1: run_chunked<1, M1>(L); return 0;
    default: return 1;
    }
}

template <bool M1, class Bases>
int dispatch_lds(const LdsGeom& g, const Bases& bases, int gw)
{
    switch (gw) {
    case 16: run_lds<16, M1>(g, bases); return 0;
    case 8: run_lds<8, M1>(g, bases); return 0;
    case 4: run_lds<4, M1>(g, bases); return 0;
    case 2: run_lds<2, M1>(g, bases); return 0;
    case 1: run_lds<1, M1>(g, bases); return 0;
    default: return 1;
    }
}

int dispatch_copy(const CopyGeom& g, int vb)
{
    switch (vb) {
    case 16: run_copy<16>(g); return 0;
    case 8: run_copy<8>(g); return 0;
    case 4: run_copy<4>(g); return 0;
    case 2: run_copy<2>(g); return 0;
    case 1: run_copy<1>(g); return 0;
    default: return 1;
    }
}
}  // namespace

int backend_current_device(int32_t* device)
{
    *device = g_device;
    return 0;
}

// The library's own window of the no-allocation entry point: host memory of
// the same size per emulated device, 256-byte aligned like the device array.
int backend_scratch_window(int32_t device, uint8_t** window)
{
    static std::vector<std::vector<uint8_t>> per_device(64);
    if (device < 0 || device >= 64) return 10;
    std::vector<uint8_t>& buf = per_device[device];
    if (buf.empty()) buf.resize(UA2A_NOALLOC_WINDOW_BYTES + 256);
    uintptr_t p = reinterpret_cast<uintptr_t>(buf.data());
    *window = buf.data() + ((256 - p % 256) % 256);
    return 0;
}

const char* backend_error_name(int) { return "emulated launch failure"; }

int backend_launch(const Launch& L, void*)
{
    if (g_fail_next) {
        const int e = g_fail_next;
        g_fail_next = 0;
        return e;
    }
    ++g_launches;
    ++g_kernel_counts[static_cast<int>(L.kernel)];
    if (g_stalled) return 0;       // queued behind an unfinished launch
    g_last_grid = L.grid;
    if (L.grid < 1) return 2;
    const uint32_t want_block = (L.kernel == Kernel::Lds || L.kernel == Kernel::LdsRanks ||
                                 L.kernel == Kernel::LdsChunked) ? kLdsBlock
                              : L.kernel == Kernel::Copy ? kCopyBlock
                              : (L.kernel == Kernel::Wait || L.kernel == Kernel::Signal) ? kWaitBlock
                              : kDirectBlock;
    if (L.block != want_block) return 5;
    switch (L.kernel) {
    case Kernel::Direct:
        if (L.grid3d) {
            // the 3-D grid must cover every tile of the launch exactly once (a
            // part of a publishing exchange covers fewer receivers than w)
            const uint64_t slabs = static_cast<uint64_t>(L.grid_y) * L.grid_z;
            if (L.grid != L.direct.tiles_per_slab || L.direct.group != 0 ||
                slabs * L.direct.tiles_per_slab != L.direct.num_tiles ||
                L.grid_y != (L.mode ? L.direct.nb : L.direct.w) || L.grid_z % (L.mode ? 1u : L.direct.nb))
                return 6;
        } else if (L.grid_y != 1 || L.grid_z != 1) {
            return 7;
        }
        return L.mode ? dispatch_direct<true>(L, L.width) : dispatch_direct<false>(L, L.width);
    case Kernel::Chunked: {
        // the 3-D grid of one plane's tiles of every rank, z = window block;
        // or, mode 0 with the grouped order, x = (tile group, r, tile), y = j
        const DirectGeom& g = L.direct;
        if (g.nb != 1 || g.sig_count != 0 || L.chunk.planes < 1 ||
            L.chunk.plane != (L.mode ? g.p_rank : g.a_rank))
            return 6;
        if (!L.grid3d) {
            // flat grid: workgroups loop over the tiles
            if (L.grid_y != 1 || L.grid_z != 1 || L.grid > g.num_tiles) return 7;
        } else if (g.group == 0 ? (L.grid != g.tiles_per_slab ||
                            static_cast<uint64_t>(L.grid_y) * L.grid_z * g.tiles_per_slab != g.num_tiles ||
                            L.grid_y != (L.mode ? 1u : g.w) || L.grid_z != g.w)
                         : (L.mode || L.grid != g.groups * g.group * g.w || L.grid_y != g.w || L.grid_z != 1 ||
                            static_cast<uint64_t>(L.grid) * L.grid_y != g.num_tiles))
            return 6;
        return L.mode ? dispatch_chunked<true>(L, L.width) : dispatch_chunked<false>(L, L.width);
    }
    case Kernel::Lds:
        if (L.grid_y != 1 || L.grid_z != 1) return 7;
        if (L.lds_bytes != L.lds.lds_bytes || L.lds.lds_bytes < 16 + L.lds.rows_per_tile * L.lds.lrow ||
            L.lds.lrow != L.lds.row + L.lds.pad || (L.lds.pad && L.width != 16) ||
            L.lds.num_slots < L.lds.num_tiles || (L.lds.xlog && L.lds.num_slots % (kXcds << L.lds.xlog) != 0) ||
            L.grid > L.lds.num_slots)
            return 3;
        return L.mode ? dispatch_lds<true>(L.lds, StackedBases{L.lds}, L.width)
                      : dispatch_lds<false>(L.lds, StackedBases{L.lds}, L.width);
    case Kernel::LdsChunked: {
        // plane 0 of every rank <-> the window (one plane of every rank); every
        // window -> output offset a multiple of the piece size
        const LdsGeom& g = L.lds;
        const LdsChunkGeom& c = L.lds_chunk;
        if (L.grid_y != 1 || L.grid_z != 1) return 7;
        if (c.image != g.lds_bytes || c.image % 16 != 0 || c.stage < 1 || c.stage > c.planes ||
            c.stage > kLdsChunkStage || (c.stage > 1 && c.plane % 16 != 0) ||
            static_cast<uint64_t>(L.lds_bytes) != static_cast<uint64_t>(c.stage) * c.image ||
            L.lds_bytes > 65536 || g.lds_bytes < 16 + g.rows_per_tile * g.lrow || g.lrow != g.row + g.pad ||
            (g.pad && L.width != 16) || g.num_slots < g.num_tiles ||
            (g.xlog && g.num_slots % (kXcds << g.xlog) != 0) || L.grid > g.num_slots || g.nb != 1 ||
            g.p_plane != 0 || g.a_plane != 0 || c.planes < 1 || c.plane % L.width != 0 ||
            (L.mode ? g.p_rank : g.a_rank) != c.plane ||
            (reinterpret_cast<uintptr_t>(c.out) - reinterpret_cast<uintptr_t>(L.mode ? g.p_ptr : g.a_ptr)) %
                static_cast<uintptr_t>(L.width))
            return 3;
        return L.mode ? dispatch_lds_chunked<true>(L) : dispatch_lds_chunked<false>(L);
    }
    case Kernel::LdsRanks:
        if (L.grid_y != 1 || L.grid_z != 1) return 7;
        if (L.lds_bytes != L.lds.lds_bytes || L.lds.lds_bytes < 16 + L.lds.rows_per_tile * L.lds.lrow ||
            L.lds.p_rank != 0 || L.lds.a_rank != 0 ||
            L.lds.num_slots < L.lds.num_tiles || (L.lds.xlog && L.lds.num_slots % (kXcds << L.lds.xlog) != 0) ||
            L.grid > L.lds.num_slots)
            return 3;
        return L.mode ? dispatch_lds<true>(L.lds, TableBases{L.lds_tab}, L.width)
                      : dispatch_lds<false>(L.lds, TableBases{L.lds_tab}, L.width);
    case Kernel::Copy:
        return dispatch_copy(L.copy, L.width);
    case Kernel::Wait:
        if (L.grid != 1 || L.grid_y != 1 || L.grid_z != 1 || L.wait.spin_limit < 1) return 9;
        run_wait(L.wait);
        return 0;
    case Kernel::Signal:
        if (L.grid != 1 || L.grid_y != 1 || L.grid_z != 1) return 9;
        for (uint32_t i = 0; i < L.signal.count; ++i) ++L.signal.credits[L.signal.first + i];
        return 0;
    case Kernel::Pack:
        if (L.grid_y < 1 || L.grid_z < 1 || L.grid_y > 65535 || L.grid_z > 65535 ||
            static_cast<uint64_t>(L.grid) * L.block > (uint64_t(1) << 31))
            return 8;
        return dispatch_pack(L, L.width);
    case Kernel::Ranks:
        // the hardware's limits on a dispatch's extents
        if (L.grid_y < 1 || L.grid_z < 1 || L.grid_y > 65535 || L.grid_z > 65535 ||
            static_cast<uint64_t>(L.grid) * L.block > (uint64_t(1) << 31))
            return 8;
        if (!L.mode) return dispatch_ranks<false, false, false>(L, L.width);
        if (L.ranks.count == L.ranks.w)
            return L.ranks.two_runs ? dispatch_ranks<true, true, false>(L, L.width)
                                    : dispatch_ranks<true, false, false>(L, L.width);
        return L.ranks.two_runs ? dispatch_ranks<true, true, true>(L, L.width)
                                : dispatch_ranks<true, false, true>(L, L.width);
    }
    return 4;
}

}  // namespace ua2a

extern "C" {

void ua2a_emu_fail_next_launch(int code) { ua2a::g_fail_next = code; }
void ua2a_emu_set_tile_budget(long long tiles)
{
    ua2a::g_tile_budget = tiles;
    ua2a::g_stalled = false;
}
void ua2a_emu_set_device(int device) { ua2a::g_device = device; }

void ua2a_emu_reset_counts(void)
{
    ua2a::g_launches = 0;
    for (int& c : ua2a::g_kernel_counts) c = 0;
}

int ua2a_emu_launches(void) { return ua2a::g_launches; }
int ua2a_emu_kernel_count(int kernel) { return ua2a::g_kernel_counts[kernel]; }
unsigned ua2a_emu_last_grid(void) { return ua2a::g_last_grid; }

/* The LDS kernels' launch-slot order for num_slots slots with 2^xlog
 * consecutive tiles per XCD turn: out[L] = the tile slot L runs. */
void ua2a_emu_lds_slot_tiles(uint32_t num_slots, uint32_t xlog, uint32_t* out)
{
    ua2a::LdsGeom g;
    memset(&g, 0, sizeof g);
    g.num_slots = num_slots;
    g.xlog = xlog;
    for (uint32_t L = 0; L < num_slots; ++L) out[L] = ua2a::lds_slot_tile(g, L);
}

/* The kernels' magic-number division, for checking against exact division. */
void ua2a_emu_fdiv(uint32_t d, const uint32_t* n, uint32_t* q, int count)
{
    const ua2a::Div32 f = ua2a::make_div32(d);
    for (int i = 0; i < count; ++i) q[i] = ua2a::fdiv(n[i], f);
}

}  // extern "C"

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

#include <vector>

#include "ua2a_bodies.h"
#include "ua2a_internal.h"

namespace ua2a {

// PlainMem, with every tile store checked against the tile's written range
// (the kernels store through a buffer resource over exactly that range).
struct CheckedMem : PlainMem {
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
int g_kernel_counts[7] = {0, 0, 0, 0, 0, 0, 0};
int g_carry_launches = 0;     // direct launches that also copied a chunked plane out
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
                    if (L.carry.dst != nullptr) {
                        // a chunked plane after the first: every lane of both
                        // waves loads, then (the barrier) every lane stores
                        uint8_t* ct = L.carry.dst + (d.dst_slab + d.u0 + static_cast<int64_t>(z) * L.carry.step) * VB;
                        std::vector<CarryVectors<VB>> v(kCarryBlock);
                        for (uint32_t tid = 0; tid < kCarryBlock; ++tid)
                            v[tid] = direct_carry_load<CheckedMem, VB, M1, kDirectBlock>(
                                g, d, tid / kDirectBlock, tid % kDirectBlock);
                        for (uint32_t tid = 0; tid < kCarryBlock; ++tid)
                            direct_carry_store<CheckedMem, VB, M1, kDirectBlock>(
                                g, d, tid / kDirectBlock, tid % kDirectBlock, ct, v[tid]);
                        continue;
                    }
                    for (uint32_t tid = 0; tid < kDirectBlock; ++tid)
                        direct_tile_body<CheckedMem, VB, M1, kDirectBlock, kDirectUnroll>(g, d, tid);
                }
        return;
    }
    if (L.carry.dst != nullptr) abort();   // the carry launch exists on the 3-D grid only
    // a capped grid loops grid-stride; every tile is visited exactly once either way
    for (uint32_t t = 0; t < g.num_tiles; ++t) {
        if (!take_tile()) return;
        const DirectTile d = direct_tile<M1>(g, t);
        for (uint32_t tid = 0; tid < kDirectBlock; ++tid)
            direct_tile_body<CheckedMem, VB, M1, kDirectBlock, kDirectUnroll>(g, d, tid);
    }
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
    if (L.kernel == Kernel::Direct && L.carry.dst != nullptr) ++g_carry_launches;
    if (g_stalled) return 0;       // queued behind an unfinished launch
    g_last_grid = L.grid;
    if (L.grid < 1) return 2;
    const uint32_t want_block = (L.kernel == Kernel::Lds || L.kernel == Kernel::LdsRanks) ? kLdsBlock
                              : L.kernel == Kernel::Copy ? kCopyBlock
                              : (L.kernel == Kernel::Wait || L.kernel == Kernel::Signal) ? kWaitBlock
                              : (L.kernel == Kernel::Direct && L.carry.dst != nullptr) ? kCarryBlock
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
            // a carry launch covers one plane (z is then the window block)
            if (L.carry.dst != nullptr && (L.direct.nb != 1 || L.direct.sig_count != 0)) return 8;
        } else if (L.grid_y != 1 || L.grid_z != 1 || L.carry.dst != nullptr) {
            return 7;
        }
        return L.mode ? dispatch_direct<true>(L, L.width) : dispatch_direct<false>(L, L.width);
    case Kernel::Lds:
        if (L.grid_y != 1 || L.grid_z != 1) return 7;
        if (L.lds_bytes != L.lds.lds_bytes || L.lds.lds_bytes < 16 + L.lds.rows_per_tile * L.lds.lrow ||
            L.lds.lrow != L.lds.row + L.lds.pad || (L.lds.pad && L.width != 16) ||
            L.lds.num_slots < L.lds.num_tiles || (L.lds.xlog && L.lds.num_slots % (kXcds << L.lds.xlog) != 0) ||
            L.grid > L.lds.num_slots)
            return 3;
        return L.mode ? dispatch_lds<true>(L.lds, StackedBases{L.lds}, L.width)
                      : dispatch_lds<false>(L.lds, StackedBases{L.lds}, L.width);
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
    ua2a::g_carry_launches = 0;
}

int ua2a_emu_launches(void) { return ua2a::g_launches; }
int ua2a_emu_kernel_count(int kernel) { return ua2a::g_kernel_counts[kernel]; }
int ua2a_emu_carry_launches(void) { return ua2a::g_carry_launches; }
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

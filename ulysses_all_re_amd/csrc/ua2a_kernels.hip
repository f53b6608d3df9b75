// gfx950 (MI355X, CDNA4) kernels of the Ulysses all_to_all_4D exchange and
// the HIP backend that launches them.
//
// The exchange is pure data movement (FastVideo "ulysses_a2a" API page,
// method run_armed: mode 0 [B,S_local,H,D] -> [B,S_local*w,H/w,D] per rank,
// mode 1 the inverse), so it is bound by HBM bandwidth: no MFMA, every byte
// read once and written once.  The kernels:
//
//  * ua2a_direct_kernel  -- each lane moves one whole vector (16 bytes when
//    the run and both bases allow) per pass; a workgroup covers one tile of
//    consecutive vectors of the side being WRITTEN (the A side in mode 0,
//    the P side in mode 1), so its stores are contiguous and its loads are
//    whole runs.  One tile per workgroup.  Used for runs of at least a few
//    cache lines.
//  * ua2a_lds_kernel     -- for short or unaligned runs: a workgroup stages
//    a contiguous span of P-side rows in LDS and moves both sides as 16-byte
//    aligned chunks, re-ordering runs inside LDS in G-byte pieces; tiles go
//    to the XCDs in runs of consecutive tiles (see LdsGeom).
//  * ua2a_chunked_kernel -- a whole chunked exchange in one launch on the
//    direct path: each workgroup owns one tile of the one-plane window and
//    moves it through every batch plane (permute into the window, read back,
//    store to the output); ua2a_chunked_flat_kernel -- the same on a flat
//    grid capped by a `blocks` hint, each workgroup looping over tiles.
//  * ua2a_lds_chunked_kernel -- a whole chunked exchange in one launch on
//    the LDS path: each workgroup keeps its LDS tile through every batch
//    plane (fill from the input, then each lane stores its chunks into the
//    window, reads them back and stores them to the output).
//  * ua2a_copy_kernel    -- contiguous block copy: mode 0's unpack of a
//    receiver's window into its output.
//  * ua2a_ranks_kernel   -- the direct kernel's scheme over per-rank
//    allocations (pointer tables) and a range of sending ranks;
//    ua2a_lds_ranks_kernel -- the LDS kernel over them.
//  * ua2a_pack_kernel    -- mode 1's pack into the receivers' windows:
//    contiguous blocks from every sender to every receiver.
//  * ua2a_signal_kernel  -- adds the readiness credits of a publishing
//    exchange's last part (earlier parts' credits are added by the next
//    part's first workgroup); ua2a_wait_kernel -- one wave that waits for
//    them, with a bounded number of polls.
//
// The per-thread bodies (ua2a_bodies.h) and their index math
// (ua2a_geometry.h) are shared with a host emulation used by the tests.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ua2a_bodies.h"
#include "ua2a_internal.h"

namespace ua2a {

// Every byte is read once and written once: mark the global accesses
// non-temporal so the streams do not displace other data in L2 / MALL.
typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));

// Cache-policy bits of a buffer store on gfx950: non-temporal, device scope.
// A tile's stores go out as buffer stores with both: measured +0.8 % (mode 0)
// and +1.2 % (mode 1) on the video-DiT exchange against non-temporal global
// stores, which set NT only.  Loads stay global and non-temporal (64-bit
// addresses; the same bits there gained nothing).
constexpr int kStoreCachePolicy = 2 /* nt */ | 16 /* sc1 */;
constexpr int kRawBufferFlags = 0x00020000;   // buffer resource word 3: untyped 32-bit data

struct StreamMem {
    template <class T>
    __device__ static T ld(const T* p) { return __builtin_nontemporal_load(p); }
    template <class T>
    __device__ static void st(T* p, T v) { __builtin_nontemporal_store(v, p); }
    // The window of a one-launch chunked exchange is read back right after
    // it is written, so its accesses keep the default cache policy (the
    // lines stay in the XCD's L2 between the store and the load).
    template <class T>
    __device__ static T ld_win(const T* p) { return *p; }
    template <class T>
    __device__ static void st_win(T* p, T v) { *p = v; }
    __device__ static void win_order() { asm volatile("" ::: "memory"); }
    __device__ static void win_plane(uint32_t) {}
    // A store at byte `off` of a tile's written range [base, base + nbytes),
    // through a buffer resource over that range (a store outside it would be
    // dropped by the hardware rather than land elsewhere).
    template <class T>
    __device__ static void st_tile(uint8_t* base, uint32_t nbytes, uint32_t off, T v)
    {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, nbytes, kRawBufferFlags);
        if constexpr (sizeof(T) == 16)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32, v), r, off, 0, kStoreCachePolicy);
        else if constexpr (sizeof(T) == 8)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i32, v), r, off, 0, kStoreCachePolicy);
        else if constexpr (sizeof(T) == 4)
            __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStoreCachePolicy);
        else if constexpr (sizeof(T) == 2)
            __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kStoreCachePolicy);
        else
            __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, kStoreCachePolicy);
    }
    // The first or last chunk of a span that starts or ends inside an aligned
    // 16-byte chunk is read whole, in one load like the span's other chunks
    // (reading its in-span pieces one by one stalled the wave on a chain of
    // small loads).  An aligned 16-byte chunk lies within one page, so the
    // bytes outside the span are mapped; they are never used, and only an
    // exchange's input, which nothing writes meanwhile, is read this way.
    __device__ static u32x4 ld_part(const u32x4* p, uint32_t, uint32_t) { return __builtin_nontemporal_load(p); }
    // A span's partial first or last chunk is written piece by piece with
    // plain stores (lines written partly through a buffer range and partly
    // plainly measured 9-52 % slower).
    template <class T>
    __device__ static void st_piece(T* p, T v) { *p = v; }
};

// Kernel arguments up front.  A direct, copy or per-rank workgroup moves one
// 1 KiB tile, so how soon its first load leaves decides much of its life.
// Left alone, the compiler loads each argument field where it is first used:
// behind the first branch, in two to four dependent rounds through the
// scalar cache.  These empty statements take the fields a kernel reads as
// scalar-register inputs, so they are all requested in one batch at the
// kernel's start and waited for once (measured on the direct kernel: +0.5 to
// +0.9 % on the video-DiT exchange, +1.5 to +7 % on 25-110 MB exchanges).
__device__ __forceinline__ void args_up_front(const DirectGeom& g)
{
    asm volatile("" ::"s"(g.src), "s"(g.dst), "s"(g.a_rank), "s"(g.a_plane), "s"(g.p_rank), "s"(g.p_plane),
                 "s"(g.vr), "s"(g.p_row), "s"(g.s_local), "s"(g.nb), "s"(g.slab_vecs), "s"(g.tile_vecs),
                 "s"(g.d_vr.m), "s"(g.d_vr.s), "s"(g.d_prow.m), "s"(g.d_prow.s), "s"(g.d_nb.m), "s"(g.d_nb.s));
}

// ... and the flat-grid decode's fields besides
__device__ __forceinline__ void flat_args_up_front(const DirectGeom& g)
{
    args_up_front(g);
    asm volatile("" ::"s"(g.num_tiles), "s"(g.tiles_per_slab), "s"(g.group), "s"(g.groups), "s"(g.w),
                 "s"(g.cap_tiles),
                 "s"(g.d_tps.m), "s"(g.d_tps.s), "s"(g.d_w.m), "s"(g.d_w.s), "s"(g.d_group.m),
                 "s"(g.d_group.s), "s"(g.d_groups.m), "s"(g.d_groups.s));
}

__device__ __forceinline__ void args_up_front(const CopyGeom& g)
{
    asm volatile("" ::"s"(g.src), "s"(g.dst), "s"(g.src_stride), "s"(g.dst_stride), "s"(g.span),
                 "s"(g.tile_vecs), "s"(g.tiles_per_span), "s"(g.num_tiles), "s"(g.d_tps.m), "s"(g.d_tps.s));
}

// (the per-rank tables are indexed by values computed in the kernel, so
// their entries still come in a later round)
__device__ __forceinline__ void args_up_front(const RanksGeom& g)
{
    asm volatile("" ::"s"(g.a_plane), "s"(g.p_plane), "s"(g.vr), "s"(g.p_row), "s"(g.seg), "s"(g.s_local),
                 "s"(g.w), "s"(g.nb), "s"(g.first), "s"(g.count), "s"(g.slab_vecs), "s"(g.tile_vecs),
                 "s"(g.tiles_per_slab), "s"(g.ny), "s"(g.nz), "s"(g.two_runs), "s"(g.d_vr.m), "s"(g.d_vr.s),
                 "s"(g.d_seg.m), "s"(g.d_seg.s), "s"(g.d_nb.m), "s"(g.d_nb.s), "s"(g.d_count.m),
                 "s"(g.d_count.s));
}

__device__ __forceinline__ void args_up_front(const PackGeom& g)
{
    asm volatile("" ::"s"(g.src_b), "s"(g.src_q), "s"(g.dst_b), "s"(g.dst_k), "s"(g.block_vecs),
                 "s"(g.tile_vecs), "s"(g.tiles_per_block), "s"(g.first), "s"(g.ny), "s"(g.nz), "s"(g.d_nb.d),
                 "s"(g.d_nb.m), "s"(g.d_nb.s));
}

// The LDS kernels already fetch their fields at the start, but in two rounds
// (the slot count first, the rest after the first slot check); one round
// measured +0.2 to +1 % on stacked tensors and -0.1 to -0.6 % on per-rank
// tables, so only the stacked kernel takes it.
__device__ __forceinline__ void args_up_front(const LdsGeom& g)
{
    asm volatile("" ::"s"(g.p_ptr), "s"(g.a_ptr), "s"(g.a_rank), "s"(g.a_plane), "s"(g.p_rank), "s"(g.p_plane),
                 "s"(g.run), "s"(g.row), "s"(g.pad), "s"(g.lrow), "s"(g.s_local), "s"(g.rows_per_tile),
                 "s"(g.tiles_per_plane), "s"(g.num_tiles), "s"(g.num_slots), "s"(g.xlog), "s"(g.w), "s"(g.nb),
                 "s"(g.j0), "s"(g.a_window), "s"(g.a_whole16), "s"(g.stride_full), "s"(g.stride_last));
    asm volatile("" ::"s"(g.d_tpp.m), "s"(g.d_tpp.s), "s"(g.d_nb.m), "s"(g.d_nb.s), "s"(g.d_run.m),
                 "s"(g.d_run.s), "s"(g.d_row.m), "s"(g.d_row.s), "s"(g.d_stride_full.m),
                 "s"(g.d_stride_full.s), "s"(g.d_stride_last.m), "s"(g.d_stride_last.s));
}

// Readiness credits of a publishing exchange.  A launch that follows a part
// on the same stream starts only after that part has completed, so every
// byte of the part is visible device-wide by then; a release add at device
// scope passes that on to whoever reads the counter with acquire order (the
// wait kernel), on any XCD.
__device__ __forceinline__ void add_credits(uint32_t* credits, uint32_t first, uint32_t count)
{
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x)
        __hip_atomic_fetch_add(credits + first + i, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// SIG: a later part of a publishing exchange, whose first workgroup adds the
// previous part's credits (sparing a launch between the two parts).
template <int VB, bool MODE1, bool SIG>
__global__ __launch_bounds__(kDirectBlock) void ua2a_direct_kernel(DirectGeom g)
{
    flat_args_up_front(g);
    if (SIG && blockIdx.x == 0) add_credits(g.sig_credits, g.sig_first, g.sig_count);
    // 64-bit tile counters: t + gridDim.x may pass 2^32 when num_tiles is near it.
    // With cap_tiles > 1 (a grid capped so low that one tile per workgroup
    // would keep too few loads in flight) a workgroup takes its tiles
    // kCapTiles at a time (t, t + grid, ...), all loaded before any is stored;
    // a group holding a partial or padding tile, the rest, and every other
    // grid go one tile at a time.
    static_assert(kTileBytes == 16 * kDirectBlock, "a full tile is 16 bytes per lane");
    const uint64_t step = gridDim.x;
    uint64_t t = blockIdx.x;
    for (; g.cap_tiles > 1 && t + (kCapTiles - 1) * step < g.num_tiles; t += kCapTiles * step) {
        DirectTile d[kCapTiles];
        bool full = true;
#pragma unroll
        for (uint32_t i = 0; i < kCapTiles; ++i) {
            d[i] = direct_tile<MODE1>(g, static_cast<uint32_t>(t + i * step));
            full = full && d[i].nvec == g.tile_vecs;
        }
        if (full) {
            direct_full_tiles_body<StreamMem, VB, MODE1, kDirectBlock, kCapTiles>(g, d, threadIdx.x);
        } else {
            for (uint32_t i = 0; i < kCapTiles; ++i)
                direct_tile_body<StreamMem, VB, MODE1, kDirectBlock, kDirectUnroll>(g, d[i], threadIdx.x);
        }
    }
    for (; t < g.num_tiles; t += step)
        direct_tile_body<StreamMem, VB, MODE1, kDirectBlock, kDirectUnroll>(
            g, direct_tile<MODE1>(g, static_cast<uint32_t>(t)), threadIdx.x);
}

// One tile per workgroup on a 3-D grid (see direct_tile_3d).
template <int VB, bool MODE1, bool SIG>
__global__ __launch_bounds__(kDirectBlock) void ua2a_direct3d_kernel(DirectGeom g)
{
    args_up_front(g);
    if (SIG && (blockIdx.x | blockIdx.y | blockIdx.z) == 0)
        add_credits(g.sig_credits, g.sig_first, g.sig_count);
    direct_tile_body<StreamMem, VB, MODE1, kDirectBlock, kDirectUnroll>(
        g, direct_tile_3d<MODE1>(g, blockIdx.x, blockIdx.y, blockIdx.z), threadIdx.x);
}

// A whole chunked exchange in one launch (3-D grid of one plane's tiles,
// see ChunkedGeom): every workgroup moves its window tile through all B
// planes.
template <int VB, bool MODE1>
__global__ __launch_bounds__(kDirectBlock) void ua2a_chunked_kernel(DirectGeom g, ChunkedGeom c)
{
    args_up_front(g);
    asm volatile("" ::"s"(c.out), "s"(c.step), "s"(c.plane), "s"(c.planes));
    uint32_t block;
    const DirectTile d = chunked_tile<MODE1>(g, blockIdx.x, blockIdx.y, blockIdx.z, block);
    if (d.nvec == 0) return;                                  // padding tile of the grouped order
    if (d.nvec == ChunkedLane<VB>::kVecs * kDirectBlock)      // the same for the whole workgroup
        chunked_tile_body<StreamMem, VB, MODE1, kDirectBlock, true>(g, d, c, block, threadIdx.x);
    else
        chunked_tile_body<StreamMem, VB, MODE1, kDirectBlock, false>(g, d, c, block, threadIdx.x);
}

// The same on a flat grid capped below the tile count (a `blocks` hint):
// workgroup b moves tiles b, b + gridDim.x, ... each through all B planes.
template <int VB, bool MODE1>
__global__ __launch_bounds__(kDirectBlock) void ua2a_chunked_flat_kernel(DirectGeom g, ChunkedGeom c)
{
    flat_args_up_front(g);
    asm volatile("" ::"s"(c.out), "s"(c.step), "s"(c.plane), "s"(c.planes));
    for (uint64_t t = blockIdx.x; t < g.num_tiles; t += gridDim.x) {
        uint32_t slab;
        const DirectTile d = direct_tile<MODE1>(g, static_cast<uint32_t>(t), &slab);
        if (d.nvec == 0) continue;                                // padding tile of the grouped order
        const uint32_t block = chunked_block<MODE1>(g, slab);
        if (d.nvec == ChunkedLane<VB>::kVecs * kDirectBlock)
            chunked_tile_body<StreamMem, VB, MODE1, kDirectBlock, true>(g, d, c, block, threadIdx.x);
        else
            chunked_tile_body<StreamMem, VB, MODE1, kDirectBlock, false>(g, d, c, block, threadIdx.x);
    }
}

// The credits of a publishing exchange's last part.
__global__ __launch_bounds__(kWaitBlock) void ua2a_signal_kernel(SignalGeom g)
{
    add_credits(g.credits, g.first, g.count);
}

// Wait for readiness credits (see WaitGeom): each lane polls its counters,
// sleeping briefly between polls, and gives up after spin_limit polls of one
// counter.  The kernel always ends.
__global__ __launch_bounds__(kWaitBlock) void ua2a_wait_kernel(WaitGeom g)
{
    bool ok = true;
    for (uint64_t i = threadIdx.x; i < g.count && ok; i += kWaitBlock) {
        const uint32_t* c = g.credits + g.first + i;
        uint32_t polls = 1;
        while (!credit_reached(__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT),
                               g.target)) {
            if (polls++ >= g.spin_limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
    }
    if (!ok) __hip_atomic_store(g.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, bool MODE1, class Bases>
__device__ __forceinline__ void lds_tiles(const LdsGeom& g, const Bases& bases)
{
    extern __shared__ u32x4 ua2a_lds_raw[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(ua2a_lds_raw);
    for (uint64_t slot = blockIdx.x; slot < g.num_slots; slot += gridDim.x) {
        const uint32_t t = lds_slot_tile(g, static_cast<uint32_t>(slot));
        if (t >= g.num_tiles) continue;      // the same for the whole workgroup
        const LdsTile d = lds_tile(g, bases, t);
        // two loads in flight per lane pay off only with 16-byte pieces (measured)
        lds_fill<StreamMem, G, MODE1, kLdsBlock, (G == 16 ? kLdsUnroll : 1)>(g, bases, d, threadIdx.x, lds);
        __syncthreads();
        lds_drain<StreamMem, G, MODE1, kLdsBlock>(g, bases, d, threadIdx.x, lds);
        __syncthreads();   // the next tile overwrites the LDS image
    }
}

template <int G, bool MODE1>
__global__ __launch_bounds__(kLdsBlock) void ua2a_lds_kernel(LdsGeom g)
{
    args_up_front(g);
    lds_tiles<G, MODE1>(g, StackedBases{g});
}

// The same over per-rank allocations (pointer tables); the A table, read
// per lane, is staged in LDS once per workgroup.
template <int G, bool MODE1>
__global__ __launch_bounds__(kLdsBlock) void ua2a_lds_ranks_kernel(LdsGeom g, LdsTables tab)
{
    __shared__ uint8_t* a_tab[kMaxRankTable];
    for (uint32_t i = threadIdx.x; i < g.w; i += kLdsBlock) a_tab[i] = tab.a[i];
    __syncthreads();
    lds_tiles<G, MODE1>(g, StagedTableBases{tab, a_tab});
}

// A whole chunked exchange in one launch on the LDS path (see LdsChunkGeom):
// each workgroup keeps its tile through all B planes, `stage` planes at a
// time -- fill one LDS image per plane, then every lane, plane after plane,
// stores its chunks of the tile's window spans into the window and reads
// them back, and stores them to that plane of the output.  A lane reads back
// only window bytes that it stored, so the window needs no barrier; the
// barrier after the drain keeps the next stage's fill from overwriting LDS
// that a lane still reads.
template <int G, bool MODE1>
__global__ __launch_bounds__(kLdsBlock) void ua2a_lds_chunked_kernel(LdsGeom g, LdsChunkGeom c)
{
    args_up_front(g);
    asm volatile("" ::"s"(c.out), "s"(c.rank_step), "s"(c.plane), "s"(c.planes), "s"(c.stage), "s"(c.image));
    extern __shared__ u32x4 ua2a_lds_raw[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(ua2a_lds_raw);
    // planes per stage: at least one, at most what the bodies hold
    const uint32_t per = c.stage == 0 ? 1u : umin32(c.stage, kLdsChunkStage);
    for (uint64_t slot = blockIdx.x; slot < g.num_slots; slot += gridDim.x) {
        const uint32_t t = lds_slot_tile(g, static_cast<uint32_t>(slot));
        if (t >= g.num_tiles) continue;      // the same for the whole workgroup
        for (uint32_t p0 = 0, n = 0; p0 < c.planes; p0 += n) {
            n = umin32(per, c.planes - p0);
            lds_chunked_fill<StreamMem, G, MODE1, kLdsBlock, (G == 16 ? kLdsUnroll : 1), kLdsChunkStage>(
                g, c, t, p0, n, threadIdx.x, lds);
            __syncthreads();
            lds_chunked_drain<StreamMem, G, MODE1, kLdsBlock, kLdsReadback, kLdsChunkStage>(g, c, t, p0, n,
                                                                                    threadIdx.x, lds);
            __syncthreads();   // the next stage's fill overwrites the LDS images
        }
    }
}

// Per-rank allocations (pointer tables, sender range): one tile per
// workgroup when the grid covers the slab grid, else each dimension loops.
template <int VB, bool MODE1, bool TWO, bool PART>
__global__ __launch_bounds__(kDirectBlock) void ua2a_ranks_kernel(RanksGeom g)
{
    args_up_front(g);
    for (uint32_t z = blockIdx.z; z < g.nz; z += gridDim.z)
        for (uint32_t y = blockIdx.y; y < g.ny; y += gridDim.y)
            for (uint32_t x = blockIdx.x; x < g.tiles_per_slab; x += gridDim.x)
                ranks_tile_body<StreamMem, VB, MODE1, TWO, PART, kDirectBlock>(
                    g, ranks_tile<MODE1, TWO>(g, x, y, z), threadIdx.x);
}

// Pack, mode 1: contiguous blocks from the senders' tensors into the
// receivers' windows, one tile per workgroup when the grid covers the slab
// grid, else each dimension loops.
template <int VB>
__global__ __launch_bounds__(kDirectBlock) void ua2a_pack_kernel(PackGeom g)
{
    args_up_front(g);
    for (uint32_t z = blockIdx.z; z < g.nz; z += gridDim.z)
        for (uint32_t y = blockIdx.y; y < g.ny; y += gridDim.y)
            for (uint32_t x = blockIdx.x; x < g.tiles_per_block; x += gridDim.x)
                pack_tile_body<StreamMem, VB, kDirectBlock>(pack_tile<VB>(g, x, y, z), threadIdx.x);
}

template <int VB>
__global__ __launch_bounds__(kCopyBlock) void ua2a_copy_kernel(CopyGeom g)
{
    args_up_front(g);
    for (uint64_t t = blockIdx.x; t < g.num_tiles; t += gridDim.x)
        copy_tile_body<StreamMem, VB, kCopyBlock, kDirectUnroll>(g, static_cast<uint32_t>(t), threadIdx.x);
}

namespace {

template <bool MODE1, bool SIG>
const void* direct_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_direct_kernel<16, MODE1, SIG>);
    case 8: return reinterpret_cast<const void*>(&ua2a_direct_kernel<8, MODE1, SIG>);
    case 4: return reinterpret_cast<const void*>(&ua2a_direct_kernel<4, MODE1, SIG>);
    case 2: return reinterpret_cast<const void*>(&ua2a_direct_kernel<2, MODE1, SIG>);
    case 1: return reinterpret_cast<const void*>(&ua2a_direct_kernel<1, MODE1, SIG>);
    default: return nullptr;
    }
}

template <bool MODE1, bool SIG>
const void* direct3d_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_direct3d_kernel<16, MODE1, SIG>);
    case 8: return reinterpret_cast<const void*>(&ua2a_direct3d_kernel<8, MODE1, SIG>);
    case 4: return reinterpret_cast<const void*>(&ua2a_direct3d_kernel<4, MODE1, SIG>);
    case 2: return reinterpret_cast<const void*>(&ua2a_direct3d_kernel<2, MODE1, SIG>);
    case 1: return reinterpret_cast<const void*>(&ua2a_direct3d_kernel<1, MODE1, SIG>);
    default: return nullptr;
    }
}

template <bool MODE1>
const void* chunked_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_chunked_kernel<16, MODE1>);
    case 8: return reinterpret_cast<const void*>(&ua2a_chunked_kernel<8, MODE1>);
    case 4: return reinterpret_cast<const void*>(&ua2a_chunked_kernel<4, MODE1>);
    case 2: return reinterpret_cast<const void*>(&ua2a_chunked_kernel<2, MODE1>);
    case 1: return reinterpret_cast<const void*>(&ua2a_chunked_kernel<1, MODE1>);
    default: return nullptr;
    }
}

template <bool SIG>
const void* direct_any(const Launch& L)
{
    if (L.grid3d) return L.mode ? direct3d_fn<true, SIG>(L.width) : direct3d_fn<false, SIG>(L.width);
    return L.mode ? direct_fn<true, SIG>(L.width) : direct_fn<false, SIG>(L.width);
}

template <bool MODE1>
const void* lds_fn(int g)
{
    switch (g) {
    case 16: return reinterpret_cast<const void*>(&ua2a_lds_kernel<16, MODE1>);
    case 8: return reinterpret_cast<const void*>(&ua2a_lds_kernel<8, MODE1>);
    case 4: return reinterpret_cast<const void*>(&ua2a_lds_kernel<4, MODE1>);
    case 2: return reinterpret_cast<const void*>(&ua2a_lds_kernel<2, MODE1>);
    case 1: return reinterpret_cast<const void*>(&ua2a_lds_kernel<1, MODE1>);
    default: return nullptr;
    }
}

template <bool MODE1>
const void* lds_ranks_fn(int g)
{
    switch (g) {
    case 16: return reinterpret_cast<const void*>(&ua2a_lds_ranks_kernel<16, MODE1>);
    case 8: return reinterpret_cast<const void*>(&ua2a_lds_ranks_kernel<8, MODE1>);
    case 4: return reinterpret_cast<const void*>(&ua2a_lds_ranks_kernel<4, MODE1>);
    case 2: return reinterpret_cast<const void*>(&ua2a_lds_ranks_kernel<2, MODE1>);
    case 1: return reinterpret_cast<const void*>(&ua2a_lds_ranks_kernel<1, MODE1>);
    default: return nullptr;
    }
}

template <bool MODE1, bool TWO, bool PART>
const void* ranks_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_ranks_kernel<16, MODE1, TWO, PART>);
    case 8: return reinterpret_cast<const void*>(&ua2a_ranks_kernel<8, MODE1, TWO, PART>);
    case 4: return reinterpret_cast<const void*>(&ua2a_ranks_kernel<4, MODE1, TWO, PART>);
    case 2: return reinterpret_cast<const void*>(&ua2a_ranks_kernel<2, MODE1, TWO, PART>);
    case 1: return reinterpret_cast<const void*>(&ua2a_ranks_kernel<1, MODE1, TWO, PART>);
    default: return nullptr;
    }
}

template <bool MODE1>
const void* chunked_flat_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_chunked_flat_kernel<16, MODE1>);
    case 8: return reinterpret_cast<const void*>(&ua2a_chunked_flat_kernel<8, MODE1>);
    case 4: return reinterpret_cast<const void*>(&ua2a_chunked_flat_kernel<4, MODE1>);
    case 2: return reinterpret_cast<const void*>(&ua2a_chunked_flat_kernel<2, MODE1>);
    case 1: return reinterpret_cast<const void*>(&ua2a_chunked_flat_kernel<1, MODE1>);
    default: return nullptr;
    }
}

template <bool MODE1>
const void* lds_chunked_fn(int g)
{
    switch (g) {
    case 16: return reinterpret_cast<const void*>(&ua2a_lds_chunked_kernel<16, MODE1>);
    case 8: return reinterpret_cast<const void*>(&ua2a_lds_chunked_kernel<8, MODE1>);
    case 4: return reinterpret_cast<const void*>(&ua2a_lds_chunked_kernel<4, MODE1>);
    case 2: return reinterpret_cast<const void*>(&ua2a_lds_chunked_kernel<2, MODE1>);
    case 1: return reinterpret_cast<const void*>(&ua2a_lds_chunked_kernel<1, MODE1>);
    default: return nullptr;
    }
}

const void* pack_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_pack_kernel<16>);
    case 8: return reinterpret_cast<const void*>(&ua2a_pack_kernel<8>);
    case 4: return reinterpret_cast<const void*>(&ua2a_pack_kernel<4>);
    case 2: return reinterpret_cast<const void*>(&ua2a_pack_kernel<2>);
    case 1: return reinterpret_cast<const void*>(&ua2a_pack_kernel<1>);
    default: return nullptr;
    }
}

const void* copy_fn(int vb)
{
    switch (vb) {
    case 16: return reinterpret_cast<const void*>(&ua2a_copy_kernel<16>);
    case 8: return reinterpret_cast<const void*>(&ua2a_copy_kernel<8>);
    case 4: return reinterpret_cast<const void*>(&ua2a_copy_kernel<4>);
    case 2: return reinterpret_cast<const void*>(&ua2a_copy_kernel<2>);
    case 1: return reinterpret_cast<const void*>(&ua2a_copy_kernel<1>);
    default: return nullptr;
    }
}

}  // namespace

// The window of ua2a_exchange_chunked_noalloc, for callers that cannot
// allocate: every device the library runs on holds its own copy for the life
// of the process.  In host code `scratch` names a host-side stand-in, not
// device memory, so the host passes kernels only the address that
// hipGetSymbolAddress reports for the current device, looked up once per
// device and kept.
static __device__ __align__(256) uint8_t scratch[UA2A_NOALLOC_WINDOW_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

int backend_scratch_window(int32_t device, uint8_t** window)
{
    if (device < 0 || device >= kMaxScratchDevices) return static_cast<int>(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return static_cast<int>(e);
        g_scratch_ptr[device] = static_cast<uint8_t*>(ptr);
    }
    *window = g_scratch_ptr[device];
    return 0;
}

int backend_current_device(int32_t* device)
{
    int d = -1;
    const hipError_t e = hipGetDevice(&d);
    if (e != hipSuccess) return static_cast<int>(e);
    *device = d;
    return 0;
}

const char* backend_error_name(int err) { return hipGetErrorName(static_cast<hipError_t>(err)); }

int backend_launch(const Launch& L, void* stream)
{
    const void* fn = nullptr;
    void* arg = nullptr;
    void* arg2 = nullptr;      // the second kernel argument, if any
    DirectGeom dg = L.direct;
    LdsGeom lg = L.lds;
    CopyGeom cg = L.copy;
    size_t shmem = 0;
    switch (L.kernel) {
    case Kernel::Direct:
        fn = L.direct.sig_count ? direct_any<true>(L) : direct_any<false>(L);
        arg = &dg;
        break;
    case Kernel::Chunked:
        if (L.direct.sig_count) return static_cast<int>(hipErrorInvalidValue);
        if (L.grid3d)
            fn = L.mode ? chunked_fn<true>(L.width) : chunked_fn<false>(L.width);
        else
            fn = L.mode ? chunked_flat_fn<true>(L.width) : chunked_flat_fn<false>(L.width);
        arg = &dg;
        arg2 = const_cast<ChunkedGeom*>(&L.chunk);
        break;
    case Kernel::Lds:
        fn = L.mode ? lds_fn<true>(L.width) : lds_fn<false>(L.width);
        arg = &lg;
        shmem = L.lds_bytes;
        break;
    case Kernel::LdsChunked:
        fn = L.mode ? lds_chunked_fn<true>(L.width) : lds_chunked_fn<false>(L.width);
        arg = &lg;
        arg2 = const_cast<LdsChunkGeom*>(&L.lds_chunk);
        shmem = L.lds_bytes;
        break;
    case Kernel::LdsRanks:
        fn = L.mode ? lds_ranks_fn<true>(L.width) : lds_ranks_fn<false>(L.width);
        arg = &lg;
        arg2 = const_cast<LdsTables*>(&L.lds_tab);
        shmem = L.lds_bytes;
        break;
    case Kernel::Copy:
        fn = copy_fn(L.width);
        arg = &cg;
        break;
    case Kernel::Pack:
        fn = pack_fn(L.width);
        arg = const_cast<PackGeom*>(&L.pack);
        break;
    case Kernel::Wait:
        fn = reinterpret_cast<const void*>(&ua2a_wait_kernel);
        arg = const_cast<WaitGeom*>(&L.wait);
        break;
    case Kernel::Signal:
        fn = reinterpret_cast<const void*>(&ua2a_signal_kernel);
        arg = const_cast<SignalGeom*>(&L.signal);
        break;
    case Kernel::Ranks:
        if (!L.mode)
            fn = ranks_fn<false, false, false>(L.width);
        else if (L.ranks.count == L.ranks.w)
            fn = L.ranks.two_runs ? ranks_fn<true, true, false>(L.width) : ranks_fn<true, false, false>(L.width);
        else
            fn = L.ranks.two_runs ? ranks_fn<true, true, true>(L.width) : ranks_fn<true, false, true>(L.width);
        arg = const_cast<RanksGeom*>(&L.ranks);
        break;
    }
    if (fn == nullptr) return static_cast<int>(hipErrorInvalidValue);
    void* args[] = {arg, arg2};
    const hipError_t e = hipLaunchKernel(fn, dim3(L.grid, L.grid_y, L.grid_z), dim3(L.block), args, shmem,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? 0 : static_cast<int>(e);
}

}  // namespace ua2a

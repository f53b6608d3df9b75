// Per-thread bodies of the exchange kernels.
//
// Each __global__ kernel in ua2a_kernels.hip is a thin loop over its tiles
// that calls one of these bodies with (tile, threadIdx.x); the LDS kernel
// calls lds_fill, a workgroup barrier, then lds_drain.  Because the bodies
// are __host__ __device__, a host emulation can run exactly this code for
// every (tile, thread) -- fill for all threads before drain for all threads
// -- and check it on a machine without a GPU.
#pragma once

#include "ua2a_geometry.h"

namespace ua2a {

// Global-memory access policy of the bodies.  The kernels use one that
// marks accesses non-temporal (streamed once, not worth keeping in cache);
// the host emulation uses PlainMem (with bounds checks of its own).
struct PlainMem {
    template <class T>
    UA2A_HD static T ld(const T* p) { return *p; }
    template <class T>
    UA2A_HD static void st(T* p, T v) { *p = v; }
    // Window accesses of the one-launch chunked exchange, and the order point
    // between a window store and the load that reads it back.
    template <class T>
    UA2A_HD static T ld_win(const T* p) { return *p; }
    template <class T>
    UA2A_HD static void st_win(T* p, T v) { *p = v; }
    UA2A_HD static void win_order() {}
    // The plane whose window accesses follow (the host emulation records
    // it with each window byte's writer; nothing to do elsewhere).
    UA2A_HD static void win_plane(uint32_t) {}
    // A store at byte `off` of a tile's written range [base, base + nbytes).
    template <class T>
    UA2A_HD static void st_tile(uint8_t* base, uint32_t, uint32_t off, T v)
    {
        *reinterpret_cast<T*>(base + off) = v;
    }
    // A G-byte piece of a span's partial first or last chunk (plain stores
    // in every policy: lines written partly through a buffer range and
    // partly plainly measured slower).
    template <class T>
    UA2A_HD static void st_piece(T* p, T v) { *p = v; }
    // Bytes [lo, hi) of the aligned 16-byte chunk at p, the others zero: the
    // emulation reads nothing outside a span.  (The kernels read such a chunk
    // whole; see StreamMem.)
    UA2A_HD static u32x4 ld_part(const u32x4* p, uint32_t lo, uint32_t hi)
    {
        u32x4 v = {0u, 0u, 0u, 0u};
        uint8_t* to = reinterpret_cast<uint8_t*>(&v);
        const uint8_t* from = reinterpret_cast<const uint8_t*>(p);
        for (uint32_t x = lo; x < hi; ++x) to[x] = from[x];
        return v;
    }
};

// The G-byte piece at byte `off` (a multiple of G) of a chunk held in
// registers; bytes are little-endian within each 32-bit lane of the vector.
template <int G> struct PieceOf;
template <> struct PieceOf<16> {
    UA2A_HD static u32x4 get(u32x4 v, uint32_t) { return v; }
};
template <> struct PieceOf<8> {
    UA2A_HD static uint64_t get(u32x4 v, uint32_t off)
    {
        return off == 0 ? (static_cast<uint64_t>(v[1]) << 32) | v[0]
                        : (static_cast<uint64_t>(v[3]) << 32) | v[2];
    }
};
UA2A_HD uint32_t dword_of(u32x4 v, uint32_t off)
{
    const uint32_t d = off >> 2;
    return d == 0 ? v[0] : d == 1 ? v[1] : d == 2 ? v[2] : v[3];
}
template <> struct PieceOf<4> {
    UA2A_HD static uint32_t get(u32x4 v, uint32_t off) { return dword_of(v, off); }
};
template <> struct PieceOf<2> {
    UA2A_HD static uint16_t get(u32x4 v, uint32_t off)
    {
        return static_cast<uint16_t>(dword_of(v, off) >> ((off & 2u) * 8u));
    }
};
template <> struct PieceOf<1> {
    UA2A_HD static uint8_t get(u32x4 v, uint32_t off)
    {
        return static_cast<uint8_t>(dword_of(v, off) >> ((off & 3u) * 8u));
    }
};

// The in-chunk byte range of the span [head, head + len) in the chunk at lo.
UA2A_HD uint32_t part_lo(uint32_t lo, uint32_t head) { return umax32(lo, head) - lo; }
UA2A_HD uint32_t part_hi(uint32_t lo, uint32_t head, uint32_t len) { return umin32(lo + 16, head + len) - lo; }

// Direct path: the BS lanes move whole VB-byte vectors of the tile; U
// vectors per lane are loaded before any is stored.
template <class Mem, int VB, bool MODE1, uint32_t BS, uint32_t U>
UA2A_HD void direct_tile_body(const DirectGeom& g, const DirectTile& d, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    // the tile writes one contiguous range of the written side: its nvec
    // vectors from d.dst_slab + d.u0 on
    const int64_t first = d.dst_slab + d.u0;
    uint8_t* const tile = g.dst + first * VB;
    const uint32_t tile_bytes = d.nvec * VB;
    for (uint32_t base = tid; base < d.nvec; base += BS * U) {
        T v[U];
        int64_t to[U];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k) {
            const uint32_t delta = base + k * BS;
            if (delta < d.nvec) {
                int64_t from;
                direct_vector<MODE1>(g, d, d.u0 + delta, from, to[k]);
                v[k] = Mem::ld(src + from);
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * BS < d.nvec)
                Mem::st_tile(tile, tile_bytes, static_cast<uint32_t>((to[k] - first) * VB), v[k]);
    }
}

// N full tiles of a capped flat grid at once: every lane loads its vectors
// of all N tiles before it stores any, so a workgroup that loops over several
// tiles keeps N tiles' loads in flight instead of one.  A full tile (16 * BS
// bytes) gives each lane exactly 16 / VB vectors, so no lane needs a bounds
// test (per-lane tests would split the body into masked blocks, across which
// the compiler waits for each load before going on).
template <class Mem, int VB, bool MODE1, uint32_t BS, uint32_t N>
UA2A_HD void direct_full_tiles_body(const DirectGeom& g, const DirectTile* d, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    constexpr uint32_t K = 16 / VB;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    T v[N][K];
    int64_t to[N][K];
#pragma unroll
    for (uint32_t i = 0; i < N; ++i)
#pragma unroll
        for (uint32_t k = 0; k < K; ++k) {
            int64_t from;
            direct_vector<MODE1>(g, d[i], d[i].u0 + tid + k * BS, from, to[i][k]);
            v[i][k] = Mem::ld(src + from);
        }
#pragma unroll
    for (uint32_t i = 0; i < N; ++i) {
        const int64_t first = d[i].dst_slab + d[i].u0;
#pragma unroll
        for (uint32_t k = 0; k < K; ++k)
            Mem::st_tile(g.dst + first * VB, 16 * BS, static_cast<uint32_t>((to[i][k] - first) * VB), v[i][k]);
    }
}

// Chunked exchange in one launch (see ChunkedGeom): the tile's window range
// is written and read back plane after plane by the lanes that own it.  A
// tile is 16 * BS bytes, so a lane owns K = 16 / VB window vectors,
// lane + k * BS, and moves them for U planes at a time: it loads the U
// planes' input vectors, then for each plane in order stores its vectors
// into the window and loads them back, then stores what it read to that
// plane of the output.  The window vectors a lane touches are its own for
// the whole launch, so the only ordering the window needs is that of one
// lane's accesses to one address, which the hardware keeps in program order
// (a later plane's store cannot overtake an earlier plane's load of the same
// vector, and a load sees the same lane's earlier store).  Mem::win_order()
// keeps the compiler from forwarding a stored vector to the load that reads
// it back, so every output byte really is read from the window.  Window
// accesses go through Mem::ld_win / st_win (cached: the window is re-read
// within the launch); input and output stay streamed.
template <int VB>
struct ChunkedLane {
    static constexpr uint32_t kVecs = 16 / VB;                  // window vectors per lane
    static constexpr uint32_t kPlanes = kVecs >= 4 ? 1 : 4 / kVecs;   // planes in flight per lane
};

// N consecutive planes from p0 on, for the lane's K window vectors: the N
// planes' input loads first, then per plane its window store and read-back,
// then the output stores.  ok[k]: vector k lies in the tile.
template <class Mem, int VB, uint32_t BS, uint32_t K, uint32_t N>
UA2A_HD void chunked_planes(const ChunkedGeom& c, const typename Piece<VB>::T* src, const int64_t* from,
                            const bool* ok, typename Piece<VB>::T* win, int64_t out0, uint32_t tile_bytes,
                            uint32_t lane, uint32_t p0)
{
    typedef typename Piece<VB>::T T;
    T v[N][K];
#pragma unroll
    for (uint32_t i = 0; i < N; ++i)
#pragma unroll
        for (uint32_t k = 0; k < K; ++k)
            if (ok[k]) v[i][k] = Mem::ld(src + (p0 + i) * c.plane + from[k]);
#pragma unroll
    for (uint32_t i = 0; i < N; ++i) {
#pragma unroll
        for (uint32_t k = 0; k < K; ++k)
            if (ok[k]) Mem::st_win(win + lane + k * BS, v[i][k]);
        Mem::win_order();
#pragma unroll
        for (uint32_t k = 0; k < K; ++k)
            if (ok[k]) v[i][k] = Mem::ld_win(win + lane + k * BS);
    }
#pragma unroll
    for (uint32_t i = 0; i < N; ++i) {
        uint8_t* const tile = c.out + (out0 + (p0 + i) * c.plane) * VB;
#pragma unroll
        for (uint32_t k = 0; k < K; ++k)
            if (ok[k]) Mem::st_tile(tile, tile_bytes, (lane + k * BS) * VB, v[i][k]);
    }
}

// FULL: the tile holds K vectors for every lane (all but a slab's last
// tile), so no lane needs a bounds test, and the planes go U at a time (the
// rest one by one).  A partial tile moves one plane at a time: per-lane
// tests split the body into masked blocks, across which the compiler keeps
// fewer values in flight anyway.
template <class Mem, int VB, bool MODE1, uint32_t BS, bool FULL>
UA2A_HD void chunked_tile_body(const DirectGeom& g, const DirectTile& d, const ChunkedGeom& c, uint32_t z,
                               uint32_t lane)
{
    typedef typename Piece<VB>::T T;
    constexpr uint32_t K = ChunkedLane<VB>::kVecs;
    constexpr uint32_t U = ChunkedLane<VB>::kPlanes;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    T* const win = reinterpret_cast<T*>(g.dst) + d.dst_slab + d.u0;     // the tile's window range
    const int64_t out0 = d.dst_slab + d.u0 + static_cast<int64_t>(z) * c.step;   // its range in out[z][0]
    const uint32_t tile_bytes = d.nvec * VB;
    int64_t from[K];
    bool ok[K];
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) {
        from[k] = 0;
        ok[k] = FULL || lane + k * BS < d.nvec;
        if (ok[k]) {
            int64_t to;
            direct_vector<MODE1>(g, d, d.u0 + lane + k * BS, from[k], to);
        }
    }
    uint32_t p0 = 0;
    if (FULL)
        for (; p0 + U <= c.planes; p0 += U)
            chunked_planes<Mem, VB, BS, K, U>(c, src, from, ok, win, out0, tile_bytes, lane, p0);
    for (; p0 < c.planes; ++p0)
        chunked_planes<Mem, VB, BS, K, 1>(c, src, from, ok, win, out0, tile_bytes, lane, p0);
}

// Per-rank allocations: as direct_tile_body, the tensors taken from the
// geometry's pointer tables (per tile, or per vector in mode 1).
// PART: mode 1 with part of the senders (a kernel instance of its own, so the
// others keep the plain contiguous-range stores).
template <class Mem, int VB, bool MODE1, bool TWO, bool PART, uint32_t BS>
UA2A_HD void ranks_tile_body(const RanksGeom& g, const RanksTile& d, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    if (!PART) {
        // mode 0, and mode 1 when every rank sends: the tile writes one
        // contiguous range, from its first vector on
        const int64_t first = d.dst_off + d.u0;
        uint8_t* const tile = d.dst + first * VB;
        for (uint32_t delta = tid; delta < d.nvec; delta += BS) {
            const uint8_t* sp;
            int64_t from, to;
            ranks_vector<MODE1, TWO>(g, d, d.u0 + delta, sp, from, to);
            const T v = Mem::ld(reinterpret_cast<const T*>(sp) + from);
            Mem::st_tile(tile, d.nvec * VB, static_cast<uint32_t>((to - first) * VB), v);
        }
    } else {
        // mode 1 with part of the senders: pieces of consecutive rows, stored
        // through the range from the tile's first written vector to its last
        // while that spans less than 4 GiB, else plainly
        T* dst = reinterpret_cast<T*>(d.dst);
        const uint8_t* sp;
        int64_t from, first, last;
        ranks_vector<MODE1, TWO>(g, d, d.u0, sp, from, first);
        ranks_vector<MODE1, TWO>(g, d, d.u0 + d.nvec - 1, sp, from, last);
        const int64_t span = last - first + 1;
        const bool ranged = span * VB <= static_cast<int64_t>(UINT32_MAX);
        uint8_t* const tile = d.dst + first * VB;
        for (uint32_t delta = tid; delta < d.nvec; delta += BS) {
            int64_t to;
            ranks_vector<MODE1, TWO>(g, d, d.u0 + delta, sp, from, to);
            const T v = Mem::ld(reinterpret_cast<const T*>(sp) + from);
            if (ranged)
                Mem::st_tile(tile, static_cast<uint32_t>(span * VB), static_cast<uint32_t>((to - first) * VB), v);
            else
                Mem::st(dst + to, v);
        }
    }
}

// Pack, mode 1: one tile of a contiguous block, one vector per lane per pass.
template <class Mem, int VB, uint32_t BS>
UA2A_HD void pack_tile_body(const PackTile& t, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    const T* __restrict__ src = reinterpret_cast<const T*>(t.src) + t.u0;
    uint8_t* const tile = t.dst + static_cast<int64_t>(t.u0) * VB;
    for (uint32_t i = tid; i < t.nvec; i += BS) Mem::st_tile(tile, t.nvec * VB, i * VB, Mem::ld(src + i));
}

// A chunk that an A span covers only in part: its first or last chunk when
// the span starts or ends inside an aligned 16-byte chunk.  Mode 1's fill
// numbers them as slots, slot = 2 * r + end (end 0: first chunk, 1: last).
struct PartChunk {
    const u32x4* src;    // the aligned chunk in global memory
    uint32_t lo, hi;     // its in-span bytes
    uint32_t at;         // A-span byte of the chunk's first byte
    uint32_t r;          // head block
    bool valid;
};

template <class Bases>
UA2A_HD PartChunk a_part_chunk(const LdsGeom& g, const Bases& bases, const LdsTile& d, uint32_t slot)
{
    PartChunk pc;
    pc.valid = false;
    pc.src = nullptr;
    pc.lo = pc.hi = pc.at = pc.r = 0;
    const uint32_t r = slot >> 1, end = slot & 1u;
    if (r >= g.w) return pc;
    const uint8_t* aspan = bases.a_rank_base(r) + d.a_start0;
    const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
    const uint32_t n = span_chunks(ahead, d.a_len);
    if (n == 0 || (end == 1 && n == 1)) return pc;       // no chunk, or the first is also the last
    const uint32_t c = end ? n - 1 : 0;
    if (chunk_full(c * 16, ahead, d.a_len)) return pc;
    pc.valid = true;
    pc.src = reinterpret_cast<const u32x4*>(aspan - ahead + c * 16);
    pc.lo = part_lo(c * 16, ahead);
    pc.hi = part_hi(c * 16, ahead, d.a_len);
    pc.at = c * 16 - ahead;
    pc.r = r;
    return pc;
}

// Place the in-span pieces of a partial A-span chunk, held in registers, in LDS.
template <int G>
UA2A_HD void place_a_part_chunk(const LdsGeom& g, const LdsTile& d, const PartChunk& pc, u32x4 v,
                                uint8_t* lds)
{
    typedef typename Piece<G>::T T;
    for (uint32_t o = pc.lo; o < pc.hi; o += G)
        *reinterpret_cast<T*>(lds + lds_pos_of_a(g, d, pc.r, pc.at + o)) = PieceOf<G>::get(v, o);
}

// LDS path, first phase: global -> LDS image of the tile's P rows.
//   mode 0: the P span itself (contiguous 16-byte chunks);
//   mode 1: the w A spans, each read as contiguous chunks and scattered
//           into its runs' places in the image in G-byte pieces.
// Mode 1 reads its A spans' partial first and last chunks whole as well
// (one load each, not a chain of piece-sized loads, which stalled the wave
// at every tile of a span misaligned to 16 bytes): each lane loads the
// partial chunk of slot tid before the loop, so that load is in flight with
// the others, and places its pieces after it; slots beyond the workgroup
// (w > BS / 2) follow in a loop of their own.  The loop itself moves whole
// chunks only (a heavier loop body measured slower).  Mode 0 moves the P
// span's partial chunks piece by piece in its loop: a P span starts and ends
// on a row, so they occur only with a misaligned base, and every other form
// measured slower on aligned spans.
// With S > 1 (the one-launch chunked kernel) one call fills the images of n
// <= S batch planes: plane k's spans are the tile's moved by k * plane bytes,
// its image lies k * image bytes into LDS, and every plane's loads go out
// before any of their LDS stores.  The caller guarantees that plane is a
// multiple of 16 bytes when n > 1, so `d` (the tile as the first plane sees
// it) places every plane alike.
template <class Mem, int G, bool MODE1, uint32_t BS, uint32_t U, class Bases, uint32_t S = 1>
UA2A_HD void lds_fill(const LdsGeom& g, const Bases& bases, const LdsTile& d, uint32_t tid,
                      uint8_t* lds, int64_t plane = 0, uint32_t image = 0, uint32_t n = 1)
{
    if (!MODE1) {
        const uint8_t* pchunk0 = d.p_span - d.head;   // 16-aligned
        const uint32_t pch = span_chunks(d.head, d.p_len);
        for (uint32_t c0 = tid; c0 < pch; c0 += BS * U) {
            u32x4 v[S][U] = {};
#pragma unroll
            for (uint32_t k = 0; k < S; ++k) {
                if (k >= n) break;
#pragma unroll
                for (uint32_t u = 0; u < U; ++u) {
                    const uint32_t c = c0 + u * BS;
                    if (c < pch && chunk_full(c * 16, d.head, d.p_len))
                        v[k][u] = Mem::ld(reinterpret_cast<const u32x4*>(pchunk0 + k * plane + c * 16));
                }
            }
#pragma unroll
            for (uint32_t k = 0; k < S; ++k) {
                if (k >= n) break;
                uint8_t* const img = lds + k * image;
#pragma unroll
                for (uint32_t u = 0; u < U; ++u) {
                    const uint32_t c = c0 + u * BS;
                    if (c >= pch) continue;
                    if (chunk_full(c * 16, d.head, d.p_len))
                        *reinterpret_cast<u32x4*>(img + lds_pos_of_p(g, c * 16)) = v[k][u];
                    else
                        copy_partial_chunk<G>(pchunk0 + k * plane, img, c * 16, d.head, d.p_len);
                }
            }
        }
    } else {
        // with G = 16 every A span is 16-aligned and has no partial chunk
        const PartChunk pc = G < 16 ? a_part_chunk(g, bases, d, tid) : PartChunk{};
        u32x4 pv[S] = {};
#pragma unroll
        for (uint32_t k = 0; k < S; ++k) {
            if (k >= n) break;
            if (G < 16 && pc.valid)
                pv[k] = Mem::ld_part(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(pc.src) + k * plane),
                                     pc.lo, pc.hi);
        }
        // the w spans' chunks as one flat index space, so every lane has work
        // even when one span is shorter than the workgroup; neighbouring lanes
        // take neighbouring chunks of one span (measured faster than putting
        // the head block fastest, which spreads a wave over w regions)
        const uint32_t stride = d.stride;      // chunk slots of the longest span
        const uint32_t total = g.w * stride;
        for (uint32_t i0 = tid; i0 < total; i0 += BS * U) {
            u32x4 v[S][U] = {};
#pragma unroll
            for (uint32_t k = 0; k < S; ++k) {
                if (k >= n) break;
#pragma unroll
                for (uint32_t u = 0; u < U; ++u) {
                    const uint32_t i = i0 + u * BS;
                    if (i >= total) continue;
                    const uint32_t r = fdiv(i, d.d_stride);
                    const uint32_t c = i - r * stride;
                    const uint8_t* aspan = bases.a_rank_base(r) + d.a_start0;
                    const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
                    if (c < span_chunks(ahead, d.a_len) && chunk_full(c * 16, ahead, d.a_len))
                        v[k][u] = Mem::ld(reinterpret_cast<const u32x4*>(aspan - ahead + k * plane + c * 16));
                }
            }
#pragma unroll
            for (uint32_t k = 0; k < S; ++k) {
                if (k >= n) break;
                uint8_t* const img = lds + k * image;
#pragma unroll
                for (uint32_t u = 0; u < U; ++u) {
                    const uint32_t i = i0 + u * BS;
                    if (i >= total) continue;
                    const uint32_t r = fdiv(i, d.d_stride);
                    const uint32_t c = i - r * stride;
                    const uint8_t* aspan = bases.a_rank_base(r) + d.a_start0;
                    const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
                    if (c < span_chunks(ahead, d.a_len) && chunk_full(c * 16, ahead, d.a_len))
                        scatter_a_chunk<G>(g, d, r, c * 16 - ahead, v[k][u], img);
                }
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < S; ++k) {
            if (k >= n) break;
            if (G < 16 && pc.valid) place_a_part_chunk<G>(g, d, pc, pv[k], lds + k * image);
        }
        for (uint32_t slot = tid + BS; G < 16 && slot < 2 * g.w; slot += BS) {
            const PartChunk more = a_part_chunk(g, bases, d, slot);
            if (!more.valid) continue;
            for (uint32_t k = 0; k < n; ++k)
                place_a_part_chunk<G>(g, d, more,
                                      Mem::ld_part(reinterpret_cast<const u32x4*>(
                                                       reinterpret_cast<const uint8_t*>(more.src) + k * plane),
                                                   more.lo, more.hi),
                                      lds + k * image);
        }
    }
}

// LDS path, second phase (after a workgroup barrier): LDS image -> global.
//   mode 0: each of the w A spans, gathered from the image, written as
//           contiguous 16-byte chunks;
//   mode 1: the P span, copied out of the image as contiguous chunks.
template <class Mem, int G, bool MODE1, uint32_t BS, class Bases>
UA2A_HD void lds_drain(const LdsGeom& g, const Bases& bases, const LdsTile& d, uint32_t tid,
                       const uint8_t* lds)
{
    if (!MODE1) {
        // the w spans' chunks as one flat index space (see lds_fill)
        const uint32_t stride = d.stride;
        const uint32_t total = g.w * stride;
        // Rank-stacked tensors whose tile spans are all 16-aligned and whole
        // chunks (always with 16-byte pieces; with 4- and 8-byte pieces when
        // the A base, rank stride, tile start and span length allow): with
        // a_window, one range from head block 0's span holds all w spans of
        // the tile, and the chunks are stored through it.  Otherwise (per-rank
        // tables, spans with partial chunks, which are written plainly --
        // lines written both ways measured 9-52 % slower -- and 1- or 2-byte
        // pieces, whose whole-chunk spans measured 3-9 % slower this way)
        // plain stores.  Measured with whole-chunk spans: 60-byte runs
        // +2.4 %, 24-byte runs +1.5 %.
        bool whole = false;
        if constexpr (Bases::kStacked)
            whole = G == 16 ||
                    (G >= 4 && g.a_whole16 && ((d.a_start0 | static_cast<int64_t>(d.a_len)) & 15) == 0);
        if (whole) {
            uint8_t* const win = g.a_ptr + d.a_start0;      // 16-aligned
            const uint32_t win_bytes = g.a_window
                ? static_cast<uint32_t>(static_cast<int64_t>(g.w - 1) * g.a_rank + d.a_len + 32) : 0u;
            for (uint32_t i = tid; i < total; i += BS) {
                const uint32_t r = fdiv(i, d.d_stride);
                const uint32_t c = i - r * stride;
                uint8_t* const p = bases.a_rank_base(r) + d.a_start0 + c * 16;
                if (c * 16 >= d.a_len) continue;
                const u32x4 v = gather_a_chunk<G>(g, d, r, c * 16, lds);
                if (g.a_window)
                    Mem::st_tile(win, win_bytes, static_cast<uint32_t>(p - win), v);
                else
                    Mem::st(reinterpret_cast<u32x4*>(p), v);
            }
        } else {
            for (uint32_t i = tid; i < total; i += BS) {
                const uint32_t r = fdiv(i, d.d_stride);
                const uint32_t c = i - r * stride;
                uint8_t* aspan = bases.a_rank_base(r) + d.a_start0;
                const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
                if (c >= span_chunks(ahead, d.a_len)) continue;
                const uint32_t lo = c * 16;
                if (chunk_full(lo, ahead, d.a_len))
                    Mem::st(reinterpret_cast<u32x4*>(aspan - ahead + lo), gather_a_chunk<G>(g, d, r, lo - ahead, lds));
                else
                    a_partial_from_lds<Mem, G>(g, d, r, lo, ahead, lds, aspan - ahead);
            }
        }
    } else {
        uint8_t* pchunk0 = d.p_span - d.head;
        const uint32_t pch = span_chunks(d.head, d.p_len);
        for (uint32_t c = tid; c < pch; c += BS) {
            const uint32_t lo = c * 16;
            if (chunk_full(lo, d.head, d.p_len))     // the P span: one contiguous range per tile
                Mem::st_tile(pchunk0, pch * 16, lo, *reinterpret_cast<const u32x4*>(lds + lds_pos_of_p(g, lo)));
            else
                p_partial_from_lds<Mem, G>(lds, pchunk0, lo, d.head, d.p_len);
        }
    }
}

// A 16-byte chunk held in registers, stored at `to` (G-aligned): one 16-byte
// store when `to` is 16-aligned, else its G-byte pieces.
template <class Mem, int G>
UA2A_HD void st_chunk(uint8_t* to, u32x4 v)
{
    typedef typename Piece<G>::T T;
    if (G == 16 || (reinterpret_cast<uintptr_t>(to) & 15u) == 0) {
        Mem::st(reinterpret_cast<u32x4*>(to), v);
        return;
    }
#pragma unroll
    for (uint32_t o = 0; o < 16; o += G) Mem::st_piece(reinterpret_cast<T*>(to + o), PieceOf<G>::get(v, o));
}

// Mode 1 of lds_drain_through_window: the tile's P span, LDS images ->
// window (at wchunk0) -> output (at ochunk0 for the first plane, plane bytes
// further for each next one); OUT16: the output shares the window's 16-byte
// chunks, so whole chunks go out through the span's buffer range.
template <class Mem, int G, uint32_t BS, uint32_t U, uint32_t S, bool OUT16>
UA2A_HD void p_span_through_window(const LdsGeom& g, const LdsTile& d, const LdsChunkGeom& c, uint32_t p0,
                                   uint32_t n, uint32_t tid, const uint8_t* lds, uint8_t* wchunk0,
                                   uint8_t* ochunk0)
{
    typedef typename Piece<G>::T T;
    const uint32_t pch = span_chunks(d.head, d.p_len);
    for (uint32_t c0 = tid; c0 < pch; c0 += BS * U) {
        u32x4 v[S][U] = {};
        bool full[U];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            const uint32_t ci = c0 + u * BS;
            full[u] = ci < pch && chunk_full(ci * 16, d.head, d.p_len);
        }
#pragma unroll
        for (uint32_t k = 0; k < S; ++k) {
            if (k >= n) break;
            Mem::win_plane(p0 + k);
            const uint8_t* img = lds + k * c.image;
            uint8_t* const och = ochunk0 + static_cast<int64_t>(k) * c.plane;
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                const uint32_t ci = c0 + u * BS;
                const uint32_t lo = ci * 16;
                if (full[u]) {
                    Mem::st_win(reinterpret_cast<u32x4*>(wchunk0 + lo),
                                *reinterpret_cast<const u32x4*>(img + lds_pos_of_p(g, lo)));
                } else if (ci < pch) {
                    const uint32_t x1 = umin32(lo + 16, d.head + d.p_len);
                    for (uint32_t x = umax32(lo, d.head); x < x1; x += G) {
                        T* const wp = reinterpret_cast<T*>(wchunk0 + x);
                        Mem::st_win(wp, *reinterpret_cast<const T*>(img + x));
                        Mem::win_order();
                        Mem::st_piece(reinterpret_cast<T*>(och + x), Mem::ld_win(wp));
                    }
                }
            }
            Mem::win_order();
#pragma unroll
            for (uint32_t u = 0; u < U; ++u)
                if (full[u]) v[k][u] = Mem::ld_win(reinterpret_cast<const u32x4*>(wchunk0 + (c0 + u * BS) * 16));
        }
#pragma unroll
        for (uint32_t k = 0; k < S; ++k) {
            if (k >= n) break;
            uint8_t* const och = ochunk0 + static_cast<int64_t>(k) * c.plane;
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                if (!full[u]) continue;
                if (OUT16)
                    Mem::st_tile(och, pch * 16, (c0 + u * BS) * 16, v[k][u]);
                else
                    st_chunk<Mem, G>(och + (c0 + u * BS) * 16, v[k][u]);
            }
        }
    }
}

// One-launch chunked exchange on the LDS path, second phase for planes p0 ..
// p0 + n - 1 (after the workgroup barrier that follows their fills; image k
// of LDS, image bytes apart, holds plane p0 + k): LDS images -> the tile's
// window spans -> those planes of the output (see LdsChunkGeom).  Each lane
// takes U of its chunks of the spans at a time and, plane after plane,
// stores them into the window and reads them back, then stores what it read
// to the planes' output.  The same lane handles the same chunks in every
// plane, so a lane reads back only what it stored itself and the window
// needs no barrier; a later plane's store to a window chunk follows the
// earlier plane's load of it in the lane's program order, which the hardware
// keeps for accesses of one lane to one address.  Window chunks are aligned
// 16-byte chunks of the window, read back as 16-byte vectors; each goes to
// the output in one 16-byte store when the output lies at the same offset
// modulo 16 (the usual case), else in G-byte pieces (every offset between
// the two is a multiple of G).  A partial first or last chunk moves as its
// in-span G-byte pieces.  With n > 1 the host guarantees that a plane is a
// multiple of 16 bytes, so `d` (the tile as seen from plane p0) places every
// plane's image alike and the output's offset modulo 16 is the same in
// every plane.
//   mode 0: the w A spans (window block r = head block r), gathered from
//           the image as lds_drain does;
//   mode 1: the P span (window block j = the tile's rank), copied out of it.
template <class Mem, int G, bool MODE1, uint32_t BS, uint32_t U, uint32_t S, class Bases>
UA2A_HD void lds_drain_through_window(const LdsGeom& g, const Bases& bases, const LdsTile& d,
                                      const LdsChunkGeom& c, uint32_t p0, uint32_t n, uint32_t tid,
                                      const uint8_t* lds)
{
    typedef typename Piece<G>::T T;
    // window -> output, for block 0 of plane p0 (plus rank_step per block)
    const uintptr_t wbase = reinterpret_cast<uintptr_t>(MODE1 ? g.p_ptr : g.a_ptr);
    const int64_t shift = static_cast<int64_t>(reinterpret_cast<uintptr_t>(c.out) - wbase) +
                          static_cast<int64_t>(p0) * c.plane;
    if (!MODE1) {
        const uint32_t stride = d.stride;
        const uint32_t total = g.w * stride;
        for (uint32_t i0 = tid; i0 < total; i0 += BS * U) {
            u32x4 v[S][U] = {};
            uint8_t* wc[U];        // the chunk's 16-aligned window span base
            uint8_t* oc[U];        // ... and the output's, plane p0
            uint32_t rr[U], lo[U], ah[U];
            int kind[U];           // 0: no chunk, 1: whole chunk, 2: partial chunk
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                kind[u] = 0;
                wc[u] = oc[u] = nullptr;
                rr[u] = lo[u] = ah[u] = 0;
                const uint32_t i = i0 + u * BS;
                if (i >= total) continue;
                const uint32_t r = fdiv(i, d.d_stride);
                const uint32_t ci = i - r * stride;
                uint8_t* wspan = bases.a_rank_base(r) + d.a_start0;
                const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(wspan) & 15u);
                if (ci >= span_chunks(ahead, d.a_len)) continue;
                wc[u] = wspan - ahead;
                oc[u] = reinterpret_cast<uint8_t*>(
                    reinterpret_cast<uintptr_t>(wc[u]) + shift + static_cast<int64_t>(r) * c.rank_step);
                rr[u] = r;
                lo[u] = ci * 16;
                ah[u] = ahead;
                kind[u] = chunk_full(lo[u], ahead, d.a_len) ? 1 : 2;
            }
#pragma unroll
            for (uint32_t k = 0; k < S; ++k) {
                if (k >= n) break;
                Mem::win_plane(p0 + k);
                const uint8_t* img = lds + k * c.image;
                const int64_t pk = static_cast<int64_t>(k) * c.plane;
#pragma unroll
                for (uint32_t u = 0; u < U; ++u) {
                    if (kind[u] == 1) {
                        Mem::st_win(reinterpret_cast<u32x4*>(wc[u] + lo[u]),
                                    gather_a_chunk<G>(g, d, rr[u], lo[u] - ah[u], img));
                    } else if (kind[u] == 2) {
                        const uint32_t x1 = umin32(lo[u] + 16, ah[u] + d.a_len);
                        for (uint32_t x = umax32(lo[u], ah[u]); x < x1; x += G) {
                            T* const wp = reinterpret_cast<T*>(wc[u] + x);
                            Mem::st_win(wp, *reinterpret_cast<const T*>(img + lds_pos_of_a(g, d, rr[u], x - ah[u])));
                            Mem::win_order();
                            Mem::st_piece(reinterpret_cast<T*>(oc[u] + pk + x), Mem::ld_win(wp));
                        }
                    }
                }
                Mem::win_order();
#pragma unroll
                for (uint32_t u = 0; u < U; ++u)
                    if (kind[u] == 1) v[k][u] = Mem::ld_win(reinterpret_cast<const u32x4*>(wc[u] + lo[u]));
            }
#pragma unroll
            for (uint32_t k = 0; k < S; ++k) {
                if (k >= n) break;
                const int64_t pk = static_cast<int64_t>(k) * c.plane;
#pragma unroll
                for (uint32_t u = 0; u < U; ++u)
                    if (kind[u] == 1) st_chunk<Mem, G>(oc[u] + pk + lo[u], v[k][u]);
            }
        }
    } else {
        uint8_t* wchunk0 = d.p_span - d.head;
        uint8_t* ochunk0 = reinterpret_cast<uint8_t*>(
            reinterpret_cast<uintptr_t>(wchunk0) + shift + static_cast<int64_t>(d.j) * c.rank_step);
        // whether the output span's chunks line up with the window's (the
        // same for the whole tile and every plane of the stage; a loop of its
        // own for each case, since a per-store test measured 6-13 % slower)
        if (G == 16 || (reinterpret_cast<uintptr_t>(ochunk0) & 15u) == 0)
            p_span_through_window<Mem, G, BS, U, S, true>(g, d, c, p0, n, tid, lds, wchunk0, ochunk0);
        else
            p_span_through_window<Mem, G, BS, U, S, false>(g, d, c, p0, n, tid, lds, wchunk0, ochunk0);
    }
}

// The first phase of one stage of the LDS chunked kernel: the images of
// planes p0 .. p0 + n - 1 of tile t, image k at lds + k * image.  Every
// plane's loads go out before any of their LDS stores (one lds_fill over
// the n planes; with two planes of 16-byte pieces 10-18 % faster than one
// plane after the other), except for mode 1 with narrower pieces, whose
// scatter of pieces measured 1.5-3 % slower that way and fills one plane
// after the other.
template <class Mem, int G, bool MODE1, uint32_t BS, uint32_t U, uint32_t S>
UA2A_HD void lds_chunked_fill(const LdsGeom& g, const LdsChunkGeom& c, uint32_t t, uint32_t p0, uint32_t n,
                              uint32_t tid, uint8_t* lds)
{
    if (!MODE1 || G == 16) {
        const int64_t off = static_cast<int64_t>(p0) * c.plane;
        const PlaneBases bases{g, MODE1 ? 0 : off, MODE1 ? off : 0};     // the input side moves
        lds_fill<Mem, G, MODE1, BS, U, PlaneBases, S>(g, bases, lds_tile(g, bases, t), tid, lds, c.plane,
                                                      c.image, n);
    } else {
        for (uint32_t k = 0; k < n; ++k) {
            const PlaneBases bases{g, 0, static_cast<int64_t>(p0 + k) * c.plane};
            lds_fill<Mem, G, true, BS, U>(g, bases, lds_tile(g, bases, t), tid, lds + k * c.image);
        }
    }
}

// The second phase of one stage of the LDS chunked kernel: planes p0 ..
// p0 + n - 1 of tile t, whose images fill LDS (image bytes apart).  Mode 0
// drains them in one pass (each lane's chunks through the window plane after
// plane, then their output stores; U0 chunks per lane at a time, S >= n);
// mode 1 one plane after the other, one chunk per lane at a time (the
// one-pass form measured 2-6 % slower there, 2.5-6 % faster in mode 0).
template <class Mem, int G, bool MODE1, uint32_t BS, uint32_t U0, uint32_t S>
UA2A_HD void lds_chunked_drain(const LdsGeom& g, const LdsChunkGeom& c, uint32_t t, uint32_t p0, uint32_t n,
                               uint32_t tid, const uint8_t* lds)
{
    if (!MODE1) {
        const PlaneBases bases{g, static_cast<int64_t>(p0) * c.plane, 0};
        lds_drain_through_window<Mem, G, false, BS, U0, S>(
            g, bases, lds_tile(g, bases, t), c, p0, n, tid, lds);
    } else {
        const PlaneBases bases{g, 0, 0};     // the drain reads no input: the tile as plane 0 sees it
        const LdsTile d = lds_tile(g, bases, t);
        for (uint32_t k = 0; k < n; ++k)
            lds_drain_through_window<Mem, G, true, BS, 1, 1>(g, bases, d, c, p0 + k, 1, tid, lds + k * c.image);
    }
}

// Strided block copy (mode 0's unpack: a receiver's window -> its output).
template <class Mem, int VB, uint32_t BS, uint32_t U>
UA2A_HD void copy_tile_body(const CopyGeom& g, uint32_t t, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    const CopyTile c = copy_tile(g, t);
    uint8_t* const tile = g.dst + c.dst_base * VB;      // the tile's contiguous written range
    for (uint32_t base = tid; base < c.nvec; base += BS * U) {
        T v[U];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * BS < c.nvec) v[k] = Mem::ld(src + c.src_base + base + k * BS);
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * BS < c.nvec) Mem::st_tile(tile, c.nvec * VB, (base + k * BS) * VB, v[k]);
    }
}

}  // namespace ua2a

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
    // A store at byte `off` of a tile's written range [base, base + nbytes).
    template <class T>
    UA2A_HD static void st_tile(uint8_t* base, uint32_t, uint32_t off, T v)
    {
        *reinterpret_cast<T*>(base + off) = v;
    }
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

// A chunked plane after the first, on two waves of BS lanes: wave 0 moves
// the tile's window range (the previous plane) out to `carry_tile`, its range
// in the output; wave 1 writes the new plane into the window.  Each lane
// loads its vectors (direct_carry_load), the workgroup waits at a barrier
// until every load has returned, then each lane stores (direct_carry_store):
// no new vector can reach the window before the old one has been read.  A
// tile is 16 * BS bytes, so a lane holds 16 / VB vectors: lane + k * BS.
// `wave` is uniform across a wave, so each wave takes one side only.
template <int VB>
struct CarryVectors {
    static constexpr uint32_t kPerLane = 16 / VB;
    typename Piece<VB>::T v[kPerLane];
};

template <class Mem, int VB, bool MODE1, uint32_t BS>
UA2A_HD CarryVectors<VB> direct_carry_load(const DirectGeom& g, const DirectTile& d, uint32_t wave,
                                           uint32_t lane)
{
    typedef typename Piece<VB>::T T;
    CarryVectors<VB> c;
#pragma unroll
    for (uint32_t k = 0; k < CarryVectors<VB>::kPerLane; ++k) {
        const uint32_t delta = lane + k * BS;
        c.v[k] = T{};
        if (delta < d.nvec) {
            if (wave == 0) {
                c.v[k] = Mem::ld(reinterpret_cast<const T*>(g.dst) + d.dst_slab + d.u0 + delta);
            } else {
                int64_t from, to;
                direct_vector<MODE1>(g, d, d.u0 + delta, from, to);
                c.v[k] = Mem::ld(reinterpret_cast<const T*>(g.src) + from);
            }
        }
    }
    return c;
}

template <class Mem, int VB, bool MODE1, uint32_t BS>
UA2A_HD void direct_carry_store(const DirectGeom& g, const DirectTile& d, uint32_t wave, uint32_t lane,
                                uint8_t* carry_tile, const CarryVectors<VB>& c)
{
    // each wave's stores go through one range: the tile's place in the output
    // (wave 0) or in the window (wave 1), written in order of its vectors
    uint8_t* const base = wave == 0 ? carry_tile : g.dst + (d.dst_slab + d.u0) * VB;
#pragma unroll
    for (uint32_t k = 0; k < CarryVectors<VB>::kPerLane; ++k) {
        const uint32_t delta = lane + k * BS;
        if (delta < d.nvec) Mem::st_tile(base, d.nvec * VB, delta * VB, c.v[k]);
    }
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
template <class Mem, int G, bool MODE1, uint32_t BS, uint32_t U, class Bases>
UA2A_HD void lds_fill(const LdsGeom& g, const Bases& bases, const LdsTile& d, uint32_t tid,
                      uint8_t* lds)
{
    if (!MODE1) {
        const uint8_t* pchunk0 = d.p_span - d.head;   // 16-aligned
        const uint32_t pch = span_chunks(d.head, d.p_len);
        for (uint32_t c0 = tid; c0 < pch; c0 += BS * U) {
            u32x4 v[U] = {};
#pragma unroll
            for (uint32_t k = 0; k < U; ++k) {
                const uint32_t c = c0 + k * BS;
                if (c < pch && chunk_full(c * 16, d.head, d.p_len))
                    v[k] = Mem::ld(reinterpret_cast<const u32x4*>(pchunk0 + c * 16));
            }
#pragma unroll
            for (uint32_t k = 0; k < U; ++k) {
                const uint32_t c = c0 + k * BS;
                if (c >= pch) continue;
                if (chunk_full(c * 16, d.head, d.p_len))
                    *reinterpret_cast<u32x4*>(lds + lds_pos_of_p(g, c * 16)) = v[k];
                else
                    copy_partial_chunk<G>(pchunk0, lds, c * 16, d.head, d.p_len);
            }
        }
    } else {
        // with G = 16 every A span is 16-aligned and has no partial chunk
        const PartChunk pc = G < 16 ? a_part_chunk(g, bases, d, tid) : PartChunk{};
        u32x4 pv = {0u, 0u, 0u, 0u};
        if (G < 16 && pc.valid) pv = Mem::ld_part(pc.src, pc.lo, pc.hi);
        // the w spans' chunks as one flat index space, so every lane has work
        // even when one span is shorter than the workgroup; neighbouring lanes
        // take neighbouring chunks of one span (measured faster than putting
        // the head block fastest, which spreads a wave over w regions)
        const uint32_t stride = d.stride;      // chunk slots of the longest span
        const uint32_t total = g.w * stride;
        for (uint32_t i0 = tid; i0 < total; i0 += BS * U) {
            u32x4 v[U] = {};
#pragma unroll
            for (uint32_t k = 0; k < U; ++k) {
                const uint32_t i = i0 + k * BS;
                if (i >= total) continue;
                const uint32_t r = fdiv(i, d.d_stride);
                const uint32_t c = i - r * stride;
                const uint8_t* aspan = bases.a_rank_base(r) + d.a_start0;
                const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
                if (c < span_chunks(ahead, d.a_len) && chunk_full(c * 16, ahead, d.a_len))
                    v[k] = Mem::ld(reinterpret_cast<const u32x4*>(aspan - ahead + c * 16));
            }
#pragma unroll
            for (uint32_t k = 0; k < U; ++k) {
                const uint32_t i = i0 + k * BS;
                if (i >= total) continue;
                const uint32_t r = fdiv(i, d.d_stride);
                const uint32_t c = i - r * stride;
                const uint8_t* aspan = bases.a_rank_base(r) + d.a_start0;
                const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
                if (c < span_chunks(ahead, d.a_len) && chunk_full(c * 16, ahead, d.a_len))
                    scatter_a_chunk<G>(g, d, r, c * 16 - ahead, v[k], lds);
            }
        }
        if (G < 16 && pc.valid) place_a_part_chunk<G>(g, d, pc, pv, lds);
        for (uint32_t slot = tid + BS; G < 16 && slot < 2 * g.w; slot += BS) {
            const PartChunk more = a_part_chunk(g, bases, d, slot);
            if (more.valid)
                place_a_part_chunk<G>(g, d, more, Mem::ld_part(more.src, more.lo, more.hi), lds);
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
        if constexpr (Bases::kStacked && G == 16) {
            // rank-stacked tensors with 16-byte pieces: with a_window, one range
            // from head block 0's span holds all w spans of the tile, and the
            // chunks are stored through it.  (Per-rank tables keep plain
            // stores, and so do narrower pieces: their spans' partial chunks are
            // written plainly, and lines written both ways by neighbouring
            // chunks measured 9-52 % slower.)
            uint8_t* const win = g.a_ptr + d.a_start0;      // 16-aligned with G = 16
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
                    a_partial_from_lds<G>(g, d, r, lo, ahead, lds, aspan - ahead);
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
                copy_partial_chunk<G>(lds, pchunk0, lo, d.head, d.p_len);
        }
    }
}

// Strided block copy (chunked exchange: window -> planes of the output).
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

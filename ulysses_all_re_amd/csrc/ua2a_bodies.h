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
// the host emulation uses PlainMem.
struct PlainMem {
    template <class T>
    UA2A_HD static T ld(const T* p) { return *p; }
    template <class T>
    UA2A_HD static void st(T* p, T v) { *p = v; }
};

// Direct path: the BS lanes move whole VB-byte vectors of the tile; U
// vectors per lane are loaded before any is stored.
template <class Mem, int VB, bool MODE1, uint32_t BS, uint32_t U>
UA2A_HD void direct_tile_body(const DirectGeom& g, const DirectTile& d, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    T* __restrict__ dst = reinterpret_cast<T*>(g.dst);
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
            if (base + k * BS < d.nvec) Mem::st(dst + to[k], v[k]);
    }
}

// Per-rank allocations: as direct_tile_body, the tensors taken from the
// geometry's pointer tables (per tile, or per vector in mode 1).
template <class Mem, int VB, bool MODE1, bool TWO, uint32_t BS>
UA2A_HD void ranks_tile_body(const RanksGeom& g, const RanksTile& d, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    T* dst = reinterpret_cast<T*>(d.dst);
    for (uint32_t delta = tid; delta < d.nvec; delta += BS) {
        const uint8_t* sp;
        int64_t from, to;
        ranks_vector<MODE1, TWO>(g, d, d.u0 + delta, sp, from, to);
        Mem::st(dst + to, Mem::ld(reinterpret_cast<const T*>(sp) + from));
    }
}

// LDS path, first phase: global -> LDS image of the tile's P rows.
//   mode 0: the P span itself (contiguous 16-byte chunks);
//   mode 1: the w A spans, each read as contiguous chunks and scattered
//           into its runs' places in the image in G-byte pieces.
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
                if (c >= span_chunks(ahead, d.a_len)) continue;
                if (chunk_full(c * 16, ahead, d.a_len))
                    scatter_a_chunk<G>(g, d, r, c * 16 - ahead, v[k], lds);
                else
                    a_partial_to_lds<G>(g, d, r, c * 16, ahead, aspan - ahead, lds);
            }
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
    } else {
        uint8_t* pchunk0 = d.p_span - d.head;
        const uint32_t pch = span_chunks(d.head, d.p_len);
        for (uint32_t c = tid; c < pch; c += BS) {
            const uint32_t lo = c * 16;
            if (chunk_full(lo, d.head, d.p_len))
                Mem::st(reinterpret_cast<u32x4*>(pchunk0 + lo),
                        *reinterpret_cast<const u32x4*>(lds + lds_pos_of_p(g, lo)));
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
    T* __restrict__ dst = reinterpret_cast<T*>(g.dst);
    const CopyTile c = copy_tile(g, t);
    for (uint32_t base = tid; base < c.nvec; base += BS * U) {
        T v[U];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * BS < c.nvec) v[k] = Mem::ld(src + c.src_base + base + k * BS);
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * BS < c.nvec) Mem::st(dst + c.dst_base + base + k * BS, v[k]);
    }
}

}  // namespace ua2a

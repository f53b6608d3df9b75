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

// Direct path: lanes move whole VB-byte vectors; U vectors per lane are
// loaded before any is stored so each lane keeps U requests in flight.
template <int VB, bool MODE1, uint32_t U>
UA2A_HD void direct_tile_body(const DirectGeom& g, uint32_t t, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    T* __restrict__ dst = reinterpret_cast<T*>(g.dst);
    const DirectTile d = direct_tile(g, t);
    for (uint32_t base = tid; base < d.nvec; base += kBlock * U) {
        T v[U];
        int64_t to[U];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k) {
            const uint32_t delta = base + k * kBlock;
            if (delta < d.nvec) {
                int64_t a, p;
                direct_vector(g, d, delta, a, p);
                v[k] = src[MODE1 ? a : p];
                to[k] = MODE1 ? p : a;
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * kBlock < d.nvec) dst[to[k]] = v[k];
    }
}

// LDS path, first phase: global -> LDS image of the tile's P rows.
//   mode 0: the P span itself (contiguous 16-byte chunks);
//   mode 1: the w A spans, each read as contiguous chunks and scattered
//           into its runs' places in the image in G-byte pieces.
template <int G, bool MODE1, uint32_t U>
UA2A_HD void lds_fill(const LdsGeom& g, const LdsTile& d, uint32_t tid, uint8_t* lds)
{
    if (!MODE1) {
        const uint8_t* pchunk0 = g.p_ptr + d.p_start - d.head;   // 16-aligned
        const uint32_t pch = span_chunks(d.head, d.p_len);
        for (uint32_t c0 = tid; c0 < pch; c0 += kBlock * U) {
            u32x4 v[U];
#pragma unroll
            for (uint32_t k = 0; k < U; ++k) {
                const uint32_t c = c0 + k * kBlock;
                if (c < pch && chunk_full(c * 16, d.head, d.p_len))
                    v[k] = *reinterpret_cast<const u32x4*>(pchunk0 + c * 16);
            }
#pragma unroll
            for (uint32_t k = 0; k < U; ++k) {
                const uint32_t c = c0 + k * kBlock;
                if (c >= pch) continue;
                if (chunk_full(c * 16, d.head, d.p_len))
                    *reinterpret_cast<u32x4*>(lds + c * 16) = v[k];
                else
                    copy_partial_chunk<G>(pchunk0, lds, c * 16, d.head, d.p_len);
            }
        }
    } else {
        for (uint32_t r = 0; r < g.w; ++r) {
            const uint8_t* aspan = g.a_ptr + d.a_start0 + static_cast<int64_t>(r) * g.a_rank;
            const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
            const uint8_t* achunk0 = aspan - ahead;
            const uint32_t ach = span_chunks(ahead, d.a_len);
            for (uint32_t c0 = tid; c0 < ach; c0 += kBlock * U) {
                u32x4 v[U];
#pragma unroll
                for (uint32_t k = 0; k < U; ++k) {
                    const uint32_t c = c0 + k * kBlock;
                    if (c < ach && chunk_full(c * 16, ahead, d.a_len))
                        v[k] = *reinterpret_cast<const u32x4*>(achunk0 + c * 16);
                }
#pragma unroll
                for (uint32_t k = 0; k < U; ++k) {
                    const uint32_t c = c0 + k * kBlock;
                    if (c >= ach) continue;
                    if (chunk_full(c * 16, ahead, d.a_len))
                        scatter_a_chunk<G>(g, d, r, c * 16 - ahead, v[k], lds);
                    else
                        a_partial_to_lds<G>(g, d, r, c * 16, ahead, achunk0, lds);
                }
            }
        }
    }
}

// LDS path, second phase (after a workgroup barrier): LDS image -> global.
//   mode 0: each of the w A spans, gathered from the image, written as
//           contiguous 16-byte chunks;
//   mode 1: the P span, copied out of the image as contiguous chunks.
template <int G, bool MODE1>
UA2A_HD void lds_drain(const LdsGeom& g, const LdsTile& d, uint32_t tid, const uint8_t* lds)
{
    if (!MODE1) {
        for (uint32_t r = 0; r < g.w; ++r) {
            uint8_t* aspan = g.a_ptr + d.a_start0 + static_cast<int64_t>(r) * g.a_rank;
            const uint32_t ahead = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aspan) & 15u);
            uint8_t* achunk0 = aspan - ahead;
            const uint32_t ach = span_chunks(ahead, d.a_len);
            for (uint32_t c = tid; c < ach; c += kBlock) {
                const uint32_t lo = c * 16;
                if (chunk_full(lo, ahead, d.a_len))
                    *reinterpret_cast<u32x4*>(achunk0 + lo) = gather_a_chunk<G>(g, d, r, lo - ahead, lds);
                else
                    a_partial_from_lds<G>(g, d, r, lo, ahead, lds, achunk0);
            }
        }
    } else {
        uint8_t* pchunk0 = g.p_ptr + d.p_start - d.head;
        const uint32_t pch = span_chunks(d.head, d.p_len);
        for (uint32_t c = tid; c < pch; c += kBlock) {
            const uint32_t lo = c * 16;
            if (chunk_full(lo, d.head, d.p_len))
                *reinterpret_cast<u32x4*>(pchunk0 + lo) = *reinterpret_cast<const u32x4*>(lds + lo);
            else
                copy_partial_chunk<G>(lds, pchunk0, lo, d.head, d.p_len);
        }
    }
}

// Strided block copy (chunked exchange: window -> planes of the output).
template <int VB, uint32_t U>
UA2A_HD void copy_tile_body(const CopyGeom& g, uint32_t t, uint32_t tid)
{
    typedef typename Piece<VB>::T T;
    const T* __restrict__ src = reinterpret_cast<const T*>(g.src);
    T* __restrict__ dst = reinterpret_cast<T*>(g.dst);
    const CopyTile c = copy_tile(g, t);
    for (uint32_t base = tid; base < c.nvec; base += kBlock * U) {
        T v[U];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * kBlock < c.nvec) v[k] = src[c.src_base + base + k * kBlock];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k)
            if (base + k * kBlock < c.nvec) dst[c.dst_base + base + k * kBlock] = v[k];
    }
}

}  // namespace ua2a

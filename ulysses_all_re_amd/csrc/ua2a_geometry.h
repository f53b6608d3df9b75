// Index geometry of the Ulysses all_to_all_4D exchange kernels.
//
// The exchange (FastVideo "ulysses_a2a" API page, method run_armed) moves
// one "run" -- the H/w * D elements of one token in one head block -- at a
// time: a run is contiguous on both sides, so the whole permutation is a copy
// of runs between two layouts of the rank-stacked tensors:
//
//   P side ("head-complete", mode-0 input / mode-1 output)
//       [j = token owner][b][s][r = head block][run]
//   A side ("sequence-gathered", mode-0 output / mode-1 input)
//       [r = head block][b][j*S_local + s][run]
//
// Mode 0 copies P -> A, mode 1 copies A -> P.  Every offset below is built
// from explicit rank and plane strides, so the same kernels serve the
// unchunked exchange (dense strides over all B planes) and the chunked one
// (one plane of every rank, into or out of a one-plane window).
//
// Everything here is __host__ __device__ so the kernels and a host-side
// emulation of their index math (used by the tests to check bounds and
// parity on a machine with no GPU) evaluate the very same expressions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define UA2A_HD __host__ __device__ __forceinline__

namespace ua2a {

// Threads per workgroup.  Direct and copy kernels: one wave64 per
// workgroup (measured fastest on MI355X for these streams); LDS kernel: four
// waves sharing one LDS tile.
constexpr uint32_t kDirectBlock = 64;
constexpr uint32_t kCopyBlock = 64;
constexpr uint32_t kLdsBlock = 256;

// ------------------------------------------------------------------------
// Division of a 32-bit unsigned n by an invariant d >= 1 via a multiply-high
// and a shift (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up variant with an N+1-bit
// multiplier): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//     q = (mulhi32(n, m) + n) >> l   for every 0 <= n < 2^32.
// The sum is formed in 64 bits so it cannot overflow.
struct Div32 {
    uint32_t d;
    uint32_t m;
    uint32_t s;
};

inline Div32 make_div32(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return Div32{d, static_cast<uint32_t>(m), l};
}

UA2A_HD uint32_t fdiv(uint32_t n, Div32 f)
{
    const uint32_t hi = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> 32);
    return static_cast<uint32_t>((static_cast<uint64_t>(hi) + n) >> f.s);
}

UA2A_HD uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// ------------------------------------------------------------------------
// Direct path: each lane moves whole VB-byte vectors.  The work is cut along
// the side the exchange WRITES, so the stores of every workgroup form one
// contiguous stretch (on MI355X the write stream is what limits a copy; the
// reads then cover whole runs, each contiguous):
//   mode 0 writes the A side, slab = (r, b, j): s_local * vr vectors
//          contiguous; t = ((r * nb + b) * w + j) * tiles_per_slab + tt
//   mode 1 writes the P side, slab = (j, b): s_local * p_row vectors
//          contiguous; t = (j * nb + b) * tiles_per_slab + tt
// A tile is tile_vecs consecutive vectors of one slab (the last tile of a
// slab is short).  Units of every stride/offset: VB-byte vectors.
//
// Tile order.  By default tiles run slab after slab.  With group = F > 0
// (mode 0 only) they run in groups of F tiles, head block r fastest:
//     t = (((j * nb + b) * groups + hi) * w + r) * F + lo,  tt = hi * F + lo
// so the workgroups active at one time read whole P rows rather than one
// head-block column of them.  The host picks this when a P-side row is a
// multiple of 4 KiB, where reading one column of power-of-two-strided rows
// measured up to 20 % slower.  Padding tiles (tt >= tiles_per_slab) are
// empty.
struct DirectGeom {
    const uint8_t* src;        // mode 0: P side; mode 1: A side
    uint8_t* dst;              // the other side
    uint32_t* sig_credits;     // part of a publishing exchange: credits of the PREVIOUS
    uint32_t sig_first;        //   part, sig_credits[sig_first .. +sig_count) get 1 each
    uint32_t sig_count;        //   (0: none)
    int64_t a_rank, a_plane;   // A-side strides
    int64_t p_rank, p_plane;   // P-side strides
    uint32_t vr;               // vectors per run
    uint32_t p_row;            // w * vr: one token of all heads
    uint32_t s_local;          // tokens per rank
    uint32_t w, nb;            // ranks; planes covered by this launch
    uint32_t slab_vecs;        // vectors per slab (< 2^32, checked by the host)
    uint32_t tile_vecs;
    uint32_t tiles_per_slab;   // ceil(slab_vecs / tile_vecs)
    uint32_t num_tiles;        // slabs * tiles_per_slab (grouped: slabs * ceil(tps / F) * F)
    uint32_t group;            // 0: slab after slab; F > 0: groups of F tiles, r fastest
    uint32_t groups;           // ceil(tiles_per_slab / F)
    uint32_t cap_tiles;        // flat grid: tiles a workgroup loads before storing (1, or more
                               //   when a capped grid would keep too few tiles in flight)
    Div32 d_vr, d_prow, d_tps, d_w, d_nb, d_group, d_groups;
};

struct DirectTile {
    int64_t dst_slab;   // write-side offset of the slab's first vector
    int64_t src_slab;   // read-side offset that the per-vector terms are added to
    uint32_t u0;        // first vector of the tile within its slab
    uint32_t nvec;      // vectors in this tile
};

// Chunked exchange in one launch (direct path, 3-D grid of one plane's
// tiles; DirectGeom then describes plane 0 of every rank into the window).
// The window is [w][one plane] in the layout of the output side, and its
// block k is the z coordinate of the grid in both modes.  Each tile's window
// range belongs to one workgroup for the whole launch, and within it each
// window vector to one lane: for every plane p that lane stores plane p's
// vector into the window, reads it back, and stores it to out[k][p], so
// window vector x of block k lands at out + x + k * step + p * plane
// (vectors; out = plane 0 of rank 0, step = rank stride - plane).  The input
// of plane p is the plane-0 input moved by p * plane.
struct ChunkedGeom {
    uint8_t* out;
    int64_t step;       // rank stride minus one plane, in vectors
    int64_t plane;      // one plane of one rank, in vectors
    uint32_t planes;    // B
};

// (`slab_out`, if given, receives the tile's slab index.)
template <bool MODE1>
UA2A_HD DirectTile direct_tile(const DirectGeom& g, uint32_t t, uint32_t* slab_out = nullptr)
{
    uint32_t slab, tt;
    if (g.group == 0) {
        slab = fdiv(t, g.d_tps);
        tt = t - slab * g.tiles_per_slab;
    } else {
        const uint32_t grp = fdiv(t, g.d_group);
        const uint32_t lo = t - grp * g.group;
        const uint32_t q = fdiv(grp, g.d_w);
        const uint32_t r = grp - q * g.w;
        const uint32_t jb = fdiv(q, g.d_groups);
        const uint32_t hi = q - jb * g.groups;
        const uint32_t j = fdiv(jb, g.d_nb);
        const uint32_t b = jb - j * g.nb;
        slab = (r * g.nb + b) * g.w + j;          // the mode-0 slab numbering
        tt = hi * g.group + lo;
    }
    if (slab_out != nullptr) *slab_out = slab;
    DirectTile d;
    if (tt >= g.tiles_per_slab) {      // padding tile of the grouped order
        d.u0 = 0;
        d.nvec = 0;
        d.dst_slab = d.src_slab = 0;
        return d;
    }
    d.u0 = tt * g.tile_vecs;
    d.nvec = umin32(g.tile_vecs, g.slab_vecs - d.u0);
    if (!MODE1) {
        const uint32_t rb = fdiv(slab, g.d_w);
        const uint32_t j = slab - rb * g.w;
        const uint32_t r = fdiv(rb, g.d_nb);
        const uint32_t b = rb - r * g.nb;
        d.dst_slab = static_cast<int64_t>(r) * g.a_rank + static_cast<int64_t>(b) * g.a_plane +
                     static_cast<int64_t>(j) * g.s_local * g.vr;
        d.src_slab = static_cast<int64_t>(j) * g.p_rank + static_cast<int64_t>(b) * g.p_plane +
                     static_cast<int64_t>(r) * g.vr;
    } else {
        const uint32_t j = fdiv(slab, g.d_nb);
        const uint32_t b = slab - j * g.nb;
        d.dst_slab = static_cast<int64_t>(j) * g.p_rank + static_cast<int64_t>(b) * g.p_plane;
        d.src_slab = static_cast<int64_t>(b) * g.a_plane +
                     static_cast<int64_t>(j) * g.s_local * g.vr;
    }
    return d;
}

// The same tile on a 3-D grid, where the hardware supplies the coordinates
// (no scalar division per workgroup): x = tile within its slab,
//   mode 0: y = j, z = r * nb + b;      mode 1: y = b, z = j.
// Used for the default slab-after-slab order when the grid fits.
template <bool MODE1>
UA2A_HD DirectTile direct_tile_3d(const DirectGeom& g, uint32_t x, uint32_t y, uint32_t z)
{
    DirectTile d;
    d.u0 = x * g.tile_vecs;
    d.nvec = umin32(g.tile_vecs, g.slab_vecs - d.u0);
    if (!MODE1) {
        const uint32_t j = y;
        const uint32_t r = fdiv(z, g.d_nb);
        const uint32_t b = z - r * g.nb;
        d.dst_slab = static_cast<int64_t>(r) * g.a_rank + static_cast<int64_t>(b) * g.a_plane +
                     static_cast<int64_t>(j) * g.s_local * g.vr;
        d.src_slab = static_cast<int64_t>(j) * g.p_rank + static_cast<int64_t>(b) * g.p_plane +
                     static_cast<int64_t>(r) * g.vr;
    } else {
        const uint32_t b = y, j = z;
        d.dst_slab = static_cast<int64_t>(j) * g.p_rank + static_cast<int64_t>(b) * g.p_plane;
        d.src_slab = static_cast<int64_t>(b) * g.a_plane +
                     static_cast<int64_t>(j) * g.s_local * g.vr;
    }
    return d;
}

// The chunked kernel's tile on its 3-D grid, and the window block it feeds
// (mode 0: the head block r; mode 1: the receiving rank j).  The chunked
// kernel's geometry has one plane (nb = 1), so on a flat grid the block is
// the slab's r = slab / w (mode 0) or j = slab (mode 1): chunked_block.  With the
// grouped order (mode 0, g.group > 0) x runs over (tile group q, head block
// r, tile within the group), the group fastest, and y is the sending rank j;
// a padding tile of the last group has nvec = 0.  Otherwise the plain 3-D
// grid of direct_tile_3d.
template <bool MODE1>
UA2A_HD DirectTile chunked_tile(const DirectGeom& g, uint32_t x, uint32_t y, uint32_t z, uint32_t& block)
{
    if (!MODE1 && g.group != 0) {
        const uint32_t grp = fdiv(x, g.d_group);
        const uint32_t lo = x - grp * g.group;
        const uint32_t q = fdiv(grp, g.d_w);
        const uint32_t r = grp - q * g.w;
        const uint32_t tt = q * g.group + lo;
        block = r;
        if (tt >= g.tiles_per_slab) {
            DirectTile d;
            d.u0 = d.nvec = 0;
            d.dst_slab = d.src_slab = 0;
            return d;
        }
        return direct_tile_3d<false>(g, tt, y, r);
    }
    block = z;
    return direct_tile_3d<MODE1>(g, x, y, z);
}

template <bool MODE1>
UA2A_HD uint32_t chunked_block(const DirectGeom& g, uint32_t slab)
{
    return MODE1 ? slab : fdiv(slab, g.d_w);
}

// Read- and write-side offsets of vector u (< slab_vecs) of the tile's slab.
template <bool MODE1>
UA2A_HD void direct_vector(const DirectGeom& g, const DirectTile& d, uint32_t u,
                           int64_t& src_off, int64_t& dst_off)
{
    dst_off = d.dst_slab + u;
    if (!MODE1) {
        const uint32_t s = fdiv(u, g.d_vr);          // token of the sending rank
        const uint32_t o = u - s * g.vr;             // vector within the run
        src_off = d.src_slab + static_cast<int64_t>(static_cast<uint64_t>(s) * g.p_row) + o;
    } else {
        const uint32_t s = fdiv(u, g.d_prow);        // token of the receiving rank
        const uint32_t rem = u - s * g.p_row;
        const uint32_t r = fdiv(rem, g.d_vr);        // head block = rank that sent it
        const uint32_t o = rem - r * g.vr;
        src_off = d.src_slab + static_cast<int64_t>(r) * g.a_rank +
                  static_cast<int64_t>(static_cast<uint64_t>(s) * g.vr) + o;
    }
}

// ------------------------------------------------------------------------
// Per-rank allocations: the same exchange when every rank's tensor is an
// allocation of its own, reached through tables of base pointers, moving only
// the runs whose SENDING rank (mode 0: the token owner j, mode 1: the head
// block r) lies in [first, first + count).  With count = 1 this is what one
// device of a multi-device exchange pushes to its peers; with count = w it is
// the whole exchange.  Tiles are still cut along the written side:
//   mode 0: slab = (r, b, j = first + y): the s_local runs that j sends to r,
//           contiguous in out[r]; each run is read from row s of in[j];
//   mode 1: slab = (j, b): the rows of out[j], of which the launch writes the
//           seg = count * vr vectors of head blocks first .. first+count-1
//           (the whole row when count = w); each vector's run comes from the
//           sender's table entry.
// Slab grid: x = tile within the slab; mode 0: y = j - first, z = r * nb + b;
// mode 1: y = b, z = j.  Units: VB-byte vectors.
//
// Mode 1 reads each vector's run from its sender's tensor.  When every tile
// lies in at most two runs (one sender, or runs of at least a tile) the
// workgroup loads the two table entries once, with wave-uniform indices, and
// each lane picks one (TWO = true); otherwise each lane loads its own entry
// before its data.  The two forms are separate kernels: code that indexes the
// table both ways makes the compiler copy the whole kernel argument into
// per-lane scratch memory.
constexpr uint32_t kMaxRankTable = 64;     // table entries carried in the kernel argument

struct RanksGeom {
    const uint8_t* src[kMaxRankTable];   // per rank: base of the tensor read
    uint8_t* dst[kMaxRankTable];         // per rank: base of the tensor written
    int64_t a_plane, p_plane;            // one batch plane of one rank, each side
    uint32_t vr;                         // vectors per run
    uint32_t p_row;                      // w * vr
    uint32_t seg;                        // count * vr: vectors a mode-1 slab writes per token
    uint32_t s_local, w, nb, first, count;
    uint32_t slab_vecs, tile_vecs, tiles_per_slab;
    uint32_t ny, nz;                     // slab grid extents along y and z
    uint32_t two_runs;                   // mode 1: every tile lies in at most two runs
    Div32 d_vr, d_seg, d_nb, d_count;
};

struct RanksTile {
    uint8_t* dst;        // the written tensor (table entry of the receiving rank)
    const uint8_t* src0; // mode 0: the read tensor; mode 1, TWO: sender of the tile's first run
    const uint8_t* src1; // mode 1, TWO: sender of the tile's last run
    uint32_t k0;         // mode 1, TWO: sender index (from first) of the tile's first run
    int64_t dst_off;     // offset of the slab's first written vector
    int64_t src_off;     // read-side term shared by the slab
    uint32_t u0;         // first vector of the tile within its slab
    uint32_t nvec;       // vectors in this tile
};

// Sender index k (0 <= k < count) of vector u of a mode-1 slab: the slab's
// runs are numbered s * count + k along it.
UA2A_HD uint32_t ranks_sender(const RanksGeom& g, uint32_t u)
{
    const uint32_t run = fdiv(u, g.d_vr);
    return run - fdiv(run, g.d_count) * g.count;
}

template <bool MODE1, bool TWO>
UA2A_HD RanksTile ranks_tile(const RanksGeom& g, uint32_t x, uint32_t y, uint32_t z)
{
    RanksTile d;
    d.u0 = x * g.tile_vecs;
    d.nvec = umin32(g.tile_vecs, g.slab_vecs - d.u0);
    if (!MODE1) {
        const uint32_t j = g.first + y;
        const uint32_t r = fdiv(z, g.d_nb);
        const uint32_t b = z - r * g.nb;
        d.dst = g.dst[r];
        d.src0 = d.src1 = g.src[j];
        d.k0 = 0;
        d.dst_off = static_cast<int64_t>(b) * g.a_plane + static_cast<int64_t>(j) * g.s_local * g.vr;
        d.src_off = static_cast<int64_t>(b) * g.p_plane + static_cast<int64_t>(r) * g.vr;
    } else {
        const uint32_t b = y, j = z;
        d.dst = g.dst[j];
        d.dst_off = static_cast<int64_t>(b) * g.p_plane + static_cast<int64_t>(g.first) * g.vr;
        d.src_off = static_cast<int64_t>(b) * g.a_plane + static_cast<int64_t>(j) * g.s_local * g.vr;
        d.src0 = d.src1 = nullptr;
        d.k0 = 0;
        if (TWO) {
            d.k0 = ranks_sender(g, d.u0);
            d.src0 = g.src[g.first + d.k0];
            d.src1 = g.src[g.first + ranks_sender(g, d.u0 + d.nvec - 1)];
        }
    }
    return d;
}

// Read tensor and offsets of vector u (< slab_vecs) of the tile's slab.
template <bool MODE1, bool TWO>
UA2A_HD void ranks_vector(const RanksGeom& g, const RanksTile& d, uint32_t u, const uint8_t*& src,
                          int64_t& src_off, int64_t& dst_off)
{
    if (!MODE1) {
        const uint32_t s = fdiv(u, g.d_vr);          // token of the sending rank
        const uint32_t o = u - s * g.vr;
        src = d.src0;
        src_off = d.src_off + static_cast<int64_t>(static_cast<uint64_t>(s) * g.p_row) + o;
        dst_off = d.dst_off + u;
    } else {
        const uint32_t s = fdiv(u, g.d_seg);         // token of the receiving rank
        const uint32_t rem = u - s * g.seg;
        const uint32_t k = fdiv(rem, g.d_vr);        // sender = head block first + k
        const uint32_t o = rem - k * g.vr;
        src = TWO ? (k == d.k0 ? d.src0 : d.src1) : g.src[g.first + k];
        src_off = d.src_off + static_cast<int64_t>(static_cast<uint64_t>(s) * g.vr) + o;
        dst_off = d.dst_off + static_cast<int64_t>(static_cast<uint64_t>(s) * g.p_row) +
                  static_cast<int64_t>(k) * g.vr + o;
    }
}

// ------------------------------------------------------------------------
// Pack, mode 1, over per-rank allocations: every sender k in [first,
// first + count) copies, for every receiver q and plane b, its token block q
// -- one contiguous block of s_local runs -- into block k of q's window
// (receive windows laid out like one rank's sequence-gathered tensor,
// [B][S_local * w][H/w][D]).  Slab grid: x = tile within the block, y = k -
// first, z = q * nb + b (looped past the grid's extent).  Units: VB-byte
// vectors; a block is block_vecs of them, contiguous on both sides.
struct PackGeom {
    const uint8_t* src[kMaxRankTable];   // per sender: its tensor [B][S_local * w][H/w][D]
    uint8_t* dst[kMaxRankTable];         // per receiver: its window
    int64_t src_b, src_q;                // sender side: plane, receiver's token block
    int64_t dst_b, dst_k;                // window side: plane, sender's token block
    uint32_t block_vecs, tile_vecs, tiles_per_block;
    uint32_t first, ny, nz;              // ny = count, nz = w * nb
    Div32 d_nb;
};

struct PackTile {
    const uint8_t* src;   // the block's first byte in the sender's tensor
    uint8_t* dst;         // ... and in the receiver's window
    uint32_t u0, nvec;    // first vector of the tile within the block; vectors in it
};

template <int VB>
UA2A_HD PackTile pack_tile(const PackGeom& g, uint32_t x, uint32_t y, uint32_t z)
{
    const uint32_t k = g.first + y;
    const uint32_t q = fdiv(z, g.d_nb);
    const uint32_t b = z - q * g.d_nb.d;
    PackTile t;
    t.u0 = x * g.tile_vecs;
    t.nvec = umin32(g.tile_vecs, g.block_vecs - t.u0);
    t.src = g.src[k] + (static_cast<int64_t>(b) * g.src_b + static_cast<int64_t>(q) * g.src_q) * VB;
    t.dst = g.dst[q] + (static_cast<int64_t>(b) * g.dst_b + static_cast<int64_t>(k) * g.dst_k) * VB;
    return t;
}

// ------------------------------------------------------------------------
// LDS path: a workgroup stages rows [s0, s0 + rows) of one (j, b) -- a
// contiguous span of rows * w * run bytes on the P side -- in LDS, laid out
// as on the P side but shifted by `head` = the span's address mod 16 so that
// 16-byte global chunks map to 16-byte aligned LDS slots.  The w A-side spans
// of the tile (one per head block r, rows * run bytes each) are then moved in
// G-byte pieces, G = the alignment shared by run and both base pointers.
// When G = 16 (every span 16-aligned, head = 0) each LDS row is padded to
// lrow = row + pad bytes with lrow = run modulo 256: the lanes that move one
// run of consecutive rows then hit disjoint LDS banks, where the bare row
// stride (a multiple of the bank period for power-of-two rows) made them
// collide.  All units here are bytes.
//     t = (j * nb + b) * tiles_per_plane + tt      (P-side memory order)
// Tiles of one plane share a cache line wherever an A span's boundary is not
// a line boundary (rows * run or the span start not a multiple of 128 bytes,
// e.g. an odd S_local * run).  Workgroups are dealt round-robin to the
// chip's XCDs, each with its own L2, so the halves of such a line would be
// written (or read) through two L2s.  Launch slot L therefore takes tile
//     t = L - L % (kXcds * K) + (L % kXcds) * K + (L / kXcds) % K,
// K = 2^xlog: every XCD gets K consecutive tiles in a row, so K - 1 of every
// K boundaries stay inside one L2, while the kXcds * K tiles in flight at one
// time still cover one contiguous region.  Slots past num_tiles are empty.
constexpr uint32_t kXcds = 8;             // XCDs per MI355X, workgroups dealt round-robin

struct LdsGeom {
    uint8_t* p_ptr;            // base of the P-side tensor (read in mode 0, written in mode 1)
    uint8_t* a_ptr;            // base of the A-side tensor (written in mode 0, read in mode 1)
    int64_t a_rank, a_plane;
    int64_t p_rank, p_plane;
    uint32_t run;              // bytes per run
    uint32_t row;              // w * run
    uint32_t pad;              // LDS padding per row (0 unless G = 16)
    uint32_t lrow;             // row + pad: LDS stride of a row
    uint32_t s_local;
    uint32_t rows_per_tile;
    uint32_t tiles_per_plane;  // ceil(s_local / rows_per_tile)
    uint32_t num_tiles;        // w * nb * tiles_per_plane
    uint32_t num_slots;        // launch slots: num_tiles rounded up to kXcds << xlog
    uint32_t xlog;             // log2 of the consecutive tiles per XCD turn (0: plain order)
    uint32_t w, nb;
    uint32_t j0;               // first P-side rank the tiles cover (per-rank form: first sender)
    uint32_t a_window;         // 1: rank-stacked A side of under 4 GiB, so a tile's w A spans
                               //    lie within 4 GiB past head block 0's (mode 0 stores through
                               //    that range); 0: per-rank tables or larger tensors
    uint32_t a_whole16;        // 1: the A base and rank stride are 16-aligned (a tile whose
                               //    start and span length are too has only whole chunks)
    uint32_t lds_bytes;        // LDS bytes the kernel reserves (>= 16 + rows_per_tile * lrow)
    uint32_t stride_full;      // 16-byte chunk slots per A span: tile of rows_per_tile rows
    uint32_t stride_last;      // ... and the plane's last tile
    Div32 d_tpp, d_nb, d_run, d_row, d_stride_full, d_stride_last;
};

struct LdsTile {
    int64_t p_start;   // byte offset of the P span from its rank's base
    int64_t a_start0;  // byte offset of each A span from its head block's base
    uint8_t* p_span;   // the P span's first byte
    uint32_t p_len;    // rows * row
    uint32_t a_len;    // rows * run (each of the w A spans)
    uint32_t head;     // (p_ptr + p_start) mod 16: LDS position of the span's first byte
    uint32_t stride;   // chunk slots per A span in the flat (span, chunk) index
    uint32_t j;        // P-side rank of the tile
    Div32 d_stride;
};

// Where a tile's spans live.  Rank-stacked tensors: bases plus rank strides.
struct StackedBases {
    static constexpr bool kStacked = true;
    const LdsGeom& g;
    UA2A_HD uint8_t* p_rank_base(uint32_t j) const { return g.p_ptr + static_cast<int64_t>(j) * g.p_rank; }
    UA2A_HD uint8_t* a_rank_base(uint32_t r) const { return g.a_ptr + static_cast<int64_t>(r) * g.a_rank; }
};

// Rank-stacked tensors with one side moved by a byte offset: a one-launch
// chunked exchange on the LDS path reads batch plane p of its input (offset
// p * plane on the input side) and writes the one-plane window (offset 0).
struct PlaneBases {
    static constexpr bool kStacked = true;
    const LdsGeom& g;
    int64_t p_off, a_off;
    UA2A_HD uint8_t* p_rank_base(uint32_t j) const { return g.p_ptr + static_cast<int64_t>(j) * g.p_rank + p_off; }
    UA2A_HD uint8_t* a_rank_base(uint32_t r) const { return g.a_ptr + static_cast<int64_t>(r) * g.a_rank + a_off; }
};

// A chunked exchange in one launch on the LDS path.  LdsGeom describes plane
// 0 of every rank and the window ([w][one plane] in the layout of the output
// side: the A side in mode 0, the P side in mode 1).  Each workgroup keeps
// its LDS tile for all planes, `stage` planes at a time: it fills one LDS
// image per plane (image bytes apart) from the input moved by p * plane
// bytes, and after a workgroup barrier each lane, plane after plane, stores
// its chunks of the tile's window spans into the window, reads them back and
// stores them to plane p of the output.  Window byte x of block k lands at
// out + x + k * rank_step + p * plane (block k is head block r in mode 0, the
// tile's rank j in mode 1; rank_step = the output's rank stride minus the
// window's, plane bytes).  Every such offset is a multiple of the piece size
// G, so a window chunk goes to the output in one 16-byte store when the two
// agree modulo 16, else in G-byte pieces.
struct LdsChunkGeom {
    uint8_t* out;          // the output: plane 0 of rank 0
    int64_t rank_step;     // B * plane - plane
    int64_t plane;         // bytes of one batch plane of one rank
    uint32_t planes;       // B
    uint32_t stage;        // planes filled into LDS before they are drained, 1..B
    uint32_t image;        // LDS bytes of one plane's image (LdsGeom::lds_bytes)
};

// Per-rank allocations: one base pointer per rank and side (the rank strides
// of the geometry are 0).  The P table is indexed by the tile's rank (one per
// workgroup), the A table by each lane's head block.
struct LdsTables {
    uint8_t* p[kMaxRankTable];
    uint8_t* a[kMaxRankTable];
};

struct TableBases {
    static constexpr bool kStacked = false;
    const LdsTables& t;
    UA2A_HD uint8_t* p_rank_base(uint32_t j) const { return t.p[j]; }
    UA2A_HD uint8_t* a_rank_base(uint32_t r) const { return t.a[r]; }
};

// The same with the A table copied to a workgroup-local array first, so the
// per-lane lookups of the (span, chunk) loops read LDS, not the kernel
// argument in memory.
struct StagedTableBases {
    static constexpr bool kStacked = false;
    const LdsTables& t;
    uint8_t* const* a;
    UA2A_HD uint8_t* p_rank_base(uint32_t j) const { return t.p[j]; }
    UA2A_HD uint8_t* a_rank_base(uint32_t r) const { return a[r]; }
};

// The tile that launch slot L runs (see LdsGeom); >= num_tiles: none.
UA2A_HD uint32_t lds_slot_tile(const LdsGeom& g, uint32_t L)
{
    const uint32_t k = g.xlog;
    const uint32_t span = kXcds << k;
    return (L - L % span) + ((L % kXcds) << k) + ((L / kXcds) & ((1u << k) - 1u));
}

template <class Bases>
UA2A_HD LdsTile lds_tile(const LdsGeom& g, const Bases& bases, uint32_t t)
{
    const uint32_t jb = fdiv(t, g.d_tpp);
    const uint32_t tt = t - jb * g.tiles_per_plane;
    const uint32_t jr = fdiv(jb, g.d_nb);
    const uint32_t b = jb - jr * g.nb;
    const uint32_t j = g.j0 + jr;
    const uint32_t s0 = tt * g.rows_per_tile;
    const uint32_t rows = umin32(g.rows_per_tile, g.s_local - s0);
    LdsTile d;
    d.p_start = static_cast<int64_t>(b) * g.p_plane + static_cast<int64_t>(s0) * g.row;
    d.a_start0 = static_cast<int64_t>(b) * g.a_plane +
                 (static_cast<int64_t>(j) * g.s_local + s0) * g.run;
    d.p_len = rows * g.row;
    d.a_len = rows * g.run;
    d.p_span = bases.p_rank_base(j) + d.p_start;
    d.head = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(d.p_span) & 15u);
    const bool full = rows == g.rows_per_tile;
    d.stride = full ? g.stride_full : g.stride_last;
    d.d_stride = full ? g.d_stride_full : g.d_stride_last;
    d.j = j;
    return d;
}

// LDS byte position of P-span byte x (counted from the span's 16-aligned
// first chunk); with padding, x is a multiple of 16 and rows start at
// multiples of row.
UA2A_HD uint32_t lds_pos_of_p(const LdsGeom& g, uint32_t x)
{
    return g.pad ? x + fdiv(x, g.d_row) * g.pad : x;
}

// LDS byte position of byte p (0 <= p < a_len) of head block r's A span.
UA2A_HD uint32_t lds_pos_of_a(const LdsGeom& g, const LdsTile& d, uint32_t r, uint32_t p)
{
    const uint32_t k = fdiv(p, g.d_run);          // row within the tile
    const uint32_t off = p - k * g.run;           // byte within the run
    return d.head + k * g.lrow + r * g.run + off;
}

// Byte-sized pieces the LDS path moves between LDS and the A side.
typedef uint32_t u32x4 __attribute__((vector_size(16)));

template <int N> struct Piece;
template <> struct Piece<16> { typedef u32x4 T; };
template <> struct Piece<8> { typedef uint64_t T; };
template <> struct Piece<4> { typedef uint32_t T; };
template <> struct Piece<2> { typedef uint16_t T; };
template <> struct Piece<1> { typedef uint8_t T; };

UA2A_HD uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// A 16-byte chunk at byte `lo` of a span that starts `head` bytes into its
// 16-aligned first chunk and is `len` bytes long lies wholly in the span.
UA2A_HD bool chunk_full(uint32_t lo, uint32_t head, uint32_t len)
{
    return lo >= head && lo + 16 <= head + len;
}

// Chunks (16-byte, aligned) that a span touches.
UA2A_HD uint32_t span_chunks(uint32_t head, uint32_t len) { return (head + len + 15) >> 4; }

// Copy the in-span G-byte pieces of a partial chunk between two buffers
// that share the span's alignment (global P span <-> its LDS image, both
// indexed from the 16-aligned chunk base).
template <int G>
UA2A_HD void copy_partial_chunk(const uint8_t* from, uint8_t* to, uint32_t lo, uint32_t head,
                                uint32_t len)
{
    typedef typename Piece<G>::T T;
    const uint32_t x1 = umin32(lo + 16, head + len);
    for (uint32_t x = umax32(lo, head); x < x1; x += G)
        *reinterpret_cast<T*>(to + x) = *reinterpret_cast<const T*>(from + x);
}

// Gather the 16 bytes of a full A-span chunk of head block r from LDS;
// p0 = byte position of the chunk's first byte in the A span.  Positions
// advance by G and wrap into the next row at the end of each run.
template <int G>
UA2A_HD u32x4 gather_a_chunk(const LdsGeom& g, const LdsTile& d, uint32_t r, uint32_t p0,
                             const uint8_t* lds)
{
    typedef typename Piece<G>::T T;
    union {
        u32x4 v;
        T p[16 / G];
    } buf;
    uint32_t k = fdiv(p0, g.d_run);
    uint32_t off = p0 - k * g.run;
    uint32_t pos = d.head + k * g.lrow + r * g.run + off;
#pragma unroll
    for (int i = 0; i < 16 / G; ++i) {
        buf.p[i] = *reinterpret_cast<const T*>(lds + pos);
        off += G;
        pos += G;
        if (off == g.run) {          // next row of the tile, same head block
            off = 0;
            pos += g.lrow - g.run;
        }
    }
    return buf.v;
}

// Scatter the 16 bytes of a full A-span chunk of head block r into LDS.
template <int G>
UA2A_HD void scatter_a_chunk(const LdsGeom& g, const LdsTile& d, uint32_t r, uint32_t p0,
                             u32x4 v, uint8_t* lds)
{
    typedef typename Piece<G>::T T;
    union {
        u32x4 v;
        T p[16 / G];
    } buf;
    buf.v = v;
    uint32_t k = fdiv(p0, g.d_run);
    uint32_t off = p0 - k * g.run;
    uint32_t pos = d.head + k * g.lrow + r * g.run + off;
#pragma unroll
    for (int i = 0; i < 16 / G; ++i) {
        *reinterpret_cast<T*>(lds + pos) = buf.p[i];
        off += G;
        pos += G;
        if (off == g.run) {
            off = 0;
            pos += g.lrow - g.run;
        }
    }
}

// Partial A-span chunk (the first or last of a span): move its in-span
// G-byte pieces one by one.  achunk0 = the span's 16-aligned first chunk
// in global memory, ahead = the span's offset inside it.
template <class Mem, int G>
UA2A_HD void a_partial_from_lds(const LdsGeom& g, const LdsTile& d, uint32_t r, uint32_t lo,
                                uint32_t ahead, const uint8_t* lds, uint8_t* achunk0)
{
    typedef typename Piece<G>::T T;
    const uint32_t x1 = umin32(lo + 16, ahead + d.a_len);
    for (uint32_t x = umax32(lo, ahead); x < x1; x += G)
        Mem::st_piece(reinterpret_cast<T*>(achunk0 + x),
                      *reinterpret_cast<const T*>(lds + lds_pos_of_a(g, d, r, x - ahead)));
}

// Partial P-span chunk, LDS image -> global (the P span's first or last
// chunk when its base is not 16-aligned): its in-span G-byte pieces.
template <class Mem, int G>
UA2A_HD void p_partial_from_lds(const uint8_t* lds, uint8_t* pchunk0, uint32_t lo, uint32_t head,
                                uint32_t len)
{
    typedef typename Piece<G>::T T;
    const uint32_t x1 = umin32(lo + 16, head + len);
    for (uint32_t x = umax32(lo, head); x < x1; x += G)
        Mem::st_piece(reinterpret_cast<T*>(pchunk0 + x), *reinterpret_cast<const T*>(lds + x));
}

// ------------------------------------------------------------------------
// Plain strided block copy: `count` blocks of span vectors, block k at
// src + k*src_stride -> dst + k*dst_stride (units: VB-byte vectors).  Used
// for mode 0's unpack of a receiver's window into its output, one block.
struct CopyGeom {
    const uint8_t* src;
    uint8_t* dst;
    int64_t src_stride, dst_stride;
    int64_t span;              // vectors per block
    uint32_t tile_vecs;
    uint32_t tiles_per_span;   // ceil(span / tile_vecs)
    uint32_t num_tiles;        // count * tiles_per_span
    Div32 d_tps;
};

struct CopyTile {
    int64_t src_base, dst_base;
    uint32_t nvec;
};

UA2A_HD CopyTile copy_tile(const CopyGeom& g, uint32_t t)
{
    const uint32_t k = fdiv(t, g.d_tps);
    const uint32_t tt = t - k * g.tiles_per_span;
    const int64_t first = static_cast<int64_t>(tt) * g.tile_vecs;
    const int64_t left = g.span - first;
    CopyTile c;
    c.src_base = static_cast<int64_t>(k) * g.src_stride + first;
    c.dst_base = static_cast<int64_t>(k) * g.dst_stride + first;
    c.nvec = left < static_cast<int64_t>(g.tile_vecs) ? static_cast<uint32_t>(left) : g.tile_vecs;
    return c;
}

// ------------------------------------------------------------------------
// Readiness credits, one counter per receiving rank.  A publishing exchange
// runs in parts (ranges of receiving ranks); after a part's launch has
// completed, a signal launch adds 1 to the counters of its receivers with
// release order at device scope, so after n publishing calls a receiver whose
// output is complete holds n.  The wait kernel polls credits[first ..
// first+count) with acquire loads until each reaches `target` (compared
// modulo 2^32) or `spin_limit` polls of one counter have passed; then it sets
// *status to 1.  Either way it ends.
struct SignalGeom {
    uint32_t* credits;
    uint32_t first, count;     // counters credits[first .. first+count) get 1 each
};

struct WaitGeom {
    const uint32_t* credits;
    uint32_t first, count;
    uint32_t target;
    uint32_t spin_limit;       // >= 1
    int32_t* status;           // set to 1 on a time-out, never cleared here
};

UA2A_HD bool credit_reached(uint32_t value, uint32_t target)
{
    return static_cast<int32_t>(value - target) >= 0;
}

}  // namespace ua2a

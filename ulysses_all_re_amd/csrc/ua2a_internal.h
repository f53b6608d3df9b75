// Internal declarations shared by the host logic (ua2a_host.cpp) and the
// device backend (ua2a_kernels.hip).  Not part of the C ABI.
#pragma once

#include "ua2a.h"
#include "ua2a_geometry.h"

struct ua2a_plan_s {
    int32_t w;
    int64_t B, S_local, H, D;
    int32_t elem_bytes;
    ua2a_layout_t layout;
    int32_t blocks;            // grid hint, 0 = auto
    uint8_t* window;           // borrowed, may be null
    int64_t window_bytes;
    int32_t device;
    int32_t path;              // UA2A_PATH_*
    int32_t disabled;          // sticky after a backend failure
    char reason[256];          // why it is disabled
};

namespace ua2a {

// Tunables (bytes / vectors / workgroups).  Measured on MI355X: one vector
// per lane per pass, single-wave workgroups, one 1 KiB tile per workgroup
// and non-temporal accesses move the most bytes per second; deeper per-lane
// unrolling, bigger workgroups or persistent grids are slower there.
constexpr uint32_t kDirectUnroll = 1;           // vectors per lane per pass (direct, copy)
constexpr uint32_t kCapTiles = 4;               // tiles in flight per workgroup of a low-capped flat grid
constexpr uint32_t kCapInFlight = 8192;         // ... used while grid * kCapTiles stays within this
constexpr uint32_t kTileBytes = 1024;           // bytes per direct / copy tile
constexpr uint32_t kLdsUnroll = 2;              // 16-byte chunks per lane per pass (LDS fill, G = 16)
constexpr uint32_t kDirectMinRun = 256;         // auto path, mode 1: least contiguous read per head block
constexpr int64_t kDirectMode1Bytes = int64_t(80) << 20;   // auto path, mode 1 short runs: direct below this per side
constexpr uint32_t kDirectGroup = 8;            // grouped tile order (mode 0, 4 KiB-multiple rows)
constexpr uint32_t kDirectGroupRowAlign = 4096;
constexpr uint32_t kMaxGridYZ = 65535;          // largest y / z grid extent used
constexpr uint64_t kMaxGridWorkItems = (uint64_t(1) << 31);   // x extent of a launch, in lanes
constexpr uint32_t kLdsTileMode0 = 8192;        // target LDS bytes per workgroup, mode 0
constexpr uint32_t kLdsTileMode1 = 16384;       // target LDS bytes per workgroup, mode 1
constexpr uint32_t kLdsTileMax = 65536;         // a tile holds at least one row, up to this
constexpr uint32_t kLdsChunkTileMode0 = 8192;   // ... in a one-launch chunked exchange, mode 0
constexpr uint32_t kLdsChunkTileMode1 = 8192;   // ... and mode 1 (half the unchunked tile: the
                                                //   window spans in flight then stay within L2)
constexpr int64_t kLineBytes = 128;             // cache line: LDS tiles align their A spans to it
constexpr uint32_t kLdsXcdLog = 2;              // LDS tiles: 2^kLdsXcdLog consecutive tiles per XCD turn
constexpr uint32_t kLdsChunkStage = 2;          // one-launch chunked LDS path: planes per LDS fill
constexpr uint32_t kLdsChunkLds = 65536;        // ... within this much LDS per workgroup
constexpr uint32_t kLdsReadback = 2;            // one-launch chunked LDS path: window chunks per lane in
                                                //   flight, mode 0 (mode 1: one; measured 5 % faster there,
                                                //   6 % slower in mode 0; four: slower in both)
constexpr uint32_t kWaitBlock = 64;             // one wave polls (or signals) the counters

enum class Kernel : int32_t { Direct = 0, Lds = 1, Copy = 2, Ranks = 3, Wait = 4, Signal = 5,
                              LdsRanks = 6, Chunked = 7, Pack = 8, LdsChunked = 9 };

// One kernel launch, fully described for the backend.
struct Launch {
    Kernel kernel;
    uint32_t block;      // threads per workgroup
    uint32_t grid_y;     // 3-D grid of the direct kernel (1 otherwise)
    uint32_t grid_z;
    int32_t grid3d;      // direct/chunked kernel: one tile per workgroup on (grid, grid_y, grid_z)
    int32_t width;       // Direct/Copy/Ranks: bytes per lane vector; Lds: LDS piece bytes G
    int32_t mode;        // Direct/Lds/Ranks: 0 or 1
    uint32_t grid;       // workgroups along x
    uint32_t lds_bytes;  // dynamic LDS (the LDS kernels)
    DirectGeom direct;   // Direct; Chunked: plane 0 of every rank into the window
    ChunkedGeom chunk;   // Chunked: output, plane strides and plane count
    LdsGeom lds;         // Lds, LdsRanks; LdsChunked: plane 0 of every rank and the window
    LdsChunkGeom lds_chunk;   // LdsChunked: output, plane strides and plane count
    CopyGeom copy;
    RanksGeom ranks;
    PackGeom pack;       // Pack: blocks from the senders' tensors into the receivers' windows
    LdsTables lds_tab;   // LdsRanks: the per-rank bases of `lds`
    WaitGeom wait;
    SignalGeom signal;
};

// Device backend.  The library implements it over HIP; a host emulation
// (tests only) implements it over ordinary memory.  Each returns 0 or a
// backend error code that backend_error_name() can name.
int backend_current_device(int32_t* device);
int backend_launch(const Launch& launch, void* stream);
const char* backend_error_name(int err);
// The device address of the library's own UA2A_NOALLOC_WINDOW_BYTES window on
// `device` (the calling thread's current device).
int backend_scratch_window(int32_t device, uint8_t** window);

}  // namespace ua2a

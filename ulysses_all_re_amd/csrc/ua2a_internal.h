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
    int32_t cus;               // compute units of `device`, 0 until first queried
    int32_t disabled;          // sticky after a backend failure
    char reason[256];          // why it is disabled
};

namespace ua2a {

// Tunables of the host logic (bytes / vectors / workgroups).
constexpr uint32_t kDirectTileVectors = 4096;   // target vectors per direct-path tile
constexpr uint32_t kDirectUnroll = 4;           // vectors in flight per lane (direct, copy)
constexpr uint32_t kLdsUnroll = 4;              // 16-byte chunks in flight per lane (LDS fill)
constexpr uint32_t kDirectMinRun = 256;         // auto path: direct only for runs >= this (bytes)
constexpr uint32_t kLdsTileBytes = 32768;       // LDS per workgroup on the LDS path
constexpr uint32_t kCopyTileVectors = 4096;     // vectors per copy-kernel tile
constexpr uint32_t kDirectBlocksPerCu = 8;      // auto grid caps (workgroups per CU)
constexpr uint32_t kLdsBlocksPerCu = 4;
constexpr uint32_t kCopyBlocksPerCu = 8;
constexpr int32_t kAssumedCus = 256;            // used by ua2a_describe before the first exchange

enum class Kernel : int32_t { Direct = 0, Lds = 1, Copy = 2 };

// One kernel launch, fully described for the backend.
struct Launch {
    Kernel kernel;
    int32_t width;       // Direct/Copy: bytes per lane vector; Lds: LDS piece bytes G
    int32_t mode;        // Direct/Lds: 0 or 1
    uint32_t grid;
    uint32_t lds_bytes;  // dynamic LDS (Lds kernel only)
    DirectGeom direct;
    LdsGeom lds;
    CopyGeom copy;
};

// Device backend.  The library implements it over HIP; a host emulation
// (tests only) implements it over ordinary memory.  Each returns 0 or a
// backend error code that backend_error_name() can name.
int backend_current_device(int32_t* device);
int backend_cu_count(int32_t device, int32_t* cus);
int backend_launch(const Launch& launch, void* stream);
const char* backend_error_name(int err);

}  // namespace ua2a

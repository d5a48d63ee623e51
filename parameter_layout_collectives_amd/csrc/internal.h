// Internal declarations of the TIDE library (host plan + HIP runtime).
//
// The plan is pure host data: shard geometry and the tile lists the kernels
// walk.  Device copies of those tables, and a small cache of uploaded
// pointer tables, live in one DeviceState per device the plan is used on.
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tide.h"

namespace tide {

// Build-time tuning constants (defaults are the measured best on MI355X).
#ifndef TIDE_RS_TILE
#define TIDE_RS_TILE 4096
#endif
#ifndef TIDE_AG_TILE
#define TIDE_AG_TILE 2048
#endif
#ifndef TIDE_AG_TILE_SMALL
#define TIDE_AG_TILE_SMALL 16384
#endif
#ifndef TIDE_RS_TILE_SMALL
#define TIDE_RS_TILE_SMALL 2048
#endif

// Elements of one parameter segment handled by one reduce-scatter tile, and
// by one all-gather tile.  Both are multiples of 8 so that tile starts keep
// the 16-byte phase of the segment they cut.
constexpr int64_t kRsTile = TIDE_RS_TILE;
constexpr int64_t kAgTile = TIDE_AG_TILE;
// Small-footprint all-gather launches keep one workgroup per CU resident, so
// each one moves a larger tile to keep enough bytes in flight.
constexpr int64_t kAgTileSmall = TIDE_AG_TILE_SMALL;
constexpr int64_t kRsTileSmall = TIDE_RS_TILE_SMALL;
static_assert(kRsTile % 8 == 0 && kAgTile % 8 == 0 && kAgTileSmall % 8 == 0 &&
                  kRsTileSmall % 8 == 0,
              "tiles must keep the 16-byte phase");
static_assert(kAgTileSmall * 4 < (int64_t(1) << 31), "all-gather tile bytes must fit in int");
constexpr int kBlock = 256;           // lanes per workgroup (4 wave64)

// Per-parameter geometry as the kernels read it.  src(r) = r*seg and
// L(r) = min(seg, max(0, numel - r*seg)) follow from seg and numel.
struct ParamDesc {
    int64_t off;     // offset of the parameter's segment in a rank block
    int64_t seg;     // c * inner: elements per rank block (padding included)
    int64_t numel;   // dim0 * inner: elements of the full tensor
    int64_t span;    // seg plus the alignment gap up to the next offset (or S)
};

// One tile: `param`'s elements [k0, k0 + tile) of rank `rank`'s segment
// (all-gather) or of the parameter's span in the block (reduce-scatter,
// where `rank` is unused: the rank is a launch argument).
struct Tile {
    int32_t param;
    int32_t rank;
    int64_t k0;
};

struct PtrTable {
    std::vector<uintptr_t> key;  // the host pointer array it was built from
    uint64_t hash = 0;
    void *dev = nullptr;         // device copy of the pointer array
    bool aligned16 = false;      // every non-null pointer is 16-byte aligned
    uint64_t last_use = 0;
};

struct DeviceState {
    int device = -1;
    int cus = 0;
    int lds_per_cu = 0;          // bytes of LDS per compute unit
    int lds_per_wg_max = 0;      // largest LDS allocation one workgroup may make
    int small_lds = 0;           // LDS a small-footprint workgroup reserves (0 = none)
    int rs_cap_lds = 0;          // LDS a default reduce-scatter workgroup reserves (0 = none)
    int ag_cap_lds = 0;          // LDS a default all-gather workgroup reserves (0 = none)
    void *d_params = nullptr;    // ParamDesc[P]
    void *d_rs_tiles = nullptr;  // Tile[n_rs]
    void *d_ag_tiles = nullptr;  // Tile[n_ag]
    void *d_ag_tiles_small = nullptr;  // Tile[n_ag_small]
    void *d_rs_tiles_small = nullptr;  // Tile[n_rs_small]
    std::vector<PtrTable> rs_cache, ag_cache;
    uint64_t tick = 0;
};

constexpr size_t kPtrCacheEntries = 8;

}  // namespace tide

struct tide_plan {
    int32_t N = 0, P = 0;
    int64_t align = 1, S = 0, psi = 0;
    std::vector<int64_t> d0, inner, c, seg, off, numel;
    std::vector<tide::ParamDesc> desc;
    std::vector<tide::Tile> rs_tiles, rs_tiles_small, ag_tiles, ag_tiles_small;
    mutable std::mutex mu;
    mutable std::vector<tide::DeviceState *> devs;
};

namespace tide {

// Thread-local error message; returns `st` for convenience.
tide_status fail(tide_status st, const std::string &msg);
void clear_error();
const char *last_error_cstr();

// src(r,i) and L(r,i).
inline void shard_run(const tide_plan *p, int32_t r, int32_t i, int64_t *src, int64_t *L) {
    const int64_t seg = p->seg[i];
    const int64_t s = static_cast<int64_t>(r) * seg;
    int64_t l = p->numel[i] - s;
    if (l < 0) l = 0;
    if (l > seg) l = seg;
    *src = s;
    *L = l;
}

// Argument checks shared by the launch paths (host only, no HIP call).
tide_status check_rs_args(const tide_plan *p, int32_t rank, const void *const *grads,
                          const float *out, uint32_t flags, int32_t max_wg);
tide_status check_ag_args(const tide_plan *p, const void *const *rank_src,
                          void *const *params, int32_t elem_bytes, uint32_t flags,
                          int32_t max_wg);

// Frees the device tables of a plan (defined next to the kernels).
void release_device_states(const tide_plan *p);

}  // namespace tide

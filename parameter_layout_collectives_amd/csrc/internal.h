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
#include "kernel_abi.h"

namespace tide {

// One slot of a plan's pointer-table cache on one device.  A slot's buffers
// are allocated once and reused for every pointer set it holds: a new set
// is written to the pinned staging copy and uploaded with an async copy on
// the caller's stream, so the launch that follows reads it in stream order.
// A stream that has read a slot, and the event recorded on it after its
// latest read (upload or launch).
struct SlotReader {
    void *stream;                // hipStream_t
    void *event;                 // hipEvent_t, owned by the slot
};

struct PtrTable {
    std::vector<uintptr_t> key;  // the host pointer array it was built from
    uint64_t hash = 0;
    void *dev = nullptr;         // device copy of the pointer array
    void *staging = nullptr;     // pinned host buffer the upload reads
    std::vector<SlotReader> readers;  // one entry per stream that has read the slot
    bool untracked = false;      // a read could not be recorded: reuse waits for the device
    void *uploaded = nullptr;    // hipEvent_t recorded after the upload of the current set
    void *upload_stream = nullptr;
    bool upload_done = false;    // the upload is known to have finished
    bool pinned = false;         // read by a captured graph: never replaced
    bool aligned16 = false;      // every non-null pointer is 16-byte aligned
    uint64_t last_use = 0;
};

// What the launch policy needs to know about one device, and the LDS
// reservations it derives from that.
struct DeviceLimits {
    int cus = 0;
    int lds_per_cu = 0;          // bytes of LDS per compute unit
    int lds_per_wg_max = 0;      // largest LDS allocation one workgroup may make
    int small_lds = 0;           // LDS a small-footprint workgroup reserves (0 = none)
    int rs_cap_lds = 0;          // LDS a default reduce-scatter workgroup reserves (0 = none)
    int ag_cap_lds = 0;          // LDS a default all-gather workgroup reserves (0 = none)
};

struct DeviceState {
    int device = -1;
    DeviceLimits lim;
    void *d_params = nullptr;    // ParamDesc[P]
    void *d_rs_tiles = nullptr;  // Tile[n_rs]
    void *d_ag_tiles = nullptr;  // Tile[n_ag]
    void *d_ag_tiles_small = nullptr;  // Tile[n_ag_small]
    void *d_rs_tiles_small = nullptr;  // Tile[n_rs_small]
    void *d_pack_tiles = nullptr;        // Tile[n_pack]
    void *d_pack_tiles_small = nullptr;  // Tile[n_pack_small]
    std::vector<PtrTable> rs_cache, ag_cache, pack_cache, slots_cache;
    uint64_t tick = 0;
};

constexpr size_t kPtrCacheEntries = 8;
constexpr size_t kMaxSlotReaders = 16;   // streams tracked per pointer-table slot

}  // namespace tide

struct tide_plan {
    int32_t N = 0, P = 0;
    int64_t align = 1, S = 0, psi = 0;
    std::vector<int64_t> d0, inner, c, seg, off, numel;
    std::vector<tide::ParamDesc> desc;
    std::vector<tide::Tile> rs_tiles, rs_tiles_small, ag_tiles, ag_tiles_small;
    std::vector<tide::Tile> pack_tiles, pack_tiles_small;
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
                          const void *out, uint32_t flags, int32_t max_wg);
tide_status check_ag_args(const tide_plan *p, const void *const *rank_src,
                          void *const *params, int32_t elem_bytes, uint32_t flags,
                          int32_t max_wg);
tide_status check_pack_args(const tide_plan *p, const void *const *tensors, const void *slot,
                            int32_t elem_bytes, uint32_t flags, int32_t max_wg);
tide_status check_rs_slots_args(const tide_plan *p, int32_t rank, const void *const *slots,
                                const void *out, uint32_t flags, int32_t max_wg);

// Frees the device tables of a plan (defined next to the kernels).
void release_device_states(const tide_plan *p);

// Launch policy (runtime.hip), shared by every entry point.
tide_status query_limits(int device, DeviceLimits *out);   // device attributes (no allocation)
// Kernel shape, tile size and LDS reservation of a reduce-scatter launch.
struct RsPolicy {
    RsKernelShape shape; // kRsSmall walks the kRsTileSmall tile list, the others kRsTile
    int64_t tile;        // kRsTile or kRsTileSmall
    int lds;
};
RsPolicy rs_policy(const DeviceLimits &lim, int32_t N, uint32_t flags);
unsigned grid_size(const DeviceLimits &lim, int64_t ntiles, uint32_t flags, int32_t max_wg);
tide_status hip_fail(const char *what, hipError_t e);

}  // namespace tide

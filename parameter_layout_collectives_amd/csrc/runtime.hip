// Runtime of the TIDE library on the HIP side: per-device tables, the
// pointer-table cache, the launch policy and the extern "C" entry points
// tide_rs, tide_ag, tide_pack and tide_rs_slots.  The kernels and their
// launch functions are in kernels.hip; the host-only plan and argument
// checks in plan.cpp.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <new>

#include "internal.h"

namespace tide {
namespace {

// Launch policy (defaults are the measured best on MI355X).
#ifndef TIDE_DEFAULT_ONE_TILE_PER_WG
#define TIDE_DEFAULT_ONE_TILE_PER_WG 1
#endif
#ifndef TIDE_SMALL_LDS_RESERVE
#define TIDE_SMALL_LDS_RESERVE 1
#endif
#ifndef TIDE_SMALL_WG_PER_CU
#define TIDE_SMALL_WG_PER_CU 1
#endif
#ifndef TIDE_SMALL_PERSISTENT
#define TIDE_SMALL_PERSISTENT 0
#endif
#ifndef TIDE_RS_WG_CAP
#define TIDE_RS_WG_CAP 2
#endif
#ifndef TIDE_AG_WG_CAP
#define TIDE_AG_WG_CAP 0
#endif
#ifndef TIDE_WG_PER_CU
#define TIDE_WG_PER_CU 8
#endif
#ifndef TIDE_SMALL_WG
#define TIDE_SMALL_WG 32
#endif
// Small-footprint TIDE-RS for at most this many ranks runs the default
// kernel shape (4 chunks per lane over 4096-element tiles) under the
// small-footprint LDS reservation; for more ranks, the lighter small shape
// (1 chunk per lane, 1024-element tiles, 16-rank batches), whose shorter
// workgroups hand CUs back sooner.  Beside a bf16 8192^3 GEMM the default
// shape cost the GEMM 0.3% (8 ranks) and 3.5% (16 ranks) but 9.9% at 64
// ranks; at 64 ranks 2048-element tiles with 2 chunks per lane cost it
// 8.9-11.2% and the shipped 1024-element shape 6.8%.
#ifndef TIDE_SMALL_FEW_RANKS
#define TIDE_SMALL_FEW_RANKS 16
#endif
constexpr int kWgPerCu = TIDE_WG_PER_CU;      // default grid: enough waves to keep HBM busy
constexpr int kSmallFootprintWg = TIDE_SMALL_WG;  // small-footprint grid

tide_status upload(const void *host, size_t bytes, void **dev, const char *what) {
    *dev = nullptr;
    if (bytes == 0) return TIDE_OK;
    hipError_t e = hipMalloc(dev, bytes);
    if (e != hipSuccess) {
        *dev = nullptr;
        if (e == hipErrorOutOfMemory) return fail(TIDE_E_NOMEM, std::string(what) + ": hipMalloc");
        return hip_fail(what, e);
    }
    e = hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(*dev);
        *dev = nullptr;
        return hip_fail(what, e);
    }
    return TIDE_OK;
}

void free_state(DeviceState *ds) {
    (void)hipFree(ds->d_params);
    (void)hipFree(ds->d_rs_tiles);
    (void)hipFree(ds->d_ag_tiles);
    (void)hipFree(ds->d_ag_tiles_small);
    (void)hipFree(ds->d_pack_tiles);
    (void)hipFree(ds->d_pack_tiles_small);
    (void)hipFree(ds->d_rs_tiles_small);
    for (auto *cache : {&ds->rs_cache, &ds->ag_cache, &ds->pack_cache, &ds->slots_cache})
        for (auto &pt : *cache) {
            (void)hipFree(pt.dev);
            (void)hipHostFree(pt.staging);
            for (const SlotReader &r : pt.readers)
                (void)hipEventDestroy(static_cast<hipEvent_t>(r.event));
            if (pt.uploaded) (void)hipEventDestroy(static_cast<hipEvent_t>(pt.uploaded));
        }
    delete ds;
}

// LDS that lets exactly `cap` workgroups share a CU (0: no cap).
int lds_for_cap(const DeviceLimits &lim, int cap) {
    if (cap <= 0 || lim.lds_per_cu <= 0) return 0;
    const int want = lim.lds_per_cu / cap - 1024;
    return (want > 0 && want <= lim.lds_per_wg_max) ? want : 0;
}

// The plan's tables on the current device (created on first use, which
// allocates and copies synchronously, so never inside a graph capture).
// Caller holds p->mu.
tide_status device_state(const tide_plan *p, bool capturing, DeviceState **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    for (DeviceState *ds : p->devs)
        if (ds->device == dev) {
            *out = ds;
            return TIDE_OK;
        }
    if (capturing)
        return fail(TIDE_E_UNSUPPORTED,
                    "the first call of a plan on a device cannot be captured into a graph: "
                    "make one call outside the capture first");
    DeviceLimits lim;
    tide_status st = query_limits(dev, &lim);
    if (st != TIDE_OK) return st;
    DeviceState *ds = new (std::nothrow) DeviceState;
    if (!ds) return fail(TIDE_E_NOMEM, "device state: out of host memory");
    ds->device = dev;
    ds->lim = lim;
    st = upload(p->desc.data(), p->desc.size() * sizeof(ParamDesc), &ds->d_params,
                            "parameter table");
    if (st == TIDE_OK)
        st = upload(p->rs_tiles.data(), p->rs_tiles.size() * sizeof(Tile), &ds->d_rs_tiles,
                    "reduce-scatter tiles");
    if (st == TIDE_OK)
        st = upload(p->rs_tiles_small.data(), p->rs_tiles_small.size() * sizeof(Tile),
                    &ds->d_rs_tiles_small, "reduce-scatter tiles (small footprint)");
    if (st == TIDE_OK)
        st = upload(p->ag_tiles.data(), p->ag_tiles.size() * sizeof(Tile), &ds->d_ag_tiles,
                    "all-gather tiles");
    if (st == TIDE_OK)
        st = upload(p->ag_tiles_small.data(), p->ag_tiles_small.size() * sizeof(Tile),
                    &ds->d_ag_tiles_small, "all-gather tiles (small footprint)");
    if (st == TIDE_OK)
        st = upload(p->pack_tiles.data(), p->pack_tiles.size() * sizeof(Tile), &ds->d_pack_tiles,
                    "pack tiles");
    if (st == TIDE_OK)
        st = upload(p->pack_tiles_small.data(), p->pack_tiles_small.size() * sizeof(Tile),
                    &ds->d_pack_tiles_small, "pack tiles (small footprint)");
    if (st != TIDE_OK) {
        free_state(ds);
        return st;
    }
    try {
        p->devs.push_back(ds);
    } catch (const std::bad_alloc &) {
        free_state(ds);
        return fail(TIDE_E_NOMEM, "device state: out of host memory");
    }
    *out = ds;
    return TIDE_OK;
}

uint64_t hash_ptrs(uint64_t h, const uintptr_t *v, size_t n) {
    for (size_t i = 0; i < n; i++) {
        h ^= static_cast<uint64_t>(v[i]);
        h *= 1099511628211ull;
    }
    return h;
}

// A pointer set as the caller passed it: `na` entries at `a`, then `nb` at
// `b` (read in place; copied only when a new table is made).
struct PtrKey {
    const uintptr_t *a;
    size_t na;
    const uintptr_t *b;
    size_t nb;
    size_t size() const { return na + nb; }
    bool equals(const std::vector<uintptr_t> &k) const {
        return k.size() == size() && std::memcmp(k.data(), a, na * sizeof(uintptr_t)) == 0 &&
               (nb == 0 || std::memcmp(k.data() + na, b, nb * sizeof(uintptr_t)) == 0);
    }
};

// Records that work on `stream` reads the slot: called after its upload
// and after every launch that reads it.  Each stream gets its own event
// (created on its first read of this slot), so reusing the slot later waits
// for exactly the streams that read it.
tide_status mark_read(PtrTable *pt, hipStream_t stream) {
    SlotReader *reader = nullptr;
    for (SlotReader &r : pt->readers)
        if (r.stream == static_cast<void *>(stream)) reader = &r;
    hipError_t e = hipSuccess;
    if (!reader && pt->readers.size() >= kMaxSlotReaders) {
        // A new stream takes over the entry of a stream whose last read has
        // finished (or, if none has, of the first one once it finishes).
        for (SlotReader &r : pt->readers)
            if (!reader && hipEventQuery(static_cast<hipEvent_t>(r.event)) == hipSuccess)
                reader = &r;
        if (!reader) {
            reader = &pt->readers.front();
            e = hipEventSynchronize(static_cast<hipEvent_t>(reader->event));
        }
        reader->stream = static_cast<void *>(stream);
    }
    if (!reader && e == hipSuccess) {
        hipEvent_t ev = nullptr;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e == hipSuccess) {
            try {
                pt->readers.push_back({static_cast<void *>(stream), ev});
                reader = &pt->readers.back();
            } catch (const std::bad_alloc &) {
                (void)hipEventDestroy(ev);
                pt->untracked = true;
                return fail(TIDE_E_NOMEM, "pointer table: out of host memory");
            }
        }
    }
    if (e == hipSuccess) e = hipEventRecord(static_cast<hipEvent_t>(reader->event), stream);
    if (e != hipSuccess) {
        // No event covers this read: reuse waits for the device.
        pt->untracked = true;
        return hip_fail("pointer table: recording its reader", e);
    }
    return TIDE_OK;
}

// OK once the slot's upload has finished (checked without waiting);
// TIDE_E_UNSUPPORTED while it is still in flight.
tide_status upload_finished(PtrTable *pt) {
    if (pt->upload_done) return TIDE_OK;
    hipError_t e = hipEventQuery(static_cast<hipEvent_t>(pt->uploaded));
    if (e == hipSuccess) {
        pt->upload_done = true;
        return TIDE_OK;
    }
    if (e != hipErrorNotReady) return hip_fail("pointer table: hipEventQuery", e);
    return fail(TIDE_E_UNSUPPORTED,
                "the pointer table is still being uploaded: synchronize before capturing");
}

// A launch on `stream` that reads the slot must not start before the upload
// (enqueued on another stream, perhaps) has finished.
tide_status order_after_upload(PtrTable *pt, hipStream_t stream) {
    if (pt->upload_done) return TIDE_OK;
    const hipEvent_t up = static_cast<hipEvent_t>(pt->uploaded);
    hipError_t e = hipEventQuery(up);
    if (e == hipSuccess) {
        pt->upload_done = true;
        return TIDE_OK;
    }
    if (e != hipErrorNotReady) return hip_fail("pointer table: hipEventQuery", e);
    if (pt->upload_stream == static_cast<void *>(stream)) return TIDE_OK;   // stream order
    e = hipStreamWaitEvent(stream, up, 0);
    if (e != hipSuccess) return hip_fail("pointer table: hipStreamWaitEvent", e);
    return TIDE_OK;
}

// Allocates a slot's device table, pinned staging buffer and upload event
// (reader events are created as streams read the slot).
tide_status new_slot(size_t bytes, PtrTable *pt) {
    hipError_t e = hipMalloc(&pt->dev, bytes);
    if (e == hipSuccess) e = hipHostMalloc(&pt->staging, bytes, hipHostMallocDefault);
    hipEvent_t up = nullptr;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&up, hipEventDisableTiming);
    pt->uploaded = up;
    if (e == hipSuccess) return TIDE_OK;
    (void)hipFree(pt->dev);
    (void)hipHostFree(pt->staging);
    if (up) (void)hipEventDestroy(up);
    pt->dev = pt->staging = pt->uploaded = nullptr;
    if (e == hipErrorOutOfMemory) return fail(TIDE_E_NOMEM, "pointer table: allocation");
    return hip_fail("pointer table: allocation", e);
}

// Waits until no launch can still read the slot's device table (and so no
// upload can still read its staging buffer): the latest event of every
// stream that read it.  Only a read that could not be recorded makes it
// wait for the whole device.
tide_status drain_slot(PtrTable *pt) {
    hipError_t e = hipSuccess;
    if (pt->untracked) {
        e = hipDeviceSynchronize();
        if (e == hipSuccess) pt->untracked = false;
    } else {
        for (const SlotReader &r : pt->readers) {
            e = hipEventSynchronize(static_cast<hipEvent_t>(r.event));
            if (e != hipSuccess) break;
        }
    }
    if (e != hipSuccess) return hip_fail("pointer table: waiting for its last readers", e);
    return TIDE_OK;
}

// Finds the slot that holds a pointer set, or fills one with it.  A hit
// costs one hash and one compare over the caller's arrays.  On a miss a
// free slot is taken (at most kPtrCacheEntries per cache), else the least
// recently used one once its last reader has finished; `order(key, dev)`
// writes the array as the kernel wants it (`dev_len` entries: a permutation
// of the key, possibly padded) into the slot's pinned staging buffer, and an
// async copy on `stream` uploads it.  After launching, the caller must call
// mark_read().  Caller holds p->mu.
template <typename Order>
tide_status pointer_table(DeviceState *ds, std::vector<PtrTable> &cache, const PtrKey &key,
                          size_t dev_len, Order order, hipStream_t stream, bool capturing,
                          PtrTable **out) {
    const uint64_t h = hash_ptrs(hash_ptrs(1469598103934665603ull, key.a, key.na), key.b, key.nb);
    for (auto &pt : cache)
        if (pt.hash == h && key.equals(pt.key)) {
            if (capturing) {
                // A graph's launches read this slot at every replay: the
                // upload must be complete now, and the slot is never reused.
                tide_status st = upload_finished(&pt);
                if (st != TIDE_OK) return st;
                pt.pinned = true;
            } else {
                tide_status st = order_after_upload(&pt, stream);
                if (st != TIDE_OK) return st;
            }
            pt.last_use = ++ds->tick;
            *out = &pt;
            return TIDE_OK;
        }
    if (capturing)
        return fail(TIDE_E_UNSUPPORTED,
                    "a pointer set the plan has not cached cannot be uploaded inside a graph "
                    "capture: make one call with the same pointers outside the capture first");
    const size_t bytes = dev_len * sizeof(uintptr_t);
    PtrTable *pt = nullptr;
    if (cache.size() < kPtrCacheEntries) {
        PtrTable fresh;
        tide_status st = new_slot(bytes, &fresh);
        if (st != TIDE_OK) return st;
        try {
            cache.reserve(kPtrCacheEntries);
            cache.push_back(std::move(fresh));
        } catch (const std::bad_alloc &) {
            (void)hipFree(fresh.dev);
            (void)hipHostFree(fresh.staging);
            (void)hipEventDestroy(static_cast<hipEvent_t>(fresh.uploaded));
            return fail(TIDE_E_NOMEM, "pointer table: out of host memory");
        }
        pt = &cache.back();
    } else {
        pt = nullptr;
        for (auto &c : cache)
            if (!c.pinned && (!pt || c.last_use < pt->last_use)) pt = &c;
        if (!pt)
            return fail(TIDE_E_UNSUPPORTED,
                        "every cached pointer set of this plan is read by a captured graph");
        tide_status drained = drain_slot(pt);
        if (drained != TIDE_OK) return drained;
    }
    // The slot holds no valid set until the upload is enqueued.  Its reader
    // events stay: they are all complete now and are re-recorded on use.
    pt->hash = 0;
    pt->key.clear();
    try {
        pt->key.resize(key.size());
    } catch (const std::bad_alloc &) {
        return fail(TIDE_E_NOMEM, "pointer table: out of host memory");
    }
    std::copy(key.a, key.a + key.na, pt->key.begin());
    if (key.nb) std::copy(key.b, key.b + key.nb, pt->key.begin() + key.na);
    uintptr_t *staged = static_cast<uintptr_t *>(pt->staging);
    std::fill(staged, staged + dev_len, uintptr_t{0});
    order(pt->key.data(), staged);
    hipError_t e = hipMemcpyAsync(pt->dev, staged, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) {
        pt->key.clear();
        return hip_fail("pointer table: upload", e);
    }
    // The copy reads the staging buffer: the slot is not reusable before it
    // ends, and launches on other streams wait for it.
    tide_status st = mark_read(pt, stream);
    if (st == TIDE_OK) {
        e = hipEventRecord(static_cast<hipEvent_t>(pt->uploaded), stream);
        if (e != hipSuccess) st = hip_fail("pointer table: hipEventRecord", e);
    }
    if (st != TIDE_OK) {
        pt->key.clear();
        return st;
    }
    pt->upload_stream = static_cast<void *>(stream);
    pt->upload_done = false;
    pt->hash = h;
    // Over the table as the kernel reads it (null padding entries are aligned).
    pt->aligned16 = true;
    for (size_t j = 0; j < dev_len; j++) pt->aligned16 = pt->aligned16 && (staged[j] & 15) == 0;
    pt->last_use = ++ds->tick;
    *out = pt;
    return TIDE_OK;
}

// The reduce-scatter launch for `flags`: kernel shape, tile list, LDS.
struct RsShape {
    RsKernelShape shape; // kernel shape (kRsSmall: the small-footprint tile list)
    const Tile *tiles;
    int64_t ntiles;
    int lds;
};

RsShape rs_shape(const tide_plan *p, const DeviceState *ds, uint32_t flags) {
    const RsPolicy pol = rs_policy(ds->lim, p->N, flags);
    RsShape r;
    const bool small_tiles = pol.shape == kRsSmall;
    r.shape = pol.shape;
    r.tiles = static_cast<const Tile *>(small_tiles ? ds->d_rs_tiles_small : ds->d_rs_tiles);
    r.ntiles = static_cast<int64_t>(small_tiles ? p->rs_tiles_small.size()
                                                : p->rs_tiles.size());
    r.lds = pol.lds;
    return r;
}

// Whether work enqueued on `stream` is being captured into a graph.
tide_status capture_status(void *stream, bool *capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs);
    if (e != hipSuccess) return hip_fail("hipStreamIsCapturing", e);
    *capturing = cs == hipStreamCaptureStatusActive;
    return TIDE_OK;
}

// After a launch: the slot's reader tracking (not while capturing - a
// captured launch reads a pinned slot).
tide_status after_launch(PtrTable *pt, hipStream_t stream, bool capturing) {
    return capturing ? TIDE_OK : mark_read(pt, stream);
}

}  // namespace

tide_status hip_fail(const char *what, hipError_t e) {
    return fail(TIDE_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

tide_status query_limits(int dev, DeviceLimits *out) {
    DeviceLimits lim;
    hipError_t e = hipDeviceGetAttribute(&lim.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&lim.lds_per_cu,
                                  hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&lim.lds_per_wg_max, hipDeviceAttributeMaxSharedMemoryPerBlock,
                                  dev);
    if (e != hipSuccess) return hip_fail("hipDeviceGetAttribute", e);
    // A small-footprint workgroup reserves just over half of a CU's LDS, so
    // no two of them share a CU: the hardware dispatcher has to spread them
    // one per CU, and a CU that holds one cannot take two workgroups of an
    // LDS-heavy kernel running beside it.  The reservation is never touched.
    lim.small_lds = 0;
    if (TIDE_SMALL_LDS_RESERVE && lim.lds_per_cu > 0) {
        const int want = lim.lds_per_cu / 2 + 1024;
        if (want <= lim.lds_per_wg_max) lim.small_lds = want;
    }
    // Optional cap on default reduce-scatter workgroups per CU (same trick:
    // an untouched LDS reservation of which exactly TIDE_RS_WG_CAP fit).
    lim.rs_cap_lds = lds_for_cap(lim, TIDE_RS_WG_CAP);
    lim.ag_cap_lds = lds_for_cap(lim, TIDE_AG_WG_CAP);
    *out = lim;
    return TIDE_OK;
}

RsPolicy rs_policy(const DeviceLimits &lim, int32_t N, uint32_t flags) {
    const bool small = (flags & TIDE_F_SMALL_FOOTPRINT) != 0;
    RsPolicy r;
    r.shape = small ? (N > TIDE_SMALL_FEW_RANKS ? kRsSmall : kRsDefault)
                    : (N >= TIDE_RS_WIDE_N ? kRsWide : kRsDefault);
    r.tile = r.shape == kRsSmall ? kRsTileSmall : kRsTile;
    r.lds = small ? lim.small_lds : lim.rs_cap_lds;
    return r;
}

// Both launch modes give every tile its own short-lived workgroup, and the
// hardware dispatcher balances them over all CUs.  Small-footprint launches
// also reserve over half a CU's LDS per workgroup, so at most one of them
// is resident on a CU at any moment, and each holds its CU for one tile
// only.  A kernel that fills every CU (a single-wave GEMM) does not place a
// workgroup on a CU that holds one of ours, so beside it these workgroups
// run in its launch gaps and tail, and it waits at most one tile for a CU.
// max_wg > 0 caps the grid (workgroups then loop over tiles and keep their
// CUs for the whole call).
unsigned grid_size(const DeviceLimits &lim, int64_t ntiles, uint32_t flags, int32_t max_wg) {
    int64_t g;
    if (flags & TIDE_F_SMALL_FOOTPRINT)
        g = !TIDE_SMALL_PERSISTENT ? ntiles
            : lim.small_lds        ? static_cast<int64_t>(lim.cus) * TIDE_SMALL_WG_PER_CU
                                   : kSmallFootprintWg;
    else if (TIDE_DEFAULT_ONE_TILE_PER_WG)
        g = ntiles;
    else
        g = static_cast<int64_t>(lim.cus) * kWgPerCu;
    if (max_wg > 0) g = max_wg;
    g = std::min<int64_t>({g, ntiles, 0x7fffffff});
    return static_cast<unsigned>(std::max<int64_t>(g, 1));
}

// Waits, before the plan's device tables are freed, for every launch that
// may read them: the events of every stream that read one of the plan's
// pointer-table slots on this device.  Launches captured into a graph
// record no event; while a slot is held by a captured launch (or a read went
// unrecorded) the whole device is waited for instead.
void release_device_states(const tide_plan *p) {
    std::lock_guard<std::mutex> lock(p->mu);
    int cur = -1;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (DeviceState *ds : p->devs) {
        if (hipSetDevice(ds->device) == hipSuccess) {
            bool whole_device = false;
            for (auto *cache : {&ds->rs_cache, &ds->ag_cache, &ds->pack_cache, &ds->slots_cache})
                for (const PtrTable &pt : *cache) whole_device |= pt.pinned || pt.untracked;
            if (whole_device) {
                (void)hipDeviceSynchronize();
            } else {
                for (auto *cache :
                     {&ds->rs_cache, &ds->ag_cache, &ds->pack_cache, &ds->slots_cache})
                    for (const PtrTable &pt : *cache)
                        for (const SlotReader &r : pt.readers)
                            (void)hipEventSynchronize(static_cast<hipEvent_t>(r.event));
            }
        }
        free_state(ds);
    }
    p->devs.clear();
    if (have_cur) (void)hipSetDevice(cur);
}

}  // namespace tide

using tide::fail;

extern "C" tide_status tide_rs(const tide_plan *plan, int32_t rank, const void *const *grads,
                               void *out, uint32_t flags, int32_t max_workgroups,
                               void *stream) {
    tide_status st = tide::check_rs_args(plan, rank, grads, out, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->S == 0) return TIDE_OK;

    // The kernel reads the table parameter-major (entry i*N + r), followed by
    // kPtrPad null entries so that a batch's pointers load in one scalar load.
    const int32_t N = plan->N, P = plan->P;
    const tide::PtrKey key{reinterpret_cast<const uintptr_t *>(grads),
                           static_cast<size_t>(N) * P, nullptr, 0};
    auto param_major = [N, P](const uintptr_t *k, uintptr_t *dev) {
        for (int32_t r = 0; r < N; r++)
            for (int32_t i = 0; i < P; i++)
                dev[static_cast<size_t>(i) * N + r] = k[static_cast<size_t>(r) * P + i];
    };

    bool capturing = false;
    st = tide::capture_status(stream, &capturing);
    if (st != TIDE_OK) return st;
    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, capturing, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->rs_cache, key, key.size() + tide::kPtrPad, param_major,
                             static_cast<hipStream_t>(stream), capturing, &pt);
    if (st != TIDE_OK) return st;

    const tide::RsShape shape = tide::rs_shape(plan, ds, flags);
    const tide::RsLaunch L{static_cast<const tide::ParamDesc *>(ds->d_params),
                           shape.tiles,
                           shape.ntiles,
                           static_cast<const char *const *>(pt->dev),
                           plan->N,
                           rank,
                           tide::avg_mode(plan->N, (flags & TIDE_F_AVG) != 0),
                           out,
                           pt->aligned16 ? 1 : 0,
                           (reinterpret_cast<uintptr_t>(out) & 15) == 0 ? 1 : 0,
                           tide::grid_size(ds->lim, shape.ntiles, flags, max_workgroups),
                           shape.lds,
                           static_cast<hipStream_t>(stream)};
    const tide::GradType type = (flags & TIDE_F_GRAD_F32)   ? tide::kF32
                                : (flags & TIDE_F_GRAD_F16) ? tide::kF16
                                                            : tide::kBf16;
    const tide::OutType otype = (flags & TIDE_F_OUT_BF16) ? tide::kOutBf16 : tide::kOutF32;
    hipError_t e = tide::launch_rs(L, type, otype, shape.shape);
    if (e != hipSuccess) return tide::hip_fail("tide_rs: kernel launch", e);
    st = tide::after_launch(pt, static_cast<hipStream_t>(stream), capturing);
    if (st != TIDE_OK) return st;
    tide::clear_error();
    return TIDE_OK;
}

namespace tide {
namespace {

// TIDE-AG placement with the SDMA engines: the same (parameter, rank) runs as
// the kernel copies, each as one device-to-device copy of the no-CU kind,
// which the HIP runtime hands to an SDMA engine.  Only 1-D copies: a 2-D
// copy of that kind runs as a blit kernel on the compute units (a kernel
// trace of it shows one copyBufferRect kernel per parameter), which is what
// this path exists to avoid.  The runtime still moves very small copies
// (around a kilobyte) with a kernel.  Each copy costs tens of microseconds
// of host time to enqueue, so the call returns once all P*N copies are
// queued.
tide_status ag_copy_engine(const tide_plan *p, const void *const *rank_src, void *const *params,
                           int32_t e, hipStream_t stream) {
    const hipMemcpyKind kind = hipMemcpyDeviceToDeviceNoCU;
    const uintptr_t eb = static_cast<uintptr_t>(e);
    for (int32_t i = 0; i < p->P; i++) {
        if (p->numel[i] == 0 || p->seg[i] == 0) continue;
        const uintptr_t off_b = static_cast<uintptr_t>(p->off[i]) * eb;
        char *dst = static_cast<char *>(params[i]);
        for (int32_t r = 0; r < p->N; r++) {
            int64_t src, L;
            shard_run(p, r, i, &src, &L);
            if (L == 0) break;   // the ranks after a short or empty shard hold nothing
            hipError_t err = hipMemcpyAsync(dst + static_cast<uintptr_t>(src) * eb,
                                            static_cast<const char *>(rank_src[r]) + off_b,
                                            static_cast<uintptr_t>(L) * eb, kind, stream);
            if (err != hipSuccess) return hip_fail("tide_ag: copy-engine copy", err);
        }
    }
    return TIDE_OK;
}

}  // namespace
}  // namespace tide

extern "C" tide_status tide_ag(const tide_plan *plan, const void *const *rank_src,
                               void *const *params, int32_t elem_bytes, uint32_t flags,
                               int32_t max_workgroups, void *stream) {
    tide_status st =
        tide::check_ag_args(plan, rank_src, params, elem_bytes, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->ag_tiles.empty()) return TIDE_OK;
    if (flags & TIDE_F_COPY_ENGINE) {
        st = tide::ag_copy_engine(plan, rank_src, params, elem_bytes,
                                  static_cast<hipStream_t>(stream));
        if (st == TIDE_OK) tide::clear_error();
        return st;
    }

    // Table: the N rank block pointers, then the P parameter pointers.
    const tide::PtrKey key{reinterpret_cast<const uintptr_t *>(rank_src),
                           static_cast<size_t>(plan->N),
                           reinterpret_cast<const uintptr_t *>(params),
                           static_cast<size_t>(plan->P)};
    const size_t n = key.size();
    auto as_is = [n](const uintptr_t *k, uintptr_t *dev) { std::copy(k, k + n, dev); };

    bool capturing = false;
    st = tide::capture_status(stream, &capturing);
    if (st != TIDE_OK) return st;
    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, capturing, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->ag_cache, key, n, as_is, static_cast<hipStream_t>(stream),
                             capturing, &pt);
    if (st != TIDE_OK) return st;

    const bool small = (flags & TIDE_F_SMALL_FOOTPRINT) != 0;
    const int64_t ntiles =
        static_cast<int64_t>(small ? plan->ag_tiles_small.size() : plan->ag_tiles.size());
    const tide::AgLaunch L{static_cast<const tide::ParamDesc *>(ds->d_params),
                           static_cast<const tide::Tile *>(small ? ds->d_ag_tiles_small
                                                                 : ds->d_ag_tiles),
                           ntiles,
                           static_cast<const uintptr_t *>(pt->dev),
                           plan->N,
                           elem_bytes,
                           tide::grid_size(ds->lim, ntiles, flags, max_workgroups),
                           small ? ds->lim.small_lds : ds->lim.ag_cap_lds,
                           static_cast<hipStream_t>(stream)};
    hipError_t e = tide::launch_ag(L, small);
    if (e != hipSuccess) return tide::hip_fail("tide_ag: kernel launch", e);
    st = tide::after_launch(pt, static_cast<hipStream_t>(stream), capturing);
    if (st != TIDE_OK) return st;
    tide::clear_error();
    return TIDE_OK;
}

extern "C" tide_status tide_pack(const tide_plan *plan, const void *const *tensors, void *slot,
                                 int32_t elem_bytes, uint32_t flags, int32_t max_workgroups,
                                 void *stream) {
    tide_status st =
        tide::check_pack_args(plan, tensors, slot, elem_bytes, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->pack_tiles.empty()) return TIDE_OK;

    // Table: the P tensor pointers, then the slot.
    const uintptr_t slot_key[1] = {reinterpret_cast<uintptr_t>(slot)};
    const tide::PtrKey key{reinterpret_cast<const uintptr_t *>(tensors),
                           static_cast<size_t>(plan->P), slot_key, 1};
    const size_t n = key.size();
    const int32_t P = plan->P;
    auto order = [P](const uintptr_t *k, uintptr_t *dev) {
        std::copy(k, k + P + 1, dev);
    };

    bool capturing = false;
    st = tide::capture_status(stream, &capturing);
    if (st != TIDE_OK) return st;
    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, capturing, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->pack_cache, key, n, order, static_cast<hipStream_t>(stream),
                             capturing, &pt);
    if (st != TIDE_OK) return st;

    const bool small = (flags & TIDE_F_SMALL_FOOTPRINT) != 0;
    const int64_t ntiles =
        static_cast<int64_t>(small ? plan->pack_tiles_small.size() : plan->pack_tiles.size());
    const tide::PackLaunch L{static_cast<const tide::ParamDesc *>(ds->d_params),
                             static_cast<const tide::Tile *>(small ? ds->d_pack_tiles_small
                                                                   : ds->d_pack_tiles),
                             ntiles,
                             static_cast<const uintptr_t *>(pt->dev),
                             plan->P,
                             elem_bytes,
                             plan->S,
                             tide::grid_size(ds->lim, ntiles, flags, max_workgroups),
                             small ? ds->lim.small_lds : ds->lim.ag_cap_lds,
                             static_cast<hipStream_t>(stream)};
    hipError_t e = tide::launch_pack(L, small);
    if (e != hipSuccess) return tide::hip_fail("tide_pack: kernel launch", e);
    st = tide::after_launch(pt, static_cast<hipStream_t>(stream), capturing);
    if (st != TIDE_OK) return st;
    tide::clear_error();
    return TIDE_OK;
}

extern "C" tide_status tide_rs_slots(const tide_plan *plan, int32_t rank,
                                     const void *const *slots, void *out, uint32_t flags,
                                     int32_t max_workgroups, void *stream) {
    tide_status st = tide::check_rs_slots_args(plan, rank, slots, out, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->S == 0) return TIDE_OK;

    // The reduce-scatter kernel reads rank r's elements of parameter i at
    // table[i*N + r] + (src(R,i) + k) * es.  Pointing that entry at
    //   slots[r] + (R*S + off_i - src(R,i)) * es
    // makes it read slot r's block R at off_i + k: the staged copy of the
    // same element.  (R*S + off_i >= R*seg_i, so the entry stays inside the
    // slot.)  The key holds the slot pointers, R and the element size.
    const int32_t N = plan->N, P = plan->P;
    const uintptr_t es = (flags & TIDE_F_GRAD_F32) ? 4u : 2u;
    const uintptr_t extra[2] = {static_cast<uintptr_t>(rank), es};
    const tide::PtrKey key{reinterpret_cast<const uintptr_t *>(slots), static_cast<size_t>(N),
                           extra, 2};
    const int64_t S = plan->S;
    const std::vector<int64_t> &off = plan->off, &seg = plan->seg;
    auto synth = [N, P, rank, es, S, &off, &seg](const uintptr_t *k, uintptr_t *dev) {
        for (int32_t i = 0; i < P; i++) {
            const int64_t rel = static_cast<int64_t>(rank) * S + off[i] -
                                static_cast<int64_t>(rank) * seg[i];
            for (int32_t r = 0; r < N; r++)
                dev[static_cast<size_t>(i) * N + r] = k[r] + static_cast<uintptr_t>(rel) * es;
        }
    };

    bool capturing = false;
    st = tide::capture_status(stream, &capturing);
    if (st != TIDE_OK) return st;
    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, capturing, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->slots_cache, key,
                             static_cast<size_t>(N) * P + tide::kPtrPad, synth,
                             static_cast<hipStream_t>(stream), capturing, &pt);
    if (st != TIDE_OK) return st;

    const tide::RsShape shape = tide::rs_shape(plan, ds, flags);
    const tide::RsLaunch L{static_cast<const tide::ParamDesc *>(ds->d_params),
                           shape.tiles,
                           shape.ntiles,
                           static_cast<const char *const *>(pt->dev),
                           N,
                           rank,
                           tide::avg_mode(plan->N, (flags & TIDE_F_AVG) != 0),
                           out,
                           pt->aligned16 ? 1 : 0,
                           (reinterpret_cast<uintptr_t>(out) & 15) == 0 ? 1 : 0,
                           tide::grid_size(ds->lim, shape.ntiles, flags, max_workgroups),
                           shape.lds,
                           static_cast<hipStream_t>(stream)};
    const tide::GradType type = (flags & TIDE_F_GRAD_F32)   ? tide::kF32
                                : (flags & TIDE_F_GRAD_F16) ? tide::kF16
                                                            : tide::kBf16;
    const tide::OutType otype = (flags & TIDE_F_OUT_BF16) ? tide::kOutBf16 : tide::kOutF32;
    hipError_t e = tide::launch_rs(L, type, otype, shape.shape);
    if (e != hipSuccess) return tide::hip_fail("tide_rs_slots: kernel launch", e);
    st = tide::after_launch(pt, static_cast<hipStream_t>(stream), capturing);
    if (st != TIDE_OK) return st;
    tide::clear_error();
    return TIDE_OK;
}

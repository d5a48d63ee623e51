// TIDE-RS and TIDE-AG placement kernels for CDNA4 (gfx950), and the launch
// paths behind tide_rs / tide_ag.
//
// Both operations stream HBM with almost no arithmetic (under half a flop
// per byte), so the design goal is bytes in flight, not ALU: 16-byte global
// loads and stores from wave64 lanes, per-tile descriptors read with scalar
// loads, non-temporal hints on data that is touched once, and persistent
// workgroups that walk a host-built tile list.
//
// TIDE-RS ("FSDP通信终局：TIDE零拷贝集合通信优化" §"TIDE的设计思路"): the
// per-parameter bf16 gradients of N ranks are read where they lie and
// reduced to this rank's fp32 shard, written straight into its block of the
// flat rank-major buffer; stock FSDP2 first packs them into a full fp32
// buffer (§"FSDP2通信开销的根源"), a copy this path never makes.
// TIDE-AG: shards are placed straight into parameter storage, removing the
// copy-out pass after the all-gather.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>

#include "internal.h"

namespace tide {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pointers the kernels fetch from tables are generic; casting them to the
// global address space lets the compiler emit global_load/store with a
// scalar (wave-uniform) base and a 32-bit per-lane offset instead of flat
// accesses.
#define GLOBAL_AS __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const GLOBAL_AS T *gload_ptr(const void *p) {
    return (const GLOBAL_AS T *)p;
}
template <class T>
__device__ __forceinline__ GLOBAL_AS T *gstore_ptr(void *p) {
    return (GLOBAL_AS T *)p;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t *p) {
    return __uint_as_float(static_cast<uint32_t>(*gload_ptr<uint16_t>(p)) << 16);
}

// Scalar path for elements [a, b) of a segment: one lane per element, the
// same rank-order sum as the vector path.
__device__ __forceinline__ void rs_elems(const uint16_t *const *__restrict__ P, int N,
                                         int64_t src, float *__restrict__ o, int64_t a,
                                         int64_t b) {
    for (int64_t k = a + threadIdx.x; k < b; k += kBlock) {
        float acc = bf16_at(P[0] + src + k);
        for (int r = 1; r < N; r++) acc = acc + bf16_at(P[r] + src + k);
        o[k] = acc;
    }
}

// Loads one batch of up to 8 ranks (16 bytes = 8 bf16 per lane and chunk),
// all issued before any add, then adds them in rank order.  FIRST: the batch
// starts at rank 0, whose value initialises the sums.
// `first` = src + (first element of this tile's vector range): a
// wave-uniform element offset; lane_off[j] is each lane's chunk start
// relative to it, in bytes (< 32 bits).
template <int CPL, bool FIRST>
__device__ __forceinline__ void rs_batch(const uint16_t *const *__restrict__ P, int r0, int nb,
                                         int64_t first, const uint32_t *lane_off, f32x4 *a0,
                                         f32x4 *a1) {
    u32x4 v[8][CPL];
#pragma unroll
    for (int q = 0; q < 8; q++) {
        if (q < nb) {
            const GLOBAL_AS char *base = gload_ptr<char>(P[r0 + q] + first);
#pragma unroll
            for (int j = 0; j < CPL; j++)
                v[q][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const GLOBAL_AS u32x4 *>(base + lane_off[j]));
        }
    }
#pragma unroll
    for (int q = 0; q < 8; q++) {
        if (q < nb) {
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                const u32x4 w = v[q][j];
                const f32x4 x0 = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
                const f32x4 x1 = {bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
                if (FIRST && q == 0) {
                    a0[j] = x0;
                    a1[j] = x1;
                } else {
                    a0[j] = a0[j] + x0;
                    a1[j] = a1[j] + x1;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// TIDE-RS kernel
// ---------------------------------------------------------------------------
//
// Tile t covers elements [k0, k0 + kRsTile) of parameter i's span in the
// rank block (its segment plus any alignment gap after it).  For rank R:
//   k <  L(R,i):  out[off_i + k] = sum_{r=0..N-1} widen(G[r][i][R*seg_i + k])
//   k >= L(R,i):  out[off_i + k] = +0.0f   (padding rows, alignment gap)
// ptrs is param-major: ptrs[i*N + r] = G[r][i].
//
// vec_in: every gradient pointer is 16-byte aligned, so lanes take chunks of
// 8 elements whose source address is 16-byte aligned (k + src = 0 mod 8);
// the few elements before the first and after the last chunk of a tile take
// the scalar path.  vec_out: `out` is 16-byte aligned; a chunk is stored as
// two 16-byte stores when its output offset is a multiple of 4 too.
template <int CPL>
__global__ __launch_bounds__(kBlock) void rs_kernel(const ParamDesc *__restrict__ pdesc,
                                                    const Tile *__restrict__ tiles,
                                                    int64_t ntiles,
                                                    const uint16_t *const *__restrict__ ptrs,
                                                    int N, int R, float *__restrict__ out,
                                                    int vec_in, int vec_out) {
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const Tile tile = tiles[t];
        const ParamDesc d = pdesc[tile.param];
        const int64_t src = static_cast<int64_t>(R) * d.seg;
        int64_t L = d.numel - src;
        L = L < 0 ? 0 : (L > d.seg ? d.seg : L);
        const int64_t kb = tile.k0;
        const int64_t ke = min(kb + kRsTile, d.span);
        const int64_t re = min(ke, L);
        float *__restrict__ o = out + d.off;
        const uint16_t *const *__restrict__ P = ptrs + static_cast<int64_t>(tile.param) * N;

        if (kb < re) {
            int64_t vs = re, ve = re;
            if (vec_in) {
                vs = min(re, kb + ((8 - ((src + kb) & 7)) & 7));
                ve = vs + ((re - vs) & ~static_cast<int64_t>(7));
            }
            rs_elems(P, N, src, o, kb, vs);
            rs_elems(P, N, src, o, ve, re);

            // A tile holds at most kRsTile/8 chunks, so every per-lane byte
            // offset below fits in 32 bits.
            const int nch = static_cast<int>((ve - vs) >> 3);
            const bool st16 = vec_out && (((d.off + vs) & 3) == 0);
            GLOBAL_AS char *obase = gstore_ptr<char>(o + vs);
            for (int c0 = 0; c0 < nch; c0 += kBlock * CPL) {
                uint32_t in_off[CPL], out_off[CPL];
                bool ok[CPL];
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    const int ch = c0 + j * kBlock + static_cast<int>(threadIdx.x);
                    ok[j] = ch < nch;
                    // Lanes past the end re-read the last chunk (in bounds)
                    // and do not store.
                    const uint32_t c = static_cast<uint32_t>(ok[j] ? ch : nch - 1);
                    in_off[j] = c * 16u;     // 8 bf16
                    out_off[j] = c * 32u;    // 8 fp32
                }
                f32x4 a0[CPL], a1[CPL];
                rs_batch<CPL, true>(P, 0, min(N, 8), src + vs, in_off, a0, a1);
                for (int r0 = 8; r0 < N; r0 += 8)
                    rs_batch<CPL, false>(P, r0, min(N - r0, 8), src + vs, in_off, a0, a1);
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    if (!ok[j]) continue;
                    if (st16) {
                        GLOBAL_AS f32x4 *dst =
                            reinterpret_cast<GLOBAL_AS f32x4 *>(obase + out_off[j]);
                        __builtin_nontemporal_store(a0[j], dst);
                        __builtin_nontemporal_store(a1[j], dst + 1);
                    } else {
                        GLOBAL_AS float *dst = reinterpret_cast<GLOBAL_AS float *>(obase + out_off[j]);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            dst[e] = a0[j][e];
                            dst[4 + e] = a1[j][e];
                        }
                    }
                }
            }
        }
        for (int64_t k = max(kb, L) + threadIdx.x; k < ke; k += kBlock) o[k] = 0.0f;
    }
}

// ---------------------------------------------------------------------------
// TIDE-AG kernel
// ---------------------------------------------------------------------------

template <int W> struct VecOf;
template <> struct VecOf<16> { typedef u32x4 type; };
template <> struct VecOf<8> { typedef u32x2 type; };
template <> struct VecOf<4> { typedef uint32_t type; };
template <> struct VecOf<2> { typedef uint16_t type; };

// Copies bytes [a, b) of a span element by element (e = 2 or 4 bytes).
__device__ __forceinline__ void copy_elems(const char *s, char *d, int a, int b, int e) {
    const GLOBAL_AS char *gs = gload_ptr<char>(s);
    GLOBAL_AS char *gd = gstore_ptr<char>(d);
    if (e == 2) {
        for (int x = a + 2 * static_cast<int>(threadIdx.x); x < b; x += 2 * kBlock)
            *reinterpret_cast<GLOBAL_AS uint16_t *>(gd + x) =
                *reinterpret_cast<const GLOBAL_AS uint16_t *>(gs + x);
    } else {
        for (int x = a + 4 * static_cast<int>(threadIdx.x); x < b; x += 4 * kBlock)
            *reinterpret_cast<GLOBAL_AS uint32_t *>(gd + x) =
                *reinterpret_cast<const GLOBAL_AS uint32_t *>(gs + x);
    }
}

// Copies n bytes from s to d where s = d (mod W): element-wise up to the
// first W-aligned destination byte, W-byte vectors (U per lane in flight),
// element-wise tail.
// n is at most kAgTile * 4 bytes, so lane offsets fit in 32 bits.
template <int W, int U>
__device__ __forceinline__ void copy_span_w(const char *s, char *d, int n, int e) {
    typedef typename VecOf<W>::type V;
    const int h = min(n, static_cast<int>((W - (reinterpret_cast<uintptr_t>(d) & (W - 1))) &
                                          (W - 1)));
    copy_elems(s, d, 0, h, e);
    const int nv = (n - h) / W;
    const GLOBAL_AS V *vs = gload_ptr<V>(s + h);
    GLOBAL_AS V *vd = gstore_ptr<V>(d + h);
    for (int b = 0; b < nv; b += kBlock * U) {
        V v[U];
#pragma unroll
        for (int j = 0; j < U; j++) {
            const int i = b + j * kBlock + static_cast<int>(threadIdx.x);
            if (i < nv) v[j] = __builtin_nontemporal_load(vs + i);
        }
#pragma unroll
        for (int j = 0; j < U; j++) {
            const int i = b + j * kBlock + static_cast<int>(threadIdx.x);
            if (i < nv) __builtin_nontemporal_store(v[j], vd + i);
        }
    }
    copy_elems(s, d, h + nv * W, n, e);
}

// Tile t covers elements [k0, k0 + kAgTile) of rank r's shard of parameter
// i: they move from rank_src[r] + off_i + k to params[i] + r*seg_i + k.
// ptrs = rank_src[0..N) followed by params[0..P).
template <int U>
__global__ __launch_bounds__(kBlock) void ag_kernel(const ParamDesc *__restrict__ pdesc,
                                                    const Tile *__restrict__ tiles,
                                                    int64_t ntiles,
                                                    const uintptr_t *__restrict__ ptrs, int N,
                                                    int e) {
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const Tile tile = tiles[t];
        const ParamDesc d = pdesc[tile.param];
        const int64_t src = static_cast<int64_t>(tile.rank) * d.seg;
        int64_t L = d.numel - src;
        L = L < 0 ? 0 : (L > d.seg ? d.seg : L);
        const int64_t len = min(kAgTile, L - tile.k0);
        const char *s = reinterpret_cast<const char *>(ptrs[tile.rank]) + (d.off + tile.k0) * e;
        char *dst = reinterpret_cast<char *>(ptrs[N + tile.param]) + (src + tile.k0) * e;
        const int n = static_cast<int>(len * e);
        const uintptr_t diff = reinterpret_cast<uintptr_t>(s) ^ reinterpret_cast<uintptr_t>(dst);
        if ((diff & 15) == 0)
            copy_span_w<16, U>(s, dst, n, e);
        else if ((diff & 7) == 0)
            copy_span_w<8, U>(s, dst, n, e);
        else if ((diff & 3) == 0)
            copy_span_w<4, U>(s, dst, n, e);
        else
            copy_span_w<2, U>(s, dst, n, e);
    }
}

// ---------------------------------------------------------------------------
// Host side: per-device tables, pointer-table cache, launch policy
// ---------------------------------------------------------------------------

constexpr int kRsChunksPerLane = 2;
constexpr int kAgVecsPerLane = 4;
constexpr int kWgPerCu = 8;           // default grid: enough waves to keep HBM busy
constexpr int kSmallFootprintWg = 32; // small-footprint grid (4 per XCD)

tide_status hip_fail(const char *what, hipError_t e) {
    return fail(TIDE_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

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
    for (auto &pt : ds->rs_cache) (void)hipFree(pt.dev);
    for (auto &pt : ds->ag_cache) (void)hipFree(pt.dev);
    delete ds;
}

// The plan's tables on the current device (created on first use).
// Caller holds p->mu.
tide_status device_state(const tide_plan *p, DeviceState **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    for (DeviceState *ds : p->devs)
        if (ds->device == dev) {
            *out = ds;
            return TIDE_OK;
        }
    DeviceState *ds = new (std::nothrow) DeviceState;
    if (!ds) return fail(TIDE_E_NOMEM, "device state: out of host memory");
    ds->device = dev;
    e = hipDeviceGetAttribute(&ds->cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) {
        delete ds;
        return hip_fail("hipDeviceGetAttribute", e);
    }
    tide_status st = upload(p->desc.data(), p->desc.size() * sizeof(ParamDesc), &ds->d_params,
                            "parameter table");
    if (st == TIDE_OK)
        st = upload(p->rs_tiles.data(), p->rs_tiles.size() * sizeof(Tile), &ds->d_rs_tiles,
                    "reduce-scatter tiles");
    if (st == TIDE_OK)
        st = upload(p->ag_tiles.data(), p->ag_tiles.size() * sizeof(Tile), &ds->d_ag_tiles,
                    "all-gather tiles");
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

uint64_t hash_ptrs(const uintptr_t *v, size_t n) {
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < n; i++) {
        h ^= static_cast<uint64_t>(v[i]);
        h *= 1099511628211ull;
    }
    return h;
}

// Finds (or uploads) the device copy of a pointer array.  `dev_order` is
// the array as the kernel wants it (it may be a permutation of `key`).
// Caller holds p->mu.
tide_status pointer_table(DeviceState *ds, std::vector<PtrTable> &cache,
                          const std::vector<uintptr_t> &key,
                          const std::vector<uintptr_t> &dev_order, PtrTable **out) {
    const uint64_t h = hash_ptrs(key.data(), key.size());
    for (auto &pt : cache)
        if (pt.hash == h && pt.key == key) {
            pt.last_use = ++ds->tick;
            *out = &pt;
            return TIDE_OK;
        }
    if (cache.size() >= kPtrCacheEntries) {
        // Evict the least recently used table once no kernel can still read it.
        auto lru = std::min_element(cache.begin(), cache.end(),
                                    [](const PtrTable &a, const PtrTable &b) {
                                        return a.last_use < b.last_use;
                                    });
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail("hipDeviceSynchronize (pointer-table eviction)", e);
        (void)hipFree(lru->dev);
        cache.erase(lru);
    }
    PtrTable pt;
    try {
        pt.key = key;
    } catch (const std::bad_alloc &) {
        return fail(TIDE_E_NOMEM, "pointer table: out of host memory");
    }
    pt.hash = h;
    pt.aligned16 = true;
    for (uintptr_t a : key) pt.aligned16 = pt.aligned16 && (a & 15) == 0;
    tide_status st = upload(dev_order.data(), dev_order.size() * sizeof(uintptr_t), &pt.dev,
                            "pointer table");
    if (st != TIDE_OK) return st;
    pt.last_use = ++ds->tick;
    try {
        cache.push_back(std::move(pt));
    } catch (const std::bad_alloc &) {
        (void)hipFree(pt.dev);
        return fail(TIDE_E_NOMEM, "pointer table: out of host memory");
    }
    *out = &cache.back();
    return TIDE_OK;
}

unsigned grid_size(const DeviceState *ds, int64_t ntiles, uint32_t flags, int32_t max_wg) {
    int64_t g = (flags & TIDE_F_SMALL_FOOTPRINT) ? kSmallFootprintWg
                                                 : static_cast<int64_t>(ds->cus) * kWgPerCu;
    if (max_wg > 0) g = max_wg;
    g = std::min(g, ntiles);
    return static_cast<unsigned>(std::max<int64_t>(g, 1));
}

}  // namespace

void release_device_states(const tide_plan *p) {
    std::lock_guard<std::mutex> lock(p->mu);
    int cur = -1;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (DeviceState *ds : p->devs) {
        if (hipSetDevice(ds->device) == hipSuccess) (void)hipDeviceSynchronize();
        free_state(ds);
    }
    p->devs.clear();
    if (have_cur) (void)hipSetDevice(cur);
}

}  // namespace tide

using tide::fail;

extern "C" tide_status tide_rs(const tide_plan *plan, int32_t rank, const void *const *grads,
                               float *out, uint32_t flags, int32_t max_workgroups,
                               void *stream) {
    tide_status st = tide::check_rs_args(plan, rank, grads, out, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->S == 0) return TIDE_OK;

    const size_t n = static_cast<size_t>(plan->N) * plan->P;
    std::vector<uintptr_t> key, dev_order;
    try {
        key.assign(reinterpret_cast<const uintptr_t *>(grads),
                   reinterpret_cast<const uintptr_t *>(grads) + n);
        dev_order.resize(n);
    } catch (const std::bad_alloc &) {
        return fail(TIDE_E_NOMEM, "tide_rs: out of host memory");
    }
    for (int32_t r = 0; r < plan->N; r++)
        for (int32_t i = 0; i < plan->P; i++)
            dev_order[static_cast<size_t>(i) * plan->N + r] = key[static_cast<size_t>(r) * plan->P + i];

    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->rs_cache, key, dev_order, &pt);
    if (st != TIDE_OK) return st;

    const int64_t ntiles = static_cast<int64_t>(plan->rs_tiles.size());
    const unsigned grid = tide::grid_size(ds, ntiles, flags, max_workgroups);
    const int vec_in = pt->aligned16 ? 1 : 0;
    const int vec_out = (reinterpret_cast<uintptr_t>(out) & 15) == 0 ? 1 : 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL(tide::rs_kernel<tide::kRsChunksPerLane>, dim3(grid), dim3(tide::kBlock), 0,
                       static_cast<hipStream_t>(stream),
                       static_cast<const tide::ParamDesc *>(ds->d_params),
                       static_cast<const tide::Tile *>(ds->d_rs_tiles), ntiles,
                       static_cast<const uint16_t *const *>(pt->dev), plan->N, rank, out, vec_in,
                       vec_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tide::hip_fail("tide_rs: kernel launch", e);
    tide::clear_error();
    return TIDE_OK;
}

extern "C" tide_status tide_ag(const tide_plan *plan, const void *const *rank_src,
                               void *const *params, int32_t elem_bytes, uint32_t flags,
                               int32_t max_workgroups, void *stream) {
    tide_status st =
        tide::check_ag_args(plan, rank_src, params, elem_bytes, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->ag_tiles.empty()) return TIDE_OK;

    std::vector<uintptr_t> key;
    try {
        key.reserve(static_cast<size_t>(plan->N) + plan->P);
        for (int32_t r = 0; r < plan->N; r++) key.push_back(reinterpret_cast<uintptr_t>(rank_src[r]));
        for (int32_t i = 0; i < plan->P; i++) key.push_back(reinterpret_cast<uintptr_t>(params[i]));
    } catch (const std::bad_alloc &) {
        return fail(TIDE_E_NOMEM, "tide_ag: out of host memory");
    }

    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->ag_cache, key, key, &pt);
    if (st != TIDE_OK) return st;

    const int64_t ntiles = static_cast<int64_t>(plan->ag_tiles.size());
    const unsigned grid = tide::grid_size(ds, ntiles, flags, max_workgroups);
    (void)hipGetLastError();
    hipLaunchKernelGGL(tide::ag_kernel<tide::kAgVecsPerLane>, dim3(grid), dim3(tide::kBlock), 0,
                       static_cast<hipStream_t>(stream),
                       static_cast<const tide::ParamDesc *>(ds->d_params),
                       static_cast<const tide::Tile *>(ds->d_ag_tiles), ntiles,
                       static_cast<const uintptr_t *>(pt->dev), plan->N, elem_bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tide::hip_fail("tide_ag: kernel launch", e);
    tide::clear_error();
    return TIDE_OK;
}

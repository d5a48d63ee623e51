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

#ifndef TIDE_NT_LOAD
#define TIDE_NT_LOAD 1
#endif
#ifndef TIDE_NT_STORE
#define TIDE_NT_STORE 1
#endif

// Streaming loads and stores: data touched once carries the non-temporal
// hint so it does not push a concurrent kernel's working set out of cache.
template <class V>
__device__ __forceinline__ V stream_load(const GLOBAL_AS V *p) {
#if TIDE_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
template <class V>
__device__ __forceinline__ void stream_store(V v, GLOBAL_AS V *p) {
#if TIDE_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// Gradient element types.  Each widens exactly to fp32: bf16 is the top
// half of an fp32 pattern, every fp16 value is an fp32 value, fp32 is kept.
enum GradType { kBf16 = 0, kF16 = 1, kF32 = 2 };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

// Per type: element bytes, the vector holding 4 consecutive elements, and
// the exact widening of such a vector and of one element.  (In a word of
// two 16-bit elements the lower address sits in the low half.)
template <int IT> struct Grad;
template <> struct Grad<kBf16> {
    static constexpr int ES = 2;
    typedef u32x2 V4;
    static __device__ __forceinline__ f32x4 widen(V4 v) {
        return f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
    }
    static __device__ __forceinline__ float one(const GLOBAL_AS char *p) {
        return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const GLOBAL_AS uint16_t *>(p))
                               << 16);
    }
};
template <> struct Grad<kF16> {
    static constexpr int ES = 2;
    typedef u32x2 V4;
    static __device__ __forceinline__ f32x4 widen(V4 v) {
        return f32x4{f16_to_f32(v.x & 0xffffu), f16_to_f32(v.x >> 16), f16_to_f32(v.y & 0xffffu),
                     f16_to_f32(v.y >> 16)};
    }
    static __device__ __forceinline__ float one(const GLOBAL_AS char *p) {
        return f16_to_f32(*reinterpret_cast<const GLOBAL_AS uint16_t *>(p));
    }
};
template <> struct Grad<kF32> {
    static constexpr int ES = 4;
    typedef u32x4 V4;
    static __device__ __forceinline__ f32x4 widen(V4 v) {
        return f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w)};
    }
    static __device__ __forceinline__ float one(const GLOBAL_AS char *p) {
        return *reinterpret_cast<const GLOBAL_AS float *>(p);
    }
};

// Scalar path for elements [a, b) of a segment: one lane per element, the
// same rank-order sum (and mean) as the vector path.  P[r] is rank r's
// gradient; src is rank R's first element in it.
template <int IT, int BLOCK>
__device__ __forceinline__ void rs_elems(const char *const *__restrict__ P, int N, int avg,
                                         int64_t src, float *__restrict__ o, int64_t a,
                                         int64_t b) {
    typedef Grad<IT> G;
    for (int64_t k = a + threadIdx.x; k < b; k += BLOCK) {
        const int64_t byte = (src + k) * G::ES;
        float acc = G::one(gload_ptr<char>(P[0] + byte));
        for (int r = 1; r < N; r++) acc = acc + G::one(gload_ptr<char>(P[r] + byte));
        if (avg) acc = acc / static_cast<float>(N);
        o[k] = acc;
    }
}

// Loads one batch of up to RB ranks (4 elements per lane and chunk), all
// issued before any add, then adds them in rank order.  FIRST: the batch
// starts at rank 0, whose value initialises the sums.  `first_byte` is the
// wave-uniform byte offset of this tile's vector range in each gradient;
// lane_off[j] is each lane's chunk start relative to it, in bytes.
template <int IT, int CPL, int RB, bool FIRST>
__device__ __forceinline__ void rs_batch(const char *const *__restrict__ P, int r0, int nb,
                                         int64_t first_byte, const uint32_t *lane_off,
                                         f32x4 *acc) {
    typedef Grad<IT> G;
    typedef typename G::V4 V;
    // All RB pointers of the batch in one go (one wide scalar load): the
    // device pointer table carries kPtrPad spare entries after its end, so
    // reading past the last rank of the last parameter stays in bounds.
    // Pointers of ranks >= nb are never dereferenced.
    const char *bp[RB];
#pragma unroll
    for (int q = 0; q < RB; q++) bp[q] = P[r0 + q];
    V v[RB][CPL];
#pragma unroll
    for (int q = 0; q < RB; q++) {
        if (q < nb) {
            const GLOBAL_AS char *base = gload_ptr<char>(bp[q] + first_byte);
#pragma unroll
            for (int j = 0; j < CPL; j++)
                v[q][j] = stream_load(reinterpret_cast<const GLOBAL_AS V *>(base + lane_off[j]));
        }
    }
#pragma unroll
    for (int q = 0; q < RB; q++) {
        if (q < nb) {
#pragma unroll
            for (int j = 0; j < CPL; j++) {
                const f32x4 x = G::widen(v[q][j]);
                if (FIRST && q == 0)
                    acc[j] = x;
                else
                    acc[j] = acc[j] + x;
            }
        }
    }
}

// Workgroup IDs are dealt to the 8 XCDs round-robin (ID mod 8), and each XCD
// has its own L2.  Virtual index v is mapped so that the workgroups of one
// XCD take one contiguous eighth of the tile list: tile-table lines and the
// data of neighbouring tiles are then fetched into one L2, not all eight.
// The map is a bijection on [0, ntiles) for any tile count.
constexpr int64_t kXcds = 8;
__device__ __forceinline__ int64_t xcd_tile(int64_t v, int64_t ntiles) {
    const int64_t q = ntiles / kXcds, rm = ntiles % kXcds;
    const int64_t x = v % kXcds, j = v / kXcds;
    return x * q + (x < rm ? x : rm) + j;
}

// ---------------------------------------------------------------------------
// TIDE-RS kernel
// ---------------------------------------------------------------------------
//
// Tile t covers elements [k0, k0 + TILE) of parameter i's span in the rank
// block (its segment plus any alignment gap after it).  For rank R:
//   k <  L(R,i):  out[off_i + k] = sum_{r=0..N-1} widen(G[r][i][R*seg_i + k])
//                 (divided by N when avg is set)
//   k >= L(R,i):  out[off_i + k] = +0.0f   (padding rows, alignment gap)
// ptrs is param-major: ptrs[i*N + r] = G[r][i].
//
// Lanes take chunks of 4 consecutive elements: 8-byte loads for 16-bit
// gradients, 16-byte loads for fp32 ones.  vec_in: every gradient pointer is
// 16-byte aligned, so chunks start where src + k is a multiple of 4; the few
// elements before the first and after the last chunk of a tile take the
// scalar path.  vec_out: `out` is 16-byte aligned; a chunk's 4 fp32 results
// go out as one 16-byte store when its output offset is a multiple of 4 too,
// so every store instruction of a wave covers one contiguous 1 KiB span.
// PACE > 0 makes each wave sleep between tiles.
template <int IT, int BLOCK, int CPL, int RB, int PACE, bool XMAP, int64_t TILE>
__global__ __launch_bounds__(BLOCK) void rs_kernel(const ParamDesc *__restrict__ pdesc,
                                                   const Tile *__restrict__ tiles,
                                                   int64_t ntiles,
                                                   const char *const *__restrict__ ptrs,
                                                   int N, int R, int avg, float *__restrict__ out,
                                                   int vec_in, int vec_out) {
    constexpr int ES = Grad<IT>::ES;
    for (int64_t v = blockIdx.x; v < ntiles; v += gridDim.x) {
        const Tile tile = tiles[XMAP ? xcd_tile(v, ntiles) : v];
        const ParamDesc d = pdesc[tile.param];
        const int64_t src = static_cast<int64_t>(R) * d.seg;
        int64_t L = d.numel - src;
        L = L < 0 ? 0 : (L > d.seg ? d.seg : L);
        const int64_t kb = tile.k0;
        const int64_t ke = min(kb + TILE, d.span);
        const int64_t re = min(ke, L);
        float *__restrict__ o = out + d.off;
        const char *const *__restrict__ P = ptrs + static_cast<int64_t>(tile.param) * N;

        if (kb < re) {
            int64_t vs = re, ve = re;
            if (vec_in) {
                vs = min(re, kb + ((4 - ((src + kb) & 3)) & 3));
                ve = vs + ((re - vs) & ~static_cast<int64_t>(3));
            }
            rs_elems<IT, BLOCK>(P, N, avg, src, o, kb, vs);
            rs_elems<IT, BLOCK>(P, N, avg, src, o, ve, re);

            // A tile holds at most TILE/4 chunks, so every per-lane byte
            // offset below fits in 32 bits.
            const int nch = static_cast<int>((ve - vs) >> 2);
            const bool st16 = vec_out && (((d.off + vs) & 3) == 0);
            GLOBAL_AS char *obase = gstore_ptr<char>(o + vs);
            for (int c0 = 0; c0 < nch; c0 += BLOCK * CPL) {
                uint32_t in_off[CPL], out_off[CPL];
                bool ok[CPL];
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    const int ch = c0 + j * BLOCK + static_cast<int>(threadIdx.x);
                    ok[j] = ch < nch;
                    // Lanes past the end re-read the last chunk (in bounds)
                    // and do not store.
                    const uint32_t c = static_cast<uint32_t>(ok[j] ? ch : nch - 1);
                    in_off[j] = c * (4u * ES);
                    out_off[j] = c * 16u;
                }
                f32x4 acc[CPL];
                const int64_t first_byte = (src + vs) * ES;
                rs_batch<IT, CPL, RB, true>(P, 0, min(N, RB), first_byte, in_off, acc);
                for (int r0 = RB; r0 < N; r0 += RB)
                    rs_batch<IT, CPL, RB, false>(P, r0, min(N - r0, RB), first_byte, in_off, acc);
                if (avg) {
                    const float n = static_cast<float>(N);
#pragma unroll
                    for (int j = 0; j < CPL; j++)
                        acc[j] = f32x4{acc[j].x / n, acc[j].y / n, acc[j].z / n, acc[j].w / n};
                }
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    if (!ok[j]) continue;
                    if (st16) {
                        stream_store(acc[j], reinterpret_cast<GLOBAL_AS f32x4 *>(obase + out_off[j]));
                    } else {
                        GLOBAL_AS float *dst = reinterpret_cast<GLOBAL_AS float *>(obase + out_off[j]);
#pragma unroll
                        for (int e = 0; e < 4; e++) dst[e] = acc[j][e];
                    }
                }
            }
        }
        for (int64_t k = max(kb, L) + threadIdx.x; k < ke; k += BLOCK) o[k] = 0.0f;
        if (PACE > 0) {
#pragma unroll
            for (int p = 0; p < PACE; p++) __builtin_amdgcn_s_sleep(32);
        }
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
template <int BLOCK>
__device__ __forceinline__ void copy_elems(const char *s, char *d, int a, int b, int e) {
    const GLOBAL_AS char *gs = gload_ptr<char>(s);
    GLOBAL_AS char *gd = gstore_ptr<char>(d);
    if (e == 2) {
        for (int x = a + 2 * static_cast<int>(threadIdx.x); x < b; x += 2 * BLOCK)
            *reinterpret_cast<GLOBAL_AS uint16_t *>(gd + x) =
                *reinterpret_cast<const GLOBAL_AS uint16_t *>(gs + x);
    } else {
        for (int x = a + 4 * static_cast<int>(threadIdx.x); x < b; x += 4 * BLOCK)
            *reinterpret_cast<GLOBAL_AS uint32_t *>(gd + x) =
                *reinterpret_cast<const GLOBAL_AS uint32_t *>(gs + x);
    }
}

// Copies n bytes from s to d where s = d (mod W): element-wise up to the
// first W-aligned destination byte, W-byte vectors (U per lane in flight),
// element-wise tail.
// n is at most one all-gather tile of 4-byte elements, so lane offsets fit in
// 32 bits.
template <int BLOCK, int W, int U>
__device__ __forceinline__ void copy_span_w(const char *s, char *d, int n, int e) {
    typedef typename VecOf<W>::type V;
    const int h = min(n, static_cast<int>((W - (reinterpret_cast<uintptr_t>(d) & (W - 1))) &
                                          (W - 1)));
    copy_elems<BLOCK>(s, d, 0, h, e);
    const int nv = (n - h) / W;
    const GLOBAL_AS V *vs = gload_ptr<V>(s + h);
    GLOBAL_AS V *vd = gstore_ptr<V>(d + h);
    for (int b = 0; b < nv; b += BLOCK * U) {
        V v[U];
#pragma unroll
        for (int j = 0; j < U; j++) {
            const int i = b + j * BLOCK + static_cast<int>(threadIdx.x);
            if (i < nv) v[j] = stream_load(vs + i);
        }
#pragma unroll
        for (int j = 0; j < U; j++) {
            const int i = b + j * BLOCK + static_cast<int>(threadIdx.x);
            if (i < nv) stream_store(v[j], vd + i);
        }
    }
    copy_elems<BLOCK>(s, d, h + nv * W, n, e);
}

// Tile t covers elements [k0, k0 + TILE) of rank r's shard of parameter
// i: they move from rank_src[r] + off_i + k to params[i] + r*seg_i + k.
// ptrs = rank_src[0..N) followed by params[0..P).
template <int BLOCK, int U, int PACE, bool XMAP, int64_t TILE>
__global__ __launch_bounds__(BLOCK) void ag_kernel(const ParamDesc *__restrict__ pdesc,
                                                    const Tile *__restrict__ tiles,
                                                    int64_t ntiles,
                                                    const uintptr_t *__restrict__ ptrs, int N,
                                                    int e) {
    for (int64_t v = blockIdx.x; v < ntiles; v += gridDim.x) {
        const Tile tile = tiles[XMAP ? xcd_tile(v, ntiles) : v];
        const ParamDesc d = pdesc[tile.param];
        const int64_t src = static_cast<int64_t>(tile.rank) * d.seg;
        int64_t L = d.numel - src;
        L = L < 0 ? 0 : (L > d.seg ? d.seg : L);
        const int64_t len = min(TILE, L - tile.k0);
        const char *s = reinterpret_cast<const char *>(ptrs[tile.rank]) + (d.off + tile.k0) * e;
        char *dst = reinterpret_cast<char *>(ptrs[N + tile.param]) + (src + tile.k0) * e;
        const int n = static_cast<int>(len * e);
        const uintptr_t diff = reinterpret_cast<uintptr_t>(s) ^ reinterpret_cast<uintptr_t>(dst);
        if ((diff & 15) == 0)
            copy_span_w<BLOCK, 16, U>(s, dst, n, e);
        else if ((diff & 7) == 0)
            copy_span_w<BLOCK, 8, U>(s, dst, n, e);
        else if ((diff & 3) == 0)
            copy_span_w<BLOCK, 4, U>(s, dst, n, e);
        else
            copy_span_w<BLOCK, 2, U>(s, dst, n, e);
        if (PACE > 0) {
#pragma unroll
            for (int p = 0; p < PACE; p++) __builtin_amdgcn_s_sleep(32);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: per-device tables, pointer-table cache, launch policy
// ---------------------------------------------------------------------------

#ifndef TIDE_RS_CPL
#define TIDE_RS_CPL 4
#endif
#ifndef TIDE_DEFAULT_ONE_TILE_PER_WG
#define TIDE_DEFAULT_ONE_TILE_PER_WG 1
#endif
#ifndef TIDE_SMALL_BLOCK
#define TIDE_SMALL_BLOCK 256
#endif
#ifndef TIDE_SMALL_PACE
#define TIDE_SMALL_PACE 0
#endif
#ifndef TIDE_SMALL_LDS_RESERVE
#define TIDE_SMALL_LDS_RESERVE 1
#endif
#ifndef TIDE_SMALL_WG_PER_CU
#define TIDE_SMALL_WG_PER_CU 1
#endif
#ifndef TIDE_RS_RB
#define TIDE_RS_RB 8
#endif
#ifndef TIDE_SMALL_CPL
#define TIDE_SMALL_CPL 2
#endif
#ifndef TIDE_SMALL_RB
#define TIDE_SMALL_RB 16
#endif
#ifndef TIDE_SMALL_PERSISTENT
#define TIDE_SMALL_PERSISTENT 0
#endif
#ifndef TIDE_XMAP_RS
#define TIDE_XMAP_RS 0
#endif
#ifndef TIDE_SMALL_AG_U
#define TIDE_SMALL_AG_U 8
#endif
#ifndef TIDE_RS_WG_CAP
#define TIDE_RS_WG_CAP 2
#endif
#ifndef TIDE_AG_WG_CAP
#define TIDE_AG_WG_CAP 0
#endif
#ifndef TIDE_XMAP_AG
#define TIDE_XMAP_AG 1
#endif
#ifndef TIDE_AG_U
#define TIDE_AG_U 1
#endif
#ifndef TIDE_WG_PER_CU
#define TIDE_WG_PER_CU 8
#endif
#ifndef TIDE_SMALL_WG
#define TIDE_SMALL_WG 32
#endif
constexpr int kRsChunksPerLane = TIDE_RS_CPL;
// Spare (null) entries after the reduce-scatter pointer table: a batch of RB
// ranks loads its RB pointers unconditionally.
constexpr size_t kPtrPad = 32;
static_assert(TIDE_RS_RB <= static_cast<int>(kPtrPad) && TIDE_SMALL_RB <= static_cast<int>(kPtrPad),
              "rank batch larger than the pointer-table padding");
constexpr int kAgVecsPerLane = TIDE_AG_U;
constexpr int kWgPerCu = TIDE_WG_PER_CU;      // default grid: enough waves to keep HBM busy
constexpr int kSmallFootprintWg = TIDE_SMALL_WG;  // small-footprint grid

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
    (void)hipFree(ds->d_ag_tiles_small);
    (void)hipFree(ds->d_rs_tiles_small);
    for (auto &pt : ds->rs_cache) (void)hipFree(pt.dev);
    for (auto &pt : ds->ag_cache) (void)hipFree(pt.dev);
    delete ds;
}

// LDS that lets exactly `cap` workgroups share a CU (0: no cap).
int lds_for_cap(const DeviceState *ds, int cap) {
    if (cap <= 0 || ds->lds_per_cu <= 0) return 0;
    const int want = ds->lds_per_cu / cap - 1024;
    return (want > 0 && want <= ds->lds_per_wg_max) ? want : 0;
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
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&ds->lds_per_cu,
                                  hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&ds->lds_per_wg_max, hipDeviceAttributeMaxSharedMemoryPerBlock,
                                  dev);
    if (e != hipSuccess) {
        delete ds;
        return hip_fail("hipDeviceGetAttribute", e);
    }
    // A small-footprint workgroup reserves just over half of a CU's LDS, so
    // no two of them share a CU: the hardware dispatcher has to spread them
    // one per CU, and a CU that holds one cannot take two workgroups of an
    // LDS-heavy kernel running beside it.  The reservation is never touched.
    ds->small_lds = 0;
    if (TIDE_SMALL_LDS_RESERVE && ds->lds_per_cu > 0) {
        const int want = ds->lds_per_cu / 2 + 1024;
        if (want <= ds->lds_per_wg_max) ds->small_lds = want;
    }
    // Optional cap on default reduce-scatter workgroups per CU (same trick:
    // an untouched LDS reservation of which exactly TIDE_RS_WG_CAP fit).
    ds->rs_cap_lds = lds_for_cap(ds, TIDE_RS_WG_CAP);
    ds->ag_cap_lds = lds_for_cap(ds, TIDE_AG_WG_CAP);
    tide_status st = upload(p->desc.data(), p->desc.size() * sizeof(ParamDesc), &ds->d_params,
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

// Finds (or uploads) the device copy of a pointer set.  A hit costs one hash
// and one compare over the caller's arrays.  On a miss `order(key, dev)`
// writes the array as the kernel wants it (`dev_len` entries: a permutation
// of the key, possibly padded) and it is uploaded.  Caller holds p->mu.
template <typename Order>
tide_status pointer_table(DeviceState *ds, std::vector<PtrTable> &cache, const PtrKey &key,
                          size_t dev_len, Order order, PtrTable **out) {
    const uint64_t h = hash_ptrs(hash_ptrs(1469598103934665603ull, key.a, key.na), key.b, key.nb);
    for (auto &pt : cache)
        if (pt.hash == h && key.equals(pt.key)) {
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
    std::vector<uintptr_t> dev;
    try {
        pt.key.resize(key.size());
        dev.assign(dev_len, 0);
    } catch (const std::bad_alloc &) {
        return fail(TIDE_E_NOMEM, "pointer table: out of host memory");
    }
    std::copy(key.a, key.a + key.na, pt.key.begin());
    if (key.nb) std::copy(key.b, key.b + key.nb, pt.key.begin() + key.na);
    order(pt.key.data(), dev.data());
    pt.hash = h;
    pt.aligned16 = true;
    for (uintptr_t a : pt.key) pt.aligned16 = pt.aligned16 && (a & 15) == 0;
    tide_status st = upload(dev.data(), dev.size() * sizeof(uintptr_t), &pt.dev, "pointer table");
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

// Both launch modes give every tile its own short-lived workgroup, and the
// hardware dispatcher balances them over all CUs.  Small-footprint launches
// also reserve over half a CU's LDS per workgroup, so at most one of them
// is resident on a CU at any moment: a concurrent GEMM keeps its place on
// every CU and loses only a little issue bandwidth there.  max_wg > 0 caps
// the grid (workgroups then loop over tiles).
unsigned grid_size(const DeviceState *ds, int64_t ntiles, uint32_t flags, int32_t max_wg) {
    int64_t g;
    if (flags & TIDE_F_SMALL_FOOTPRINT)
        g = !TIDE_SMALL_PERSISTENT ? ntiles
            : ds->small_lds        ? static_cast<int64_t>(ds->cus) * TIDE_SMALL_WG_PER_CU
                                   : kSmallFootprintWg;
    else if (TIDE_DEFAULT_ONE_TILE_PER_WG)
        g = ntiles;
    else
        g = static_cast<int64_t>(ds->cus) * kWgPerCu;
    if (max_wg > 0) g = max_wg;
    g = std::min<int64_t>({g, ntiles, 0x7fffffff});
    return static_cast<unsigned>(std::max<int64_t>(g, 1));
}

// Lets `kernel` launch with `bytes` of dynamic LDS (needed above 64 KiB).
tide_status allow_lds(const void *kernel, int bytes) {
    if (bytes <= 65536) return TIDE_OK;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return hip_fail("hipFuncSetAttribute (LDS reservation)", e);
    return TIDE_OK;
}

// Everything one tide_rs launch needs.
struct RsLaunch {
    const ParamDesc *pd;
    const Tile *tiles;
    int64_t ntiles;
    const char *const *ptrs;
    int N, R, avg;
    float *out;
    int vec_in, vec_out;
    unsigned grid;
    int lds;
    hipStream_t stream;
};

// Default launches: one 256-lane workgroup per 4096-element tile, at most
// TIDE_RS_WG_CAP per CU.  Small-footprint launches: the small tile list and
// its kernel shape, at most one workgroup per CU.
template <int IT, bool SMALL>
tide_status launch_rs(const RsLaunch &a) {
    auto k = SMALL ? rs_kernel<IT, TIDE_SMALL_BLOCK, TIDE_SMALL_CPL, TIDE_SMALL_RB, TIDE_SMALL_PACE,
                               TIDE_XMAP_RS, kRsTileSmall>
                   : rs_kernel<IT, kBlock, kRsChunksPerLane, TIDE_RS_RB, 0, TIDE_XMAP_RS, kRsTile>;
    tide_status st = allow_lds(reinterpret_cast<const void *>(k), a.lds);
    if (st != TIDE_OK) return st;
    hipLaunchKernelGGL(k, dim3(a.grid), dim3(SMALL ? TIDE_SMALL_BLOCK : kBlock), a.lds, a.stream,
                       a.pd, a.tiles, a.ntiles, a.ptrs, a.N, a.R, a.avg, a.out, a.vec_in,
                       a.vec_out);
    return TIDE_OK;
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

    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->rs_cache, key, key.size() + tide::kPtrPad, param_major, &pt);
    if (st != TIDE_OK) return st;

    const bool small = (flags & TIDE_F_SMALL_FOOTPRINT) != 0;
    const int64_t ntiles =
        static_cast<int64_t>(small ? plan->rs_tiles_small.size() : plan->rs_tiles.size());
    const tide::RsLaunch L{static_cast<const tide::ParamDesc *>(ds->d_params),
                           static_cast<const tide::Tile *>(small ? ds->d_rs_tiles_small
                                                                 : ds->d_rs_tiles),
                           ntiles,
                           static_cast<const char *const *>(pt->dev),
                           plan->N,
                           rank,
                           (flags & TIDE_F_AVG) ? 1 : 0,
                           out,
                           pt->aligned16 ? 1 : 0,
                           (reinterpret_cast<uintptr_t>(out) & 15) == 0 ? 1 : 0,
                           tide::grid_size(ds, ntiles, flags, max_workgroups),
                           small ? ds->small_lds : ds->rs_cap_lds,
                           static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    if (flags & TIDE_F_GRAD_F32)
        st = small ? tide::launch_rs<tide::kF32, true>(L) : tide::launch_rs<tide::kF32, false>(L);
    else if (flags & TIDE_F_GRAD_F16)
        st = small ? tide::launch_rs<tide::kF16, true>(L) : tide::launch_rs<tide::kF16, false>(L);
    else
        st = small ? tide::launch_rs<tide::kBf16, true>(L) : tide::launch_rs<tide::kBf16, false>(L);
    if (st != TIDE_OK) return st;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tide::hip_fail("tide_rs: kernel launch", e);
    tide::clear_error();
    return TIDE_OK;
}

namespace tide {
namespace {

// TIDE-AG placement with the SDMA engines: the same (parameter, rank) runs as
// the kernel copies, as device-to-device copies that use no compute unit.
// The ranks holding a full shard of parameter i form a prefix 0..F-1; when
// the rank blocks are equally spaced (one gathered buffer) those F runs are
// one 2-D copy: F rows of seg_i elements, source pitch = block spacing,
// destination pitch = seg_i.  The one short rank (if any) is a 1-D copy.
tide_status ag_copy_engine(const tide_plan *p, const void *const *rank_src, void *const *params,
                           int32_t e, hipStream_t stream) {
    const hipMemcpyKind kind = hipMemcpyDeviceToDeviceNoCU;
    const uintptr_t eb = static_cast<uintptr_t>(e);
    bool equal = p->N > 1;
    uintptr_t pitch = 0;
    if (equal) {
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(rank_src[0]);
        const uintptr_t b1 = reinterpret_cast<uintptr_t>(rank_src[1]);
        equal = b1 > b0;
        pitch = b1 - b0;
        for (int32_t r = 2; equal && r < p->N; r++)
            equal = reinterpret_cast<uintptr_t>(rank_src[r]) ==
                    reinterpret_cast<uintptr_t>(rank_src[r - 1]) + pitch;
    }
    for (int32_t i = 0; i < p->P; i++) {
        if (p->numel[i] == 0 || p->seg[i] == 0) continue;
        const uintptr_t seg_b = static_cast<uintptr_t>(p->seg[i]) * eb;
        const uintptr_t off_b = static_cast<uintptr_t>(p->off[i]) * eb;
        char *dst = static_cast<char *>(params[i]);
        int32_t full = 0;
        while (full < p->N) {
            int64_t src, L;
            shard_run(p, full, i, &src, &L);
            if (L != p->seg[i]) break;
            full++;
        }
        hipError_t err = hipSuccess;
        if (equal && full > 1 && pitch >= seg_b) {
            err = hipMemcpy2DAsync(dst, seg_b, static_cast<const char *>(rank_src[0]) + off_b,
                                   pitch, seg_b, static_cast<size_t>(full), kind, stream);
        } else {
            for (int32_t r = 0; r < full && err == hipSuccess; r++)
                err = hipMemcpyAsync(dst + static_cast<uintptr_t>(r) * seg_b,
                                     static_cast<const char *>(rank_src[r]) + off_b, seg_b, kind,
                                     stream);
        }
        if (err == hipSuccess && full < p->N) {
            int64_t src, L;
            shard_run(p, full, i, &src, &L);
            if (L > 0)
                err = hipMemcpyAsync(dst + static_cast<uintptr_t>(src) * eb,
                                     static_cast<const char *>(rank_src[full]) + off_b,
                                     static_cast<uintptr_t>(L) * eb, kind, stream);
        }
        if (err != hipSuccess) return hip_fail("tide_ag: copy-engine copy", err);
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

    std::lock_guard<std::mutex> lock(plan->mu);
    tide::DeviceState *ds = nullptr;
    st = tide::device_state(plan, &ds);
    if (st != TIDE_OK) return st;
    tide::PtrTable *pt = nullptr;
    st = tide::pointer_table(ds, ds->ag_cache, key, n, as_is, &pt);
    if (st != TIDE_OK) return st;

    const bool small = (flags & TIDE_F_SMALL_FOOTPRINT) != 0;
    const int64_t ntiles =
        static_cast<int64_t>(small ? plan->ag_tiles_small.size() : plan->ag_tiles.size());
    const unsigned grid = tide::grid_size(ds, ntiles, flags, max_workgroups);
    (void)hipGetLastError();
    const auto *pd = static_cast<const tide::ParamDesc *>(ds->d_params);
    const auto *pp = static_cast<const uintptr_t *>(pt->dev);
    if (small) {
        auto k = tide::ag_kernel<TIDE_SMALL_BLOCK, TIDE_SMALL_AG_U, TIDE_SMALL_PACE, TIDE_XMAP_AG,
                                 tide::kAgTileSmall>;
        st = tide::allow_lds(reinterpret_cast<const void *>(k), ds->small_lds);
        if (st != TIDE_OK) return st;
        hipLaunchKernelGGL(k, dim3(grid), dim3(TIDE_SMALL_BLOCK), ds->small_lds,
                           static_cast<hipStream_t>(stream), pd,
                           static_cast<const tide::Tile *>(ds->d_ag_tiles_small), ntiles, pp,
                           plan->N, elem_bytes);
    } else {
        auto k = tide::ag_kernel<tide::kBlock, tide::kAgVecsPerLane, 0, TIDE_XMAP_AG, tide::kAgTile>;
        st = tide::allow_lds(reinterpret_cast<const void *>(k), ds->ag_cap_lds);
        if (st != TIDE_OK) return st;
        hipLaunchKernelGGL(k, dim3(grid), dim3(tide::kBlock), ds->ag_cap_lds,
                           static_cast<hipStream_t>(stream), pd,
                           static_cast<const tide::Tile *>(ds->d_ag_tiles), ntiles, pp, plan->N,
                           elem_bytes);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tide::hip_fail("tide_ag: kernel launch", e);
    tide::clear_error();
    return TIDE_OK;
}

// tide_rs_noalloc: TIDE-RS for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  tide_rs keeps the tables its kernel walks - parameter
// descriptors, the tile list and the pointer table - in device memory the
// plan allocates on first use and in a cache of uploaded pointer tables.
// This entry point keeps them instead in one fixed per-device array,
// `scratch`, and rewrites what a call needs there on the call's stream:
//   1. the descriptors, per-parameter tile starts and pointer table, carried
//      as kernel arguments of small copy launches (no host staging buffer
//      and no host-to-device copy);
//   2. the tile list, generated on the device from the tile starts;
//   3. the same reduce-scatter kernel and launch policy as tide_rs, reading
//      the tables from `scratch`.
// The result is bit-identical to tide_rs with the same arguments.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

namespace {

// The per-device working memory.  Each device the library runs on holds its
// own copy until the process ends.  Host code never uses this name as an
// address: it stands for a host-side shadow, so every host-side use goes
// through the device address hipGetSymbolAddress returns for the current
// device.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// 64-bit words copied by one table launch (the words travel as the kernel's
// by-value argument, which stays under the 4 KiB kernel-argument limit).
constexpr int kChunkWords = 448;
struct WordChunk {
    uint64_t w[kChunkWords];
};
static_assert(sizeof(WordChunk) + 16 <= 4096, "table chunk exceeds the kernel-argument limit");

__global__ __launch_bounds__(256) void put_words(uint64_t *__restrict__ dst, int n, WordChunk c) {
    for (int i = static_cast<int>(threadIdx.x); i < n; i += 256) dst[i] = c.w[i];
}

// Tile v of the reduce-scatter tile list: parameter i with
// tstart[i] <= v < tstart[i+1] (tstart[0] = 0, tstart[P] = ntiles), first
// element (v - tstart[i]) * tile of its span.  The same list, in the same
// order, as the plan's own tile list for this tile size.
__global__ __launch_bounds__(256) void make_rs_tiles(tide::Tile *__restrict__ tiles,
                                                     const int64_t *__restrict__ tstart, int P,
                                                     int64_t ntiles, int64_t tile) {
    const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (v >= ntiles) return;
    int lo = 0, hi = P;   // tstart[lo] <= v < tstart[hi]
    while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if (tstart[mid] <= v)
            lo = mid;
        else
            hi = mid;
    }
    tiles[v] = tide::Tile{lo, 0, (v - tstart[lo]) * tile};
}

constexpr int kMaxDevices = 64;

struct ScratchDevice {
    char *ptr = nullptr;   // this device's copy of `scratch`
    tide::DeviceLimits lim;
};

std::mutex g_mu;               // guards g_dev and g_words
ScratchDevice g_dev[kMaxDevices];
// Host image of the tables copied by put_words (descriptors, tile starts,
// pointer table): at most the whole scratch array.
uint64_t g_words[kScratchBytes / sizeof(uint64_t)];

// Byte offsets of the tables inside `scratch` for one call.
struct ScratchLayout {
    size_t desc, tstart, ptrs, tiles, end;
    size_t words;          // 64-bit words before `tiles` (what put_words writes)
    int64_t ntiles;
};

ScratchLayout layout_for(const tide_plan *p, int64_t tile) {
    ScratchLayout L;
    L.ntiles = 0;
    for (int32_t i = 0; i < p->P; i++) L.ntiles += (p->desc[i].span + tile - 1) / tile;
    L.desc = 0;
    L.tstart = L.desc + sizeof(tide::ParamDesc) * static_cast<size_t>(p->P);
    L.ptrs = L.tstart + sizeof(int64_t) * (static_cast<size_t>(p->P) + 1);
    L.words = (L.ptrs + sizeof(uintptr_t) * (static_cast<size_t>(p->N) * p->P + tide::kPtrPad)) /
              sizeof(uint64_t);
    L.tiles = (L.words * sizeof(uint64_t) + 255) / 256 * 256;
    L.end = L.tiles + sizeof(tide::Tile) * static_cast<size_t>(L.ntiles);
    return L;
}

// This device's scratch address and launch limits, looked up on the first
// call on the device.  Caller holds g_mu.
tide_status scratch_device(ScratchDevice **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return tide::hip_fail("tide_rs_noalloc: hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices)
        return tide::fail(TIDE_E_UNSUPPORTED, "tide_rs_noalloc: device index beyond 63");
    ScratchDevice &d = g_dev[dev];
    if (!d.ptr) {
        tide_status st = tide::query_limits(dev, &d.lim);
        if (st != TIDE_OK) return st;
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return tide::hip_fail("tide_rs_noalloc: hipGetSymbolAddress", e);
        if (!ptr) return tide::fail(TIDE_E_HIP, "tide_rs_noalloc: scratch has no device address");
        d.ptr = static_cast<char *>(ptr);
    }
    *out = &d;
    return TIDE_OK;
}

}  // namespace

extern "C" tide_status tide_rs_noalloc(const tide_plan *plan, int32_t rank,
                                       const void *const *grads, void *out, uint32_t flags,
                                       int32_t max_workgroups, void *stream) {
    tide_status st = tide::check_rs_args(plan, rank, grads, out, flags, max_workgroups);
    if (st != TIDE_OK) return st;
    if (plan->S == 0) return TIDE_OK;
    // The tile size depends only on N and the flags (not on the device).
    const int64_t tile = tide::rs_policy(tide::DeviceLimits{}, plan->N, flags).tile;
    const ScratchLayout L = layout_for(plan, tile);
    if (L.end > kScratchBytes)
        return tide::fail(TIDE_E_INVALID,
                          "tide_rs_noalloc: the plan's tables need " + std::to_string(L.end) +
                              " bytes of scratch, more than its " +
                              std::to_string(kScratchBytes) + " (use tide_rs)");

    std::lock_guard<std::mutex> lock(g_mu);
    ScratchDevice *dev = nullptr;
    st = scratch_device(&dev);
    if (st != TIDE_OK) return st;
    const tide::RsPolicy pol = tide::rs_policy(dev->lim, plan->N, flags);
    const hipStream_t s = static_cast<hipStream_t>(stream);

    // Host image of the tables, in the layout the kernels read.
    const int32_t N = plan->N, P = plan->P;
    std::fill(g_words, g_words + L.words, uint64_t{0});
    char *img = reinterpret_cast<char *>(g_words);
    std::copy(plan->desc.begin(), plan->desc.end(),
              reinterpret_cast<tide::ParamDesc *>(img + L.desc));
    int64_t *tstart = reinterpret_cast<int64_t *>(img + L.tstart);
    tstart[0] = 0;
    for (int32_t i = 0; i < P; i++) tstart[i + 1] = tstart[i] + (plan->desc[i].span + tile - 1) / tile;
    // Param-major pointer table (entry i*N + r), then kPtrPad null entries.
    uintptr_t *ptrs = reinterpret_cast<uintptr_t *>(img + L.ptrs);
    bool aligned16 = true;
    for (int32_t r = 0; r < N; r++)
        for (int32_t i = 0; i < P; i++) {
            const uintptr_t g = reinterpret_cast<uintptr_t>(grads[static_cast<size_t>(r) * P + i]);
            ptrs[static_cast<size_t>(i) * N + r] = g;
            aligned16 = aligned16 && (g & 15) == 0;
        }

    // 1. The tables, one kernel-argument chunk per launch.
    uint64_t *dwords = reinterpret_cast<uint64_t *>(dev->ptr);
    WordChunk chunk;
    for (size_t w0 = 0; w0 < L.words; w0 += kChunkWords) {
        const int n = static_cast<int>(std::min<size_t>(kChunkWords, L.words - w0));
        std::copy(g_words + w0, g_words + w0 + n, chunk.w);
        hipLaunchKernelGGL(put_words, dim3(1), dim3(256), 0, s, dwords + w0, n, chunk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return tide::hip_fail("tide_rs_noalloc: table launch", e);
    }
    // 2. The tile list.
    tide::Tile *tiles = reinterpret_cast<tide::Tile *>(dev->ptr + L.tiles);
    const int64_t tgrid = (L.ntiles + 255) / 256;
    hipLaunchKernelGGL(make_rs_tiles, dim3(static_cast<unsigned>(tgrid)), dim3(256), 0, s, tiles,
                       reinterpret_cast<const int64_t *>(dev->ptr + L.tstart), P, L.ntiles, tile);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tide::hip_fail("tide_rs_noalloc: tile-list launch", e);

    // 3. The reduce-scatter, exactly as tide_rs launches it.
    const tide::RsLaunch launch{reinterpret_cast<const tide::ParamDesc *>(dev->ptr + L.desc),
                                tiles,
                                L.ntiles,
                                reinterpret_cast<const char *const *>(dev->ptr + L.ptrs),
                                N,
                                rank,
                                tide::avg_mode(plan->N, (flags & TIDE_F_AVG) != 0),
                                out,
                                aligned16 ? 1 : 0,
                                (reinterpret_cast<uintptr_t>(out) & 15) == 0 ? 1 : 0,
                                tide::grid_size(dev->lim, L.ntiles, flags, max_workgroups),
                                pol.lds,
                                s};
    const tide::GradType type = (flags & TIDE_F_GRAD_F32)   ? tide::kF32
                                : (flags & TIDE_F_GRAD_F16) ? tide::kF16
                                                            : tide::kBf16;
    const tide::OutType otype = (flags & TIDE_F_OUT_BF16) ? tide::kOutBf16 : tide::kOutF32;
    e = tide::launch_rs(launch, type, otype, pol.shape);
    if (e != hipSuccess) return tide::hip_fail("tide_rs_noalloc: kernel launch", e);
    tide::clear_error();
    return TIDE_OK;
}

// TIDE-RS and TIDE-AG placement kernels for CDNA4 (gfx950), and the
// functions that launch them.
//
// Both operations stream HBM with almost no arithmetic (under half a flop
// per byte), so the design goal is bytes in flight, not ALU: 16-byte global
// loads and stores from wave64 lanes, per-tile descriptors read with scalar
// loads, non-temporal hints on data that is touched once, and short-lived
// workgroups, one per entry of a host-built tile list.
//
// TIDE-RS ("FSDP通信终局：TIDE零拷贝集合通信优化" §"TIDE的设计思路"): the
// per-parameter bf16 gradients of N ranks are read where they lie and
// reduced to this rank's fp32 shard, written straight into its block of the
// flat rank-major buffer; stock FSDP2 first packs them into a full fp32
// buffer (§"FSDP2通信开销的根源"), a copy this path never makes.
// TIDE-AG: shards are placed straight into parameter storage, removing the
// copy-out pass after the all-gather.
#include <hip/hip_runtime.h>

#include "kernel_abi.h"

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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

// fp32 -> bf16 bits, round to nearest with ties to even, on the pattern:
// adding 0x7fff plus the lowest kept bit, then cutting the low 16 bits,
// carries into the kept part exactly when the cut part is above half a
// unit, or equal to it with an odd kept part.  A carry out of the fraction
// raises the exponent (to infinity past the largest finite bf16), which is
// the rounded value.  Subnormals need no special case.  A NaN keeps its top
// bits with the quiet bit set, so it cannot turn into an infinity.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Output element types of the reduce-scatter: the fp32 sum as is, or
// rounded once to bf16.
template <int OT> struct Out;
template <> struct Out<kOutF32> {
    static constexpr int ES = 4;
    typedef f32x4 V4;
    static __device__ __forceinline__ V4 pack(f32x4 v) { return v; }
    static __device__ __forceinline__ void one(GLOBAL_AS char *p, float v) {
        *reinterpret_cast<GLOBAL_AS float *>(p) = v;
    }
};
template <> struct Out<kOutBf16> {
    static constexpr int ES = 2;
    typedef u32x2 V4;
    static __device__ __forceinline__ V4 pack(f32x4 v) {
        return V4{bf16_rne(v.x) | (bf16_rne(v.y) << 16), bf16_rne(v.z) | (bf16_rne(v.w) << 16)};
    }
    static __device__ __forceinline__ void one(GLOBAL_AS char *p, float v) {
        *reinterpret_cast<GLOBAL_AS uint16_t *>(p) = static_cast<uint16_t>(bf16_rne(v));
    }
};

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
// same rank-order sum (and mean, and bf16 rounding) as the vector path.
// P[r] is rank r's gradient; src is rank R's first element in it; o is the
// segment's first output element.
template <int IT, int OT, int BLOCK>
__device__ __forceinline__ void rs_elems(const char *const *__restrict__ P, int N, int avg,
                                         int64_t src, GLOBAL_AS char *o, int64_t a, int64_t b) {
    typedef Grad<IT> G;
    for (int64_t k = a + threadIdx.x; k < b; k += BLOCK) {
        const int64_t byte = (src + k) * G::ES;
        float acc = G::one(gload_ptr<char>(P[0] + byte));
        for (int r = 1; r < N; r++) acc = acc + G::one(gload_ptr<char>(P[r] + byte));
        if (avg == kAvgMul)
            acc = acc * (1.0f / static_cast<float>(N));
        else if (avg == kAvgDiv)
            acc = acc / static_cast<float>(N);
        Out<OT>::one(o + k * Out<OT>::ES, acc);
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
//                 (divided by N when avg is set: kAvgDiv divides, kAvgMul
//                 multiplies by 1/N, which the host picks only when N is a
//                 power of two, where both give the same bits)
//   k >= L(R,i):  out[off_i + k] = +0.0f   (padding rows, alignment gap)
// ptrs is param-major: ptrs[i*N + r] = G[r][i].  OT: fp32 output, or the
// fp32 result rounded to bf16 (padding then +0 in bf16).
//
// Lanes take chunks of 4 consecutive elements: 8-byte loads for 16-bit
// gradients, 16-byte loads for fp32 ones.  vec_in: every gradient pointer is
// 16-byte aligned, so chunks start where src + k is a multiple of 4; the few
// elements before the first and after the last chunk of a tile take the
// scalar path.  vec_out: `out` is 16-byte aligned; a chunk's 4 results go
// out as one 16-byte (fp32) or 8-byte (bf16) store when its output offset is
// a multiple of 4 too, so every store instruction of a wave covers one
// contiguous span.
// PACE > 0 makes each wave sleep between tiles.
template <int IT, int OT, int BLOCK, int CPL, int RB, int PACE, bool XMAP, int64_t TILE>
__global__ __launch_bounds__(BLOCK) void rs_kernel(const ParamDesc *__restrict__ pdesc,
                                                   const Tile *__restrict__ tiles,
                                                   int64_t ntiles,
                                                   const char *const *__restrict__ ptrs,
                                                   int N, int R, int avg, void *__restrict__ out,
                                                   int vec_in, int vec_out) {
    constexpr int ES = Grad<IT>::ES;
    typedef Out<OT> O;
    for (int64_t v = blockIdx.x; v < ntiles; v += gridDim.x) {
        const Tile tile = tiles[XMAP ? xcd_tile(v, ntiles) : v];
        const ParamDesc d = pdesc[tile.param];
        const int64_t src = static_cast<int64_t>(R) * d.seg;
        int64_t L = d.numel - src;
        L = L < 0 ? 0 : (L > d.seg ? d.seg : L);
        const int64_t kb = tile.k0;
        const int64_t ke = min(kb + TILE, d.span);
        const int64_t re = min(ke, L);
        GLOBAL_AS char *o = gstore_ptr<char>(out) + d.off * O::ES;
        const char *const *__restrict__ P = ptrs + static_cast<int64_t>(tile.param) * N;

        if (kb < re) {
            int64_t vs = re, ve = re;
            if (vec_in) {
                vs = min(re, kb + ((4 - ((src + kb) & 3)) & 3));
                ve = vs + ((re - vs) & ~static_cast<int64_t>(3));
            }
            rs_elems<IT, OT, BLOCK>(P, N, avg, src, o, kb, vs);
            rs_elems<IT, OT, BLOCK>(P, N, avg, src, o, ve, re);

            // A tile holds at most TILE/4 chunks, so every per-lane byte
            // offset below fits in 32 bits.
            const int nch = static_cast<int>((ve - vs) >> 2);
            const bool st16 = vec_out && (((d.off + vs) & 3) == 0);
            GLOBAL_AS char *obase = o + vs * O::ES;
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
                    out_off[j] = c * (4u * O::ES);
                }
                f32x4 acc[CPL];
                const int64_t first_byte = (src + vs) * ES;
                rs_batch<IT, CPL, RB, true>(P, 0, min(N, RB), first_byte, in_off, acc);
                for (int r0 = RB; r0 < N; r0 += RB)
                    rs_batch<IT, CPL, RB, false>(P, r0, min(N - r0, RB), first_byte, in_off, acc);
                if (avg == kAvgMul) {
                    const float inv = 1.0f / static_cast<float>(N);   // exact: N = 2^k
#pragma unroll
                    for (int j = 0; j < CPL; j++)
                        acc[j] = f32x4{acc[j].x * inv, acc[j].y * inv, acc[j].z * inv,
                                       acc[j].w * inv};
                } else if (avg == kAvgDiv) {
                    const float n = static_cast<float>(N);
#pragma unroll
                    for (int j = 0; j < CPL; j++)
                        acc[j] = f32x4{acc[j].x / n, acc[j].y / n, acc[j].z / n, acc[j].w / n};
                }
#pragma unroll
                for (int j = 0; j < CPL; j++) {
                    if (!ok[j]) continue;
                    if (st16) {
                        stream_store(O::pack(acc[j]),
                                     reinterpret_cast<GLOBAL_AS typename O::V4 *>(obase + out_off[j]));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++) O::one(obase + out_off[j] + e * O::ES, acc[j][e]);
                    }
                }
            }
        }
        for (int64_t k = max(kb, L) + threadIdx.x; k < ke; k += BLOCK) O::one(o + k * O::ES, 0.0f);
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
// Pack kernel (stage 1 of the two-stage reduce-scatter)
// ---------------------------------------------------------------------------
//
// The inverse placement of TIDE-AG: one rank's per-parameter tensors laid
// out rank-major in a staging slot (for Slot-Reuse, the vacated all-gather
// buffer).  Tile t covers elements [k0, k0 + TILE) of parameter i's span in
// block q = tile.rank:
//   k <  L(q,i):  slot[q*S + off_i + k] = tensors[i][q*seg_i + k]
//   k >= L(q,i):  slot[q*S + off_i + k] = 0   (padding rows, alignment gap)
// ptrs = tensors[0..P) followed by the slot.  The copy takes the widest
// vector both addresses allow, as in ag_kernel.
template <int BLOCK, int U, bool XMAP, int64_t TILE>
__global__ __launch_bounds__(BLOCK) void pack_kernel(const ParamDesc *__restrict__ pdesc,
                                                      const Tile *__restrict__ tiles,
                                                      int64_t ntiles,
                                                      const uintptr_t *__restrict__ ptrs, int P,
                                                      int64_t S, int e) {
    for (int64_t v = blockIdx.x; v < ntiles; v += gridDim.x) {
        const Tile tile = tiles[XMAP ? xcd_tile(v, ntiles) : v];
        const ParamDesc d = pdesc[tile.param];
        const int64_t src = static_cast<int64_t>(tile.rank) * d.seg;
        int64_t L = d.numel - src;
        L = L < 0 ? 0 : (L > d.seg ? d.seg : L);
        const int64_t kb = tile.k0;
        const int64_t ke = min(kb + TILE, d.span);
        char *blk = reinterpret_cast<char *>(ptrs[P]) +
                    (static_cast<int64_t>(tile.rank) * S + d.off) * e;
        const int64_t re = min(ke, L);
        if (kb < re) {
            const char *s = reinterpret_cast<const char *>(ptrs[tile.param]) + (src + kb) * e;
            char *dst = blk + kb * e;
            const int n = static_cast<int>((re - kb) * e);
            const uintptr_t diff = reinterpret_cast<uintptr_t>(s) ^ reinterpret_cast<uintptr_t>(dst);
            if ((diff & 15) == 0)
                copy_span_w<BLOCK, 16, U>(s, dst, n, e);
            else if ((diff & 7) == 0)
                copy_span_w<BLOCK, 8, U>(s, dst, n, e);
            else if ((diff & 3) == 0)
                copy_span_w<BLOCK, 4, U>(s, dst, n, e);
            else
                copy_span_w<BLOCK, 2, U>(s, dst, n, e);
        }
        GLOBAL_AS char *z = gstore_ptr<char>(blk);
        for (int64_t k = max(kb, L) + threadIdx.x; k < ke; k += BLOCK) {
            if (e == 2)
                *reinterpret_cast<GLOBAL_AS uint16_t *>(z + k * 2) = 0;
            else
                *reinterpret_cast<GLOBAL_AS uint32_t *>(z + k * 4) = 0;
        }
    }
}

// ---------------------------------------------------------------------------
// Launch functions
// ---------------------------------------------------------------------------

// Lets `kernel` launch with `bytes` of dynamic LDS (needed above 64 KiB).
hipError_t allow_lds(const void *kernel, int bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// Default launches: one 256-lane workgroup per 4096-element tile (8-rank
// batches, or 2-rank batches for many ranks).  Small-footprint launches:
// the small tile list and its kernel shape.
template <int IT, int OT, int SHAPE>
hipError_t launch_rs_t(const RsLaunch &a) {
    auto k = SHAPE == kRsSmall
                 ? rs_kernel<IT, OT, TIDE_SMALL_BLOCK, TIDE_SMALL_CPL, TIDE_SMALL_RB,
                             TIDE_SMALL_PACE, TIDE_XMAP_RS, kRsTileSmall>
             : SHAPE == kRsWide
                 ? rs_kernel<IT, OT, kBlock, kRsChunksPerLane, TIDE_RS_WIDE_RB, 0, TIDE_XMAP_RS,
                             kRsTile>
                 : rs_kernel<IT, OT, kBlock, kRsChunksPerLane, TIDE_RS_RB, 0, TIDE_XMAP_RS,
                             kRsTile>;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(k), a.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(a.grid), dim3(SHAPE == kRsSmall ? TIDE_SMALL_BLOCK : kBlock),
                       a.lds, a.stream, a.pd, a.tiles, a.ntiles, a.ptrs, a.N, a.R, a.avg, a.out,
                       a.vec_in, a.vec_out);
    return hipGetLastError();
}

template <bool SMALL>
hipError_t launch_ag_t(const AgLaunch &a) {
    auto k = SMALL ? ag_kernel<TIDE_SMALL_AG_BLOCK, TIDE_SMALL_AG_U, TIDE_SMALL_PACE, TIDE_XMAP_AG,
                               kAgTileSmall>
                   : ag_kernel<kBlock, kAgVecsPerLane, 0, TIDE_XMAP_AG, kAgTile>;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(k), a.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(a.grid), dim3(SMALL ? TIDE_SMALL_AG_BLOCK : kBlock), a.lds,
                       a.stream, a.pd, a.tiles, a.ntiles, a.ptrs, a.N, a.elem_bytes);
    return hipGetLastError();
}

template <bool SMALL>
hipError_t launch_pack_t(const PackLaunch &a) {
    auto k = SMALL ? pack_kernel<TIDE_SMALL_AG_BLOCK, TIDE_SMALL_AG_U, TIDE_XMAP_AG, kAgTileSmall>
                   : pack_kernel<kBlock, kAgVecsPerLane, TIDE_XMAP_AG, kAgTile>;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(k), a.lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(a.grid), dim3(SMALL ? TIDE_SMALL_AG_BLOCK : kBlock), a.lds,
                       a.stream, a.pd, a.tiles, a.ntiles, a.ptrs, a.P, a.S, a.elem_bytes);
    return hipGetLastError();
}

template <int IT, int OT>
hipError_t launch_rs_s(const RsLaunch &a, RsKernelShape shape) {
    switch (shape) {
    case kRsSmall: return launch_rs_t<IT, OT, kRsSmall>(a);
    case kRsWide: return launch_rs_t<IT, OT, kRsWide>(a);
    default: return launch_rs_t<IT, OT, kRsDefault>(a);
    }
}

template <int OT>
hipError_t launch_rs_o(const RsLaunch &a, GradType type, RsKernelShape shape) {
    switch (type) {
    case kF32: return launch_rs_s<kF32, OT>(a, shape);
    case kF16: return launch_rs_s<kF16, OT>(a, shape);
    default: return launch_rs_s<kBf16, OT>(a, shape);
    }
}

}  // namespace

hipError_t launch_rs(const RsLaunch &a, GradType type, OutType out, RsKernelShape shape) {
    (void)hipGetLastError();
    return out == kOutBf16 ? launch_rs_o<kOutBf16>(a, type, shape)
                           : launch_rs_o<kOutF32>(a, type, shape);
}

hipError_t launch_ag(const AgLaunch &a, bool small) {
    (void)hipGetLastError();
    return small ? launch_ag_t<true>(a) : launch_ag_t<false>(a);
}

hipError_t launch_pack(const PackLaunch &a, bool small) {
    (void)hipGetLastError();
    return small ? launch_pack_t<true>(a) : launch_pack_t<false>(a);
}

}  // namespace tide

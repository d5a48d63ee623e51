// What the TIDE kernels read and how they are launched: table formats, tile
// sizes, kernel shapes and the launch descriptors.  The kernels and their
// launch functions live in kernels.hip; the runtime (runtime.hip) builds the
// tables and calls the launch functions.  Nothing here changes without
// changing the kernels' machine code.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace tide {

// Build-time tuning constants (defaults are the measured best on MI355X).
#ifndef TIDE_RS_TILE
#define TIDE_RS_TILE 4096
#endif
#ifndef TIDE_AG_TILE
#define TIDE_AG_TILE 2048
#endif
#ifndef TIDE_AG_TILE_SMALL
#define TIDE_AG_TILE_SMALL 32768
#endif
#ifndef TIDE_RS_TILE_SMALL
#define TIDE_RS_TILE_SMALL 1024
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

// Kernel shapes (defaults are the measured best on MI355X).
#ifndef TIDE_RS_CPL
#define TIDE_RS_CPL 4
#endif
#ifndef TIDE_SMALL_BLOCK
#define TIDE_SMALL_BLOCK 256
#endif
#ifndef TIDE_SMALL_PACE
#define TIDE_SMALL_PACE 0
#endif
#ifndef TIDE_RS_RB
#define TIDE_RS_RB 8
#endif
// Default TIDE-RS launches for at least TIDE_RS_WIDE_N ranks load the ranks
// in batches of TIDE_RS_WIDE_RB instead of TIDE_RS_RB.  With the N gradients
// of one element at the same offset in N buffers, fewer of them in flight at
// once per wave measured faster from 16 ranks up (the MoE layer at 16 ranks
// +3.2%, the 70B shapes at 24 ranks +3%) and slower at 8 and 12.
#ifndef TIDE_RS_WIDE_N
#define TIDE_RS_WIDE_N 16
#endif
#ifndef TIDE_RS_WIDE_RB
#define TIDE_RS_WIDE_RB 2
#endif
#ifndef TIDE_SMALL_CPL
#define TIDE_SMALL_CPL 1
#endif
#ifndef TIDE_SMALL_RB
#define TIDE_SMALL_RB 16
#endif
#ifndef TIDE_XMAP_RS
#define TIDE_XMAP_RS 0
#endif
#ifndef TIDE_SMALL_AG_U
#define TIDE_SMALL_AG_U 4
#endif
// Small-footprint copies (all-gather placement, pack): one 1024-lane
// workgroup per CU.  Its 16 light waves (few VGPRs, no ALU work) keep many
// bytes in flight, so each workgroup finishes its tile, and frees its CU,
// quickly.
#ifndef TIDE_SMALL_AG_BLOCK
#define TIDE_SMALL_AG_BLOCK 1024
#endif
#ifndef TIDE_XMAP_AG
#define TIDE_XMAP_AG 1
#endif
#ifndef TIDE_AG_U
#define TIDE_AG_U 1
#endif

constexpr int kRsChunksPerLane = TIDE_RS_CPL;
constexpr int kAgVecsPerLane = TIDE_AG_U;
// Spare (null) entries after the reduce-scatter pointer table: a batch of RB
// ranks loads its RB pointers unconditionally.
constexpr size_t kPtrPad = 32;
static_assert(TIDE_RS_RB <= static_cast<int>(kPtrPad) && TIDE_SMALL_RB <= static_cast<int>(kPtrPad) &&
                  TIDE_RS_WIDE_RB <= static_cast<int>(kPtrPad),
              "rank batch larger than the pointer-table padding");

// The TIDE-RS kernel shapes: the default one (4096-element tiles, 8-rank
// batches), the same over 2-rank batches for many ranks, and the
// small-footprint one (its own tile list).
enum RsKernelShape { kRsDefault = 0, kRsWide = 1, kRsSmall = 2 };

// Gradient element types.  Each widens exactly to fp32: bf16 is the top
// half of an fp32 pattern, every fp16 value is an fp32 value, fp32 is kept.
enum GradType { kBf16 = 0, kF16 = 1, kF32 = 2 };

// Output element types of the reduce-scatter: the fp32 result, or that
// result rounded once to bf16 (nearest, ties to even).
enum OutType { kOutF32 = 0, kOutBf16 = 1 };

// How a TIDE-RS launch turns the rank-order sum into the mean (TIDE_F_AVG):
// not at all, by one correctly rounded division by N, or, when N is a power
// of two, by one multiplication by 1/N = 2^-k.  The exact quotient x/2^k and
// the exact product x*2^-k are the same real number, and each operation
// rounds it once, so the two give identical bits (subnormal results, zeros,
// infinities included; a NaN stays a NaN).
enum AvgMode { kAvgNone = 0, kAvgDiv = 1, kAvgMul = 2 };
inline int avg_mode(int N, bool avg) {
    if (!avg) return kAvgNone;
    return (N & (N - 1)) == 0 ? kAvgMul : kAvgDiv;
}

// Everything one TIDE-RS launch needs.  ptrs is the param-major pointer
// table (entry i*N + r = rank r's gradient of parameter i) plus kPtrPad
// null entries.  vec_in: every gradient pointer is 16-byte aligned; vec_out:
// out is 16-byte aligned.  lds: dynamic LDS each workgroup reserves (never
// touched; it only caps workgroups per CU).
struct RsLaunch {
    const ParamDesc *pd;
    const Tile *tiles;
    int64_t ntiles;
    const char *const *ptrs;
    int N, R, avg;               // avg: an AvgMode
    void *out;                   // S elements of the output type
    int vec_in, vec_out;
    unsigned grid;
    int lds;
    hipStream_t stream;
};

// Everything one TIDE-AG kernel launch needs.  ptrs: the N rank block
// pointers, then the P parameter pointers.
struct AgLaunch {
    const ParamDesc *pd;
    const Tile *tiles;
    int64_t ntiles;
    const uintptr_t *ptrs;
    int N, elem_bytes;
    unsigned grid;
    int lds;
    hipStream_t stream;
};

// Everything one pack launch (stage 1 of the two-stage reduce-scatter)
// needs.  ptrs: the P tensor pointers, then the slot pointer.  S: elements
// per rank block of the slot.
struct PackLaunch {
    const ParamDesc *pd;
    const Tile *tiles;
    int64_t ntiles;
    const uintptr_t *ptrs;
    int P, elem_bytes;
    int64_t S;
    unsigned grid;
    int lds;
    hipStream_t stream;
};

// Enqueue one launch.  For TIDE-RS `shape` picks the kernel shape; for the
// other two `small` selects the small-footprint kernel shape.  The caller
// passes the matching tile list (kRsSmall and `small` walk the
// small-footprint tile lists).  Returns the HIP error of
// the launch (or of allowing its LDS reservation).
hipError_t launch_rs(const RsLaunch &a, GradType type, OutType out, RsKernelShape shape);
hipError_t launch_ag(const AgLaunch &a, bool small);
hipError_t launch_pack(const PackLaunch &a, bool small);

}  // namespace tide

/*
 * tide.h - C ABI of the TIDE placement collectives on one MI355X (gfx950).
 *
 * TIDE keeps FSDP2's per-parameter storage and folds the rank-major layout
 * into the collective's addressing, so neither a gradient pack copy nor an
 * all-gather copy-out pass is needed ("FSDP通信终局：TIDE零拷贝集合通信优化",
 * kongchang.com, §"FSDP2通信开销的根源" and §"TIDE的设计思路：布局感知的零拷贝通信").
 * This library implements one GPU's share of that hot path, with the N ranks
 * of a data-parallel group held as N pointer sets in one device's memory:
 *
 *   tide_plan_*  dim-0 shard geometry with ceil padding and the offsets of
 *                every parameter inside a rank block;
 *   tide_rs      TIDE-RS: per-parameter bf16 gradients of N ranks -> this
 *                rank's fp32 block of the flat rank-major shard buffer,
 *                summed in fp32 in rank order (no pack copy);
 *   tide_ag      TIDE-AG placement: a rank-major gathered buffer -> full
 *                per-parameter tensors (no copy-out pass).
 *
 * Notation.  N = world (ranks), P = nparams.  Parameter i is a row-major
 * tensor viewed as [dim0_i, inner_i] (inner = product of the trailing dims;
 * a 0-dim tensor is [1, 1]).  Psi = sum_i dim0_i * inner_i.
 *   c_i     = ceil(dim0_i / N)              rows of parameter i per rank
 *   seg_i   = c_i * inner_i                 elements of parameter i per rank block
 *   off_0   = 0, off_{i+1} = roundup(off_i + seg_i, align)
 *   S       = roundup(off_{P-1} + seg_{P-1}, align)    elements per rank block
 *   src(r,i)= r * c_i * inner_i             first element of rank r's shard
 *   L(r,i)  = min(c_i, max(0, dim0_i - r*c_i)) * inner_i   real elements of it
 * Rank r's block holds, at off_i + k for k < L(r,i), element src(r,i)+k of
 * parameter i; positions off_i+L(r,i) .. off_i+seg_i-1 are padding, and the
 * positions between segments (align > 1) are gaps.  Each rank keeps 1/N of
 * every parameter (tqpw.cn "FSDP技术演进全景图" §2.1); trailing ranks may hold
 * fewer rows, or none.
 *
 * Ownership and threading.  The caller owns every device buffer and stream.
 * A plan owns its host geometry and, per device it is used on, small device
 * tables (parameter descriptors, tile lists and a cache of uploaded pointer
 * tables).  Host pointer arrays passed to tide_rs / tide_ag are read during
 * the call only.  A plan may be used from several host threads at once.
 *
 * Errors.  Every call returns a tide_status and never aborts.  All argument
 * checks run before anything is enqueued: on an error nothing is launched
 * and no output is touched.  tide_last_error() gives a message for the last
 * non-OK status returned on the calling thread.  A device fault inside a
 * launched kernel surfaces, as for any HIP launch, at the caller's next
 * synchronisation.
 *
 * Streams.  tide_rs and tide_ag are asynchronous and stream-ordered on the
 * given hipStream_t (passed as void*; NULL = the null stream).  The first
 * call of a plan on a device uploads its geometry tables with blocking
 * copies.  Device pointer tables are cached per plan and device (8 pointer
 * sets per operation, least recently used replaced): a set already cached
 * costs a hash and a compare on the host and no upload; a new set is copied
 * through a pinned staging buffer by an async copy on the call's stream.
 * Replacing a set waits (on the host) until the launches that read it have
 * finished, through one event per stream that read it (up to 16 streams per
 * cached set; a further stream takes over the entry of one whose reads have
 * finished).  It synchronises the whole device only if recording such an
 * event failed.  A call on another stream that hits a set whose upload may
 * still be in flight makes its stream wait for that upload.
 *
 * Graph capture.  tide_rs, tide_ag, tide_pack and tide_rs_slots may be
 * captured into a HIP graph (stream capture) once the plan has been used on
 * the device and the call's pointer set is cached and uploaded: make the
 * same call once outside the capture and synchronize first.  Otherwise the
 * call returns TIDE_E_UNSUPPORTED and enqueues nothing.  A pointer set read
 * by a captured launch keeps its cache slot for the plan's lifetime (the
 * graph reads that slot at every replay); once all 8 slots of an operation
 * are held that way, calls with a new pointer set return TIDE_E_UNSUPPORTED.
 * Destroy the graphs before the plan.
 */
#ifndef TIDE_H
#define TIDE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tide_status {
    TIDE_OK = 0,
    TIDE_E_INVALID = 1,      /* argument out of range, null, misaligned or overlapping */
    TIDE_E_UNSUPPORTED = 2,  /* well-formed request the library does not implement */
    TIDE_E_NOMEM = 3,        /* host or device allocation failed */
    TIDE_E_HIP = 4           /* a HIP runtime call failed; message names it */
} tide_status;

/* Opaque plan: the shard geometry of one parameter list for one world size. */
typedef struct tide_plan tide_plan;

/* Launch flag: small-footprint mode, for running beside a compute kernel on
 * another stream (e.g. a bf16 GEMM).  Every tile still gets a short-lived
 * workgroup, but each one reserves just over half of a compute unit's LDS,
 * so at most one is resident per compute unit at any moment, and it holds
 * that unit for one tile only.  A compute kernel that fills every unit
 * waits at most one tile for a unit; beside such a kernel (a single-wave
 * GEMM) the collective makes progress mainly in the kernel's launch gaps and
 * tail.  The pages trace the interference to collectives that occupy the
 * compute units a concurrent GEMM needs (TIDE article, §"FSDP2通信开销的根源");
 * TIDE's answer is to keep collectives off them, with copy engines and
 * short-lived thread blocks (§"TIDE的设计思路").  max_workgroups > 0 with
 * this flag runs a persistent grid instead: more progress beside a compute
 * kernel, which then loses the units that grid holds. */
#define TIDE_F_SMALL_FOOTPRINT 0x1u

/* Launch flag, tide_ag only: place the shards with the SDMA copy engines
 * (hipMemcpyDeviceToDeviceNoCU copies) and no kernel of the library's own,
 * so a concurrent compute kernel keeps the compute units.  This is the
 * analogue of TIDE-AG moving data without occupying SMs (TIDE article,
 * §"TIDE的设计思路").  One 1-D copy per (parameter, rank) run with real
 * elements: P*N copies at most, each costing some tens of microseconds of
 * host time to enqueue (the call returns when all are queued).  The HIP
 * runtime itself may still move copies of about a kilobyte or less with a
 * small kernel.  tide_rs rejects the flag with TIDE_E_UNSUPPORTED: a
 * reduction needs arithmetic. */
#define TIDE_F_COPY_ENGINE 0x2u

/* Flags, tide_rs only: the gradient element type.  Without either flag the
 * gradients are bf16 (the TIDE-RS case).  TIDE_F_GRAD_F16 reads IEEE fp16
 * gradients (FSDP mixed precision with fp16 parameters and an fp32 reduce,
 * tqpw.cn blog §3.2); TIDE_F_GRAD_F32 reads fp32 gradients.  Both widen
 * exactly to fp32 before the rank-order sum.  Setting both is rejected. */
#define TIDE_F_GRAD_F16 0x8u
#define TIDE_F_GRAD_F32 0x10u

/* Flag, tide_rs only: write the shard in bf16 - each fp32 result (sum or
 * mean, computed exactly as without the flag) rounded once to bf16, to
 * nearest with ties to even (a NaN stays a NaN).  The reduction itself stays
 * in fp32, the reduction dtype of FSDP mixed precision (tqpw.cn blog §3.2);
 * only the stored shard is narrowed, halving its bytes. */
#define TIDE_F_OUT_BF16 0x20u

/* Flag, tide_rs only: write the mean instead of the sum - each rank-order
 * fp32 sum divided by N with one correctly rounded binary32 division
 * (apxml "Communication volume analysis" §"分片中的通信原语" describes the
 * gradient reduce-scatter as averaging).  Padding and gaps stay +0.0f.  When
 * N is a power of two the kernel multiplies by 1/N instead, which rounds the
 * same exact value once and so gives the same bits. */
#define TIDE_F_AVG 0x4u

/* ---------------------------------------------------------------------- */
/* Plan (host only; makes no HIP call).                                    */
/* ---------------------------------------------------------------------- */

/* Build the geometry above.
 *   world        N >= 1 ranks (at most 65536).
 *   nparams      P >= 1 parameters (at most 1<<24).
 *   dim0, inner  host arrays of P non-negative sizes; dim0*inner and the
 *                rank block size must fit in int64 (and N*S too).
 *   align_elems  >= 1: offset granularity inside a rank block (1 = tight).
 *   out_plan     receives the plan; set to NULL on error.
 * Returns TIDE_E_INVALID on a bad size, TIDE_E_NOMEM if allocation fails. */
tide_status tide_plan_create(int32_t world, int32_t nparams, const int64_t *dim0,
                             const int64_t *inner, int64_t align_elems,
                             tide_plan **out_plan);

/* Release a plan.  Before freeing its device tables it waits for the launches
 * that may read them (an event per stream that used the plan); if a graph
 * captured a launch of the plan, it waits for the whole device instead.
 * NULL is ignored. */
void tide_plan_destroy(tide_plan *plan);

int32_t tide_plan_world(const tide_plan *plan);          /* N, or -1 if plan is NULL */
int32_t tide_plan_nparams(const tide_plan *plan);        /* P, or -1 */
int64_t tide_plan_shard_numel(const tide_plan *plan);    /* S, or -1 */

/* Geometry of parameter i: off_i, c_i, seg_i (any output may be NULL). */
tide_status tide_plan_param(const tide_plan *plan, int32_t i, int64_t *off,
                            int64_t *rows_per_rank, int64_t *seg_numel);

/* Rank r's shard of parameter i: src(r,i) and L(r,i) (outputs may be NULL). */
tide_status tide_plan_real(const tide_plan *plan, int32_t rank, int32_t i,
                           int64_t *src_off, int64_t *real_numel);

/* ---------------------------------------------------------------------- */
/* TIDE-RS (TIDE article §"TIDE的设计思路"; reduce-scatter semantics from   */
/* §"FSDP2通信开销的根源" and apxml "Communication volume analysis"         */
/* §"分片中的通信原语"; fp32 reduction dtype, tqpw.cn blog §3.2).            */
/* ---------------------------------------------------------------------- */

/* Write rank `rank`'s block (S elements, fp32 or by flag bf16) of the
 * reduce-scatter:
 *   out[off_i + k] = sum over r = 0..N-1, in that order, of
 *                    widen(grads[r*P + i][src(rank,i) + k])   for k < L(rank,i)
 *                    (divided by N with TIDE_F_AVG)
 *   out[off_i + k] = +0.0f for L(rank,i) <= k < seg_i, and gaps are +0.0f.
 * widen(b) is exact (bf16 bits shifted into the top of an fp32; fp16 and
 * fp32 convert exactly); every add is one IEEE binary32 round-to-nearest-even
 * addition with subnormals kept, so the result is bit-for-bit reproducible.
 * With TIDE_F_OUT_BF16 each value above is then rounded once to bf16.
 *   plan    a plan from tide_plan_create.
 *   rank    0 <= rank < N.
 *   grads   host array of N*P device pointers; entry r*P + i is rank r's
 *           gradient of parameter i, dim0_i*inner_i elements, row-major,
 *           aligned to its element size (bf16 by default, fp16 or fp32 by
 *           flag).  Only the elements of rank `rank`'s shard are read.
 *           Entries with L(rank,i) = 0 may be NULL.
 *   out     device pointer to S floats (4-byte aligned), or with
 *           TIDE_F_OUT_BF16 to S bf16 values (2-byte aligned), e.g. block
 *           `rank` of an N*S buffer; must not overlap any element that is read.
 *   flags   any of TIDE_F_SMALL_FOOTPRINT, TIDE_F_AVG, TIDE_F_OUT_BF16 and
 *           one of TIDE_F_GRAD_F16 / TIDE_F_GRAD_F32 (both: TIDE_E_INVALID);
 *           TIDE_F_COPY_ENGINE or other bits -> TIDE_E_UNSUPPORTED.
 *   max_workgroups  0 = the policy for `flags`; > 0 caps the grid.
 *   stream  hipStream_t (NULL = null stream).
 * 16-byte aligned pointers take the vector path; other alignments are
 * handled element by element with identical results. */
tide_status tide_rs(const tide_plan *plan, int32_t rank, const void *const *grads,
                    void *out, uint32_t flags, int32_t max_workgroups, void *stream);

/* ---------------------------------------------------------------------- */
/* TIDE-AG placement (TIDE article §"TIDE的设计思路"; all-gather semantics  */
/* from apxml "Communication volume analysis" §"分片中的通信原语").          */
/* ---------------------------------------------------------------------- */

/* Scatter N rank blocks straight into full per-parameter tensors:
 *   params[i][src(r,i) + k] = rank_src[r][off_i + k]   for every r, i, k < L(r,i)
 * as an exact copy of elem_bytes-byte elements.  Padding and gaps are never
 * read; every element of every parameter is written exactly once.
 *   rank_src    host array of N device pointers, each to a rank block of S
 *               elements (e.g. base + r*S*elem_bytes of a gathered buffer).
 *   params      host array of P device pointers to the full tensors
 *               (dim0_i*inner_i elements; NULL allowed when that is 0).
 *   elem_bytes  2 (bf16/fp16) or 4 (fp32).
 *   flags       0, TIDE_F_SMALL_FOOTPRINT or TIDE_F_COPY_ENGINE (not both);
 *               other bits -> TIDE_E_UNSUPPORTED.
 *   max_workgroups, stream  as for tide_rs (max_workgroups is ignored with
 *               TIDE_F_COPY_ENGINE).
 * Destinations must not overlap one another or any element that is read.
 * With TIDE_F_COPY_ENGINE the call enqueues several copies; if the runtime
 * rejects one of them (TIDE_E_HIP), copies enqueued before it still run. */
tide_status tide_ag(const tide_plan *plan, const void *const *rank_src,
                    void *const *params, int32_t elem_bytes, uint32_t flags,
                    int32_t max_workgroups, void *stream);

/* ---------------------------------------------------------------------- */
/* Two-stage TIDE-RS with Slot-Reuse (TIDE article §"TIDE的设计思路": the  */
/* two-stage pipeline separates gradient reads from network progress, and  */
/* Slot-Reuse stages gradients in vacated all-gather slots).               */
/* ---------------------------------------------------------------------- */

/* Stage 1: lay one rank's per-parameter tensors out rank-major in a staging
 * slot of N*S elements - the layout of the all-gather buffer, so a vacated
 * all-gather buffer can serve as the slot:
 *   slot[q*S + off_i + k] = tensors[i][src(q,i) + k]   for k < L(q,i)
 *   slot[q*S + off_i + k] = 0 for L(q,i) <= k < seg_i, and gaps are 0,
 * for every destination rank q.  Block q is this rank's contribution to
 * rank q's shard.  An exact copy of elem_bytes-byte elements.
 *   tensors     host array of P device pointers (dim0_i*inner_i elements;
 *               NULL allowed when that is 0), element-aligned.
 *   slot        device pointer to N*S elements, element-aligned; it must not
 *               overlap any tensor.
 *   elem_bytes  2 (bf16/fp16) or 4 (fp32).
 *   flags       0 or TIDE_F_SMALL_FOOTPRINT; other bits -> TIDE_E_UNSUPPORTED.
 *   max_workgroups, stream  as for tide_rs. */
tide_status tide_pack(const tide_plan *plan, const void *const *tensors, void *slot,
                      int32_t elem_bytes, uint32_t flags, int32_t max_workgroups,
                      void *stream);

/* Stage 2: rank `rank`'s block of the reduce-scatter from N staged slots:
 *   out[off_i + k] = rank-order fp32 sum over r of widen(slots[r][rank*S + off_i + k])
 * for k < L(rank,i), and +0 elsewhere - bit-identical to tide_rs over the
 * gradients the slots were packed from (same order, same widening, and the
 * same flags: TIDE_F_SMALL_FOOTPRINT, TIDE_F_AVG, TIDE_F_OUT_BF16, and
 * TIDE_F_GRAD_F16 / TIDE_F_GRAD_F32 for the slot element type).
 *   slots   host array of N device pointers; slots[r] = rank r's slot (N*S
 *           elements, aligned to the element size).  Only block `rank` of
 *           each slot is read, and of it only the real elements.
 *   out     as for tide_rs; must not overlap any element that is read.
 * Errors and streams as for tide_rs. */
tide_status tide_rs_slots(const tide_plan *plan, int32_t rank, const void *const *slots,
                          void *out, uint32_t flags, int32_t max_workgroups, void *stream);

/* ---------------------------------------------------------------------- */
/* Allocation-free TIDE-RS.                                                */
/* ---------------------------------------------------------------------- */

/* tide_rs for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, flags, validation and result as tide_rs, bit for bit; it
 * calls no hipMalloc, hipFree or other allocating HIP routine and keeps no
 * per-plan device state.  The tables tide_rs keeps in plan-owned device
 * memory (parameter descriptors, tile list, pointer table) are instead
 * written, on `stream`, into one fixed 8 MiB array per device that the
 * library holds until the process ends; the first call on a device only
 * looks up that array's address.  Each call enqueues small table-writing
 * launches (the tables travel as kernel arguments, about 3.5 KiB per launch)
 * and then the reduce-scatter kernel.
 *   Limit: 32*P + 8*(P+1) + 8*(N*P + 32) bytes of tables, rounded up to 256,
 *   plus 16 bytes per tile (ceil(span_i / 4096) tiles per parameter, or
 *   ceil(span_i / 1024) with TIDE_F_SMALL_FOOTPRINT above 16 ranks) must fit
 *   in 8 MiB; a larger plan returns TIDE_E_INVALID before anything is
 *   enqueued.
 *   Sharing: every call on one device uses that device's one array.  Calls
 *   ordered on one stream are safe; calls that overlap on one device (other
 *   streams, or other host threads without ordering between them) race on
 *   the array and may read each other's tables.  Order them with events or
 *   use one stream. */
tide_status tide_rs_noalloc(const tide_plan *plan, int32_t rank, const void *const *grads,
                            void *out, uint32_t flags, int32_t max_workgroups, void *stream);

/* ---------------------------------------------------------------------- */
/* Diagnostics.                                                            */
/* ---------------------------------------------------------------------- */

/* Message for the last non-OK status on this thread ("" if none). */
const char *tide_last_error(void);

/* Fixed name of a status code. */
const char *tide_status_string(tide_status status);

#ifdef __cplusplus
}
#endif

#endif /* TIDE_H */

// Host side of the TIDE library: plan construction, geometry queries,
// argument validation and error reporting.  Makes no HIP call.
//
// Geometry: dim-0 shards with ceil(dim0/N) rows per rank, every shard padded
// to that many rows, parameters packed in caller order inside a rank block
// ("FSDP通信终局：TIDE零拷贝集合通信优化" §"FSDP2通信开销的根源" for the
// rank-major block layout; tqpw.cn "FSDP技术演进全景图" §2.1 for 1/N of every
// parameter per rank).
#include <algorithm>
#include <cstring>
#include <new>

#include "internal.h"

namespace {
bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_add_overflow(a, b, r); }

bool round_up_ok(int64_t x, int64_t a, int64_t *r) {
    int64_t t;
    if (!add_ok(x, a - 1, &t)) return false;
    *r = t / a * a;
    return true;
}
}  // namespace

namespace tide {

namespace {
thread_local std::string g_last_error;

// One half-open byte interval [lo, hi).
struct Span {
    uintptr_t lo, hi;
};

bool overlap(const Span &a, const Span &b) { return a.lo < b.hi && b.lo < a.hi; }

// Sorts `dst` and reports whether two of its spans overlap.
bool sort_and_check_disjoint(std::vector<Span> &dst) {
    std::sort(dst.begin(), dst.end(), [](const Span &a, const Span &b) { return a.lo < b.lo; });
    for (size_t k = 1; k < dst.size(); k++)
        if (dst[k].lo < dst[k - 1].hi) return false;
    return true;
}

// True if `s` overlaps a span of `dst` (sorted, disjoint: hi ascends too).
bool hits_sorted(const std::vector<Span> &dst, const Span &s) {
    auto it = std::upper_bound(dst.begin(), dst.end(), s.lo,
                               [](uintptr_t v, const Span &d) { return v < d.hi; });
    return it != dst.end() && it->lo < s.hi;
}
}  // namespace

tide_status fail(tide_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

void clear_error() { g_last_error.clear(); }

const char *last_error_cstr() { return g_last_error.c_str(); }

tide_status check_rs_args(const tide_plan *p, int32_t rank, const void *const *grads,
                          const void *out, uint32_t flags, int32_t max_wg) {
    if (!p) return fail(TIDE_E_INVALID, "tide_rs: plan is NULL");
    if (rank < 0 || rank >= p->N)
        return fail(TIDE_E_INVALID, "tide_rs: rank " + std::to_string(rank) +
                                        " outside [0, " + std::to_string(p->N) + ")");
    if (flags & TIDE_F_COPY_ENGINE)
        return fail(TIDE_E_UNSUPPORTED,
                    "tide_rs: TIDE_F_COPY_ENGINE is for tide_ag (a reduction needs arithmetic)");
    if (flags & ~(TIDE_F_SMALL_FOOTPRINT | TIDE_F_AVG | TIDE_F_GRAD_F16 | TIDE_F_GRAD_F32 |
                  TIDE_F_OUT_BF16))
        return fail(TIDE_E_UNSUPPORTED, "tide_rs: unknown flag bits");
    if ((flags & TIDE_F_GRAD_F16) && (flags & TIDE_F_GRAD_F32))
        return fail(TIDE_E_INVALID, "tide_rs: TIDE_F_GRAD_F16 and TIDE_F_GRAD_F32 both set");
    const uintptr_t es = (flags & TIDE_F_GRAD_F32) ? 4u : 2u;
    const uintptr_t os = (flags & TIDE_F_OUT_BF16) ? 2u : 4u;
    if (max_wg < 0) return fail(TIDE_E_INVALID, "tide_rs: max_workgroups < 0");
    if (p->S == 0) return TIDE_OK;
    if (!grads) return fail(TIDE_E_INVALID, "tide_rs: grads array is NULL");
    if (!out) return fail(TIDE_E_INVALID, "tide_rs: out is NULL");
    if (reinterpret_cast<uintptr_t>(out) % os)
        return fail(TIDE_E_INVALID, "tide_rs: out is not aligned to its element size");
    // One pass over the N*P gradient runs rank `rank` reads (no allocation):
    // each must be non-null, element-aligned and disjoint from `out`.
    const uintptr_t o = reinterpret_cast<uintptr_t>(out);
    const Span written{o, o + static_cast<uintptr_t>(p->S) * os};
    for (int32_t i = 0; i < p->P; i++) {
        int64_t src, L;
        shard_run(p, rank, i, &src, &L);
        if (L == 0) continue;
        for (int32_t r = 0; r < p->N; r++) {
            const void *g = grads[static_cast<int64_t>(r) * p->P + i];
            if (!g)
                return fail(TIDE_E_INVALID, "tide_rs: grads[" + std::to_string(r) + "*P+" +
                                                std::to_string(i) + "] is NULL");
            const uintptr_t a = reinterpret_cast<uintptr_t>(g);
            if (a % es)
                return fail(TIDE_E_INVALID, "tide_rs: grads[" + std::to_string(r) + "*P+" +
                                                std::to_string(i) +
                                                "] is not aligned to its element size");
            const Span read{a + static_cast<uintptr_t>(src) * es,
                            a + static_cast<uintptr_t>(src + L) * es};
            if (overlap(read, written))
                return fail(TIDE_E_INVALID, "tide_rs: out overlaps gradient elements it would read");
        }
    }
    return TIDE_OK;
}

tide_status check_ag_args(const tide_plan *p, const void *const *rank_src,
                          void *const *params, int32_t elem_bytes, uint32_t flags,
                          int32_t max_wg) {
    if (!p) return fail(TIDE_E_INVALID, "tide_ag: plan is NULL");
    if (elem_bytes != 2 && elem_bytes != 4)
        return fail(TIDE_E_INVALID, "tide_ag: elem_bytes must be 2 or 4");
    if (flags & ~(TIDE_F_SMALL_FOOTPRINT | TIDE_F_COPY_ENGINE))
        return fail(TIDE_E_UNSUPPORTED, "tide_ag: unknown flag bits");
    if ((flags & TIDE_F_SMALL_FOOTPRINT) && (flags & TIDE_F_COPY_ENGINE))
        return fail(TIDE_E_UNSUPPORTED,
                    "tide_ag: TIDE_F_SMALL_FOOTPRINT and TIDE_F_COPY_ENGINE exclude each other");
    if (max_wg < 0) return fail(TIDE_E_INVALID, "tide_ag: max_workgroups < 0");
    if (p->psi == 0) return TIDE_OK;
    if (!rank_src) return fail(TIDE_E_INVALID, "tide_ag: rank_src array is NULL");
    if (!params) return fail(TIDE_E_INVALID, "tide_ag: params array is NULL");
    const uintptr_t e = static_cast<uintptr_t>(elem_bytes);
    // Destinations: sorted once (P log P) and checked pairwise disjoint.  A
    // rank block is then checked against them whole, and run by run (binary
    // searches) only if it touches one: padding may lie under a destination.
    thread_local std::vector<Span> dst;
    dst.clear();
    for (int32_t i = 0; i < p->P; i++) {
        if (p->numel[i] == 0) continue;
        const uintptr_t d = reinterpret_cast<uintptr_t>(params[i]);
        if (!d)
            return fail(TIDE_E_INVALID, "tide_ag: params[" + std::to_string(i) + "] is NULL");
        if (d % e)
            return fail(TIDE_E_INVALID, "tide_ag: params[" + std::to_string(i) +
                                            "] is not aligned to its element size");
        dst.push_back({d, d + static_cast<uintptr_t>(p->numel[i]) * e});
    }
    if (!sort_and_check_disjoint(dst))
        return fail(TIDE_E_INVALID, "tide_ag: a destination overlaps another destination");
    const uintptr_t block_bytes = static_cast<uintptr_t>(p->S) * e;
    for (int32_t r = 0; r < p->N; r++) {
        const uintptr_t s = reinterpret_cast<uintptr_t>(rank_src[r]);
        // A rank block that no destination touches needs no per-run check.
        if (s && s % e == 0 && !hits_sorted(dst, Span{s, s + block_bytes})) continue;
        bool checked = false;
        for (int32_t i = 0; i < p->P; i++) {
            int64_t src, L;
            shard_run(p, r, i, &src, &L);
            if (L == 0) continue;
            if (!checked) {
                if (!s)
                    return fail(TIDE_E_INVALID,
                                "tide_ag: rank_src[" + std::to_string(r) + "] is NULL");
                if (s % e)
                    return fail(TIDE_E_INVALID, "tide_ag: rank_src[" + std::to_string(r) +
                                                    "] is not aligned to its element size");
                checked = true;
            }
            const Span read{s + static_cast<uintptr_t>(p->off[i]) * e,
                            s + static_cast<uintptr_t>(p->off[i] + L) * e};
            if (hits_sorted(dst, read))
                return fail(TIDE_E_INVALID,
                            "tide_ag: a destination overlaps a source element that is read");
        }
    }
    return TIDE_OK;
}

tide_status check_pack_args(const tide_plan *p, const void *const *tensors, const void *slot,
                            int32_t elem_bytes, uint32_t flags, int32_t max_wg) {
    if (!p) return fail(TIDE_E_INVALID, "tide_pack: plan is NULL");
    if (elem_bytes != 2 && elem_bytes != 4)
        return fail(TIDE_E_INVALID, "tide_pack: elem_bytes must be 2 or 4");
    if (flags & ~TIDE_F_SMALL_FOOTPRINT)
        return fail(TIDE_E_UNSUPPORTED, "tide_pack: unsupported flag bits");
    if (max_wg < 0) return fail(TIDE_E_INVALID, "tide_pack: max_workgroups < 0");
    if (p->S == 0) return TIDE_OK;
    if (!tensors) return fail(TIDE_E_INVALID, "tide_pack: tensors array is NULL");
    const uintptr_t e = static_cast<uintptr_t>(elem_bytes);
    const uintptr_t d = reinterpret_cast<uintptr_t>(slot);
    if (!d) return fail(TIDE_E_INVALID, "tide_pack: slot is NULL");
    if (d % e) return fail(TIDE_E_INVALID, "tide_pack: slot is not aligned to its element size");
    // The slot (N*S elements) is written whole; each tensor is read whole.
    const Span written{d, d + static_cast<uintptr_t>(p->N) * static_cast<uintptr_t>(p->S) * e};
    for (int32_t i = 0; i < p->P; i++) {
        if (p->numel[i] == 0) continue;
        const uintptr_t a = reinterpret_cast<uintptr_t>(tensors[i]);
        if (!a) return fail(TIDE_E_INVALID, "tide_pack: tensors[" + std::to_string(i) + "] is NULL");
        if (a % e)
            return fail(TIDE_E_INVALID, "tide_pack: tensors[" + std::to_string(i) +
                                            "] is not aligned to its element size");
        if (overlap(Span{a, a + static_cast<uintptr_t>(p->numel[i]) * e}, written))
            return fail(TIDE_E_INVALID, "tide_pack: the slot overlaps tensors[" +
                                            std::to_string(i) + "]");
    }
    return TIDE_OK;
}

tide_status check_rs_slots_args(const tide_plan *p, int32_t rank, const void *const *slots,
                                const void *out, uint32_t flags, int32_t max_wg) {
    if (!p) return fail(TIDE_E_INVALID, "tide_rs_slots: plan is NULL");
    if (rank < 0 || rank >= p->N)
        return fail(TIDE_E_INVALID, "tide_rs_slots: rank " + std::to_string(rank) +
                                        " outside [0, " + std::to_string(p->N) + ")");
    if (flags & TIDE_F_COPY_ENGINE)
        return fail(TIDE_E_UNSUPPORTED, "tide_rs_slots: TIDE_F_COPY_ENGINE is for tide_ag");
    if (flags & ~(TIDE_F_SMALL_FOOTPRINT | TIDE_F_AVG | TIDE_F_GRAD_F16 | TIDE_F_GRAD_F32 |
                  TIDE_F_OUT_BF16))
        return fail(TIDE_E_UNSUPPORTED, "tide_rs_slots: unknown flag bits");
    if ((flags & TIDE_F_GRAD_F16) && (flags & TIDE_F_GRAD_F32))
        return fail(TIDE_E_INVALID,
                    "tide_rs_slots: TIDE_F_GRAD_F16 and TIDE_F_GRAD_F32 both set");
    const uintptr_t es = (flags & TIDE_F_GRAD_F32) ? 4u : 2u;
    const uintptr_t os = (flags & TIDE_F_OUT_BF16) ? 2u : 4u;
    if (max_wg < 0) return fail(TIDE_E_INVALID, "tide_rs_slots: max_workgroups < 0");
    if (p->S == 0) return TIDE_OK;
    if (!slots) return fail(TIDE_E_INVALID, "tide_rs_slots: slots array is NULL");
    if (!out) return fail(TIDE_E_INVALID, "tide_rs_slots: out is NULL");
    const uintptr_t o = reinterpret_cast<uintptr_t>(out);
    if (o % os) return fail(TIDE_E_INVALID, "tide_rs_slots: out is not aligned to its element size");
    const Span written{o, o + static_cast<uintptr_t>(p->S) * os};
    for (int32_t r = 0; r < p->N; r++) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(slots[r]);
        if (!a)
            return fail(TIDE_E_INVALID, "tide_rs_slots: slots[" + std::to_string(r) + "] is NULL");
        if (a % es)
            return fail(TIDE_E_INVALID, "tide_rs_slots: slots[" + std::to_string(r) +
                                            "] is not aligned to its element size");
        // Block `rank` of slot r: the runs of real elements are read.
        const uintptr_t blk = a + static_cast<uintptr_t>(rank) * static_cast<uintptr_t>(p->S) * es;
        for (int32_t i = 0; i < p->P; i++) {
            int64_t src, L;
            shard_run(p, rank, i, &src, &L);
            if (L == 0) continue;
            const Span read{blk + static_cast<uintptr_t>(p->off[i]) * es,
                            blk + static_cast<uintptr_t>(p->off[i] + L) * es};
            if (overlap(read, written))
                return fail(TIDE_E_INVALID,
                            "tide_rs_slots: out overlaps slot elements it would read");
        }
    }
    return TIDE_OK;
}

}  // namespace tide

using tide::fail;

extern "C" {

tide_status tide_plan_create(int32_t world, int32_t nparams, const int64_t *dim0,
                             const int64_t *inner, int64_t align_elems,
                             tide_plan **out_plan) {
    if (!out_plan) return fail(TIDE_E_INVALID, "tide_plan_create: out_plan is NULL");
    *out_plan = nullptr;
    if (world < 1 || world > 65536)
        return fail(TIDE_E_INVALID, "tide_plan_create: world must be in [1, 65536]");
    if (nparams < 1 || nparams > (1 << 24))
        return fail(TIDE_E_INVALID, "tide_plan_create: nparams must be in [1, 2^24]");
    if (!dim0 || !inner) return fail(TIDE_E_INVALID, "tide_plan_create: size array is NULL");
    if (align_elems < 1) return fail(TIDE_E_INVALID, "tide_plan_create: align_elems < 1");

    tide_plan *p = new (std::nothrow) tide_plan;
    if (!p) return fail(TIDE_E_NOMEM, "tide_plan_create: out of host memory");
    try {
        p->N = world;
        p->P = nparams;
        p->align = align_elems;
        p->d0.assign(dim0, dim0 + nparams);
        p->inner.assign(inner, inner + nparams);
        p->c.resize(nparams);
        p->seg.resize(nparams);
        p->off.resize(nparams);
        p->numel.resize(nparams);
        p->desc.resize(nparams);
        int64_t pos = 0, psi = 0;
        for (int32_t i = 0; i < nparams; i++) {
            const int64_t d = dim0[i], n = inner[i];
            if (d < 0 || n < 0) {
                delete p;
                return fail(TIDE_E_INVALID, "tide_plan_create: negative size for param " +
                                                std::to_string(i));
            }
            const int64_t c = d / world + (d % world != 0);
            int64_t seg, numel, off, end;
            if (!mul_ok(c, n, &seg) || !mul_ok(d, n, &numel) || !round_up_ok(pos, align_elems, &off) ||
                !add_ok(off, seg, &end) || !add_ok(psi, numel, &psi)) {
                delete p;
                return fail(TIDE_E_INVALID, "tide_plan_create: sizes overflow int64");
            }
            p->c[i] = c;
            p->seg[i] = seg;
            p->numel[i] = numel;
            p->off[i] = off;
            p->desc[i] = {off, seg, numel, seg};
            if (i > 0) p->desc[i - 1].span = off - p->off[i - 1];
            pos = end;
        }
        int64_t S, total;
        if (!round_up_ok(pos, align_elems, &S) || !mul_ok(S, world, &total) ||
            !mul_ok(total, 4, &total)) {
            delete p;
            return fail(TIDE_E_INVALID, "tide_plan_create: rank block size overflows int64");
        }
        p->S = S;
        p->psi = psi;
        p->desc[nparams - 1].span = S - p->off[nparams - 1];

        // Reduce-scatter tiles cover every position of a rank block: each
        // parameter's segment and the alignment gap after it (padding and
        // gaps are written as zeros).  They do not depend on the rank.
        for (int32_t i = 0; i < nparams; i++) {
            for (int64_t k = 0; k < p->desc[i].span; k += tide::kRsTile)
                p->rs_tiles.push_back({i, 0, k});
            for (int64_t k = 0; k < p->desc[i].span; k += tide::kRsTileSmall)
                p->rs_tiles_small.push_back({i, 0, k});
        }
        // All-gather tiles cover the real elements of every (param, rank);
        // ranks of one parameter are adjacent so the destination tensor is
        // written front to back.
        for (int32_t i = 0; i < nparams; i++)
            for (int32_t r = 0; r < world; r++) {
                int64_t src, L;
                tide::shard_run(p, r, i, &src, &L);
                for (int64_t k = 0; k < L; k += tide::kAgTile) p->ag_tiles.push_back({i, r, k});
                for (int64_t k = 0; k < L; k += tide::kAgTileSmall)
                    p->ag_tiles_small.push_back({i, r, k});
            }
        // Pack tiles cover every position of every (param, rank) span of a
        // staging slot: real elements are copied, padding and gaps zeroed.
        for (int32_t i = 0; i < nparams; i++)
            for (int32_t r = 0; r < world; r++) {
                for (int64_t k = 0; k < p->desc[i].span; k += tide::kAgTile)
                    p->pack_tiles.push_back({i, r, k});
                for (int64_t k = 0; k < p->desc[i].span; k += tide::kAgTileSmall)
                    p->pack_tiles_small.push_back({i, r, k});
            }
    } catch (const std::bad_alloc &) {
        delete p;
        return fail(TIDE_E_NOMEM, "tide_plan_create: out of host memory");
    }
    *out_plan = p;
    return TIDE_OK;
}

void tide_plan_destroy(tide_plan *plan) {
    if (!plan) return;
    tide::release_device_states(plan);
    delete plan;
}

int32_t tide_plan_world(const tide_plan *plan) { return plan ? plan->N : -1; }
int32_t tide_plan_nparams(const tide_plan *plan) { return plan ? plan->P : -1; }
int64_t tide_plan_shard_numel(const tide_plan *plan) { return plan ? plan->S : -1; }

tide_status tide_plan_param(const tide_plan *plan, int32_t i, int64_t *off,
                            int64_t *rows_per_rank, int64_t *seg_numel) {
    if (!plan) return fail(TIDE_E_INVALID, "tide_plan_param: plan is NULL");
    if (i < 0 || i >= plan->P) return fail(TIDE_E_INVALID, "tide_plan_param: index out of range");
    if (off) *off = plan->off[i];
    if (rows_per_rank) *rows_per_rank = plan->c[i];
    if (seg_numel) *seg_numel = plan->seg[i];
    return TIDE_OK;
}

tide_status tide_plan_real(const tide_plan *plan, int32_t rank, int32_t i, int64_t *src_off,
                           int64_t *real_numel) {
    if (!plan) return fail(TIDE_E_INVALID, "tide_plan_real: plan is NULL");
    if (rank < 0 || rank >= plan->N) return fail(TIDE_E_INVALID, "tide_plan_real: rank out of range");
    if (i < 0 || i >= plan->P) return fail(TIDE_E_INVALID, "tide_plan_real: index out of range");
    int64_t src, L;
    tide::shard_run(plan, rank, i, &src, &L);
    if (src_off) *src_off = src;
    if (real_numel) *real_numel = L;
    return TIDE_OK;
}

const char *tide_last_error(void) { return tide::last_error_cstr(); }

const char *tide_status_string(tide_status status) {
    switch (status) {
        case TIDE_OK: return "TIDE_OK";
        case TIDE_E_INVALID: return "TIDE_E_INVALID";
        case TIDE_E_UNSUPPORTED: return "TIDE_E_UNSUPPORTED";
        case TIDE_E_NOMEM: return "TIDE_E_NOMEM";
        case TIDE_E_HIP: return "TIDE_E_HIP";
    }
    return "TIDE_E_UNKNOWN";
}

}  // extern "C"

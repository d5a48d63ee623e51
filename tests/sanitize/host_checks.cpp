// The library's host code (plan geometry, argument checks, error strings)
// run under AddressSanitizer and UndefinedBehaviorSanitizer.  Built with g++
// from csrc/plan.cpp and this file only, so no HIP call and no GPU is
// involved: the one runtime function plan.cpp needs, which frees device
// tables, is a no-op here.  Every call must return a valid status, and the
// cases with a known answer must give it; any memory error or undefined
// behaviour aborts the program with the sanitizer's report.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "../../parameter_layout_collectives_amd/csrc/internal.h"

namespace tide {
void release_device_states(const tide_plan *) {}
}  // namespace tide

namespace {

int failures = 0;

void expect(bool ok, const char *what, int line) {
    if (!ok) {
        std::fprintf(stderr, "FAILED at line %d: %s (last error: %s)\n", line, what,
                     tide_last_error());
        failures++;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

bool valid_status(tide_status s) {
    return s == TIDE_OK || s == TIDE_E_INVALID || s == TIDE_E_UNSUPPORTED ||
           s == TIDE_E_NOMEM || s == TIDE_E_HIP;
}

// Fake device addresses: never dereferenced by the checks.
constexpr uintptr_t kBase = uintptr_t(0x7f0000000000ull);
const void *addr(uintptr_t a) { return reinterpret_cast<const void *>(a); }

void plan_errors() {
    int64_t d0[2] = {4, 5}, in[2] = {3, 1};
    tide_plan *p = reinterpret_cast<tide_plan *>(1);
    EXPECT(tide_plan_create(0, 2, d0, in, 1, &p) == TIDE_E_INVALID && p == nullptr);
    EXPECT(tide_plan_create(65537, 2, d0, in, 1, &p) == TIDE_E_INVALID);
    EXPECT(tide_plan_create(4, 0, d0, in, 1, &p) == TIDE_E_INVALID);
    EXPECT(tide_plan_create(4, 2, nullptr, in, 1, &p) == TIDE_E_INVALID);
    EXPECT(tide_plan_create(4, 2, d0, nullptr, 1, &p) == TIDE_E_INVALID);
    EXPECT(tide_plan_create(4, 2, d0, in, 0, &p) == TIDE_E_INVALID);
    EXPECT(tide_plan_create(4, 2, d0, in, 1, nullptr) == TIDE_E_INVALID);
    int64_t neg[2] = {-1, 5};
    EXPECT(tide_plan_create(4, 2, neg, in, 1, &p) == TIDE_E_INVALID);
    const int64_t big = std::numeric_limits<int64_t>::max() / 2;
    int64_t bd[2] = {big, 1}, bi[2] = {3, 1};
    EXPECT(tide_plan_create(4, 2, bd, bi, 1, &p) == TIDE_E_INVALID);   // dim0 * inner
    int64_t hd[2] = {int64_t(1) << 40, 1}, hi[2] = {int64_t(1) << 22, 1};
    EXPECT(tide_plan_create(64, 2, hd, hi, 1, &p) == TIDE_E_INVALID);  // 4*N*S
    int64_t ad[1] = {7}, ai[1] = {1};
    EXPECT(tide_plan_create(2, 1, ad, ai, std::numeric_limits<int64_t>::max(), &p) ==
           TIDE_E_INVALID);                                               // rounding up
    EXPECT(std::strlen(tide_last_error()) > 0);
    EXPECT(tide_plan_world(nullptr) == -1 && tide_plan_nparams(nullptr) == -1 &&
           tide_plan_shard_numel(nullptr) == -1);
    EXPECT(tide_plan_param(nullptr, 0, nullptr, nullptr, nullptr) == TIDE_E_INVALID);
    tide_plan_destroy(nullptr);
    for (int s = -2; s < 8; s++) EXPECT(tide_status_string(static_cast<tide_status>(s)) != nullptr);
}

void random_plan(std::mt19937_64 &g) {
    const int32_t N = 1 + static_cast<int32_t>(g() % 70);
    const int32_t P = 1 + static_cast<int32_t>(g() % 12);
    const int64_t align = int64_t(1) << (g() % 4);
    std::vector<int64_t> d0(P), in(P);
    for (int32_t i = 0; i < P; i++) {
        d0[i] = (g() % 9 == 0) ? 0 : static_cast<int64_t>(g() % 300);
        in[i] = (g() % 11 == 0) ? 0 : 1 + static_cast<int64_t>(g() % 40);
    }
    tide_plan *p = nullptr;
    EXPECT(tide_plan_create(N, P, d0.data(), in.data(), align, &p) == TIDE_OK);
    if (!p) return;
    const int64_t S = tide_plan_shard_numel(p);
    EXPECT(S >= 0 && S % align == 0);
    int64_t prev_end = 0;
    for (int32_t i = 0; i < P; i++) {
        int64_t off = -1, c = -1, seg = -1;
        EXPECT(tide_plan_param(p, i, &off, &c, &seg) == TIDE_OK);
        EXPECT(off % align == 0 && off >= prev_end && off + seg <= S);
        EXPECT(c == (d0[i] + N - 1) / N && seg == c * in[i]);
        prev_end = off + seg;
        int64_t total = 0;
        for (int32_t r = 0; r < N; r++) {
            int64_t src = -1, L = -1;
            EXPECT(tide_plan_real(p, r, i, &src, &L) == TIDE_OK);
            EXPECT(src == r * seg && L >= 0 && L <= seg);
            total += L;
        }
        EXPECT(total == d0[i] * in[i]);
    }
    int64_t o1, o2, o3;   // real outputs, so an index past the end would be read
    EXPECT(tide_plan_param(p, P, &o1, &o2, &o3) == TIDE_E_INVALID);
    EXPECT(tide_plan_param(p, -1, &o1, &o2, &o3) == TIDE_E_INVALID);
    EXPECT(tide_plan_real(p, N, 0, &o1, &o2) == TIDE_E_INVALID);
    EXPECT(tide_plan_real(p, 0, P, &o1, &o2) == TIDE_E_INVALID);

    // tide_rs arguments: every gradient its own range, 1 MiB apart; `out` far away.
    const int32_t R = static_cast<int32_t>(g() % N);
    std::vector<const void *> grads(static_cast<size_t>(N) * P);
    for (size_t k = 0; k < grads.size(); k++) grads[k] = addr(kBase + (k << 20));
    const uintptr_t far = kBase + (uintptr_t(1) << 36);
    int64_t psi = 0;
    for (int32_t i = 0; i < P; i++) psi += d0[i] * in[i];
    // An empty rank block (S = 0) or an empty model (psi = 0) has nothing to
    // move: those calls succeed without looking at the pointers.
    EXPECT(tide::check_rs_args(p, R, grads.data(), addr(far), 0, 0) == TIDE_OK);
    EXPECT(tide::check_rs_args(p, N, grads.data(), addr(far), 0, 0) == TIDE_E_INVALID);
    EXPECT(tide::check_rs_args(p, R, grads.data(), addr(far + 2), 0, 0) ==
           (S > 0 ? TIDE_E_INVALID : TIDE_OK));   // fp32 out not 4-byte aligned
    EXPECT(tide::check_rs_args(p, R, nullptr, addr(far), 0, 0) ==
           (S > 0 ? TIDE_E_INVALID : TIDE_OK));
    EXPECT(tide::check_rs_args(p, R, grads.data(), addr(far), 0x80000000u, 0) != TIDE_OK);
    // `out` placed at a random gradient's address: an error exactly when
    // that gradient's run for rank R is non-empty and S > 0
    const size_t victim = g() % grads.size();
    const int32_t vi = static_cast<int32_t>(victim % P);
    int64_t vsrc = 0, vL = 0;
    tide_plan_real(p, R, vi, &vsrc, &vL);
    const tide_status ov = tide::check_rs_args(p, R, grads.data(),
                                               addr(kBase + (victim << 20) + 2 * vsrc), 0, 0);
    EXPECT(valid_status(ov));
    if (vL > 0 && S > 0) EXPECT(ov == TIDE_E_INVALID);
    // random pointers: any status is fine, but it must be a valid one
    for (int t = 0; t < 4; t++) {
        std::vector<const void *> rnd(grads.size());
        for (auto &q : rnd) q = addr(kBase + 2 * (g() % (uintptr_t(1) << 30)));
        EXPECT(valid_status(tide::check_rs_args(p, R, rnd.data(),
                                                addr(kBase + 4 * (g() % (uintptr_t(1) << 28))),
                                                static_cast<uint32_t>(g() % 64), 0)));
    }

    // tide_ag arguments: one rank-major buffer, parameters far away and apart.
    for (int32_t e : {2, 4}) {
        std::vector<const void *> src(N);
        for (int32_t r = 0; r < N; r++) src[r] = addr(kBase + uintptr_t(r) * S * e);
        std::vector<void *> dst(P);
        for (int32_t i = 0; i < P; i++)
            dst[i] = const_cast<void *>(addr(far + (uintptr_t(i) << 24)));
        EXPECT(tide::check_ag_args(p, src.data(), dst.data(), e, 0, 0) == TIDE_OK);
        EXPECT(tide::check_ag_args(p, src.data(), dst.data(), 3, 0, 0) == TIDE_E_INVALID);
        EXPECT(tide::check_ag_args(p, nullptr, dst.data(), e, 0, 0) ==
               (psi > 0 ? TIDE_E_INVALID : TIDE_OK));
        // two parameters at one address: an error when both have elements
        if (P >= 2) {
            std::vector<void *> dup(dst);
            dup[1] = dup[0];
            const tide_status st = tide::check_ag_args(p, src.data(), dup.data(), e, 0, 0);
            EXPECT(valid_status(st));
            if (d0[0] * in[0] > 0 && d0[1] * in[1] > 0) EXPECT(st == TIDE_E_INVALID);
        }
        for (int t = 0; t < 4; t++) {
            std::vector<void *> rnd(P);
            for (auto &q : rnd)
                q = const_cast<void *>(addr(kBase + uintptr_t(e) * (g() % (uintptr_t(1) << 26))));
            EXPECT(valid_status(tide::check_ag_args(p, src.data(), rnd.data(), e,
                                                    static_cast<uint32_t>(g() % 64), 0)));
            EXPECT(valid_status(tide::check_pack_args(p, grads.data(), rnd[0], e,
                                                      static_cast<uint32_t>(g() % 64), 0)));
        }
        EXPECT(valid_status(tide::check_rs_slots_args(p, R, src.data(), addr(far), 0, 0)));
    }
    tide_plan_destroy(p);
}

}  // namespace

int main() {
    plan_errors();
    std::mt19937_64 g(20261202);
    for (int it = 0; it < 1500; it++) random_plan(g);
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}

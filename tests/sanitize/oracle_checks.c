/* The oracle's C code (oracle/oracle.c) run under AddressSanitizer and
 * UndefinedBehaviorSanitizer on buffers of exactly the sizes its contract
 * names, so a read or write one element past any of them is reported.  It
 * also checks one property the contract fixes: packing a rank's tensors and
 * all-gathering the packed slot gives the tensors back.  Test
 * infrastructure: built by tests/test_host_sanitizers.py with gcc. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_geometry(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                    int64_t align, int64_t *c, int64_t *seg, int64_t *off, int64_t *S);
int oracle_rs_typed(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                    int64_t align, int32_t R, int dtype, int avg, const void *const *grads,
                    float *out);
int oracle_pack(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner, int64_t align,
                int32_t elem_bytes, const void *const *tensors, void *slot);
int oracle_ag(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner, int64_t align,
              int32_t elem_bytes, const void *const *rank_src, void *const *params);
int oracle_round_bf16(const float *in, uint16_t *out, int64_t n);
int oracle_rs_traffic(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                      int64_t align, int32_t R, int64_t *real, int64_t *padded);

static uint64_t state = 88172645463325252ull;
static uint64_t next(void) {   /* xorshift64 */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c); failures++; } } while (0)

static void *xmalloc(size_t n) {   /* n = 0 still gives a distinct block */
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static void fill(void *p, size_t n) {
    unsigned char *b = p;
    for (size_t k = 0; k < n; k++) b[k] = (unsigned char)next();
}

static void one_case(void) {
    const int32_t N = 1 + (int32_t)(next() % 9), P = 1 + (int32_t)(next() % 6);
    const int64_t align = (int64_t)1 << (next() % 3);
    int64_t d0[6], in[6], c[6], seg[6], off[6], S;
    for (int32_t i = 0; i < P; i++) {
        d0[i] = (next() % 7 == 0) ? 0 : (int64_t)(next() % 40);
        in[i] = (next() % 9 == 0) ? 0 : 1 + (int64_t)(next() % 9);
    }
    EXPECT(oracle_geometry(N, P, d0, in, align, c, seg, off, &S) == 0);
    const int dtype = (int)(next() % 3);
    const size_t es = dtype == 2 ? 4 : 2;
    /* every rank's full gradients, each its own exact-size block */
    void **grads = xmalloc(sizeof(void *) * (size_t)N * P);
    for (int32_t r = 0; r < N; r++)
        for (int32_t i = 0; i < P; i++) {
            size_t n = (size_t)(d0[i] * in[i]) * es;
            grads[(size_t)r * P + i] = xmalloc(n);
            fill(grads[(size_t)r * P + i], n);
        }
    float *out = xmalloc(sizeof(float) * (size_t)S);
    const int32_t R = (int32_t)(next() % N);
    EXPECT(oracle_rs_typed(N, P, d0, in, align, R, dtype, (int)(next() % 2),
                           (const void *const *)grads, out) == 0);
    int64_t real, padded;
    EXPECT(oracle_rs_traffic(N, P, d0, in, align, R, &real, &padded) == 0);
    EXPECT(padded == (int64_t)(N - 1) * S && real <= padded);
    uint16_t *rounded = xmalloc(sizeof(uint16_t) * (size_t)S);
    EXPECT(oracle_round_bf16(out, rounded, S) == 0);

    /* pack rank 0's tensors into an exact N*S slot, all-gather it back */
    const int32_t e = (next() % 2) ? 4 : 2;
    void **t = xmalloc(sizeof(void *) * P), **back = xmalloc(sizeof(void *) * P);
    for (int32_t i = 0; i < P; i++) {
        size_t n = (size_t)(d0[i] * in[i]) * (size_t)e;
        t[i] = xmalloc(n);
        fill(t[i], n);
        back[i] = xmalloc(n);
        memset(back[i], 0, n ? n : 1);
    }
    void *slot = xmalloc((size_t)N * (size_t)S * (size_t)e);
    EXPECT(oracle_pack(N, P, d0, in, align, e, (const void *const *)t, slot) == 0);
    const void **blocks = xmalloc(sizeof(void *) * N);
    for (int32_t r = 0; r < N; r++) blocks[r] = (const char *)slot + (size_t)r * S * e;
    EXPECT(oracle_ag(N, P, d0, in, align, e, blocks, back) == 0);
    for (int32_t i = 0; i < P; i++)
        EXPECT(memcmp(t[i], back[i], (size_t)(d0[i] * in[i]) * (size_t)e) == 0);

    for (int32_t i = 0; i < P; i++) { free(t[i]); free(back[i]); }
    free(t); free(back); free(slot); free(blocks); free(rounded); free(out);
    for (size_t k = 0; k < (size_t)N * P; k++) free(grads[k]);
    free(grads);
}

int main(void) {
    int64_t d0 = 3, in = 2, c, seg, off, S;
    EXPECT(oracle_geometry(0, 1, &d0, &in, 1, &c, &seg, &off, &S) != 0);
    EXPECT(oracle_geometry(2, 1, &d0, &in, 0, &c, &seg, &off, &S) != 0);
    for (int it = 0; it < 3000; it++) one_case();
    if (failures) { fprintf(stderr, "%d check(s) failed\n", failures); return 1; }
    printf("oracle checks passed\n");
    return 0;
}

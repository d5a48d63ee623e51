/*
 * CPU oracle for the TIDE layout-aware reduce-scatter / all-gather placement.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the placement collectives compute.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or constant with the HIP library, and the HIP
 * library never calls it.
 *
 * Sources (cited by page title and section):
 *   [TIDE] "FSDP通信终局：TIDE零拷贝集合通信优化" (kongchang.com)
 *          §"FSDP2通信开销的根源"  - per-parameter storage versus the flat
 *            rank-major buffer (all elements of one rank contiguous, rank
 *            blocks one after another); reduce-scatter leaves each rank with
 *            the reduced shard it owns.
 *          §"TIDE的设计思路"        - TIDE-RS reads per-parameter bf16
 *            gradients and reduces them to fp32 shards; TIDE-AG delivers
 *            shards straight into parameter storage.
 *   [VOL]  apxml "Communication volume analysis" (FSDP course, ch. 1)
 *          §"分片中的通信原语"      - all-gather rebuilds full parameters
 *            from the shards; reduce-scatter hands each rank its shard.
 *          §"带宽饱和和节点扩展"    - a ring all-gather or reduce-scatter
 *            moves (N-1)/N * Psi elements per rank.
 *   [BLOG] tqpw.cn "FSDP技术演进全景图" §2.1 - each of N GPUs keeps 1/N of
 *            the parameters; §3.2 - fp16 parameters with reduction dtype
 *            float32 (hence fp16 gradients reduced in fp32).
 *
 * Readings taken where the pages are silent (each one listed in the design
 * notes of the repository):
 *   - shards are taken along dim 0 with c = ceil(d0/N) rows per rank; the
 *     trailing ranks may own fewer rows (or none) and their shard is padded
 *     to c rows;
 *   - inside one rank block the parameters follow the caller's order, each
 *     at an offset rounded up to `align` elements (1 = tightly packed);
 *   - padding and alignment gaps of the reduce-scatter output are +0.0f;
 *   - the reduction is a SUM in binary32, in rank order 0..N-1, starting
 *     from rank 0's widened value (not from +0.0), round-to-nearest-even on
 *     every add, no fused operations, subnormals kept;
 *   - bf16 -> fp32 widening is exact: the fp32 bit pattern is the bf16
 *     pattern shifted left by 16; fp16 -> fp32 widening is exact too;
 *   - the mean (when asked for) is the rank-order sum divided by N with one
 *     correctly rounded binary32 division (the volume page describes the
 *     reduce-scatter of gradients as averaging; the TIDE article as a
 *     reduction to fp32; the sum is the default contract);
 *   - a bf16 shard (when asked for) is the fp32 result above rounded once
 *     to bf16, to nearest with ties to even (the reduction itself stays in
 *     fp32, as the blog's reduction dtype and the TIDE article require).
 *
 * Build: gcc -std=c11 -O2 -fno-fast-math -ffp-contract=off -fopenmp
 *        (see oracle/build_oracle.py).  OpenMP splits independent output
 *        elements only; the per-element rank loop is always sequential, so the
 *        thread count never changes a bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>
#if defined(__x86_64__)
#include <xmmintrin.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* The oracle relies on IEEE binary32 with subnormals kept.  Some shared
 * libraries switch the SSE flush-to-zero / denormals-are-zero bits on when
 * they load, so every thread clears them before it adds anything. */
static unsigned keep_subnormals(void)
{
#if defined(__x86_64__)
    unsigned old = _mm_getcsr();
    _mm_setcsr(old & ~(0x8000u /* FTZ */ | 0x0040u /* DAZ */));
    return old;
#else
    return 0;
#endif
}

static void restore_fp_mode(unsigned old)
{
#if defined(__x86_64__)
    _mm_setcsr(old);
#else
    (void)old;
#endif
}

/* bf16 -> fp32, exact: the bf16 bits are the upper half of the fp32 bits. */
static float widen_bf16(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* IEEE binary16 -> binary32, exact (every half value is a float value).
 * Fields: sign 1 bit, exponent 5 bits (bias 15), fraction 10 bits.
 *   exponent 0:  zero or subnormal, value = fraction * 2^-24
 *   exponent 31: infinity (fraction 0) or NaN (payload kept in the top
 *                fraction bits of the float)
 *   otherwise:   normal, float exponent = e - 15 + 127, fraction << 13 */
static float widen_f16(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1fu;
    uint32_t frac = (uint32_t)h & 0x3ffu;
    uint32_t bits;
    float f;
    if (e == 0) {
        f = (float)frac * 0x1p-24f;     /* frac < 2^10: product exact */
        return sign ? -f : f;
    }
    if (e == 31)
        bits = (sign << 31) | 0x7f800000u | (frac << 13);
    else
        bits = (sign << 31) | ((e - 15u + 127u) << 23) | (frac << 13);
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Gradient element types of the reduce-scatter. */
#define ORACLE_BF16 0
#define ORACLE_F16 1
#define ORACLE_F32 2

/* Element k of a gradient run, as an exact fp32 value. */
static float load_elem(const void *run, int64_t k, int dtype)
{
    if (dtype == ORACLE_BF16) return widen_bf16(((const uint16_t *)run)[k]);
    if (dtype == ORACLE_F16) return widen_f16(((const uint16_t *)run)[k]);
    float f;
    memcpy(&f, (const char *)run + 4 * k, sizeof f);
    return f;
}

static int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

/* ---------------------------------------------------------------------- */
/* Shard geometry ([TIDE] §"FSDP2通信开销的根源": rank-major layout;       */
/* [BLOG] §2.1: 1/N per GPU; dim-0 rows with ceil padding).                */
/* ---------------------------------------------------------------------- */

/* For every parameter i: c[i] rows per rank, seg[i] = c[i]*inner[i] elements
 * per rank block, off[i] its offset inside a rank block; *S = rank block size. */
int oracle_geometry(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                    int64_t align, int64_t *c, int64_t *seg, int64_t *off, int64_t *S)
{
    if (N <= 0 || P <= 0 || align <= 0) return ORACLE_EINVAL;
    int64_t pos = 0;
    for (int32_t i = 0; i < P; i++) {
        if (d0[i] < 0 || inner[i] < 0) return ORACLE_EINVAL;
        c[i] = (d0[i] + N - 1) / N;
        seg[i] = c[i] * inner[i];
        off[i] = round_up(pos, align);
        pos = off[i] + seg[i];
    }
    *S = round_up(pos, align);
    return ORACLE_OK;
}

/* Rank r's shard of parameter i: it starts at element src of the full tensor
 * and holds L real (non-padding) elements. */
static void shard_run(int32_t r, int64_t d0, int64_t inner, int64_t c,
                      int64_t *src, int64_t *L)
{
    int64_t rows = d0 - (int64_t)r * c;
    if (rows < 0) rows = 0;
    if (rows > c) rows = c;
    *src = (int64_t)r * c * inner;
    *L = rows * inner;
}

int oracle_shard_run(int32_t N, int64_t d0, int64_t inner, int32_t r,
                     int64_t *src, int64_t *L)
{
    if (N <= 0 || r < 0 || r >= N || d0 < 0 || inner < 0) return ORACLE_EINVAL;
    shard_run(r, d0, inner, (d0 + N - 1) / N, src, L);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Reduce-scatter into this rank's fp32 block ([TIDE] §"TIDE的设计思路":    */
/* bf16 per-parameter gradients in, fp32 shard out; [VOL] §"分片中的通信原语"). */
/* ---------------------------------------------------------------------- */

/* Shared body: `first[r*P + i]` points at element 0 of rank r's contribution
 * to rank R's shard of parameter i, i.e. at G[r][i] + src(R,i) for the
 * full-tensor entry points, or at the slice itself for the slice entry
 * points.  dtype is the gradient element type; avg != 0 divides each sum by
 * N (one correctly rounded binary32 division), giving the mean. */
static int rs_body(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                   int64_t align, int32_t R, int dtype, int avg, const void *const *first,
                   float *out)
{
    int64_t S;
    if (N <= 0 || P <= 0 || R < 0 || R >= N) return ORACLE_EINVAL;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16 && dtype != ORACLE_F32) return ORACLE_EINVAL;
    int64_t *c = malloc(3 * sizeof(int64_t) * (size_t)P);
    if (!c) return ORACLE_EINVAL;
    int64_t *seg = c + P, *off = c + 2 * P;
    if (oracle_geometry(N, P, d0, inner, align, c, seg, off, &S) != ORACLE_OK) {
        free(c);
        return ORACLE_EINVAL;
    }

    unsigned mode = keep_subnormals();

    /* Every position of the block starts as +0.0f: padding rows and the
     * alignment gaps keep that value. */
    for (int64_t j = 0; j < S; j++) out[j] = 0.0f;

    for (int32_t i = 0; i < P; i++) {
        int64_t src, L;
        shard_run(R, d0[i], inner[i], c[i], &src, &L);
        (void)src;
#pragma omp parallel
        {
            keep_subnormals();
#pragma omp for schedule(static)
            for (int64_t k = 0; k < L; k++) {
                float acc = load_elem(first[(int64_t)0 * P + i], k, dtype);
                for (int32_t r = 1; r < N; r++)
                    acc = acc + load_elem(first[(int64_t)r * P + i], k, dtype);
                if (avg) acc = acc / (float)N;
                out[off[i] + k] = acc;
            }
        }
    }
    restore_fp_mode(mode);
    free(c);
    return ORACLE_OK;
}

static size_t elem_size(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* grads[r*P + i] = rank r's full gradient of parameter i (d0*inner
 * elements of type dtype, row-major).  out = S fp32 values, rank R's block. */
int oracle_rs_typed(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                    int64_t align, int32_t R, int dtype, int avg, const void *const *grads,
                    float *out)
{
    if (N <= 0 || P <= 0 || R < 0 || R >= N) return ORACLE_EINVAL;
    const void **first = malloc(sizeof(void *) * (size_t)N * (size_t)P);
    if (!first) return ORACLE_EINVAL;
    for (int32_t r = 0; r < N; r++)
        for (int32_t i = 0; i < P; i++) {
            int64_t src, L;
            shard_run(R, d0[i], inner[i], (d0[i] + N - 1) / N, &src, &L);
            first[(int64_t)r * P + i] =
                L > 0 ? (const char *)grads[(int64_t)r * P + i] + (size_t)src * elem_size(dtype)
                      : NULL;
        }
    int rc = rs_body(N, P, d0, inner, align, R, dtype, avg, first, out);
    free(first);
    return rc;
}

/* slices[r*P + i] = the L(R,i) elements of rank r's gradient of parameter i
 * that belong to rank R's shard (G[r][i][src(R,i) .. src(R,i)+L(R,i)) ). */
int oracle_rs_slices_typed(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                           int64_t align, int32_t R, int dtype, int avg,
                           const void *const *slices, float *out)
{
    return rs_body(N, P, d0, inner, align, R, dtype, avg, slices, out);
}

/* The TIDE-RS contract: bf16 gradients, fp32 sum. */
int oracle_rs(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
              int64_t align, int32_t R, const uint16_t *const *grads, float *out)
{
    return oracle_rs_typed(N, P, d0, inner, align, R, ORACLE_BF16, 0,
                           (const void *const *)grads, out);
}

int oracle_rs_slices(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                     int64_t align, int32_t R, const uint16_t *const *slices, float *out)
{
    return rs_body(N, P, d0, inner, align, R, ORACLE_BF16, 0, (const void *const *)slices, out);
}

/* ---------------------------------------------------------------------- */
/* Staging for the two-stage reduce-scatter ([TIDE] §"TIDE的设计思路": the  */
/* pipeline stages gradients, optionally in vacated all-gather slots).      */
/* ---------------------------------------------------------------------- */

/* One rank's per-parameter tensors laid out rank-major, as the all-gather
 * buffer is: for every destination rank q, parameter i and k < seg_i
 *   slot[q*S + off_i + k] = tensors[i][src(q,i) + k]   if k < L(q,i)
 *                         = 0                           otherwise (padding),
 * and every alignment gap is 0.  elem_bytes-byte elements, copied exactly.
 * Block q of the slot is what this rank contributes to rank q's shard. */
int oracle_pack(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                int64_t align, int32_t elem_bytes, const void *const *tensors, void *slot)
{
    int64_t S;
    if (N <= 0 || P <= 0 || (elem_bytes != 2 && elem_bytes != 4)) return ORACLE_EINVAL;
    int64_t *c = malloc(3 * sizeof(int64_t) * (size_t)P);
    if (!c) return ORACLE_EINVAL;
    int64_t *seg = c + P, *off = c + 2 * P;
    if (oracle_geometry(N, P, d0, inner, align, c, seg, off, &S) != ORACLE_OK) {
        free(c);
        return ORACLE_EINVAL;
    }
    /* Everything starts as zero: padding rows and gaps keep it. */
    memset(slot, 0, (size_t)N * (size_t)S * (size_t)elem_bytes);
    for (int32_t q = 0; q < N; q++) {
        for (int32_t i = 0; i < P; i++) {
            int64_t src, L;
            shard_run(q, d0[i], inner[i], c[i], &src, &L);
            char *to = (char *)slot + ((int64_t)q * S + off[i]) * elem_bytes;
            const char *from = (const char *)tensors[i] + src * elem_bytes;
            if (L > 0) memcpy(to, from, (size_t)L * (size_t)elem_bytes);
        }
    }
    free(c);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* fp32 -> bf16 rounding of a reduced shard.                               */
/* ---------------------------------------------------------------------- */

/* The value of a bf16 pattern, as a double (exact). */
static double bf16_value(uint16_t b) { return (double)widen_bf16(b); }

/* x rounded to bf16: IEEE round to nearest, ties to even.
 * A bf16 keeps an fp32's sign, 8-bit exponent and top 7 fraction bits, so
 * the bf16 values around a finite x are t, x's pattern with its low 16 bits
 * cleared (x cut toward zero), and t + 1 as a pattern, the next bf16 away
 * from zero (sign-magnitude patterns grow with magnitude).  x goes to the
 * nearer of the two, and on a tie to the one whose last bit is 0.  Above
 * the largest finite bf16 the upper neighbour is infinity, whose distance
 * is measured as if it were 2^128 (IEEE's rule for overflow).  All
 * distances are exact in double.  Zeros and infinities are kept; a NaN stays
 * a NaN (its quiet bit set, so that cutting the payload cannot give an
 * infinity). */
static uint16_t round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
    uint16_t t = (uint16_t)(u >> 16);
    if ((u & 0xffffu) == 0) return t;          /* representable (zeros, infinities too) */
    uint16_t up = (uint16_t)(t + 1u);
    double ax = fabs((double)x);
    double at = fabs(bf16_value(t));
    double aup = ((up & 0x7fffu) == 0x7f80u) ? ldexp(1.0, 128) : fabs(bf16_value(up));
    double d_t = ax - at, d_up = aup - ax;
    if (d_t < d_up) return t;
    if (d_up < d_t) return up;
    return (t & 1u) ? up : t;
}

/* out[k] = round_bf16(in[k]) for k < n. */
int oracle_round_bf16(const float *in, uint16_t *out, int64_t n)
{
    if (n < 0 || (n > 0 && (!in || !out))) return ORACLE_EINVAL;
    for (int64_t k = 0; k < n; k++) out[k] = round_bf16(in[k]);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* All-gather placement ([TIDE] §"TIDE的设计思路": shards delivered straight */
/* into parameter storage; [VOL] §"分片中的通信原语": full parameters rebuilt). */
/* ---------------------------------------------------------------------- */

/* rank_src[r] = rank r's block (S elements of elem_bytes each);
 * params[i]   = full tensor of parameter i (d0*inner elements).
 * For every r, i and k < L(r,i): params[i][src(r,i)+k] = rank_src[r][off_i+k].
 * Padding is never read; nothing else in params is written. */
int oracle_ag(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
              int64_t align, int32_t elem_bytes, const void *const *rank_src,
              void *const *params)
{
    int64_t S;
    if (N <= 0 || P <= 0 || (elem_bytes != 2 && elem_bytes != 4)) return ORACLE_EINVAL;
    int64_t *c = malloc(3 * sizeof(int64_t) * (size_t)P);
    if (!c) return ORACLE_EINVAL;
    int64_t *seg = c + P, *off = c + 2 * P;
    if (oracle_geometry(N, P, d0, inner, align, c, seg, off, &S) != ORACLE_OK) {
        free(c);
        return ORACLE_EINVAL;
    }
    for (int32_t r = 0; r < N; r++) {
        for (int32_t i = 0; i < P; i++) {
            int64_t src, L;
            shard_run(r, d0[i], inner[i], c[i], &src, &L);
            if (elem_bytes == 2) {
                const uint16_t *from = (const uint16_t *)rank_src[r];
                uint16_t *to = (uint16_t *)params[i];
#pragma omp parallel for schedule(static)
                for (int64_t k = 0; k < L; k++) to[src + k] = from[off[i] + k];
            } else {
                const uint32_t *from = (const uint32_t *)rank_src[r];
                uint32_t *to = (uint32_t *)params[i];
#pragma omp parallel for schedule(static)
                for (int64_t k = 0; k < L; k++) to[src + k] = from[off[i] + k];
            }
        }
    }
    free(c);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* Traffic counts ([VOL] §"带宽饱和和节点扩展").                              */
/* ---------------------------------------------------------------------- */

/* Elements rank R pulls from the other N-1 ranks in a reduce-scatter:
 * *real = sum over params of (N-1)*L(R,i), *padded = (N-1)*S. */
int oracle_rs_traffic(int32_t N, int32_t P, const int64_t *d0, const int64_t *inner,
                      int64_t align, int32_t R, int64_t *real, int64_t *padded)
{
    int64_t S;
    if (N <= 0 || P <= 0 || R < 0 || R >= N) return ORACLE_EINVAL;
    int64_t *c = malloc(3 * sizeof(int64_t) * (size_t)P);
    if (!c) return ORACLE_EINVAL;
    int64_t *seg = c + P, *off = c + 2 * P;
    if (oracle_geometry(N, P, d0, inner, align, c, seg, off, &S) != ORACLE_OK) {
        free(c);
        return ORACLE_EINVAL;
    }
    int64_t sum = 0;
    for (int32_t i = 0; i < P; i++) {
        int64_t src, L;
        shard_run(R, d0[i], inner[i], c[i], &src, &L);
        sum += L;
    }
    *real = (int64_t)(N - 1) * sum;
    *padded = (int64_t)(N - 1) * S;
    free(c);
    return ORACLE_OK;
}

/* Threads an OpenMP region of the oracle will use. */
int oracle_threads(void) { return omp_get_max_threads(); }

void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

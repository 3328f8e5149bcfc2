/*
 * Plain CPU oracle for paged grouped-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call this.  It shares no code, header or
 * constant with the HIP library and must never stand in for it.
 *
 * It is the definition written out, following the f64 reference in the span-02
 * GPU test page (respanai/span-02, engine/crates/kernels/tests/gpu.rs, function
 * `reference`):
 *   - scale 1.0: scores are the plain dot product q . k (no 1/sqrt(hd));
 *   - GQA: query head h reads kv head kh = h / (nh / nkv);
 *   - causal with an optional sliding window: key position p is visible to a
 *     row at position qpos iff lo <= p <= hi, lo = max(0, qpos + 1 - window)
 *     when window > 0 (else 0), hi = the row's last visible key (the page passes
 *     the query positions for it, so hi = qpos in every call it shows);
 *   - every bf16 input is widened exactly, dot products, exponentials, the
 *     normaliser and the weighted sum of V are all taken in f64:
 *       m = max_p s_p,  e_p = exp(s_p - m),  z = sum_p e_p,
 *       o_d = sum_p (e_p / z) * v_{p,d};
 *   - the f64 result is rounded once to bf16, round-to-nearest-even.  (The
 *     page's own `bf` helper truncates; rounding is the reading taken here, the
 *     two differ by at most one bf16 ulp.)
 * Addressing (same page, the pool layout and the `mapped_pool` helper):
 *   table entry = page_origin[row] + p / 16, physical page = block_table[entry]
 *   (then page_map[physical page] when a page map is given), element
 *   ((phys * nkv + kh) * 16 + p % 16) * hd + d of the K (or V) pool.
 *
 * Sums run over p in increasing order, then over d in increasing order, with
 * no blocking, fusion or reordering.  Built without -ffast-math and with
 * -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PAGE 16

static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Correctly rounded f64 -> bf16 (nearest, ties to even). */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    if (isinf(x))
        return signbit(x) ? 0xff80 : 0x7f80;
    if (x == 0.0)
        return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(fabs(x), &e);            /* |x| = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;                /* floor(log2 |x|) */
    if (ex < -126)
        ex = -126;                 /* subnormal bf16 spacing is fixed */
    double ulp = ldexp(1.0, ex - 7);   /* 7 stored mantissa bits */
    double y = rint(x / ulp) * ulp;    /* default rounding mode: ties to even */
    float f = (float)y;            /* exact (or overflow to inf) */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Error codes: 0 ok; -1 bad shape; -2 table index out of range; -3 page out of
 * range; -4 page-map index out of range; -5 out of memory. */
int pgqa_oracle_decode(uint16_t *out, double *out_f64,
                       const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                       const int32_t *block_table, int64_t table_len,
                       const int32_t *page_origin, const int32_t *qpos,
                       const int32_t *kv_last,
                       const int32_t *page_map, int64_t map_len,
                       int64_t npages,
                       int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                       int64_t window, int nthreads)
{
    if (rows < 0 || nh <= 0 || nkv <= 0 || hd <= 0 || nh % nkv != 0 || window < 0)
        return -1;
    const int64_t group = nh / nkv;
    int status = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t job = 0; job < rows * nh; ++job) {
        const int64_t t = job / nh, h = job % nh;
        const int64_t kh = h / group;
        const int64_t qp = qpos[t];
        const int64_t lo = window > 0 ? (qp + 1 - window > 0 ? qp + 1 - window : 0) : 0;
        const int64_t hi = kv_last[t];
        const uint16_t *qrow = q + (t * nh + h) * hd;
        uint16_t *orow = out + (t * nh + h) * hd;
        double *o = calloc((size_t)hd, sizeof(double));
        int64_t n = hi >= lo ? hi - lo + 1 : 0;
        double *s = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        int64_t *base = malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        if (!o || !s || !base) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -5;
            free(o); free(s); free(base);
            continue;
        }
        int bad = 0;
        /* Resolve every visible key's address: origin + p/16 -> table -> (map) -> pool. */
        for (int64_t i = 0; i < n && !bad; ++i) {
            const int64_t p = lo + i;
            const int64_t entry = (int64_t)page_origin[t] + p / ORACLE_PAGE;
            if (entry < 0 || entry >= table_len) { bad = -2; break; }
            int64_t phys = block_table[entry];
            if (page_map) {
                if (phys < 0 || phys >= map_len) { bad = -4; break; }
                phys = page_map[phys];
            }
            if (phys < 0 || phys >= npages) { bad = -3; break; }
            base[i] = ((phys * nkv + kh) * ORACLE_PAGE + p % ORACLE_PAGE) * hd;
        }
        if (bad) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = bad;
            free(o); free(s); free(base);
            continue;
        }
        /* s_p = sum_d q_d k_{p,d} */
        double m = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int64_t d = 0; d < hd; ++d)
                acc += bf16_to_f64(qrow[d]) * bf16_to_f64(k_pool[base[i] + d]);
            s[i] = acc;
            if (acc > m)
                m = acc;
        }
        /* e_p = exp(s_p - m), z = sum_p e_p */
        double z = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            s[i] = exp(s[i] - m);
            z += s[i];
        }
        /* o_d = sum_p (e_p / z) v_{p,d}, p ascending for every d */
        for (int64_t i = 0; i < n; ++i) {
            const double w = s[i] / z;
            for (int64_t d = 0; d < hd; ++d)
                o[d] += w * bf16_to_f64(v_pool[base[i] + d]);
        }
        for (int64_t d = 0; d < hd; ++d) {
            orow[d] = oracle_f64_to_bf16(o[d]);
            if (out_f64)
                out_f64[(t * nh + h) * hd + d] = o[d];
        }
        free(o); free(s); free(base);
    }
    return status;
}

/* rel-RMS of a against reference b, both bf16 bit patterns, accumulated in f64:
 * sqrt(sum (a-b)^2 / max(sum b^2, 1e-30)) -- the span-02 test's `rel_rms`. */
double pgqa_oracle_rel_rms(const uint16_t *a, const uint16_t *b, int64_t n)
{
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double x = bf16_to_f64(a[i]), y = bf16_to_f64(b[i]);
        num += (x - y) * (x - y);
        den += y * y;
    }
    return sqrt(num / (den > 1e-30 ? den : 1e-30));
}

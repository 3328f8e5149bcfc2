/*
 * Plain CPU oracle for paged grouped-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call this.  It shares no code, header or
 * constant with the HIP library and must never stand in for it.
 *
 * What is computed is the definition of the span-02 GPU kernel test page
 * (respanai/span-02, engine/crates/kernels/tests/gpu.rs): the quantities of its
 * `reference` function, extended to the decode call's full contract (per-row
 * page origins, a page map, a last-visible-key array).  For query row t and
 * query head h:
 *   - kv head kh = h / (nh / nkv) (grouped-query sharing);
 *   - visible keys p: lo_t <= p <= hi_t, lo_t = max(0, qpos_t + 1 - window)
 *     for a sliding layer (window > 0), else 0; hi_t = the row's last visible
 *     key (the page passes the query positions there, so hi_t = qpos_t in
 *     every call it shows);
 *   - score s_p = q_t,h . k_p (scale 1.0, no 1/sqrt(hd));
 *   - out_t,h = sum_p softmax(s)_p v_p = N / Z with, for any shift c,
 *       N = sum_p exp(s_p - c) v_p,   Z = sum_p exp(s_p - c).
 *     The shift c is the largest visible score, so no exponential overflows.
 *   - every bf16 input is widened exactly; scores, exponentials, N and Z are
 *     f64; out = N_d / Z is rounded once to bf16, nearest-even.  (The page's
 *     own rounding helper truncates; nearest-even is the reading taken, the two
 *     differ by at most one bf16 ulp.)
 * Addressing (same page: pool layout [page][nkv][16][hd] and its page-map
 * helper): the row's table starts at entry page_origin[t]; logical page
 * j = p / 16 lives at physical page block_table[origin + j] (then
 * page_map[that] when a map is given), slot p % 16.
 *
 * The visible keys are walked page by page in increasing position; within a
 * key the hd products are summed in increasing d.  No blocking, fusion or
 * reordering beyond that.  Built without -ffast-math, with -ffp-contract=off.
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

/* One (row, head): the element offsets of its visible keys' K/V rows, then the
 * shifted exponentials and the unnormalised sum.  Returns 0, or a negative
 * addressing error. */
static int attend_one(uint16_t *orow, double *ofrow, const uint16_t *qrow,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      const int32_t *block_table, int64_t table_len, int64_t origin,
                      const int32_t *page_map, int64_t map_len, int64_t npages,
                      int64_t nkv, int64_t kh, int64_t hd, int64_t lo, int64_t hi,
                      int64_t *row_at, double *score, double *num)
{
    int64_t n = 0;
    /* resolve the keys one page at a time: table entry -> (map) -> pool page */
    for (int64_t page = lo >= 0 ? lo / ORACLE_PAGE : 0; hi >= lo && page <= hi / ORACLE_PAGE; ++page) {
        const int64_t entry = origin + page;
        if (entry < 0 || entry >= table_len)
            return -2;
        int64_t phys = block_table[entry];
        if (page_map) {
            if (phys < 0 || phys >= map_len)
                return -4;
            phys = page_map[phys];
        }
        if (phys < 0 || phys >= npages)
            return -3;
        const int64_t first = page * ORACLE_PAGE > lo ? page * ORACLE_PAGE : lo;
        const int64_t last = page * ORACLE_PAGE + ORACLE_PAGE - 1 < hi ? page * ORACLE_PAGE + ORACLE_PAGE - 1 : hi;
        for (int64_t p = first; p <= last; ++p)
            row_at[n++] = ((phys * nkv + kh) * ORACLE_PAGE + p % ORACLE_PAGE) * hd;
    }
    double top = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        double dot = 0.0;
        for (int64_t d = 0; d < hd; ++d)
            dot += bf16_to_f64(qrow[d]) * bf16_to_f64(k_pool[row_at[i] + d]);
        score[i] = dot;
        top = dot > top ? dot : top;
    }
    for (int64_t d = 0; d < hd; ++d)
        num[d] = 0.0;
    double z = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double e = exp(score[i] - top);
        z += e;
        const uint16_t *vrow = v_pool + row_at[i];
        for (int64_t d = 0; d < hd; ++d)
            num[d] += e * bf16_to_f64(vrow[d]);
    }
    for (int64_t d = 0; d < hd; ++d) {
        const double o = n > 0 ? num[d] / z : 0.0;   /* nothing visible: 0 */
        orow[d] = oracle_f64_to_bf16(o);
        if (ofrow)
            ofrow[d] = o;
    }
    return 0;
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
        const int64_t qp = qpos[t];
        int64_t lo = 0;
        if (window > 0 && qp + 1 - window > 0)
            lo = qp + 1 - window;
        const int64_t hi = kv_last[t];
        const int64_t n = hi >= lo ? hi - lo + 1 : 0;
        int64_t *row_at = malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        double *score = malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        double *num = malloc((size_t)hd * sizeof(double));
        int rc = -5;
        if (row_at && score && num)
            rc = attend_one(out + job * hd, out_f64 ? out_f64 + job * hd : NULL, q + job * hd,
                            k_pool, v_pool, block_table, table_len, page_origin[t], page_map, map_len,
                            npages, nkv, h / group, hd, lo, hi, row_at, score, num);
        if (rc != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = rc;
        }
        free(row_at);
        free(score);
        free(num);
    }
    return status;
}

/* Root-mean-square difference of a from the reference b, relative to the
 * root-mean-square of b, both bf16 bit patterns, in f64.  A zero reference
 * gives 0 when a equals it and +inf otherwise. */
static double rel_rms_span(const uint16_t *a, const uint16_t *b, int64_t n)
{
    double diff2 = 0.0, ref2 = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double y = bf16_to_f64(b[i]);
        const double dv = bf16_to_f64(a[i]) - y;
        diff2 += dv * dv;
        ref2 += y * y;
    }
    if (ref2 == 0.0)
        return diff2 == 0.0 ? 0.0 : INFINITY;
    return sqrt(diff2 / ref2);
}

double pgqa_oracle_rel_rms(const uint16_t *a, const uint16_t *b, int64_t n)
{
    return rel_rms_span(a, b, n);
}

/* The same measure for each of nvec consecutive vectors of len elements
 * (e.g. every (row, head) output row of hd values). */
void pgqa_oracle_rel_rms_each(const uint16_t *a, const uint16_t *b, int64_t nvec, int64_t len, double *out)
{
    for (int64_t i = 0; i < nvec; ++i)
        out[i] = rel_rms_span(a + i * len, b + i * len, len);
}

/*
 * Plain CPU oracle for the QK-norm + RoPE prep that fills the paged KV pool.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call this.  It shares no code, header or
 * constant with the HIP library and must never stand in for it.
 *
 * Source: the pegainfer pull request page #1002 ("reduce the duplicated CPU
 * operator oracles in the HD256/HD512 QK-RoPE smokes"), its description of
 * the operator the QK-RoPE gates check: RMSNorm of the query and key heads
 * with norm weights, rotary embedding from position tables over the first
 * rotary_dim elements as a low and a high half, a pass-through tail when
 * rotary_dim < hd, a weightless norm for V (and V taken from the K input in
 * the hd-512 "K = V" form), and the results landing at paged-pool layout
 * addresses through per-token page origins.  The page prints no formulas; the
 * plainest reading is taken, written out here per (token, head):
 *
 *   x_d      = the bf16 input, widened exactly to f64           (d < hd)
 *   r        = 1 / sqrt( (sum_d x_d^2) / hd + eps )             (sum in d order)
 *   n_d      = x_d * r * w_d       (w_d = 1 for V or a NULL weight)
 *   h        = rotary_dim / 2,  c_i = cos[pos][i],  s_i = sin[pos][i] (f32 table
 *              entries widened; i < h)
 *   y_i      = n_i c_i - n_{i+h} s_i                            (i < h)
 *   y_{i+h}  = n_{i+h} c_i + n_i s_i                            (i < h)
 *   y_d      = n_d                                              (d >= rotary_dim)
 *   V heads are never rotated.
 *   out      = y rounded once from f64 to bf16, nearest-even.
 *
 * Addressing (the same as the decode oracle's): the token's table entry is
 * page_origin[token] + pos / 16, its physical page block_table[entry] (then
 * page_map[that] when a map is given), and head kh of K (or V) lands at
 * element ((phys * nkv + kh) * 16 + pos % 16) * hd + d of the pool.  Nothing
 * else in the pools is written.
 *
 * Built without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_PAGE 16

uint16_t oracle_f64_to_bf16(double x); /* pgqa_oracle.c: correctly rounded f64 -> bf16 */

static double widen_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * RMSNorm of one head, then the rotation of its first rotary_dim elements
 * (rotary_dim 0: none).  y receives hd f64 values.
 */
static void norm_rotate(double *y, const uint16_t *x_bf16, const uint16_t *w_bf16, int64_t hd,
                        const float *cos_row, const float *sin_row, int64_t rotary_dim, double eps)
{
    double ss = 0.0;
    for (int64_t d = 0; d < hd; ++d) {
        double x = widen_bf16(x_bf16[d]);
        ss += x * x;
    }
    double r = 1.0 / sqrt(ss / (double)hd + eps);
    double n[512];
    for (int64_t d = 0; d < hd; ++d) {
        double w = w_bf16 ? widen_bf16(w_bf16[d]) : 1.0;
        n[d] = widen_bf16(x_bf16[d]) * r * w;
    }
    int64_t h = rotary_dim / 2;
    for (int64_t i = 0; i < h; ++i) {
        double c = (double)cos_row[i], s = (double)sin_row[i];
        y[i] = n[i] * c - n[i + h] * s;
        y[i + h] = n[i + h] * c + n[i] * s;
    }
    for (int64_t d = rotary_dim; d < hd; ++d)
        y[d] = n[d];
}

/*
 * Error codes: 0 ok; -1 bad shape; -2 table index out of range; -3 page out of
 * range; -4 page-map index out of range; -5 position outside the RoPE tables
 * (or negative).
 *
 * q_out      bf16 [tokens][nh][hd]; q_f64 (optional) the same before rounding
 * k_pool, v_pool  bf16 [npages][nkv][16][hd], written only at the tokens' slots
 * k_f64, v_f64    optional f64 shadows of the pools, written at the same places
 * v_in       NULL: V is taken from k_in (the K = V form)
 * q_w, k_w   bf16 [hd] or NULL (weight 1)
 * rope_cos, rope_sin  f32 [table_rows][rotary_dim / 2]
 */
int pgqa_oracle_qk_rope_prep(uint16_t *q_out, double *q_f64, uint16_t *k_pool, uint16_t *v_pool,
                             double *k_f64, double *v_f64,
                             const uint16_t *q_in, const uint16_t *k_in, const uint16_t *v_in,
                             const uint16_t *q_w, const uint16_t *k_w,
                             const float *rope_cos, const float *rope_sin, int64_t table_rows,
                             const int32_t *pos, const int32_t *block_table, int64_t table_len,
                             const int32_t *page_origin, const int32_t *page_map, int64_t map_len,
                             int64_t npages, int64_t tokens, int64_t nh, int64_t nkv, int64_t hd,
                             int64_t rotary_dim, double eps)
{
    if (tokens < 0 || nh < 1 || nkv < 1 || hd < 2 || hd > 512 || rotary_dim < 0 || rotary_dim > hd ||
        rotary_dim % 2 != 0 || !(eps >= 0.0))
        return -1;
    int64_t h = rotary_dim / 2;
    double y[512];
    for (int64_t t = 0; t < tokens; ++t) {
        int64_t p = pos[t];
        if (p < 0 || (rotary_dim > 0 && p >= table_rows))
            return -5;
        const float *cr = rotary_dim > 0 ? rope_cos + p * h : NULL;
        const float *sr = rotary_dim > 0 ? rope_sin + p * h : NULL;

        for (int64_t qh = 0; qh < nh; ++qh) {
            int64_t base = (t * nh + qh) * hd;
            norm_rotate(y, q_in + base, q_w, hd, cr, sr, rotary_dim, eps);
            for (int64_t d = 0; d < hd; ++d) {
                q_out[base + d] = oracle_f64_to_bf16(y[d]);
                if (q_f64)
                    q_f64[base + d] = y[d];
            }
        }

        int64_t entry = (int64_t)page_origin[t] + p / ORACLE_PAGE;
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
        for (int64_t kh = 0; kh < nkv; ++kh) {
            int64_t src = (t * nkv + kh) * hd;
            int64_t dst = ((phys * nkv + kh) * ORACLE_PAGE + p % ORACLE_PAGE) * hd;
            norm_rotate(y, k_in + src, k_w, hd, cr, sr, rotary_dim, eps);
            for (int64_t d = 0; d < hd; ++d) {
                k_pool[dst + d] = oracle_f64_to_bf16(y[d]);
                if (k_f64)
                    k_f64[dst + d] = y[d];
            }
            norm_rotate(y, (v_in ? v_in : k_in) + src, NULL, hd, NULL, NULL, 0, eps);
            for (int64_t d = 0; d < hd; ++d) {
                v_pool[dst + d] = oracle_f64_to_bf16(y[d]);
                if (v_f64)
                    v_f64[dst + d] = y[d];
            }
        }
    }
    return 0;
}

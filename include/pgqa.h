/*
 * pgqa — paged grouped-query decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpgqa.so.  Plain pointers and sizes only; no framework types.
 *
 * Source of the contract: the span-02 GPU kernel test page
 * (respanai/span-02, engine/crates/kernels/tests/gpu.rs), function `run()`:
 * its `attn::choose_splits`, `attn::decode_part_bytes` and `attn::attn_decode`
 * calls fix the argument list and order, the pool layout, the 4096-entry
 * counter buffer, the "null counters selects a separate combine kernel" rule
 * and the page-map argument.  The page does not give the split rule, the
 * partial-buffer size formula or the second position array's meaning; the
 * readings taken here are stated at each declaration.
 *
 * Conventions for every entry point:
 *   - Device pointers point to memory of the current HIP device, owned by the
 *     caller.  The library allocates nothing and never synchronises: work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns.
 *   - bf16 tensors are arrays of uint16_t bit patterns.
 *   - A negative return code means the call was refused *before* anything was
 *     enqueued (buffers untouched); pgqa_last_error() then describes why.
 */
#ifndef PGQA_H
#define PGQA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PGQA_OK 0
#define PGQA_EINVAL (-1)  /* bad pointer, shape, window or split count           */
#define PGQA_ECAP (-2)    /* more merge units than the counter buffer holds       */
#define PGQA_ELAUNCH (-3) /* the HIP runtime reported an error at launch          */

/* Tokens per KV page; the pool layout fixes it. */
#define PGQA_PAGE 16
/* Largest split count attn_decode accepts. */
#define PGQA_MAX_SPLITS 256

/*
 * Number of KV splits for a decode call (span-02 test page, `run()`: the
 * `choose_splits` call, made with the visible span, the row count, nkv and the
 * row count again).
 *   kv_span      - keys a row can see: min(ctx, window) for a sliding layer,
 *                  ctx otherwise (longest sequence for a batch).
 *   rows         - query rows in the call.
 *   nkv          - kv heads.
 *   rows_per_seq - query rows that share one sequence (one block-table span);
 *                  the page passes `rows` (all rows on one sequence).  Values
 *                  < 1 or > rows are read as rows.
 * Returns a split count in [1, PGQA_MAX_SPLITS].  It only affects speed: every
 * count in that range gives a correct result.  Never fails.
 */
int32_t pgqa_choose_splits(int64_t kv_span, int64_t rows, int64_t nkv, int64_t rows_per_seq);

/*
 * pgqa_choose_splits with the head layout (ours: the page's call passes no
 * head count, and the best count also depends on which kernel the call
 * takes).  Same arguments, plus nh (query heads) and hd (head dimension).
 * Batches (more than one sequence) whose tiles go to the shared-page kernel
 * -- groups of more than 16 query heads per kv head from hd 128 -- hold one
 * workgroup per CU, so the count aims at W = 256 workgroups (one round)
 * below 64 units and W = 512 (two rounds, rows taken longest first) from 64:
 * min(floor(W / units), 16, pages / 16), units = sequences * nkv, at least
 * the short-span count and 1.  Every other call, and arguments that
 * attn_decode would refuse (nh not a multiple of nkv, hd outside
 * {64, 128, 256, 512}), gets pgqa_choose_splits's count.  Returns a count in
 * [1, PGQA_MAX_SPLITS]; it only affects speed.  Never fails.
 */
int32_t pgqa_choose_splits_heads(int64_t kv_span, int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                                 int64_t rows_per_seq);

/*
 * Bytes of the partial-result buffer attn_decode needs for `splits` splits
 * (span-02 test page, `run()`: the `decode_part_bytes` call).  Formula (ours):
 * rows * nh * splits * (hd + 2) * 4 -- an f32 unnormalised output row plus the
 * running max and sum for every (row, query head, split).  Returns 0 for
 * non-positive arguments.  With splits == 1 the buffer is not used.
 */
uint64_t pgqa_decode_part_bytes(int64_t rows, int64_t nh, int64_t splits, int64_t hd);

/*
 * Splits that a tile of a decode call actually works on (ours; the pages
 * leave the split of a row to the implementation).  A tile is a run of rows
 * on one sequence that attn_decode processes together; `pages` is the number
 * of KV pages its rows can see (the pages from the first visible key of any
 * of its rows to the last).  Result: min(splits, ceil(pages / 4)), at least
 * 1, with splits clamped to PGQA_MAX_SPLITS -- so every split of a tile
 * covers at least 4 pages (or all of them), the floor pgqa_choose_splits
 * itself keeps.  Splits of the tile past that
 * count do no work, and the merge reads only the partials of the others; a
 * tile of one split is written without a merge.  Never fails.
 */
int32_t pgqa_tile_splits(int64_t pages, int64_t splits);

/* Entries of int32 the merge-counter buffer must hold: 4096 (span-02 test page,
 * `run()`, the zeroed `cnt` buffer of 4096 * 4 bytes). */
int32_t pgqa_counter_capacity(void);

/*
 * Paged GQA decode attention (span-02 test page, `run()`: the `attn_decode`
 * calls, and the `reference` function for what is computed).
 *
 * For every query row t and query head h, with kv head kh = h / (nh / nkv):
 *   visible keys p:  lo_t <= p <= kv_last[t],
 *                    lo_t = max(0, qpos[t] + 1 - window) if window > 0, else 0
 *   key p's K/V row: pool[phys][kh][p % 16][0..hd), where
 *                    phys = block_table[page_origin[t] + p / 16],
 *                    then phys = page_map[phys] if page_map != NULL
 *   out[t][h][:] = sum_p softmax_p(q[t][h] . K_p) * V_p   (scale 1.0)
 * rounded to bf16 (nearest even); 0 if no key is visible.
 *
 * Arguments (order as on the page, with the stream last):
 *   out         bf16 [rows][nh][hd]                      (written)
 *   part        partial buffer, >= pgqa_decode_part_bytes(rows, nh, splits, hd)
 *               bytes, 4-byte aligned; may be NULL when splits == 1.  Contents
 *               are undefined after the call.
 *   q           bf16 [rows][nh][hd]
 *   k_pool      bf16 [npages][nkv][16][hd]
 *   v_pool      bf16 [npages][nkv][16][hd]
 *   block_table int32 page ids; row t's table starts at entry page_origin[t]
 *   page_origin int32 [rows]
 *   qpos        int32 [rows] query positions (the window is anchored here)
 *   kv_last     int32 [rows] last visible key per row.  The page passes the
 *               query positions again here (causal decode); only
 *               kv_last == qpos is checked against its reference.
 *   rows, nh, nkv, hd  shapes: nh % nkv == 0, hd in {64, 128, 256, 512}
 *   window      0 = global causal, > 0 = sliding window of that many keys
 *   splits      1..PGQA_MAX_SPLITS, normally from pgqa_choose_splits; a tile
 *               of rows works on pgqa_tile_splits(its pages, splits) of them
 *   counters    NULL: a separate combine kernel merges the splits.  Non-NULL:
 *               int32 [pgqa_counter_capacity()], all zero before the first
 *               call, and the merge happens inside the decode launch: the last
 *               workgroup of each merge unit merges and resets its counter;
 *               when one unit's merge would read 64 KB or more of partials
 *               (hd 256 and up in the per-wave kernel), the unit's
 *               workgroups wait briefly (at most 20 us each, see
 *               pgqa_set_merge_wait_ticks) for the last one and merge it
 *               together, each its own blocks, through three counter words
 *               per unit (entries unit, 2048 + unit and 3072 + unit, so
 *               at most 1024 such units).  Either way the buffer is all zero again when
 *               the call completes and can be reused without clearing.  The
 *               result is the same as with NULL counters, bit for bit.  For
 *               calls with one or two merge units and many splits the
 *               separate combine kernel is the faster choice.
 *   page_map    NULL, or int32 indexed by block-table entries (see above)
 *   stream      hipStream_t
 *
 * The caller guarantees: every block-table entry, page-map entry and pool page
 * reached for a visible key is in range (pages that hold no visible key of any
 * row sharing the origin are never read, so they may point anywhere -- e.g. at
 * a NaN-filled null page); the K/V rows of visible keys are finite.
 * Rows that share an origin and sit next to each other are processed together
 * and read each KV page once.  Bitwise properties, for a given split count:
 * the result does not depend on `counters` (fused merge == separate combine),
 * nor on where pages live in the pool (identity table == permuted pool behind
 * a page map).  Different split counts may differ in the last bits (calls
 * whose tiles all get the same pgqa_tile_splits counts give the same bits).
 * `out` must not alias any input or `part`.  Calls that share `part` or
 * `counters` must not run concurrently.
 * Returns PGQA_OK, PGQA_EINVAL (also for shapes whose launch grid would
 * exceed 2^32 - 1 threads), PGQA_ECAP (counters given and
 * rows * nkv * ceil(nh / nkv / 16) > pgqa_counter_capacity()) or PGQA_ELAUNCH.
 */
int pgqa_attn_decode(void *out, void *part, const void *q, const void *k_pool,
                     const void *v_pool, const int32_t *block_table,
                     const int32_t *page_origin, const int32_t *qpos,
                     const int32_t *kv_last, int64_t rows, int64_t nh, int64_t nkv,
                     int64_t hd, int64_t window, int64_t splits, int32_t *counters,
                     const int32_t *page_map, void *stream);

/* Bytes of partial results pgqa_attn_decode_noalloc can hold: 32 MiB. */
#define PGQA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * pgqa_attn_decode without the caller's partial buffer and counters, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  It allocates
 * nothing: the split partials live in a static device array of
 * PGQA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up once per device, with
 * that device current; no hipMalloc, hipFree or allocating library call),
 * and the splits are merged by the separate combine kernel.
 * Arguments, computation, rounding and return codes: as pgqa_attn_decode with
 * part = the scratch and counters = NULL, so the result is bit for bit that
 * call's for the same split count.  In addition it returns PGQA_EINVAL when
 * splits > 1 and rows * nh * splits * (hd + 2) * 4 exceeds
 * PGQA_NOALLOC_SCRATCH_BYTES (use fewer splits or pgqa_attn_decode), and
 * PGQA_ELAUNCH when the scratch address cannot be had.
 * Every call on one GPU uses that GPU's one scratch array, which keeps the
 * last call's contents (nothing in it needs to start at zero): calls that
 * overlap on one GPU (concurrent streams, other threads) race and must not
 * happen.
 */
int pgqa_attn_decode_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                             const int32_t *block_table, const int32_t *page_origin, const int32_t *qpos,
                             const int32_t *kv_last, int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                             int64_t window, int64_t splits, const int32_t *page_map, void *stream);

/*
 * Rows per prefill tile (span-02 test page, `run()`, the prefill section: the
 * `prefill_rows_per_tile(hd)` argument of `make_tiles`).  64 for every
 * supported hd (the kernels cut a tile further into the rows they hold at
 * once); 0 for an unsupported hd.
 */
int32_t pgqa_prefill_rows_per_tile(int64_t hd);

/*
 * Prefill tiles from the rows' page origins (span-02 test page, `run()`: the
 * `make_tiles` call).  HOST pointers.  Consecutive rows with equal origin
 * form runs; each run is cut into tiles of at most rows_per_tile rows.  Tile
 * n covers rows tile_row0[n] .. tile_row0[n] + tile_rows[n] - 1.
 *   page_origin  int32 [rows]      (host)
 *   rows_per_tile 1 .. pgqa_prefill_rows_per_tile(hd)
 *   tile_row0, tile_rows  int32 [capacity]  (host, written)
 * Returns the number of tiles, PGQA_EINVAL for bad arguments, or PGQA_ECAP
 * when more than `capacity` tiles would be needed.
 */
int64_t pgqa_make_tiles(const int32_t *page_origin, int64_t rows, int64_t rows_per_tile, int32_t *tile_row0,
                        int32_t *tile_rows, int64_t capacity);

/*
 * Paged prefill attention (span-02 test page, `run()`: the `attn_prefill`
 * calls, checked against the same `reference` as decode with every context
 * row causal).  Computes exactly what pgqa_attn_decode computes for the same
 * rows (same visibility rule, pool addressing, page map and rounding), with
 * the rows grouped by the caller's tiles instead of split across KV: each
 * (tile, kv head) is one pass over the tile's pages, with no partials.
 * Arguments as for pgqa_attn_decode, plus:
 *   tile_row0, tile_rows  int32 [ntiles] DEVICE arrays, normally from
 *                pgqa_make_tiles: every tile's rows share one page origin,
 *                1 <= tile_rows[n] <= pgqa_prefill_rows_per_tile(hd), and
 *                the tiles cover rows 0 .. rows - 1 without overlap.  A tile
 *                reaching outside 0 .. rows - 1 is skipped; a tile whose rows
 *                change origin is cut at the change (rows after it are not
 *                written).
 *   ntiles       1 .. rows
 *   rows         query rows (q and out hold rows * nh * hd values); the
 *                page's call leaves it implicit in the tiles.
 * No partial buffer, no counters, no split count.  The result equals
 * pgqa_attn_decode's for the same rows within the rel-RMS bound (not bit for
 * bit: decode may group rows and split keys differently), and is bit for bit
 * the same for an identity pool and a permuted pool behind a page map.
 * Returns PGQA_OK, PGQA_EINVAL or PGQA_ELAUNCH.
 */
int pgqa_attn_prefill(void *out, const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                      const int32_t *page_origin, const int32_t *qpos, const int32_t *kv_last,
                      const int32_t *tile_row0, const int32_t *tile_rows, int64_t ntiles, int64_t rows, int64_t nh,
                      int64_t nkv, int64_t hd, int64_t window, const int32_t *page_map, void *stream);

/*
 * QK-norm + RoPE prep: the step before decode that fills the paged pool
 * (pegainfer pull request page #1002, the HD256/HD512 QK-RoPE gates: RMSNorm
 * of the query and key heads with norm weights, rotary embedding from
 * position tables over the first rotary_dim elements as a low and a high
 * half with a pass-through tail, a weightless norm for V, V from the K input
 * in the hd-512 "K = V" form, the results landing at the paged layout's
 * addresses through per-token page origins).  The page prints no formulas;
 * the reading taken, per token t and head:
 *   n_d = x_d * w_d / sqrt(sum_d(x_d^2) / hd + eps)   (w_d = 1: V, or no weight)
 *   for i < rotary_dim / 2, h = rotary_dim / 2, c = cos[pos_t][i], s = sin[pos_t][i]:
 *     y_i = n_i c - n_{i+h} s,   y_{i+h} = n_{i+h} c + n_i s
 *   y_d = n_d for d >= rotary_dim; V heads are never rotated.
 * Computed in f32, stored as bf16 rounded to nearest even.
 *   q_out        bf16 [tokens][nh][hd]: the rotated query heads.  May be q_in
 *                itself (in place); must not overlap anything else.
 *   k_pool, v_pool  bf16 [npages][nkv][16][hd]: kv head kh of token t is
 *                written at page phys = block_table[page_origin[t] + pos[t] / 16]
 *                (then page_map[phys] when page_map is not NULL), slot
 *                pos[t] % 16 -- the addressing pgqa_attn_decode reads.  Nothing
 *                else in the pools is touched.  Two tokens with the same slot
 *                race.
 *   q_in         bf16 [tokens][nh][hd];  k_in bf16 [tokens][nkv][hd]
 *   v_in         bf16 [tokens][nkv][hd], or NULL: V is normalised from k_in
 *   q_weight, k_weight  bf16 [hd] norm weights, or NULL for weight 1
 *   rope_cos, rope_sin  f32 [positions][rotary_dim / 2] (row pos[t] is read);
 *                may be NULL when rotary_dim is 0
 *   pos          int32 [tokens], >= 0 (and < the tables' rows when rotating)
 *   block_table, page_origin (int32 [tokens]), page_map: as for decode; the
 *                caller guarantees every reached entry and page is valid
 *   rotary_dim   a multiple of 16 in 0 .. hd;  eps finite, >= 0
 * Every bf16 buffer and both tables must be 16-byte aligned.  tokens == 0
 * enqueues nothing.  Returns PGQA_OK, PGQA_EINVAL or PGQA_ELAUNCH.
 */
int pgqa_qk_rope_prep(void *q_out, void *k_pool, void *v_pool, const void *q_in, const void *k_in, const void *v_in,
                      const void *q_weight, const void *k_weight, const float *rope_cos, const float *rope_sin,
                      const int32_t *pos, const int32_t *block_table, const int32_t *page_origin,
                      const int32_t *page_map, int64_t tokens, int64_t nh, int64_t nkv, int64_t hd,
                      int64_t rotary_dim, float eps, void *stream);

/*
 * Test hook for the fused merge's give-up path (no page defines it).  When one
 * merge unit's partials reach 2 MB, the unit's workgroups merge it together,
 * each waiting at most `ticks` ticks of the GPU's 100 MHz real-time counter
 * for the unit's last arrival before it leaves the merge to the others (the
 * last arrival merges whatever nobody took).  Any ticks >= 1 gives the same
 * result bit for bit; it only changes how the work is shared.  0 restores the
 * default (2000 ticks = 20 us).  Applies to the calls enqueued after it, from
 * any thread.  Returns the previous setting, or PGQA_EINVAL for ticks < 0.
 */
int32_t pgqa_set_merge_wait_ticks(int32_t ticks);

/*
 * Test hook for the two page steps of narrow tiles (no page defines it).
 * Tiles of at most 4 columns (columns = rows of the tile x heads per kv
 * head) at hd 64, 128 and 256 can run their scores and P.V either on MFMA, in
 * 16-column blocks of which the tile fills at most 4, or on the vector ALU
 * with packed bf16 dot products.  mode 0 (the default) takes the vector-ALU
 * step at hd 64 and 128 in launches of more than 512 workgroups and MFMA
 * otherwise; 1 takes the vector-ALU step wherever it applies (hd 256
 * included); 2 never.  The two steps round differently, so their outputs
 * differ in the last bits; each matches the definition to the same bound.
 * Applies to the calls enqueued after it, from any thread.  Returns the
 * previous mode, or PGQA_EINVAL for a mode outside 0..2.
 */
int32_t pgqa_set_narrow_path(int32_t mode);

/* Message for the last non-zero return on this thread ("" if none). */
const char *pgqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PGQA_H */

// Paged grouped-query decode (and prefill) attention for CDNA4 (gfx950):
// kernels + C ABI.
//
// What is computed is fixed by the span-02 GPU kernel test page
// (respanai/span-02, engine/crates/kernels/tests/gpu.rs): its `reference`
// function (scale 1.0, kv head h / (nh / nkv), causal with an optional sliding
// window, pool [page][nkv][16][hd]) and its `attn_decode` / `attn_prefill`
// calls (block table with per-row origins, split partials merged by the last
// workgroup through a counter or by a separate combine kernel, optional page
// map whose out-of-window pages may point at a NaN-filled null page).  The
// page shows no kernel code; everything below is designed for MI355X.
//
// Work decomposition
//   * A "tile" is a run of consecutive rows that share a page origin (rows of
//     one sequence).  Its query heads for one kv head form "columns" (row,
//     head); one tile reads each KV page once for all of its columns.  Groups
//     wider than a tile are cut into head blocks.
//   * Scores are S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 tokens x 16
//     columns); the softmax weights come out laid out as the A operand of
//     v_mfma_f32_16x16x16_bf16, so P V needs no shuffle of P; V reaches the B
//     operand through the LDS transpose read; a column of ones appended to V
//     yields the softmax denominators from the same MFMA.
//   * pgqa_wave_kernel (hd 64 to 256): 16-column tiles, 4 waves each taking
//     every 4th page of the split with their own softmax state (K straight
//     from HBM into MFMA operand registers); narrow groups, batched decode.
//     Its vector-ALU form takes tiles of at most 4 columns in large launches:
//     packed bf16 dot products and DPP sums instead of mostly empty MFMA
//     tiles, K and V both straight into registers.
//   * pgqa_slice_kernel (hd 512, tiles of up to 16 columns): the 4 waves take
//     every page, each a quarter of hd, with RING pages in flight per wave in
//     registers; the partial scores are summed through LDS, so all waves hold
//     one softmax state and no cross-wave merge is needed; one-row and
//     few-row decode of wide heads.
//   * pgqa_shared_kernel: up to 64-column tiles, 8 waves in two teams taking
//     alternating pages staged in LDS by direct-to-LDS loads; groups of 8+
//     with several rows, hd-512 tiles of more than 16 columns.  Its WIDE form
//     (prefill) gives the teams separate column blocks of a tile twice as
//     wide, both computing every page.
//   * With S splits, each (tile, kv head, head block, split) workgroup writes
//     an f32 partial (o, m, l); the merge (fixed order: 8 interleaved groups of
//     splits, each an fma chain) runs in the last workgroup of the unit, in
//     all of the unit's workgroups together (large merges: each its own
//     32-element blocks, one wave per block), or in the separate combine
//     kernel -- the same arithmetic per element, so the same bits.
//   * Masked scores are replaced by -inf with a select and V rows of tokens no
//     column can see are zeroed with a select, so a NaN page or NaN slot outside
//     every window cannot leak into the result.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <type_traits>
#include <utility>

#include "errors.h"
#include "pgqa.h"

// Bytes of the allocation-free entry point's partial-result scratch, and the
// scratch itself (see noalloc_scratch).
constexpr uint64_t kNoAllocScratchBytes = uint64_t(PGQA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace pgqa_detail {
namespace {
thread_local char g_error[512] = "";
}  // namespace

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

const char *error_text() { return g_error; }
}  // namespace pgqa_detail

namespace {

constexpr int kPage = PGQA_PAGE;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSplits = PGQA_MAX_SPLITS;
constexpr int kCounterCap = 4096;
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

struct DecodeArgs {
  uint16_t *out;
  float *part_o;   // [rows][nh][splits][hd]
  float *part_ml;  // [rows][nh][splits][2] = (running max in log2 units, sum)
  const uint16_t *q;
  const uint16_t *k_pool;
  const uint16_t *v_pool;
  const int32_t *block_table;
  const int32_t *page_origin;
  const int32_t *qpos;
  const int32_t *kv_last;
  int32_t *counters;
  const int32_t *page_map;
  int rows, nh, nkv, group, window, splits, rmax, hblocks;
  int cap;  // columns per tile: 16 (per-wave kernel) or 16 * column blocks (shared-page kernel)
  int rank_rows;  // take rows longest first (large launches; the shared-page kernel with one-row tiles)
  int spin_ticks;  // fused merge: > 0 selects the parallel (owned-block) merge and bounds each
                   // workgroup's wait for the unit's last arrival (100 MHz ticks)
  // prefill: caller-made tiles (runs of rows on one sequence, at most
  // kPrefillRowsPerTile rows each), cut into nsub sub-tiles of rmax rows;
  // NULL for decode
  const int32_t *tile_row0;
  const int32_t *tile_nrows;
  int ntiles, nsub;
};

// Orders this wave's LDS accesses around the point (a wave executes its LDS
// instructions in order, so only compiler reordering has to be prevented).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16-byte direct load global -> LDS: every lane's 16 bytes land at
// lds_base + 16 * lane (lds_base must be the same for the whole wave).
__device__ __forceinline__ void load_to_lds16(const void *src, void *lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16) of a tile that direct-to-LDS loads
// filled: within each 16-lane group, lane i receives elements i, i+16, i+32 and
// i+48 of the group's concatenated 8-byte rows.  Written as inline assembly
// because the compiler's own form of this read carries no record of which LDS
// object it reads, so the compiler would wait for every direct load still in
// flight (the whole prefetch ring) before it; here the caller waits instead:
// results are valid only after lds_wait_reads().
template <int OFFSET>
__device__ __forceinline__ s16x4 lds_read_tr16(uint32_t lds_addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(OFFSET));
  return r;
}
__device__ __forceinline__ void lds_wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// Workgroup barrier for LDS exchanges only: waits for this wave's LDS traffic,
// not for its vector-memory loads (which stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// Four softmax weights -> bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ s16x4 pack_weights(float p0, float p1, float p2, float p3) {
  const bf16x2 lo = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
  const bf16x2 hi = __builtin_convertvector(f32x2{p2, p3}, bf16x2);
  const unsigned u0 = __builtin_bit_cast(unsigned, lo), u1 = __builtin_bit_cast(unsigned, hi);
  return s16x4{static_cast<short>(u0 & 0xffff), static_cast<short>(u0 >> 16), static_cast<short>(u1 & 0xffff),
               static_cast<short>(u1 >> 16)};
}

// Two bf16 packed in a 32-bit word, as the operand of v_dot2_f32_bf16.  (A
// bit cast applied directly to an element of a vector value compiled to a
// read of element 0 with this toolchain; the copy goes through a scalar.)
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned u) {
  bf16x2 r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

// DPP lane moves within 16-lane rows: row_ror:8 (lane i <- i ^ 8),
// row_half_mirror (i <- 7 - i within 8), quad_perm [2,3,0,1] (i <- i ^ 2) and
// [1,0,3,2] (i <- i ^ 1).
constexpr int kDppRor8 = 0x128, kDppHalfMirror = 0x141, kDppXor2 = 0x4E, kDppXor1 = 0xB1;
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// One level of a transposing sum over lane pairs (i, partner(i)) whose
// `upper` flags differ: of its N values the lane keeps the upper half if
// `upper`, else the lower, and adds the partner's copy of that half.  After
// log2(N) such levels over distinct lane bits each lane holds one full sum,
// the one whose index has the lane's bits.
template <int CTRL, int N>
__device__ __forceinline__ void fold_half(float *v, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float lo = v[i], hi = v[i + N / 2];
    const float keep = upper ? hi : lo, send = upper ? lo : hi;
    v[i] = keep + dpp_move<CTRL>(send);
  }
}
// The same level for partners across rows (lane ^ OFF, OFF 16 or 32).
template <int OFF, int N>
__device__ __forceinline__ void fold_half_xor(float *v, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float lo = v[i], hi = v[i + N / 2];
    const float keep = upper ? hi : lo, send = upper ? lo : hi;
    v[i] = keep + __shfl_xor(send, OFF);
  }
}

// Agent-coherent 32-bit accesses for the partial results.  The stores go past
// this XCD's L2 (write-through), so the fused merge needs no L2 write-back
// fence -- its ordering comes from waiting for the stores to complete before
// the counter ticket, and from the ticket's result gating the loads -- and a
// launch that leaves its partials for the combine kernel ends without
// megabytes of dirty L2 lines to write back.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
struct LoadPlain {
  __device__ __forceinline__ float operator()(const float *p) const { return *p; }
};
struct LoadCoherent {
  __device__ __forceinline__ float operator()(const float *p) const {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// ---- cross-split merge -------------------------------------------------
// The merge of S split partials (o_s[hd], m_s, l_s) of one (row, query head):
//   M   = max m_s over non-empty splits (l_s > 0),  w_s = exp2(m_s - M) (else 0)
//   num = sum_g ( sum_{s = g mod 8, s ascending} w_s o_s[d] ),  g = 0..7 in order
//   den = the same grouping over w_s l_s,  out = num / den  (0 if den == 0).
// The eight strided groups let the loads of a merge run in parallel; the order
// is fixed, and both the fused last-workgroup merge and the combine kernel
// take exactly these steps per output element, so the two paths give the same
// bits.
constexpr int kMergeGroups = 8;

// LDS scratch of the fused merge: weights and sums of up to NT (column,
// split) pairs, per-column max and denominator (NT = workgroup size).
template <int NT>
struct FusedScratch {
  float w[NT];
  float l[NT];
  float mx[NT];
  float den[NT];
};

// Column c (0 .. cap-1) of a tile -> (row offset, head within the kv group),
// or off if the tile has no such column.  A group of at most `cap` heads keeps
// whole rows in a tile; a wider group is cut into head blocks of `cap`.
struct Column {
  int row, head;
  bool on;
};
__device__ __forceinline__ Column tile_column(int c, int group, int nrows, int hb, int cap) {
  Column col;
  if (group <= cap) {
    col.row = c / group;
    col.head = c - col.row * group;
    col.on = col.row < nrows;
  } else {
    col.row = 0;
    col.head = hb * cap + c;
    col.on = col.head < group;
  }
  return col;
}

// Rows t0 .. t0+nrows-1 (nrows <= rmax) that share row t0's page origin and
// stay inside one rmax-aligned block.  Lane r < rmax keeps row t0 + r's
// visible range [lo_l, hi_l]; lo_min / hi_max span the tile's rows.  A
// workgroup whose t0 does not start a tile has nothing to do (lead false).
struct Tile {
  int origin, nrows, lo_l, hi_l, lo_min, hi_max;
  int fp0, fp1;  // pages [fp0, fp1) are visible in full to every row of the tile
  bool lead;
};
// With force_rows > 0 (prefill) the tile is rows t0 .. t0 + force_rows - 1 as
// the caller cut them, shortened to the run that shares row t0's origin.
// The tile from lane l's row t0 + l (lrow: that row exists and is within
// the tile's span; org_l, qp_l, hi_l: its page origin, query position and
// last visible key) and row t0 - 1's origin.
__device__ __forceinline__ Tile tile_from(const DecodeArgs &a, int t0, int lane, int force_rows, bool lrow, int org_l,
                                          int qp_l, int hi_l, int prev_origin) {
  Tile t;
  t.hi_l = lrow ? hi_l : -1;
  t.origin = __builtin_amdgcn_readfirstlane(org_l);
  if (force_rows > 0) {
    t.lead = true;
    const uint64_t stop = __ballot(lane >= 1 && (!lrow || org_l != t.origin));
    t.nrows = stop ? static_cast<int>(__builtin_ctzll(stop)) : 64;
  } else {
    t.lead = t0 % a.rmax == 0 || prev_origin != t.origin;
    const uint64_t stop = __ballot(lane >= 1 && (!lrow || org_l != t.origin || (t0 + lane) % a.rmax == 0));
    t.nrows = stop ? static_cast<int>(__builtin_ctzll(stop)) : 64;
  }
  t.lo_l = a.window > 0 ? max(0, qp_l + 1 - a.window) : 0;
  const bool live = lane < t.nrows && t.hi_l >= t.lo_l;
  int lo = live ? t.lo_l : INT_MAX, hi = live ? t.hi_l : -1;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off));
    hi = max(hi, __shfl_xor(hi, off));
  }
  t.lo_min = __builtin_amdgcn_readfirstlane(lo);
  t.hi_max = __builtin_amdgcn_readfirstlane(hi);
  int lo_all = lane < t.nrows ? t.lo_l : INT_MIN, hi_all = lane < t.nrows ? t.hi_l : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo_all = max(lo_all, __shfl_xor(lo_all, off));
    hi_all = min(hi_all, __shfl_xor(hi_all, off));
  }
  lo_all = __builtin_amdgcn_readfirstlane(lo_all);
  hi_all = __builtin_amdgcn_readfirstlane(hi_all);
  t.fp0 = (lo_all + kPage - 1) / kPage;
  t.fp1 = hi_all >= lo_all ? (hi_all + 1) / kPage : t.fp0;
  return t;
}

// Launches of at most 64 rows that rank them (large launches, whose later
// workgroups start while the earlier ones stream): every row's page origin,
// query position and last visible key read once through the scalar cache,
// into lane r = row r.  A workgroup that starts while the others stream K/V waits
// behind their loads in the vector memory queue (measured on the batched
// decode: 12-27 us per dependent round trip); scalar loads take another
// path, and the tile is then built from these lanes without a second load.
// Whole 16-row chunks are read with one wide load per array, the rest row
// by row: nothing past row rows - 1 is read.
struct LaneRows {
  int org, qp, kl;
};
typedef const __attribute__((address_space(4))) int32_t ScalarInt;
__device__ __forceinline__ LaneRows rows_by_lane(const DecodeArgs &a, int lane) {
  LaneRows m{INT_MIN, 0, -1};
  ScalarInt *po = (ScalarInt *)a.page_origin;
  ScalarInt *pq = (ScalarInt *)a.qpos;
  ScalarInt *pk = (ScalarInt *)a.kv_last;
#pragma unroll
  for (int c = 0; c < 64; c += 16) {
    if (c + 16 <= a.rows) {
      int o[16], q[16], k[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        o[j] = po[c + j];
        q[j] = pq[c + j];
        k[j] = pk[c + j];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (lane == c + j) {
          m.org = o[j];
          m.qp = q[j];
          m.kl = k[j];
        }
      }
    } else if (c < a.rows) {
      // the last, partial chunk: rows past rows - 1 read row rows - 1 again
      // (no branch per row, so the loads are waited for together)
      int o[16], q[16], k[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = min(c + j, a.rows - 1);
        o[j] = po[r];
        q[j] = pq[r];
        k[j] = pk[r];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (lane == c + j && c + j < a.rows) {
          m.org = o[j];
          m.qp = q[j];
          m.kl = k[j];
        }
      }
    }
  }
  return m;
}

// The tile starting at row t0 from the lanes of rows_by_lane.
__device__ __forceinline__ Tile tile_of_lanes(const DecodeArgs &a, const LaneRows &m, int t0, int lane) {
  const int r = min(t0 + lane, 63);
  const bool lrow = lane < a.rmax && t0 + lane < a.rows;
  const int org_l = __shfl(m.org, r), qp_l = __shfl(m.qp, r), hi_l = __shfl(m.kl, r);
  const int prev_origin = t0 > 0 ? __builtin_amdgcn_readlane(m.org, t0 - 1) : INT_MIN;
  return tile_from(a, t0, lane, 0, lrow, org_l, qp_l, hi_l, prev_origin);
}

// The tile starting at row t0, its rows' metadata loaded (vector loads).
__device__ __forceinline__ Tile tile_rows(const DecodeArgs &a, int t0, int lane, int force_rows = 0) {
  const int span = force_rows > 0 ? force_rows : a.rmax;
  const bool lrow = lane < span && t0 + lane < a.rows;
  const int org_l = lrow ? a.page_origin[t0 + lane] : INT_MIN;
  const int qp_l = lrow ? a.qpos[t0 + lane] : 0;
  const int hi_l = lrow ? a.kv_last[t0 + lane] : -1;
  const int prev_origin = force_rows == 0 && t0 > 0 ? a.page_origin[t0 - 1] : INT_MIN;
  return tile_from(a, t0, lane, force_rows, lrow, org_l, qp_l, hi_l, prev_origin);
}

// Prefill: sub-tile p of the launch -> its first row and row count (0: none,
// also for a caller tile that would reach outside rows 0 .. rows - 1).  The
// sub-tiles are taken last first: in a causal prefill the later rows of a
// sequence see the most keys, so the longest work is dispatched first and
// the launch ends on short pieces.
constexpr int kPrefillRowsPerTile = 64;
__device__ __forceinline__ int prefill_subtile(const DecodeArgs &a, int p, int &nrows) {
  p = a.ntiles * a.nsub - 1 - p;
  const int i = p / a.nsub, j = p - i * a.nsub;
  const int r0 = a.tile_row0[i], n = a.tile_nrows[i];
  nrows = 0;
  if (r0 < 0 || n < 1 || n > kPrefillRowsPerTile || r0 > a.rows - n) return 0;
  nrows = max(0, min(a.rmax, n - j * a.rmax));
  return r0 + j * a.rmax;
}

// The row of rank p when the rows are ordered by decreasing visible length
// (ties: lower row first), the same in every lane.  Workgroups take rows in
// this order, so the first dispatched take the longest rows and a batch of
// uneven sequences ends on short pieces of work, not on one long row.  Rank
// selection is a binary search on the length with wave-wide counts.  Small
// launches and batches of more than kRankRows rows keep their own order.
constexpr int kRankRows = 1024;
constexpr int64_t kRankMinBlocks = 512;  // launches this large take rows longest first
constexpr int64_t kSharedRankMinBlocks = 256;  // ... on the shared-page kernel (one workgroup per CU)
constexpr int kRankLenMax = (1 << 30) - 1;  // longer rows rank as equals
__device__ __forceinline__ int row_of_rank(const DecodeArgs &a, int p, int lane) {
  if (!a.rank_rows || a.rows > kRankRows) return p;
  constexpr int R = kRankRows / 64;
  const int nr = (a.rows + 63) / 64;
  int len[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int r = 64 * k + lane;
    len[k] = -1;
    if (k < nr && r < a.rows) {
      const int lo = a.window > 0 ? max(0, a.qpos[r] + 1 - a.window) : 0;
      len[k] = min(max(a.kv_last[r] - lo + 1, 0), kRankLenMax);
    }
  }
  auto count_gt = [&](int x) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < R; ++k)
      if (k < nr) c += __builtin_popcountll(__ballot(len[k] > x));
    return c;
  };
  // smallest length x with at most p rows longer than x: the rank-p length
  int lo_x = -1, hi_x = kRankLenMax;
  while (hi_x - lo_x > 1) {
    const int mid = lo_x + (hi_x - lo_x) / 2;
    if (count_gt(mid) <= p) hi_x = mid;
    else lo_x = mid;
  }
  int q = p - count_gt(hi_x);  // position among the rows of that length
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k < nr) {
      uint64_t m = __ballot(len[k] == hi_x);
      const int c = __builtin_popcountll(m);
      if (q < c) {
        for (int i = 0; i < q; ++i) m &= m - 1;
        return 64 * k + static_cast<int>(__builtin_ctzll(m));
      }
      q -= c;
    }
  }
  return p;  // not reached
}

// row_of_rank from the lanes: the rank of lane r's row is the number of
// rows that see more keys, plus the rows that see as many with a smaller
// index -- the same order.
__device__ __forceinline__ int rank_of_lanes(const DecodeArgs &a, const LaneRows &m, int p, int lane) {
  int len = -1;
  if (lane < a.rows) {
    const int lo = a.window > 0 ? max(0, m.qp + 1 - a.window) : 0;
    len = min(max(m.kl - lo + 1, 0), kRankLenMax);
  }
  int rank = 0;
  for (int j = 0; j < a.rows; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += lj > len || (lj == len && j < lane) ? 1 : 0;
  }
  const uint64_t hit = __ballot(lane < a.rows && rank == p);
  return hit ? static_cast<int>(__builtin_ctzll(hit)) : p;
}

// Split `split` of S covers pages [pbeg, pend) of the tile's visible page
// range [lo_min / 16, hi_max / 16], cut into S contiguous near-equal chunks
// from logical positions only (some may be empty).
__device__ __forceinline__ void split_range(const Tile &t, int split, int splits, int &pbeg, int &pend) {
  pbeg = pend = 0;
  if (t.hi_max >= 0) {
    const int p0 = t.lo_min / kPage;
    const int64_t npg = t.hi_max / kPage - p0 + 1;
    pbeg = p0 + static_cast<int>(npg * split / splits);
    pend = p0 + static_cast<int>(npg * (split + 1) / splits);
  }
}

// Splits a tile uses of the call's S: one per kSplitPages pages of its
// visible page range (at least 1, at most S).  4 pages is the split
// heuristic's own floor (its latency regime), so the counts it chooses are
// kept; a tile far shorter than the call's longest row gives up the rest.  Splits st .. S - 1 of the tile
// do no work: they write no partial -- with the separate combine only an
// empty (m, l) = (-inf, 0) in their slots, which the merge skips exactly --
// and take no part in the fused merge, which reads st partials.  A tile of
// one split writes its output directly when the merge is fused, and its slot
// 0 for the combine otherwise (whose merge of one split gives the same bits:
// weight exp2(0) = 1).
constexpr int kSplitPages = 4;
__host__ __device__ constexpr int splits_for_pages(int64_t pages, int64_t splits) {
  const int64_t s = (pages + kSplitPages - 1) / kSplitPages;
  return static_cast<int>(pages < 1 ? 1 : s < splits ? s : splits);
}
__device__ __forceinline__ int tile_splits(const Tile &t, int splits) {
  if (t.hi_max < 0) return 1;
  return splits_for_pages(t.hi_max / kPage - t.lo_min / kPage + 1, splits);
}

// The empty (m, l) of split `split` for the tile's columns (separate
// combine; plain stores, read after the launch).
__device__ __forceinline__ void mark_empty_split(const DecodeArgs &a, int t0, int kh, int hb, int nrows, int ncols,
                                                 int cap, int split) {
  for (int c = threadIdx.x; c < ncols; c += blockDim.x) {
    const Column rc = tile_column(c, a.group, nrows, hb, cap);
    const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
    float *ml = a.part_ml + 2 * (th * a.splits + split);
    ml[0] = -INFINITY;
    ml[1] = 0.f;
  }
}

// ---- fused merge: the last workgroup of a merge unit merges every split ----
// Called by all threads once this workgroup's partial stores are issued; st
// is the tile's split count.  The unit's counter is a ticket: the workgroup
// that draws st - 1 merges the st partials and resets the counter to zero.  Columns are taken CG at a time (CG * S <= NT):
// one round of loads fetches every (m, l) of the group, a second every partial
// element; each thread keeps the eight group sums of its elements, which is
// the combine kernel's arithmetic element for element.
template <int HD, int NT>
__device__ void fused_merge(const DecodeArgs &a, int t0, int kh, int hb, int nrows, int ncols, int cap, int st,
                            FusedScratch<NT> *fsp, int *s_is_last) {
  wait_all_memory();  // this workgroup's partial stores have completed
  __syncthreads();
  const int unit = (t0 * a.nkv + kh) * a.hblocks + hb;
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(&a.counters[unit], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_is_last = prev == st - 1;
  }
  __syncthreads();
  if (!*s_is_last) return;
  FusedScratch<NT> &fs = *fsp;
  const LoadCoherent ld;
  const int S = st;           // partials merged
  const int SS = a.splits;    // slots per (row, head)
  const int tid = threadIdx.x;
  const int cg_max = max(1, min(ncols, NT / S));
  for (int c0 = 0; c0 < ncols; c0 += cg_max) {
    const int cg = min(cg_max, ncols - c0);
    // (m, l) of every (column, split) of the group
    for (int idx = tid; idx < cg * S; idx += NT) {
      const int c = idx / S, sp = idx - c * S;
      const Column rc = tile_column(c0 + c, a.group, nrows, hb, cap);
      const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
      const float m = ld(a.part_ml + (th * SS + sp) * 2);
      const float l = ld(a.part_ml + (th * SS + sp) * 2 + 1);
      fs.l[idx] = l;
      fs.w[idx] = l > 0.f ? m : -INFINITY;
    }
    __syncthreads();
    if (tid < cg) {
      float mx = -INFINITY;
      for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, fs.w[tid * S + sp]);
      fs.mx[tid] = mx;
    }
    __syncthreads();
    for (int idx = tid; idx < cg * S; idx += NT) {
      const int c = idx / S;
      fs.w[idx] = fs.l[idx] > 0.f ? fast_exp2(fs.w[idx] - fs.mx[c]) : 0.f;
    }
    __syncthreads();
    if (tid < cg) {
      float dg[kMergeGroups];
#pragma unroll
      for (int g = 0; g < kMergeGroups; ++g) dg[g] = 0.f;
      for (int s0 = 0; s0 < S; s0 += kMergeGroups)
#pragma unroll
        for (int g = 0; g < kMergeGroups; ++g) {
          const int sp = s0 + g;
          if (sp < S) {
            const float ws = fs.w[tid * S + sp];
            dg[g] = ws != 0.f ? __builtin_fmaf(ws, fs.l[tid * S + sp], dg[g]) : dg[g];
          }
        }
      float den = 0.f;
#pragma unroll
      for (int g = 0; g < kMergeGroups; ++g) den += dg[g];
      fs.den[tid] = den;
    }
    __syncthreads();
    // every partial element of the group
    for (int idx = tid; idx < cg * HD; idx += NT) {
      const int c = idx / HD, d = idx - c * HD;
      const Column rc = tile_column(c0 + c, a.group, nrows, hb, cap);
      const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
      const float *o = a.part_o + th * SS * HD + d;
      const float *w = fs.w + c * S;
      float num[kMergeGroups];
#pragma unroll
      for (int g = 0; g < kMergeGroups; ++g) num[g] = 0.f;
      for (int s0 = 0; s0 < S; s0 += kMergeGroups) {
        float v[kMergeGroups];
#pragma unroll
        for (int g = 0; g < kMergeGroups; ++g) v[g] = ld(o + static_cast<int64_t>(min(s0 + g, S - 1)) * HD);
#pragma unroll
        for (int g = 0; g < kMergeGroups; ++g) {
          const int sp = s0 + g;
          if (sp < S) {
            const float ws = w[sp];
            num[g] = ws != 0.f ? __builtin_fmaf(ws, v[g], num[g]) : num[g];
          }
        }
      }
      float n = 0.f;
#pragma unroll
      for (int g = 0; g < kMergeGroups; ++g) n += num[g];
      const float den = fs.den[c];
      a.out[th * HD + d] = f32_to_bf16_rne(den > 0.f ? n / den : 0.f);
    }
    __syncthreads();
  }
  if (tid == 0) __hip_atomic_store(&a.counters[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The running max of a column only moves when a page's max exceeds it by more
// than this (log2 units), so the output accumulators are rescaled rarely;
// softmax weights then stay below 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.f;

// The parallel fused merge (defined with the combine kernel below).
template <int HD, int NT, bool WIDE = true>
__device__ void owned_merge(const DecodeArgs &a, int t0, int kh, int hb, int nrows, int ncols, int cap, int split,
                            int st, int *s_word);

// Tiles of at most this many columns may take the vector-ALU page step.
constexpr int kNarrowCols = 4;

// OWNED: the parallel fused merge is compiled in (hd 256; at hd 128 a form of
// its own, launched only for merges that use it, since it costs the kernel a
// wave per SIMD: 192 against 152 VGPRs).
// VALU = false: scores and P.V on MFMA, 16-column tiles.
// VALU = true (hd 64 to 256, tiles of at most kNarrowCols columns): the page
// step runs on the vector ALU with packed bf16 dot products
// (v_dot2_f32_bf16), cross-lane sums through DPP, and no LDS staging of V;
// the wave's state is moved into the MFMA form's output layout at the end,
// so the merges and the epilogue are shared.
template <int HD, bool VALU = false, bool OWNED = (HD >= 256)>
__global__ __launch_bounds__(kThreads) void pgqa_wave_kernel(DecodeArgs a) {
  constexpr int KJ = HD / 32;   // QK^T MFMA steps (32 hd elements each)
  constexpr int DJ = HD / 16;   // PV MFMA output blocks (16 hd columns each)
  constexpr int VLD = HD / 32;  // 16-byte V loads per lane per page
  constexpr int VSTR = HD + 8;  // LDS row stride of a staged V page (elements)
  // Per-wave V staging; reused at the end for the cross-wave merge.
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kWaves][kPage * VSTR];
  __shared__ float xfer[kWaves][16];
  __shared__ int s_is_last;
  static_assert(2 * (16 * HD + 32) * 4 <= kWaves * kPage * VSTR * 2, "merge slots must fit the V staging area");
  static_assert(sizeof(FusedScratch<kThreads>) <= sizeof(vtile), "merge scratch must fit the V staging area");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15;  // MFMA row/column index of this lane
  const int lc = lane >> 4;  // MFMA k-group of this lane

  int b = blockIdx.x;
  const int split = b % a.splits;
  b /= a.splits;
  const int hb = b % a.hblocks;
  b /= a.hblocks;
  const int kh = b % a.nkv;
  // ---- the tile: row metadata through the scalar cache in large ranked
  // launches of up to 64 rows, else vector loads; Q is requested afterwards,
  // with the first page-table window, so the two share one memory round
  // trip ----
  int sub_rows = 0;
  const int pos = b / a.nkv;
  const bool lane_rows = !a.tile_row0 && a.rank_rows && a.rows <= 64;
  LaneRows lr{INT_MIN, 0, -1};
  if (lane_rows) lr = rows_by_lane(a, lane);
  const int t0 = a.tile_row0   ? prefill_subtile(a, pos, sub_rows)
                 : lane_rows ? rank_of_lanes(a, lr, pos, lane)
                             : row_of_rank(a, pos, lane);
  if (a.tile_row0 && sub_rows == 0) return;
  const Tile tile = lane_rows ? tile_of_lanes(a, lr, t0, lane) : tile_rows(a, t0, lane, sub_rows);
  if (!tile.lead) return;
  const int origin = tile.origin;
  const int nrows = tile.nrows;
  const int lo_l = tile.lo_l, hi_l = tile.hi_l;
  const int ncols = a.group <= 16 ? nrows * a.group : min(16, a.group - hb * 16);
  const int st = tile_splits(tile, a.splits);
  if (split >= st) {
    if (a.counters == nullptr) mark_empty_split(a, t0, kh, hb, nrows, ncols, 16, split);
    return;
  }
  int pbeg, pend;
  split_range(tile, split, st, pbeg, pend);

  // ---- this lane's score column and its Q (zero for a column without a row) ----
  const Column col = tile_column(ln, a.group, nrows, hb, 16);
  const int col_lo = __shfl(lo_l, col.row);
  // shuffle with every lane active, then drop columns without a row
  const int col_hi_any = __shfl(hi_l, col.row);
  const int col_hi = col.on ? col_hi_any : -1;
  bf16x8 qop[KJ];
  {
    const uint16_t *qrow = a.q + (static_cast<int64_t>(t0 + (col.on ? col.row : 0)) * a.nh + kh * a.group +
                                  (col.on ? col.head : 0)) * HD;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      if (col.on) {
        qop[j] = *reinterpret_cast<const bf16x8 *>(qrow + (4 * j + lc) * 8);
      } else {
        u32x4 z = {0u, 0u, 0u, 0u};
        qop[j] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  // ---- vector-ALU form: K and V both arrive as 16-byte chunks, lane l of
  // load j holding chunk cl = l % CH of token TPL*j + tg (tg = l / CH).  A
  // lane computes the partial dot products of its chunk for all NLD tokens
  // and kNarrowCols columns; a transposing sum over the CH lanes of a token
  // row leaves lane l with the full score of column vc = cl % 4 and token
  // vtok.  The weights go through LDS (64 floats); each lane then accumulates
  // P.V for its own chunk over its NLD tokens, and the tg lanes of a chunk
  // are summed once, after the last page. ----
  constexpr int CH = HD / 8;        // 16-byte chunks per token row
  constexpr int TPL = 64 / CH;      // tokens per 64-lane load
  constexpr int NLD = kPage / TPL;  // loads per page, of K and of V
  static_assert(!VALU || ((HD == 64 || HD == 128 || HD == 256) && NLD * kNarrowCols == CH && NLD == VLD),
                "the vector-ALU form is built for hd 64 to 256");
  const int cl = lane % CH, tg = lane / CH;
  const int vc = cl % kNarrowCols;                 // score column of this lane
  const int vtok = TPL * (cl / kNarrowCols) + tg;  // and its token in the page
  const Column vcol = tile_column(vc, a.group, nrows, hb, 16);
  const int vcol_lo = __shfl(lo_l, vcol.row);
  const int vcol_hi_any = __shfl(hi_l, vcol.row);
  const int vcol_hi = vcol.on ? vcol_hi_any : -1;
  u32x4 qv[kNarrowCols];               // Q chunk cl of every column
  float vacc[kNarrowCols][8];          // o[column][8 cl + e] over this lane's tokens
  float vl = 0.f, vm = -INFINITY;      // weight sum of this lane's (token, column); reference max of column vc
  if constexpr (VALU) {
#pragma unroll
    for (int c = 0; c < kNarrowCols; ++c) {
      const Column cc = tile_column(c, a.group, nrows, hb, 16);
      qv[c] = u32x4{0u, 0u, 0u, 0u};
      if (cc.on)
        qv[c] = *reinterpret_cast<const u32x4 *>(
            a.q + (static_cast<int64_t>(t0 + cc.row) * a.nh + kh * a.group + cc.head) * HD + cl * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) vacc[c][e] = 0.f;
    }
  }

  float m_run = -INFINITY;  // reference max (log2 units) of column ln
  f32x4 oacc[DJ];           // rows 4*lc+i of the column block, hd column 16*jj+ln
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < DJ; ++jj) oacc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  const s16x4 ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80};
  const int64_t kv_head_off = static_cast<int64_t>(kh) * kPage * HD;
  const int64_t page_elems = static_cast<int64_t>(a.nkv) * kPage * HD;
  uint16_t *vt = vtile[wave];
  // V operand of step jj via the LDS transpose read: lane (4m+q) of k-group lc
  // points at token row 4*lc+m, hd column 16*jj + 4q, and receives
  // V[4*lc .. 4*lc+3][16*jj + ln] (the 16 lanes' 4-element rows are
  // redistributed column-wise).
  const uint16_t *vtr = vt + (4 * lc + (ln >> 2)) * VSTR + 4 * (ln & 3);

  // This wave's pages: pbeg + wave + kWaves * k, k = 0 .. nk-1.  They are
  // walked in windows of 128; the physical pages of a window are fetched (lane
  // l of pv0 / pv1: page w0 + l / w0 + 64 + l) and waited for before the
  // window's pipelined loop, so page loads never wait on the table.
  const int first = pbeg + wave;
  const int nk = first < pend ? (pend - first + kWaves - 1) / kWaves : 0;
  int pv0 = 0, pv1 = 0;
  auto fetch_window = [&](int w0) {
    int ph[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = w0 + 64 * h + lane;
      ph[h] = 0;
      if (k < nk) {
        ph[h] = a.block_table[origin + first + kWaves * k];
        if (a.page_map) ph[h] = a.page_map[ph[h]];
      }
    }
    pv0 = ph[0];
    pv1 = ph[1];
    wait_all_memory();
  };
  auto load_page = [&](int kw, bf16x8(&kop)[KJ], u32x4(&vreg)[VLD]) {
    const int phys = kw < 64 ? __builtin_amdgcn_readlane(pv0, kw) : __builtin_amdgcn_readlane(pv1, kw - 64);
    const int64_t page_off = static_cast<int64_t>(phys) * page_elems + kv_head_off;
    const uint16_t *kp = a.k_pool + page_off;
    const uint16_t *vp = a.v_pool + page_off;
    if constexpr (VALU) {
#pragma unroll
      for (int j = 0; j < KJ; ++j)
        kop[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(kp + (j * 64 + lane) * 8));
    } else {
#pragma unroll
      for (int j = 0; j < KJ; ++j)
        kop[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(kp + ln * HD + (4 * j + lc) * 8));
    }
#pragma unroll
    for (int j = 0; j < VLD; ++j)
      vreg[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + (j * 64 + lane) * 8));
  };
  // The vector-ALU page step (same masking, lazy rescale and bf16 weights as
  // the MFMA step below).
  auto compute_page_valu = [&](int k, const bf16x8(&kop)[KJ], const u32x4(&vreg)[VLD]) {
    const int p = first + kWaves * k;
    const bool full = p >= tile.fp0 && p < tile.fp1;
    float part[NLD * kNarrowCols];  // index j * 4 + column
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const u32x4 kw = __builtin_bit_cast(u32x4, kop[j]);
#pragma unroll
      for (int c = 0; c < kNarrowCols; ++c) {
        float sdot = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          sdot = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw[d]), as_bf16x2(qv[c][d]), sdot, false);
        part[j * kNarrowCols + c] = sdot;
      }
    }
    // sum over the CH lanes of a token row: lane bit 4 (hd 256), 3 (hd 128 and
    // 256), 2, 1, 0
    if constexpr (CH == 32) fold_half_xor<16, 32>(part, (lane & 16) != 0);
    if constexpr (CH >= 16) fold_half<kDppRor8, 16>(part, (lane & 8) != 0);
    fold_half<kDppHalfMirror, 8>(part, (lane & 4) != 0);
    fold_half<kDppXor2, 4>(part, (lane & 2) != 0);
    fold_half<kDppXor1, 2>(part, (lane & 1) != 0);
    bool vis = true;
    uint64_t bal = ~0ull;
    if (!full) {
      const int pos = p * kPage + vtok;
      vis = vcol.on && pos >= vcol_lo && pos <= vcol_hi;
      bal = __ballot(vis);
      if (bal == 0) return;
    }
    const float sv = vis ? part[0] : -INFINITY;
    if (__ballot(sv * kLog2e > vm + kRescaleSlack) != 0) {
      // the column's max over its 16 lanes (lane bits 2-5)
      float mx = sv;
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m2 = mx * kLog2e;
      const bool grow = m2 > vm + kRescaleSlack;
      const float m_new = grow ? m2 : vm;
      const float alpha = grow ? fast_exp2(vm - m_new) : 1.f;
      vm = m_new;
      vl *= alpha;
#pragma unroll
      for (int c = 0; c < kNarrowCols; ++c) {
        const float ac = __shfl(alpha, c);  // lane c holds column c
#pragma unroll
        for (int e = 0; e < 8; ++e) vacc[c][e] *= ac;
      }
    }
    float pw = fast_exp2(__builtin_fmaf(sv, kLog2e, -vm));
    if (!full) pw = sv == -INFINITY ? 0.f : pw;
    {
      // the sum takes the bf16-rounded weight, as P.V does
      const bf16x2 pb = __builtin_convertvector(f32x2{pw, 0.f}, bf16x2);
      vl += __uint_as_float(__builtin_bit_cast(unsigned, pb) << 16);
    }
    float *pbuf = reinterpret_cast<float *>(vt);
    pbuf[lane] = pw;
    wave_lds_sync();
    // weights of this lane's tokens: (token TPL*j + tg, column c) sits in lane
    // tg*CH + 4j + c
    f32x4 pj[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) pj[j] = reinterpret_cast<const f32x4 *>(pbuf + tg * CH)[j];
#pragma unroll
    for (int j2 = 0; j2 < NLD / 2; ++j2) {
      const int j0 = 2 * j2, j1 = 2 * j2 + 1;
      u32x4 v0 = vreg[j0], v1 = vreg[j1];
      if (!full) {
        // tokens no column sees may hold NaN
        if (((bal >> (tg * CH + kNarrowCols * j0)) & 0xfull) == 0) v0 = u32x4{0u, 0u, 0u, 0u};
        if (((bal >> (tg * CH + kNarrowCols * j1)) & 0xfull) == 0) v1 = u32x4{0u, 0u, 0u, 0u};
      }
      // element e of both tokens in one word: (v0[e], v1[e])
      unsigned vpair[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        vpair[2 * d] = __builtin_amdgcn_perm(v1[d], v0[d], 0x05040100u);
        vpair[2 * d + 1] = __builtin_amdgcn_perm(v1[d], v0[d], 0x07060302u);
      }
#pragma unroll
      for (int c = 0; c < kNarrowCols; ++c) {
        const bf16x2 pp = __builtin_convertvector(f32x2{pj[j0][c], pj[j1][c]}, bf16x2);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vacc[c][e] = __builtin_amdgcn_fdot2_f32_bf16(pp, as_bf16x2(vpair[e]), vacc[c][e], false);
      }
    }
    wave_lds_sync();
  };
  auto compute_page = [&](int k, const bf16x8(&kop)[KJ], const u32x4(&vreg)[VLD]) {
    const int p = first + kWaves * k;
    // Pages every row sees in full need no per-token masks (columns without a
    // row hold Q = 0 and are never written out).
    const bool full = p >= tile.fp0 && p < tile.fp1;
    const int pos0 = p * kPage + 4 * lc;
    bool vis[4] = {true, true, true, true};
    uint32_t tokmask = 0xffffu;
    if (!full) {
      tokmask = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vis[i] = col.on && pos0 + i >= col_lo && pos0 + i <= col_hi;
        const uint64_t bal = __ballot(vis[i]);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if ((bal >> (16 * g)) & 0xffffull) tokmask |= 1u << (4 * g + i);
      }
      if (tokmask == 0) return;
    }

    // S^T: lane holds scores of tokens 4*lc+i for column ln.
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j], qop[j], sc, 0, 0, 0);

    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = vis[i] ? sc[i] : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m2 = mx * kLog2e;
    // Move the reference max only when this page exceeds it by the slack.
    const bool grow = m2 > m_run + kRescaleSlack;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? m2 : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      // factors move from the column layout (lane ln) to the output layout
      // (lane holds rows 4*lc .. 4*lc+3)
      if (lc == 0) xfer[wave][ln] = alpha;
      wave_lds_sync();
      const f32x4 al = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);
#pragma unroll
      for (int jj = 0; jj < DJ; ++jj) oacc[jj] *= al;
      lacc *= al;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(__builtin_fmaf(sv[i], kLog2e, -m_run));
      if (!full) pr[i] = sv[i] == -INFINITY ? 0.f : pr[i];
    }
    const s16x4 pa = pack_weights(pr[0], pr[1], pr[2], pr[3]);

    // Stage V; tokens no column can see are zeroed (they may hold NaN).
#pragma unroll
    for (int j = 0; j < VLD; ++j) {
      const int e = (j * 64 + lane) * 8;
      const int tok = e / HD;
      u32x4 v = vreg[j];
      if (!full && !((tokmask >> tok) & 1u)) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(vt + tok * VSTR + (e - tok * HD)) = v;
    }
    wave_lds_sync();
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj) {
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)(vtr + 16 * jj));
      oacc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, oacc[jj], 0, 0, 0);
    }
    lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ones, lacc, 0, 0, 0);
    wave_lds_sync();
  };

  // Two register sets (hd <= 128, and the vector-ALU form up to hd 256): the
  // next page's K and V are in flight while the current page is computed;
  // past the window's end its last page is loaded again (already cached) so
  // every step issues the same loads.  The MFMA form at hd 256 holds one page
  // (214 VGPRs, two waves per SIMD, against 280 and one wave with two sets:
  // 4-17% faster on batched and multi-row decode, the same bits); the other
  // wave of the SIMD covers the load latency.
  for (int w0 = 0; w0 < nk; w0 += 128) {
    const int wn = min(128, nk - w0);
    fetch_window(w0);
    bf16x8 kA[KJ];
    u32x4 vA[VLD];
    load_page(0, kA, vA);
    if constexpr (HD <= 128 || VALU) {
      bf16x8 kB[KJ];
      u32x4 vB[VLD];
      for (int k = 0; k < wn; k += 2) {
        load_page(min(k + 1, wn - 1), kB, vB);
        if constexpr (VALU)
          compute_page_valu(w0 + k, kA, vA);
        else
          compute_page(w0 + k, kA, vA);
        load_page(min(k + 2, wn - 1), kA, vA);
        if (k + 1 < wn) {
          if constexpr (VALU)
            compute_page_valu(w0 + k + 1, kB, vB);
          else
            compute_page(w0 + k + 1, kB, vB);
        }
      }
    } else {
      for (int k = 0; k < wn; ++k) {
        if (k > 0) load_page(k, kA, vA);
        compute_page(w0 + k, kA, vA);
      }
    }
    wait_all_memory();
  }

  if constexpr (VALU) {
    // P.V partials: transposing sum over the lanes of one chunk (lane bit 5;
    // 4 from hd 128 down; 3 at hd 64) leaves each lane NKEEP outputs
    float fv[kNarrowCols * 8];
#pragma unroll
    for (int c = 0; c < kNarrowCols; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) fv[c * 8 + e] = vacc[c][e];
    fold_half_xor<32, 32>(fv, (lane & 32) != 0);
    if constexpr (CH <= 16) fold_half_xor<16, 16>(fv, (lane & 16) != 0);
    if constexpr (CH == 8) fold_half<kDppRor8, 8>(fv, (lane & 8) != 0);
    // the lane keeps values v = vbase + i (v = 8 column + element)
    constexpr int NKEEP = CH / 2;
    const int vbase = ((lane >> 5) & 1) * 16 + (CH <= 16 ? ((lane >> 4) & 1) * 8 : 0) +
                      (CH == 8 ? ((lane >> 3) & 1) * 4 : 0);
    // weight sums over each column's 16 lanes
    vl += __shfl_xor(vl, 4);
    vl += __shfl_xor(vl, 8);
    vl += __shfl_xor(vl, 16);
    vl += __shfl_xor(vl, 32);
    // into the MFMA output layout through the wave's LDS area:
    // o[column][hd], then the columns' sums and reference maxes
    float *ob = reinterpret_cast<float *>(vt);
    static_assert((kNarrowCols * HD + 2 * kNarrowCols) * 4 <= kPage * VSTR * 2, "state must fit the V staging area");
#pragma unroll
    for (int i = 0; i < NKEEP; ++i) ob[((vbase + i) >> 3) * HD + cl * 8 + ((vbase + i) & 7)] = fv[i];
    if (lane < kNarrowCols) {
      ob[kNarrowCols * HD + lane] = vl;
      ob[kNarrowCols * HD + kNarrowCols + lane] = vm;
    }
    wave_lds_sync();
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[jj][i] = lc == 0 ? ob[i * HD + 16 * jj + ln] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lacc[i] = lc == 0 ? ob[kNarrowCols * HD + i] : 0.f;
    m_run = ln < kNarrowCols ? ob[kNarrowCols * HD + kNarrowCols + ln] : -INFINITY;
    wave_lds_sync();
  }
  // ---- reference max into the output layout ----
  if (lc == 0) xfer[wave][ln] = m_run;
  wave_lds_sync();
  f32x4 mo = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);

  // ---- merge the 4 wave states through LDS: (0 <- 2, 1 <- 3), then 0 <- 1 ----
  float *slot_base = reinterpret_cast<float *>(&vtile[0][0]);
  constexpr int kSlot = 16 * HD + 32;  // floats: o[16][HD], m[16], l[16]
  auto put_state = [&](int slot) {
    float *sp = slot_base + slot * kSlot;
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[(4 * lc + i) * HD + 16 * jj + ln] = oacc[jj][i];
    if (ln == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sp[16 * HD + 4 * lc + i] = mo[i];
        sp[16 * HD + 16 + 4 * lc + i] = lacc[i];
      }
    }
  };
  auto take_state = [&](int slot) {
    const float *sp = slot_base + slot * kSlot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mb = sp[16 * HD + 4 * lc + i];
      const float lb = sp[16 * HD + 16 + 4 * lc + i];
      const float ma = mo[i];
      const float mn = fmaxf(ma, mb);
      const float wa = ma == -INFINITY ? 0.f : fast_exp2(ma - mn);
      const float wb = mb == -INFINITY ? 0.f : fast_exp2(mb - mn);
#pragma unroll
      for (int jj = 0; jj < DJ; ++jj)
        oacc[jj][i] = oacc[jj][i] * wa + sp[(4 * lc + i) * HD + 16 * jj + ln] * wb;
      lacc[i] = lacc[i] * wa + lb * wb;
      mo[i] = mn;
    }
  };
  __syncthreads();
  if (wave >= 2) put_state(wave - 2);
  __syncthreads();
  if (wave < 2) take_state(wave);
  __syncthreads();
  if (wave == 1) put_state(0);
  __syncthreads();
  if (wave == 0) take_state(0);

  const bool fused = st > 1 && a.counters != nullptr;
  const bool direct = st == 1 && (a.splits == 1 || a.counters != nullptr);
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lc + i;
      if (r >= ncols) continue;
      const Column rc = tile_column(r, a.group, nrows, hb, 16);
      const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
      if (direct) {
        const float l = lacc[i];
#pragma unroll
        for (int jj = 0; jj < DJ; ++jj) {
          const float v = l > 0.f ? oacc[jj][i] / l : 0.f;
          a.out[th * HD + 16 * jj + ln] = f32_to_bf16_rne(v);
        }
      } else {
        const int64_t ps = th * a.splits + split;
        float *po = a.part_o + ps * HD;
#pragma unroll
        for (int jj = 0; jj < DJ; ++jj) store_coherent(po + 16 * jj + ln, oacc[jj][i]);
        if (ln == 0) {
          store_coherent(a.part_ml + 2 * ps, mo[i]);
          store_coherent(a.part_ml + 2 * ps + 1, lacc[i]);
        }
      }
    }
  }
  if (!fused) return;

  // Large merges (OWNED forms only; the host sets spin_ticks for those): all
  // of the unit's workgroups together.  Otherwise the last one alone.
  if constexpr (OWNED) {
    if (a.spin_ticks > 0) {
      __syncthreads();  // the V staging area is free for the merge scratch
      owned_merge<HD, kThreads>(a, t0, kh, hb, nrows, ncols, 16, split, st, &s_is_last);
      return;
    }
  }
  fused_merge<HD, kThreads>(a, t0, kh, hb, nrows, ncols, 16, st,
                            reinterpret_cast<FusedScratch<kThreads> *>(&vtile[0][0]), &s_is_last);
}

// ---------------------------------------------------------------------------
// hd-sliced kernel: tiles of up to 16 columns at large hd (one-row and
// few-row decode of wide heads).  The 4 waves of a workgroup split hd into 4
// slices and all walk every page of the split: wave w loads, for each page,
// only its slice of K and V (HD / 4 elements of each of the 16 tokens), so a
// page costs a wave HD / 8 registers of K and as many of V, and RING pages are
// in flight per wave at once -- loads of page k + RING are issued as soon as
// page k's registers are consumed (K after the scores, V after its staging).
// Each wave's partial scores (its slice of q . k) go through LDS; every wave
// adds the 4 slices in the same order, so all 4 hold the same scores and the
// same softmax state, and each accumulates P V for its own hd slice.  At the
// end no cross-wave merge is needed: wave w owns output elements
// [w HD / 4, (w + 1) HD / 4) of every column.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(kThreads) void pgqa_slice_kernel(DecodeArgs a) {
  constexpr int HS = HD / kWaves;  // hd slice of one wave
  constexpr int KS = HS / 32;      // QK^T MFMA steps over the slice
  constexpr int DS = HS / 16;      // PV output blocks of the slice
  constexpr int VL = HS / 32;      // 16-byte V loads per lane per page
  constexpr int RING = 3;          // pages in flight per wave (RING + 1 register sets)
  constexpr int VSTR = HS + 8;     // LDS row stride of a staged V slice (elements)
  // The reference max follows every new column max (no slack): the largest
  // weight of the row is then exactly 1 before bf16 rounding, which keeps the
  // rounding of the weights out of the dominant term (measured: worst
  // per-head error against the f64 oracle 1.45e-3 instead of 2.2e-3 on a
  // 32K-key global layer, at the same speed).
  constexpr float SLACK = 0.f;
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kWaves][kPage * VSTR];
  // partial scores of every wave, two buffers used in turn: a wave can only
  // write one again after passing the next exchange's barrier, which every
  // wave reaches after reading it
  __shared__ __attribute__((aligned(16))) f32x4 xs[2][kWaves][64];
  __shared__ float xfer[kWaves][16];
  __shared__ int s_is_last;
  static_assert(KS >= 1 && DS >= 1, "the hd-sliced kernel needs hd >= 128");
  static_assert(sizeof(FusedScratch<kThreads>) <= sizeof(vtile), "merge scratch must fit the V staging area");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15;
  const int lc = lane >> 4;
  const int h0 = wave * HS;  // first hd element of this wave's slice

  int b = blockIdx.x;
  const int split = b % a.splits;
  b /= a.splits;
  const int hb = b % a.hblocks;
  b /= a.hblocks;
  const int kh = b % a.nkv;
  // ---- the tile (row metadata through the scalar cache in large ranked
  // launches of up to 64 rows); Q follows, requested with the first
  // page-table window ----
  const int pos = b / a.nkv;
  const bool lane_rows = a.rank_rows && a.rows <= 64;
  LaneRows lr{INT_MIN, 0, -1};
  if (lane_rows) lr = rows_by_lane(a, lane);
  const int t0 = lane_rows ? rank_of_lanes(a, lr, pos, lane) : row_of_rank(a, pos, lane);
  const Tile tile = lane_rows ? tile_of_lanes(a, lr, t0, lane) : tile_rows(a, t0, lane);
  if (!tile.lead) return;
  const int origin = tile.origin;
  const int nrows = tile.nrows;
  const int ncols = a.group <= 16 ? nrows * a.group : min(16, a.group - hb * 16);
  const int st = tile_splits(tile, a.splits);
  if (split >= st) {
    if (a.counters == nullptr) mark_empty_split(a, t0, kh, hb, nrows, ncols, 16, split);
    return;
  }
  int pbeg, pend;
  split_range(tile, split, st, pbeg, pend);

  const Column col = tile_column(ln, a.group, nrows, hb, 16);
  const int col_lo = __shfl(tile.lo_l, col.row);
  const int col_hi_any = __shfl(tile.hi_l, col.row);
  const int col_hi = col.on ? col_hi_any : -1;
  // Q of this wave's slice (zero for a column without a row)
  bf16x8 qop[KS];
  {
    const uint16_t *qrow = a.q + (static_cast<int64_t>(t0 + (col.on ? col.row : 0)) * a.nh + kh * a.group +
                                  (col.on ? col.head : 0)) * HD + h0;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (col.on) {
        qop[j] = *reinterpret_cast<const bf16x8 *>(qrow + (4 * j + lc) * 8);
      } else {
        u32x4 z = {0u, 0u, 0u, 0u};
        qop[j] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  float m_run = -INFINITY;
  f32x4 oacc[DS];
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < DS; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const s16x4 ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80};
  const int64_t kv_head_off = static_cast<int64_t>(kh) * kPage * HD + h0;
  const int64_t page_elems = static_cast<int64_t>(a.nkv) * kPage * HD;
  uint16_t *vt = vtile[wave];
  const uint16_t *vtr = vt + (4 * lc + (ln >> 2)) * VSTR + 4 * (ln & 3);

  // Physical pages of the split, 128 per window in two VGPRs per lane.  Page
  // ids are looked up only for the page being requested, which runs RING
  // pages ahead.  When it leaves the window, the next window is fetched and
  // waited for (every load in flight drains once per 128 pages): the window
  // registers are then never waited on inside the page loop.
  const int nk = pend - pbeg;
  int cur0 = 0, cur1 = 0, cur_w = 0;
  int xpar = 0;  // score-exchange buffer in use (flips on every exchange; uniform)
  auto fetch_window = [&](int w0) {
    int ph[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = w0 + 64 * h + lane;
      ph[h] = 0;
      if (k < nk) {
        ph[h] = a.block_table[origin + pbeg + k];
        if (a.page_map) ph[h] = a.page_map[ph[h]];
      }
    }
    cur0 = ph[0];
    cur1 = ph[1];
    cur_w = w0;
    wait_all_memory();
  };
  auto phys_of = [&](int k) -> int {
    const int off = k - cur_w;  // 0 .. 127
    return __builtin_amdgcn_readlane(off < 64 ? cur0 : cur1, off & 63);
  };
  // The loads of page k into a register set.  With real false (a refill past
  // the last page) load j of every lane reads the 16 bytes at j * 16 of the
  // window's first page instead (a page of the split): the same number of
  // load instructions, distinct (so none is merged into another) but all
  // within one cache line, and the data is never used.
  auto load_k = [&](int k, bool real, bf16x8(&kr)[KS]) {
    const uint16_t *kp = a.k_pool + static_cast<int64_t>(phys_of(real ? k : cur_w)) * page_elems + kv_head_off;
#pragma unroll
    for (int j = 0; j < KS; ++j)
      kr[j] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8 *>(kp + (real ? ln * HD + (4 * j + lc) * 8 : 8 * j)));
  };
  auto load_v = [&](int k, bool real, u32x4(&vr)[VL]) {
    const uint16_t *vp = a.v_pool + static_cast<int64_t>(phys_of(real ? k : cur_w)) * page_elems + kv_head_off;
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int e = (j * 64 + lane) * 8;  // element of the [16][HS] slice
      const int tok = e / HS;
      vr[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(vp + (real ? tok * HD + (e - tok * HS) : 8 * (KS + j))));
    }
  };

  // Step k: first the register set that page k - 1 used (consumed in the
  // previous step) is refilled with page k + RING, then page k is computed
  // from its own set (kr, vr).  Every step -- also the steps past the last
  // page, which only refill -- issues the same loads in the same order, and a
  // refill never shares a basic block with the last use of its registers, so
  // the compiler's counted waits leave RING pages in flight.  All 4 waves take
  // every page, so the per-page decisions (visibility, skip) are the same in
  // all of them.
  auto page = [&](int k, bf16x8(&kr)[KS], u32x4(&vr)[VL], bf16x8(&kf)[KS], u32x4(&vf)[VL]) {
    const int p = pbeg + k;
    const int kn = k + RING;  // >= 0
    const bool real = kn < nk;
    if (real && kn - cur_w >= 128) fetch_window(cur_w + 128);  // the page to request leaves the window
    load_k(kn, real, kf);
    load_v(kn, real, vf);
    if (k < 0) return;  // the first RING steps only request pages
    const bool full = p >= tile.fp0 && p < tile.fp1;
    const int pos0 = p * kPage + 4 * lc;
    bool vis[4] = {true, true, true, true};
    uint32_t tokmask = 0xffffu;
    if (!full) {
      tokmask = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vis[i] = col.on && pos0 + i >= col_lo && pos0 + i <= col_hi;
        const uint64_t bal = __ballot(vis[i]);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if ((bal >> (16 * g)) & 0xffffull) tokmask |= 1u << (4 * g + i);
      }
    }
    if (k >= nk) tokmask = 0;  // past the last page
    if (tokmask == 0) return;  // no column sees this page (or no page)
    // partial scores over this wave's slice
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[j], qop[j], sc, 0, 0, 0);
    // stage this wave's V slice (tokens no column sees are zeroed: they may
    // hold NaN)
#pragma unroll
    for (int j = 0; j < VL; ++j) {
      const int e = (j * 64 + lane) * 8;
      const int tok = e / HS;
      u32x4 v = vr[j];
      if (!full && !((tokmask >> tok) & 1u)) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(vt + tok * VSTR + (e - tok * HS)) = v;
    }
    // whole scores: the 4 slices added in wave order, the same in every wave
    f32x4 *xp = xs[xpar][0];
    xpar ^= 1;
    xp[wave * 64 + lane] = sc;
    lds_barrier();
    sc = xp[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sc += xp[w * 64 + lane];

    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = vis[i] ? sc[i] : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m2 = mx * kLog2e;
    const bool grow = m2 > m_run + SLACK;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? m2 : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      if (lc == 0) xfer[wave][ln] = alpha;
      wave_lds_sync();
      const f32x4 al = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);
#pragma unroll
      for (int u = 0; u < DS; ++u) oacc[u] *= al;
      lacc *= al;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(__builtin_fmaf(sv[i], kLog2e, -m_run));
      if (!full) pr[i] = sv[i] == -INFINITY ? 0.f : pr[i];
    }
    const s16x4 pa = pack_weights(pr[0], pr[1], pr[2], pr[3]);
    wave_lds_sync();  // the staged V slice is visible to the whole wave
#pragma unroll
    for (int u = 0; u < DS; ++u) {
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)(vtr + 16 * u));
      oacc[u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, oacc[u], 0, 0, 0);
    }
    lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ones, lacc, 0, 0, 0);
    wave_lds_sync();  // the V slice's reads are done before the next page stages its own
  };

  if (nk > 0) {
    fetch_window(0);
    bf16x8 kset[RING + 1][KS];
    u32x4 vset[RING + 1][VL];
    // The loop starts RING steps early: those steps only request pages 0 ..
    // RING - 1, through the same code as every later refill (a separate
    // prologue would be scheduled differently, and the compiler would then
    // wait as if its last loads were the ones still in flight).  Step k uses
    // set (k + RING) mod (RING + 1) and refills the set of step k - 1.
    for (int k = -RING; k < nk; k += RING + 1) {
#pragma unroll
      for (int r = 0; r <= RING; ++r) page(k + r, kset[r], vset[r], kset[(r + RING) % (RING + 1)], vset[(r + RING) % (RING + 1)]);
    }
  }
  wait_all_memory();

  // ---- results: every wave holds the same (m, l) and its own hd slice ----
  if (lc == 0) xfer[wave][ln] = m_run;
  wave_lds_sync();
  const f32x4 mo = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);
  const bool fused = st > 1 && a.counters != nullptr;
  const bool direct = st == 1 && (a.splits == 1 || a.counters != nullptr);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * lc + i;
    if (r >= ncols) continue;
    const Column rc = tile_column(r, a.group, nrows, hb, 16);
    const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
    if (direct) {
      const float l = lacc[i];
#pragma unroll
      for (int u = 0; u < DS; ++u) {
        const float v = l > 0.f ? oacc[u][i] / l : 0.f;
        a.out[th * HD + h0 + 16 * u + ln] = f32_to_bf16_rne(v);
      }
    } else {
      const int64_t ps = th * a.splits + split;
      float *po = a.part_o + ps * HD + h0;
#pragma unroll
      for (int u = 0; u < DS; ++u) store_coherent(po + 16 * u + ln, oacc[u][i]);
      if (wave == 0 && ln == 0) {
        store_coherent(a.part_ml + 2 * ps, mo[i]);
        store_coherent(a.part_ml + 2 * ps + 1, lacc[i]);
      }
    }
  }
  if (!fused) return;
  __syncthreads();  // the V staging area is free for the merge scratch
  if (a.spin_ticks > 0) {
    owned_merge<HD, kThreads>(a, t0, kh, hb, nrows, ncols, 16, split, st, &s_is_last);
    return;
  }
  fused_merge<HD, kThreads>(a, t0, kh, hb, nrows, ncols, 16, st,
                            reinterpret_cast<FusedScratch<kThreads> *>(&vtile[0][0]), &s_is_last);
}

// ---- merge of one block of 32 consecutive hd elements of one (row, query head) ----
// The per-element arithmetic: M = max m_s over the non-empty splits
// (l_s > 0), w_s = exp2(m_s - M) (0 for an empty split); for each of the 8
// split groups g (split s is in group s mod 8) an fma chain over the group's
// splits in increasing order gives num_g = sum w_s o_s[d] and
// den_g = sum w_s l_s; out = (num_0 + ... + num_7) / (den_0 + ... + den_7),
// the sums taken in group order (0 if the denominator is 0).  The combine
// kernel and both forms of the fused merge run exactly this, so their bits
// agree.
// One wave merges a block: lane l takes split group l / 8 and elements
// 4 (l mod 8) .. 4 (l mod 8) + 3.  It loads the (m, l) and the 4 partial
// elements of every split of its group (16-byte loads, BATCH splits of each
// group per memory round trip: one round trip for up to 8 BATCH splits, all
// loads of a round issued before any is used), and the block max,
// the group denominators and the group sums are exchanged between lanes: no
// LDS, no barrier.  CPOL is the loads' cache policy: plain after a kernel
// boundary, device-coherent (read past this XCD's L2) inside the decode
// launch.  `live` false: nothing is loaded or written.
constexpr int kCpolPlain = 0;
constexpr int kCpolDevice = 16;           // sc1
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer
// Splits per group per round trip: 16 (measured: 32, one round trip for
// every S, is no faster in either merge and costs the combine 55 VGPRs).
constexpr int kMergeBatch = 16;
template <int CPOL, int BATCH, int WB = 1>
__device__ __forceinline__ void merge_wave32(const DecodeArgs &a, int64_t th, int d0, int hd, int lane, bool live,
                                             int S) {
  // WB > 1: the block is WB * 32 elements, lane (g, q) taking elements
  // d0 + 32 w + 4 q .. + 3 for w < WB (BATCH splits of a group, each WB loads,
  // per round trip).  Every element's arithmetic is the same as with WB = 1.
  if (!live) return;
  const int g = lane >> 3, q = lane & 7;
  const int ni = (S + kMergeGroups - 1) / kMergeGroups;  // splits per group (at most)
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o + th * a.splits * hd, 0, S * hd * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rml =
      __builtin_amdgcn_make_buffer_rsrc(a.part_ml + th * a.splits * 2, 0, S * 8, kBufferWord3);
  // (m, l) of the group's splits: the group's i-th split (s = g + 8 i) is
  // loaded by lane 8 g + (i mod 8), as its (i / 8)-th pair (past split S - 1:
  // split S - 1 again, never used)
  constexpr int kPairs = kMaxSplits / kMergeGroups / 8;  // pairs per lane
  f32x2 mlk[kPairs];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int i = q + 8 * k;
    mlk[k] = f32x2{0.f, 0.f};
    if (8 * k < ni) {
      mlk[k] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             rml, min(g + kMergeGroups * i, S - 1) * 8, 0, CPOL));
    }
  }
  f32x4 v[BATCH][WB];
  auto load_batch = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i)
      if (i0 + i < ni)
#pragma unroll
        for (int w = 0; w < WB; ++w)
          v[i][w] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         ro, (min(g + kMergeGroups * (i0 + i), S - 1) * hd + d0 + 32 * w + 4 * q) * 4, 0, CPOL));
  };
  load_batch(0);
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int i = q + 8 * k;
    if (i < ni && g + kMergeGroups * i < S && mlk[k].y > 0.f) mx = fmaxf(mx, mlk[k].x);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float dg = 0.f;
  f32x4 num[WB];
#pragma unroll
  for (int w = 0; w < WB; ++w) num[w] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lead = lane & ~7;  // lane 8 g
  auto chain = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int ii = i0 + i;
      if (ii < ni) {
        const float m_s = __shfl(mlk[ii >> 3].x, lead + (ii & 7));
        const float l_s = __shfl(mlk[ii >> 3].y, lead + (ii & 7));
        if (g + kMergeGroups * ii < S) {
          const float ws = l_s > 0.f ? fast_exp2(m_s - mx) : 0.f;
          if (ws != 0.f) {
            dg = __builtin_fmaf(ws, l_s, dg);
#pragma unroll
            for (int w = 0; w < WB; ++w)
#pragma unroll
              for (int c = 0; c < 4; ++c) num[w][c] = __builtin_fmaf(ws, v[i][w][c], num[w][c]);
          }
        }
      }
    }
  };
  chain(0);
#pragma unroll
  for (int i0 = BATCH; i0 < kMaxSplits / kMergeGroups; i0 += BATCH) {
    if (ni > i0) {  // more than 8 i0 splits: another round trip
      load_batch(i0);
      chain(i0);
    }
  }
  // sums over the 8 groups in group order
  float den = 0.f;
  f32x4 n[WB];
#pragma unroll
  for (int w = 0; w < WB; ++w) n[w] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gg = 0; gg < kMergeGroups; ++gg) {
    den += __shfl(dg, gg * 8);
#pragma unroll
    for (int w = 0; w < WB; ++w)
#pragma unroll
      for (int c = 0; c < 4; ++c) n[w][c] += __shfl(num[w][c], gg * 8 + q);
  }
  if (g == 0) {
#pragma unroll
    for (int w = 0; w < WB; ++w) {
      uint16_t *op = a.out + th * hd + d0 + 32 * w + 4 * q;
#pragma unroll
      for (int c = 0; c < 4; ++c) op[c] = f32_to_bf16_rne(den > 0.f ? n[w][c] / den : 0.f);
    }
  }
}

// The same arithmetic for up to 16 splits with one lane per 4 elements: lane l
// takes elements d0 + 4 l .. + 3 (a block of 256) and loads every split's
// partial and (m, l) itself (one round trip), then runs the 8 group chains
// and their in-order sum on its own -- no exchange between lanes.
constexpr int kLaneMergeSplits = 16;
template <int CPOL>
__device__ __forceinline__ void merge_lanes256(const DecodeArgs &a, int64_t th, int d0, int hd, int lane, int S) {
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o + th * a.splits * hd, 0, S * hd * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rml =
      __builtin_amdgcn_make_buffer_rsrc(a.part_ml + th * a.splits * 2, 0, S * 8, kBufferWord3);
  f32x2 ml[kLaneMergeSplits];
  f32x4 v[kLaneMergeSplits];
#pragma unroll
  for (int s = 0; s < kLaneMergeSplits; ++s) {
    if (s < S) {
      ml[s] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rml, s * 8, 0, CPOL));
      v[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (s * hd + d0 + 4 * lane) * 4, 0, CPOL));
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kLaneMergeSplits; ++s)
    if (s < S && ml[s].y > 0.f) mx = fmaxf(mx, ml[s].x);
  float dg[kMergeGroups];
  f32x4 num[kMergeGroups];
#pragma unroll
  for (int g = 0; g < kMergeGroups; ++g) {
    dg[g] = 0.f;
    num[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < kLaneMergeSplits; ++s) {
    if (s < S) {
      const int g = s % kMergeGroups;
      const float ws = ml[s].y > 0.f ? fast_exp2(ml[s].x - mx) : 0.f;
      if (ws != 0.f) {
        dg[g] = __builtin_fmaf(ws, ml[s].y, dg[g]);
#pragma unroll
        for (int c = 0; c < 4; ++c) num[g][c] = __builtin_fmaf(ws, v[s][c], num[g][c]);
      }
    }
  }
  float den = 0.f;
  f32x4 n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < kMergeGroups; ++g) {
    den += dg[g];
#pragma unroll
    for (int c = 0; c < 4; ++c) n[c] += num[g][c];
  }
  uint16_t *op = a.out + th * hd + d0 + 4 * lane;
#pragma unroll
  for (int c = 0; c < 4; ++c) op[c] = f32_to_bf16_rne(den > 0.f ? n[c] / den : 0.f);
}

// Separate merge: one wave per (row, query head, 32 hd elements).
__global__ __launch_bounds__(64) void pgqa_combine_kernel(DecodeArgs a, int hd) {
  const int chunks = hd / 32;
  const int64_t th = blockIdx.x / chunks;
  const int d0 = static_cast<int>(blockIdx.x - th * chunks) * 32;
  merge_wave32<kCpolPlain, kMergeBatch>(a, th, d0, hd, threadIdx.x, true, a.splits);
}

// ---- parallel fused merge of one unit (owned blocks) ----
// S below is the tile's split count (pgqa_tile_splits): only those
// workgroups of the unit take part.
// The unit's outputs are cut into blocks of 32 elements and the blocks into
// chunks of one block per wave of a workgroup; chunk c belongs to the
// workgroup of split c mod S, whose waves merge its blocks one each.  Only
// the workgroups of splits below the chunk count own a chunk.  The others
// neither wait nor merge, so their done counts (step 3) land while the last
// arrivals are still running instead of after the merge.  Three counter
// words per unit, on separate cache lines: arrivals, a ready flag and a done
// count.
//  1. Every workgroup, once its partial stores have completed (they write
//     through to memory), adds 1 to the arrival word.  The one that draws
//     S - 1 is the last to arrive: every partial of the unit is in memory,
//     and it sets the ready flag.
//  2. A workgroup that owns a chunk polls the flag -- a word written once,
//     so polling it does not slow the arrivals down -- for at most
//     spin_ticks of the 100 MHz real-time counter, then merges its blocks
//     with the combine kernel's per-element arithmetic (device-coherent
//     loads).  One that gives up merges nothing.
//  3. Every workgroup adds 1 + (blocks merged << 16) to the done word.  The
//     one that completes it (low half S - 1) is the last to touch any of the
//     three words: if fewer than all blocks were merged (a workgroup gave up),
//     it merges every block itself -- merging a block twice writes the same
//     bits -- and then it resets the three words to zero for the next call.
// No workgroup waits on another for more than spin_ticks, and none needs
// another to be resident: a launch larger than the device holds only merges
// later.
constexpr int64_t kParallelMergeBytes = int64_t(64) << 10;  // per-unit partials from which the merge goes parallel
constexpr int kClaimSpinTicks = 2000;                        // 20 us
constexpr int kFlagBase = 2048;  // ready flags: counters[kFlagBase + unit]
constexpr int kDoneBase = 3072;  // done counts: counters[kDoneBase + unit]
constexpr int kOwnedMergeUnits = 1024;  // units the three-word layout holds
// Bound of the parallel merge's waits for the calls that follow, set by
// pgqa_set_merge_wait_ticks (0: kClaimSpinTicks).
std::atomic<int> g_merge_wait_ticks{0};
// Page step of narrow tiles (pgqa_set_narrow_path): 0 chooses by launch size,
// 1 takes the vector-ALU step wherever it applies, 2 never.
std::atomic<int> g_narrow_path{0};

// Chunks first, first + step, ... of the unit (chunk c: blocks c * waves ..
// c * waves + waves - 1 below nblocks, one per wave; block b: column
// b / (HD / 32), elements (b mod (HD / 32)) 32 ..).  Returns how many blocks
// this workgroup merged (the same in every thread).
template <int HD, int NT, int WB>
__device__ int merge_blocks(const DecodeArgs &a, int t0, int kh, int hb, int nrows, int nblocks, int cap, int first,
                            int step, int S) {
  constexpr int per_col = HD / (32 * WB);
  static_assert(per_col >= 1 && HD % (32 * WB) == 0, "a merge block must divide hd");
  constexpr int waves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int merged = 0;
  for (int c = first; c * waves < nblocks; c += step) {
    const int b = c * waves + wave;
    if (b < nblocks) {
      const Column rc = tile_column(b / per_col, a.group, nrows, hb, cap);
      const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
      if constexpr (WB == 1) merge_wave32<kCpolDevice, kMergeBatch>(a, th, (b % per_col) * 32, HD, lane, true, S);
      else if constexpr (WB == 8) merge_lanes256<kCpolDevice>(a, th, (b % per_col) * 256, HD, lane, S);
      else merge_wave32<kCpolDevice, kMergeBatch / WB, WB>(a, th, (b % per_col) * 32 * WB, HD, lane, true, S);
    }
    merged += min(waves, nblocks - c * waves);
  }
  return merged;
}

template <int HD, int NT, int WB>
__device__ void owned_merge_wb(const DecodeArgs &a, int t0, int kh, int hb, int nrows, int ncols, int cap, int split,
                               int st, int *s_word) {
  const int unit = (t0 * a.nkv + kh) * a.hblocks + hb;
  int32_t *arrive = a.counters + unit;
  int32_t *flag = a.counters + kFlagBase + unit;
  int32_t *done = a.counters + kDoneBase + unit;
  const int S = st;  // the tile's splits: arrivals, owners and partials merged
  const int nblocks = ncols * (HD / (32 * WB));
  const int nchunks = (nblocks + NT / 64 - 1) / (NT / 64);
  const int tid = threadIdx.x;
  wait_all_memory();  // this workgroup's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const int t = __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ready = t == S - 1;
    if (ready) {
      __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (split < nchunks) {
      const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
      while (__builtin_amdgcn_s_memrealtime() - t_start < static_cast<uint64_t>(a.spin_ticks)) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
          ready = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    *s_word = ready;
  }
  __syncthreads();
  // pass 0: this workgroup's own blocks (if it saw the flag); pass 1, only in
  // the last workgroup to finish and only if some workgroup gave up: every
  // block (a block merged twice gets the same bits).  One call site keeps
  // the merge code in the kernel once.
  int first = split, step = S;
  for (int pass = 0; pass < 2; ++pass) {
    int merged = 0;
    if (*s_word > 0) merged = merge_blocks<HD, NT, WB>(a, t0, kh, hb, nrows, nblocks, cap, first, step, S);
    __syncthreads();  // every thread has read s_word
    if (pass == 1) break;
    if (tid == 0) {
      const int d = __hip_atomic_fetch_add(done, 1 + (merged << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_word = (d & 0xffff) != S - 1 ? -1 : ((d >> 16) + merged < nblocks ? 1 : 0);
    }
    __syncthreads();
    if (*s_word < 0) return;  // not the last to finish
    first = 0;
    step = 1;
  }
  // the last workgroup to finish: nobody touches the three words any more
  if (tid == 0) {
    __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Up to 16 splits (hd 256 and 512), blocks of 256 elements merged lane by
// lane; up to 32, blocks of 128 elements (a merge of a few splits is one
// short round trip, so fewer, wider blocks leave fewer rounds per owner);
// 32 elements otherwise.  WIDE false: 32 elements always.
template <int HD, int NT, bool WIDE>
__device__ void owned_merge(const DecodeArgs &a, int t0, int kh, int hb, int nrows, int ncols, int cap, int split,
                            int st, int *s_word) {
  if constexpr (WIDE && HD >= 256) {
    if (st <= kLaneMergeSplits) {
      owned_merge_wb<HD, NT, 8>(a, t0, kh, hb, nrows, ncols, cap, split, st, s_word);
      return;
    }
  }
  if (WIDE && st <= 4 * kMergeGroups) owned_merge_wb<HD, NT, 4>(a, t0, kh, hb, nrows, ncols, cap, split, st, s_word);
  else owned_merge_wb<HD, NT, 1>(a, t0, kh, hb, nrows, ncols, cap, split, st, s_word);
}

// ---------------------------------------------------------------------------
// Shared-page kernel: tiles of up to 64 columns (e.g. 8 rows x 8 heads of one
// sequence) and hd-512 tiles too wide for the per-wave kernel or in calls of
// fewer than 64 splits.  8 waves in two teams of 4; team t takes
// the split's pages 2j + t, so every SIMD holds two waves whose latency chains
// (LDS reads, MFMA, exp) overlap.  Both teams stage their pages' K and V in
// LDS with direct-to-LDS loads (global_load_lds_dwordx4) into a ring of NP
// slots of one page pair each, NP - 1 pairs ahead of the pair being computed.
//   LDS K layout: MFMA operand order -- 16-byte chunk s is the A operand of
//     step s / 64 for lane s % 64 (token s % 16, hd (4 (s/64) + (s/16) % 4) * 8).
//   LDS V layout: [hd block of 16][token][16] -- the 16 lanes of a transpose
//     read group cover 4 tokens x 16 columns contiguously.
// Within a team the waves form 4/NSL column blocks x NSL hd slices: wave w
// scores column block w / NSL over hd slice w % NSL; with NSL > 1 the slices'
// partial scores are summed through LDS in slice order, so the waves of a
// block hold identical scores and softmax state, and each accumulates P V for
// its own slice.  NSL is fixed per launch (from the widest tile the shapes
// allow), so every MFMA is unconditional.  At the end team 1's softmax state
// is merged into team 0's in a fixed order.
// Every wave waits for its own loads of a pair, then a barrier makes the pair
// complete; the same barrier tells that the slot refilled next is free.
// ---------------------------------------------------------------------------
constexpr int kSharedThreads = 512;
template <int HD, int NSL, bool WIDE>
__global__ __launch_bounds__(kSharedThreads) void pgqa_shared_kernel(DecodeArgs a) {
  constexpr int KJ = HD / 32;              // QK^T MFMA steps over the whole hd
  constexpr int DJ = HD / 16;              // PV MFMA output blocks over the whole hd
  constexpr int KS = KJ / NSL;             // ... per slice
  constexpr int DS = DJ / NSL;
  constexpr int QBM = kWaves / NSL;        // column blocks per team
  constexpr int CAP = 16 * QBM;            // columns per team
  // WIDE (prefill, one split): the teams take different column blocks of a
  // tile twice as wide and both compute every page of a pair, so a page is
  // read once per 2 CAP columns and there is no team merge.
  constexpr int TCAP = WIDE ? 2 * CAP : CAP;  // columns per tile
  constexpr int PAGE_ELEMS = kPage * HD;   // bf16 elements of one K (or V) page
  constexpr int SLOT_ELEMS = 4 * PAGE_ELEMS;  // a page pair: team 0's K, V, then team 1's
  constexpr int NP = HD == 512 ? 2 : HD == 256 ? 4 : 6;  // ring slots (128, 128, 96 KB)
  constexpr int LW = HD / 128;             // 1 KB direct loads per wave per page, each of K and V
  constexpr int INFLIGHT = (NP - 2) * 2 * LW;  // this wave's loads still allowed in flight
  constexpr int MCH = HD / 32 < DS ? HD / 32 : DS;  // output blocks per team-merge round
  static_assert(LW >= 1 && KS >= 1, "the shared-page kernel needs hd >= 128 and hd / 32 >= slices");
  static_assert(DS % MCH == 0, "team merge rounds must cover the slice");
  // One object per ring slot and a pair loop unrolled by NP, so every LDS
  // access names its slot at compile time and the compiler can tell reads of
  // one slot from the direct loads still landing in the others.
  __shared__ __attribute__((aligned(16))) uint16_t slot0[SLOT_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t slot1[SLOT_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t slot2[NP > 2 ? SLOT_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t slot3[NP > 3 ? SLOT_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t slot4[NP > 4 ? SLOT_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t slot5[NP > 5 ? SLOT_ELEMS : 8];
  // partial scores per wave (WIDE: per wave and page of the pair, so the
  // second page's exchange cannot overwrite the first's before it is read)
  __shared__ __attribute__((aligned(16))) f32x4 xscore[(WIDE ? 4 : 2) * kWaves][64];
  __shared__ float xfer[2 * kWaves][16];
  __shared__ int s_is_last;
  __shared__ int4 s_tiles[64];  // tiles whose parallel merge follows the page loop (row, rows, columns, splits)
  static_assert(sizeof(FusedScratch<kSharedThreads>) <= sizeof(slot0), "merge scratch must fit a ring slot");
  static_assert(256 * MCH * 16 <= sizeof(slot0), "team merge round must fit a ring slot");
  // Ring slot I as a direct reference to its own object (no pointer table):
  // the compiler then knows which object every LDS access touches.
  auto slot = [&](auto I) __attribute__((always_inline)) -> uint16_t * {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return slot0;
    else if constexpr (i == 1) return slot1;
    else if constexpr (i == 2) return slot2;
    else if constexpr (i == 3) return slot3;
    else if constexpr (i == 4) return slot4;
    else return slot5;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave >> 2;  // wave-uniform
  const int w4 = wave & 3;     // wave within the team
  const int ln = lane & 15;
  const int lc = lane >> 4;
  const int cb = w4 / NSL;     // this wave's column block
  const int sl = w4 % NSL;     // ... and hd slice
  const int cbt = cb + (WIDE ? team * QBM : 0);  // column block within the tile
  const int j0 = sl * KS;      // first QK step of the slice
  const int jj0 = sl * DS;     // first PV block of the slice

  int b = blockIdx.x;
  const int split = b % a.splits;
  b /= a.splits;
  const int hb = b % a.hblocks;
  b /= a.hblocks;
  const int kh = b % a.nkv;
  // this workgroup's rmax-aligned block of rows; it takes the block's tiles
  // (runs of rows on one sequence) one after another
  // (prefill: one caller-made sub-tile)
  int sub_rows = 0;
  int rb0 = a.rank_rows ? row_of_rank(a, b / a.nkv, lane) : (b / a.nkv) * a.rmax;  // ranked: one-row blocks
  int rb1 = min(rb0 + a.rmax, a.rows);
  if (a.tile_row0) {
    rb0 = prefill_subtile(a, b / a.nkv, sub_rows);
    rb1 = sub_rows > 0 ? rb0 + 1 : rb0;
  }
  int n_tiles = 0;  // wave-uniform count of s_tiles entries
  for (int t0 = rb0; t0 < rb1;) {
    const Tile tile = tile_rows(a, t0, lane, sub_rows);
    const int nrows = tile.nrows;
    const int ncols = a.group <= TCAP ? nrows * a.group : min(TCAP, a.group - hb * TCAP);
    const int st = tile_splits(tile, a.splits);
    if (split >= st) {
      if (a.counters == nullptr) mark_empty_split(a, t0, kh, hb, nrows, ncols, TCAP, split);
      t0 += nrows;
      continue;
    }
    int pbeg, pend;
    split_range(tile, split, st, pbeg, pend);
    const bool active = 16 * cbt < ncols;  // this wave's column block exists (wave-uniform)

    const Column col = tile_column(16 * cbt + ln, a.group, nrows, hb, TCAP);
    const int col_lo = __shfl(tile.lo_l, col.row);
    // shuffle with every lane active, then drop columns without a row
    const int col_hi_any = __shfl(tile.hi_l, col.row);
    const int col_hi = col.on ? col_hi_any : -1;
    bf16x8 qop[KS];
    {
      const uint16_t *qrow = a.q + (static_cast<int64_t>(t0 + (col.on ? col.row : 0)) * a.nh + kh * a.group + col.head) * HD;
  #pragma unroll
      for (int u = 0; u < KS; ++u) {
        u32x4 z = {0u, 0u, 0u, 0u};
        qop[u] = __builtin_bit_cast(bf16x8, z);
        if (col.on) qop[u] = *reinterpret_cast<const bf16x8 *>(qrow + (4 * (j0 + u) + lc) * 8);
      }
    }

    float m_run = -INFINITY;  // reference max (log2 units) of column ln, the same in the column's 4 lanes
    f32x4 oacc[DS];
    f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
    for (int u = 0; u < DS; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const s16x4 ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80};
    const int64_t kv_head_off = static_cast<int64_t>(kh) * kPage * HD;
    const int64_t page_elems = static_cast<int64_t>(a.nkv) * kPage * HD;

    // Global source (element offset in the page) of this lane's chunk of each
    // of the wave's 1 KB direct loads: K chunk s = 64 i + lane, V chunk likewise.
    int k_src[LW], v_src[LW];
  #pragma unroll
    for (int r = 0; r < LW; ++r) {
      const int s = (w4 * LW + r) * 64 + lane;
      k_src[r] = (s & 15) * HD + (4 * (s >> 6) + ((s >> 4) & 3)) * 8;
      v_src[r] = ((s & 31) >> 1) * HD + (s >> 5) * 16 + (s & 1) * 8;
    }

    const int nk = pend - pbeg;
    const int npairs = (nk + 1) / 2;
    int pv0 = 0, pv1 = 0, pw0 = -1;  // physical pages of pages [pw0, pw0 + 128)
    auto fetch_window = [&](int w0) __attribute__((always_inline)) {
      int ph[2];
  #pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = w0 + 64 * h + lane;
        ph[h] = 0;
        if (k < nk) {
          ph[h] = a.block_table[tile.origin + pbeg + k];
          if (a.page_map) ph[h] = a.page_map[ph[h]];
        }
      }
      pv0 = ph[0];
      pv1 = ph[1];
      pw0 = w0;
      wait_all_memory();
    };
    // Requests this team's page of pair j into ring slot `dst`.  Past the
    // split's end it requests the last page again: every step issues the same
    // number of loads, so the counted waits below stay exact (and the compiler
    // can tell which loads an LDS read must wait for).
    auto issue_pair = [&](int j, uint16_t *dst) __attribute__((always_inline)) {
      const int k = min(2 * j + team, nk - 1);
      if (k - pw0 >= 128) fetch_window(k - team);  // drains the ring once per 128 pages
      const int kw = k - pw0;
      const int phys = kw < 64 ? __builtin_amdgcn_readlane(pv0, kw) : __builtin_amdgcn_readlane(pv1, kw - 64);
      const int64_t page_off = static_cast<int64_t>(phys) * page_elems + kv_head_off;
      const uint16_t *kp = a.k_pool + page_off;
      const uint16_t *vp = a.v_pool + page_off;
      uint16_t *kdst = dst + team * 2 * PAGE_ELEMS + w4 * LW * 512;
      uint16_t *vdst = kdst + PAGE_ELEMS;
  #pragma unroll
      for (int r = 0; r < LW; ++r) {
        load_to_lds16(kp + k_src[r], kdst + r * 512);
        load_to_lds16(vp + v_src[r], vdst + r * 512);
      }
    };

    // Page pk of pair j (in the pair's ring slot `buf`) for this wave's
    // columns: scores, online softmax, P V.
    auto page = [&](int j, int pk, const uint16_t *buf) __attribute__((always_inline)) {
      const int k = 2 * j + pk;
      const int p = pbeg + k;
      const bool full = p >= tile.fp0 && p < tile.fp1;  // the same in every wave of the team
      uint32_t tokmask = 0;
      if (k < nk) {
        tokmask = 0xffffu;
        if (!full) {
          // tokens of this page some row of the tile can see
          uint32_t mrow = 0;
          if (lane < nrows) {
            const int lo = max(tile.lo_l - p * kPage, 0), hi = min(tile.hi_l - p * kPage, kPage - 1);
            if (hi >= lo) mrow = ((2u << hi) - 1u) & ~((1u << lo) - 1u);
          }
  #pragma unroll
          for (int off = 32; off >= 1; off >>= 1) mrow |= __shfl_xor(mrow, off);
          tokmask = __builtin_amdgcn_readfirstlane(mrow);
        }
      }
      const bool work = tokmask != 0;  // the same in every wave of the team

      const uint16_t *kt = buf + pk * 2 * PAGE_ELEMS;
      const uint16_t *vt = kt + PAGE_ELEMS;
      // lane (4m+q) of group lc reads token 4 lc + m, columns 4q..4q+3 of each block
      const uint16_t *vtr = vt + (4 * lc + (ln >> 2)) * 16 + 4 * (ln & 3) + jj0 * 256;
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
      s16x4 vb[DS];
      if (work) {
        // partial scores over this wave's hd slice: all K operands read first,
        // two accumulation chains; V operands requested meanwhile
        bf16x8 kop[KS];
  #pragma unroll
        for (int u = 0; u < KS; ++u) kop[u] = *reinterpret_cast<const bf16x8 *>(kt + ((j0 + u) * 64 + lane) * 8);
        {
          const uint32_t va = lds_address(vtr);
          [&]<int... U>(std::integer_sequence<int, U...>) {
            ((vb[U] = lds_read_tr16<U * 512>(va)), ...);
          }(std::make_integer_sequence<int, DS>{});
        }
        f32x4 sc1 = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int u = 0; u < KS; ++u) {
          if ((u & 1) == 0) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u], qop[u], sc, 0, 0, 0);
          else sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u], qop[u], sc1, 0, 0, 0);
        }
        if constexpr (KS > 1) sc += sc1;
      }
      if constexpr (NSL > 1) {
        // every wave of both teams takes part in the exchange barrier
        const int xr = WIDE ? 2 : 1, xp = WIDE ? pk : 0;  // rows per wave, this page's row
        if (work) xscore[xr * wave + xp][lane] = sc;
        lds_barrier();
        if (work) {
          const int w0 = 4 * team + cb * NSL;
          sc = xscore[xr * w0 + xp][lane];
  #pragma unroll
          for (int s2 = 1; s2 < NSL; ++s2) sc += xscore[xr * (w0 + s2) + xp][lane];
        }
      }
      if (!work || !active) return;

      bool vis[4] = {true, true, true, true};
      if (!full) {
        const int pos0 = p * kPage + 4 * lc;
  #pragma unroll
        for (int t = 0; t < 4; ++t) vis[t] = pos0 + t >= col_lo && pos0 + t <= col_hi;
      }
      float sv[4];
      float lmx = -INFINITY;
  #pragma unroll
      for (int t = 0; t < 4; ++t) {
        sv[t] = vis[t] ? sc[t] : -INFINITY;
        lmx = fmaxf(lmx, sv[t]);
      }
      // The column's reference max moves only when one of its scores passes it
      // by more than the slack; only then is the column max taken across lanes.
      if (__ballot(lmx * kLog2e > m_run + kRescaleSlack) != 0) {
        float mx = lmx;
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m2 = mx * kLog2e;
        const bool grow = m2 > m_run + kRescaleSlack;  // the same in the column's 4 lanes
        const float m_new = grow ? m2 : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
        m_run = m_new;
        if (lc == 0) xfer[wave][ln] = alpha;
        wave_lds_sync();
        const f32x4 al = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);
  #pragma unroll
        for (int u = 0; u < DS; ++u) oacc[u] *= al;
        lacc *= al;
      }
      float pr[4];
  #pragma unroll
      for (int t = 0; t < 4; ++t) {
        pr[t] = fast_exp2(__builtin_fmaf(sv[t], kLog2e, -m_run));
        if (!full) pr[t] = sv[t] == -INFINITY ? 0.f : pr[t];
      }
      const s16x4 pa = pack_weights(pr[0], pr[1], pr[2], pr[3]);
      lds_wait_reads();  // the V operands have arrived
      if (!full) {
        // tokens no column can see may hold NaN: zero their V entries
        const uint32_t keep = (tokmask >> (4 * lc)) & 0xfu;
  #pragma unroll
        for (int u = 0; u < DS; ++u)
  #pragma unroll
          for (int r = 0; r < 4; ++r) vb[u][r] = (keep >> r) & 1u ? vb[u][r] : static_cast<short>(0);
      }
  #pragma unroll
      for (int u = 0; u < DS; ++u) oacc[u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb[u], oacc[u], 0, 0, 0);
      lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ones, lacc, 0, 0, 0);
    };

    // One pair: wait for it, refill the slot of the pair before it, compute this
    // team's page of it (WIDE: both pages, for this team's columns).
    auto step = [&](int j, const uint16_t *buf, uint16_t *refill) __attribute__((always_inline)) {
      // this wave's loads of pair j have landed once at most the loads of the
      // pairs after it are outstanding; the barrier then makes the whole pair
      // visible and tells that the slot of pair j - 1 is no longer read
      __builtin_amdgcn_s_waitcnt((INFLIGHT & 15) | ((INFLIGHT >> 4) << 14) | 0x0f70);
      lds_barrier();
      issue_pair(j + NP - 1, refill);
      if constexpr (WIDE) {
        page(j, 0, buf);
        page(j, 1, buf);
      } else {
        page(j, team, buf);
      }
    };

    if (npairs > 0) {
      fetch_window(0);
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (issue_pair(I, slot(std::integral_constant<int, I>{})), ...);
      }(std::make_integer_sequence<int, NP - 1>{});
      for (int j = 0; j < npairs; j += NP) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (step(j + I, slot(std::integral_constant<int, I>{}), slot(std::integral_constant<int, (I + NP - 1) % NP>{})), ...);
        }(std::make_integer_sequence<int, NP>{});
      }
    }
    wait_all_memory();
    __syncthreads();

    // ---- team 1's state joins team 0's: per column, the larger reference max
    // wins and both sums are scaled to it (team 0 first) ----
    float mo[4], lo[4];
    {
      if (lc == 0) xfer[wave][ln] = m_run;
      wave_lds_sync();
      const f32x4 m4 = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        mo[i] = m4[i];
        lo[i] = lacc[i];
      }
    }
    if constexpr (!WIDE) {
      float sa[4] = {1.f, 1.f, 1.f, 1.f}, sb[4] = {0.f, 0.f, 0.f, 0.f};
      f32x4 *xm = reinterpret_cast<f32x4 *>(&xscore[0][0]);  // [w4][lane] (m x4, l x4)
      __syncthreads();
      if (team == 1) {
        xm[(w4 * 64 + lane) * 2] = f32x4{mo[0], mo[1], mo[2], mo[3]};
        xm[(w4 * 64 + lane) * 2 + 1] = f32x4{lo[0], lo[1], lo[2], lo[3]};
      }
      __syncthreads();
      if (team == 0) {
        const f32x4 mb = xm[(w4 * 64 + lane) * 2];
        const f32x4 lb = xm[(w4 * 64 + lane) * 2 + 1];
    #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float mm = fmaxf(mo[i], mb[i]);
          sa[i] = mm == -INFINITY ? 0.f : fast_exp2(mo[i] - mm);
          sb[i] = mm == -INFINITY ? 0.f : fast_exp2(mb[i] - mm);
          lo[i] = lo[i] * sa[i] + lb[i] * sb[i];
          mo[i] = mm;
        }
      }
      {
        f32x4 *xo = reinterpret_cast<f32x4 *>(slot0);  // [w4][u][lane]
    #pragma unroll
        for (int u0 = 0; u0 < DS; u0 += MCH) {
          __syncthreads();
          if (team == 1) {
    #pragma unroll
            for (int u = 0; u < MCH; ++u) xo[(w4 * MCH + u) * 64 + lane] = oacc[u0 + u];
          }
          __syncthreads();
          if (team == 0) {
    #pragma unroll
            for (int u = 0; u < MCH; ++u) {
              const f32x4 ob = xo[(w4 * MCH + u) * 64 + lane];
    #pragma unroll
              for (int i = 0; i < 4; ++i) oacc[u0 + u][i] = oacc[u0 + u][i] * sa[i] + ob[i] * sb[i];
            }
          }
        }
      }
    }

    // ---- results: team 0 (WIDE: both teams), this wave's hd slice of its
    // column block ----
    const bool fused = !WIDE && st > 1 && a.counters != nullptr;
    const bool direct = st == 1 && (a.splits == 1 || a.counters != nullptr);
    if ((WIDE || team == 0) && active) {
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * cbt + 4 * lc + i;
        if (r >= ncols) continue;
        const Column rc = tile_column(r, a.group, nrows, hb, TCAP);
        const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
        if (direct) {
          const float l = lo[i];
  #pragma unroll
          for (int u = 0; u < DS; ++u) {
            const float v = l > 0.f ? oacc[u][i] / l : 0.f;
            a.out[th * HD + 16 * (jj0 + u) + ln] = f32_to_bf16_rne(v);
          }
        } else {
          const int64_t ps = th * a.splits + split;
          float *po = a.part_o + ps * HD + 16 * jj0;
  #pragma unroll
          for (int u = 0; u < DS; ++u) store_coherent(po + 16 * u + ln, oacc[u][i]);
          if (sl == 0 && ln == 0) {
            store_coherent(a.part_ml + 2 * ps, mo[i]);
            store_coherent(a.part_ml + 2 * ps + 1, lo[i]);
          }
        }
      }
    }
    __syncthreads();  // the team-merge area (slot 0) is free again
    if constexpr (!WIDE) {
      if (fused) {
        if (a.spin_ticks > 0) {
          // merged after the page loop (its registers are free then)
          if (tid == 0) s_tiles[n_tiles] = int4{t0, nrows, ncols, st};
          ++n_tiles;
        } else {
          fused_merge<HD, kSharedThreads>(a, t0, kh, hb, nrows, ncols, CAP, st,
                                          reinterpret_cast<FusedScratch<kSharedThreads> *>(slot0), &s_is_last);
        }
      }
    }
    t0 += nrows;
    __syncthreads();  // LDS is reused by the next tile
  }
  if constexpr (WIDE) return;
  for (int i = 0; i < n_tiles; ++i) {
    const int4 tl = s_tiles[i];
    owned_merge<HD, kSharedThreads, false>(a, tl.x, kh, hb, tl.y, tl.z, CAP, split, tl.w, &s_is_last);
    __syncthreads();
  }
}


using pgqa_detail::fail;

// Which kernel runs and how rows are tiled, from the call's shapes only (so
// calls that differ only in data -- merge mode, page placement -- run the same
// code).  The shared-page kernel takes, from hd 128 up, tiles of more than 16
// columns (groups of 8 or more; every group at hd 512); hd-512 tiles of up to
// 16 columns go to the hd-sliced kernel (measured against the per-wave kernel
// at hd 512: 28.3 against 31.8 us of kernel time on a 32K-key, 8-column call,
// and faster from 11 to 256 splits); the per-wave kernel takes the rest.
// With fewer columns than the shared-page kernel's 64 the hd is cut into
// slices so that all 4 waves still have work.
struct Plan {
  int kind;     // 0: per-wave kernel, 1: shared-page kernel, 2: hd-sliced kernel
  int wide = 0; // shared-page kernel with the teams on separate columns (prefill)
  int nsl;      // hd slices per column block (shared-page kernel)
  int cap;      // columns per tile
  int rmax;     // rows per tile
  int hblocks;  // head blocks per kv head
  int valu = 0; // per-wave kernel with the vector-ALU page step
};
// The largest split count pgqa_choose_splits gives a batch of sequences (its
// bandwidth regime's cap; its latency regime stays at or below it from 4
// (sequence, kv head) units up).
constexpr int64_t kBatchMaxSplits = 16;

Plan make_plan(int64_t rows, int64_t group, int64_t hd, int64_t splits, int64_t nkv) {
  Plan p;
  // The host cannot see whether the rows share a sequence (the origins are
  // device data).  Tiles are sized for several rows of one sequence only
  // when the split count is above what any batch is given (a one-sequence
  // call over a long span); otherwise for one row per sequence.  Sized for
  // several rows, a batch of one-row sequences would leave each shared-page
  // workgroup walking rmax one-row tiles in turn, each on a fraction of its
  // columns (measured 1.4-2x slower at 8 and 16 heads per kv head).
  // Shorter one-sequence spans then run as if each row were its own
  // sequence: more workgroups read each page.
  const bool one_sequence = splits > kBatchMaxSplits;
  const int64_t trows = one_sequence ? rows : 1;
  int64_t cols = group <= 64 ? group * (trows < 64 / group ? trows : 64 / group) : 64;
  // Several-row tiles at hd 128 and 256 keep to 32 columns (two hd slices
  // per column block) while the launch, with twice the tiles, still fits one
  // round of 256 workgroups (one per CU): more workgroups share the span's
  // latency-bound page loop (measured 5-10% faster on windowed and 4K-16K
  // multi-row calls; longer spans, whose split counts fill the round, keep
  // 64 columns)
  if (one_sequence && (hd == 128 || hd == 256) && group <= 32 && cols > 32) {
    const int64_t half_rows = 32 / group;
    if (nkv * splits * ((rows + half_rows - 1) / half_rows) <= 256) cols = group * half_rows;
  }
  // groups of 8+ heads: several rows of one sequence fill a 64-column tile
  // (multi-row decode), as do groups of more than 16 heads on their own;
  // narrower groups keep the per-wave kernel, whose 16-column tiles waste
  // nothing when every row has its own sequence
  p.kind = hd >= 128 && cols > 16 && (group >= 8 || hd == 512) ? 1 : 0;
  // hd-512 tiles of up to 16 columns: the hd-sliced kernel
  if (hd == 512 && cols <= 16) p.kind = 2;
  p.nsl = p.kind == 1 ? (cols <= 16 ? 4 : cols <= 32 ? 2 : 1) : 1;
  if (p.kind == 1 && hd == 128 && p.nsl == 4) p.nsl = 2;  // hd 128 has 4 QK steps
  if (p.kind == 1 && hd == 512 && p.nsl == 1) p.nsl = 2;  // a whole hd-512 slice needs too many registers
  p.cap = p.kind == 1 ? 16 * (kWaves / p.nsl) : 16;
  p.rmax = group <= p.cap ? static_cast<int>(p.cap / group) : 1;
  p.hblocks = group <= p.cap ? 1 : static_cast<int>((group + p.cap - 1) / p.cap);
  return p;
}

// Prefill: tiles have many rows, so the shared-page kernel takes every hd
// from 128 up.  Its two teams take separate column blocks of one tile
// (128 columns, 64 at hd 512: each page read once per tile) when a caller
// tile's rows fill it -- at least 2 heads per kv head below hd 512 --, and
// alternate pages of 64-column tiles otherwise; hd 64 keeps the per-wave
// kernel's 16-column tiles.  At hd 256 a launch of fewer than 512 (tile, kv
// head) units takes the 64-column form too: twice the workgroups fill the
// GPU better (measured: the page's 1500-row shape 83.6 -> 70.6 us, a 2048-row
// context 126.7 -> 106.4 us; at hd 128 the narrow form is slower, 108 -> 142
// us, and from 512 units the wide form is faster at both).
constexpr int64_t kPrefillWideUnits = 512;
Plan make_prefill_plan(int64_t group, int64_t hd, int64_t units) {
  Plan p;
  p.kind = hd >= 128 ? 1 : 0;
  p.nsl = p.kind == 1 ? (hd == 512 ? 2 : 1) : 1;
  const int team_cap = 16 * (kWaves / p.nsl);
  p.wide = p.kind == 1 && 2 * team_cap <= kPrefillRowsPerTile * group && !(hd == 256 && units < kPrefillWideUnits);
  p.cap = p.kind == 1 ? (p.wide ? 2 : 1) * team_cap : 16;
  p.rmax = group <= p.cap ? static_cast<int>(p.cap / group) : 1;
  p.hblocks = group <= p.cap ? 1 : static_cast<int>((group + p.cap - 1) / p.cap);
  return p;
}

template <int HD, int NSL, bool WIDE = false>
hipError_t launch_shared(const DecodeArgs &a, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((pgqa_shared_kernel<HD, NSL, WIDE>), dim3(static_cast<unsigned>(blocks)), dim3(kSharedThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_decode(const DecodeArgs &a, const Plan &p, int64_t blocks, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if constexpr (HD >= 128) {
    if (p.kind == 1 && p.wide) {
      if constexpr (HD == 512) {
        if (p.nsl == 2) return launch_shared<HD, 2, true>(a, blocks, stream);
      } else {
        if (p.nsl == 1) return launch_shared<HD, 1, true>(a, blocks, stream);
      }
      return hipErrorInvalidValue;
    }
    if (p.kind == 1) {
      if (p.nsl == 2) return launch_shared<HD, 2>(a, blocks, stream);
      if constexpr (HD < 512) {
        if (p.nsl == 1) return launch_shared<HD, 1>(a, blocks, stream);
      }
      if constexpr (HD >= 256) {
        if (p.nsl == 4) return launch_shared<HD, 4>(a, blocks, stream);
      }
      return hipErrorInvalidValue;
    }
  }
  if constexpr (HD == 512) {
    // every hd-512 plan is the shared-page or the hd-sliced kernel
    if (p.kind != 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pgqa_slice_kernel<HD>, grid, block, 0, stream, a);
  } else {
    if constexpr (HD <= 256) {
      if (p.valu) {
        hipLaunchKernelGGL((pgqa_wave_kernel<HD, true>), grid, block, 0, stream, a);
        return hipGetLastError();
      }
    }
    if constexpr (HD == 128) {
      if (a.spin_ticks > 0) {
        hipLaunchKernelGGL((pgqa_wave_kernel<HD, false, true>), grid, block, 0, stream, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL(pgqa_wave_kernel<HD>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

// ---- the allocation-free entry point's scratch ----
// Partials of pgqa_attn_decode_noalloc live in the file-scope array `scratch`
// (below, outside this namespace); each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address of this GPU's copy is
// taken once per device with hipGetSymbolAddress (device current) and kept in
// `g_noalloc_ptr`; only that address is ever passed to a kernel.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_noalloc_ptr[kMaxDevices];

// This device's scratch address, looked up on its first use (nullptr, with
// the runtime's error in *err, if it cannot be had).
void *noalloc_scratch(int *err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? static_cast<int>(e) : static_cast<int>(hipErrorInvalidDevice);
    return nullptr;
  }
  void *p = g_noalloc_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    *err = static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
    return nullptr;
  }
  g_noalloc_ptr[dev].store(p, std::memory_order_release);  // the same address whichever thread stores it
  return p;
}

// One decode call.  With `scratch_of` (the allocation-free entry point) the
// partials go to this device's static scratch array instead of `part`, after
// the shapes have been checked against its size.
int decode_call(void *out, void *part, const void *q, const void *k_pool, const void *v_pool,
                const int32_t *block_table, const int32_t *page_origin, const int32_t *qpos, const int32_t *kv_last,
                int64_t rows, int64_t nh, int64_t nkv, int64_t hd, int64_t window, int64_t splits, int32_t *counters,
                const int32_t *page_map, void *stream, void *(*scratch_of)(int *)) {
  if (!out || !q || !k_pool || !v_pool || !block_table || !page_origin || !qpos || !kv_last)
    return fail(PGQA_EINVAL, "a required pointer is NULL");
  if (rows < 1 || rows > INT_MAX / 2) return fail(PGQA_EINVAL, "rows=%lld out of range", (long long)rows);
  if (nh < 1 || nkv < 1 || nh % nkv != 0 || nh > 65536)
    return fail(PGQA_EINVAL, "nh=%lld must be a positive multiple of nkv=%lld", (long long)nh, (long long)nkv);
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512)
    return fail(PGQA_EINVAL, "hd=%lld unsupported (64, 128, 256 or 512)", (long long)hd);
  if (window < 0 || window > INT_MAX) return fail(PGQA_EINVAL, "window=%lld out of range", (long long)window);
  if (splits < 1 || splits > kMaxSplits)
    return fail(PGQA_EINVAL, "splits=%lld outside 1..%d", (long long)splits, kMaxSplits);
  if (scratch_of && splits > 1) {
    // (hd + 2) * 4 >= 264 bytes per (row, head, split): the first test keeps
    // the product below from overflowing
    const bool too_big = static_cast<uint64_t>(rows) * nh * splits > kNoAllocScratchBytes / 264;
    const uint64_t need = too_big ? 0 : static_cast<uint64_t>(rows) * nh * splits * (hd + 2) * 4;
    if (too_big || need > kNoAllocScratchBytes)
      return fail(PGQA_EINVAL,
                  "partials of %llu bytes exceed the %llu-byte scratch of the allocation-free entry point "
                  "(fewer splits, or pgqa_attn_decode with a partial buffer)",
                  (unsigned long long)need, (unsigned long long)kNoAllocScratchBytes);
    int err = 0;
    part = scratch_of(&err);
    if (!part) return fail(PGQA_ELAUNCH, "scratch address of this device: %s", hipGetErrorString((hipError_t)err));
  }
  if (splits > 1 && !part) return fail(PGQA_EINVAL, "splits > 1 needs a partial buffer");
  if (part && (reinterpret_cast<uintptr_t>(part) & 3u)) return fail(PGQA_EINVAL, "partial buffer not 4-byte aligned");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15u)
    return fail(PGQA_EINVAL, "q and the pools must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(out) & 1u) return fail(PGQA_EINVAL, "out must be 2-byte aligned");

  const int64_t group = nh / nkv;
  Plan plan = make_plan(rows, group, hd, splits, nkv);
  // the per-wave kernel's workgroups each take one row (working only if it
  // starts a tile); the shared-page kernel's an rmax-aligned block of rows
  const int64_t grid_rows = plan.kind == 1 ? (rows + plan.rmax - 1) / plan.rmax : rows;
  // the documented (kernel-independent) bound: at most rows * nkv * ceil(group / 16) units
  if (counters && splits > 1 && rows * nkv * ((group + 15) / 16) > kCounterCap)
    return fail(PGQA_ECAP, "rows * nkv * ceil(group / 16) = %lld exceeds the %d counters",
                (long long)(rows * nkv * ((group + 15) / 16)), kCounterCap);
  if (rows * nh * (hd > 128 ? hd / 128 : 1) > INT_MAX) return fail(PGQA_EINVAL, "rows * nh too large");
  const int64_t blocks = grid_rows * nkv * plan.hblocks * splits;
  // every grid is checked before anything is enqueued: a launch holds at most
  // 2^32 - 1 threads in all
  const int64_t block_threads = plan.kind == 1 ? kSharedThreads : kThreads;
  if (blocks > INT_MAX || blocks * block_threads > int64_t(UINT32_MAX))
    return fail(PGQA_EINVAL, "grid of %lld workgroups too large", (long long)blocks);
  // Tiles of at most 4 columns (one row of a group of up to 4 heads, or a few
  // rows of a narrower group) at hd 64 and 128 take the vector-ALU page step
  // in launches of more than kRankMinBlocks workgroups: measured level with
  // the MFMA step at hd 128 and 4% faster at hd 64 on batched decode, but
  // 1.6 us slower on a one-workgroup call, so smaller launches keep MFMA.  At
  // hd 256 the MFMA form (one register set, two waves per SIMD) is 2-8%
  // faster, so the vector-ALU form runs there only when forced (mode 1).
  // Rows per tile then drop to 4 / group, so no tile has more columns.
  {
    const int mode = g_narrow_path.load(std::memory_order_relaxed);
    const bool fits = plan.kind == 0 && (hd == 64 || hd == 128 || (hd == 256 && mode == 1)) && group <= kNarrowCols;
    if (fits && mode != 2 && (mode == 1 || blocks > kRankMinBlocks)) {
      plan.valu = 1;
      plan.rmax = static_cast<int>(kNarrowCols / group);
    }
  }
  const int64_t combine_blocks = rows * nh * (hd / 32);
  if (splits > 1 && !counters && combine_blocks * 64 > int64_t(UINT32_MAX))
    return fail(PGQA_EINVAL, "combine grid of %lld workgroups too large", (long long)combine_blocks);

  DecodeArgs a;
  a.out = static_cast<uint16_t *>(out);
  a.part_o = static_cast<float *>(part);
  a.part_ml = part ? static_cast<float *>(part) + rows * nh * splits * hd : nullptr;
  a.q = static_cast<const uint16_t *>(q);
  a.k_pool = static_cast<const uint16_t *>(k_pool);
  a.v_pool = static_cast<const uint16_t *>(v_pool);
  a.block_table = block_table;
  a.page_origin = page_origin;
  a.qpos = qpos;
  a.kv_last = kv_last;
  a.counters = counters;
  a.page_map = page_map;
  a.rows = static_cast<int>(rows);
  a.nh = static_cast<int>(nh);
  a.nkv = static_cast<int>(nkv);
  a.group = static_cast<int>(group);
  a.window = static_cast<int>(window);
  a.splits = static_cast<int>(splits);
  a.rmax = plan.rmax;
  a.hblocks = plan.hblocks;
  a.cap = plan.cap;
  a.tile_row0 = nullptr;
  a.tile_nrows = nullptr;
  a.ntiles = 0;
  a.nsub = 0;
  // Ordering rows costs a dependent memory round trip before a workgroup can
  // start; it pays only when the launch is larger than what the GPU holds at
  // once (2-3 per-wave workgroups per CU), so that the order of dispatch
  // decides how the launch ends.
  // Rows longest first where a launch takes more than one round of
  // workgroups: the per-wave kernel's large launches, and the shared-page
  // kernel's one-row tiles beyond the 256 workgroups (one per CU) it holds.
  a.rank_rows = (plan.kind != 1 || plan.rmax == 1) && rows > 1 &&
                blocks > (plan.kind == 1 ? kSharedRankMinBlocks : kRankMinBlocks);

  // The merge of one unit reads splits * cap * hd floats of partials: from
  // kParallelMergeBytes up the unit's workgroups merge it together, each its
  // own blocks (every kernel from hd 256; the shared-page kernel and the
  // per-wave kernel's MFMA step from hd 128; at most kOwnedMergeUnits units,
  // the counter layout of that merge), below that the last one to arrive
  // merges it alone.  Both give the same bits.
  const int wait_ticks = g_merge_wait_ticks.load(std::memory_order_relaxed);
  a.spin_ticks = counters != nullptr && splits > 1 && (plan.kind != 0 || hd >= 256 || (hd == 128 && !plan.valu)) &&
                         rows * nkv * plan.hblocks <= kOwnedMergeUnits &&
                         splits * plan.cap * hd * 4 >= kParallelMergeBytes
                     ? (wait_ticks > 0 ? wait_ticks : kClaimSpinTicks)
                     : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (hd) {
    case 64: err = launch_decode<64>(a, plan, blocks, st); break;
    case 128: err = launch_decode<128>(a, plan, blocks, st); break;
    case 256: err = launch_decode<256>(a, plan, blocks, st); break;
    default: err = launch_decode<512>(a, plan, blocks, st); break;
  }
  if (err != hipSuccess) return fail(PGQA_ELAUNCH, "split kernel launch: %s", hipGetErrorString(err));
  if (splits > 1 && !counters) {
    hipLaunchKernelGGL(pgqa_combine_kernel, dim3(static_cast<unsigned>(rows * nh * (hd / 32))), dim3(64), 0, st, a,
                       static_cast<int>(hd));
    err = hipGetLastError();
    if (err != hipSuccess) return fail(PGQA_ELAUNCH, "combine kernel launch: %s", hipGetErrorString(err));
  }
  return PGQA_OK;
}

}  // namespace

extern "C" {

int32_t pgqa_choose_splits(int64_t kv_span, int64_t rows, int64_t nkv, int64_t rows_per_seq) {
  if (kv_span < 1 || rows < 1 || nkv < 1) return 1;
  if (rows_per_seq < 1 || rows_per_seq > rows) rows_per_seq = rows;
  const int64_t nseq = (rows + rows_per_seq - 1) / rows_per_seq;
  const int64_t units = nseq * nkv;
  const int64_t pages = (kv_span + kPage - 1) / kPage;
  // Two regimes, measured over split counts 1..256 on every configuration
  // and on sweeps of further lengths, head layouts and batch sizes:
  //  - long spans are bandwidth-bound.  One sequence: about one workgroup per
  //    CU on the 256 CUs (each workgroup's prologue and epilogue then come
  //    once), at least 8 pages per split.  A batch: about 4 workgroups per CU
  //    up to 256 (sequence, kv head) units, 6 above (with the longest rows
  //    dispatched first, uneven lengths still balance), at most 16 splits, at
  //    least 16 pages per split;
  //  - short spans are latency-bound: about 64 workgroups in all, at least 4
  //    pages per split.
  // The larger of the two wins.
  auto cdiv = [](int64_t x, int64_t y) { return (x + y - 1) / y; };
  const int64_t batch_wgs = units <= 256 ? 1024 : 1536;
  const int64_t s_long = nseq == 1 ? std::min(cdiv(256, units), pages / 8)
                                   : std::min(std::min(cdiv(batch_wgs, units), kBatchMaxSplits), pages / 16);
  const int64_t s_short = std::min(cdiv(64, units), pages / 4);
  int64_t s = std::max(s_long, s_short);
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return static_cast<int32_t>(s);
}

int32_t pgqa_choose_splits_heads(int64_t kv_span, int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                                 int64_t rows_per_seq) {
  const int32_t s = pgqa_choose_splits(kv_span, rows, nkv, rows_per_seq);
  if (kv_span < 1 || rows < 1 || nkv < 1 || nh < nkv || nh % nkv != 0) return s;
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512) return s;
  if (rows_per_seq < 1 || rows_per_seq > rows) rows_per_seq = rows;
  const int64_t nseq = (rows + rows_per_seq - 1) / rows_per_seq;
  if (nseq == 1 || make_plan(rows, nh / nkv, hd, s, nkv).kind != 1) return s;
  // The shared-page kernel holds one workgroup per CU.  Below 64 units one
  // round of 256 workgroups is best; from 64 units two rounds, whose rows
  // are taken longest first, balance the uneven lengths better (measured
  // over split counts 2..16 on batches of 16..128 sequences with 32 and 64
  // heads per kv head).
  const int64_t units = nseq * nkv;
  const int64_t pages = (kv_span + kPage - 1) / kPage;
  const int64_t wgs = units < 64 ? 256 : 512;
  const int64_t s_round = std::min(std::min(wgs / units, kBatchMaxSplits), pages / 16);
  const int64_t s_short = std::min((64 + units - 1) / units, pages / 4);
  return static_cast<int32_t>(std::max(std::max(s_round, s_short), int64_t(1)));
}

int32_t pgqa_tile_splits(int64_t pages, int64_t splits) {
  if (splits < 1) return 1;
  return splits_for_pages(pages, splits < kMaxSplits ? splits : kMaxSplits);
}

uint64_t pgqa_decode_part_bytes(int64_t rows, int64_t nh, int64_t splits, int64_t hd) {
  if (rows < 1 || nh < 1 || splits < 1 || hd < 1) return 0;
  return static_cast<uint64_t>(rows) * nh * splits * (hd + 2) * 4;
}

int32_t pgqa_counter_capacity(void) { return kCounterCap; }

const char *pgqa_last_error(void) { return pgqa_detail::error_text(); }

int32_t pgqa_set_merge_wait_ticks(int32_t ticks) {
  if (ticks < 0) return PGQA_EINVAL;
  return g_merge_wait_ticks.exchange(ticks, std::memory_order_relaxed);
}

int32_t pgqa_set_narrow_path(int32_t mode) {
  if (mode < 0 || mode > 2) return PGQA_EINVAL;
  return g_narrow_path.exchange(mode, std::memory_order_relaxed);
}

int pgqa_attn_decode(void *out, void *part, const void *q, const void *k_pool, const void *v_pool,
                     const int32_t *block_table, const int32_t *page_origin, const int32_t *qpos,
                     const int32_t *kv_last, int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                     int64_t window, int64_t splits, int32_t *counters, const int32_t *page_map,
                     void *stream) {
  pgqa_detail::clear_error();
  return decode_call(out, part, q, k_pool, v_pool, block_table, page_origin, qpos, kv_last, rows, nh, nkv, hd, window,
                     splits, counters, page_map, stream, nullptr);
}

int pgqa_attn_decode_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                             const int32_t *block_table, const int32_t *page_origin, const int32_t *qpos,
                             const int32_t *kv_last, int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                             int64_t window, int64_t splits, const int32_t *page_map, void *stream) {
  pgqa_detail::clear_error();
  return decode_call(out, nullptr, q, k_pool, v_pool, block_table, page_origin, qpos, kv_last, rows, nh, nkv, hd,
                     window, splits, nullptr, page_map, stream, &noalloc_scratch);
}

int32_t pgqa_prefill_rows_per_tile(int64_t hd) {
  return hd == 64 || hd == 128 || hd == 256 || hd == 512 ? kPrefillRowsPerTile : 0;
}

int64_t pgqa_make_tiles(const int32_t *page_origin, int64_t rows, int64_t rows_per_tile, int32_t *tile_row0,
                        int32_t *tile_rows, int64_t capacity) {
  pgqa_detail::clear_error();
  if (!page_origin || !tile_row0 || !tile_rows || rows < 0 || rows > INT_MAX || rows_per_tile < 1 ||
      rows_per_tile > kPrefillRowsPerTile)
    return fail(PGQA_EINVAL, "make_tiles: bad arguments");
  int64_t n = 0;
  for (int64_t r = 0; r < rows;) {
    int64_t e = r + 1;
    while (e < rows && e - r < rows_per_tile && page_origin[e] == page_origin[r]) ++e;
    if (n >= capacity) return fail(PGQA_ECAP, "make_tiles: more than %lld tiles", (long long)capacity);
    tile_row0[n] = static_cast<int32_t>(r);
    tile_rows[n] = static_cast<int32_t>(e - r);
    ++n;
    r = e;
  }
  return n;
}

int pgqa_attn_prefill(void *out, const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                      const int32_t *page_origin, const int32_t *qpos, const int32_t *kv_last,
                      const int32_t *tile_row0, const int32_t *tile_rows, int64_t ntiles, int64_t rows, int64_t nh,
                      int64_t nkv, int64_t hd, int64_t window, const int32_t *page_map, void *stream) {
  pgqa_detail::clear_error();
  if (!out || !q || !k_pool || !v_pool || !block_table || !page_origin || !qpos || !kv_last || !tile_row0 ||
      !tile_rows)
    return fail(PGQA_EINVAL, "a required pointer is NULL");
  if (rows < 1 || rows > INT_MAX / 2) return fail(PGQA_EINVAL, "rows=%lld out of range", (long long)rows);
  if (ntiles < 1 || ntiles > rows) return fail(PGQA_EINVAL, "ntiles=%lld out of range", (long long)ntiles);
  if (nh < 1 || nkv < 1 || nh % nkv != 0 || nh > 65536)
    return fail(PGQA_EINVAL, "nh=%lld must be a positive multiple of nkv=%lld", (long long)nh, (long long)nkv);
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512)
    return fail(PGQA_EINVAL, "hd=%lld unsupported (64, 128, 256 or 512)", (long long)hd);
  if (window < 0 || window > INT_MAX) return fail(PGQA_EINVAL, "window=%lld out of range", (long long)window);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15u)
    return fail(PGQA_EINVAL, "q and the pools must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(out) & 1u) return fail(PGQA_EINVAL, "out must be 2-byte aligned");

  const int64_t group = nh / nkv;
  const Plan plan = make_prefill_plan(group, hd, ntiles * nkv);
  const int64_t nsub = (kPrefillRowsPerTile + plan.rmax - 1) / plan.rmax;
  const int64_t blocks = ntiles * nsub * nkv * plan.hblocks;
  const int64_t block_threads = plan.kind == 1 ? kSharedThreads : kThreads;
  if (blocks > INT_MAX || blocks * block_threads > int64_t(UINT32_MAX))
    return fail(PGQA_EINVAL, "grid of %lld workgroups too large", (long long)blocks);

  DecodeArgs a;
  a.out = static_cast<uint16_t *>(out);
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.q = static_cast<const uint16_t *>(q);
  a.k_pool = static_cast<const uint16_t *>(k_pool);
  a.v_pool = static_cast<const uint16_t *>(v_pool);
  a.block_table = block_table;
  a.page_origin = page_origin;
  a.qpos = qpos;
  a.kv_last = kv_last;
  a.counters = nullptr;
  a.page_map = page_map;
  a.rows = static_cast<int>(rows);
  a.nh = static_cast<int>(nh);
  a.nkv = static_cast<int>(nkv);
  a.group = static_cast<int>(group);
  a.window = static_cast<int>(window);
  a.splits = 1;
  a.rmax = plan.rmax;
  a.hblocks = plan.hblocks;
  a.cap = plan.cap;
  a.rank_rows = 0;
  a.spin_ticks = 0;
  a.tile_row0 = tile_row0;
  a.tile_nrows = tile_rows;
  a.ntiles = static_cast<int>(ntiles);
  a.nsub = static_cast<int>(nsub);

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (hd) {
    case 64: err = launch_decode<64>(a, plan, blocks, st); break;
    case 128: err = launch_decode<128>(a, plan, blocks, st); break;
    case 256: err = launch_decode<256>(a, plan, blocks, st); break;
    default: err = launch_decode<512>(a, plan, blocks, st); break;
  }
  if (err != hipSuccess) return fail(PGQA_ELAUNCH, "prefill kernel launch: %s", hipGetErrorString(err));
  return PGQA_OK;
}

}  // extern "C"

// Paged grouped-query decode attention for CDNA4 (gfx950): kernels + C ABI.
//
// What is computed is fixed by the span-02 GPU kernel test page
// (respanai/span-02, engine/crates/kernels/tests/gpu.rs): its `reference`
// function (scale 1.0, kv head h / (nh / nkv), causal with an optional sliding
// window, pool [page][nkv][16][hd]) and its `attn_decode` calls (block table
// with per-row origins, split partials merged by the last workgroup through a
// counter or by a separate combine kernel, optional page map whose
// out-of-window pages may point at a NaN-filled null page).  The page shows no
// kernel code; everything below is designed for MI355X.
//
// Work decomposition
//   * A "tile" is a run of up to `rmax` consecutive rows that share a page
//     origin (rows of one sequence).  Its query heads for one kv head form up to
//     16 "columns" (row, head), so one tile reads each KV page once for all of
//     them.  Groups wider than 16 heads are cut into head blocks of 16.
//   * A workgroup (4 waves) owns one (tile, kv head, head block, split).  The
//     split is a contiguous range of the tile's visible pages; the 4 waves take
//     its pages round robin and each keeps its own online-softmax state.
//   * Per page and wave: K (16 tokens x hd) is loaded straight into MFMA
//     operand registers and S^T = K Q^T is formed with
//     v_mfma_f32_16x16x32_bf16 (tokens x columns).  The softmax weights come out
//     laid out as the A operand of v_mfma_f32_16x16x16_bf16, so P V needs no
//     shuffle of P; V is staged through LDS to read it token-major.  A column
//     of ones appended to V yields the softmax denominators from the same MFMA.
//   * The 4 wave states are merged through LDS (fixed tree), then the
//     workgroup either writes the normalised bf16 output (1 split) or an f32
//     partial (o, m, l).  Partials are merged, in split order 0..S-1, by one
//     device routine used both by the last workgroup of a merge unit (fused,
//     counter ticket) and by the separate combine kernel, so the two paths give
//     the same bits.
//   * Masked scores are replaced by -inf with a select and V rows of tokens no
//     column can see are zeroed with a select, so a NaN page or NaN slot outside
//     every window cannot leak into the result.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "pgqa.h"

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
};

// Orders this wave's LDS accesses around the point (a wave executes its LDS
// instructions in order, so only compiler reordering has to be prevented).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge of S split partials for one output element, in split order.  Used by
// both the fused last-workgroup merge and the combine kernel: the only merge
// arithmetic in the library, with explicit fused multiply-adds so both callers
// compile to the same operations.
__device__ __forceinline__ float merge_splits(const float *__restrict__ o, const float *__restrict__ ml,
                                              int splits, int hd, int d) {
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) {
    const float l = ml[2 * s + 1];
    if (l > 0.f) mx = fmaxf(mx, ml[2 * s]);
  }
  float num = 0.f, den = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float l = ml[2 * s + 1];
    if (l > 0.f) {
      const float w = fast_exp2(ml[2 * s] - mx);
      den = __builtin_fmaf(w, l, den);
      num = __builtin_fmaf(w, o[static_cast<int64_t>(s) * hd + d], num);
    }
  }
  return den > 0.f ? num / den : 0.f;
}

// Column c (0..15) of a tile -> (row offset, head within the kv group), or
// off if the tile has no such column.
struct Column {
  int row, head;
  bool on;
};
__device__ __forceinline__ Column tile_column(int c, int group, int nrows, int hb) {
  Column col;
  if (group <= 16) {
    col.row = c / group;
    col.head = c - col.row * group;
    col.on = col.row < nrows;
  } else {
    col.row = 0;
    col.head = hb * 16 + c;
    col.on = col.head < group;
  }
  return col;
}

template <int HD>
__global__ __launch_bounds__(kThreads) void pgqa_split_kernel(DecodeArgs a) {
  constexpr int KJ = HD / 32;   // QK^T MFMA steps (32 hd elements each)
  constexpr int DJ = HD / 16;   // PV MFMA output blocks (16 hd columns each)
  constexpr int VLD = HD / 32;  // 16-byte V loads per lane per page
  constexpr int VSTR = HD + 8;  // LDS row stride of a staged V page (elements)
  // Per-wave V staging; reused at the end for the cross-wave merge.
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kWaves][kPage * VSTR];
  __shared__ float xfer[kWaves][16];
  __shared__ int s_is_last;
  static_assert(2 * (16 * HD + 32) * 4 <= kWaves * kPage * VSTR * 2, "merge slots must fit the V staging area");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 15;  // MFMA row/column index of this lane
  const int lc = lane >> 4;  // MFMA k-group of this lane

  int b = blockIdx.x;
  const int split = b % a.splits;
  b /= a.splits;
  const int hb = b % a.hblocks;
  b /= a.hblocks;
  const int kh = b % a.nkv;
  const int t0 = b / a.nkv;

  // ---- tile: rows t0 .. t0+nrows-1 share the origin; t0 must lead it ----
  const int origin = a.page_origin[t0];
  if (t0 % a.rmax != 0 && a.page_origin[t0 - 1] == origin) return;
  int nrows = 1;
  while (nrows < a.rmax && t0 + nrows < a.rows && (t0 + nrows) % a.rmax != 0 &&
         a.page_origin[t0 + nrows] == origin)
    ++nrows;

  int lo_min = INT_MAX, hi_max = -1;
  for (int r = 0; r < nrows; ++r) {
    const int qp = a.qpos[t0 + r];
    const int hi = a.kv_last[t0 + r];
    const int lo = a.window > 0 ? max(0, qp + 1 - a.window) : 0;
    if (hi >= lo) {
      lo_min = min(lo_min, lo);
      hi_max = max(hi_max, hi);
    }
  }
  int pbeg = 0, pend = 0;
  if (hi_max >= 0) {
    const int p0 = lo_min / kPage;
    const int64_t npg = hi_max / kPage - p0 + 1;
    pbeg = p0 + static_cast<int>(npg * split / a.splits);
    pend = p0 + static_cast<int>(npg * (split + 1) / a.splits);
  }

  // ---- this lane's score column ----
  const Column col = tile_column(ln, a.group, nrows, hb);
  const int col_t = t0 + (col.on ? col.row : 0);
  const int col_h = kh * a.group + col.head;
  int col_lo = 0, col_hi = -1;
  if (col.on) {
    const int qp = a.qpos[col_t];
    col_hi = a.kv_last[col_t];
    col_lo = a.window > 0 ? max(0, qp + 1 - a.window) : 0;
  }

  // Q^T as the B operand: step j, lane (ln, lc) holds hd elements (4j+lc)*8..+8
  // of column ln -- the same hd chunk the K operand lanes load for step j.
  bf16x8 qop[KJ];
  {
    const uint16_t *qrow = a.q + (static_cast<int64_t>(col_t) * a.nh + col_h) * HD;
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

  float m_run = -INFINITY;  // running max (log2 units) of column ln
  f32x4 oacc[DJ];           // rows 4*lc+i of the column block, hd column 16*jj+ln
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < DJ; ++jj) oacc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  const s16x4 ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80};
  const int64_t kv_head_off = static_cast<int64_t>(kh) * kPage * HD;
  uint16_t *vt = vtile[wave];

  for (int p = pbeg + wave; p < pend; p += kWaves) {
    // Visibility of the 4 tokens this lane scores, and of each token for any column.
    const int pos0 = p * kPage + 4 * lc;
    bool vis[4];
    uint32_t tokmask = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vis[i] = col.on && pos0 + i >= col_lo && pos0 + i <= col_hi;
      const uint64_t bal = __ballot(vis[i]);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if ((bal >> (16 * g)) & 0xffffull) tokmask |= 1u << (4 * g + i);
    }
    if (tokmask == 0) continue;

    int phys = a.block_table[origin + p];
    if (a.page_map) phys = a.page_map[phys];
    const int64_t page_off = static_cast<int64_t>(phys) * a.nkv * kPage * HD + kv_head_off;
    const uint16_t *kp = a.k_pool + page_off;
    const uint16_t *vp = a.v_pool + page_off;

    bf16x8 kop[KJ];
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      kop[j] = *reinterpret_cast<const bf16x8 *>(kp + ln * HD + (4 * j + lc) * 8);
    u32x4 vreg[VLD];
#pragma unroll
    for (int j = 0; j < VLD; ++j)
      vreg[j] = *reinterpret_cast<const u32x4 *>(vp + (j * 64 + lane) * 8);

    // S^T: lane holds scores of tokens 4*lc+i for column ln.
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j], qop[j], sc, 0, 0, 0);

    float s2[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s2[i] = vis[i] ? sc[i] * kLog2e : -INFINITY;
      mx = fmaxf(mx, s2[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
    s16x4 pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = none ? 0.f : fast_exp2(s2[i] - m_new);
      pa[i] = static_cast<short>(f32_to_bf16_rne(pr));
    }
    m_run = m_new;

    // Rescale factors move from the column layout (lane ln) to the output layout
    // (lane holds rows 4*lc .. 4*lc+3).
    if (lc == 0) xfer[wave][ln] = alpha;
    wave_lds_sync();
    const f32x4 al = *reinterpret_cast<const f32x4 *>(&xfer[wave][4 * lc]);
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj) oacc[jj] *= al;
    lacc *= al;

    // Stage V; tokens no column can see are zeroed (they may hold NaN).
#pragma unroll
    for (int j = 0; j < VLD; ++j) {
      const int e = (j * 64 + lane) * 8;
      const int tok = e / HD;
      u32x4 v = vreg[j];
      if (!((tokmask >> tok) & 1u)) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(vt + tok * VSTR + (e - tok * HD)) = v;
    }
    wave_lds_sync();
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj) {
      s16x4 vb;
#pragma unroll
      for (int r = 0; r < 4; ++r) vb[r] = static_cast<short>(vt[(4 * lc + r) * VSTR + 16 * jj + ln]);
      oacc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, oacc[jj], 0, 0, 0);
    }
    lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ones, lacc, 0, 0, 0);
    wave_lds_sync();
  }

  // ---- running max into the output layout ----
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

  const int ncols = a.group <= 16 ? nrows * a.group : min(16, a.group - hb * 16);
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lc + i;
      if (r >= ncols) continue;
      const Column rc = tile_column(r, a.group, nrows, hb);
      const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
      if (a.splits == 1) {
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
        for (int jj = 0; jj < DJ; ++jj) po[16 * jj + ln] = oacc[jj][i];
        if (ln == 0) {
          a.part_ml[2 * ps] = mo[i];
          a.part_ml[2 * ps + 1] = lacc[i];
        }
      }
    }
  }
  if (a.splits == 1 || a.counters == nullptr) return;

  // ---- fused merge: the last workgroup of this unit merges every split ----
  __threadfence();
  __syncthreads();
  const int unit = (t0 * a.nkv + kh) * a.hblocks + hb;
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(&a.counters[unit], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_is_last = prev == a.splits - 1;
  }
  __syncthreads();
  if (!s_is_last) return;
  __threadfence();
  for (int idx = threadIdx.x; idx < ncols * HD; idx += kThreads) {
    const int c = idx / HD;
    const int d = idx - c * HD;
    const Column rc = tile_column(c, a.group, nrows, hb);
    const int64_t th = static_cast<int64_t>(t0 + rc.row) * a.nh + kh * a.group + rc.head;
    const float v = merge_splits(a.part_o + th * a.splits * HD, a.part_ml + th * a.splits * 2, a.splits, HD, d);
    a.out[th * HD + d] = f32_to_bf16_rne(v);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&a.counters[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Separate merge: one workgroup per (row, query head).
__global__ __launch_bounds__(256) void pgqa_combine_kernel(DecodeArgs a, int hd) {
  const int64_t th = blockIdx.x;
  const float *po = a.part_o + th * a.splits * hd;
  const float *pml = a.part_ml + th * a.splits * 2;
  for (int d = threadIdx.x; d < hd; d += blockDim.x)
    a.out[th * hd + d] = f32_to_bf16_rne(merge_splits(po, pml, a.splits, hd, d));
}

thread_local char g_error[512] = "";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

template <int HD>
hipError_t launch_decode(const DecodeArgs &a, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL(pgqa_split_kernel<HD>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int32_t pgqa_choose_splits(int64_t kv_span, int64_t rows, int64_t nkv, int64_t rows_per_seq) {
  if (kv_span < 1 || rows < 1 || nkv < 1) return 1;
  if (rows_per_seq < 1 || rows_per_seq > rows) rows_per_seq = rows;
  const int64_t nseq = (rows + rows_per_seq - 1) / rows_per_seq;
  const int64_t units = nseq * nkv;
  const int64_t pages = (kv_span + kPage - 1) / kPage;
  // Aim at two 4-wave workgroups per CU on the 256 CUs, with at least 8 pages
  // (2 per wave) in every split.
  const int64_t target = 512;
  int64_t s = (target + units - 1) / units;
  int64_t smax = pages / 8;
  if (smax < 1) smax = 1;
  if (smax > kMaxSplits) smax = kMaxSplits;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return static_cast<int32_t>(s);
}

uint64_t pgqa_decode_part_bytes(int64_t rows, int64_t nh, int64_t splits, int64_t hd) {
  if (rows < 1 || nh < 1 || splits < 1 || hd < 1) return 0;
  return static_cast<uint64_t>(rows) * nh * splits * (hd + 2) * 4;
}

int32_t pgqa_counter_capacity(void) { return kCounterCap; }

const char *pgqa_last_error(void) { return g_error; }

int pgqa_attn_decode(void *out, void *part, const void *q, const void *k_pool, const void *v_pool,
                     const int32_t *block_table, const int32_t *page_origin, const int32_t *qpos,
                     const int32_t *kv_last, int64_t rows, int64_t nh, int64_t nkv, int64_t hd,
                     int64_t window, int64_t splits, int32_t *counters, const int32_t *page_map,
                     void *stream) {
  g_error[0] = '\0';
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
  if (splits > 1 && !part) return fail(PGQA_EINVAL, "splits > 1 needs a partial buffer");
  if (part && (reinterpret_cast<uintptr_t>(part) & 3u)) return fail(PGQA_EINVAL, "partial buffer not 4-byte aligned");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15u)
    return fail(PGQA_EINVAL, "q and the pools must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(out) & 1u) return fail(PGQA_EINVAL, "out must be 2-byte aligned");

  const int64_t group = nh / nkv;
  const int64_t hblocks = group <= 16 ? 1 : (group + 15) / 16;
  const int64_t rmax = group <= 16 ? 16 / group : 1;
  const int64_t units = rows * nkv * hblocks;
  if (counters && splits > 1 && units > kCounterCap)
    return fail(PGQA_ECAP, "%lld merge units exceed the %d counters", (long long)units, kCounterCap);
  if (rows * nh > INT_MAX) return fail(PGQA_EINVAL, "rows * nh too large");
  const int64_t blocks = units * splits;
  if (blocks > INT_MAX) return fail(PGQA_EINVAL, "grid of %lld workgroups too large", (long long)blocks);

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
  a.rmax = static_cast<int>(rmax);
  a.hblocks = static_cast<int>(hblocks);

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (hd) {
    case 64: err = launch_decode<64>(a, blocks, st); break;
    case 128: err = launch_decode<128>(a, blocks, st); break;
    case 256: err = launch_decode<256>(a, blocks, st); break;
    default: err = launch_decode<512>(a, blocks, st); break;
  }
  if (err != hipSuccess) return fail(PGQA_ELAUNCH, "split kernel launch: %s", hipGetErrorString(err));
  if (splits > 1 && !counters) {
    hipLaunchKernelGGL(pgqa_combine_kernel, dim3(static_cast<unsigned>(rows * nh)), dim3(256), 0, st, a,
                       static_cast<int>(hd));
    err = hipGetLastError();
    if (err != hipSuccess) return fail(PGQA_ELAUNCH, "combine kernel launch: %s", hipGetErrorString(err));
  }
  return PGQA_OK;
}

}  // extern "C"

// QK-norm + RoPE prep for paged attention on CDNA4 (gfx950): kernel + C ABI.
//
// The step before decode that the pegainfer pull request page (#1002, the
// HD256/HD512 QK-RoPE gates) describes: per token, an RMSNorm of every query
// and key head with a norm weight, a rotary embedding of the first
// rotary_dim elements taken as a low and a high half (the rest pass
// through), a weightless RMSNorm of V (V taken from the K input in the
// "K = V" form), and the key and value heads landing in the paged pool
// [page][nkv][16][hd] at the token's position, found through a per-token
// page origin into the block table (and the page map, when given).  The page
// prints no formulas; the readings are stated in pgqa.h.
//
// Work decomposition.  A token's heads, in the order [nh query | nkv key |
// nkv value], form one row of (nh + 2 nkv) * hd elements, cut into chunks of
// 512: hd / 8 lanes per head, 8 consecutive elements (one 16-byte load and
// one 16-byte store) per lane, 512 / hd whole heads per chunk.  One wave
// takes up to 4 chunks of one token and issues all of its loads -- the data,
// the per-token chain position -> table entry -> page (-> map), the norm
// weights and the lane's rotary-table row, which depend on the lane's
// position in a head only -- before the first result is needed, so a wave
// pays the dependent chain's latency once for 4 KB in and 4 KB out (small
// launches: one chunk per wave, for more waves in flight).  The
// memory traffic is the inputs read once and the outputs written once, fully
// coalesced.
//   * Sum of squares: each lane's 8 squares in element order, then a
//     butterfly over the head's lanes (xor 1, 2, 4, ...): every lane of the
//     head ends with the same bits.
//   * Rotation: element i < rotary_dim / 2 pairs with i + rotary_dim / 2;
//     since rotary_dim is a multiple of 16 the partner of a lane's 8 elements
//     is the 8 elements of the lane rotary_dim / 16 away, fetched with a
//     cross-lane permute.
//   * Rounding: f32 arithmetic, bf16 nearest-even on the store
//     (v_cvt_pk_bf16_f32).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "errors.h"
#include "pgqa.h"

namespace {

using pgqa_detail::fail;

constexpr int kPrepWaves = 4;
constexpr int kPrepThreads = 64 * kPrepWaves;
constexpr int kRowChunk = 512;   // bf16 elements of a token's row per chunk
constexpr int kGroupChunks = 4;  // most chunks per wave
// Launches of at most this many chunks give every chunk its own wave: they
// fill only part of the device, and more, shorter waves finish sooner.
constexpr int64_t kSmallLaunchChunks = 8192;

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

struct PrepArgs {
  uint16_t *q_out;
  uint16_t *k_pool;
  uint16_t *v_pool;
  const uint16_t *q_in;
  const uint16_t *k_in;
  const uint16_t *v_in;  // the K input again in the K = V form
  const uint16_t *q_w;   // nullptr: weight 1
  const uint16_t *k_w;
  const float *rope_cos;  // [position][rotary_dim / 2]
  const float *rope_sin;
  const int32_t *pos;
  const int32_t *block_table;
  const int32_t *page_origin;
  const int32_t *page_map;
  int64_t waves;  // tokens * groups
  int chunks;     // 512-element chunks per token
  int groups;     // waves per token
  int per_group;  // chunks per wave: ceil(chunks / groups) <= kGroupChunks
  int nh, nkv, rd;
  float eps;
};

__device__ __forceinline__ void widen8(const u32x4 r, float *x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(r[j] << 16);
    x[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
  }
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int HD>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(4))) void pgqa_prep_kernel(PrepArgs a) {
  constexpr int LPH = HD / 8;          // lanes per head
  constexpr int HPW = kRowChunk / HD;  // heads per chunk
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kPrepWaves + (threadIdx.x >> 6);
  if (gw >= a.waves) return;  // whole waves
  const int t = static_cast<int>(gw / a.groups);
  const int c0 = static_cast<int>(gw - static_cast<int64_t>(t) * a.groups) * a.per_group;
  const int c1 = min(c0 + a.per_group, a.chunks);  // this wave's chunks: c0 .. c1 - 1
  const int d0 = (lane % LPH) * 8;  // the same elements of every head this lane takes
  const int nall = a.nh + 2 * a.nkv;

  // Every load of the wave is issued before any result is needed: the
  // per-token chain (position -> table entry -> page -> map), the norm
  // weights and the rotary-table row (one per lane: they depend on d0 only),
  // and the group's data.
  const int p = a.pos[t];
  int ph = a.block_table[a.page_origin[t] + (p >> 4)];
  if (a.page_map) ph = a.page_map[ph];
  u32x4 qw = {0u, 0u, 0u, 0u}, kw = {0u, 0u, 0u, 0u};
  if (a.q_w) qw = *reinterpret_cast<const u32x4 *>(a.q_w + d0);
  if (a.k_w) kw = *reinterpret_cast<const u32x4 *>(a.k_w + d0);
  const int half = a.rd >> 1;
  const bool in_rot = d0 < a.rd;  // this lane's elements are rotated (query and key heads)
  const bool lo = d0 < half;
  f32x4 c0v = {1.f, 1.f, 1.f, 1.f}, c1v = c0v, s0v = {0.f, 0.f, 0.f, 0.f}, s1v = s0v;
  if (in_rot) {
    const int64_t ti = static_cast<int64_t>(p) * half + (lo ? d0 : d0 - half);
    c0v = *reinterpret_cast<const f32x4 *>(a.rope_cos + ti);
    c1v = *reinterpret_cast<const f32x4 *>(a.rope_cos + ti + 4);
    s0v = *reinterpret_cast<const f32x4 *>(a.rope_sin + ti);
    s1v = *reinterpret_cast<const f32x4 *>(a.rope_sin + ti + 4);
  }
  u32x4 raw[kGroupChunks];
#pragma unroll
  for (int g = 0; g < kGroupChunks; ++g) {
    raw[g] = u32x4{0u, 0u, 0u, 0u};
    const int head = (c0 + g) * HPW + lane / LPH;
    if (c0 + g < c1 && head < nall) {
      const uint16_t *src = head < a.nh ? a.q_in + (static_cast<int64_t>(t) * a.nh + head) * HD
                                        : (head < a.nh + a.nkv ? a.k_in + (static_cast<int64_t>(t) * a.nkv + head - a.nh) * HD
                                                               : a.v_in + (static_cast<int64_t>(t) * a.nkv + head - a.nh - a.nkv) * HD);
      raw[g] = *reinterpret_cast<const u32x4 *>(src + d0);
    }
  }

  float qwf[8], kwf[8];
  widen8(qw, qwf);
  widen8(kw, kwf);
  const float c[8] = {c0v[0], c0v[1], c0v[2], c0v[3], c1v[0], c1v[1], c1v[2], c1v[3]};
  const float sn[8] = {s0v[0], s0v[1], s0v[2], s0v[3], s1v[0], s1v[1], s1v[2], s1v[3]};
  const int partner = in_rot ? (lo ? lane + (half >> 3) : lane - (half >> 3)) : lane;
  const float sgn = lo ? -1.f : 1.f;  // low half: a c - b s; high half: b c + a s
  const int64_t kv_row = ((static_cast<int64_t>(ph) * a.nkv) * 16 + (p & 15)) * HD + d0;  // kv head 0

#pragma unroll
  for (int g = 0; g < kGroupChunks; ++g) {
    if (c0 + g >= c1) break;  // wave-uniform
    const int head = (c0 + g) * HPW + lane / LPH;
    // section: 0 query, 1 key, 2 value, 3 past the row's end (last chunk only)
    const int sec = head < a.nh ? 0 : head < a.nh + a.nkv ? 1 : head < nall ? 2 : 3;
    float x[8];
    widen8(raw[g], x);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(x[j], x[j], ss);
#pragma unroll
    for (int off = 1; off < LPH; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / HD) + a.eps);
    const bool weighted = sec == 0 ? a.q_w != nullptr : sec == 1 && a.k_w != nullptr;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = sec == 0 ? qwf[j] : kwf[j];
      y[j] = weighted ? x[j] * inv * w : x[j] * inv;
    }
    // rotation of the query and key heads' first rd elements; the partner
    // lane belongs to the same head, so every lane shuffles
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = __shfl(y[j], partner);
    if (sec < 2 && in_rot) {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = __builtin_fmaf(sgn * pv[j], sn[j], y[j] * c[j]);
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16(y[2 * j], y[2 * j + 1]);
    if (sec == 0)
      *reinterpret_cast<u32x4 *>(a.q_out + (static_cast<int64_t>(t) * a.nh + head) * HD + d0) = o;
    else if (sec == 1)
      *reinterpret_cast<u32x4 *>(a.k_pool + kv_row + static_cast<int64_t>(head - a.nh) * 16 * HD) = o;
    else if (sec == 2)
      *reinterpret_cast<u32x4 *>(a.v_pool + kv_row + static_cast<int64_t>(head - a.nh - a.nkv) * 16 * HD) = o;
  }
}

template <int HD>
hipError_t launch_prep(const PrepArgs &a, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL(pgqa_prep_kernel<HD>, dim3(static_cast<unsigned>(blocks)), dim3(kPrepThreads), 0, stream, a);
  return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int pgqa_qk_rope_prep(void *q_out, void *k_pool, void *v_pool, const void *q_in, const void *k_in, const void *v_in,
                      const void *q_weight, const void *k_weight, const float *rope_cos, const float *rope_sin,
                      const int32_t *pos, const int32_t *block_table, const int32_t *page_origin,
                      const int32_t *page_map, int64_t tokens, int64_t nh, int64_t nkv, int64_t hd,
                      int64_t rotary_dim, float eps, void *stream) {
  pgqa_detail::clear_error();
  if (tokens < 0 || tokens > INT_MAX) return fail(PGQA_EINVAL, "tokens=%lld out of range", (long long)tokens);
  if (nh < 1 || nkv < 1 || nh > 65536 || nkv > 65536)
    return fail(PGQA_EINVAL, "nh=%lld / nkv=%lld out of range", (long long)nh, (long long)nkv);
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512)
    return fail(PGQA_EINVAL, "hd=%lld unsupported (64, 128, 256 or 512)", (long long)hd);
  if (rotary_dim < 0 || rotary_dim > hd || rotary_dim % 16 != 0)
    return fail(PGQA_EINVAL, "rotary_dim=%lld must be a multiple of 16 in 0..hd", (long long)rotary_dim);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(PGQA_EINVAL, "eps must be finite and >= 0");
  if (!q_out || !k_pool || !v_pool || !q_in || !k_in || !pos || !block_table || !page_origin)
    return fail(PGQA_EINVAL, "a required pointer is NULL");
  if (rotary_dim > 0 && (!rope_cos || !rope_sin))
    return fail(PGQA_EINVAL, "rotary_dim > 0 needs both rotary tables");
  const void *a16[] = {q_out, k_pool, v_pool, q_in, k_in, v_in, q_weight, k_weight, rope_cos, rope_sin};
  for (const void *ptr : a16)
    if (ptr && !aligned16(ptr)) return fail(PGQA_EINVAL, "bf16 buffers and rotary tables must be 16-byte aligned");
  if (tokens == 0) return PGQA_OK;

  const int64_t row = (nh + 2 * nkv) * hd;
  const int64_t chunks = (row + kRowChunk - 1) / kRowChunk;
  const int64_t groups = tokens * chunks <= kSmallLaunchChunks ? chunks : (chunks + kGroupChunks - 1) / kGroupChunks;
  const int64_t waves = tokens * groups;
  const int64_t blocks = (waves + kPrepWaves - 1) / kPrepWaves;
  if (blocks * kPrepThreads > static_cast<int64_t>(UINT32_MAX))
    return fail(PGQA_EINVAL, "tokens * (nh + 2 nkv) * hd = %lld elements: grid too large", (long long)(tokens * row));

  PrepArgs a;
  a.q_out = static_cast<uint16_t *>(q_out);
  a.k_pool = static_cast<uint16_t *>(k_pool);
  a.v_pool = static_cast<uint16_t *>(v_pool);
  a.q_in = static_cast<const uint16_t *>(q_in);
  a.k_in = static_cast<const uint16_t *>(k_in);
  a.v_in = static_cast<const uint16_t *>(v_in ? v_in : k_in);
  a.q_w = static_cast<const uint16_t *>(q_weight);
  a.k_w = static_cast<const uint16_t *>(k_weight);
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.pos = pos;
  a.block_table = block_table;
  a.page_origin = page_origin;
  a.page_map = page_map;
  a.waves = waves;
  a.chunks = static_cast<int>(chunks);
  a.groups = static_cast<int>(groups);
  a.per_group = static_cast<int>((chunks + groups - 1) / groups);
  a.nh = static_cast<int>(nh);
  a.nkv = static_cast<int>(nkv);
  a.rd = static_cast<int>(rotary_dim);
  a.eps = eps;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (hd) {
    case 64: err = launch_prep<64>(a, blocks, st); break;
    case 128: err = launch_prep<128>(a, blocks, st); break;
    case 256: err = launch_prep<256>(a, blocks, st); break;
    default: err = launch_prep<512>(a, blocks, st); break;
  }
  if (err != hipSuccess) return fail(PGQA_ELAUNCH, "prep kernel launch: %s", hipGetErrorString(err));
  return PGQA_OK;
}

}  // extern "C"

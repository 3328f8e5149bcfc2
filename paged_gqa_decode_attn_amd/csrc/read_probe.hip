// Streaming-read probe for the benchmark: how fast this GPU reads HBM with
// the load form the decode kernels use (16-byte nontemporal vector loads into
// registers), for two access patterns:
//   * contiguous: workgroup b reads bytes [b * chunk, (b + 1) * chunk) of the
//     buffer, every lane keeping UNROLL 16-byte loads in flight;
//   * scattered 4 KB blocks: the buffer is read as 4 KB blocks in a
//     permuted order (block j -> (j * 2654435761 + 12345) mod nblocks, a
//     bijection for a power-of-two count), the way a batched decode reads
//     randomly placed K/V pages; each workgroup takes a run of consecutive
//     slots of that order;
//   * paired 4 KB blocks: the two halves of the buffer stand for a K pool and
//     a V pool; consecutive 4 KB slots read block j of the first half, then
//     block j of the second half, j in the permuted order above -- a page's K
//     then its V, as the per-wave decode kernel requests them.
// Every byte is read exactly once per launch.  The loaded words are folded
// with XOR and each workgroup writes one word to `sink`, so no load can be
// dropped.  Not part of the attention path: a measuring instrument only,
// built into its own library (libpgqa_probe.so).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <int UNROLL, int SCATTER>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *buf, uint64_t n16, uint64_t per_block,
                                                         uint32_t nblocks4k, unsigned *sink) {
  const uint64_t b = blockIdx.x;
  const uint64_t begin = b * per_block;
  uint64_t end = begin + per_block;
  if (end > n16) end = n16;
  unsigned acc = 0;
  // one step: every lane issues UNROLL loads of 16 bytes, 256 * 16 * UNROLL
  // bytes per workgroup, then folds them
  constexpr uint64_t kStep = 256ull * UNROLL;
  for (uint64_t base = begin; base < end; base += kStep) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      uint64_t i = base + static_cast<uint64_t>(u) * 256 + threadIdx.x;
      if (i >= end) i = begin;  // past the end: read the first word again (cached)
      if constexpr (SCATTER == 1) {
        // 16-byte word i of the slot order -> the word of the permuted 4 KB block
        const uint64_t slot = i >> 8, word = i & 255;
        const uint64_t blk = (slot * 2654435761ull + 12345ull) & (nblocks4k - 1);
        i = (blk << 8) | word;
      } else if constexpr (SCATTER == 2) {
        // slot 2 j + h -> block perm(j) of half h (nblocks4k / 2 blocks each)
        const uint64_t slot = i >> 8, word = i & 255;
        const uint64_t half = nblocks4k >> 1;
        const uint64_t blk = ((slot >> 1) * 2654435761ull + 12345ull) & (half - 1);
        i = (((slot & 1) * half + blk) << 8) | word;
      }
      v[u] = __builtin_nontemporal_load(buf + i);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // fold the workgroup's lanes into one word
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ unsigned red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[b] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

template <int UNROLL>
hipError_t launch(const void *buf, uint64_t bytes, int64_t blocks, int scatter, unsigned *sink, hipStream_t st) {
  const uint64_t n16 = bytes / 16;
  const uint64_t per_block = (n16 + blocks - 1) / blocks;
  const uint32_t nblocks4k = static_cast<uint32_t>(bytes / 4096);
  const dim3 grid(static_cast<unsigned>(blocks)), blk(256);
  if (scatter == 2)
    hipLaunchKernelGGL((read_probe_kernel<UNROLL, 2>), grid, blk, 0, st, static_cast<const u32x4 *>(buf), n16,
                       per_block, nblocks4k, sink);
  else if (scatter)
    hipLaunchKernelGGL((read_probe_kernel<UNROLL, 1>), grid, blk, 0, st, static_cast<const u32x4 *>(buf), n16,
                       per_block, nblocks4k, sink);
  else
    hipLaunchKernelGGL((read_probe_kernel<UNROLL, 0>), grid, blk, 0, st, static_cast<const u32x4 *>(buf), n16,
                       per_block, nblocks4k, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Reads `bytes` of the device buffer `buf` once (see above).
//   bytes     a multiple of 4096; with scatter, bytes / 4096 a power of two
//   blocks    workgroups of 256 threads, 1 .. 2^20; with scatter, each
//             workgroup's share must be whole 4 KB blocks
//   unroll    16-byte loads in flight per lane: 1, 2, 4, 8 or 16
//   scatter   0: contiguous shares; 1: permuted 4 KB blocks
//   sink      device array of `blocks` uint32 (written)
//   stream    hipStream_t
// Returns 0, -1 for bad arguments (nothing enqueued) or -3 if the launch failed.
int pgqa_probe_read(const void *buf, uint64_t bytes, int64_t blocks, int32_t unroll, int32_t scatter,
                    unsigned *sink, void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 4096 != 0 || blocks < 1 || blocks > (1 << 20)) return -1;
  if (reinterpret_cast<uintptr_t>(buf) & 15u) return -1;
  if (scatter < 0 || scatter > 2) return -1;
  if (scatter) {
    const uint64_t nb = bytes / 4096;
    if (nb < 2 || (nb & (nb - 1)) != 0 || nb % static_cast<uint64_t>(blocks) != 0) return -1;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (unroll) {
    case 1: e = launch<1>(buf, bytes, blocks, scatter, sink, st); break;
    case 2: e = launch<2>(buf, bytes, blocks, scatter, sink, st); break;
    case 4: e = launch<4>(buf, bytes, blocks, scatter, sink, st); break;
    case 8: e = launch<8>(buf, bytes, blocks, scatter, sink, st); break;
    case 16: e = launch<16>(buf, bytes, blocks, scatter, sink, st); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -3;
}

}  // extern "C"

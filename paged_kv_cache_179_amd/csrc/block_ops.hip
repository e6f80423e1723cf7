// Whole-block copies for the block pool (gfx950).
//
// Two pool operations the serving engines on the pages build on the block
// cache:
// * copy-on-write of a shared block: prefix sharing makes several block
//   tables name one physical block (wLLM case study, ADR-001 on the KV-cache
//   layout), so a sequence that is about to write into a shared block first
//   gets a private copy of it (mini-vLLM README, "Limitations": block
//   reference counts are kept for prefix caching);
// * swapping blocks out to host memory and back, which lets a preempted
//   sequence resume where it stopped (wLLM PyPI page, "Features -- Core
//   engine": CPU-swap preemption).
//
// Both are the same data movement: for each (src, dst) pair of a mapping,
// copy one block of `block_bytes` from the source pool to the destination
// pool, for one or two pools (K and V) at once.  A pool may be device memory
// or host memory the device can address (pinned).  One launch covers every
// pair: workgroup w copies one 4 KiB chunk of one pair's block, 16 bytes a
// lane, with non-temporal loads and stores (the copied blocks are not read
// again soon).  Many small workgroups with streaming accesses moved 128 KiB
// blocks at 72% of the HBM peak (read plus write), where 16 KiB chunks with
// cached accesses reached 50%.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kChunk = kThreads * 16;  // bytes per workgroup

__global__ __launch_bounds__(kThreads) void block_copy_kernel(BlockCopyArgs a, int64_t chunks,
                                                              int64_t total) {
  for (int64_t w = blockIdx.x; w < total; w += gridDim.x) {
    const int64_t chunk = w % chunks;
    const int64_t r = w / chunks;
    const int64_t pair = r % a.num_pairs;
    const int pool = static_cast<int>(r / a.num_pairs);
    const int64_t src_blk = a.block_mapping[2 * pair];
    const int64_t dst_blk = a.block_mapping[2 * pair + 1];
    if (src_blk < 0 || src_blk >= a.src_blocks || dst_blk < 0 || dst_blk >= a.dst_blocks) continue;
    const char* src = static_cast<const char*>(a.src[pool]) + src_blk * a.block_bytes;
    char* dst = static_cast<char*>(a.dst[pool]) + dst_blk * a.block_bytes;
    const int64_t off = chunk * kChunk + threadIdx.x * 16;
    if (off < a.block_bytes)
      __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off)),
                                  reinterpret_cast<u32x4*>(dst + off));
  }
}

// Streaming-read probe: workgroup w reads bytes [w kProbeSpan, (w + 1)
// kProbeSpan) of the source with non-temporal 16-byte loads, eight per lane in
// flight, and stores the XOR of all its 32-bit words to sink[w] (so the loads
// cannot be dropped, and a test can check what was read).
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  constexpr int64_t kSpan16 = kProbeSpan / 16;
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * kSpan16;
  const int64_t end = begin + kSpan16 < n16 ? begin + kSpan16 : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i0 = begin + threadIdx.x; i0 < end; i0 += kThreads * kProbeUnroll) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t i = i0 + u * kThreads;
      v[u] = i < end ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x ^= __shfl_xor(x, off, kWave);
  __shared__ uint32_t s_x[kThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) s_x[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) y ^= s_x[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t grid = (bytes + kProbeSpan - 1) / kProbeSpan;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_block_copy(const BlockCopyArgs& a, hipStream_t stream) {
  if (a.num_pairs <= 0 || a.num_pools <= 0 || a.block_bytes <= 0) return hipSuccess;
  const int64_t chunks = (a.block_bytes + kChunk - 1) / kChunk;
  const int64_t total = chunks * a.num_pairs * a.num_pools;
  const int64_t grid = total < (int64_t(1) << 20) ? total : (int64_t(1) << 20);  // grid-stride beyond
  hipLaunchKernelGGL(block_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                     a, chunks, total);
  return hipGetLastError();
}

}  // namespace pa

// Slot-mapped K/V cache write for gfx950.
//
// The new tokens' keys and values are scattered into their pool slots in one
// launch for all sequences, not one sequence at a time (mini-vLLM README,
// "End-to-end throughput vs baselines").  Each
// lane moves 16 bytes; the 16-byte chunks of one (token, KV head) row are
// consecutive lanes, so both the read of key/value and the write into the
// [block][head][offset][dim] pool are contiguous per row.  Pure bit copy.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ key_cache,
    u32x4* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int64_t total,
    int32_t chunks_per_row, int32_t num_kv_heads, int32_t log2_bs, int64_t num_slots) {
  copy_rows_to_cache(key, value, key_cache, value_cache, slot_mapping, total, chunks_per_row,
                     num_kv_heads, log2_bs, num_slots,
                     static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                     static_cast<int64_t>(gridDim.x) * blockDim.x);
}

// E4M3 byte of y (round to nearest, ties to even), saturating to +-448;
// NaN gives 0x7F.  The hardware conversion rounds to nearest even on the
// E4M3 grid but turns values past the range into NaN, hence the clamp.
__device__ inline unsigned e4m3_byte(float y) {
  if (y != y) return 0x7Fu;
  const float c = fminf(fmaxf(y, -448.f), 448.f);
  return static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xFFu;
}

// Slot-mapped write into E4M3 caches: each work item quantises 16 elements of
// one (token, KV head) row, key[...] / k_scale and value[...] / v_scale (the
// division correctly rounded in fp32), and stores their 16 bytes.
template <typename E>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const char* __restrict__ key, const char* __restrict__ value, u32x4* __restrict__ key_cache,
    u32x4* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int64_t total,
    int32_t chunks_per_row, int32_t num_kv_heads, int32_t log2_bs, int64_t num_slots, float k_scale,
    float v_scale) {
  constexpr int G = E::kPerGroup;  // elements per 16-byte source group
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t per_token = static_cast<int64_t>(chunks_per_row) * num_kv_heads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    const int64_t n = i / per_token;
    const int64_t rem = i - n * per_token;  // = head * chunks_per_row + chunk
    const int64_t slot = slot_mapping[n];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot >> log2_bs;
    const int64_t off = slot & ((int64_t(1) << log2_bs) - 1);
    const int64_t head = rem / chunks_per_row;
    const int64_t chunk = rem - head * chunks_per_row;
    const int64_t dst = (((blk * num_kv_heads + head) << log2_bs) + off) * chunks_per_row + chunk;
    const int64_t src = i * 16 * E::kBytes;  // 16 source elements per item
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const char* in = (kv == 0 ? key : value) + src;
      const float sc = kv == 0 ? k_scale : v_scale;
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * w + j;
          const u32x4 g = *reinterpret_cast<const u32x4*>(in + (e / G) * 16);
          word |= e4m3_byte(E::elem(g, e % G) / sc) << (8 * j);
        }
        out[w] = word;
      }
      (kv == 0 ? key_cache : value_cache)[dst] = out;
    }
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.kv_fp8) {
    const int32_t chunks_per_row = a.head_dim / 16;  // 16 E4M3 bytes per item
    const int64_t total = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * chunks_per_row;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    const int64_t num_slots = static_cast<int64_t>(a.num_blocks) << a.log2_block_size;
    auto go = [&](auto tag) {
      using E = decltype(tag);
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<E>, dim3(static_cast<unsigned>(blocks)),
                         dim3(threads), 0, stream, static_cast<const char*>(a.key),
                         static_cast<const char*>(a.value), static_cast<u32x4*>(a.key_cache),
                         static_cast<u32x4*>(a.value_cache), a.slot_mapping, total, chunks_per_row,
                         a.num_kv_heads, a.log2_block_size, num_slots, a.k_scale, a.v_scale);
    };
    if (a.src_dtype == PA_DTYPE_F32) go(F32{});
    else if (a.src_dtype == PA_DTYPE_F16) go(F16{});
    else go(BF16{});
    return hipGetLastError();
  }
  const int32_t chunks_per_row = a.head_dim * a.elem_bytes / 16;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * chunks_per_row;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  const int64_t num_slots = static_cast<int64_t>(a.num_blocks) << a.log2_block_size;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads),
                     0, stream, static_cast<const u32x4*>(a.key),
                     static_cast<const u32x4*>(a.value), static_cast<u32x4*>(a.key_cache),
                     static_cast<u32x4*>(a.value_cache), a.slot_mapping, total, chunks_per_row,
                     a.num_kv_heads, a.log2_block_size, num_slots);
  return hipGetLastError();
}

}  // namespace pa

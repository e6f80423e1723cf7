// C-ABI entry points: argument validation, workspace sizing and dispatch to the
// gfx950 kernels.  Validation happens entirely on the host and before any HIP
// call, so every error path returns a status with nothing enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "paged_attention.h"
#include "pa_internal.h"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

bool supported_dtype(int d) { return d == PA_DTYPE_F32 || d == PA_DTYPE_F16 || d == PA_DTYPE_BF16; }
bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
bool supported_block_size(int b) { return is_pow2(b) && b <= 256; }
int elem_bytes(int d) { return d == PA_DTYPE_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int32_t clamp_i32(int64_t v) {
  return static_cast<int32_t>(std::min<int64_t>(std::max<int64_t>(v, 0), INT32_MAX));
}

// Decode geometry shared by the sizing function and both decode halves.
struct DecodeGeom {
  int32_t ctx_limit;
  int32_t part_tokens;
  int32_t num_parts;
};

DecodeGeom decode_geom(int64_t ctx_limit, int32_t partition_size) {
  DecodeGeom g{};
  g.ctx_limit = clamp_i32(ctx_limit);
  g.part_tokens = partition_size > 0 ? partition_size : std::max<int32_t>(g.ctx_limit, 1);
  g.num_parts = std::max<int32_t>(
      1, static_cast<int32_t>((static_cast<int64_t>(g.ctx_limit) + g.part_tokens - 1) / g.part_tokens));
  return g;
}

pa_status check_decode_shapes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int32_t num_blocks, int32_t max_context_len, int32_t partition_size,
                              int dtype) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      max_context_len < 0)
    return PA_ERR_BAD_SHAPE;
  if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (max_blocks_per_seq <= 0 || num_blocks <= 0)) return PA_ERR_BAD_SHAPE;
  if (partition_size < 0 || (partition_size > 0 && (partition_size % 64 != 0 ||
                                                     partition_size % block_size != 0)))
    return PA_ERR_BAD_SHAPE;
  return PA_OK;
}

// An E4M3 cache scale: positive and finite.
bool valid_scale(float s) { return s > 0.f && s <= 3.0e38f; }

// Logit soft-cap (>= 0, finite; 0 = none) and sliding window (>= 0; 0 = none).
bool valid_variant(float logit_softcap, int32_t sliding_window) {
  return logit_softcap >= 0.f && logit_softcap <= 3.0e38f && sliding_window >= 0;
}

pa_status check_workspace(size_t needed, const void* workspace, size_t workspace_bytes) {
  if (needed == 0) return PA_OK;
  if (workspace == nullptr) return PA_ERR_NULL_POINTER;
  if (workspace_bytes < needed) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(workspace, 16)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

pa_status decode_args(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t num_blocks, int32_t max_context_len, float scale,
                      float logit_softcap, int32_t sliding_window, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, pa_dtype dtype,
                      pa::DecodeArgs* a) {
  pa_status st = check_decode_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_blocks_per_seq, num_blocks, max_context_len,
                                     partition_size, dtype);
  if (st != PA_OK) return st;
  if (!valid_variant(logit_softcap, sliding_window)) return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return st;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_POINTER;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_UNSUPPORTED;
  const DecodeGeom g = decode_geom(
      std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * block_size),
      partition_size);
  const pa::DecodeWorkspace w =
      pa::decode_workspace_layout(num_seqs, num_heads, head_dim, g.num_parts);
  st = check_workspace(w.bytes, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  *a = pa::DecodeArgs{};
  a->out = out;
  a->query = query;
  a->key_cache = key_cache;
  a->value_cache = value_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->ws_max = g.num_parts > 1 ? reinterpret_cast<float*>(ws + w.off_max) : nullptr;
  a->ws_sum = g.num_parts > 1 ? reinterpret_cast<float*>(ws + w.off_sum) : nullptr;
  a->ws_acc = g.num_parts > 1 ? reinterpret_cast<float*>(ws + w.off_acc) : nullptr;
  a->plan = reinterpret_cast<int4*>(ws + w.off_plan);
  a->plan_count = reinterpret_cast<int32_t*>(ws + w.off_count);
  a->seq_shared = g.num_parts > 1 ? reinterpret_cast<int32_t*>(ws + w.off_shared) : nullptr;
  a->members = g.num_parts > 1 ? reinterpret_cast<int32_t*>(ws + w.off_members) : nullptr;
  a->num_seqs = num_seqs;
  a->num_heads = num_heads;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->log2_block_size = log2i(block_size);
  a->num_blocks = num_blocks;
  a->ctx_limit = g.ctx_limit;
  a->part_tokens = g.part_tokens;
  a->num_parts = g.num_parts;
  a->scale = scale;
  a->softcap = logit_softcap;
  a->window = sliding_window;
  a->dtype = dtype;
  return PA_OK;
}

pa_status to_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// True if a kernel may dereference `p`: device memory, or pinned host memory
// that HIP maps at the same address.  Pageable host memory (and anything HIP
// does not know) is refused, since a kernel touching it would fault.
bool device_addressable(const void* p) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return false;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return true;
  return attr.type == hipMemoryTypeHost && attr.devicePointer == p;
}

}  // namespace

namespace {

pa_status prefill_impl(void* out, const void* query, const int32_t* query_start_loc,
                           int32_t num_q_tokens, int32_t max_query_len, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_context_len, float scale, float logit_softcap,
                           int32_t sliding_window, void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, int32_t kv_fp8, float k_scale, float v_scale,
                           const void* new_key, const void* new_value,
                           const int64_t* slot_mapping, void* stream) {
  if (num_q_tokens < 0 || max_query_len < 0) return PA_ERR_BAD_SHAPE;
  const bool fused = new_key != nullptr || new_value != nullptr || slot_mapping != nullptr;
  if (!valid_variant(logit_softcap, sliding_window)) return PA_ERR_BAD_SHAPE;
  pa_status st = check_decode_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                     max_blocks_per_seq, num_blocks, max_context_len, 0, dtype);
  if (st != PA_OK) return st;
  if (dtype == PA_DTYPE_F32 || num_heads / num_kv_heads > 128) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_q_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !query || !query_start_loc || !key_cache || !value_cache || !block_tables ||
      !context_lens)
    return PA_ERR_NULL_POINTER;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      !aligned(query_start_loc, 4))
    return PA_ERR_UNSUPPORTED;
  if (fused) {
    if (!new_key || !new_value || !slot_mapping) return PA_ERR_NULL_POINTER;
    if (!aligned(new_key, 16) || !aligned(new_value, 16) || !aligned(slot_mapping, 8))
      return PA_ERR_UNSUPPORTED;
  }
  const int32_t ctx_limit = clamp_i32(
      std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * block_size));
  if (ctx_limit == 0) return PA_OK;
  const pa::PrefillWorkspace w = pa::prefill_workspace_layout(
      num_q_tokens, num_heads, head_dim, pa::prefill_num_splits(ctx_limit), num_seqs,
      pa::prefill_num_tiles(num_heads, num_kv_heads, max_query_len));
  st = check_workspace(w.bytes, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  pa::PrefillArgs a{};
  a.out = out;
  a.query = query;
  a.query_start_loc = query_start_loc;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_q_tokens = num_q_tokens;
  a.max_query_len = max_query_len;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.log2_block_size = log2i(block_size);
  a.num_blocks = num_blocks;
  a.ctx_limit = ctx_limit;
  a.window = sliding_window;
  a.scale = scale;
  a.softcap = logit_softcap;
  a.dtype = dtype;
  a.kv_fp8 = kv_fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.new_key = new_key;
  a.new_value = new_value;
  a.slot_mapping = slot_mapping;
  a.fused = fused ? 1 : 0;
  return to_status(pa::launch_prefill(a, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "null pointer argument";
    case PA_ERR_BAD_SHAPE: return "inconsistent or negative size argument";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, block_size or alignment";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_TOO_LARGE: return "call needs more than the fixed scratch of pa_decode_noalloc";
    default: return "unknown status";
  }
}

int pa_version(void) { return 104; }

pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                               void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PA_ERR_BAD_SHAPE;
  if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_UNSUPPORTED;
  pa::CacheWriteArgs a{key, value, key_cache, value_cache, slot_mapping, num_tokens,
                       num_kv_heads, head_dim, log2i(block_size), num_blocks, elem_bytes(dtype),
                       dtype, 0, 1.f, 1.f};
  return to_status(pa::launch_reshape_and_cache(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                   void* value_cache, const int64_t* slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                                   float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PA_ERR_BAD_SHAPE;
  if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_BAD_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_UNSUPPORTED;
  pa::CacheWriteArgs a{key, value, key_cache, value_cache, slot_mapping, num_tokens,
                       num_kv_heads, head_dim, log2i(block_size), num_blocks, elem_bytes(dtype),
                       dtype, 1, k_scale, v_scale};
  return to_status(pa::launch_reshape_and_cache(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks < 0) return PA_ERR_BAD_SHAPE;
  if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(block_mapping, 8))
    return PA_ERR_UNSUPPORTED;
  pa::BlockCopyArgs a{};
  a.src[0] = key_cache;
  a.src[1] = value_cache;
  a.dst[0] = key_cache;
  a.dst[1] = value_cache;
  a.num_pools = 2;
  a.block_mapping = block_mapping;
  a.num_pairs = num_pairs;
  a.block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  a.src_blocks = num_blocks;
  a.dst_blocks = num_blocks;
  return to_status(pa::launch_block_copy(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_stream_read_probe(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words,
                               void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || sink_words < 0) return PA_ERR_BAD_SHAPE;
  if (!src || !sink) return PA_ERR_NULL_POINTER;
  if (!aligned(src, 16) || !aligned(sink, 4)) return PA_ERR_UNSUPPORTED;
  if (sink_words < (bytes + pa::kProbeSpan - 1) / pa::kProbeSpan) return PA_ERR_WORKSPACE_TOO_SMALL;
  return to_status(pa::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

pa_status pa_swap_blocks(const void* src_cache, void* dst_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int64_t block_bytes, int32_t src_num_blocks,
                         int32_t dst_num_blocks, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!src_cache || !dst_cache || !block_mapping) return PA_ERR_NULL_POINTER;
  if (!aligned(src_cache, 16) || !aligned(dst_cache, 16) || !aligned(block_mapping, 8))
    return PA_ERR_UNSUPPORTED;
  if (!device_addressable(src_cache) || !device_addressable(dst_cache) ||
      !device_addressable(block_mapping))
    return PA_ERR_UNSUPPORTED;
  pa::BlockCopyArgs a{};
  a.src[0] = src_cache;
  a.dst[0] = dst_cache;
  a.num_pools = 1;
  a.block_mapping = block_mapping;
  a.num_pairs = num_pairs;
  a.block_bytes = block_bytes;
  a.src_blocks = src_num_blocks;
  a.dst_blocks = dst_num_blocks;
  return to_status(pa::launch_block_copy(a, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || partition_size < 0) return 0;
  const DecodeGeom g = decode_geom(max_context_len, partition_size);
  return pa::decode_workspace_layout(num_seqs, num_heads, head_dim, g.num_parts).bytes;
}

pa_status pa_decode_partitions(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_context_len, float scale, float logit_softcap,
                               int32_t sliding_window, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, pa_dtype dtype, void* stream) {
  pa::DecodeArgs a;
  pa_status st = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, max_context_len, scale, logit_softcap,
                             sliding_window, partition_size, workspace, workspace_bytes, dtype,
                             &a);
  if (st != PA_OK || num_seqs == 0) return st;
  return to_status(pa::launch_decode_partitions(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_decode_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t max_context_len, int32_t sliding_window,
                           int32_t partition_size, const void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0 || sliding_window < 0)
    return PA_ERR_BAD_SHAPE;
  if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs > 0 && max_blocks_per_seq <= 0) return PA_ERR_BAD_SHAPE;
  if (partition_size < 0 || (partition_size > 0 && (partition_size % 64 != 0 ||
                                                     partition_size % block_size != 0)))
    return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !context_lens) return PA_ERR_NULL_POINTER;
  if (!aligned(out, 16) || !aligned(context_lens, 4)) return PA_ERR_UNSUPPORTED;
  const DecodeGeom g = decode_geom(
      std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * block_size),
      partition_size);
  if (g.num_parts <= 1) return PA_OK;  // the partition kernel wrote the output
  const pa::DecodeWorkspace w = pa::decode_workspace_layout(num_seqs, num_heads, head_dim, g.num_parts);
  pa_status st = check_workspace(w.bytes, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  pa::DecodeArgs a{};
  const char* ws = static_cast<const char*>(workspace);
  a.out = out;
  a.context_lens = context_lens;
  a.ws_max = reinterpret_cast<float*>(const_cast<char*>(ws) + w.off_max);
  a.ws_sum = reinterpret_cast<float*>(const_cast<char*>(ws) + w.off_sum);
  a.ws_acc = reinterpret_cast<float*>(const_cast<char*>(ws) + w.off_acc);
  // The partition call's plan: the reduce reads how many partitions an item joined.
  a.plan_count = reinterpret_cast<int32_t*>(const_cast<char*>(ws) + w.off_count);
  a.seq_shared = reinterpret_cast<int32_t*>(const_cast<char*>(ws) + w.off_shared);
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.ctx_limit = g.ctx_limit;
  a.part_tokens = g.part_tokens;
  a.num_parts = g.num_parts;
  a.window = sliding_window;
  a.dtype = dtype;
  return to_status(pa::launch_decode_reduce(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_context_len, float scale,
                    float logit_softcap, int32_t sliding_window, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, pa_dtype dtype, void* stream) {
  pa::DecodeArgs a;
  pa_status st = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, max_context_len, scale, logit_softcap,
                             sliding_window, partition_size, workspace, workspace_bytes, dtype,
                             &a);
  if (st != PA_OK || num_seqs == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = to_status(pa::launch_decode_partitions(a, s));
  if (st != PA_OK) return st;
  return to_status(pa::launch_decode_reduce(a, s));
}

pa_status pa_decode_fused_write(void* out, const void* query, const void* key, const void* value,
                                const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                                void* value_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, float logit_softcap,
                                int32_t sliding_window, int32_t partition_size, void* workspace,
                                size_t workspace_bytes, pa_dtype dtype, void* stream) {
  // The write's checks (as pa_reshape_and_cache), then the decode's.
  if (num_tokens < 0) return PA_ERR_BAD_SHAPE;
  if (num_tokens > 0) {
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
        !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
      return PA_ERR_UNSUPPORTED;
  }
  pa::DecodeArgs a{};
  pa_status st = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, max_context_len, scale, logit_softcap,
                             sliding_window, partition_size, workspace, workspace_bytes, dtype,
                             &a);
  if (st != PA_OK) return st;
  const pa::CacheWriteArgs w{key, value, key_cache, value_cache, slot_mapping, num_tokens,
                             num_kv_heads, head_dim, log2i(block_size), num_blocks,
                             elem_bytes(dtype), dtype, 0, 1.f, 1.f};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (num_seqs == 0)  // a write only
    return num_tokens > 0 ? to_status(pa::launch_reshape_and_cache(w, s)) : PA_OK;
  st = to_status(pa::launch_decode_partitions_write(a, num_tokens > 0 ? &w : nullptr, s));
  if (st != PA_OK) return st;
  return to_status(pa::launch_decode_reduce(a, s));
}

pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_context_len, float scale, float logit_softcap,
                            int32_t sliding_window, int32_t partition_size, pa_dtype dtype,
                            void* stream) {
  // Host validation first, before any HIP call: the placeholder workspace
  // address only lets decode_args check the other arguments and the size; it
  // is never passed on.
  pa::DecodeArgs a;
  void* const placeholder = reinterpret_cast<void*>(uintptr_t(256));
  pa_status st = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, max_context_len, scale, logit_softcap,
                             sliding_window, partition_size, placeholder,
                             pa::kNoAllocScratchBytes, dtype, &a);
  if (st == PA_ERR_WORKSPACE_TOO_SMALL) return PA_ERR_TOO_LARGE;
  if (st != PA_OK || num_seqs == 0) return st;
  void* scratch = nullptr;
  if (pa::noalloc_scratch(&scratch) != hipSuccess) return PA_ERR_LAUNCH;
  st = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                   context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                   num_blocks, max_context_len, scale, logit_softcap, sliding_window,
                   partition_size, scratch, pa::kNoAllocScratchBytes, dtype, &a);
  if (st != PA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = to_status(pa::launch_decode_partitions(a, s));
  if (st != PA_OK) return st;
  return to_status(pa::launch_decode_reduce(a, s));
}

pa_status pa_decode_partitions_fp8(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_context_len, float scale, float logit_softcap,
                                   int32_t sliding_window, int32_t partition_size, float k_scale,
                                   float v_scale, void* workspace, size_t workspace_bytes,
                                   pa_dtype dtype, void* stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_BAD_SHAPE;
  pa::DecodeArgs a;
  pa_status st = decode_args(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                             context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, max_context_len, scale, logit_softcap,
                             sliding_window, partition_size, workspace, workspace_bytes, dtype,
                             &a);
  if (st != PA_OK || num_seqs == 0) return st;
  a.kv_fp8 = 1;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return to_status(pa::launch_decode_partitions(a, static_cast<hipStream_t>(stream)));
}

pa_status pa_decode_fp8(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                        float scale, float logit_softcap, int32_t sliding_window,
                        int32_t partition_size, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, pa_dtype dtype, void* stream) {
  pa_status st = pa_decode_partitions_fp8(
      out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
      num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale,
      logit_softcap, sliding_window, partition_size, k_scale, v_scale, workspace, workspace_bytes,
      dtype, stream);
  if (st != PA_OK || num_seqs == 0) return st;
  return pa_decode_reduce(out, context_lens, num_seqs, num_heads, head_dim, max_blocks_per_seq,
                          block_size, max_context_len, sliding_window, partition_size, workspace,
                          workspace_bytes, dtype, stream);
}

size_t pa_prefill_workspace_bytes(int32_t num_q_tokens, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                  int32_t max_context_len) {
  if (num_q_tokens <= 0 || num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0 || head_dim <= 0 || max_query_len <= 0 || max_context_len <= 0)
    return 0;
  return pa::prefill_workspace_layout(num_q_tokens, num_heads, head_dim,
                                      pa::prefill_num_splits(max_context_len), num_seqs,
                                      pa::prefill_num_tiles(num_heads, num_kv_heads, max_query_len))
      .bytes;
}

pa_status pa_prefill_chunk(void* out, const void* query, const int32_t* query_start_loc,
                           int32_t num_q_tokens, int32_t max_query_len, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_context_len, float scale, float logit_softcap,
                           int32_t sliding_window, void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, void* stream) {
  return prefill_impl(out, query, query_start_loc, num_q_tokens, max_query_len, key_cache,
                      value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                      scale, logit_softcap, sliding_window, workspace, workspace_bytes, dtype, 0,
                      1.f, 1.f, nullptr, nullptr, nullptr, stream);
}

pa_status pa_prefill_chunk_fused(void* out, const void* query, const void* key, const void* value,
                                 const int64_t* slot_mapping, const int32_t* query_start_loc,
                                 int32_t num_q_tokens, int32_t max_query_len, void* key_cache,
                                 void* value_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_context_len, float scale, float logit_softcap,
                                 int32_t sliding_window, void* workspace, size_t workspace_bytes,
                                 pa_dtype dtype, void* stream) {
  if (num_q_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_NULL_POINTER;
  return prefill_impl(out, query, query_start_loc, num_q_tokens, max_query_len, key_cache,
                      value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                      scale, logit_softcap, sliding_window, workspace, workspace_bytes, dtype, 0,
                      1.f, 1.f, key, value, slot_mapping, stream);
}

pa_status pa_prefill_chunk_fp8(void* out, const void* query, const int32_t* query_start_loc,
                               int32_t num_q_tokens, int32_t max_query_len, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_context_len, float scale, float logit_softcap,
                               int32_t sliding_window, float k_scale, float v_scale,
                               void* workspace, size_t workspace_bytes, pa_dtype dtype,
                               void* stream) {
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_BAD_SHAPE;
  return prefill_impl(out, query, query_start_loc, num_q_tokens, max_query_len, key_cache,
                      value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                      scale, logit_softcap, sliding_window, workspace, workspace_bytes, dtype, 1,
                      k_scale, v_scale, nullptr, nullptr, nullptr, stream);
}

}  // extern "C"

// Host-side interface between the C-ABI shim (pa_api.cpp) and the kernel
// translation units.  Every argument here has already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_attention.h"

namespace pa {

constexpr int kDecodeThreads = 256;  // 4 waves per decode workgroup
constexpr int kSegTokens = 512;      // tokens whose block ids are staged in LDS at once
constexpr int kMaxHeadsPerWg = 8;    // query heads of one KV head handled by one workgroup
constexpr int kShareMaxSeqs = 2048;  // decode calls of at most this many sequences look for shared partitions
// Query rows of one group work unit of the MFMA decode kernel (all the
// sequences of a shared partition, times the group's query heads): one
// 16-row tile per wave of its workgroup at head_dim 64 and 256 (four waves)
// and at 128 over 16-bit caches (eight waves); two per wave at 128 over E4M3
// caches (four waves), the only E4M3 head_dim with group units.
constexpr int decode_group_rows(int head_dim) { return head_dim == 128 ? 128 : 64; }

struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int64_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t log2_block_size;
  int32_t num_blocks;
  int32_t elem_bytes;
  int32_t src_dtype;  // key/value dtype (pa_dtype)
  int32_t kv_fp8;     // quantise into E4M3 caches: byte = E4M3(key / k_scale), saturating
  float k_scale, v_scale;
};

// Whole-block copies from one or two source pools to destination pools of the
// same block size (block_ops.hip).
struct BlockCopyArgs {
  const void* src[2];
  void* dst[2];
  int32_t num_pools;             // 1 or 2 (K and V)
  const int64_t* block_mapping;  // [num_pairs][2] = (source block, destination block)
  int64_t num_pairs;
  int64_t block_bytes;           // multiple of 16
  int64_t src_blocks, dst_blocks;
};

struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_max;   // [S][Hq][P] running max (log2 units)
  float* ws_sum;   // [S][Hq][P] softmax denominators
  float* ws_acc;   // [S][Hq][P][D] un-normalised partial outputs
  int4* plan;      // [S * P] work items, group items first, then the others longest first:
                   //   (seq, first partition, span | single << 8, ctx), or for a group item
                   //   (offset in members, partition p, 1 | 1 << 9 | member count << 16, (p + 1) * P)
  int32_t* plan_count;  // [0] valid items in `plan`, [1] log2 of the partitions an item joins,
                        // [2] units taken from the partition kernel's queue, [3] group items
  int32_t* seq_shared;  // [S] leading partitions of each sequence that group items compute
  int32_t* members;     // [S * P] the sequences of each group item, one run per item
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t log2_block_size;
  int32_t num_blocks;
  int32_t ctx_limit;       // min(max_context_len, max_blocks_per_seq * block_size)
  int32_t part_tokens;     // tokens per partition (> 0)
  int32_t num_parts;       // partitions covering ctx_limit
  int32_t plan_min_items;  // the plan may join partitions while it keeps this many items (0: never)
  int32_t window;          // sliding window (tokens attended, ending at the query); 0 = whole context
  int32_t share;           // look for partitions whose blocks several sequences' tables share
  int32_t share_max_members;  // sequences one group item may hold (its query rows fit a unit)
  int32_t share_vec;       // the search may read a partition's block ids 16 bytes at a time
  int32_t static_plan;     // no plan kernel: one (sequence, partition, head chunk) slot per
                           // workgroup, partition-major (decode_mfma.hip, Unit info)
  float scale;
  float softcap;           // logit soft-cap; 0 = none
  pa_dtype dtype;          // query, output (and cache unless kv_fp8)
  int32_t kv_fp8;          // caches hold E4M3 bytes, value = byte * k_scale (v_scale)
  float k_scale, v_scale;
};

struct DecodeWorkspace {
  size_t bytes;
  size_t off_max, off_sum, off_acc;  // partition states (only when P > 1)
  size_t off_count, off_plan;        // work plan (always)
  size_t off_shared, off_members;    // shared-partition plan (only when P > 1)
};
DecodeWorkspace decode_workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t num_parts);

struct PrefillArgs {
  void* out;
  const void* query;
  const int32_t* query_start_loc;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_q_tokens;
  int32_t max_query_len;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t log2_block_size;
  int32_t num_blocks;
  int32_t ctx_limit;
  int32_t window;  // sliding window (keys attended, ending at the row's own position); 0 = none
  float scale;
  float softcap;   // logit soft-cap; 0 = none
  pa_dtype dtype;  // query, output (and cache unless kv_fp8)
  int32_t kv_fp8;  // caches hold E4M3 bytes, value = byte * k_scale (v_scale)
  float k_scale, v_scale;
  // Fused write (fused != 0): the chunk tokens' own K/V ([num_q_tokens][Hkv][D])
  // are read from new_key/new_value instead of the cache, and written into the
  // cache at slot_mapping by the kernel.
  const void* new_key;
  const void* new_value;
  const int64_t* slot_mapping;
  int32_t fused;
};

// Size of the fixed device scratch that pa_decode_noalloc uses in place of a
// workspace (decode_scratch.hip), and its address on the current device.
constexpr size_t kNoAllocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_block_copy(const BlockCopyArgs& a, hipStream_t stream);
// Bytes each workgroup of the streaming-read probe reads (one sink word each).
constexpr int64_t kProbeSpan = 256 * 1024;
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream);
// As launch_decode_partitions, with the step's cache write (16-bit or fp32
// caches, write->kv_fp8 == 0) done in the plan's launch, or, for a call with
// the static plan, in a launch of its own first.
hipError_t launch_decode_partitions_write(const DecodeArgs& a, const CacheWriteArgs* write,
                                          hipStream_t stream);
// 16-bit caches: the MFMA kernel (decode_mfma.hip), any group size.
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream);
// Workgroups one launch of the MFMA kernel keeps resident (its persistent grid).
int decode_mfma_grid(const DecodeArgs& a);
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream);
struct PrefillWorkspace {
  size_t bytes;
  size_t off_max, off_sum, off_acc;  // key-range partial states (only when nsplit > 1)
  size_t off_count, off_plan;        // work plan (always)
  size_t off_toklim;                 // last key of each query token's rows, or -1, for the merge (only when nsplit > 1)
};
int32_t prefill_num_splits(int32_t ctx_limit);
int32_t prefill_num_tiles(int32_t num_heads, int32_t num_kv_heads, int32_t max_query_len);
PrefillWorkspace prefill_workspace_layout(int32_t num_q_tokens, int32_t num_heads,
                                          int32_t head_dim, int32_t nsplit, int32_t num_seqs,
                                          int32_t ntiles);
hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream);

}  // namespace pa

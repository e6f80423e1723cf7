/*
 * paged_attention.h -- C ABI of the MI355X (gfx950) paged-attention library.
 *
 * The operation: each query token attends to the keys and values of its own
 * sequence, which sit in fixed-size physical blocks of a shared pool and are
 * reached through a per-sequence block table (mini-vLLM README, "How it works
 * -- Paged KV-cache").  Three operations make up the path:
 *
 *   pa_reshape_and_cache  write the new tokens' K/V into their pool slots
 *                         (mini-vLLM README, "End-to-end throughput vs
 *                         baselines": one scatter for all sequences' K/V);
 *   pa_decode             one query token per sequence attends its whole
 *                         context (wLLM PyPI page, "Features -- Core engine":
 *                         the PagedAttention kernel over a block-based cache),
 *                         split into context partitions plus a merge;
 *   pa_prefill_chunk      a chunk of a prompt attends the cached context before
 *                         it and itself causally (wLLM PyPI page, "Features --
 *                         Core engine": chunked prefill).
 *
 * Two block-pool operations sit beside them: pa_copy_blocks (copy-on-write of
 * a shared block) and pa_swap_blocks (blocks to and from a host pool); the
 * _fp8 calls at the end are the same operations over E4M3 caches.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are DEVICE pointers into memory the caller owns
 *   (pa_swap_blocks also takes pinned host pools); the library allocates
 *   nothing and keeps no state between calls.  Every call
 *   only enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 *   returns; results are ready when the stream reaches that point.
 * - Element type `dtype` is shared by query, key/value, caches and output.
 * - Cache layout (K and V alike): [num_blocks][num_kv_heads][block_size][head_dim],
 *   contiguous.  Token t of a sequence lives in block table[t / block_size]
 *   at offset t % block_size.  Query/key/value/output are contiguous
 *   [tokens][heads][head_dim].
 * - Grouped-query heads: query head h reads KV head h / (num_heads /
 *   num_kv_heads) (contiguous groups; mini-vLLM's GQA-aware kernel maps each
 *   query head to its KV head instead of expanding K/V).
 * - Supported: head_dim 64, 128 or 256; block_size a power of two 1..256;
 *   dtype F32, F16 or BF16 (prefill: F16 or BF16).  Softmax and accumulation
 *   run in fp32; outputs are rounded to `dtype` to nearest-even.
 * - Host-side arguments are validated before anything is launched and a bad
 *   one returns an error status with nothing enqueued.  Device arrays are NOT
 *   inspected (that would need a synchronisation).  Their contents are
 *   preconditions: block ids in [0, num_blocks), context_lens in
 *   [0, min(max_context_len, max_blocks_per_seq * block_size)], slots unique.
 *   Kernels clamp every index to the buffers they were given, so violating a
 *   precondition gives wrong numbers, never an out-of-bounds access: a slot or
 *   block id outside the pool is skipped (write) or replaced by block 0
 *   (read); lengths are clamped to the limits above.
 * - Launch failures are reported as PA_ERR_LAUNCH.
 */
#ifndef PAGED_ATTENTION_H_
#define PAGED_ATTENTION_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,
  PA_ERR_BAD_SHAPE = 2,
  PA_ERR_UNSUPPORTED = 3,
  PA_ERR_WORKSPACE_TOO_SMALL = 4,
  PA_ERR_LAUNCH = 5,
  PA_ERR_TOO_LARGE = 6 /* pa_decode_noalloc: the call needs more than its fixed scratch */
} pa_status;

typedef enum pa_dtype { PA_DTYPE_F32 = 0, PA_DTYPE_F16 = 1, PA_DTYPE_BF16 = 2 } pa_dtype;

/* Static string naming a status code ("unknown status" for other values). */
const char* pa_status_str(int status);

/* Library ABI version (major * 100 + minor). */
int pa_version(void);

/*
 * Slot-mapped cache write.  For every n < num_tokens with
 * s = slot_mapping[n] >= 0:  key_cache[s / block_size][h][s % block_size][:] =
 * key[n][h][:] and the same for value, for every KV head h.  A pure bit copy.
 *   key, value          [num_tokens][num_kv_heads][head_dim]
 *   key_cache, value_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *   slot_mapping        int64 [num_tokens]; negative = skip this token;
 *                       slots >= num_blocks * block_size are skipped too.
 * num_tokens == 0 is a valid no-op.  Duplicate slots: which write lands is
 * unspecified.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                               void* stream);

/*
 * Block copy inside one pool, for copy-on-write of a block that several
 * block tables share (wLLM case study, ADR-001 on the KV-cache layout: prefix
 * sharing is a block-table operation; mini-vLLM README, "Limitations": block
 * reference counts are kept for prefix caching).  For every pair
 * i < num_pairs with (src, dst) = (block_mapping[2i], block_mapping[2i+1]):
 * key_cache[dst] = key_cache[src] and value_cache[dst] = value_cache[src],
 * whole blocks ([num_kv_heads][block_size][head_dim] each).  A bit copy.
 *   key_cache, value_cache  [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_mapping           int64 [num_pairs][2], device-addressable memory
 * A pair with an id outside [0, num_blocks) is skipped.  Destinations must be
 * distinct and no destination may be another pair's source (the pairs run in
 * no particular order).  num_pairs == 0 is a valid no-op.
 */
pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * Block copy between two pools of the same block size, for swapping a
 * preempted sequence's blocks out to host memory and back (wLLM PyPI page,
 * "Features -- Core engine": CPU-swap preemption).  For every pair i:
 * dst_cache block block_mapping[2i+1] = src_cache block block_mapping[2i],
 * block_bytes bytes each.  Call it once per pool (K, then V).
 *   src_cache, dst_cache  [src_num_blocks] and [dst_num_blocks] blocks of
 *                         block_bytes; either may be host memory that the
 *                         device can address (pinned: hipHostMalloc, or
 *                         torch's pin_memory), the other device memory
 *   block_mapping         int64 [num_pairs][2], device-addressable memory
 *   block_bytes           > 0, a multiple of 16
 * A pair with an id outside its pool is skipped; destinations must be
 * distinct.  The copy is asynchronous on `stream` like every other call.
 * Each pointer is checked with hipPointerGetAttributes before the launch:
 * pageable host memory (or a pointer HIP does not know) gives
 * PA_ERR_UNSUPPORTED, since the kernel could not read it.
 */
pa_status pa_swap_blocks(const void* src_cache, void* dst_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int64_t block_bytes, int32_t src_num_blocks,
                         int32_t dst_num_blocks, void* stream);

/*
 * Measurement aid, not part of the attention path: a plain streaming read of
 * `bytes` of device memory with non-temporal 16-byte loads, to compare the
 * kernels' HBM rates with what a bare read reaches on the same device.
 * Workgroup w reads bytes [w * 262144, (w + 1) * 262144) and writes the XOR of
 * their 32-bit words to sink[w].
 *   src    device memory, 16-byte aligned; bytes > 0, a multiple of 16
 *   sink   device memory, sink_words >= ceil(bytes / 262144) uint32 words
 * Returns PA_ERR_BAD_SHAPE for a bad size and PA_ERR_WORKSPACE_TOO_SMALL for a
 * short sink.
 */
pa_status pa_stream_read_probe(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words,
                               void* stream);

/*
 * Workspace bytes pa_decode needs (0 only when num_seqs <= 0), with
 * P = ceil(max_context_len / partition_size) (1 when partition_size == 0 or
 * the context fits one partition).  The regions, in this order, each starting
 * 256-byte aligned: when P > 1, the partial results (num_seqs * num_heads * P
 * maxima, as many sums, and as many rows of head_dim floats); then the work
 * plan: 256 bytes of counts (int32: items, log2 of the partitions an item
 * joins, units taken from the queue, items of shared partitions) and 16 bytes
 * per item for num_seqs * P items; when P > 1, num_seqs int32 counts of
 * shared partitions and num_seqs * P int32 sequence ids of shared-partition
 * items.  The contents are the library's and change with every call; the
 * layout is stated for tools that read the plan back.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * Decode attention: row s of `query` is the token at position
 * context_lens[s] - 1 of sequence s and attends all context_lens[s] cached
 * tokens of that sequence (the current token's K/V must already be written).
 *   out, query      [num_seqs][num_heads][head_dim]
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]
 *   context_lens    int32 [num_seqs]; 0 gives an all-zero output row
 *   max_context_len host-side upper bound of context_lens; sizes the grid
 *   scale           multiplies q.k before the softmax (e.g. 1/sqrt(head_dim))
 *   logit_softcap   0, or a cap c > 0: every scaled score x becomes
 *                   c * tanh(x / c) before the softmax
 *   sliding_window  0, or a window W > 0: a row at position p attends only
 *                   keys p - W + 1 .. p (its W most recent tokens).  The two
 *                   are the Gemma-2-style variants that the wLLM PyPI page
 *                   ("Supported models") names as kernel work; the pages do
 *                   not define them further, so these are the usual forms.
 *                   A negative window, or a negative or non-finite cap, is
 *                   PA_ERR_BAD_SHAPE.
 *   partition_size  tokens per context partition; 0 = never split.  Otherwise
 *                   a positive multiple of 64 and of block_size.  Sequences
 *                   longer than one partition are processed by several
 *                   workgroups whose partial softmax states are merged by a
 *                   second kernel through `workspace`.
 *   workspace       device scratch of >= pa_decode_workspace_bytes(...) bytes
 *                   (may be NULL when that is 0); overwritten, no alignment
 *                   requirement beyond 256 bytes.  It holds the call's work
 *                   plan and the counter from which the attention kernel's
 *                   workgroups take their work, so two calls in flight at once
 *                   (on different streams) need different workspaces.
 */
pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                    float scale, float logit_softcap, int32_t sliding_window,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    pa_dtype dtype, void* stream);

/*
 * The two halves of pa_decode, for callers that time or schedule them apart
 * (pa_decode == pa_decode_partitions followed by pa_decode_reduce on the same
 * stream with the same arguments).  pa_decode_partitions writes the output of
 * every sequence whose context one work item covers (one partition, or a run
 * of up to four consecutive partitions that the work plan joins into one item
 * when there are enough items to fill the device) and the partial softmax
 * states of the others into `workspace`; pa_decode_reduce merges those partial
 * states (log-sum-exp weighted) into `out` and leaves the other rows
 * untouched.  The reduce reads the plan's choice from `workspace`, so it must
 * get the workspace the partition call wrote.
 */
pa_status pa_decode_partitions(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_context_len, float scale, float logit_softcap,
                               int32_t sliding_window, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, pa_dtype dtype, void* stream);

pa_status pa_decode_reduce(void* out, const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t max_context_len,
                           int32_t sliding_window, int32_t partition_size,
                           const void* workspace, size_t workspace_bytes, pa_dtype dtype,
                           void* stream);

/*
 * pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, semantics and results as pa_decode without the workspace: the
 * work plan and partition states go to a fixed scratch array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds in device memory (one per
 * device it runs on, kept until the process ends).  Nothing is allocated,
 * freed or memset by this call; the kernels reset every counter they read.
 *   - A call whose pa_decode_workspace_bytes(num_seqs, num_heads, head_dim,
 *     min(max_context_len, max_blocks_per_seq * block_size), partition_size)
 *     exceeds PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_TOO_LARGE with nothing
 *     enqueued.
 *   - All calls on one device share that device's scratch, which keeps the
 *     last call's contents: two calls that can overlap on one device (other
 *     streams, other host threads) race and give wrong results.  Serialise
 *     them, or use pa_decode with a workspace per stream.
 *   - The first call on a device looks up the scratch's device address (no
 *     allocation, nothing enqueued); a failure there is PA_ERR_LAUNCH.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_context_len, float scale, float logit_softcap,
                            int32_t sliding_window, int32_t partition_size, pa_dtype dtype,
                            void* stream);

/*
 * Workspace bytes pa_prefill_chunk needs for these sizes (0 if none).
 */
size_t pa_prefill_workspace_bytes(int32_t num_q_tokens, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_query_len, int32_t max_context_len);

/*
 * Chunked-prefill attention.  Sequence s owns query rows
 * query_start_loc[s] .. query_start_loc[s+1]-1 (L rows, L may be 1) and a
 * context of context_lens[s] tokens that already includes those L tokens (their
 * K/V must be written first).  Row i sits at position C - L + i and attends
 * keys 0 .. C - L + i: the causal mask is aligned to the end of the context.
 * logit_softcap and sliding_window as for pa_decode (with a window W, row i
 * attends keys C - L + i - W + 1 .. C - L + i).
 *   out, query       [num_q_tokens][num_heads][head_dim]
 *   query_start_loc  int32 [num_seqs + 1], non-decreasing, last = num_q_tokens
 *   max_query_len    host-side upper bound of the chunk lengths (grid size)
 *   other arguments  as for pa_decode.  Rows of a sequence with L > C are
 *                    preconditions violations (their keys are clamped to C).
 */
pa_status pa_prefill_chunk(void* out, const void* query, const int32_t* query_start_loc,
                           int32_t num_q_tokens, int32_t max_query_len, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_context_len, float scale, float logit_softcap,
                           int32_t sliding_window, void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, void* stream);

/*
 * A decode step in one call: the step's slot-mapped cache write
 * (pa_reshape_and_cache of key/value [num_tokens][num_kv_heads][head_dim],
 * `dtype`, at the int64 slot_mapping [num_tokens]; negative or out-of-pool
 * slots are skipped) followed by pa_decode over the written caches, with the
 * write done in the same launch as the decode's work plan (neither reads what
 * the other writes), so the step takes one launch fewer than the two calls.
 * After the call the caches and `out` are those of pa_reshape_and_cache then
 * pa_decode with the same arguments.  16-bit and fp32 caches (E4M3 caches:
 * pa_reshape_and_cache_fp8 then pa_decode_fp8).  num_tokens may be 0 (a
 * plain pa_decode); num_seqs may be 0 (a plain write).  Arguments, workspace
 * and errors as pa_reshape_and_cache and pa_decode.  (mini-vLLM README,
 * "End-to-end throughput vs baselines": launch overhead is the dominant cost
 * for small models, and the new tokens' K/V go into the pool in one scatter.)
 */
pa_status pa_decode_fused_write(void* out, const void* query, const void* key, const void* value,
                                const int64_t* slot_mapping, int32_t num_tokens, void* key_cache,
                                void* value_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_context_len, float scale, float logit_softcap,
                                int32_t sliding_window, int32_t partition_size, void* workspace,
                                size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * Chunked prefill with the chunk's own cache write fused in (one call for a
 * mixed step: decode rows are chunks of L = 1).  As pa_prefill_chunk, plus
 * the chunk tokens' new K and V ([num_q_tokens][num_kv_heads][head_dim],
 * `dtype`) and their int64 slot_mapping [num_q_tokens] (negative or outside
 * the pool: not written).  The attention reads the chunk's own keys and
 * values from `key`/`value` (never from the cache, so no part of the launch
 * waits for another's write), and the kernel writes them into the caches as
 * pa_reshape_and_cache would; after the call the caches and the output are
 * those of pa_reshape_and_cache followed by pa_prefill_chunk.  context_lens
 * still include the chunk.  16-bit caches only.  (wLLM PyPI page, "Features --
 * Core engine": chunked prefill; mini-vLLM README, "End-to-end throughput vs
 * baselines": one scatter for all sequences' K/V.)
 */
pa_status pa_prefill_chunk_fused(void* out, const void* query, const void* key, const void* value,
                                 const int64_t* slot_mapping, const int32_t* query_start_loc,
                                 int32_t num_q_tokens, int32_t max_query_len, void* key_cache,
                                 void* value_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_context_len, float scale, float logit_softcap,
                                 int32_t sliding_window, void* workspace, size_t workspace_bytes,
                                 pa_dtype dtype, void* stream);

/*
 * fp8 KV cache.  The vLLM native-Windows build README lists fp8 among its
 * KV-cache compression options ("KV compression" column of its release
 * table); the pages say no more, so this is the usual form: each cached K and
 * V element is one byte in the OCP 8-bit float format E4M3 (bias 7, 3
 * mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest finite
 * 448) and a cached value is byte * k_scale (K) or byte * v_scale (V), one
 * scale per tensor.  The caches are uint8 [num_blocks][num_kv_heads]
 * [block_size][head_dim]; everything else is as in the calls above.
 *
 * pa_reshape_and_cache_fp8: the slot-mapped write, quantising each element:
 * byte = E4M3(key / k_scale) -- the division correctly rounded in fp32, then
 * round to nearest with ties to even, saturating to +-448; NaN -> 0x7F.  key
 * and value are `dtype` (F32, F16 or BF16).  k_scale, v_scale > 0 and finite,
 * else PA_ERR_BAD_SHAPE.
 */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                   void* value_cache, const int64_t* slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                                   float k_scale, float v_scale, void* stream);

/*
 * Decode (and its first half) over E4M3 caches: as pa_decode /
 * pa_decode_partitions with the K and V scales; the second half is the same
 * pa_decode_reduce.  `dtype` (query and output) must be F16 or BF16 (else
 * PA_ERR_UNSUPPORTED).  The bytes are widened exactly to `dtype` in LDS; the K
 * scale multiplies the scores and the V scale the output.
 */
pa_status pa_decode_fp8(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                        float scale, float logit_softcap, int32_t sliding_window,
                        int32_t partition_size, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, pa_dtype dtype, void* stream);

pa_status pa_decode_partitions_fp8(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_context_len, float scale, float logit_softcap,
                                   int32_t sliding_window, int32_t partition_size, float k_scale,
                                   float v_scale, void* workspace, size_t workspace_bytes,
                                   pa_dtype dtype, void* stream);

/*
 * Chunked prefill over E4M3 caches: as pa_prefill_chunk with the K and V
 * scales (same workspace size).
 */
pa_status pa_prefill_chunk_fp8(void* out, const void* query, const int32_t* query_start_loc,
                               int32_t num_q_tokens, int32_t max_query_len, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_context_len, float scale, float logit_softcap,
                               int32_t sliding_window, float k_scale, float v_scale,
                               void* workspace, size_t workspace_bytes, pa_dtype dtype,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H_ */

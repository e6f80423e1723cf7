// Work items of the decode partition kernels.
//
// A planning kernel lists every non-empty (sequence, partition) pair, longest
// first, before the partition kernel runs.  Workgroup b of the partition
// kernel then takes item b / (Hkv * head_chunks) of that list, for KV head and
// head chunk b % (Hkv * head_chunks).  The grid is sized for the worst case
// (every sequence at the full context), so the workgroups past the end of the
// list, all at the end of the grid, exit at once.
#pragma once

#include "pa_internal.h"

namespace pa {

struct DecodeItem {
  int seq, part, ctx, kvh, chunk;
  bool valid;
  bool single;  // the sequence's attended tokens lie in one partition: final output
};

// First token a decode row attends: the start of its sliding window (the
// window ends at the row's own token, context_lens - 1), or 0 without one.
__device__ inline int window_start(const DecodeArgs& a, int ctx) {
  return a.window > 0 ? max(0, ctx - a.window) : 0;
}

__device__ inline DecodeItem decode_item(const DecodeArgs& a, int head_chunks) {
  const uint32_t per = static_cast<uint32_t>(a.num_kv_heads * head_chunks);
  const uint32_t j = blockIdx.x / per;
  const uint32_t r = blockIdx.x - j * per;
  const int count = *a.plan_count;
  const int4 it = a.plan[j];  // in bounds: the grid has S * P * per workgroups
  DecodeItem d;
  d.valid = static_cast<int>(j) < count;
  d.seq = it.x;
  d.part = it.y;
  d.ctx = it.w;
  d.single = (it.z >> 8) & 1;
  d.kvh = static_cast<int>(r) / head_chunks;
  d.chunk = static_cast<int>(r) - d.kvh * head_chunks;
  return d;
}

// Grid of a partition kernel: one workgroup per possible item and KV head chunk.
inline uint64_t decode_grid(const DecodeArgs& a, int head_chunks) {
  return static_cast<uint64_t>(a.num_seqs) * a.num_parts * a.num_kv_heads * head_chunks;
}

}  // namespace pa

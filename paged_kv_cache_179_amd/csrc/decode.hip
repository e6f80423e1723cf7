// Paged-attention decode for gfx950: one query token per sequence attends its
// whole context, read block by block through the sequence's block table.
// This file holds the parts shared by both element widths -- the work plan,
// the merge of partition states (decode_reduce) -- and the fp32 partition
// kernel; 16-bit caches use the MFMA kernel of decode_mfma.hip.
//
// The operation is the PagedAttention decode the wLLM PyPI page lists under
// "Features -- Core engine" (a block-based KV cache read by a custom kernel),
// with the grouped-query head mapping of the mini-vLLM README ("End-to-end
// throughput vs baselines": each query head reads its KV head directly).
//
// fp32 partition kernel.  One workgroup (4 waves) handles one
// (sequence, KV head, context partition) and all query heads of that KV head
// (up to 8; larger groups are split over several workgroups).  Inside a
// wave, a token's head_dim row is spread over LPT lanes that each load 16
// contiguous bytes, so one wave-wide load covers TPL = 64 / LPT whole rows
// and every (block, head) run of the [block][head][offset][dim] pool is read
// with fully coalesced 16-byte loads.  q.k is a per-lane dot product followed
// by a DPP butterfly over the LPT lanes of the row.  Each lane keeps an
// online-softmax state (running max m, denominator l, un-normalised
// accumulator) for its own token stream; the states are merged across the
// wave, then across the 4 waves through LDS, at the end of the partition.
//
// A sequence that fits one partition gets its output directly; longer ones
// write (m, l, acc) per partition to the workspace and decode_reduce merges
// them: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
// Scores are kept in log2 units (scale * log2(e) folded in) so every
// exponential is one v_exp_f32.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "decode_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = kDecodeThreads / kWave;

template <typename E, int D>
struct RowLayout {
  static constexpr int kEpl = E::kPerGroup;       // elements per lane load
  static constexpr int kLpt = D / kEpl;           // lanes per token row
  static constexpr int kTpl = kWave / kLpt;       // token rows per wave load
  static constexpr int kUnroll = kTpl >= 8 ? 2 : 4;  // wave loads per tile
  static constexpr int kTile = kUnroll * kTpl;    // tokens per wave iteration
  static_assert(kLpt >= 1 && kLpt <= kWave, "row must fit one wave");
};

template <typename E, int D, int GT, typename S>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(
    DecodeArgs a, int32_t head_chunks, S score) {
  using R = RowLayout<E, D>;
  constexpr int EPL = R::kEpl, LPT = R::kLpt, TPL = R::kTpl, U = R::kUnroll, TILE = R::kTile;

  __shared__ int32_t s_tbl[kSegTokens];
  __shared__ u32x4 s_q[GT * LPT];
  __shared__ float s_max[kWaves][GT];
  __shared__ float s_sum[kWaves][GT];
  __shared__ float s_acc[kWaves][GT][D];

  const DecodeItem item = decode_item(a, head_chunks);
  if (!item.valid) return;
  const int seq = item.seq, part = item.part, ctx = item.ctx, kvh = item.kvh, chunk = item.chunk;

  const int group = a.num_heads / a.num_kv_heads;
  const int h_first = kvh * group + chunk * GT;
  const int nh = min(GT, group - chunk * GT);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int sub = lane % LPT;  // which 16-byte slice of the row
  const int grp = lane / LPT;  // which token row of a wave load

  // Stage the query rows of this head group, then take this lane's slice.
  {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(a.query) +
        (static_cast<int64_t>(seq) * a.num_heads + h_first) * D * E::kBytes);
    for (int i = tid; i < GT * LPT; i += kDecodeThreads) {
      const int h = i / LPT;
      s_q[i] = (h < nh) ? qsrc[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  u32x4 q[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) q[h] = s_q[h * LPT + sub];

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int lbs = a.log2_block_size;
  const int off_mask = (1 << lbs) - 1;
  const char* kbase = static_cast<const char*>(a.key_cache);
  const char* vbase = static_cast<const char*>(a.value_cache);
  const int64_t row_bytes = static_cast<int64_t>(D) * E::kBytes;
  const int64_t lane_bytes = static_cast<int64_t>(sub) * 16;
  const int32_t* table = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;

  const int tok_begin = max(part * a.part_tokens, window_start(a, ctx));
  const int tok_end = min(part * a.part_tokens + a.part_tokens, ctx);
  for (int seg = tok_begin; seg < tok_end; seg += kSegTokens) {
    const int seg_end = min(seg + kSegTokens, tok_end);
    const int first_blk = seg >> lbs;
    const int nblk = ((seg_end - 1) >> lbs) - first_blk + 1;
    __syncthreads();  // previous segment's ids are no longer read
    for (int i = tid; i < nblk; i += kDecodeThreads) {
      const int b = table[first_blk + i];
      s_tbl[i] = (b < 0 || b >= a.num_blocks) ? 0 : b;
    }
    __syncthreads();

    const int ntiles = (seg_end - seg + TILE - 1) / TILE;
    for (int tile = wave; tile < ntiles; tile += kWaves) {
      const int tbase = seg + tile * TILE;
      u32x4 kr[U], vr[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tbase + u * TPL + grp;
        ok[u] = t < seg_end;
        if (ok[u]) {
          const int64_t blk = s_tbl[(t >> lbs) - first_blk];
          const int64_t off =
              ((blk * a.num_kv_heads + kvh) << lbs | (t & off_mask)) * row_bytes + lane_bytes;
          kr[u] = load16(kbase + off);
          vr[u] = load16(vbase + off);
        } else {
          kr[u] = u32x4{0u, 0u, 0u, 0u};
          vr[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }

      float s[GT][U];
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float d = score(group_sum<LPT>(E::dot(q[h], kr[u], 0.f)));
          s[h][u] = ok[u] ? d : -__builtin_inff();
        }

      float vf[U][EPL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[u][e] = E::elem(vr[u], e);

#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float tmax = s[h][0];
#pragma unroll
        for (int u = 1; u < U; ++u) tmax = fmaxf(tmax, s[h][u]);
        const float m_new = fmaxf(m[h], tmax);
        const float m_use = safe_max(m_new);
        const float alpha = exp2_fast(m[h] - m_use);
        m[h] = m_new;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = exp2_fast(s[h][u] - m_use);
          l[h] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = __builtin_fmaf(p, vf[u][e], acc[h][e]);
        }
      }
    }
  }

  // Merge the token streams of this wave (lanes with the same slice).
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const float mw = across_groups_max<LPT>(m[h]);
    const float f = exp2_fast(m[h] - safe_max(mw));
    l[h] = across_groups_sum<LPT>(l[h] * f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = across_groups_sum<LPT>(acc[h][e] * f);
    m[h] = mw;
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][sub * EPL + e] = acc[h][e];
      if (lane == 0) {
        s_max[wave][h] = m[h];
        s_sum[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the 4 waves and write the output or this partition's state.
  for (int idx = tid; idx < nh * D; idx += kDecodeThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    float mx = s_max[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_max[w][h]);
    const float mu = safe_max(mx);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2_fast(s_max[w][h] - mu);
      den = __builtin_fmaf(f, s_sum[w][h], den);
      num = __builtin_fmaf(f, s_acc[w][h][d], num);
    }
    const int64_t row = static_cast<int64_t>(seq) * a.num_heads + h_first + h;
    if (item.single) {
      E::store(a.out, row * D + d, den == 0.f ? 0.f : num / den);
    } else {
      const int64_t ws = row * a.num_parts + part;
      a.ws_acc[ws * D + d] = num;
      if (d == 0) {
        a.ws_max[ws] = mx;
        a.ws_sum[ws] = den;
      }
    }
  }
}

template <typename E, int D, bool WIN>
__global__ __launch_bounds__(kDecodeThreads) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / kWave;
  const int row = blockIdx.x * kWaves + threadIdx.x / kWave;  // seq * Hq + head
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= a.num_seqs * a.num_heads) return;
  const int seq = row / a.num_heads;
  const int64_t base = static_cast<int64_t>(row) * a.num_parts;
  // Without a window a row's partitions start at 0: lane p's max and sum are
  // loaded before the row is known to need merging, in the same round trip as
  // the context length and the plan's counts (lanes past the row's partitions
  // read states no call wrote, and drop them).
  float m_spec = -__builtin_inff(), s_spec = 0.f;
  if (!WIN && lane < a.num_parts) {
    m_spec = a.ws_max[base + lane];
    s_spec = a.ws_sum[base + lane];
  }
  // Everything the skip test below reads, loaded up front (the shared count
  // is only meaningful when the plan made group items, and is then written).
  const int c_raw = a.context_lens[seq];
  const int span_log2 = a.plan_count[1];
  const int n_group = a.plan_count[3];
  const int shared = WIN ? 0 : a.seq_shared[seq];
  const int ctx = max(0, min(c_raw, a.ctx_limit));
  // Partitions holding the attended tokens (the window's, or all of them).
  const int p0 = WIN ? window_start(a, ctx) / a.part_tokens : 0;
  const int p1 = (ctx - 1) / a.part_tokens + 1;
  // Nothing to do for an empty context (its rows are zeros, written by the
  // partition kernel) or for rows whose partitions fit one work item, which
  // the partition kernel wrote, unless group items computed some of their
  // partitions.  One test, without short-circuits, so that all its loads go
  // out together.
  const bool skip = (ctx == 0) | ((p1 - p0 <= (1 << span_log2)) & (WIN | (n_group == 0) | (shared == 0)));
  if (skip) return;
  typedef float vecf __attribute__((ext_vector_type(PER)));
  vecf num = {};
  float den;
  if (p1 - p0 <= kWave) {
    // One partition per lane: the max, the weights and the denominator come
    // from one load per lane, and the partial outputs of the live partitions
    // (a partition joined to an earlier one's work item holds no state: max
    // -inf, sum 0, output never written) are read four at a time, their loads
    // issued before any of them is used.
    const bool in = lane < p1 - p0;
    const float m_l = !in ? -__builtin_inff() : WIN ? a.ws_max[base + p0 + lane] : m_spec;
    const float s_l = !in ? 0.f : WIN ? a.ws_sum[base + p0 + lane] : s_spec;
    const float mu = safe_max(across_groups_max<1>(m_l));
    const float f_l = m_l == -__builtin_inff() ? 0.f : exp2_fast(m_l - mu);
    den = across_groups_sum<1>(f_l * s_l);
    uint64_t live = __builtin_amdgcn_ballot_w64(m_l != -__builtin_inff());
    while (live != 0) {  // wave-uniform
      int q[4];
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[i] = live != 0 ? __builtin_ctzll(live) : q[0];  // a live one again, weight 0
        f[i] = live != 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f_l), q[i])) : 0.f;
        live &= live - 1;
      }
      vecf v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = *reinterpret_cast<const vecf*>(a.ws_acc + (base + p0 + q[i]) * D + lane * PER);
#pragma unroll
      for (int i = 0; i < 4; ++i) num += f[i] * v[i];
    }
  } else {
    float mx = -__builtin_inff();
    for (int p = p0 + lane; p < p1; p += kWave) mx = fmaxf(mx, a.ws_max[base + p]);
    mx = across_groups_max<1>(mx);
    const float mu = safe_max(mx);
    den = 0.f;
    for (int p = p0 + lane; p < p1; p += kWave) den += exp2_fast(a.ws_max[base + p] - mu) * a.ws_sum[base + p];
    den = across_groups_sum<1>(den);
    for (int p = p0; p < p1; ++p) {
      const float m = a.ws_max[base + p];
      if (m == -__builtin_inff()) continue;  // a joined partition: no state
      num += exp2_fast(m - mu) * *reinterpret_cast<const vecf*>(a.ws_acc + (base + p) * D + lane * PER);
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    E::store(a.out, static_cast<int64_t>(row) * D + lane * PER + j, den == 0.f ? 0.f : num[j] / den);
}

template <typename E, int D, int GT>
hipError_t launch_partitions_gt(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_heads / a.num_kv_heads;
  const int chunks = (group + GT - 1) / GT;
  const uint64_t n = decode_grid(a, chunks);
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffffu) return hipErrorInvalidValue;
  // The window only moves this kernel's token range: no per-score form needed.
  if (a.softcap > 0.f)
    hipLaunchKernelGGL((decode_partition_kernel<E, D, GT, ScoreMap<true, false, true>>),
                       dim3(static_cast<uint32_t>(n)), dim3(kDecodeThreads), 0, stream, a, chunks,
                       make_score_map<true, false, true>(a.scale, a.softcap));
  else
    hipLaunchKernelGGL((decode_partition_kernel<E, D, GT, ScoreMap<false, false>>),
                       dim3(static_cast<uint32_t>(n)), dim3(kDecodeThreads), 0, stream, a, chunks,
                       make_score_map<false, false>(a.scale, a.softcap));
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_partitions_d(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_heads / a.num_kv_heads;
  switch (group < kMaxHeadsPerWg ? group : kMaxHeadsPerWg) {
    case 1: return launch_partitions_gt<E, D, 1>(a, stream);
    case 2: return launch_partitions_gt<E, D, 2>(a, stream);
    case 3: return launch_partitions_gt<E, D, 3>(a, stream);
    case 4: return launch_partitions_gt<E, D, 4>(a, stream);
    case 5: return launch_partitions_gt<E, D, 5>(a, stream);
    case 6: return launch_partitions_gt<E, D, 6>(a, stream);
    case 7: return launch_partitions_gt<E, D, 7>(a, stream);
    default: return launch_partitions_gt<E, D, 8>(a, stream);
  }
}

template <typename E>
hipError_t launch_partitions_e(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_partitions_d<E, 64>(a, stream);
    case 128: return launch_partitions_d<E, 128>(a, stream);
    default: return launch_partitions_d<E, 256>(a, stream);
  }
}

// Work plan: every non-empty work item, ordered longest first.  An item is a
// span of 1, 2 or 4 consecutive partitions of one sequence: always 1 unless
// a.plan_min_items > 0, and then the widest span of at most kSpanTokens
// tokens that still leaves a.plan_min_items items (each item costs the
// partition kernel a merge and a refill of its DMA pipeline).  The partial
// last items come after the full ones, in decreasing length, so the short
// ones fill the tail of the partition kernel instead of a long one starting
// last.  A counting sort over kPlanBuckets length classes (descending); the
// order inside a class is whatever the LDS atomics give, which changes only
// the dispatch order, never a result.  With a sliding window, a sequence's
// items start at the partition holding its first attended token, so
// partitions wholly before the window get no work at all.  One workgroup; it
// sits on the critical path of every decode call, so it reads each context
// length once.
//
// Shared partitions (a.share).  Sharing a prompt prefix means that several
// block tables name the same physical blocks (wLLM case study, ADR-001 on
// the KV-cache layout).  A partition whose blocks several sequences' tables
// name alike is then read once for all of them by a group item: the query
// rows of all its sequences (up to a.share_max_members per item) against the
// one stream of keys and values.  The search runs level by level from
// partition 0.  At level p, every sequence whose partitions 0..p-1 were
// shared, and whose partition p is full and not its last, hashes the
// partition's first block id into an LDS table; the smallest sequence with
// that id leads, and every other one whose whole partition (every block id)
// matches the leader's joins it.  Group items take the first plan positions;
// a member's own items start after its shared partitions, and the reduce
// merges its row.  Which sequences share a group item changes no result: the
// group path computes each query row on its own.
constexpr int kPlanThreads = 1024;  // the most threads; a launch uses plan_threads(num_seqs)
// Threads of one plan launch: one per sequence, in whole waves, at least 256
// (wave 0 scans the class histogram, the first 192 threads clear it).  Every
// wave runs every phase, so spare waves only add issue time (tinyllama's plan
// took 7.8 us with 1,024 threads for 64 sequences).
inline int plan_threads(int num_seqs) {
  const int t = (num_seqs + kWave - 1) / kWave * kWave;
  return t < 256 ? 256 : (t > kPlanThreads ? kPlanThreads : t);
}
constexpr int kPlanBuckets = 64;
constexpr int kSpanTokens = 2048;
constexpr int kPlanCtxCache = 8192;  // context lengths kept in LDS
constexpr int kShareHashBits = 12;
constexpr int kShareHash = 1 << kShareHashBits;  // twice the sequences searched: probes stay short
static_assert(kShareHash >= 2 * kShareMaxSeqs, "hash table load: the search sizes it to 2 S");
static_assert(kShareMaxSeqs <= kPlanCtxCache, "searched sequences keep their context in LDS");

template <bool WIN>
__device__ __forceinline__ void plan_body(const DecodeArgs& a) {
  __shared__ int hist[3][kPlanBuckets];  // per span choice 1, 2, 4
  __shared__ int s_ctx[kPlanCtxCache];
  __shared__ int s_tot[3];  // items per span choice
  // Shared-partition search (see above).
  __shared__ int h_key[kShareHash], h_lead[kShareHash], h_cnt[kShareHash];
  __shared__ int h_off[kShareHash], h_fill[kShareHash];
  __shared__ int s_qs[kShareMaxSeqs];    // leading partitions of a sequence that group items cover
  __shared__ int s_slot[kShareMaxSeqs];  // the sequence's hash slot at the current level, or -1
  __shared__ int s_key[kShareMaxSeqs];   // first block id of the partition searched
  __shared__ int s_key1[kShareMaxSeqs];  // and of the next partition, read ahead
  __shared__ int s_ngroup, s_nmem, s_more, s_hit;
  const int tid = threadIdx.x;
  const int nthr = static_cast<int>(blockDim.x);  // whole waves, >= 256
  const bool share = !WIN && a.share != 0;
  const int P = a.part_tokens;
  const int64_t mbps = a.max_blocks_per_seq;
  if (tid < 3 * kPlanBuckets) hist[tid / kPlanBuckets][tid % kPlanBuckets] = 0;
  if (tid == 0) {
    s_ngroup = 0;
    s_nmem = 0;
  }
  for (int s = tid; s < a.num_seqs; s += nthr) {
    // The context length and, for the search, the first block id: loads
    // issued together, one round trip.
    const int cl = a.context_lens[s];
    const int key = share ? a.block_tables[s * mbps] : 0;
    // Partition 1's first block id: a table entry whenever the table reaches
    // past partition 0 (checked against the context below).
    const int bpp0 = P >> a.log2_block_size;
    const int key1 = share && mbps > bpp0 ? a.block_tables[s * mbps + bpp0] : -1;
    const int c = max(0, min(cl, a.ctx_limit));
    if (s < kPlanCtxCache) s_ctx[s] = c;
    if (share) {
      s_qs[s] = 0;
      s_key[s] = key;
      s_key1[s] = key1;
    }
  }
  __syncthreads();

  if (share) {  // a.num_seqs <= kShareMaxSeqs, block_size <= P (host-checked)
    const int bpp = P >> a.log2_block_size;  // blocks per partition
    // Hash slots: the power of two >= twice the sequences (at least 64).
    int hbits = 6;
    while ((1 << hbits) < 2 * a.num_seqs) ++hbits;
    const int hsize = 1 << hbits;
    for (int p = 0; p + 1 < a.num_parts; ++p) {  // a shared partition is never a sequence's last
      for (int i = tid; i < hsize; i += nthr) {
        h_key[i] = -1;
        h_lead[i] = 0x7fffffff;
        h_cnt[i] = 0;
        h_fill[i] = 0;
      }
      if (tid == 0) {
        s_more = 0;
        s_hit = 0;
      }
      __syncthreads();
      for (int s = tid; s < a.num_seqs; s += nthr) {
        int slot = -1;
        const int key = s_key[s];
        if (s_qs[s] == p && s_ctx[s] > (p + 1) * P && key >= 0 && key < a.num_blocks) {
          slot = static_cast<int>((static_cast<uint32_t>(key) * 0x9E3779B1u) >> (32 - hbits));
          while (true) {  // at most a.num_seqs keys in twice as many slots
            const int old = atomicCAS(&h_key[slot], -1, key);
            if (old == -1) break;
            if (old == key) {
              s_hit = 1;  // another sequence starts the partition with this block
              break;
            }
            slot = (slot + 1) & (hsize - 1);
          }
          atomicMin(&h_lead[slot], s);
        }
        s_slot[s] = slot;
      }
      __syncthreads();
      if (s_hit == 0) break;  // no partition begins with another's block: nothing shared
      for (int s = tid; s < a.num_seqs; s += nthr) {
        const int slot = s_slot[s];
        if (slot < 0) continue;
        const int lead = h_lead[slot];
        if (lead == s) continue;
        // Compare the whole partition's block ids, the loads all in flight at
        // once (16-byte loads when the table rows allow them).
        const int32_t* mine = a.block_tables + s * mbps + p * bpp;
        const int32_t* theirs = a.block_tables + lead * mbps + p * bpp;
        int diff = 0;
        if (a.share_vec) {
          for (int i = 0; i < bpp; i += 4) {
            const int4 x = *reinterpret_cast<const int4*>(mine + i);
            const int4 y = *reinterpret_cast<const int4*>(theirs + i);
            diff |= (x.x ^ y.x) | (x.y ^ y.y) | (x.z ^ y.z) | (x.w ^ y.w);
          }
        } else {
          for (int i = 1; i < bpp; ++i) diff |= mine[i] ^ theirs[i];
        }
        if (diff == 0) atomicAdd(&h_cnt[slot], 1);
        else s_slot[s] = -1;  // first block alike, the rest not: read on its own
      }
      __syncthreads();
      for (int s = tid; s < a.num_seqs; s += nthr) {
        const int slot = s_slot[s];
        if (slot < 0 || h_lead[slot] != s || h_cnt[slot] == 0) continue;
        // A group's leader reserves its member run and its items: runs of
        // up to share_max_members sequences, the last one shorter.
        const int n = h_cnt[slot] + 1;
        const int off = atomicAdd(&s_nmem, n);
        const int nit = (n + a.share_max_members - 1) / a.share_max_members;
        const int first = atomicAdd(&s_ngroup, nit);
        h_off[slot] = off;
        for (int i = 0; i < nit; ++i) {
          const int cnt = min(a.share_max_members, n - i * a.share_max_members);
          a.plan[first + i] =
              make_int4(off + i * a.share_max_members, p, 1 | (1 << 9) | (cnt << 16), (p + 1) * P);
        }
      }
      __syncthreads();
      for (int s = tid; s < a.num_seqs; s += nthr) {
        const int slot = s_slot[s];
        if (slot < 0 || h_cnt[slot] == 0) continue;  // not shared at this level
        a.members[h_off[slot] + atomicAdd(&h_fill[slot], 1)] = s;
        s_qs[s] = p + 1;
        if (s_ctx[s] > (p + 2) * P) {  // the next level's key
          s_key[s] = p == 0 ? s_key1[s] : a.block_tables[s * mbps + (p + 1) * bpp];
          s_more = 1;
        }
      }
      __syncthreads();
      if (s_more == 0) break;
    }
    if (s_ngroup > 0)
      for (int s = tid; s < a.num_seqs; s += nthr) a.seq_shared[s] = s_qs[s];
  }
  const int ngroup = share ? s_ngroup : 0;

  // log2 of the widest span considered: at most 4 partitions, kSpanTokens
  // tokens and the partitions there are.
  int max_k = 0;
  if (a.plan_min_items > 0)
    while (max_k < 2 && (P << (max_k + 1)) <= kSpanTokens && (2 << max_k) <= a.num_parts) ++max_k;
  int shift[3] = {0, 0, 0};
  for (int k = 0; k <= max_k; ++k)
    while ((((P << k) - 1) >> shift[k]) >= kPlanBuckets) ++shift[k];
  auto ctx_of = [&](int s) {
    return s < kPlanCtxCache ? s_ctx[s] : max(0, min(a.context_lens[s], a.ctx_limit));
  };
  // A sequence's own items: spans of 2^k partitions from `base` (a partition
  // boundary: the partition holding the window's first token, the first one
  // after the shared ones, or 0), the attended tokens from `lo` on.  Every
  // span is full except, without a window, the last one and, with a window,
  // the first and the last; a sequence with an empty context still owns one
  // item, whose output rows are zeros.
  struct Own {
    int c, base, lo;
  };
  auto own = [&](int s) {
    Own o;
    o.c = ctx_of(s);
    if constexpr (WIN) {
      o.lo = window_start(a, o.c);
      o.base = o.lo - o.lo % P;
    } else {
      o.base = share ? s_qs[s] * P : 0;
      o.lo = o.base;
    }
    return o;
  };
  auto span_tokens = [&](const Own& o, int k, int slot) {
    if (slot == 0 && o.c == 0) return 1;
    const int first = o.base + slot * (P << k);
    return min(first + (P << k), o.c) - max(first, o.lo);
  };
  auto bucket = [&](int k, int t) { return kPlanBuckets - 1 - ((t - 1) >> shift[k]); };
  // A sequence's spans for span choice k: n of them, the first and the last
  // placed one by one, those between always full.
  auto n_spans = [&](const Own& o, int k) {
    return o.c == 0 ? 1 : (o.c - o.base + (P << k) - 1) / (P << k);
  };
  const int lane = tid & (kWave - 1);
  const int nloop = (a.num_seqs + nthr - 1) / nthr;  // whole waves in step

  // 1. Item counts of each span choice (wave sums, one atomic per wave).
  if (tid < 3) s_tot[tid] = 0;
  __syncthreads();
  for (int i = 0; i < nloop; ++i) {
    const int s = i * nthr + tid;
    const bool live = s < a.num_seqs;
    const Own o = own(live ? s : 0);
    for (int k = 1; k <= max_k; ++k) {
      int total;
      wave_scan(live ? n_spans(o, k) : 0, &total);
      if (lane == 0) atomicAdd(&s_tot[k], total);
    }
  }
  __syncthreads();
  int k = 0;  // the widest span that keeps plan_min_items items
  for (int kk = max_k; kk >= 1; --kk)
    if (s_tot[kk] + ngroup >= a.plan_min_items) {
      k = kk;
      break;
    }
  const int span = 1 << k;
  // 2. Histogram of the chosen spans' lengths.  Full spans all fall in the
  // top bucket (0): those are summed over the wave first.
  struct Spans {
    int n, b_first, b_last, top;  // b_last only when n >= 2; top: spans in bucket 0
  };
  auto spans = [&](const Own& o) {
    Spans x;
    x.n = n_spans(o, k);
    x.b_first = bucket(k, span_tokens(o, k, 0));
    x.b_last = x.n >= 2 ? bucket(k, span_tokens(o, k, x.n - 1)) : -1;
    x.top = (x.b_first == 0) + max(0, x.n - 2) + (x.b_last == 0);
    return x;
  };
  for (int i = 0; i < nloop; ++i) {
    const int s = i * nthr + tid;
    const bool live = s < a.num_seqs;
    const Spans x = spans(own(live ? s : 0));
    int total;
    wave_scan(live ? x.top : 0, &total);
    if (lane == 0 && total > 0) atomicAdd(&hist[k][0], total);
    if (live && x.b_first > 0) atomicAdd(&hist[k][x.b_first], 1);
    if (live && x.b_last > 0) atomicAdd(&hist[k][x.b_last], 1);
  }
  __syncthreads();
  static_assert(kPlanBuckets == kWave, "one bucket per lane of wave 0");
  if (tid < kWave) {
    // Wave 0, one bucket per lane: the exclusive prefix sum of the histogram
    // (the bucket offsets, after the group items).
    const int c = hist[k][tid];
    int tot;
    const int incl = wave_scan(c, &tot);
    hist[k][tid] = ngroup + incl - c;
    if (tid == 0) {
      *a.plan_count = ngroup + tot;
      a.plan_count[1] = k;  // log2 of the span, for the reduce
      a.plan_count[2] = 0;  // units taken from the partition kernel's queue
      a.plan_count[3] = ngroup;
    }
  }
  __syncthreads();
  // 3. The items, each at its bucket's next position; a wave's top-bucket
  // items take one run (one atomic), each lane its part by a prefix sum.
  const int64_t cap = static_cast<int64_t>(a.num_seqs) * a.num_parts;  // plan entries
  for (int i = 0; i < nloop; ++i) {
    const int s = i * nthr + tid;
    const bool live = s < a.num_seqs;
    const Own o = own(live ? s : 0);
    const Spans x = spans(o);
    int total;
    const int top = live ? x.top : 0;
    const int incl = wave_scan(top, &total);
    int run = 0;
    if (lane == 0 && total > 0) run = atomicAdd(&hist[k][0], total);
    run = __builtin_amdgcn_readlane(run, 0);
    if (!live) continue;
    int top_pos = run + incl - top;
    const int p0 = o.base / P;
    // One item covers the sequence: its output is final, and the reduce skips the row.
    const int single = (o.base == 0 || WIN) && o.c <= o.base + (P << k) ? 1 : 0;
    auto put = [&](int slot, int pos) {
      if (pos >= 0 && pos < cap) a.plan[pos] = make_int4(s, p0 + slot * span, span | (single << 8), o.c);
    };
    put(0, x.b_first == 0 ? top_pos++ : atomicAdd(&hist[k][x.b_first], 1));
    for (int slot = 1; slot < x.n - 1; ++slot) put(slot, top_pos++);
    if (x.n >= 2) put(x.n - 1, x.b_last == 0 ? top_pos++ : atomicAdd(&hist[k][x.b_last], 1));
  }
}

template <bool WIN>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a) {
  plan_body<WIN>(a);
}

// The step's new K/V rows for the plan-and-write launch (16-bit and fp32
// caches; a bit copy, as pa_reshape_and_cache).
struct WriteRows {
  const u32x4* key;
  const u32x4* value;
  u32x4* key_cache;
  u32x4* value_cache;
  const int64_t* slot_mapping;
  int64_t total;  // 16-byte items: tokens x KV heads x chunks per row
  int32_t chunks_per_row, num_kv_heads, log2_bs;
  int64_t num_slots;
};

// The plan and the step's cache write in one launch: neither reads what the
// other writes (the plan reads context lengths and block tables only), and
// the partition kernel after it sees both.  Workgroup 0 plans; the others
// copy the rows.  Every workgroup carries the plan's LDS, so each holds a CU.
template <bool WIN>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_write_kernel(DecodeArgs a, WriteRows w) {
  if (blockIdx.x == 0) {
    plan_body<WIN>(a);
    return;
  }
  copy_rows_to_cache(w.key, w.value, w.key_cache, w.value_cache, w.slot_mapping, w.total,
                     w.chunks_per_row, w.num_kv_heads, w.log2_bs, w.num_slots,
                     static_cast<int64_t>(blockIdx.x - 1) * blockDim.x + threadIdx.x,
                     static_cast<int64_t>(gridDim.x - 1) * blockDim.x);
}

template <typename E, bool WIN>
hipError_t launch_reduce_w(const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + kWaves - 1) / kWaves));
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL((decode_reduce_kernel<E, 64, WIN>), grid, dim3(kDecodeThreads), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((decode_reduce_kernel<E, 128, WIN>), grid, dim3(kDecodeThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_reduce_kernel<E, 256, WIN>), grid, dim3(kDecodeThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_reduce_e(const DecodeArgs& a, hipStream_t stream) {
  return a.window > 0 ? launch_reduce_w<E, true>(a, stream) : launch_reduce_w<E, false>(a, stream);
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

DecodeWorkspace decode_workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t num_parts) {
  DecodeWorkspace w{};
  if (num_seqs <= 0) return w;
  size_t off = 0;
  if (num_parts > 1) {
    const size_t n = static_cast<size_t>(num_seqs) * num_heads * num_parts;
    w.off_max = 0;
    w.off_sum = align256(n * sizeof(float));
    w.off_acc = w.off_sum + align256(n * sizeof(float));
    off = w.off_acc + align256(n * head_dim * sizeof(float));
  }
  w.off_count = off;
  w.off_plan = off + 256;
  const size_t items = static_cast<size_t>(num_seqs) * std::max(num_parts, 1);
  w.bytes = w.off_plan + align256(items * sizeof(int4));
  if (num_parts > 1) {
    w.off_shared = w.bytes;
    w.off_members = w.off_shared + align256(static_cast<size_t>(num_seqs) * sizeof(int32_t));
    w.bytes = w.off_members + align256(items * sizeof(int32_t));
  }
  return w;
}

// PA_DECODE_KERNEL=vector in the environment (read once): 16-bit caches go
// through the vector kernel too, the baseline the MFMA kernel is measured
// against (same results within the 16-bit tolerance; E4M3 caches always take
// the MFMA kernel).
static bool vector_kernel_forced() {
  static const bool forced = [] {
    const char* e = std::getenv("PA_DECODE_KERNEL");
    return e != nullptr && std::strcmp(e, "vector") == 0;
  }();
  return forced;
}

hipError_t launch_decode_partitions(const DecodeArgs& args, hipStream_t stream) {
  return launch_decode_partitions_write(args, nullptr, stream);
}

hipError_t launch_decode_partitions_write(const DecodeArgs& args, const CacheWriteArgs* write,
                                          hipStream_t stream) {
  if (args.num_seqs <= 0) return write ? launch_reshape_and_cache(*write, stream) : hipSuccess;
  DecodeArgs a = args;
  const bool mfma = a.dtype != PA_DTYPE_F32 && (a.kv_fp8 || !vector_kernel_forced());
  a.plan_min_items = 0;
  a.share = 0;
  a.static_plan = 0;
  if (mfma) {
    const int group = a.num_heads / a.num_kv_heads;
    // Shared partitions: whole contexts, one head chunk per KV head, blocks
    // of 16+ tokens (one scalar table read per pass); E4M3 caches only at
    // head_dim 128 (the kernel's only E4M3 form with a group path).
    a.share = (a.window == 0 && group <= 16 && a.num_seqs >= 2 && (!a.kv_fp8 || a.head_dim == 128) &&
               a.num_seqs <= kShareMaxSeqs && a.num_parts > 1 && a.log2_block_size >= 4 &&
               a.seq_shared != nullptr && a.members != nullptr) ? 1 : 0;
    a.share_max_members = decode_group_rows(a.head_dim) / group;
    // The search compares a partition's block ids 16 bytes at a time when
    // every table row's partitions start 16-byte aligned.
    const int bpp = a.part_tokens >> a.log2_block_size;
    a.share_vec = (reinterpret_cast<uintptr_t>(a.block_tables) % 16 == 0 && a.max_blocks_per_seq % 4 == 0 &&
                   bpp % 4 == 0) ? 1 : 0;
  }
  if (mfma) {
    // Small calls: when every (sequence, partition, head chunk) slot has a
    // workgroup of the persistent grid, each workgroup takes the slot its
    // index names (empty ones exit at once), and the plan launch -- a third
    // of such a call -- is left out.  No spans are joined and no shared
    // partitions are looked for; the counts the reduce reads (one partition
    // per item, no group items) are written by the partition kernel.
    const int group = a.num_heads / a.num_kv_heads;
    const uint64_t slots = decode_grid(a, (group + 15) / 16);
    DecodeArgs st = a;  // the grid of the kernel a static launch takes (no group path)
    st.static_plan = 1;
    a.static_plan = slots <= static_cast<uint64_t>(decode_mfma_grid(st)) ? 1 : 0;
    if (!a.static_plan) {
      // Join partitions while every persistent workgroup still gets a unit.
      const int per = a.num_kv_heads * ((group + 15) / 16);
      a.plan_min_items = std::max(1, (decode_mfma_grid(a) + per - 1) / per);
    }
  }
  const int pthreads = plan_threads(a.num_seqs);
  WriteRows wr{};
  if (write) {
    wr.key = static_cast<const u32x4*>(write->key);
    wr.value = static_cast<const u32x4*>(write->value);
    wr.key_cache = static_cast<u32x4*>(write->key_cache);
    wr.value_cache = static_cast<u32x4*>(write->value_cache);
    wr.slot_mapping = write->slot_mapping;
    wr.chunks_per_row = write->head_dim * write->elem_bytes / 16;
    wr.num_kv_heads = write->num_kv_heads;
    wr.log2_bs = write->log2_block_size;
    wr.num_slots = static_cast<int64_t>(write->num_blocks) << write->log2_block_size;
    wr.total = static_cast<int64_t>(write->num_tokens) * write->num_kv_heads * wr.chunks_per_row;
  }
  if (a.static_plan) {
    if (write) {  // no plan to share a launch with
      const hipError_t e = launch_reshape_and_cache(*write, stream);
      if (e != hipSuccess) return e;
    }
  } else {
    if (wr.total > 0) {
      // One copying workgroup per CU at most besides the planner (each holds a CU's LDS).
      const int64_t need = (wr.total + pthreads - 1) / pthreads;
      const unsigned copiers = static_cast<unsigned>(std::min<int64_t>(need, 255));
      if (a.window > 0)
        hipLaunchKernelGGL(decode_plan_write_kernel<true>, dim3(1 + copiers), dim3(pthreads), 0, stream, a, wr);
      else
        hipLaunchKernelGGL(decode_plan_write_kernel<false>, dim3(1 + copiers), dim3(pthreads), 0, stream, a, wr);
    } else if (a.window > 0) {
      hipLaunchKernelGGL(decode_plan_kernel<true>, dim3(1), dim3(pthreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL(decode_plan_kernel<false>, dim3(1), dim3(pthreads), 0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mfma) return launch_decode_mfma(a, stream);
  switch (a.dtype) {
    case PA_DTYPE_F16: return launch_partitions_e<F16>(a, stream);
    case PA_DTYPE_BF16: return launch_partitions_e<BF16>(a, stream);
    default: return launch_partitions_e<F32>(a, stream);
  }
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_parts <= 1) return hipSuccess;
  if (a.plan_count == nullptr || a.ws_max == nullptr || a.ws_sum == nullptr || a.ws_acc == nullptr ||
      a.seq_shared == nullptr)
    return hipErrorInvalidValue;  // the kernel reads the plan's span and the partial states
  switch (a.dtype) {
    case PA_DTYPE_F32: return launch_reduce_e<F32>(a, stream);
    case PA_DTYPE_F16: return launch_reduce_e<F16>(a, stream);
    default: return launch_reduce_e<BF16>(a, stream);
  }
}

}  // namespace pa

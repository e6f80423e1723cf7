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
  const int ctx = max(0, min(a.context_lens[seq], a.ctx_limit));
  if (ctx == 0) return;
  // Partitions holding the attended tokens (the window's, or all of them).
  const int p0 = WIN ? window_start(a, ctx) / a.part_tokens : 0;
  const int p1 = (ctx - 1) / a.part_tokens + 1;
  // Rows whose partitions fit one work item were written by the partition kernel.
  if (p1 - p0 <= (1 << a.plan_count[1])) return;
  const int64_t base = static_cast<int64_t>(row) * a.num_parts;
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
    const float m_l = in ? a.ws_max[base + p0 + lane] : -__builtin_inff();
    const float s_l = in ? a.ws_sum[base + p0 + lane] : 0.f;
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
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 64;
constexpr int kSpanTokens = 2048;
constexpr int kPlanCtxCache = 8192;  // context lengths kept in LDS

template <bool WIN>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a) {
  __shared__ int hist[3][kPlanBuckets];  // per span choice 1, 2, 4
  __shared__ int s_ctx[kPlanCtxCache];
  __shared__ int s_span;
  const int tid = threadIdx.x;
  if (tid < 3 * kPlanBuckets) hist[tid / kPlanBuckets][tid % kPlanBuckets] = 0;
  __syncthreads();

  const int P = a.part_tokens;
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
  // Tokens of span slot `slot` (2^k partitions, counted from the partition
  // that holds the first attended token `lo`, which starts at token `base`) of
  // a sequence; a sequence with an empty context still owns one item, whose
  // output rows are zeros.
  auto span_tokens = [&](int c, int lo, int base, int k, int slot) {
    if (slot == 0 && c == 0) return 1;
    if constexpr (!WIN) return min(P << k, c - slot * (P << k));
    const int first = base + slot * (P << k);
    return min(first + (P << k), c) - max(first, lo);
  };
  auto first_part_token = [&](int lo) { return lo > 0 ? lo - lo % P : 0; };
  for (int s = tid; s < a.num_seqs; s += kPlanThreads) {
    const int c = max(0, min(a.context_lens[s], a.ctx_limit));
    if (s < kPlanCtxCache) s_ctx[s] = c;
    const int lo = WIN ? window_start(a, c) : 0;
    const int base = WIN ? first_part_token(lo) : 0;
    for (int k = 0; k <= max_k; ++k)
      for (int slot = 0;; ++slot) {
        const int t = span_tokens(c, lo, base, k, slot);
        if (t <= 0) break;
        atomicAdd(&hist[k][kPlanBuckets - 1 - ((t - 1) >> shift[k])], 1);
      }
  }
  __syncthreads();
  static_assert(kPlanBuckets == kWave, "one bucket per lane of wave 0");
  if (tid < kWave) {
    // Wave 0, one bucket per lane: item counts per span, then the exclusive
    // prefix sum of the chosen span's histogram (the bucket offsets).
    int k_use = 0;
    for (int k = max_k; k >= 1; --k) {
      int items = hist[k][tid];
      for (int off = 1; off < kWave; off <<= 1) items += __shfl_xor(items, off, kWave);
      if (items >= a.plan_min_items) {
        k_use = k;
        break;
      }
    }
    const int c = hist[k_use][tid];
    int incl = c;
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off, kWave);
      if (tid >= off) incl += v;
    }
    hist[k_use][tid] = incl - c;
    if (tid == kWave - 1) {
      *a.plan_count = incl;
      a.plan_count[1] = k_use;  // log2 of the span, for the reduce
      a.plan_count[2] = 0;      // units taken from the partition kernel's queue
      s_span = k_use;
    }
  }
  __syncthreads();
  const int k = s_span;
  const int span = 1 << k;
  for (int s = tid; s < a.num_seqs; s += kPlanThreads) {
    const int c = ctx_of(s);
    const int lo = WIN ? window_start(a, c) : 0;
    const int base = WIN ? first_part_token(lo) : 0;
    const int p0 = base > 0 ? base / P : 0;
    // One item covers the sequence: its output is final, and the reduce skips the row.
    const int single = c <= base + (P << k) ? 1 : 0;
    for (int slot = 0;; ++slot) {
      const int t = span_tokens(c, lo, base, k, slot);
      if (t <= 0) break;
      const int pos = atomicAdd(&hist[k][kPlanBuckets - 1 - ((t - 1) >> shift[k])], 1);
      a.plan[pos] = make_int4(s, p0 + slot * span, span | (single << 8), c);
    }
  }
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
  w.bytes = w.off_plan + align256(static_cast<size_t>(num_seqs) * std::max(num_parts, 1) * sizeof(int4));
  return w;
}

hipError_t launch_decode_partitions(const DecodeArgs& args, hipStream_t stream) {
  if (args.num_seqs <= 0) return hipSuccess;
  DecodeArgs a = args;
  const bool mfma = a.dtype != PA_DTYPE_F32;
  a.plan_min_items = 0;
  if (mfma) {
    // Join partitions while every persistent workgroup still gets two units.
    const int group = a.num_heads / a.num_kv_heads;
    const int per = a.num_kv_heads * ((group + 15) / 16);
    a.plan_min_items = std::max(1, (2 * decode_mfma_grid(a) + per - 1) / per);
  }
  if (a.window > 0)
    hipLaunchKernelGGL(decode_plan_kernel<true>, dim3(1), dim3(kPlanThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_plan_kernel<false>, dim3(1), dim3(kPlanThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mfma) return launch_decode_mfma(a, stream);
  return launch_partitions_e<F32>(a, stream);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_parts <= 1) return hipSuccess;
  if (a.plan_count == nullptr || a.ws_max == nullptr || a.ws_sum == nullptr || a.ws_acc == nullptr)
    return hipErrorInvalidValue;  // the kernel reads the plan's span and the partial states
  switch (a.dtype) {
    case PA_DTYPE_F32: return launch_reduce_e<F32>(a, stream);
    case PA_DTYPE_F16: return launch_reduce_e<F16>(a, stream);
    default: return launch_reduce_e<BF16>(a, stream);
  }
}

}  // namespace pa

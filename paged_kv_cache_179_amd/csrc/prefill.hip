// Chunked-prefill paged attention for gfx950 (MFMA).
//
// A chunk of L prompt tokens at the end of a context of C cached tokens attends
// the context before it and itself causally: row i sits at position C - L + i
// and sees keys 0 .. C - L + i.  Chunked prefill is listed on the wLLM PyPI
// page ("Features -- Core engine"; long prompts are split so they do not stall
// other requests' decode); the GQA mapping is the mini-vLLM one (each query
// head reads its own KV head).
//
// A tile of query rows makes both products dense, so both run on the matrix
// cores (v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulate):
//
// * A workgroup has 128 query rows: 4 waves x 32 rows (8 waves x 16 rows at
//   head_dim 256).  Rows are (position, head) pairs of one KV head,
//   head-minor, so the G query heads that share a KV head share every K/V tile
//   (for MQA, 16 positions x 8 heads).  A wave's rows are 16-row MFMA tiles;
//   their query rows stay in registers.
// * Keys go by passes of 32.  Each pass's K and V rows are copied HBM -> LDS by
//   the gfx950 global-to-LDS DMA, an equal share of the rows by every wave
//   (the block's rows a wave-uniform base, each lane adding a 32-bit offset),
//   into one of three buffers (four at head_dim 256): the next passes are in
//   flight while one is computed.
//   Rows are stored with their 16-byte chunks rotated (K by the row, V by twice
//   the row) so that the compute reads below are bank-conflict free.
// * Scores, transposed: S^T = K Q^T (keys x rows).  Lane l of the accumulator
//   holds row l % 16's scores of keys 4 (l / 16) + 0..3 of each 16-key half,
//   so the row max of the online softmax is one in-lane max and two lane swaps.
// * O^T += V^T P^T with the 32 keys of the pass as the contraction: the score
//   registers (exp2, rounded to the input type) are already P^T's operand once
//   the key order inside the pass is taken as (first half's 4 keys, second
//   half's 4 keys) per lane; V^T's operand, in the same key order, comes from
//   two transposing LDS reads (ds_read_b64_tr_b16).  One more MFMA against a
//   ones operand sums the rounded probabilities (the softmax denominator).
// * The keys of a chunk are split in ranges of kSplitKeys so that long contexts
//   spread over several workgroups; each range writes an (m, l, acc) partial
//   per row and prefill_merge_kernel combines them by log-sum-exp weights, as
//   the decode reduce does.  Rows whose keys fit one range are written directly.
//
// Scores are kept in log2 units (scale * log2 e folded in): one v_exp_f32 per
// probability.  The running max is only moved when a score passes it by 2^8.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMergeWaves = 4;  // merge kernel: rows (one per wave) per workgroup
constexpr int kRowsPerWg = 128;  // query rows sharing each K/V tile
// 16-row MFMA tiles per wave: two, except at head_dim 256 where one keeps a
// wave's registers (accumulators 16 x 256 fp32 per tile) low enough for two
// waves per SIMD; a workgroup then has 8 waves.
constexpr int prefill_row_tiles(int head_dim) { return head_dim == 256 ? 1 : 2; }
constexpr int prefill_threads(int head_dim) { return kRowsPerWg / (16 * prefill_row_tiles(head_dim)) * 64; }
constexpr int kKeyTile = 32;  // keys per pass
// Head dims whose prefill launch is persistent (see prefill_kernel).
template <int D>
constexpr bool kPersistentPrefill = D == 256;
constexpr int kSplitKeys = 1024;
constexpr float kLazyMax = 8.f;

template <typename E>
struct Mma;
template <>
struct Mma<BF16> {
  static constexpr unsigned kOnePair = 0x3F803F80u;
  __device__ static inline f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline unsigned pack(float lo, float hi) {
    const bf16x2 r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(unsigned, r);
  }
  // Two E4M3 values (low or high half of w) as an exact bf16 pair.
  template <bool HIGH>
  __device__ static inline unsigned from_fp8(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HIGH));
  }
};
template <>
struct Mma<F16> {
  static constexpr unsigned kOnePair = 0x3C003C00u;
  __device__ static inline f32x4 run(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline unsigned pack(float lo, float hi) {
    const f16x2 r = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(unsigned, r);
  }
  // Two E4M3 values as an exact fp16 pair.
  template <bool HIGH>
  __device__ static inline unsigned from_fp8(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HIGH));
  }
};

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (each swap hands a lane its own
// value and its partner's, in some order).
__device__ inline float max_across_rows(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// The chunk, row tile and key range of one item, and the keys its rows see.
struct PrefillItem {
  int q_begin, qlen, ctx, pos0, npos, last_key, key_lo, key_hi;
  bool valid;
};

// From the chunk's query_start_loc entries and context length as given.
__device__ inline PrefillItem prefill_item_at(const PrefillArgs& a, int qsl_begin, int qsl_end, int context_len,
                                              int tile, int split, int pos_per_tile) {
  PrefillItem it{};
  it.q_begin = min(max(qsl_begin, 0), a.num_q_tokens);
  const int q_end = min(max(qsl_end, it.q_begin), a.num_q_tokens);
  it.ctx = max(0, min(context_len, a.ctx_limit));
  it.qlen = min(q_end - it.q_begin, it.ctx);
  it.pos0 = tile * pos_per_tile;
  it.valid = it.qlen > 0 && it.pos0 < it.qlen;
  if (!it.valid) return it;
  it.npos = min(pos_per_tile, it.qlen - it.pos0);
  it.last_key = it.ctx - it.qlen + it.pos0 + it.npos - 1;  // last key any row of the tile sees
  // First key any row sees: the window start of the tile's first row.  The
  // range starts on a pass boundary (keys below the window are masked).
  const int first_key = a.window > 0 ? max(0, it.ctx - it.qlen + it.pos0 - a.window + 1) : 0;
  const int split_lo = split * kSplitKeys;
  it.key_lo = max(split_lo, first_key & ~(kKeyTile - 1));
  it.valid = split_lo <= it.last_key && split_lo + kSplitKeys > first_key;
  it.key_hi = min(split_lo + kSplitKeys, it.last_key + 1);
  return it;
}

__device__ inline PrefillItem prefill_item(const PrefillArgs& a, int seq, int tile, int split,
                                           int pos_per_tile) {
  return prefill_item_at(a, a.query_start_loc[seq], a.query_start_loc[seq + 1], a.context_lens[seq], tile,
                         split, pos_per_tile);
}

// Work plan of one prefill call: every (chunk, row tile, key range) item that
// has keys, longest key range first (a counting sort over 64 classes), so the
// dispatcher starts the long items first and fills the tail with short ones.
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 64;

constexpr int kPlanSeqCache = 4096;  // chunks whose bounds and context lengths the plan keeps in LDS

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillArgs a, int32_t pos_per_tile,
                                                                   int32_t ntiles, int32_t nsplit,
                                                                   int4* plan, int32_t* plan_count,
                                                                   int32_t* tok_lim) {
  __shared__ int hist[kPlanBuckets];
  __shared__ int s_qs[kPlanSeqCache];  // query_start_loc as given
  __shared__ int s_cl[kPlanSeqCache];  // context_lens as given
  __shared__ int s_off[kPlanSeqCache];  // first row tile of each chunk among all chunks' tiles
  __shared__ int s_wsum[kPlanThreads / kWave];
  const int tid = threadIdx.x;
  const int S = a.num_seqs;
  if (tid < kPlanBuckets) hist[tid] = 0;
  // Every chunk's bounds and context length, read once (the item loops below
  // visit each chunk ntiles * nsplit times).
  const bool cached = S + 1 <= kPlanSeqCache;
  if (cached) {
    for (int s = tid; s <= S; s += kPlanThreads) {
      s_qs[s] = a.query_start_loc[s];
      if (s < S) s_cl[s] = a.context_lens[s];
    }
  }
  __syncthreads();
  // For the merge kernel (only when key ranges are split): the last key of
  // every query token's rows when those keys span more than one range, else
  // -1 (tokens outside every chunk or past its attended rows, and rows whose
  // keys fit one range, which the prefill kernel writes itself).
  if (tok_lim != nullptr) {
    auto start = [&](int s) { return min(max(cached ? s_qs[s] : a.query_start_loc[s], 0), a.num_q_tokens); };
    // Token t of chunk s.
    auto lim = [&](int s, int t) {
      const int q_begin = start(s);
      const int q_end = max(q_begin, start(s + 1));
      const int ctx = max(0, min(cached ? s_cl[s] : a.context_lens[s], a.ctx_limit));
      const int qlen = min(q_end - q_begin, ctx);
      const int pos = t - q_begin;
      if (pos >= qlen) return -1;
      const int row_lim = ctx - qlen + pos;
      const int p0 = a.window > 0 ? max(0, row_lim - a.window + 1) / kSplitKeys : 0;
      return row_lim / kSplitKeys + 1 - p0 > 1 ? row_lim : -1;
    };
    if (cached) {
      for (int t = tid; t < a.num_q_tokens; t += kPlanThreads) {
        if (t < start(0) || t >= start(S)) {
          tok_lim[t] = -1;
          continue;
        }
        // The last chunk whose start is <= t (the starts do not decrease).
        int lo = 0, hi = S;  // start(lo) <= t < start(hi)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (start(mid) <= t) lo = mid; else hi = mid;
        }
        tok_lim[t] = lim(lo, t);
      }
    } else {
      for (int t = tid; t < a.num_q_tokens; t += kPlanThreads) tok_lim[t] = -1;
      __syncthreads();
      for (int s = tid; s < S; s += kPlanThreads) {
        const int b = start(s), e = max(b, start(s + 1));
        for (int t = b; t < e; ++t) tok_lim[t] = lim(s, t);
      }
    }
  }
  __syncthreads();
  static_assert((kSplitKeys - 1) >> 4 < kPlanBuckets, "one class per 16 keys");
  // Items by (chunk, row tile) pair, one pair per thread: a pair past its
  // chunk's rows has none, the others one per key range their rows reach.
  // Items of a whole range (the top class) are counted and placed per wave
  // (one LDS atomic per wave), the rest one by one.
  const int lane = tid & (kWave - 1);
  // With the chunks in LDS, only the row tiles that hold rows are visited:
  // chunk s has ceil(rows / pos_per_tile) of them (at most ntiles), and
  // s_off is their exclusive prefix sum (thread t sums chunks 4t .. 4t + 3).
  int npairs = S * ntiles;  // < 2^31 (host-checked)
  if (cached) {
    static_assert(kPlanSeqCache == 4 * kPlanThreads, "four chunks per thread");
    int nt[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sq = 4 * tid + j;
      nt[j] = 0;
      if (sq < S) {
        const int qb = min(max(s_qs[sq], 0), a.num_q_tokens);
        const int qe = min(max(s_qs[sq + 1], qb), a.num_q_tokens);
        const int rows = min(qe - qb, max(0, min(s_cl[sq], a.ctx_limit)));
        nt[j] = rows > 0 ? min(ntiles, (rows + pos_per_tile - 1) / pos_per_tile) : 0;
      }
      sum += nt[j];
    }
    int wtotal;
    const int incl = wave_scan(sum, &wtotal);
    if (lane == 0) s_wsum[tid / kWave] = wtotal;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / kWave; ++w) {
      before += w < tid / kWave ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
    int off = before + incl - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sq = 4 * tid + j;
      if (sq < S) s_off[sq] = off;
      off += nt[j];
    }
    npairs = total;
    __syncthreads();
  }
  auto bucket = [](int t) { return kPlanBuckets - 1 - ((t - 1) >> 4); };
  struct Pair {
    int seq, tile, s_lo, s_hi;  // key ranges s_lo .. s_hi (none when s_hi < s_lo)
    int key_lo, key_end;        // the keys the tile's rows see: key_lo (a pass boundary) .. key_end - 1
  };
  auto pair_of = [&](int pr) {
    Pair x{};
    x.s_lo = 0;
    x.s_hi = -1;
    if (pr >= npairs) return x;
    if (cached) {  // the last chunk whose first tile is <= pr
      int lo = 0, hi = S;  // s_off[lo] <= pr < s_off[hi] (s_off[S] taken as npairs)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= pr) lo = mid; else hi = mid;
      }
      x.seq = lo;
      x.tile = pr - s_off[lo];
    } else {
      x.seq = pr / ntiles;
      x.tile = pr - x.seq * ntiles;
    }
    const int qb = cached ? s_qs[x.seq] : a.query_start_loc[x.seq];
    const int qe = cached ? s_qs[x.seq + 1] : a.query_start_loc[x.seq + 1];
    const int cl = cached ? s_cl[x.seq] : a.context_lens[x.seq];
    const PrefillItem it = prefill_item_at(a, qb, qe, cl, x.tile, 0, pos_per_tile);
    if (it.qlen <= 0 || it.pos0 >= it.qlen) return x;  // no rows in this tile
    const int first_key = a.window > 0 ? max(0, it.ctx - it.qlen + it.pos0 - a.window + 1) : 0;
    x.s_lo = first_key / kSplitKeys;
    x.s_hi = it.last_key / kSplitKeys;
    x.key_lo = first_key & ~(kKeyTile - 1);
    x.key_end = it.last_key + 1;
    return x;
  };
  // Keys of item (x, split), split in s_lo .. s_hi: the key range of
  // prefill_item_at, from the pair's bounds.
  auto keys_of = [&](const Pair& x, int split) {
    return min((split + 1) * kSplitKeys, x.key_end) - max(split * kSplitKeys, x.key_lo);
  };
  for (int p0 = 0; p0 < npairs; p0 += kPlanThreads) {  // uniform trip count: whole waves
    const Pair x = pair_of(p0 + tid);
    int top = 0;
    for (int sp = x.s_lo; sp <= x.s_hi; ++sp) {
      const int t = keys_of(x, sp);
      if (t <= 0) continue;
      if (bucket(t) == 0) ++top;
      else atomicAdd(&hist[bucket(t)], 1);
    }
    int wtop;
    wave_scan(top, &wtop);
    if (lane == 0 && wtop > 0) atomicAdd(&hist[0], wtop);
  }
  __syncthreads();
  static_assert(kPlanBuckets == kWave, "one class per lane of wave 0");
  if (tid < kWave) {  // wave 0: the classes' offsets (exclusive prefix sum)
    const int c = hist[tid];
    int total;
    const int incl = wave_scan(c, &total);
    hist[tid] = incl - c;
    if (tid == 0) *plan_count = total;
  }
  __syncthreads();
  for (int p0 = 0; p0 < npairs; p0 += kPlanThreads) {
    const Pair x = pair_of(p0 + tid);
    int top = 0;
    for (int sp = x.s_lo; sp <= x.s_hi; ++sp) {
      const int t = keys_of(x, sp);
      if (t > 0 && bucket(t) == 0) ++top;
    }
    // This lane's top-class items go to base + (the top items of the lanes
    // below it) + 0, 1, ...
    int wtop;
    const int below = wave_scan(top, &wtop);  // inclusive
    int base = 0;
    if (lane == 0 && wtop > 0) base = atomicAdd(&hist[0], wtop);
    int pos_top = __builtin_amdgcn_readfirstlane(base) + below - top;
    for (int sp = x.s_lo; sp <= x.s_hi; ++sp) {
      const int t = keys_of(x, sp);
      if (t <= 0) continue;
      const int pos = bucket(t) == 0 ? pos_top++ : atomicAdd(&hist[bucket(t)], 1);
      plan[pos] = make_int4(x.seq, x.tile, sp, t);
    }
  }
}

// FUSED: the chunk's own K/V come from the call's new rows (a.fused), a
// compile-time choice so that calls without it carry none of its code in the
// pass loop (the Gemma chunks' prefill kernel 61.4-61.8 -> 59.9-60.0 us).
template <typename E, int D, typename S, bool KV8, bool FUSED>
__global__ __launch_bounds__(prefill_threads(D)) void prefill_kernel(PrefillArgs a, int32_t group,
                                                          int32_t pos_per_tile, int32_t nsplit,
                                                          const int4* plan, const int32_t* plan_count,
                                                          S score, float* ws_max,
                                                          float* ws_sum, float* ws_acc) {
  static_assert(!(KV8 && FUSED), "the fused write takes 16-bit caches");
  using M = Mma<E>;
  constexpr int NC = D / 8;             // 16-byte chunks per row
  constexpr int RB = 2 * D;             // row bytes
  constexpr int RPI = 1024 / RB;        // rows per DMA instruction
  constexpr int NTW = prefill_row_tiles(D);  // row tiles per wave
  constexpr int WAVES = prefill_threads(D) / 64;
  constexpr int RPW = 16 * NTW;              // rows per wave
  // Waves that issue the DMA: all of them, each for an equal share of the
  // keys.  (With only the first four of eight issuing, those waves reached
  // each pass's barrier about a third of a pass after the other four; spread
  // over all eight, the Gemma chunks' prefill ran 2-3% faster.)
  constexpr int DW = WAVES;
  constexpr int WKEYS = kKeyTile / DW;       // keys each of them copies per pass
  static_assert(KV8 || WKEYS % RPI == 0, "a wave copies whole DMA instructions");
  // Cached rows: 2 D bytes (16-bit) or D bytes (E4M3, converted in LDS into
  // the 16-bit tile the MFMAs read).
  constexpr int CNC = KV8 ? NC / 2 : NC;                 // 16-byte chunks per cached row
  constexpr int NDK = (WKEYS * CNC + 63) / 64;          // DMA instructions per issuing wave per pass, K or V
  constexpr int NDW = 2 * NDK;                          // ... K and V
  constexpr int KB = D / 32;            // k-steps of the score product
  constexpr int MT = D / 16;            // 16-dim output tiles
  // [buffer][K or V][key][chunk]; NBUF - 1 passes in flight ahead of the one
  // computed (at head_dim 256 the 8-wave workgroup has the CU to itself).
  constexpr int NBUF = D == 256 ? 4 : 3;
  // K tiles and V tiles, each at an address known when the kernel is built:
  // a pass reads its operands at a lane offset plus a constant.
  __shared__ u32x4 s_k[NBUF][kKeyTile][CNC];
  __shared__ u32x4 s_v[NBUF][kKeyTile][CNC];
  __shared__ u32x4 s_cv[KV8 ? 2 : 1][kKeyTile][KV8 ? NC : 1];  // converted pass (E4M3 caches)

  // At head_dim 256 (one 8-wave workgroup per CU) the launch is persistent:
  // workgroup b takes the plan's units (item, KV head) b, then 2G - 1 - b, then
  // 2G + b, ... (G workgroups).  The plan is longest first, so the workgroups
  // that drew the shortest units of one round draw the longest of the next;
  // one workgroup per unit left the last units waiting for the hardware to
  // hand them a CU well after others had gone idle.  At smaller head dims,
  // where several workgroups share a CU, one workgroup per unit is faster (the
  // loop costs registers and so occupancy there).
  const int n_units = *plan_count * a.num_kv_heads;
  auto run_unit = [&](const int unit) {
    const int j = unit / a.num_kv_heads;
    const int kvh = unit - j * a.num_kv_heads;
    const int4 pi = plan[j];
    const int seq = pi.x, split = pi.z;
    const PrefillItem item = prefill_item(a, seq, pi.y, split, pos_per_tile);
    if (!item.valid) return;
    const int q_begin = item.q_begin, ctx = item.ctx, qlen = item.qlen, pos0 = item.pos0;
    const int npos = item.npos, last_key = item.last_key, key_lo = item.key_lo, key_hi = item.key_hi;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane & 15;
    const int g4 = lane >> 4;

    // This lane's query rows (one per 16-row tile of the wave): the keys
    // row_lo .. row_lim it attends (row_lo <= 0 without a window).
    int row_lim[NTW], row_lo[NTW], rpos[NTW], rhead[NTW];
    bool row_ok[NTW];
    const int win = a.window > 0 ? a.window : 0x40000000;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int row = wave * RPW + 16 * t + hl;
      rpos[t] = row / group;
      rhead[t] = row - rpos[t] * group;
      row_ok[t] = rpos[t] < npos;
      row_lim[t] = row_ok[t] ? ctx - qlen + pos0 + rpos[t] : -1;
      row_lo[t] = row_lim[t] - win + 1;
    }
    // The same bounds as seen from this lane's first key of a pass (4 g4):
    // lane_lim also stops at the range's end.
    int lane_lim[NTW], lane_lo[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      lane_lim[t] = min(row_lim[t], key_hi - 1) - 4 * g4;
      lane_lo[t] = row_lo[t] - 4 * g4;
    }
    // Keys any row of this wave sees (wave-uniform): passes outside are skipped.
    const int wave_last = min(last_key, ctx - qlen + pos0 + min(npos - 1, (wave * RPW + RPW - 1) / group));
    const int wave_first = ctx - qlen + pos0 + (wave * RPW) / group - win + 1;
    // Passes whose 32 keys every row of the wave sees need no mask: keys up to
    // the smallest row limit, from the largest window start, below key_hi.
    // (Rows past the chunk see no key when masked; unmasked they score zeros
    // against their zero query and are never written.)
    const int wave_min_lim = ctx - qlen + pos0 + (wave * RPW) / group;
    const int wave_max_lo = ctx - qlen + pos0 + min(npos - 1, (wave * RPW + RPW - 1) / group) - win + 1;

    // B operands of the scores: lane (hl, g4) of tile t holds dims 32 kb + 8 g4 .. + 7.
    u32x4 q[NTW][KB];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const char* qp = static_cast<const char*>(a.query) +
                       ((static_cast<int64_t>(q_begin) + pos0 + (row_ok[t] ? rpos[t] : 0)) * a.num_heads +
                        kvh * group + rhead[t]) * static_cast<int64_t>(RB);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        q[t][kb] = row_ok[t] ? load16(qp + (32 * kb + 8 * g4) * 2) : u32x4{0u, 0u, 0u, 0u};
    }

    const int lbs = a.log2_block_size;
    const int off_mask = (1 << lbs) - 1;
    const char* kbase = static_cast<const char*>(a.key_cache);
    const char* vbase = static_cast<const char*>(a.value_cache);
    const int64_t trow = static_cast<int64_t>(seq) * a.max_blocks_per_seq;
    // Block of this wave's share of each pass, lane i holding pass i's (a key
    // range has at most kSplitKeys / kKeyTile passes): read once here, so that
    // the pass loop takes it with a lane read instead of a memory round trip.
    static_assert(kSplitKeys / kKeyTile <= 64, "one lane per pass");
    int blk_lane = 0;
    if ((1 << lbs) >= WKEYS && wave < DW && lane * kKeyTile < key_hi - key_lo) {
      blk_lane = a.block_tables[trow + (min(key_lo + lane * kKeyTile + wave * WKEYS, key_hi - 1) >> lbs)];
      blk_lane = (blk_lane < 0 || blk_lane >= a.num_blocks) ? 0 : blk_lane;
    }
    wait_vmcnt<0>();  // once, before any DMA: no compiler wait inside the pass loop

    // Fused write: keys from chunk_start on are the chunk's own tokens.  The
    // workgroups read them from new_key/new_value (never from the cache, so no
    // workgroup waits for another's write), and the workgroup of the tile's
    // first key range writes the tile's tokens (this KV head) into the cache.
    constexpr bool fused = FUSED;
    const int chunk_start = ctx - qlen;
    if (fused) {
      const int first_key = a.window > 0 ? max(0, chunk_start + pos0 - a.window + 1) : 0;
      if (split == first_key / kSplitKeys) {
        const int64_t num_slots = static_cast<int64_t>(a.num_blocks) << lbs;
        for (int i = tid; i < 2 * npos * NC; i += 64 * WAVES) {
          const int kv = i / (npos * NC);
          const int r = i - kv * npos * NC;
          const int64_t tok = static_cast<int64_t>(q_begin) + pos0 + r / NC;
          const int64_t slot = a.slot_mapping[tok];
          if (slot < 0 || slot >= num_slots) continue;
          const char* src = static_cast<const char*>(kv ? a.new_value : a.new_key) +
                            (tok * a.num_kv_heads + kvh) * RB + (r % NC) * 16;
          char* dst = const_cast<char*>(kv ? vbase : kbase) +
                      ((((slot >> lbs) * a.num_kv_heads + kvh) << lbs) + (slot & off_mask)) * RB +
                      (r % NC) * 16;
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        }
        wait_vmcnt<0>();  // the DMA pipeline below counts only its own transfers
      }
    }
    // Source row of key `key` (K or V): the chunk's input row or the cache row.
    auto fused_row = [&](const void* in, int key) {
      return static_cast<const char*>(in) +
             ((static_cast<int64_t>(q_begin) + key - chunk_start) * a.num_kv_heads + kvh) * RB;
    };

    // Rotation (in chunks) of key row r and value row r of a tile.
    // A shift of 2 r rather than r: the 16-row operand reads then take the
    // LDS cycles of a contiguous read instead of twice as many.
    auto rot_k = [](int r) { return D == 64 ? r % NC : (2 * r) % NC; };
    auto rot_v = [](int r) { return D == 64 ? (r & ~1) % NC : (2 * r) % NC; };

    // This wave's share of pass `p`'s DMA (keys WKEYS wave .. WKEYS (wave + 1)
    // - 1 of the pass; none for waves past DW) into buffer `b`.  Keys past the
    // range are clamped to its last key.
    auto issue = [&](int p, int b) {
      if (wave >= DW) return;
      const int k0 = key_lo + p * kKeyTile + wave * WKEYS;
      const char* kd = reinterpret_cast<const char*>(&s_k[b][wave * WKEYS][0]);
      const char* vd = reinterpret_cast<const char*>(&s_v[b][wave * WKEYS][0]);
      if constexpr (KV8) {
        // E4M3 rows (D bytes) land unrotated, WKEYS * CNC 16-byte pieces per
        // wave: the conversion applies the rotations.  Lanes past the wave's
        // pieces sit out (an instruction still counts once in vmcnt).
        // The block id comes from the lanes read at the start, or, for blocks
        // smaller than the wave's share, from a vector load in a loop of its
        // own (a vector load joined into this loop would make every DMA wait
        // for all earlier ones).
        if ((1 << lbs) >= WKEYS) {
          const int blk = __builtin_amdgcn_readlane(blk_lane, p);
#pragma unroll
          for (int r = 0; r < NDK; ++r) {
            const int piece = r * 64 + lane;
            if (piece < WKEYS * CNC) {
              // The block's rows of this KV head as a wave-uniform base and a
              // 32-bit offset per lane.
              const int key = min(k0 + piece / CNC, key_hi - 1);
              const int64_t head_off = ((static_cast<int64_t>(blk) * a.num_kv_heads + kvh) << lbs) * D;
              const uint32_t roff = static_cast<uint32_t>(key & off_mask) * D + (piece % CNC) * 16;
              dma16_sv(kbase + head_off, roff, kd + r * 1024);
              dma16_sv(vbase + head_off, roff, vd + r * 1024);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < NDK; ++r) {
            const int piece = r * 64 + lane;
            if (piece < WKEYS * CNC) {
              const int key = min(k0 + piece / CNC, key_hi - 1);
              int blk = a.block_tables[trow + (key >> lbs)];
              blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
              const int64_t roff =
                  (((static_cast<int64_t>(blk) * a.num_kv_heads + kvh) << lbs) | (key & off_mask)) * D +
                  (piece % CNC) * 16;
              dma16(kbase + roff, kd + r * 1024);
              dma16(vbase + roff, vd + r * 1024);
            }
          }
        }
        return;
      }
      if ((1 << lbs) >= WKEYS) {
        // The wave's keys lie in one block, read at the start.
        int blk = __builtin_amdgcn_readlane(blk_lane, p);
        blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
        const int64_t head_off = ((static_cast<int64_t>(blk) * a.num_kv_heads + kvh) << lbs) * RB;
        if (!fused) {
          // The block's rows of this KV head as a wave-uniform base, and a
          // 32-bit offset per lane (a block of at most 256 tokens holds at most
          // 128 KiB of one head).
          const char* kb = kbase + head_off;
          const char* vb = vbase + head_off;
#pragma unroll
          for (int r = 0; r < WKEYS / RPI; ++r) {
            const int row = wave * WKEYS + r * RPI + lane / NC;  // row of the tile
            const int pos = lane % NC;
            const int key = min(k0 + r * RPI + lane / NC, key_hi - 1);
            const uint32_t roff = static_cast<uint32_t>(key & off_mask) * RB;
            dma16_sv(kb, roff + ((pos + rot_k(row)) % NC) * 16, kd + r * RPI * RB);
            dma16_sv(vb, roff + ((pos + rot_v(row)) % NC) * 16, vd + r * RPI * RB);
          }
          return;
        }
#pragma unroll
        for (int r = 0; r < WKEYS / RPI; ++r) {
          const int row = wave * WKEYS + r * RPI + lane / NC;  // row of the tile
          const int pos = lane % NC;
          const int key = min(k0 + r * RPI + lane / NC, key_hi - 1);
          const int64_t roff = head_off + static_cast<int64_t>(key & off_mask) * RB;
          const bool own = fused && key >= chunk_start;
          const char* ksrc = own ? fused_row(a.new_key, key) : kbase + roff;
          const char* vsrc = own ? fused_row(a.new_value, key) : vbase + roff;
          dma16(ksrc + ((pos + rot_k(row)) % NC) * 16, kd + r * RPI * RB);
          dma16(vsrc + ((pos + rot_v(row)) % NC) * 16, vd + r * RPI * RB);
        }
      } else {
#pragma unroll
        for (int r = 0; r < WKEYS / RPI; ++r) {
          const int row = wave * WKEYS + r * RPI + lane / NC;
          const int pos = lane % NC;
          const int key = min(k0 + r * RPI + lane / NC, key_hi - 1);
          int blk = a.block_tables[trow + (key >> lbs)];
          blk = (blk < 0 || blk >= a.num_blocks) ? 0 : blk;
          const int64_t roff = (((static_cast<int64_t>(blk) * a.num_kv_heads + kvh) << lbs) | (key & off_mask)) * RB;
          const bool own = fused && key >= chunk_start;
          const char* ksrc = own ? fused_row(a.new_key, key) : kbase + roff;
          const char* vsrc = own ? fused_row(a.new_value, key) : vbase + roff;
          dma16(ksrc + ((pos + rot_k(row)) % NC) * 16, kd + r * RPI * RB);
          dma16(vsrc + ((pos + rot_v(row)) % NC) * 16, vd + r * RPI * RB);
        }
      }
    };

    // Per-lane LDS offsets (bytes within one K or V tile), as a row base and a
    // rotated chunk position; NC is a power of two.
    //   keys: row 16 h + hl, chunk 4 kb + g4;
    //   values (transposing reads): row 16 h + 4 g4 + hl / 4, dims 16 mt + 4 (hl % 4).
    static_assert((NC & (NC - 1)) == 0, "chunk count is a power of two");
    const int vrow0 = 4 * g4 + (hl >> 2);
    const int q4 = hl & 3;
    const int vpos0 = (q4 >> 1) - rot_v(vrow0);  // row 16 + vrow0: rotation + 32, the same mod NC
    auto koff = [&](int h, int kb) {
      return (16 * h + hl) * RB + ((g4 - rot_k(16 * h + hl) + 4 * kb) & (NC - 1)) * 16;
    };
    auto voff = [&](int h, int mt) {
      return (16 * h + vrow0) * RB + ((vpos0 + 2 * mt) & (NC - 1)) * 16 + (q4 & 1) * 8;
    };

    const u32x4 ones = {M::kOnePair, M::kOnePair, M::kOnePair, M::kOnePair};
    f32x4 acc[NTW][MT];
    f32x4 lacc[NTW];
    float m[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      lacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[t] = -__builtin_inff();
    }

    // This lane's operand LDS addresses in buffer 0, for the key rows 0-15 of
    // a pass (rows 16-31 sit 16 rows further on at the same rotation: both
    // rotations repeat every 16 rows).  Held in registers for the unit, so
    // that each operand read in the pass loop is a lane address plus a
    // constant (buffer, half) in the instruction's offset field.  E4M3 caches
    // read the converted tile.
    typedef __attribute__((address_space(3))) const char lds_char;
    const uint32_t k_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (lds_char*)(KV8 ? static_cast<const void*>(&s_cv[0][0][0]) : static_cast<const void*>(&s_k[0][0][0]))));
    const uint32_t v_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (lds_char*)(KV8 ? static_cast<const void*>(&s_cv[1][0][0]) : static_cast<const void*>(&s_v[0][0][0]))));
    uint32_t kop[KB], vop[MT];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kop[kb] = k_lds + koff(0, kb);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vop[mt] = v_lds + voff(0, mt);

    // A pass out of buffer B (a compile-time constant, so that the buffer's
    // offset folds into the LDS instructions), in two halves: the scores
    // S^T = K Q^T (qk), then the online softmax and O^T += V^T P^T (smpv).
    // Unless `full` (every row of the wave sees every key of the pass), each
    // score is checked against its row's range (the diagonal and window edges).
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    // The empty asm makes the lane offsets opaque at each use, so that the
    // tile's address is added in the LDS instructions' offset field rather
    // than precomputed for every buffer outside the loop (in registers).
    auto opaque_k = [&]() {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(kop[kb]));
    };
    auto opaque_v = [&]() {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(vop[mt]));
    };
    // s[h][t] holds keys k0 + 16 h + 4 g4 + i of row 16 t + hl.
    auto qk = [&](auto b_const, f32x4 (&s)[2][NTW]) {
      constexpr int B = decltype(b_const)::value;
      constexpr uint32_t BO = KV8 ? 0 : B * kKeyTile * RB;  // the buffer's offset from buffer 0
      static_assert(BO + 16 * RB < 65536, "fits the LDS instruction offset");
      opaque_k();
      // Every key operand of the pass is read before its product, the reads
      // for later products during the earlier ones, so that their latencies
      // overlap instead of adding up (an order the scheduler keeps: left to
      // itself it holds one read in flight at a time, to save registers).  The
      // two halves' score chains alternate, so that each product has two
      // before its dependence (1% on the Gemma chunks against one chain after
      // the other, same result bits).
      u32x4 ka[2][KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ka[h][kb] = *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(kop[kb] + BO + h * 16 * RB));
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < NTW; ++t) s[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < NTW; ++t) s[h][t] = M::run(ka[h][kb], q[t][kb], s[h][t]);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTW, 0);
        if (kb + 2 < KB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    };
    auto smpv = [&](int p, auto b_const, bool full, f32x4 (&s)[2][NTW]) {
      constexpr int B = decltype(b_const)::value;
      constexpr uint32_t BO = KV8 ? 0 : B * kKeyTile * RB;
      opaque_v();
      const int k0 = key_lo + p * kKeyTile;
      auto read_v = [&](int mt) {
        const u32x2 v0 = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(static_cast<uintptr_t>(vop[mt] + BO))));
        const u32x2 v1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(
                                                       static_cast<uintptr_t>(vop[mt] + BO + 16 * RB))));
        return u32x4{v0[0], v0[1], v1[0], v1[1]};
      };
      // The first PV value operands are read during the softmax (issued
      // before it); each product then reads the operand PV tiles ahead.
      constexpr int PV = MT < 8 ? MT : 8;
      u32x4 va[MT];
#pragma unroll
      for (int mt = 0; mt < PV; ++mt) va[mt] = read_v(mt);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV, 0);
      u32x4 pb[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        // Exponents against the row's current max (an fma each without
        // capping); masked keys get -inf.  Key k0 + 16 h + 4 g4 + i is in the
        // row's range when 16 h + i lies in [lo_t - k0, lim_t - k0].
        const float mu_old = safe_max(m[t]);
        float e[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) e[4 * h + i] = score.exponent(s[h][t][i], mu_old);
        if (!full) {
          const int dhi = lane_lim[t] - k0;
          const int dlo = lane_lo[t] - k0;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool in = 16 * h + i <= dhi && (!S::kWindow || 16 * h + i >= dlo);
              e[4 * h + i] = in ? e[4 * h + i] : -__builtin_inff();
            }
        }
        float mx = e[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, e[i]);
        mx = max_across_rows(mx);  // the pass's max, relative to mu_old
        // Move the max when this pass's passes it by 2^kLazyMax (or is the
        // row's first finite score); otherwise the exponents stay below it.
        const bool move = m[t] == -__builtin_inff() ? mx > -__builtin_inff() : mx > kLazyMax;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {  // wave-uniform
          const float m_new = fmaxf(m[t], mx + mu_old);
          const float alpha = exp2_fast(m[t] - safe_max(m_new));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] *= alpha;
          lacc[t] *= alpha;
          const float shift = safe_max(m_new) - mu_old;
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] -= shift;
          m[t] = m_new;
        }
        pb[t] = u32x4{M::pack(exp2_fast(e[0]), exp2_fast(e[1])), M::pack(exp2_fast(e[2]), exp2_fast(e[3])),
                      M::pack(exp2_fast(e[4]), exp2_fast(e[5])), M::pack(exp2_fast(e[6]), exp2_fast(e[7]))};
        lacc[t] = M::run(ones, pb[t], lacc[t]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + PV < MT) va[mt + PV] = read_v(mt + PV);
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[t][mt] = M::run(va[mt], pb[t], acc[t][mt]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        __builtin_amdgcn_sched_group_barrier(0x008, NTW, 1);
        if (mt + PV < MT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
    };

    auto compute = [&](int p, auto b_const, bool full) {
      f32x4 s[2][NTW];
      qk(b_const, s);
      smpv(p, b_const, full, s);
    };

    const int npass = (key_hi - key_lo + kKeyTile - 1) / kKeyTile;
    auto sees = [&](int p) {  // wave-uniform: some row of this wave sees a key of pass p
      const int k0 = key_lo + p * kKeyTile;
      return p < npass && k0 <= wave_last && k0 + kKeyTile > wave_first;
    };
    auto full_pass = [&](int p) {  // wave-uniform: every row of this wave sees every key of pass p
      const int k0 = key_lo + p * kKeyTile;
      return k0 + kKeyTile - 1 <= wave_min_lim && k0 + kKeyTile <= key_hi && (!S::kWindow || k0 >= wave_max_lo);
    };
    for (int p = 0; p < NBUF - 1 && p < npass; ++p) issue(p, p);
    // Pass p uses buffer p % NBUF: the loop runs NBUF passes at a time so that
    // each one's buffer is a constant.
    auto step = [&](int p, auto b_const) {
      constexpr int B = decltype(b_const)::value;
      // Wait for this wave's share of pass p: the passes issued after it may stay in flight.
      static_assert(NBUF == 3 || NBUF == 4, "wait cases and the unrolled pass loop");
      switch (min(NBUF - 2, npass - 1 - p)) {
        case 2: wait_vmcnt<2 * NDW>(); break;
        case 1: wait_vmcnt<NDW>(); break;
        default: wait_vmcnt<0>(); break;
      }
      // Every wave's share of pass p has landed, and every wave is done with
      // pass p - 1, whose buffer the next DMA reuses.
      __syncthreads();
      if (p + NBUF - 1 < npass) issue(p + NBUF - 1, (B + NBUF - 1) % NBUF);
      if constexpr (KV8) {
        // All threads turn the pass's E4M3 K and V rows into the rotated 16-bit
        // tile; the next iteration's barrier keeps it until every wave is
        // done with it.
        const int b = B;
#pragma unroll
        for (int i = 0; i < 2 * kKeyTile * CNC / (64 * WAVES); ++i) {
          const int idx = static_cast<int>(threadIdx.x) + i * 64 * WAVES;
          const int kv = idx / (kKeyTile * CNC);
          const int t = (idx / CNC) % kKeyTile;
          const int c = 2 * (idx % CNC);
          const u32x4 w = kv ? s_v[b][t][idx % CNC] : s_k[b][t][idx % CNC];
          const u32x4 lo = {M::template from_fp8<false>(w[0]), M::template from_fp8<true>(w[0]),
                            M::template from_fp8<false>(w[1]), M::template from_fp8<true>(w[1])};
          const u32x4 hi = {M::template from_fp8<false>(w[2]), M::template from_fp8<true>(w[2]),
                            M::template from_fp8<false>(w[3]), M::template from_fp8<true>(w[3])};
          const int rot = kv == 0 ? rot_k(t) : rot_v(t);
          s_cv[kv][t][(c - rot) & (NC - 1)] = lo;
          s_cv[kv][t][(c + 1 - rot) & (NC - 1)] = hi;
        }
        __syncthreads();
      }
      if (sees(p)) compute(p, b_const, full_pass(p));
    };
    for (int p0 = 0; p0 < npass; p0 += NBUF) {
      step(p0, std::integral_constant<int, 0>{});
      if (p0 + 1 < npass) step(p0 + 1, std::integral_constant<int, 1>{});
      if (p0 + 2 < npass) step(p0 + 2, std::integral_constant<int, 2 % NBUF>{});
      if constexpr (NBUF > 3)
        if (p0 + 3 < npass) step(p0 + 3, std::integral_constant<int, 3 % NBUF>{});
    }

#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if (!row_ok[t] || key_lo > row_lim[t] || key_hi <= row_lo[t]) continue;  // no key of this range for this row
      const float lsum = lacc[t][0];
      const int nsplit_row = row_lim[t] / kSplitKeys - max(row_lo[t], 0) / kSplitKeys + 1;
      const int64_t out_row = (static_cast<int64_t>(q_begin) + pos0 + rpos[t]) * a.num_heads + kvh * group + rhead[t];
      // Output register i of tile mt holds dim 16 mt + 4 g4 + i.
      if constexpr (KV8) {  // values were read without their scale
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] *= a.v_scale;
      }
      if (nsplit_row == 1) {
        const float inv = 1.f / lsum;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4 o = acc[t][mt] * inv;
          const u32x2 packed = {M::pack(o[0], o[1]), M::pack(o[2], o[3])};
          *reinterpret_cast<u32x2*>(static_cast<char*>(a.out) + (out_row * D + 16 * mt + 4 * g4) * 2) = packed;
        }
      } else {
        const int64_t ws = out_row * nsplit + split;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4*>(&ws_acc[ws * D + 16 * mt + 4 * g4]) = acc[t][mt];
        if (g4 == 0) {
          ws_max[ws] = m[t];
          ws_sum[ws] = lsum;
        }
      }
    }

  };
  if constexpr (kPersistentPrefill<D>) {
    const int g = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
    for (int round = 0;; ++round) {
      const int unit = round * g + ((round & 1) ? g - 1 - b : b);
      if (unit >= n_units) break;  // units only grow with the round
      run_unit(unit);
      __syncthreads();  // every wave is done with this unit's LDS before the next one's DMA
    }
  } else {
    if (static_cast<int>(blockIdx.x) < n_units) run_unit(static_cast<int>(blockIdx.x));
  }
}

// One wave per (query token, head): merge the key-range partials of rows
// whose keys spanned more than one range.  Each wave issues its loads in two
// rounds (the token's last key from the plan's map, then up to four ranges'
// states at once), so the kernel costs two memory latencies.
template <typename E, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void prefill_merge_kernel(PrefillArgs a, int32_t nsplit,
                                                                const int32_t* tok_lim,
                                                                const float* ws_max,
                                                                const float* ws_sum,
                                                                const float* ws_acc) {
  constexpr int PER = D / 64;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rowid >= static_cast<int64_t>(a.num_q_tokens) * a.num_heads) return;
  const int t = static_cast<int>(rowid / a.num_heads);
  const int row_lim = tok_lim[t];
  if (row_lim < 0) return;  // nothing to merge
  // Key ranges holding the row's keys (those of its window, or 0 .. row_lim).
  const int p0 = a.window > 0 ? max(0, row_lim - a.window + 1) / kSplitKeys : 0;
  const int p1 = row_lim / kSplitKeys + 1;
  if (p1 - p0 <= 1) return;
  const int64_t base = rowid * nsplit;

  // Online merge over groups of four ranges (one group unless the row spans
  // more than 4096 keys), each group's loads issued together.
  typedef float vecp __attribute__((ext_vector_type(PER)));
  vecp num = {};
  float mrun = -__builtin_inff(), den = 0.f;
  for (int p = p0; p < p1; p += 4) {
    vecp v[4];
    float mp[4], sp[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pu = min(p + u, p1 - 1);
      v[u] = *reinterpret_cast<const vecp*>(&ws_acc[(base + pu) * D + lane * PER]);
      mp[u] = p + u < p1 ? ws_max[base + pu] : -__builtin_inff();
      sp[u] = ws_sum[base + pu];
    }
    const float mnew = fmaxf(fmaxf(mrun, fmaxf(mp[0], mp[1])), fmaxf(mp[2], mp[3]));
    const float mu = safe_max(mnew);
    const float alpha = exp2_fast(mrun - mu);
    num *= alpha;
    den *= alpha;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float f = exp2_fast(mp[u] - mu);
      num += f * v[u];
      den = __builtin_fmaf(f, sp[u], den);
    }
    mrun = mnew;
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int j = 0; j < PER; ++j) E::store(a.out, rowid * D + lane * PER + j, num[j] * inv);
}

// Workgroups of one persistent prefill launch: as many as fit on the device at once.
template <typename E, int D, typename S, bool KV8, bool FUSED>
uint64_t prefill_grid() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g > 0) return static_cast<uint64_t>(g);
  int ncu = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) ncu = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_kernel<E, D, S, KV8, FUSED>,
                                                    prefill_threads(D), 0) != hipSuccess)
    per_cu = 1;
  g = std::max(1, ncu) * std::max(1, per_cu);
  cache[dev].store(g, std::memory_order_relaxed);
  return static_cast<uint64_t>(g);
}

template <typename E, int D>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream, void* workspace) {
  const int group = a.num_heads / a.num_kv_heads;
  const int pos_per_tile = kRowsPerWg / group;
  const int ntiles = prefill_num_tiles(a.num_heads, a.num_kv_heads, a.max_query_len);
  const int nsplit = prefill_num_splits(a.ctx_limit);
  const uint64_t items = static_cast<uint64_t>(a.num_seqs) * ntiles * nsplit;
  if (items == 0) return hipSuccess;
  const uint64_t n = items * a.num_kv_heads;
  if (n > 0x7fffffffu) return hipErrorInvalidValue;
  const PrefillWorkspace w = prefill_workspace_layout(a.num_q_tokens, a.num_heads, a.head_dim, nsplit,
                                                      a.num_seqs, ntiles);
  char* base = static_cast<char*>(workspace);
  float* ws_max = nsplit > 1 ? reinterpret_cast<float*>(base + w.off_max) : nullptr;
  float* ws_sum = nsplit > 1 ? reinterpret_cast<float*>(base + w.off_sum) : nullptr;
  float* ws_acc = nsplit > 1 ? reinterpret_cast<float*>(base + w.off_acc) : nullptr;
  int4* plan = reinterpret_cast<int4*>(base + w.off_plan);
  int32_t* plan_count = reinterpret_cast<int32_t*>(base + w.off_count);
  int32_t* tok_lim = nsplit > 1 ? reinterpret_cast<int32_t*>(base + w.off_toklim) : nullptr;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, pos_per_tile, ntiles,
                     nsplit, plan, plan_count, tok_lim);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // An E4M3 cache's K scale folds into the score scale.
  const float qk_scale = a.kv_fp8 ? a.scale * a.k_scale : a.scale;
  with_score_map(qk_scale, a.softcap, a.window, [&](auto map) {
    using S = decltype(map);
    if (a.kv_fp8) {
      const uint64_t grid = kPersistentPrefill<D> ? std::min<uint64_t>(n, prefill_grid<E, D, S, true, false>()) : n;
      hipLaunchKernelGGL((prefill_kernel<E, D, S, true, false>), dim3(static_cast<uint32_t>(grid)),
                         dim3(prefill_threads(D)), 0, stream, a, group, pos_per_tile, nsplit, plan,
                         plan_count, map, ws_max, ws_sum, ws_acc);
    } else if (a.fused) {
      const uint64_t grid = kPersistentPrefill<D> ? std::min<uint64_t>(n, prefill_grid<E, D, S, false, true>()) : n;
      hipLaunchKernelGGL((prefill_kernel<E, D, S, false, true>), dim3(static_cast<uint32_t>(grid)),
                         dim3(prefill_threads(D)), 0, stream, a, group, pos_per_tile, nsplit, plan,
                         plan_count, map, ws_max, ws_sum, ws_acc);
    } else {
      const uint64_t grid = kPersistentPrefill<D> ? std::min<uint64_t>(n, prefill_grid<E, D, S, false, false>()) : n;
      hipLaunchKernelGGL((prefill_kernel<E, D, S, false, false>), dim3(static_cast<uint32_t>(grid)),
                         dim3(prefill_threads(D)), 0, stream, a, group, pos_per_tile, nsplit, plan,
                         plan_count, map, ws_max, ws_sum, ws_acc);
    }
    return 0;
  });
  err = hipGetLastError();
  if (err != hipSuccess || nsplit <= 1) return err;
  const int64_t rows = static_cast<int64_t>(a.num_q_tokens) * a.num_heads;
  if (rows == 0) return hipSuccess;
  if ((rows + kMergeWaves - 1) / kMergeWaves > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_merge_kernel<E, D>), dim3(static_cast<unsigned>((rows + kMergeWaves - 1) / kMergeWaves)),
                     dim3(kMergeWaves * 64), 0,
                     stream, a, nsplit, tok_lim, ws_max, ws_sum, ws_acc);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_prefill_e(const PrefillArgs& a, hipStream_t stream, void* workspace) {
  switch (a.head_dim) {
    case 64: return launch_prefill_d<E, 64>(a, stream, workspace);
    case 128: return launch_prefill_d<E, 128>(a, stream, workspace);
    default: return launch_prefill_d<E, 256>(a, stream, workspace);
  }
}

}  // namespace

static size_t align256p(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int32_t prefill_num_splits(int32_t ctx_limit) { return (ctx_limit + kSplitKeys - 1) / kSplitKeys; }

int32_t prefill_num_tiles(int32_t num_heads, int32_t num_kv_heads, int32_t max_query_len) {
  const int pos_per_tile = kRowsPerWg / (num_heads / num_kv_heads);
  return (max_query_len + pos_per_tile - 1) / pos_per_tile;
}

PrefillWorkspace prefill_workspace_layout(int32_t num_q_tokens, int32_t num_heads, int32_t head_dim,
                                          int32_t nsplit, int32_t num_seqs, int32_t ntiles) {
  PrefillWorkspace w{};
  if (num_q_tokens <= 0 || num_seqs <= 0 || ntiles <= 0 || nsplit <= 0) return w;
  size_t off = 0;
  if (nsplit > 1) {
    const size_t n = static_cast<size_t>(num_q_tokens) * num_heads * nsplit;
    w.off_max = 0;
    w.off_sum = align256p(n * sizeof(float));
    w.off_acc = w.off_sum + align256p(n * sizeof(float));
    off = w.off_acc + align256p(n * head_dim * sizeof(float));
  }
  w.off_count = off;
  w.off_plan = off + 256;
  w.bytes = w.off_plan + align256p(static_cast<size_t>(num_seqs) * ntiles * nsplit * sizeof(int4));
  if (nsplit > 1) {
    w.off_toklim = w.bytes;
    w.bytes += align256p(static_cast<size_t>(num_q_tokens) * sizeof(int32_t));
  }
  return w;
}

hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream) {
  if (a.dtype == PA_DTYPE_F16) return launch_prefill_e<F16>(a, stream, workspace);
  return launch_prefill_e<BF16>(a, stream, workspace);
}

}  // namespace pa

// Chunked-prefill paged attention for gfx950 (MFMA).
//
// A chunk of L prompt tokens at the end of a context of C cached tokens attends
// the context before it and itself causally: row i sits at position C - L + i
// and sees keys 0 .. C - L + i.  Chunked prefill is listed on the wLLM PyPI
// page ("Features -- Core engine"; long prompts are split so they do not stall
// other requests' decode); the GQA mapping is the mini-vLLM one (each query
// head reads its own KV head).
//
// Unlike decode, a tile of query rows makes both products dense, so they run
// on the matrix cores (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulate):
//
// * A workgroup is 4 waves x 32 query rows.  Rows are (position, head) pairs of
//   one KV head, head-minor, so the G query heads that share a KV head share
//   every K/V tile that is staged (for MQA, 16 positions x 8 heads).
// * Scores are computed transposed, S^T = K Q^T (keys x rows), so that each
//   lane of the accumulator holds one query row: the row max and sum of the
//   online softmax stay inside a lane apart from one exchange between the two
//   half-waves, and rescaling the output is a per-lane multiply.
// * O^T += V^T P^T.  P^T comes straight from the score accumulator registers
//   (exp2, rounded to the input type); V is staged transposed in LDS
//   ([dim][key]) so its operand is two 8-byte LDS reads per MFMA.
// * The keys of a tile are split in ranges of kSplitKeys so that long contexts
//   spread over several workgroups; each range writes an (m, l, acc) partial
//   per row and prefill_merge combines them by log-sum-exp weights, as the
//   decode reduce does.  Rows whose keys fit one range are written directly.
//
// Scores are kept in log2 units (scale * log2 e folded in): one v_exp_f32 per
// probability.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWg = 4 * kRowsPerWave;
constexpr int kKeyTile = 32;
constexpr int kSplitKeys = 1024;

template <typename E>
struct Mfma;
template <>
struct Mfma<BF16> {
  __device__ static inline f32x16 run(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round to bf16 (nearest-even); returns the 16-bit pattern.
  __device__ static inline unsigned short round_bits(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
  }
  __device__ static inline float from_bits(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
  }
};
template <>
struct Mfma<F16> {
  __device__ static inline f32x16 run(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline unsigned short round_bits(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
  }
  __device__ static inline float from_bits(unsigned short b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
};

// Byte-select of v_perm_b32: result byte i = byte sel[i] of {hi:lo}.
__device__ inline unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a, int32_t group,
                                                          int32_t pos_per_tile, int32_t ntiles,
                                                          int32_t nsplit, uint32_t n_logical,
                                                          uint32_t per_xcd, float scale_log2,
                                                          float* ws_max, float* ws_sum,
                                                          float* ws_acc) {
  constexpr int KPAD = D + 8;          // K tile row stride (elements)
  constexpr int VPAD = kKeyTile + 4;   // V^T tile row stride (elements)
  constexpr int NKS = D / 16;          // k-steps of the score product
  constexpr int NDB = D / 32;          // 32-wide output column blocks
  __shared__ __attribute__((aligned(16))) unsigned short s_k[kKeyTile * KPAD];
  __shared__ __attribute__((aligned(16))) unsigned short s_vt[D * VPAD];
  __shared__ int32_t s_tbl[kSplitKeys];

  const uint32_t logical = xcd_remap(blockIdx.x, per_xcd);
  if (logical >= n_logical) return;
  // Logical order ((seq * Hkv + kv_head) * nsplit + split) * ntiles + tile,
  // with tiles from the end of the chunk (most keys) first.
  uint32_t rem = logical;
  const int tile = ntiles - 1 - static_cast<int>(rem % ntiles);
  rem /= ntiles;
  const int split = rem % nsplit;
  rem /= nsplit;
  const int kvh = rem % a.num_kv_heads;
  const int seq = rem / a.num_kv_heads;

  const int q_begin = min(max(a.query_start_loc[seq], 0), a.num_q_tokens);
  const int q_end = min(max(a.query_start_loc[seq + 1], q_begin), a.num_q_tokens);
  const int ctx = max(0, min(a.context_lens[seq], a.ctx_limit));
  const int qlen = min(q_end - q_begin, ctx);
  const int pos0 = tile * pos_per_tile;
  if (qlen <= 0 || pos0 >= qlen) return;
  const int npos = min(pos_per_tile, qlen - pos0);
  const int last_key = ctx - qlen + pos0 + npos - 1;  // last key any row of the tile sees
  const int key_lo = split * kSplitKeys;
  if (key_lo > last_key) return;
  const int key_hi = min(key_lo + kSplitKeys, last_key + 1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // This lane's query row.
  const int row = wave * kRowsPerWave + l32;
  const int rpos = row / group;
  const int rhead = row - rpos * group;
  const bool row_ok = rpos < npos;
  const int row_lim = row_ok ? ctx - qlen + pos0 + rpos : -1;
  const int hq = kvh * group + rhead;
  const int64_t q_row = static_cast<int64_t>(q_begin) + pos0 + rpos;

  u32x4 qf[NKS];
  {
    const char* qp = static_cast<const char*>(a.query) +
                     (q_row * a.num_heads + hq) * static_cast<int64_t>(D) * 2;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = row_ok ? load16(qp + (16 * ks + 8 * half) * 2) : u32x4{0u, 0u, 0u, 0u};
  }

  // Block ids of this key range.
  const int lbs = a.log2_block_size;
  const int off_mask = (1 << lbs) - 1;
  const int first_blk = key_lo >> lbs;
  {
    const int nblk = ((key_hi - 1) >> lbs) - first_blk + 1;
    const int32_t* table = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;
    for (int i = tid; i < nblk; i += kThreads) {
      const int b = table[first_blk + i];
      s_tbl[i] = (b < 0 || b >= a.num_blocks) ? 0 : b;
    }
  }

  const char* kbase = static_cast<const char*>(a.key_cache);
  const char* vbase = static_cast<const char*>(a.value_cache);
  constexpr int64_t kRowBytes = static_cast<int64_t>(D) * 2;

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -__builtin_inff();
  float lsum = 0.f;

  for (int k0 = key_lo; k0 < key_hi; k0 += kKeyTile) {
    __syncthreads();  // the table is staged / the previous tile is consumed
    // K tile: [key][dim] (16-byte chunks).
    for (int c = tid; c < kKeyTile * D / 8; c += kThreads) {
      const int key = c / (D / 8);
      const int dc = c - key * (D / 8);
      const int kabs = k0 + key;
      u32x4 v{0u, 0u, 0u, 0u};
      if (kabs < key_hi) {
        const int64_t blk = s_tbl[(kabs >> lbs) - first_blk];
        v = load16(kbase + ((blk * a.num_kv_heads + kvh) << lbs | (kabs & off_mask)) * kRowBytes +
                   dc * 16);
      }
      *reinterpret_cast<u32x4*>(&s_k[key * KPAD + dc * 8]) = v;
    }
    // V tile, transposed: [dim][key], 4 keys x 8 dims per unit.
    for (int u = tid; u < (kKeyTile / 4) * (D / 8); u += kThreads) {
      const int kg = u / (D / 8);
      const int dc = u - kg * (D / 8);
      u32x4 r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kabs = k0 + 4 * kg + j;
        r[j] = u32x4{0u, 0u, 0u, 0u};
        if (kabs < key_hi) {
          const int64_t blk = s_tbl[(kabs >> lbs) - first_blk];
          r[j] = load16(vbase + ((blk * a.num_kv_heads + kvh) << lbs | (kabs & off_mask)) * kRowBytes +
                        dc * 16);
        }
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 lo{perm(r[1][w], r[0][w], 0x05040100u), perm(r[3][w], r[2][w], 0x05040100u)};
        const u32x2 hi{perm(r[1][w], r[0][w], 0x07060302u), perm(r[3][w], r[2][w], 0x07060302u)};
        *reinterpret_cast<u32x2*>(&s_vt[(dc * 8 + 2 * w) * VPAD + 4 * kg]) = lo;
        *reinterpret_cast<u32x2*>(&s_vt[(dc * 8 + 2 * w + 1) * VPAD + 4 * kg]) = hi;
      }
    }
    __syncthreads();

    // S^T (32 keys x 32 rows of this wave).
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(&s_k[l32 * KPAD + 16 * ks + 8 * half]);
      st = Mfma<E>::run(ka, qf[ks], st);
    }

    // Online softmax for this lane's row (accumulator register r holds key
    // 8*(r/4) + 4*half + r%4 of the tile).
    float s[16];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      s[r] = (key <= row_lim && key < key_hi) ? st[r] * scale_log2 : -__builtin_inff();
      tmax = fmaxf(tmax, s[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float mu = safe_max(m_new);
    const float alpha = exp2_fast(m - mu);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    u32x4 pb[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned short b0 = Mfma<E>::round_bits(exp2_fast(s[8 * ks2 + 2 * w] - mu));
        const unsigned short b1 = Mfma<E>::round_bits(exp2_fast(s[8 * ks2 + 2 * w + 1] - mu));
        lsum += Mfma<E>::from_bits(b0) + Mfma<E>::from_bits(b1);
        pb[ks2][w] = static_cast<unsigned>(b0) | (static_cast<unsigned>(b1) << 16);
      }
    }

    // O^T (dims x rows) += V^T P^T.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const unsigned short* vrow = &s_vt[(32 * db + l32) * VPAD + 16 * ks2 + 4 * half];
        const u32x2 x = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 y = *reinterpret_cast<const u32x2*>(vrow + 8);
        o[db] = Mfma<E>::run(u32x4{x[0], x[1], y[0], y[1]}, pb[ks2], o[db]);
      }
    }
  }

  if (!row_ok || key_lo > row_lim) return;  // no key of this range for this row
  lsum += __shfl_xor(lsum, 32, 64);
  const int nsplit_row = (row_lim + kSplitKeys) / kSplitKeys;
  const int64_t out_row = q_row * a.num_heads + hq;
  if (nsplit_row == 1) {
    const float inv = 1.f / lsum;
    // Output register r of block db holds dim 32*db + 8*(r/4) + 4*half + r%4.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        unsigned short bits[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bits[i] = Mfma<E>::round_bits(o[db][4 * j + i] * inv);
        const u32x2 pk{static_cast<unsigned>(bits[0]) | (static_cast<unsigned>(bits[1]) << 16),
                       static_cast<unsigned>(bits[2]) | (static_cast<unsigned>(bits[3]) << 16)};
        *reinterpret_cast<u32x2*>(static_cast<char*>(a.out) +
                                  (out_row * D + 32 * db + 8 * j + 4 * half) * 2) = pk;
      }
  } else {
    const int64_t ws = out_row * nsplit + split;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(&ws_acc[ws * D + 32 * db + 8 * j + 4 * half]) =
            u32x4{__float_as_uint(o[db][4 * j]), __float_as_uint(o[db][4 * j + 1]),
                  __float_as_uint(o[db][4 * j + 2]), __float_as_uint(o[db][4 * j + 3])};
    if (half == 0) {
      ws_max[ws] = m;
      ws_sum[ws] = lsum;
    }
  }
}

// One wave per (query token, head): merge the key-range partials of rows
// whose keys spanned more than one range.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_merge_kernel(PrefillArgs a, int32_t nsplit,
                                                                const float* ws_max,
                                                                const float* ws_sum,
                                                                const float* ws_acc) {
  constexpr int PER = D / 64;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (rowid >= static_cast<int64_t>(a.num_q_tokens) * a.num_heads) return;
  const int t = static_cast<int>(rowid / a.num_heads);
  // Sequence of token t: last s with query_start_loc[s] <= t.
  int lo = 0, hi = a.num_seqs;  // invariant: qsl[lo] <= t < qsl[hi]
  if (t < a.query_start_loc[0] || t >= a.query_start_loc[a.num_seqs]) return;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.query_start_loc[mid] <= t) lo = mid; else hi = mid;
  }
  const int q_begin = min(max(a.query_start_loc[lo], 0), a.num_q_tokens);
  const int q_end = min(max(a.query_start_loc[lo + 1], q_begin), a.num_q_tokens);
  const int ctx = max(0, min(a.context_lens[lo], a.ctx_limit));
  const int qlen = min(q_end - q_begin, ctx);
  const int pos = t - q_begin;
  if (pos >= qlen) return;
  const int row_lim = ctx - qlen + pos;
  const int nsplit_row = (row_lim + kSplitKeys) / kSplitKeys;
  if (nsplit_row <= 1) return;
  const int64_t base = rowid * nsplit;

  float mx = -__builtin_inff();
  for (int p = lane; p < nsplit_row; p += 64) mx = fmaxf(mx, ws_max[base + p]);
  mx = across_groups_max<1>(mx);
  const float mu = safe_max(mx);
  float den = 0.f;
  for (int p = lane; p < nsplit_row; p += 64) den += exp2_fast(ws_max[base + p] - mu) * ws_sum[base + p];
  den = across_groups_sum<1>(den);
  float num[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) num[j] = 0.f;
  for (int p = 0; p < nsplit_row; ++p) {
    const float f = exp2_fast(ws_max[base + p] - mu);
#pragma unroll
    for (int j = 0; j < PER; ++j) num[j] = __builtin_fmaf(f, ws_acc[(base + p) * D + lane * PER + j], num[j]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) E::store(a.out, rowid * D + lane * PER + j, num[j] / den);
}

template <typename E, int D>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream, void* workspace) {
  const int group = a.num_heads / a.num_kv_heads;
  const int pos_per_tile = kRowsPerWg / group;
  const int ntiles = (a.max_query_len + pos_per_tile - 1) / pos_per_tile;
  const int nsplit = (a.ctx_limit + kSplitKeys - 1) / kSplitKeys;
  const uint64_t n = static_cast<uint64_t>(a.num_seqs) * a.num_kv_heads * (nsplit > 0 ? nsplit : 1) * ntiles;
  if (n == 0 || nsplit == 0) return hipSuccess;
  const uint32_t per = static_cast<uint32_t>((n + 7) / 8);
  float* ws_max = nullptr;
  float* ws_sum = nullptr;
  float* ws_acc = nullptr;
  if (nsplit > 1) {
    const PrefillWorkspace w = prefill_workspace_layout(a.num_q_tokens, a.num_heads, a.head_dim, nsplit);
    char* base = static_cast<char*>(workspace);
    ws_max = reinterpret_cast<float*>(base + w.off_max);
    ws_sum = reinterpret_cast<float*>(base + w.off_sum);
    ws_acc = reinterpret_cast<float*>(base + w.off_acc);
  }
  hipLaunchKernelGGL((prefill_kernel<E, D>), dim3(per * 8), dim3(kThreads), 0, stream, a, group,
                     pos_per_tile, ntiles, nsplit, static_cast<uint32_t>(n), per,
                     a.scale * kLog2e, ws_max, ws_sum, ws_acc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nsplit <= 1) return err;
  const int64_t rows = static_cast<int64_t>(a.num_q_tokens) * a.num_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_merge_kernel<E, D>), dim3(static_cast<unsigned>((rows + 3) / 4)),
                     dim3(kThreads), 0, stream, a, nsplit, ws_max, ws_sum, ws_acc);
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

PrefillWorkspace prefill_workspace_layout(int32_t num_q_tokens, int32_t num_heads,
                                          int32_t head_dim, int32_t nsplit) {
  PrefillWorkspace w{};
  if (nsplit <= 1 || num_q_tokens <= 0) return w;
  const size_t n = static_cast<size_t>(num_q_tokens) * num_heads * nsplit;
  w.off_max = 0;
  w.off_sum = align256p(n * sizeof(float));
  w.off_acc = w.off_sum + align256p(n * sizeof(float));
  w.bytes = w.off_acc + align256p(n * head_dim * sizeof(float));
  return w;
}

hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream) {
  if (a.dtype == PA_DTYPE_F16) return launch_prefill_e<F16>(a, stream, workspace);
  return launch_prefill_e<BF16>(a, stream, workspace);
}

}  // namespace pa

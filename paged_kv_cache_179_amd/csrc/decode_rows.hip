// Paged-attention decode for 16-bit caches: a software-pipelined kernel that
// streams each sequence's K/V blocks through LDS.
//
// Same operation, work split, partition states and reduce as decode.hip (the
// PagedAttention decode of the wLLM PyPI page, "Features -- Core engine", with
// mini-vLLM's grouped-query head mapping: each query head reads its KV head).
// The design targets the cost of grouped-query heads, where every cached
// element feeds G multiply-adds for q.k and G more for p.V:
//
// * Passes of TP tokens (16; 8 for head_dim 256), one 4 KB (block, head) run
//   of K and of V per pass at block_size 16.  Both are copied by the gfx950
//   global-to-LDS DMA (16-byte lanes, fully coalesced, non-temporal) into a
//   per-wave slot; two slots per wave, so pass i+1 is in flight while pass i
//   is computed.  No K/V bytes pass through VGPRs on the way to LDS.
// * q.k: LQ = 64 / TP lanes per token, each reading CPL 16-byte chunks of its
//   token's key row from LDS (chunks are rotated per row when loaded, so
//   these reads are bank-conflict free) and the group's query chunks from
//   LDS (same address across tokens: broadcast).  v_dot2 per head, then a
//   2- or 3-step DPP sum over the token's lanes.
// * Online softmax with lazy rescaling: probabilities are taken against the
//   wave's running max m, which is refreshed (wave-wide max, rescale of the
//   accumulators) only when some score exceeds m by more than 2^8 -- a
//   ballot per head per pass.  Probabilities therefore stay <= 256.
// * p.V: lanes own 16-byte slices of the value rows; two tokens' values are
//   interleaved with v_perm so that one v_dot2 adds both tokens' products to
//   one output element.  The (p_t, p_t+1) pairs, rounded to the cache type,
//   reach the slice lanes through a small LDS table; the denominator sums the
//   same rounded values.
//
// One workgroup of 4 waves handles one (sequence, KV head, partition, head
// chunk); the waves take the passes of each 512-token segment in turn and are
// merged through LDS at the end.
#include "device_common.h"
#include "lds_dma.h"
#include "decode_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = kDecodeThreads / kWave;
constexpr float kLazyMax = 8.f;  // log2 of the largest unnormalised probability

template <typename E>
struct Pack16;
template <>
struct Pack16<BF16> {
  __device__ static inline unsigned round(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
  }
  __device__ static inline float widen(unsigned b) { return __uint_as_float(b << 16); }
  __device__ static inline float dot(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           c, false);
  }
};
template <>
struct Pack16<F16> {
  __device__ static inline unsigned round(float x) {
    return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
  }
  __device__ static inline float widen(unsigned b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(b)));
  }
  __device__ static inline float dot(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
};

__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
  // The swap hands each lane the value of lane ^ 32 in one of its two results.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float wave_sum(float x) {
  x = group_sum<32>(x);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct Geo {
  static constexpr int TP = D == 256 ? 8 : 16;  // tokens per pass
  static constexpr int LQ = kWave / TP;         // lanes per token (scores)
  static constexpr int NC = D / 8;              // 16-byte chunks per row
  static constexpr int CPL = NC / LQ;           // chunks per lane (scores)
  static constexpr int RB = D * 2;              // row bytes
  static constexpr int RPI = 1024 / RB;         // rows per DMA instruction
  static constexpr int NDMA = TP / RPI;         // DMA instructions per pass, K or V
  static constexpr int LPT = NC;                // lanes per value row (p.V)
  static constexpr int TPL = kWave / LPT;       // value rows per wave load
  static constexpr int NPG = (TP / 2) / TPL;    // token pairs per lane group
  // Rotation (in chunks) of key row t in LDS.  Lane p of a token reads chunks
  // p, p + LQ, ...; with these rotations the 16 lanes that one LDS cycle
  // serves touch 16 different bank groups.
  __device__ static inline int rot(int t) { return D == 64 ? (LQ * (t >> 1)) % NC : (LQ * t) % NC; }
};

template <typename E, int D, int GT>
__global__ __launch_bounds__(kDecodeThreads) void decode_rows_kernel(DecodeArgs a, int32_t head_chunks,
                                                                     float scale_log2) {
  using P = Pack16<E>;
  using G = Geo<D>;
  constexpr int TP = G::TP, LQ = G::LQ, NC = G::NC, CPL = G::CPL, RPI = G::RPI, NDMA = G::NDMA;
  constexpr int LPT = G::LPT, TPL = G::TPL, NPG = G::NPG;
  constexpr int kPSlots = TP / 2 + kWave;  // pair slots read + one dummy per lane

  __shared__ int32_t s_tbl[kSegTokens];
  __shared__ u32x4 s_q[GT][NC];
  // Two pipeline slots per wave, K and V, each [TP rows][NC chunks].
  __shared__ u32x4 s_k0[kWaves][TP][NC];
  __shared__ u32x4 s_v0[kWaves][TP][NC];
  __shared__ u32x4 s_k1[kWaves][TP][NC];
  __shared__ u32x4 s_v1[kWaves][TP][NC];
  __shared__ unsigned s_p[kWaves][kPSlots][8];
  __shared__ float s_max[kWaves][GT];
  __shared__ float s_sum[kWaves][GT];
  // After its last pass, a wave's partial output rows go into its own slot-0
  // buffers: the K half first, the V half for the heads that do not fit.
  auto s_acc = [&](int w, int h, int d) -> float& {
    constexpr int kHeadsInK = static_cast<int>(sizeof(s_k0[0]) / (D * sizeof(float)));
    static_assert(2 * kHeadsInK >= GT, "partial outputs must fit a slot");
    float* base = h < kHeadsInK ? reinterpret_cast<float*>(&s_k0[w][0][0])
                                : reinterpret_cast<float*>(&s_v0[w][0][0]) - kHeadsInK * D;
    return base[h * D + d];
  };

  const DecodeItem item = decode_item(a, head_chunks);
  if (!item.valid) return;
  const int seq = item.seq, part = item.part, ctx = item.ctx, kvh = item.kvh, chunk = item.chunk;
  const int nparts = max(1, (ctx + a.part_tokens - 1) / a.part_tokens);

  const int group = a.num_heads / a.num_kv_heads;
  const int h_first = kvh * group + chunk * GT;
  const int nh = min(GT, group - chunk * GT);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar branches
  const int tq = lane / LQ;    // token of this lane in the score phase
  const int pq = lane % LQ;    // its chunk set: pq, pq + LQ, ...
  const int sub = lane % LPT;  // value slice owned in the p.V phase
  const int grp = lane / LPT;  // value-row group in the p.V phase
  // Probability-pair slot written by this lane: the first lane of token 2j+1
  // holds the pair (2j, 2j+1) and writes slot j; every other lane writes a
  // slot nobody reads, so the store needs no branch.
  const int pslot = (lane % (2 * LQ) == LQ) ? lane / (2 * LQ) : TP / 2 + lane;

  // Stage the group's query rows in LDS (rows past the group are zero).
  {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(a.query) + (static_cast<int64_t>(seq) * a.num_heads + h_first) * D * 2);
    for (int i = tid; i < GT * NC; i += kDecodeThreads) {
      const int h = i / NC;
      s_q[h][i - h * NC] = h < nh ? qsrc[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m[GT], lsum[GT], acc[GT][8];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -__builtin_inff();
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int lbs = a.log2_block_size;
  const int off_mask = (1 << lbs) - 1;
  const char* kbase = static_cast<const char*>(a.key_cache);
  const char* vbase = static_cast<const char*>(a.value_cache);
  constexpr int64_t kRowBytes = G::RB;
  const int32_t* table = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks_per_seq;

  const int tok_begin = part * a.part_tokens;
  const int tok_end = min(tok_begin + a.part_tokens, ctx);
  for (int seg = tok_begin; seg < tok_end; seg += kSegTokens) {
    const int seg_end = min(seg + kSegTokens, tok_end);
    const int first_blk = seg >> lbs;
    const int nblk = ((seg_end - 1) >> lbs) - first_blk + 1;
    __syncthreads();  // also orders the query staging before its first read
    for (int i = tid; i < nblk; i += kDecodeThreads) {
      const int b = table[first_blk + i];
      s_tbl[i] = (b < 0 || b >= a.num_blocks) ? 0 : b;
    }
    __syncthreads();

    const int npass = (seg_end - seg + TP - 1) / TP;
    const int my_passes = npass > wave ? (npass - wave + kWaves - 1) / kWaves : 0;

    // DMA of this wave's pass `it` into one slot.  Rows past the segment are
    // clamped to its last token (read, then given probability 0).
    auto issue = [&](int it, u32x4 (*sk)[NC], u32x4 (*sv)[NC]) {
      const int t0 = seg + (it * kWaves + wave) * TP;
#pragma unroll
      for (int r = 0; r < NDMA; ++r) {
        const int row = r * RPI + lane / NC;
        const int slot = lane % NC;
        int t = t0 + row;
        t = t < seg_end ? t : seg_end - 1;
        const int64_t blk = s_tbl[(t >> lbs) - first_blk];
        const int64_t roff = ((blk * a.num_kv_heads + kvh) << lbs | (t & off_mask)) * kRowBytes;
        const int kchunk = (slot + G::rot(row)) % NC;
        dma16(kbase + roff + kchunk * 16, &sk[r * RPI][0]);
        dma16(vbase + roff + slot * 16, &sv[r * RPI][0]);
      }
    };

    // Scores, softmax and p.V of this wave's pass `it` from one slot.
    auto compute = [&](int it, u32x4 (*sk)[NC], u32x4 (*sv)[NC]) {
      const int t0 = seg + (it * kWaves + wave) * TP;
      const bool ok = t0 + tq < seg_end;
      u32x4 k[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) k[j] = sk[tq][(pq + LQ * j - G::rot(tq) + NC) % NC];
      float s[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const u32x4 qc = s_q[h][pq + LQ * j];
#pragma unroll
          for (int w = 0; w < 4; ++w) d = P::dot(qc[w], k[j][w], d);
        }
        s[h] = group_sum<LQ>(d);
      }

#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float sc = ok ? s[h] * scale_log2 : -__builtin_inff();
        if (__builtin_amdgcn_ballot_w64(sc > m[h] + kLazyMax) != 0) {  // wave-uniform
          const float m_new = fmaxf(m[h], wave_max(sc));
          const float alpha = exp2_fast(m[h] - m_new);  // 0 on the first update
          lsum[h] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
          m[h] = m_new;
        }
        const unsigned pb = P::round(exp2_fast(sc - safe_max(m[h])));
        lsum[h] += pq == 0 ? P::widen(pb) : 0.f;
        // lane (2j+1)*LQ takes token 2j's probability from lane 2j*LQ (same DPP row).
        const unsigned lo = static_cast<unsigned>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(pb), 0x110 + LQ, 0xF, 0xF, false));
        s_p[wave][pslot][h] = lo | (pb << 16);
      }
      wave_lds_sync();

#pragma unroll
      for (int pj = 0; pj < NPG; ++pj) {
        const int j = pj * TPL + grp;
        const u32x4 v1 = sv[2 * j][sub];
        const u32x4 v2 = sv[2 * j + 1][sub];
        unsigned pr[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) pr[h] = s_p[wave][j][h];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned lo = __builtin_amdgcn_perm(v2[w], v1[w], 0x05040100u);
          const unsigned hi = __builtin_amdgcn_perm(v2[w], v1[w], 0x07060302u);
#pragma unroll
          for (int h = 0; h < GT; ++h) {
            acc[h][2 * w] = P::dot(pr[h], lo, acc[h][2 * w]);
            acc[h][2 * w + 1] = P::dot(pr[h], hi, acc[h][2 * w + 1]);
          }
        }
      }
      wave_lds_sync();
    };

    // Two-slot pipeline over this wave's passes of the segment: the DMA of
    // the next pass is issued before waiting for (and computing) this one.
    if (my_passes > 0) issue(0, s_k0[wave], s_v0[wave]);
    for (int it = 0; it < my_passes; it += 2) {
      if (it + 1 < my_passes) {
        issue(it + 1, s_k1[wave], s_v1[wave]);
        wait_vmcnt<2 * NDMA>();
      } else {
        wait_vmcnt<0>();
      }
      wave_lds_sync();
      compute(it, s_k0[wave], s_v0[wave]);
      if (it + 1 >= my_passes) break;
      if (it + 2 < my_passes) {
        issue(it + 2, s_k0[wave], s_v0[wave]);
        wait_vmcnt<2 * NDMA>();
      } else {
        wait_vmcnt<0>();
      }
      wave_lds_sync();
      compute(it + 1, s_k1[wave], s_v1[wave]);
    }
  }

  // Per-wave totals (every lane shares the wave's running max m).
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    lsum[h] = wave_sum(lsum[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = across_groups_sum<LPT>(acc[h][e]);
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc(wave, h, sub * 8 + e) = acc[h][e];
      if (lane == 0) {
        s_max[wave][h] = m[h];
        s_sum[wave][h] = lsum[h];
      }
    }
  }
  __syncthreads();

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
      num = __builtin_fmaf(f, s_acc(w, h, d), num);
    }
    const int64_t row = static_cast<int64_t>(seq) * a.num_heads + h_first + h;
    if (nparts == 1) {
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

template <typename E, int D, int GT>
hipError_t launch_gt(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_heads / a.num_kv_heads;
  const int chunks = (group + GT - 1) / GT;
  const uint64_t n = decode_grid(a, chunks);
  if (n == 0) return hipSuccess;
  if (n > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_rows_kernel<E, D, GT>), dim3(static_cast<uint32_t>(n)),
                     dim3(kDecodeThreads), 0, stream, a, chunks, a.scale * kLog2e);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_heads / a.num_kv_heads;
  switch (group < kMaxHeadsPerWg ? group : kMaxHeadsPerWg) {
    case 1: return launch_gt<E, D, 1>(a, stream);
    case 2: return launch_gt<E, D, 2>(a, stream);
    case 3: return launch_gt<E, D, 3>(a, stream);
    case 4: return launch_gt<E, D, 4>(a, stream);
    case 5: return launch_gt<E, D, 5>(a, stream);
    case 6: return launch_gt<E, D, 6>(a, stream);
    case 7: return launch_gt<E, D, 7>(a, stream);
    default: return launch_gt<E, D, 8>(a, stream);
  }
}

template <typename E>
hipError_t launch_e(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_d<E, 64>(a, stream);
    case 128: return launch_d<E, 128>(a, stream);
    default: return launch_d<E, 256>(a, stream);
  }
}

}  // namespace

hipError_t launch_decode_rows(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == PA_DTYPE_F16) return launch_e<F16>(a, stream);
  return launch_e<BF16>(a, stream);
}

}  // namespace pa

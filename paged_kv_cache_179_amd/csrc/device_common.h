// Device-side helpers shared by the gfx950 kernels of this library:
// element-type traits for 16-byte register groups, wavefront reductions built
// on DPP row operations, and small math wrappers over the hardware
// instructions.  wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Element types.  A "group" is the 16 bytes one lane moves per load.
// ---------------------------------------------------------------------------
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerGroup = 4;
  __device__ static inline float elem(const u32x4& g, int e) { return __uint_as_float(g[e]); }
  // sum_e q[e] * k[e] + acc over one group
  __device__ static inline float dot(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(__uint_as_float(q[e]), __uint_as_float(k[e]), acc);
    return acc;
  }
  __device__ static inline void store(void* base, int64_t idx, float v) {
    static_cast<float*>(base)[idx] = v;
  }
};

struct F16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerGroup = 8;
  __device__ static inline float elem(const u32x4& g, int e) {
    // A vector subscript is copied to a scalar before __builtin_bit_cast: bit-casting
    // the subscript expression itself reads element 0 with this compiler.
    const unsigned w = g[e >> 1];
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    return static_cast<float>(h[e & 1]);
  }
  __device__ static inline float dot(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned qw = q[w], kw = k[w];
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qw), __builtin_bit_cast(f16x2, kw), acc,
                                   false);
    }
    return acc;
  }
  __device__ static inline void store(void* base, int64_t idx, float v) {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(v);
  }
};

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerGroup = 8;
  __device__ static inline float elem(const u32x4& g, int e) {
    const unsigned w = g[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static inline float dot(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned qw = q[w], kw = k[w];
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw),
                                            __builtin_bit_cast(bf16x2, kw), acc, false);
    }
    return acc;
  }
  __device__ static inline void store(void* base, int64_t idx, float v) {
    static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(v);
  }
};

// ---------------------------------------------------------------------------
// Cross-lane helpers.
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, ..., 64); every lane of a
// group ends with the group's sum.  Within a 16-lane row the exchanges are
// DPP quad permutes and row mirrors; wider groups use a swizzle (xor 16) and
// a cross-half exchange (xor 32).
template <int N>
__device__ inline float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32)
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // xor 16
  if constexpr (N >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// Max / sum across groups: lanes l, l ^ N, l ^ 2N, ... (N = group width).
template <int N>
__device__ inline float across_groups_max(float x) {
#pragma unroll
  for (int off = N; off < kWave; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}
template <int N>
__device__ inline float across_groups_sum(float x) {
#pragma unroll
  for (int off = N; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Inclusive prefix sum over a wave (all 64 lanes active); *total gets the
// wave's sum.  Within each row of 16 lanes by DPP row shifts (lanes shifted
// in from outside the row add 0), then the row totals by lane reads.
__device__ inline int wave_scan(int x, int* total) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
  const int row = (threadIdx.x & (kWave - 1)) >> 4;
  *total = r0 + r1 + r2 + r3;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Offset used to exponentiate scores against a running max that may still be
// -inf (no finite score seen yet): then every exponent is -inf and gives 0.
__device__ inline float safe_max(float m) { return m == -__builtin_inff() ? 0.f : m; }

__device__ inline u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }

// Raw score q.k -> exponent of the kernels' base-2 softmax.  Plain attention:
// scale * s * log2(e).  With logit soft-capping at `cap` (the Gemma-2 style
// capping that the wLLM PyPI page, "Supported models", names as kernel work):
// cap * tanh(scale * s / cap) * log2(e), which bounds every score by +-cap.
// CAP selects the capped form at compile time, so that plain attention
// carries no tanh in its inner loop; WIN tells the kernels that mask scores
// one by one whether a sliding window's lower bound takes part (the window
// itself is in the kernel arguments).  The capped form evaluates
// tanh(y) = 1 - 2 / (1 + e^(2y)) with the hardware exp2 and reciprocal (a few
// instructions; absolute error a few 1e-7, which the cap scales), except in
// the fp32 kernel (PRECISE), which calls the library tanhf.
template <bool CAP, bool WIN, bool PRECISE = false>
struct ScoreMap {
  static constexpr bool kWindow = WIN;
  float mul;       // scale * log2(e); without capping the whole map
  float cap_log2;  // cap * log2(e) when capping
  float cap_in;    // 2 * scale / cap * log2(e): exp2 argument of e^(2y), y = scale * s / cap
  __device__ inline float operator()(float s) const {
    if constexpr (CAP) {
      if constexpr (PRECISE) return cap_log2 * tanhf(s * mul);
      return cap_log2 * (1.f - 2.f * __builtin_amdgcn_rcpf(1.f + exp2_fast(s * cap_in)));
    }
    return s * mul;
  }
  // operator()(s) - mu, the exponent of the softmax term of s against a max
  // mu (one fma without capping).
  __device__ inline float exponent(float s, float mu) const {
    if constexpr (CAP) return (*this)(s) - mu;
    return __builtin_fmaf(s, mul, -mu);
  }
};
template <bool CAP, bool WIN, bool PRECISE = false>
inline ScoreMap<CAP, WIN, PRECISE> make_score_map(float scale, float softcap) {
  if constexpr (CAP)
    return ScoreMap<CAP, WIN, PRECISE>{scale / softcap, softcap * kLog2e, 2.f * scale / softcap * kLog2e};
  return ScoreMap<CAP, WIN, PRECISE>{scale * kLog2e, 0.f, 0.f};
}

// Calls launch(map) with the compile-time form of the variant: capped or
// not, windowed or not.
template <typename F>
inline auto with_score_map(float scale, float softcap, int32_t window, F&& launch) {
  if (softcap > 0.f) {
    if (window > 0) return launch(make_score_map<true, true>(scale, softcap));
    return launch(make_score_map<true, false>(scale, softcap));
  }
  if (window > 0) return launch(make_score_map<false, true>(scale, softcap));
  return launch(make_score_map<false, false>(scale, softcap));
}

// Slot-mapped bit copy of new K/V rows into the pools.  Item i is 16-byte
// chunk i of the [token][KV head][chunk] inputs; it goes to its token's slot
// (block slot >> log2_bs, offset slot & (2^log2_bs - 1)) in the
// [block][KV head][offset][chunk] pools.  Tokens whose slot is negative or
// past the pool are skipped.  This thread takes items first, first + step, ...
__device__ inline void copy_rows_to_cache(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                                          u32x4* __restrict__ key_cache, u32x4* __restrict__ value_cache,
                                          const int64_t* __restrict__ slot_mapping, int64_t total,
                                          int32_t chunks_per_row, int32_t num_kv_heads, int32_t log2_bs,
                                          int64_t num_slots, int64_t first, int64_t step) {
  const int64_t per_token = static_cast<int64_t>(chunks_per_row) * num_kv_heads;
  for (int64_t i = first; i < total; i += step) {
    const int64_t n = i / per_token;
    const int64_t rem = i - n * per_token;  // = head * chunks_per_row + chunk
    const int64_t slot = slot_mapping[n];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot >> log2_bs;
    const int64_t off = slot & ((int64_t(1) << log2_bs) - 1);
    const int64_t head = rem / chunks_per_row;
    const int64_t chunk = rem - head * chunks_per_row;
    const int64_t dst = (((blk * num_kv_heads + head) << log2_bs) + off) * chunks_per_row + chunk;
    key_cache[dst] = key[i];
    value_cache[dst] = value[i];
  }
}

}  // namespace pa

// Paged-attention decode for grouped-query heads on the matrix cores.
//
// Same operation, work split, partition states and reduce as the other decode
// kernels: the PagedAttention decode of the wLLM PyPI page ("Features -- Core
// engine"), with the grouped-query mapping of the mini-vLLM README ("End-to-end
// throughput vs baselines": each query head reads its KV head).  When G query
// heads share a KV head, every cached element feeds 2G flops.  q.k and p.V
// are then a real [G x D] x [D x T] contraction, so both run on MFMA:
//
// * A pass is one 16-token tile.  Its K and V rows are copied HBM -> LDS by the
//   gfx950 global-to-LDS DMA, as in the vector kernel: two slots per wave,
//   with the next pass in flight while this one is computed (three slots and
//   two passes in flight for E4M3 caches, whose passes are half the bytes).
//   The block id of a pass comes through a scalar load, so the only
//   vector-memory operations in flight are the DMAs that the explicit waits
//   count; the block's rows are the DMA's wave-uniform base, each lane adding
//   a 32-bit offset.
// * E4M3 caches: keys are widened to 16 bits in registers, right before the
//   score MFMAs; values into a per-wave 16-bit tile in LDS that the
//   transposing reads below use.
// * Scores: S^T = K Q^T with v_mfma_f32_16x16x32_{bf16,f16}.  The A operand is
//   the tile's key rows, one 16-byte LDS read per lane per 32 dims.  The B
//   operand is the group's query rows, loaded once into registers; up to 16
//   heads, unused heads are zero.  Lane l ends up with the scores of head
//   l % 16 for tokens 4 * (l / 16) + 0..3.
// * Probabilities, rounded to the cache type, are then already laid out as
//   the B operand of O^T += V^T P^T with v_mfma_f32_16x16x16: no exchange
//   between lanes.  The A operand V^T comes from LDS through the gfx950
//   transposing read (ds_read_b64_tr_b16): four tokens of one value column
//   per lane.  One more MFMA against a ones operand sums the same rounded
//   probabilities for the denominator.
// * Online softmax in base 2 with lazy rescaling.  The running max of a head
//   only moves when a score passes it by more than 2^8, so probabilities stay
//   <= 256.
// * Key and value rows are stored in LDS with their 16-byte chunks rotated
//   per row: chunk c of row t at (c - 2t) mod NC (keys at head_dim 64:
//   (c - t) mod 8; values: (c - (t & ~1)) mod 8).  Measured with the LDS
//   bank-conflict counter, a key operand read then costs what a contiguous
//   16-byte read does (a shift of t costs twice that), and so does a
//   transposing value read.
//
// The kernel is persistent: as many workgroups as fit on the device, each
// looping over work units (one (sequence, partition) item of the plan, one KV
// head, up to 16 of its query heads) of the longest-first plan: statically in
// alternating order (units b, 2 grid - 1 - b, 2 grid + b, ...), or, in
// launches of more than one round, from the third unit on whichever is next
// in a device-wide queue.  Calls small enough that every (sequence,
// partition, head chunk) slot has a workgroup skip the plan: each workgroup
// takes the slot its index names (the static plan).  The workgroup's waves
// (eight at head_dim 128 over 16-bit caches, four otherwise) take the unit's
// 16-token passes in turn and merge through LDS at the end of the unit; the
// first pass of the next unit is already in flight by then.  Group units
// (a partition several sequences' tables share, for all their query rows)
// are described with their code below.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "decode_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Waves of one workgroup.  Eight at head_dim 128, so that one workgroup holds
// a CU and its waves, all of the same age, get the same share of the memory
// pipeline (two workgroups on one CU do not: the older one's loads issue
// first, and the younger one streams at about half its rate).  Four at 256,
// where eight would not fit the LDS, and at 64, where four workgroups share a
// CU and small launches fill the device in one round; four for E4M3 caches,
// whose three pipeline slots per wave would leave room for one workgroup of
// eight (measured slower: llama2-shaped fp8 decode 0.46 against 0.40-0.44 ms).
template <int D, bool KV8>
constexpr int waves_for() {
  return D == 128 && !KV8 ? 8 : 4;
}
constexpr int kTile = 16;       // tokens per pass
constexpr int kHeadTile = 16;   // query heads per workgroup (MFMA N)
// Launches of at least this many rounds of the grid take their units from a
// queue rather than in a fixed order.
constexpr int kQueueRounds = 1;
constexpr float kLazyMax = 8.f; // log2 of the largest unnormalised probability

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Mma;
template <>
struct Mma<BF16> {
  static constexpr unsigned kOnePair = 0x3F803F80u;
  __device__ static inline f32x4 qk(const u32x4& k, const u32x4& q, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
  __device__ static inline f32x4 pv(const u32x2& v, const u32x2& p, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v),
                                                     __builtin_bit_cast(s16x4, p), c, 0, 0, 0);
  }
  __device__ static inline unsigned pack(float lo, float hi) {
    const bf16x2 r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(unsigned, r);
  }
  // Two E4M3 values (the low or high half of w) as a bf16 pair, in one gfx950
  // scaled conversion with scale 1.  Exact: every E4M3 value (4 significant
  // bits, exponents -9..8) is a bf16 value.
  template <bool HIGH>
  __device__ static inline unsigned from_fp8(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HIGH));
  }
};
template <>
struct Mma<F16> {
  static constexpr unsigned kOnePair = 0x3C003C00u;
  __device__ static inline f32x4 qk(const u32x4& k, const u32x4& q, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
  }
  __device__ static inline f32x4 pv(const u32x2& v, const u32x2& p, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, v),
                                                 __builtin_bit_cast(f16x4, p), c, 0, 0, 0);
  }
  __device__ static inline unsigned pack(float lo, float hi) {
    const f16x2 r = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(unsigned, r);
  }
  // Two E4M3 values as an fp16 pair (scaled conversion, scale 1); every E4M3
  // value is an fp16 value, so this is exact.
  template <bool HIGH>
  __device__ static inline unsigned from_fp8(unsigned w) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HIGH));
  }
};

template <int D>
struct TileGeo {
  static constexpr int NC = D / 8;           // 16-byte chunks per row
  static constexpr int RB = 2 * D;           // row bytes
  static constexpr int RPI = 1024 / RB;      // rows per DMA instruction
  static constexpr int NDMA = kTile / RPI;   // DMA instructions per pass, K or V
  static constexpr int KB = D / 32;          // q.k MFMAs per pass
  static constexpr int MT = D / 16;          // p.V MFMAs per pass
  // Key and query rows: chunk c of row t sits at (c - rot_k(t)) mod NC.  A
  // shift of 2 t, not t: with a shift of t the 16-byte reads of one MFMA
  // operand (16 rows, one chunk column each) take twice the LDS cycles of a
  // contiguous read, with 2 t (and for the value rows' 2 t) they take the same.
  __device__ static inline int rot_k(int t) { return D == 64 ? t % NC : (2 * t) % NC; }
  __device__ static inline int rot_v(int t) { return D == 64 ? (t & ~1) % NC : (2 * t) % NC; }
};

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48.  Each swap hands a lane its own
// value and its partner's (in some order), so the max of the two is the pair max.
__device__ inline float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Read-only data loaded through the scalar unit: the work plan, its length and
// the block tables.  Scalar loads are counted by lgkmcnt, apart from the
// vector-memory counter that orders the DMA pipeline.
typedef __attribute__((address_space(4))) const int32_t cint;

template <typename T>
__device__ inline T scalar_ptr(const void* p) {
  return reinterpret_cast<T>(reinterpret_cast<uintptr_t>(p));
}

// One work unit: one (sequence, partition) item of the plan, for one KV head
// and one chunk of up to 16 of its query heads.  All fields are wave-uniform.
struct Unit {
  bool valid;
  int seq, kvh, h_first, nh;
  int tb, te, ctx;  // token range [tb, te) of the item (tb a multiple of 16); context length
  int lo;           // first attended token (sliding window); tokens below it are masked
  int span;         // partitions joined in the item (its state goes to the first)
  bool single;      // the sequence has one partition: write the output directly
  int mine;         // passes of this wave (passes w, w + 4, ... of the unit)
  bool group;       // a shared partition for several sequences: nh = their query rows
  int moff;         // group: the item's run in a.members (seq = its first member)
};

// GROUPS: the launch's plan may hold group items (its search for shared
// partitions ran).  Launches without them use a copy of the kernel with no
// group path compiled in.
template <typename E, int D, typename S, bool KV8, bool GROUPS>
__global__ __launch_bounds__((waves_for<D, KV8>() * kWave)) void decode_mfma_kernel(DecodeArgs a, int32_t head_chunks,
                                                                            S score) {
  constexpr int kWaves = waves_for<D, KV8>();
  constexpr int kThreads = kWaves * kWave;
  using M = Mma<E>;
  using G = TileGeo<D>;
  constexpr int NC = G::NC, RB = G::RB, RPI = G::RPI, KB = G::KB, MT = G::MT;
  // Cached rows: 2 D bytes (16-bit) or D bytes (E4M3, converted in LDS to the
  // 16-bit tile the MFMAs read).
  constexpr int CRB = KV8 ? D : RB;            // cached row bytes
  constexpr int CNC = CRB / 16;                // 16-byte chunks per cached row
  constexpr int CRPI = 1024 / CRB;             // cached rows per DMA instruction
  constexpr int NDMA = kTile / CRPI;           // DMA instructions per pass, K or V
  constexpr int NQ = kHeadTile * RB / 1024;  // DMA instructions per query tile

  // Per wave, NS pipeline slots, each a key tile and a value tile of
  // [kTile rows][CNC chunks].  16-bit caches: two slots, one pass in flight
  // while the other is computed; a slot is exactly one wave's partial output
  // [16 heads][D] in fp32, which is where that goes at the end of a unit.
  // E4M3 caches: a pass is half the bytes, so three slots keep two passes in
  // flight (the bytes in flight per wave of the 16-bit kernel).
  constexpr int NS = KV8 ? 3 : 2;
  // Group units (see below) exist for 16-bit caches and for E4M3 caches at
  // head_dim 128, in launches whose plan may hold them.  Compiled in, the
  // group path's registers crowd the regular path's: measured at E4M3 64 and
  // 256, TinyLlama-shaped fp8 decode 5% slower, Gemma-shaped 2.5%; 16-bit
  // TinyLlama-shaped decode (static plan) 23.5-23.7 against 22.8-23.0 us.
  constexpr bool kGroupUnits = GROUPS && (!KV8 || D == 128);
  __shared__ u32x4 s_kv[kWaves][NS][2][kTile][CNC];
  // E4M3 caches: each wave's value tile of the pass it computes, widened to
  // 16 bits and rotated as the 16-bit value slots are (keys are widened in
  // registers).  At the end of a unit it holds heads 0-7 of the wave's
  // partial output, and a free slot heads 8-15.
  __shared__ u32x4 s_cv[KV8 ? kWaves : 1][kTile][KV8 ? NC : 1];
  // Query tile of the current unit and of the next one.
  __shared__ u32x4 s_q[2][kHeadTile][NC];
  __shared__ float s_max[kWaves][kHeadTile];
  __shared__ float s_sum[kWaves][kHeadTile];
  __shared__ int s_part[kWaves];
  // The workgroup's unit after the next one, from the queue.  Written by
  // thread 0 before a barrier and read by every wave after it; the next write
  // comes after the next unit's first barrier, so one copy is enough.
  __shared__ int s_next;
  static_assert(sizeof(s_kv[0][0]) == (KV8 ? kHeadTile / 2 : kHeadTile) * D * sizeof(float),
                "partial output fills a slot");
  static_assert(!KV8 || sizeof(s_cv[0]) == kHeadTile / 2 * D * sizeof(float),
                "half the partial output fills the value tile");
  // Partial output row of wave w, head h, when the wave's free slot is `sl`.
  auto part_row = [&](int w, int sl, int h) -> float* {
    if constexpr (KV8) {
      if (h < kHeadTile / 2) return reinterpret_cast<float*>(&s_cv[w][0][0]) + h * D;
      return reinterpret_cast<float*>(&s_kv[w][sl][0][0][0]) + (h - kHeadTile / 2) * D;
    }
    return reinterpret_cast<float*>(&s_kv[w][sl][0][0][0]) + h * D;
  };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hl = lane & 15;  // head (scores, outputs); key row (score A operand)
  const int g4 = lane >> 4;  // 16-lane row of the wave

  const int per = a.num_kv_heads * head_chunks;
  // Static plan: one slot per (sequence, partition, head chunk), one per
  // workgroup; workgroup 0 leaves the counts the reduce reads (items of one
  // partition, no group items).
  const bool stat = a.static_plan != 0;
  if (stat && blockIdx.x == 0 && threadIdx.x == 0) {
    a.plan_count[0] = a.num_seqs * a.num_parts;
    a.plan_count[1] = 0;
    a.plan_count[2] = 0;
    a.plan_count[3] = 0;
  }
  const int n_units = stat ? a.num_seqs * a.num_parts * per : *scalar_ptr<cint*>(a.plan_count) * per;
  const int u = blockIdx.x;
  if (u >= n_units) return;
  // Workgroup b of N takes units b and 2 N - 1 - b first.  Launches of more
  // than one round of the grid then hand out the units from 2 N on in plan
  // order from a counter of units taken, plan_count[2], which the plan kernel
  // zeroes, so that the workgroups that run fast take more of the short units
  // at the end (per-workgroup traces show rates apart by up to 2x, so a fixed
  // order leaves a long tail).  A workgroup takes one per unit it starts from
  // its second on and stops at the first past the end, so every workgroup
  // leaves the loop.  (Without the queue, in round r a workgroup takes unit
  // r N + b, or r N + N - 1 - b in odd rounds: over the longest-first plan,
  // one that drew a short unit in one round draws a long one in the next.)
  const int NG = static_cast<int>(gridDim.x);
  const bool queued = !stat && n_units >= kQueueRounds * NG;
  int32_t* const queue = a.plan_count + 2;
  int rnd = 1;  // round of nxt
  auto next_unit = [&]() {
    if (queued) return __builtin_amdgcn_readfirstlane(s_next);
    ++rnd;
    return rnd * NG + ((rnd & 1) ? NG - 1 - u : u);
  };

  const int group = a.num_heads / a.num_kv_heads;
  const int P = a.part_tokens;
  const int lbs = a.log2_block_size;
  const int off_mask = (1 << lbs) - 1;
  const char* kbase = static_cast<const char*>(a.key_cache);
  const char* vbase = static_cast<const char*>(a.value_cache);
  const char* qbase = static_cast<const char*>(a.query);
  cint* plan = scalar_ptr<cint*>(a.plan);  // [item][seq, part, run, ctx]
  cint* tables = scalar_ptr<cint*>(a.block_tables);
  cint* ctx_lens = scalar_ptr<cint*>(a.context_lens);
  cint* members = scalar_ptr<cint*>(a.members);

  auto info = [&](int uu) {
    Unit x;
    x.valid = uu < n_units;
    const int j = x.valid ? uu / per : 0;
    const int r = x.valid ? uu - j * per : 0;
    int pfirst;     // the item's first partition
    int members_n = 0;  // group item: its sequences
    if (stat) {
      // Slot j: partition p = j / num_seqs of sequence ((j % num_seqs) + p
      // ceil(num_seqs / num_parts)) % num_seqs, when it holds attended tokens
      // (a sequence with an empty context keeps partition 0, whose output
      // rows are zeros).  Workgroups go round-robin to the 8 XCDs and round
      // each XCD's CUs, so workgroups 256 apart share a CU (the timings here
      // bear that out): without the rotation by p, partition-major slots of 64 sequences x 4 KV heads
      // put all four partitions of one sequence on one CU (TinyLlama-shaped
      // decode 25.8 us against 24.0 with the rotation; sequence-major slots
      // 26.3 us).
      pfirst = j / a.num_seqs;
      x.seq = j - pfirst * a.num_seqs;
      x.seq = (x.seq + pfirst * ((a.num_seqs + a.num_parts - 1) / a.num_parts)) % a.num_seqs;
      x.ctx = max(0, min(ctx_lens[x.seq], a.ctx_limit));
      const int p0 = S::kWindow ? window_start(a, x.ctx) / P : 0;
      const int p1 = max(1, (x.ctx + P - 1) / P);
      x.valid = x.valid && pfirst >= p0 && pfirst < p1;
      x.span = 1;
      x.single = p1 - p0 <= 1;
      x.group = false;
    } else {
      x.seq = plan[4 * static_cast<int64_t>(j)];
      pfirst = plan[4 * static_cast<int64_t>(j) + 1];
      const int span_word = plan[4 * static_cast<int64_t>(j) + 2];
      x.ctx = plan[4 * static_cast<int64_t>(j) + 3];
      x.span = span_word & 0xff;
      x.single = (span_word >> 8) & 1;
      x.group = kGroupUnits && ((span_word >> 9) & 1);
      // A group item in a launch without the group path cannot come from
      // this library's plan (the host gives both the same flags); dropped
      // rather than read as a sequence.
      if (!kGroupUnits && ((span_word >> 9) & 1)) x.valid = false;
      members_n = span_word >> 16;
    }
    x.kvh = r / head_chunks;
    const int chunk = r - x.kvh * head_chunks;
    x.h_first = x.kvh * group + chunk * kHeadTile;
    x.nh = min(kHeadTile, group - chunk * kHeadTile);
    x.moff = 0;
    if (x.group) {  // one head chunk per KV head; rows = members x group
      x.moff = x.seq;
      x.seq = members[x.moff];
      x.nh = members_n * group;
    }
    const int pb = pfirst * P;
    x.lo = window_start(a, x.ctx);
    // Passes start on a 16-token boundary so that each one stays inside one
    // block; the tokens before the window in the first pass are masked.
    x.tb = S::kWindow ? max(pb, x.lo & ~(kTile - 1)) : pb;
    x.te = min(pb + x.span * P, x.ctx);
    const int npass = (x.valid && x.te > x.tb) ? (x.te - x.tb + kTile - 1) / kTile : 0;
    x.mine = npass > wave ? (npass - wave + kWaves - 1) / kWaves : 0;
    return x;
  };

  // Per-lane LDS offsets of the compute reads (bytes within one tile).  Key
  // and query rows share the rotation (chunk c of row t at (c - rot_k(t)) mod NC).
  int koff[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) koff[kb] = hl * RB + ((4 * kb + g4 - G::rot_k(hl) + NC) % NC) * 16;
  // E4M3 keys: lane (hl, g4) reads the 16 key bytes of dims 16 c ..+15,
  // c = 4 j + g4, for the MFMA pair 2 j (dims ..+7) and 2 j + 1 (dims 8..15);
  // the query operands of that pair are the matching 16-bit chunks 2 c and
  // 2 c + 1.  Raw key rows are stored with chunk c at (c - rot8(t)) mod CNC,
  // rot8(t) = t CNC / 16, so the 16 rows of a read cover all 64 banks.
  int k8off[KB / 2 > 0 ? KB / 2 : 1];
  if constexpr (KV8) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      koff[kb] = hl * RB + ((2 * (4 * (kb / 2) + g4) + (kb & 1) - G::rot_k(hl) + NC) % NC) * 16;
#pragma unroll
    for (int j = 0; j < KB / 2; ++j) k8off[j] = hl * CRB + ((4 * j + g4 - hl * CNC / 16 + CNC) % CNC) * 16;
  }
  int voff[MT];
  {
    const int vrow = 4 * g4 + (hl >> 2);
    const int q4 = hl & 3;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      voff[mt] = vrow * RB + ((2 * mt + (q4 >> 1) - G::rot_v(vrow) + NC) % NC) * 16 + (q4 & 1) * 8;
  }

  // DMA of pass k of unit x (tokens x.tb + (4 k + wave) * 16 ...) into slot
  // `sl`.  Rows past the partition are clamped to its last token (read, then
  // given probability 0).
  auto issue = [&](const Unit& x, int k, int sl) {
    const int t0 = x.tb + (k * kWaves + wave) * kTile;
    const char* kd = reinterpret_cast<const char*>(&s_kv[wave][sl][0][0][0]);
    const char* vd = reinterpret_cast<const char*>(&s_kv[wave][sl][1][0][0]);
    const int64_t trow = static_cast<int64_t>(x.seq) * a.max_blocks_per_seq;
    if constexpr (KV8) {
      // E4M3 key rows land rotated by rot8(row) (see k8off); value rows land
      // unrotated, since the widening pass reads them in order.  As below,
      // the table read is a scalar load for blocks of 16 or more tokens: a
      // vector load here would make every DMA wait for all earlier ones.
      if (lbs >= 4) {
        int b = tables[trow + (t0 >> lbs)];
        b = (b < 0 || b >= a.num_blocks) ? 0 : b;
        const int64_t head_off = ((static_cast<int64_t>(b) * a.num_kv_heads + x.kvh) << lbs) * CRB;
        // The block's rows of this KV head as a wave-uniform base, a 32-bit
        // offset per lane (blocks of at most 256 tokens).
#pragma unroll
        for (int r = 0; r < NDMA; ++r) {
          const int row = r * CRPI + lane / CNC;
          const int pos = lane % CNC;
          const int t = min(t0 + row, x.te - 1);
          const uint32_t roff = static_cast<uint32_t>(t & off_mask) * CRB;
          dma16_sv(kbase + head_off, roff + ((pos + row * CNC / 16) % CNC) * 16, kd + r * 1024);
          dma16_sv(vbase + head_off, roff + pos * 16, vd + r * 1024);
        }
      } else {
#pragma unroll
        for (int r = 0; r < NDMA; ++r) {
          const int row = r * CRPI + lane / CNC;
          const int pos = lane % CNC;
          const int t = min(t0 + row, x.te - 1);
          int b = a.block_tables[trow + (t >> lbs)];
          b = (b < 0 || b >= a.num_blocks) ? 0 : b;
          const int64_t roff =
              (((static_cast<int64_t>(b) * a.num_kv_heads + x.kvh) << lbs) | (t & off_mask)) * CRB;
          dma16(kbase + roff + ((pos + row * CNC / 16) % CNC) * 16, kd + r * 1024);
          dma16(vbase + roff + pos * 16, vd + r * 1024);
        }
      }
      return;
    }
    if (lbs >= 4) {
      // The 16 tokens lie in one block: one scalar table read per pass.  The
      // block's rows of this KV head as a wave-uniform base, a 32-bit offset
      // per lane (blocks of at most 256 tokens).
      int b = tables[trow + (t0 >> lbs)];
      b = (b < 0 || b >= a.num_blocks) ? 0 : b;
      const int64_t head_off = ((static_cast<int64_t>(b) * a.num_kv_heads + x.kvh) << lbs) * RB;
#pragma unroll
      for (int r = 0; r < NDMA; ++r) {
        const int row = r * RPI + lane / NC;
        const int pos = lane % NC;
        const int t = min(t0 + row, x.te - 1);
        const uint32_t roff = static_cast<uint32_t>(t & off_mask) * RB;
        dma16_sv(kbase + head_off, roff + ((pos + G::rot_k(row)) % NC) * 16, kd + r * RPI * RB);
        dma16_sv(vbase + head_off, roff + ((pos + G::rot_v(row)) % NC) * 16, vd + r * RPI * RB);
      }
    } else {
      // Small blocks: each row reads its own table entry (vector loads; the
      // compiler then waits for them before the DMA, which is correct but
      // drains the pipeline -- a layout kept for completeness, not speed).
#pragma unroll
      for (int r = 0; r < NDMA; ++r) {
        const int row = r * RPI + lane / NC;
        const int pos = lane % NC;
        const int t = min(t0 + row, x.te - 1);
        int b = a.block_tables[trow + (t >> lbs)];
        b = (b < 0 || b >= a.num_blocks) ? 0 : b;
        const int64_t roff =
            (((static_cast<int64_t>(b) * a.num_kv_heads + x.kvh) << lbs) | (t & off_mask)) * RB;
        dma16(kbase + roff + ((pos + G::rot_k(row)) % NC) * 16, kd + r * RPI * RB);
        dma16(vbase + roff + ((pos + G::rot_v(row)) % NC) * 16, vd + r * RPI * RB);
      }
    }
  };

  // DMA of unit x's query rows into query buffer `qb` (wave 0 only).  Rows
  // past the head chunk repeat its last row; their outputs are never written.
  auto issue_q = [&](const Unit& x, int qb) {
    const char* qd = reinterpret_cast<const char*>(&s_q[qb][0][0]);
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      const int row = r * RPI + lane / NC;
      const int pos = lane % NC;
      const int h = min(row, x.nh - 1);
      const char* src = qbase + (static_cast<int64_t>(x.seq) * a.num_heads + x.h_first + h) * RB;
      dma16(src + ((pos + G::rot_k(row)) % NC) * 16, qd + r * RPI * RB);
    }
  };

  // 16 E4M3 values (one 16-byte chunk) as two 16-bit chunks: dims 0..7 and 8..15.
  auto widen = [](const u32x4& w, u32x4& lo, u32x4& hi) {
    lo = u32x4{M::template from_fp8<false>(w[0]), M::template from_fp8<true>(w[0]),
               M::template from_fp8<false>(w[1]), M::template from_fp8<true>(w[1])};
    hi = u32x4{M::template from_fp8<false>(w[2]), M::template from_fp8<true>(w[2]),
               M::template from_fp8<false>(w[3]), M::template from_fp8<true>(w[3])};
  };

  // E4M3 caches: widen this wave's value tile in slot `sl` into its 16-bit
  // tile.  Lane l takes 16-byte chunks l, l + 64, ... (chunk q: row q / CNC,
  // dims 16 (q % CNC) ..+15) and writes the two 16-bit chunks they become at
  // their rotated places.
  auto convert = [&](int sl) {
    if constexpr (KV8) {
#pragma unroll
      for (int i = 0; i < kTile * CNC / 64; ++i) {
        const int q = lane + 64 * i;
        const int t = q / CNC;
        const int c = 2 * (q % CNC);
        u32x4 lo, hi;
        widen(s_kv[wave][sl][1][t][q % CNC], lo, hi);
        s_cv[wave][t][(c - G::rot_v(t) + NC) % NC] = lo;
        s_cv[wave][t][(c + 1 - G::rot_v(t) + NC) % NC] = hi;
      }
      wave_lds_sync();
    }
  };

  const u32x2 ones = {M::kOnePair, M::kOnePair};
  f32x4 acc[MT];
  f32x4 lacc;
  float m;

  auto compute = [&](const Unit& x, int k, int sl, int qb) {
    const int t0 = x.tb + (k * kWaves + wave) * kTile;
    const char* kt = reinterpret_cast<const char*>(&s_kv[wave][sl][0][0][0]);
    const char* vt = KV8 ? reinterpret_cast<const char*>(&s_cv[wave][0][0]) : kt + kTile * RB;
    const char* qt = reinterpret_cast<const char*>(&s_q[qb][0][0]);

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KV8) {
#pragma unroll
      for (int j = 0; j < KB / 2; ++j) {
        u32x4 lo, hi;
        widen(*reinterpret_cast<const u32x4*>(kt + k8off[j]), lo, hi);
        s = M::qk(lo, *reinterpret_cast<const u32x4*>(qt + koff[2 * j]), s);
        s = M::qk(hi, *reinterpret_cast<const u32x4*>(qt + koff[2 * j + 1]), s);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s = M::qk(*reinterpret_cast<const u32x4*>(kt + koff[kb]),
                  *reinterpret_cast<const u32x4*>(qt + koff[kb]), s);
    }

    // Lane (hl, g4) holds head hl's scores of tokens t0 + 4 g4 + i.
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g4 + i;
      sc[i] = ((!S::kWindow || t >= x.lo) && t < x.te) ? score(s[i]) : -__builtin_inff();
    }
    const float mx = max_across_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazyMax) != 0) {  // wave-uniform
      const float m_new = fmaxf(m, mx);
      const float alpha = exp2_fast(m - m_new);  // 0 on the first update
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
      lacc *= alpha;
      m = m_new;
    }
    const u32x2 pb = {M::pack(exp2_fast(sc[0] - m), exp2_fast(sc[1] - m)),
                      M::pack(exp2_fast(sc[2] - m), exp2_fast(sc[3] - m))};
    lacc = M::pv(ones, pb, lacc);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + voff[mt]));
      acc[mt] = M::pv(__builtin_bit_cast(u32x2, v), pb, acc[mt]);
    }
    wave_lds_sync();
  };

  // Merge of the four waves' partial states of unit x (slot `pr` of each
  // wave is free and holds its partial output, or half of it) and the output
  // or workspace writes.
  // take: also take the unit after the next one from the queue (into s_next).
  auto finish = [&](const Unit& x, int pr, bool take) {
    float* part_out = part_row(wave, pr, hl);
    if (hl < x.nh) {  // the merge reads only the unit's heads
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4*>(part_out + 16 * mt + 4 * g4) = acc[mt];
    }
    if (lane < kHeadTile) {
      s_max[wave][hl] = m;
      s_sum[wave][hl] = lacc[0];
    }
    if (lane == 0) s_part[wave] = pr;
    __syncthreads();
    // Taken before the merge, so that the atomic's latency hides behind it.
    int taken = 0;
    if (take && tid == 0) taken = 2 * NG + atomicAdd(queue, 1);
    const int nparts = max(1, (x.ctx + P - 1) / P);
    const int part = x.tb / P;
    const int part_end = min(part + x.span, nparts);
    // Four consecutive dims of one head per thread and step.
    constexpr int D4 = D / 4;
    for (int idx = tid; idx < x.nh * D4; idx += kThreads) {
      const int h = idx / D4;
      const int d = (idx - h * D4) * 4;
      float mw[kWaves];
      float mx = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = s_max[w][h];
        mx = fmaxf(mx, mw[w]);
      }
      const float mu = safe_max(mx);
      float den = 0.f;
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2_fast(mw[w] - mu);
        den = __builtin_fmaf(f, s_sum[w][h], den);
        num += f * *reinterpret_cast<const f32x4*>(part_row(w, s_part[w], h) + d);
      }
      if constexpr (KV8) num *= a.v_scale;  // values were read without their scale
      const int64_t row = static_cast<int64_t>(x.seq) * a.num_heads + x.h_first + h;
      if (x.single) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        if (den != 0.f) o = num / den;
        const u32x2 packed = {M::pack(o[0], o[1]), M::pack(o[2], o[3])};
        *reinterpret_cast<u32x2*>(static_cast<char*>(a.out) + (row * D + d) * 2) = packed;
      } else {
        const int64_t ws = row * a.num_parts + part;
        *reinterpret_cast<f32x4*>(a.ws_acc + ws * D + d) = num;
        if (d == 0) {
          a.ws_max[ws] = mx;
          a.ws_sum[ws] = den;
          for (int q = part + 1; q < part_end; ++q) {  // joined partitions: empty states
            a.ws_max[ws + q - part] = -__builtin_inff();
            a.ws_sum[ws + q - part] = 0.f;
          }
        }
      }
    }
    if (take && tid == 0) s_next = taken;
    __syncthreads();
  };

  // Group units: one partition that the block tables of several sequences
  // share, for all their query rows (member m, head j -> row m * group + j;
  // GT row tiles of 16 per wave, so the partition is read once for up to
  // decode_group_rows(D) rows).  Every wave computes every pass: wave w still
  // DMAs passes w, w + kWaves, ... into its own slots, and after each round of
  // kWaves passes (one per wave) each wave runs its row tiles over all of
  // them.  Query rows come straight from global memory into registers.  A
  // row's running max moves only on its own scores (the rescale factor is 1
  // for the other rows of the tile, an exact no-op), so a row's result does
  // not depend on which rows share its tile.  Each wave writes its rows'
  // partition states itself: no merge across waves.
  //   Per-wave timestamps of a traced copy (16-bit caches, head_dim 128, 112
  // rows): a round of eight passes takes 10-16 K cycles of computing, each
  // pass a chain of dependent steps (LDS reads, score MFMAs, max across
  // lanes, exponentials, p.V MFMAs) of ~1,250 cycles per row tile.  Four
  // computing waves with two tiles each (half the LDS reads) were slower
  // (group units 32.6 against 29.5 us), as were two passes per step.
  constexpr int GCW = kWaves;                                    // computing waves
  constexpr int GT = decode_group_rows(D) / (GCW * kHeadTile);  // row tiles per wave
  static_assert(GT >= 1 && GT * GCW * kHeadTile == decode_group_rows(D), "group rows");
  u32x4 qr[GT][KB];     // score B operands of this lane's row, per tile
  f32x4 gacc[GT][MT];
  f32x4 glacc[GT];
  float gm[GT];
  int64_t grow[GT];     // this lane's row: sequence * num_heads + head, or -1
  int gtiles = 0;       // row tiles of the unit (wave-uniform)
  // Loads this wave's query rows of group unit x and clears their states.
  // The chunk of a row that lane (hl, g4) supplies to score MFMA kb matches
  // the key chunk that koff[kb] (k8off for E4M3 keys) gives the same lane.
  auto group_begin = [&](const Unit& x) {
    const int rows = x.nh;
    gtiles = (rows + kHeadTile - 1) / kHeadTile;
#pragma unroll
    for (int i = 0; i < GT; ++i) {
      const int r = (wave + GCW * i) * kHeadTile + hl;
      grow[i] = -1;
      if (r < rows) {
        const int mem = r / group;
        const int sq = a.members[x.moff + mem];
        grow[i] = static_cast<int64_t>(sq) * a.num_heads + x.kvh * group + (r - mem * group);
      }
      const char* qsrc = qbase + (grow[i] < 0 ? 0 : grow[i]) * RB;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int c = KV8 ? 2 * (4 * (kb / 2) + g4) + (kb & 1) : 4 * kb + g4;
        qr[i][kb] = grow[i] < 0 ? u32x4{0u, 0u, 0u, 0u} : load16(qsrc + c * 16);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) gacc[i][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      glacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      gm[i] = -__builtin_inff();
    }
  };
  // One pass of 16 tokens for this wave's row tiles: ka are the keys as score
  // A operands, vv the values as transposed p.V A operands.
  auto group_pass = [&](const u32x4 (&ka)[KB], const s16x4 (&vv)[MT]) {
#pragma unroll
    for (int i = 0; i < GT; ++i) {
      if (wave + GCW * i >= gtiles) continue;  // wave-uniform
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc = M::qk(ka[kb], qr[i][kb], sacc);
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = score(sacc[e]);
      const float mx = max_across_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      const bool up = mx > gm[i] + kLazyMax;  // this row's own decision
      if (__builtin_amdgcn_ballot_w64(up) != 0) {  // wave-uniform
        const float alpha = up ? exp2_fast(gm[i] - mx) : 1.f;  // 0 on the first update
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) gacc[i][mt] *= alpha;
        glacc[i] *= alpha;
        gm[i] = up ? mx : gm[i];
      }
      const u32x2 pb = {M::pack(exp2_fast(sc[0] - gm[i]), exp2_fast(sc[1] - gm[i])),
                        M::pack(exp2_fast(sc[2] - gm[i]), exp2_fast(sc[3] - gm[i]))};
      glacc[i] = M::pv(ones, pb, glacc[i]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) gacc[i][mt] = M::pv(__builtin_bit_cast(u32x2, vv[mt]), pb, gacc[i][mt]);
    }
  };
  // The partition states of this wave's rows of group unit x.
  auto group_store = [&](const Unit& x) {
    const int part = x.tb / P;
#pragma unroll
    for (int i = 0; i < GT; ++i) {
      if (wave + GCW * i >= gtiles || grow[i] < 0) continue;
      const int64_t ws = grow[i] * a.num_parts + part;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 o = gacc[i][mt];
        if constexpr (KV8) o *= a.v_scale;  // values were read without their scale
        *reinterpret_cast<f32x4*>(a.ws_acc + ws * D + 16 * mt + 4 * g4) = o;
      }
      if (g4 == 0) {
        a.ws_max[ws] = gm[i];
        a.ws_sum[ws] = glacc[i][0];
      }
    }
  };

  // Group unit over 16-bit caches: two slots per wave, so a round's DMA is
  // issued once the barrier that ends the previous round has passed.
  //   On entry this wave's pass 0 is in flight in `slot`; on exit the next
  // unit's first pass is in flight in `slot` and, for a regular next unit,
  // its query tile has landed in s_q[qb ^ 1] (as after a regular unit).
  auto group_unit = [&](const Unit& x, const Unit& nx, int& slot, int qb, bool take) {
    if constexpr (!KV8) {
      group_begin(x);
      auto gpass = [&](const char* kt) {  // a slot: keys, then values
        u32x4 ka[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) ka[kb] = *reinterpret_cast<const u32x4*>(kt + koff[kb]);
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        s16x4 vv[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          vv[mt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kt + kTile * RB + voff[mt]));
        group_pass(ka, vv);
      };
      const int npass = (x.te - x.tb) / kTile;  // full partition
      const int nround = (npass + kWaves - 1) / kWaves;  // the last one may be short
      // Where this wave's pass 0 lands (read after round 0's barrier; a wave
      // with no pass in a round still keeps its slot parity in step).
      if (lane == 0) s_part[wave] = slot;
      int gs[kWaves];
      // At least one round (a shared partition is a full one, of at least 64
      // tokens), written so that the compiler sees the wait below on every
      // path out of the query loads; otherwise it would wait for them, and so
      // for every DMA in flight, in the regular units' pass loop.
      int r = 0;
      do {
        wait_vmcnt<0>();  // this wave's pass of round r (and at r = 0 its query rows)
        __syncthreads();  // every wave's pass of round r; every wave done with round r - 1
        if (r == 0) {
#pragma unroll
          for (int w = 0; w < kWaves; ++w) gs[w] = __builtin_amdgcn_readfirstlane(s_part[w]);
        }
        if (r + 1 < nround) {
          if ((r + 1) * kWaves + wave < npass) issue(x, r + 1, slot ^ 1);
        } else {
          if (wave == 0 && nx.valid && !nx.group) issue_q(nx, qb ^ 1);  // before nx's pass 0
          if (nx.valid && nx.mine > 0) issue(nx, 0, slot ^ 1);
        }
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (r * kWaves + w < npass) gpass(reinterpret_cast<const char*>(&s_kv[w][(gs[w] + r) & 1][0][0][0]));
        slot ^= 1;
      } while (++r < nround);
      // The next regular unit's query tile has landed before the barrier below.
      if (wave == 0 && nx.valid && !nx.group) {
        if (nx.mine > 0) wait_vmcnt<2 * NDMA>();
        else wait_vmcnt<0>();
      }
      group_store(x);
      if (take && tid == 0) s_next = 2 * NG + atomicAdd(queue, 1);
      __syncthreads();  // slots free for the next unit; s_next published
    }
  };

  // Persistent loop over the workgroup's units (the plan being ordered
  // longest first, each round of the grid takes units of similar length).
  // Each wave keeps one
  // DMA in flight ahead of the pass it computes, and the first pass of the
  // next unit is issued before the current unit's merge, so its latency
  // overlaps the merge.  Wave 0 also stages the next unit's query rows; those
  // NQ DMAs are ordered before a pass's and waited with it.
  Unit cur = info(u);
  if (!cur.valid) return;  // a static slot past its sequence's context (workgroup-uniform)
  int qb = 0;
  int slot = 0;
  if constexpr (KV8) {
    if (wave == 0 && !cur.group) {
      issue_q(cur, 0);
      wait_vmcnt<0>();
    }
  } else {
    // The first pass goes out with the query tile, and only the query tile
    // is waited for before the barrier: one round trip, not two, before the
    // first pass can be computed.
    if (wave == 0 && !cur.group) issue_q(cur, 0);
    if (cur.mine > 0) issue(cur, 0, slot);
    if (wave == 0 && !cur.group) {
      if (cur.mine > 0) wait_vmcnt<2 * NDMA>();
      else wait_vmcnt<0>();
    }
  }
  __syncthreads();
  Unit nxt = info(2 * NG - 1 - u);
  if constexpr (KV8) {
    // Three slots.  A wave's passes, unit after unit, form one stream: pass i
    // of the stream uses slot i mod 3, and up to two passes are in flight
    // ahead of the one computed (reaching into the next unit at the end of
    // this one, so the merge overlaps them too).  Each wait leaves in flight
    // exactly the DMAs issued after the pass it waits for: two per later pass
    // and, for wave 0, the query tile if it was issued after that pass.
    int issued = 0, done = 0;  // passes of the stream issued, computed
    int ic = 0, in = 0;        // passes of cur, of nxt issued
    int isl = 0, csl = 0;      // slots of the next pass to issue, to compute
    int q_after = 0;           // wave 0: passes issued before the last query tile
    auto issue_next = [&]() -> bool {
      if (ic < cur.mine) {
        issue(cur, ic++, isl);
      } else if (nxt.valid && in < nxt.mine) {
        issue(nxt, in++, isl);
      } else {
        return false;
      }
      ++issued;
      isl = isl == NS - 1 ? 0 : isl + 1;
      return true;
    };
    // Waits until at most n DMAs are in flight (n a multiple of 2 NDMA; the
    // query tile is NQ = 2 NDMA).
    static_assert(NQ == 2 * NDMA, "query tile counts as one pass");
    auto wait_upto = [](int n) {
      if (n >= 6 * NDMA) wait_vmcnt<6 * NDMA>();
      else if (n >= 4 * NDMA) wait_vmcnt<4 * NDMA>();
      else if (n >= 2 * NDMA) wait_vmcnt<2 * NDMA>();
      else wait_vmcnt<0>();
    };
    // One pass of 16 E4M3 keys (slot tile kt) and their widened values (vt)
    // for this wave's group rows.
    auto gpass8 = [&](const char* kt, const char* vt) {
      u32x4 ka[KB];
#pragma unroll
      for (int j = 0; j < KB / 2; ++j) widen(*reinterpret_cast<const u32x4*>(kt + k8off[j]), ka[2 * j], ka[2 * j + 1]);
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      s16x4 vv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) vv[mt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + voff[mt]));
      group_pass(ka, vv);
    };
    // Group unit over E4M3 caches.  Before the transposing reads a value tile
    // must be widened: after the barrier that ends the previous round, each
    // wave widens the value tile of its own pass of this round into its 16-bit
    // tile, and a second barrier publishes the four.  Keys are widened in
    // registers.  Other waves read this wave's slots, so a slot is refilled
    // only after the barrier that ends the round which read it: before a
    // round's first barrier the wave's stream runs at most one pass ahead of
    // the pass it contributes, after it two.
    auto group_unit8 = [&](bool take) {
      const Unit& x = cur;
      group_begin(x);
      if (wave == 0 && nxt.valid && !nxt.group) {
        issue_q(nxt, qb ^ 1);
        q_after = issued;
      }
      if (lane == 0) s_part[wave] = csl;  // slot of this wave's pass 0 of x
      const int npass = (x.te - x.tb) / kTile;  // full partition
      const int nround = (npass + kWaves - 1) / kWaves;
      int gs[kWaves];
      // The query rows, and with them every pass issued so far, have landed
      // (a wait the compiler sees on every path, so that it adds none of its
      // own for the query registers inside the rounds).
      wait_vmcnt<0>();
      for (int r = 0; r < nround; ++r) {
        const bool own = r < x.mine;  // this wave's pass r of x is pass `done` of its stream
        while (issued - done < NS - 1 && issue_next()) {
        }
        if (own) wait_upto(2 * NDMA * (issued - done - 1) + (wave == 0 && q_after > done ? NQ : 0));
        __syncthreads();  // every wave's pass of round r landed; round r - 1 read by every wave
        if (r == 0) {
#pragma unroll
          for (int w = 0; w < kWaves; ++w) gs[w] = __builtin_amdgcn_readfirstlane(s_part[w]);
        }
        while (issued - done < NS && issue_next()) {
        }
        if (own) convert(csl);
        __syncthreads();  // the widened value tiles of round r
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (r * kWaves + w < npass)
            gpass8(reinterpret_cast<const char*>(&s_kv[w][(gs[w] + r) % NS][0][0][0]),
                   reinterpret_cast<const char*>(&s_cv[w][0][0]));
        if (own) {
          ++done;
          csl = csl == NS - 1 ? 0 : csl + 1;
        }
      }
      // The next query tile has landed before the barrier below.
      if (wave == 0 && nxt.valid && !nxt.group) wait_upto(2 * NDMA * (issued - q_after));
      group_store(x);
      if (take && tid == 0) s_next = 2 * NG + atomicAdd(queue, 1);
      __syncthreads();  // slots free for the next unit; s_next published
    };
    while (true) {
      if (kGroupUnits && cur.group) {
        if constexpr (kGroupUnits) group_unit8(queued && nxt.valid);
        if (!nxt.valid) break;
        cur = nxt;
        nxt = info(next_unit());
        qb ^= 1;
        ic = in;
        in = 0;
        continue;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      lacc = f32x4{0.f, 0.f, 0.f, 0.f};
      m = -__builtin_inff();
      if (wave == 0 && nxt.valid && !nxt.group) {
        issue_q(nxt, qb ^ 1);  // older than every pass of nxt
        q_after = issued;
      }
      for (int k = 0; k < cur.mine; ++k) {
        while (issued - done < NS && issue_next()) {
        }
        const int later = issued - done - 1;
        wait_upto(2 * NDMA * later + (wave == 0 && q_after > done ? NQ : 0));
        wave_lds_sync();
        convert(csl);
        compute(cur, k, csl, qb);
        ++done;
        csl = csl == NS - 1 ? 0 : csl + 1;
      }
      while (issued - done < NS - 1 && issue_next()) {
      }
      // The next query tile has landed before the merge's barrier.
      if (wave == 0 && nxt.valid && !nxt.group) wait_upto(2 * NDMA * (issued - q_after));
      // At most the two slots from csl on are in flight; the one before is free.
      finish(cur, csl == 0 ? NS - 1 : csl - 1, queued && nxt.valid);
      if (!nxt.valid) break;
      cur = nxt;
      nxt = info(next_unit());
      qb ^= 1;
      ic = in;
      in = 0;
    }
    return;
  }
  while (true) {
    if (cur.group) {
      group_unit(cur, nxt, slot, qb, queued && nxt.valid);
      if (!nxt.valid) break;
      cur = nxt;
      nxt = info(next_unit());
      qb ^= 1;
      continue;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    lacc = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -__builtin_inff();
    bool q_todo = wave == 0 && nxt.valid && !nxt.group;
    const bool next_first = nxt.valid && nxt.mine > 0;
    for (int k = 0; k < cur.mine; ++k) {
      if (k + 1 < cur.mine) {
        issue(cur, k + 1, slot ^ 1);
        if (q_todo) {
          issue_q(nxt, qb ^ 1);  // waited by the next iteration's wait
          q_todo = false;
          wait_vmcnt<2 * NDMA + NQ>();
        } else {
          wait_vmcnt<2 * NDMA>();
        }
      } else {
        if (q_todo) {
          issue_q(nxt, qb ^ 1);  // older than the pass below: waited with it
          q_todo = false;
        }
        if (next_first) {
          issue(nxt, 0, slot ^ 1);
          wait_vmcnt<2 * NDMA>();
        } else {
          wait_vmcnt<0>();
        }
      }
      wave_lds_sync();
      convert(slot);
      compute(cur, k, slot, qb);
      slot ^= 1;
    }
    if (cur.mine == 0) {
      if (q_todo) issue_q(nxt, qb ^ 1);
      if (next_first) {
        issue(nxt, 0, slot);
        wait_vmcnt<2 * NDMA>();
      } else {
        wait_vmcnt<0>();
      }
    }
    // Now only the next unit's first pass (if any) is in flight, in `slot`;
    // the next query tile has landed.
    finish(cur, slot ^ 1, queued && nxt.valid);
    if (!nxt.valid) break;
    cur = nxt;
    nxt = info(next_unit());
    qb ^= 1;
  }
}

// Workgroups of one persistent launch: as many as fit on the device at once.
template <typename E, int D, typename S, bool KV8, bool GROUPS>
int persistent_grid() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g > 0) return g;
  int ncu = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) ncu = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_kernel<E, D, S, KV8, GROUPS>,
                                                    waves_for<D, KV8>() * kWave, 0) != hipSuccess)
    per_cu = 1;
  g = std::max(1, ncu) * std::max(1, per_cu);
  cache[dev].store(g, std::memory_order_relaxed);
  return g;
}

// Whether a launch takes the kernel with the group path: only when the plan
// searched for shared partitions (no static plan, the share flag set).
inline bool mfma_groups(const DecodeArgs& a) { return a.static_plan == 0 && a.share != 0; }

template <typename E, int D, typename S, bool KV8>
int grid_g(bool groups) {
  if constexpr (!KV8 || D == 128) {
    if (groups) return persistent_grid<E, D, S, KV8, true>();
  }
  return persistent_grid<E, D, S, KV8, false>();
}

template <typename E, typename S, bool KV8>
int grid_s(int head_dim, bool groups) {
  switch (head_dim) {
    case 64: return grid_g<E, 64, S, KV8>(groups);
    case 128: return grid_g<E, 128, S, KV8>(groups);
    default: return grid_g<E, 256, S, KV8>(groups);
  }
}

// Scale of q.k before the score map: an E4M3 cache's K scale folds in here.
inline float qk_scale(const DecodeArgs& a) { return a.kv_fp8 ? a.scale * a.k_scale : a.scale; }

template <typename E>
int grid_e(const DecodeArgs& a) {
  return with_score_map(qk_scale(a), a.softcap, a.window, [&](auto map) {
    return a.kv_fp8 ? grid_s<E, decltype(map), true>(a.head_dim, mfma_groups(a))
                    : grid_s<E, decltype(map), false>(a.head_dim, mfma_groups(a));
  });
}

template <typename E, int D, bool KV8>
hipError_t launch_kv(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_heads / a.num_kv_heads;
  const int chunks = (group + kHeadTile - 1) / kHeadTile;
  const uint64_t n = decode_grid(a, chunks);
  if (n == 0) return hipSuccess;
  with_score_map(qk_scale(a), a.softcap, a.window, [&](auto map) {
    using S = decltype(map);
    auto go = [&](auto groups) {
      constexpr bool GR = decltype(groups)::value;
      const uint64_t grid = std::min<uint64_t>(n, static_cast<uint64_t>(persistent_grid<E, D, S, KV8, GR>()));
      hipLaunchKernelGGL((decode_mfma_kernel<E, D, S, KV8, GR>), dim3(static_cast<uint32_t>(grid)),
                         dim3(waves_for<D, KV8>() * kWave), 0, stream, a, chunks, map);
    };
    if constexpr (!KV8 || D == 128) {
      if (mfma_groups(a)) {
        go(std::true_type{});
        return 0;
      }
    }
    go(std::false_type{});
    return 0;
  });
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  return a.kv_fp8 ? launch_kv<E, D, true>(a, stream) : launch_kv<E, D, false>(a, stream);
}

template <typename E>
hipError_t launch_e(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_d<E, 64>(a, stream);
    case 128: return launch_d<E, 128>(a, stream);
    case 256: return launch_d<E, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_mfma_grid(const DecodeArgs& a) {
  return a.dtype == PA_DTYPE_BF16 ? grid_e<BF16>(a) : grid_e<F16>(a);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (a.dtype == PA_DTYPE_BF16) return launch_e<BF16>(a, stream);
  if (a.dtype == PA_DTYPE_F16) return launch_e<F16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa

// Per-row top-K over transformed unary logits on gfx950.
//
// Operation ("[Spec] DFlash2: local convolution + candidate selector",
// implementation breakdown: deterministic per-slot top-k over the unary logits
// that output_multiplier / final_logit_softcapping transform; "DSpark
// padded-vocab d2t fix": ids in the padded tail are never selected):
//   ids[n, 0..K) = the K ids v < valid_vocab with the largest T(z[n, v]),
//   ordered by (value descending, id ascending); unary = T(z) of those ids.
// T is strictly increasing, so selection compares the raw logits exactly.
//
// Design (HBM-bound stream, one pass over the logits, no cross-workgroup
// synchronisation):
//  * Every value has an order-preserving unsigned key (-0 and +0 share a key;
//    a position outside the logical vocabulary has key 0, below every real
//    value), and every (key, id) pair a 56-bit composite
//    key << 24 | (2^24 - 1 - id) whose order is exactly (value desc, id asc)
//    and which is unique within a row.
//  * A workgroup of 4 waves owns a row (or, when rows are very few, a segment
//    of one; a small second kernel then merges segments).  The row is cut
//    into group-chunks of 16384 values; inside one, the waves interleave at
//    the granularity of one wave load (64 lanes x 16 bytes), so each wave
//    holds 64 values per lane, as eight 16-byte loads, and the four waves
//    split every group-chunk -- the row's partial last one included -- into
//    equal quarters.  Waves stream on their own, the next group-chunk's
//    loads in flight while the current one is processed, and each keeps its
//    own K best in LDS.  No workgroup barrier until the final merge.  The
//    logits are read once, with non-temporal loads.
//  * Threshold: on a wave's first chunk, the K-th largest of its 64 lane
//    maxima (found bit by bit with ballot counts; those K lanes hold K
//    distinct values that reach it); afterwards a value must beat the wave's
//    K-th key strictly (its id is larger than every id the wave holds).
//  * bf16: while that threshold is a positive value, the filter runs on the
//    raw bits (a positive bf16 read as int16 orders like its value), one
//    packed signed max per two values; keys are built only for survivors.
//    Otherwise (and for fp32) keys are built per value.  Either way a lane
//    first compares the maxima of groups of its registers with the
//    threshold, and searches register by register only a group that holds
//    a survivor (after the first chunks, most lanes hold none).
//  * Survivors are compacted into LDS; the wave's sorted list is updated with
//    ranks from a binary search in the held list plus a count among the new.
//  * If a chunk yields more survivors than LDS holds (mass ties), an exact
//    bisection on the key, then on the id among the tied key, narrows the
//    chunk to exactly its K best; that path re-reads the chunk from cache.
//  * The sorted per-wave lists are merged with one barrier: each entry's rank
//    is its own index plus, per other list, a binary-searched count of larger
//    entries.
#include "conv_slot_proj.h"
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPerLane = 64;                   // values per lane per wave-chunk
constexpr int kWaveChunk = 64 * kPerLane;      // 4096 values of one wave
constexpr int kGroupChunk = kWaves * kWaveChunk;  // 16384 values of one workgroup
// Elements between a lane's consecutive 16-byte vectors inside a group-chunk:
// the waves interleave at 1 KiB (one wave load), so each wave load of the
// four waves covers one contiguous 4 KiB (bf16) stretch.
template <int VEC> constexpr int64_t vec_stride() { return (int64_t)kWaves * 64 * VEC; }
constexpr int kWaveCap = 256;                  // LDS slots for one chunk's new candidates
constexpr int kMaxK = DFLASH_MAX_TOP_K;
constexpr int kMergeThreads = 256;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Two packed bf16 -> two packed keys.  Per half: negative -> ~b + 1
// (never carries: ~b <= 0x7fff), non-negative -> b ^ 0x8000.
__device__ __forceinline__ uint32_t bf16_key2(uint32_t w) {
  const uint32_t lo_neg = (w >> 15) & 1u, hi_neg = w >> 31;
  const uint32_t m = (lo_neg * 0xffffu) | (hi_neg * 0xffff0000u);    // sign-filled halves
  return (w ^ (m | 0x80008000u)) + (m & 0x00010001u);
}
// fp32 bits -> key in [1, 0xffffffff] (same construction on 32 bits).
__device__ __forceinline__ uint32_t f32_key(uint32_t b) {
  return (b & 0x80000000u) ? (0u - b) : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_key_value(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : (0u - k);
  return __uint_as_float(b);
}

// Within a wave: make LDS writes of all lanes visible to all lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One lane's 64 values of a group-chunk.  With the lane base
// lb = c_start + (wave * 64 + lane) * VEC, value i (0..63) sits at
// id = lb + (i / VEC) * vec_stride<VEC>() + i % VEC.
template <typename TIO> struct Chunk;

template <> struct Chunk<uint16_t> {
  static constexpr int VEC = 8, L = kPerLane / VEC, W = kPerLane / 2;
  uint32_t w[W];     // raw bits after issue(), packed keys after make_keys()

  // `full` (wave-uniform): the whole wave-chunk lies below the logical vocab
  // end, so every load is unconditional and the key conversion branch-free
  // (keeps the wait for this chunk's loads from draining the prefetch).
  // Partial group-chunk: vectors past the logical vocab end read as zero.
  __device__ __forceinline__ void issue(const uint16_t* rowp, int64_t lb, int64_t valid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = lb + l * vec_stride<VEC>();
      const uint4 r = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  // A group-chunk of a row with valid >= VEC, by unconditional loads (so the
  // wait for them is an exact in-order count): a vector past last_vec, the
  // last whole vector below the logical end, re-reads that one instead; its
  // values are replaced in make_keys.  In a whole group-chunk every vector
  // lies at or below last_vec.
  __device__ __forceinline__ void issue_clamped(const uint16_t* rowp, int32_t lb, int32_t last_vec) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int32_t e0 = min(lb + l * (int32_t)vec_stride<VEC>(), last_vec);
      const u32x4 rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + e0));   // streamed once
      const uint4 r = make_uint4(rv.x, rv.y, rv.z, rv.w);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  __device__ __forceinline__ void keys_full() {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j] = bf16_key2(w[j]);
  }
  // Keys of a partial group-chunk (issue() read the vectors below the end).
  __device__ __forceinline__ void make_keys(const uint16_t* rowp, int64_t lb, int64_t valid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = lb + l * vec_stride<VEC>();
      if (e0 + VEC <= valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[l * 4 + q] = bf16_key2(w[l * 4 + q]);
      } else {   // the one vector that straddles the logical end, or beyond it
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t a = e0 + 2 * q;
          const uint32_t lo = a < valid ? bf16_key(rowp[a]) : 0u;
          const uint32_t hi = a + 1 < valid ? bf16_key(rowp[a + 1]) : 0u;
          w[l * 4 + q] = lo | (hi << 16);
        }
      }
    }
  }
  __device__ uint32_t max_key() const {
    u16x2 m = __builtin_bit_cast(u16x2, w[0]);
#pragma unroll
    for (int j = 1; j < W; ++j) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j]));
    return max((uint32_t)m.x, (uint32_t)m.y);
  }
  // On raw bits: the largest lane value read as int16 (the largest positive
  // value, when the lane has one).
  __device__ int raw_max_i16() const {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    s16x2 m = __builtin_bit_cast(s16x2, w[0]);
#pragma unroll
    for (int j = 1; j < W; ++j) m = __builtin_elementwise_max(m, __builtin_bit_cast(s16x2, w[j]));
    return max((int)m.x, (int)m.y);
  }
  static constexpr bool kHasRawFilter = true;
  // Wave-uniform scans.  The group pre-test is taken for the whole wave (a
  // ballot), and f(pass, key, value index) is called by every lane for every
  // value of a group where some lane holds a survivor, so f may use ballots.
  // scan_ge: keys >= tau (1 <= tau < 0x10000).  scan_raw_ge (before
  // make_keys): positive values whose bits, read as int16, are >= r
  // (1 <= r <= 0x7fff), i.e. key >= r + 0x8000; negative values never pass.
  template <class F> __device__ void scan_ge(uint64_t tau, F&& f) const {
    const uint32_t t1 = (uint32_t)(tau - 1);
    u16x2 gm[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      gm[g] = __builtin_bit_cast(u16x2, w[8 * g]);
#pragma unroll
      for (int j = 1; j < 8; ++j) gm[g] = __builtin_elementwise_max(gm[g], __builtin_bit_cast(u16x2, w[8 * g + j]));
    }
    const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(gm[0], gm[1]),
                                              __builtin_elementwise_max(gm[2], gm[3]));
    if (__ballot(max((uint32_t)m.x, (uint32_t)m.y) > t1) == 0) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (__ballot(max((uint32_t)gm[g].x, (uint32_t)gm[g].y) > t1) == 0) continue;
#pragma unroll
      for (int j = 8 * g; j < 8 * g + 8; ++j) {
        const uint32_t lo = w[j] & 0xffffu, hi = w[j] >> 16;
        f(lo > t1, lo, 2 * j);
        f(hi > t1, hi, 2 * j + 1);
      }
    }
  }
  template <class F> __device__ void scan_raw_ge(uint32_t r, F&& f) const {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const short r1 = (short)(r - 1);
    s16x2 gm[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      gm[g] = __builtin_bit_cast(s16x2, w[8 * g]);
#pragma unroll
      for (int j = 1; j < 8; ++j) gm[g] = __builtin_elementwise_max(gm[g], __builtin_bit_cast(s16x2, w[8 * g + j]));
    }
    const s16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(gm[0], gm[1]),
                                              __builtin_elementwise_max(gm[2], gm[3]));
    if (__ballot(max(m.x, m.y) > r1) == 0) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (__ballot(max(gm[g].x, gm[g].y) > r1) == 0) continue;
#pragma unroll
      for (int j = 8 * g; j < 8 * g + 8; ++j) {
        const s16x2 x = __builtin_bit_cast(s16x2, w[j]);
        f(x.x > r1, (w[j] & 0xffffu) | 0x8000u, 2 * j);
        f(x.y > r1, (w[j] >> 16) | 0x8000u, 2 * j + 1);
      }
    }
  }
  static constexpr uint64_t kKeyLimit = 0x10000u;   // keys are < this
  static constexpr int kKeyBits = 16;
  __device__ static uint32_t key_at(const uint16_t* p) { return bf16_key(*p); }
  __device__ static float value(uint32_t k) { return bf16_key_value(k); }
};

template <> struct Chunk<float> {
  static constexpr int VEC = 4, L = kPerLane / VEC;
  uint32_t w[kPerLane];

  __device__ __forceinline__ void issue(const float* rowp, int64_t lb, int64_t valid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = lb + l * vec_stride<VEC>();
      const uint4 r = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  __device__ __forceinline__ void issue_clamped(const float* rowp, int32_t lb, int32_t last_vec) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int32_t e0 = min(lb + l * (int32_t)vec_stride<VEC>(), last_vec);
      const u32x4 rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + e0));   // streamed once
      const uint4 r = make_uint4(rv.x, rv.y, rv.z, rv.w);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  __device__ __forceinline__ void keys_full() {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) w[j] = f32_key(w[j]);
  }
  __device__ __forceinline__ void make_keys(const float* rowp, int64_t lb, int64_t valid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = lb + l * vec_stride<VEC>();
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[l * 4 + q] = (e0 + VEC <= valid) ? f32_key(w[l * 4 + q])
                       : (e0 + q < valid) ? f32_key(__float_as_uint(rowp[e0 + q])) : 0u;
    }
  }
  __device__ uint32_t max_key() const {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) m = max(m, w[j]);
    return m;
  }
  static constexpr bool kHasRawFilter = false;
  __device__ int raw_max_i16() const { return 0; }
  // Wave-uniform scan as in the bf16 chunk: keys >= tau (eight groups of
  // eight keys).  There is no raw scan for fp32.
  template <class F> __device__ void scan_ge(uint64_t tau, F&& f) const {
    uint32_t gm[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      gm[g] = w[8 * g];
#pragma unroll
      for (int j = 1; j < 8; ++j) gm[g] = max(gm[g], w[8 * g + j]);
    }
    uint32_t m = gm[0];
#pragma unroll
    for (int g = 1; g < 8; ++g) m = max(m, gm[g]);
    if (__ballot((uint64_t)m >= tau) == 0) return;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (__ballot((uint64_t)gm[g] >= tau) == 0) continue;
#pragma unroll
      for (int j = 8 * g; j < 8 * g + 8; ++j) f((uint64_t)w[j] >= tau, w[j], j);
    }
  }
  template <class F> __device__ void scan_raw_ge(uint32_t, F&&) const {}
  static constexpr uint64_t kKeyLimit = 0x100000000ull;
  static constexpr int kKeyBits = 32;
  __device__ static uint32_t key_at(const float* p) { return f32_key(__float_as_uint(*p)); }
  __device__ static float value(uint32_t k) { return f32_key_value(k); }
};

struct WaveLds {
  uint64_t pool[kMaxK + kWaveCap];   // a chunk's survivors; at the end the sorted best
  uint64_t tmp[kMaxK];
  uint32_t count;
  uint32_t nbest;
};

struct Shared {
  WaveLds wave[kWaves];
  // Keys below which every wave may drop values (not ties: another wave's
  // values can have smaller ids), each valid because at least K values of
  // the row reach it:
  //  * bound: the largest K-th held key of any wave;
  //  * qkey[w]: wave w's ceil(K/4)-th held key (0 until it holds that many);
  //    the smallest of the four is reached by 4 ceil(K/4) >= K values, and
  //    sits near the K-th best of the values seen so far (the largest K-th
  //    key only near the 4K-th).
  uint32_t bound;
  uint32_t qkey[kWaves];
};

template <int VEC>
__device__ __forceinline__ int64_t value_id(int64_t lb, int i) {
  return lb + (i / VEC) * vec_stride<VEC>() + (i % VEC);
}

// Counts, over this lane's chunk values re-read from memory, those with
// key >= lo_key (mode 0), key > key_eq (mode 1), or key == key_eq and
// id < id_bound (mode 2); then sums over the wave.
template <typename TIO>
__device__ uint32_t count_pass(const TIO* rowp, int64_t lb, int64_t valid, int mode,
                               uint64_t lo_key, uint32_t key_eq, int64_t id_bound) {
  constexpr int VEC = Chunk<TIO>::VEC;
  uint32_t c = 0;
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t id = value_id<VEC>(lb, i);
    if (id >= valid) continue;
    const uint32_t k = Chunk<TIO>::key_at(rowp + id);
    if (mode == 0) c += ((uint64_t)k >= lo_key) ? 1u : 0u;
    else if (mode == 1) c += (k > key_eq) ? 1u : 0u;
    else c += (k == key_eq && id < id_bound) ? 1u : 0u;
  }
  return wave_sum_u32(c);
}

// Exact narrowing when a wave-chunk yields more than kWaveCap candidates:
// replaces the new candidates (pool[nbest, ...)) by exactly the chunk's K
// best (or all its real values if fewer); returns their number.
template <typename TIO>
__device__ __noinline__ uint32_t narrow_exact(const TIO* rowp, int64_t lb, int64_t c_start, int64_t valid, int lane,
                                              int K, int nbest, WaveLds& wl) {
  constexpr int VEC = Chunk<TIO>::VEC;
  const uint32_t n_real = count_pass(rowp, lb, valid, 0, 1, 0, 0);
  uint32_t kt = 1;                                     // take every real value when there are few
  int64_t id_bound = INT64_MAX;
  if (n_real > (uint32_t)K) {
    uint64_t lo = 1, hi = Chunk<TIO>::kKeyLimit;       // count(>= lo) >= K > count(>= hi)
    while (hi - lo > 1) {
      const uint64_t mid = lo + (hi - lo) / 2;
      if (count_pass(rowp, lb, valid, 0, mid, 0, 0) >= (uint32_t)K) lo = mid; else hi = mid;
    }
    kt = (uint32_t)lo;
    const uint32_t c_gt = count_pass(rowp, lb, valid, 1, 0, kt, 0);
    const uint32_t need = (uint32_t)K - c_gt;          // ties at kt to take, lowest ids first
    int64_t lo_i = c_start, hi_i = c_start + kGroupChunk;  // count(id < lo_i) < need <= count(id < hi_i)
    while (hi_i - lo_i > 1) {
      const int64_t mid = lo_i + (hi_i - lo_i) / 2;
      if (count_pass(rowp, lb, valid, 2, 0, kt, mid) >= need) hi_i = mid; else lo_i = mid;
    }
    id_bound = hi_i;
  }
  wave_sync();
  if (lane == 0) wl.count = 0;
  wave_sync();
  for (int i = 0; i < kPerLane; ++i) {
    const int64_t id = value_id<VEC>(lb, i);
    if (id >= valid) continue;
    const uint32_t k = Chunk<TIO>::key_at(rowp + id);
    if (k > kt || (k == kt && id < id_bound)) {
      const uint32_t pos = atomicAdd(&wl.count, 1u);
      if (pos < (uint32_t)kWaveCap) wl.pool[nbest + pos] = composite(k, id);
    }
  }
  wave_sync();
  return __builtin_amdgcn_readfirstlane(wl.count);
}


// K-th largest of the 64 lane values m (unsigned, below 2^bits): the largest
// t with #{lanes : m >= t} >= K, found bit by bit with ballot counts.  Those
// K lanes each hold a distinct value >= t.  Returns 0 when fewer than K
// lanes have m >= 1.
__device__ __forceinline__ uint32_t kth_largest_lane(uint32_t m, int K, int bits) {
  uint32_t t = 0;
  for (int b = bits - 1; b >= 0; --b) {
    const uint32_t cand = t | (1u << b);
    if (__popcll(__ballot(m >= cand)) >= K) t = cand;
  }
  return t;
}

// One workgroup of the top-K: `block` = row * segs + segment.
template <typename TIO>
__device__ __forceinline__ void topk_rows_body(int block, const TIO* __restrict__ logits, int64_t row_stride,
                                               int64_t valid_vocab, int32_t K, int32_t wchunks, int32_t segs,
                                               int32_t wchunks_per_seg, float mult, float cap,
                                               uint64_t* __restrict__ parts, int64_t* __restrict__ ids_out,
                                               float* __restrict__ unary_out) {
  __shared__ Shared sh;
  const int lane = threadIdx.x & 63;
  // wave index through readfirstlane: provably uniform, so chunk bounds and
  // tests below are scalar and the loads need no exec masking
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WaveLds& wl = sh.wave[wave];
  const int64_t row = block / segs;
  const int seg = (int)(block % segs);
  const int c_begin = seg * wchunks_per_seg;
  const int c_end = min(wchunks, c_begin + wchunks_per_seg);
  const TIO* rowp = logits + row * row_stride;

  // The wave's sorted best composites live in registers: lane i < nbest holds
  // the i-th (hv); nbest and the K-th key are wave-uniform.
  int nbest = 0;
  uint64_t hv = 0;
  uint32_t kth_key = 0;                          // key of the K-th held one once nbest == K
  int n_new = 0;                                 // this chunk's survivors in wl.pool[0, n_new) (wave-uniform)
  if (threadIdx.x == 0) sh.bound = 0;
  if (threadIdx.x < kWaves) sh.qkey[threadIdx.x] = 0;
  __syncthreads();
  // The workgroup's shared bound (a key; 0 = none yet), read without ordering:
  // any value another wave has published is valid.
  auto shared_bound = [&]() -> uint32_t {
    uint32_t q = __hip_atomic_load(&sh.qkey[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      q = min(q, __hip_atomic_load(&sh.qkey[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    const uint32_t b = __hip_atomic_load(&sh.bound, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(max(b, q));
  };
  // (readlane returns a signed int: widen each half through uint32_t)
  auto readlane64 = [](uint64_t v, int j) -> uint64_t {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), j) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, j);
  };

  constexpr int VEC = Chunk<TIO>::VEC;
  // Called by every lane (uniform control flow) for one value index i of the
  // lane's values: the lanes where it passes append its composite to
  // wl.pool[n_new, ...) in lane order (slots from a ballot count, no atomics).
  auto push = [&](bool pass, uint32_t k, int i, uint32_t id_base) {
    const uint64_t m = __ballot(pass);
    if (m == 0) return;
    if (pass) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint32_t pos = (uint32_t)n_new + below;
      // ids < 2^24: the 32-bit lane base plus the value's compile-time offset
      const uint32_t id = id_base + (uint32_t)((i / VEC) * vec_stride<VEC>() + i % VEC);
      if (pos < (uint32_t)kWaveCap) wl.pool[pos] = ((uint64_t)k << 24) | (uint64_t)(kIdMask - id);
    }
    n_new += (int)__popcll(m);
  };
  // After the survivors of one chunk are in the pool: exact narrowing if they
  // overflowed, then merge them into the held list, 64 at a time (one per
  // lane).  Ranks: a held entry's is its index plus the new ones above it; a
  // new one's is the held ones above it plus the new ones above it.  Per new
  // candidate j (read with readlane): the held lanes it beats come from one
  // compare, whose ballot also gives, by complement over the held lanes, the
  // count of held entries above it (composites are unique) -- no pass over
  // the held list.  Ranks are distinct.  The K best are reordered through
  // LDS.  A chunk without survivors costs nothing here.
  auto update = [&](int64_t lb, int64_t c_start) {
    if (n_new == 0) return;
    if (n_new > kWaveCap) n_new = (int)narrow_exact<TIO>(rowp, lb, c_start, valid_vocab, lane, K, 0, wl);
    wave_sync();
    for (int b0 = 0; b0 < n_new; b0 += 64) {
      const int m = min(64, n_new - b0);
      const uint64_t held = (1ull << nbest) - 1ull;   // lanes holding an entry (nbest <= K <= 32)
      const uint64_t cv = lane < m ? wl.pool[b0 + lane] : 0ull;
      int rank_h = lane, rank_c = 0, above_c = 0;
      for (int j = 0; j < m; ++j) {
        const uint64_t cj = readlane64(cv, j);
        const bool beats = cj > hv;
        rank_h += beats ? 1 : 0;
        rank_c += cj > cv ? 1 : 0;
        const int above = (int)__popcll(held & ~__ballot(beats));
        if (lane == j) above_c = above;
      }
      rank_c += above_c;
      if (lane < nbest && rank_h < K) wl.tmp[rank_h] = hv;
      if (lane < m && rank_c < K) wl.tmp[rank_c] = cv;
      wave_sync();
      nbest = min(K, nbest + m);
      hv = lane < nbest ? wl.tmp[lane] : 0ull;
      wave_sync();
    }
    n_new = 0;
    const int q = (K + 3) / 4;
    if (nbest >= q) {
      const uint32_t qk = composite_key(readlane64(hv, q - 1));
      if (lane == 0) __hip_atomic_store(&sh.qkey[wave], qk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (nbest == K) {
      kth_key = composite_key(readlane64(hv, K - 1));
      if (lane == 0) atomicMax(&sh.bound, kth_key);
    }
  };
  // General path: `ch` holds keys.  Threshold, compaction, update.
  auto process_keys = [&](const Chunk<TIO>& ch, int64_t lb, int64_t c_start) {
    const uint32_t sb = shared_bound();
    uint64_t tau;
    if (nbest < K) {
      // K-th largest lane maximum: at least K values reach it (key 0 =
      // no real value; too few real lanes -> every real value)
      const uint32_t t = kth_largest_lane(ch.max_key(), K, Chunk<TIO>::kKeyBits);
      tau = t ? (uint64_t)t : 1u;
    } else {
      // a later value has a larger id than every held one: it must beat the
      // K-th key strictly
      tau = (uint64_t)kth_key + 1;
    }
    if ((uint64_t)sb > tau) tau = sb;
    if (tau < Chunk<TIO>::kKeyLimit)
      ch.scan_ge(tau, [&](bool pass, uint32_t k, int i) { push(pass, k, i, (uint32_t)lb); });
    update(lb, c_start);
  };
  // One full chunk whose raw bits are in `ch`.  bf16: while the threshold is
  // a positive value the filter runs on raw bits (keys are built only for
  // survivors); otherwise the chunk goes through the key path.
  auto process_full = [&](Chunk<TIO>& ch, int64_t lb, int64_t c_start) {
    if (Chunk<TIO>::kHasRawFilter) {
      // key bound (values below it are dropped): the workgroup's, or the
      // wave's own K-th key + 1 (strict, as above) when that is higher
      uint32_t tau = shared_bound();
      if (nbest == K && kth_key + 1 > tau) tau = kth_key + 1;
      int r = 0;                                                 // raw int16 threshold, >= 1 when usable
      if (tau > 0x8000u && tau < 0x10000u) {
        r = (int)(tau - 0x8000u);
      } else if (nbest == 0 && tau <= 0x8000u) {
        // first chunk: K-th largest positive raw lane maximum (a positive
        // int16 orders like its value); 0 when fewer than K lanes hold a
        // positive value
        r = (int)kth_largest_lane((uint32_t)max(ch.raw_max_i16(), 0), K, 15);
      }
      if (r >= 1) {
        ch.scan_raw_ge((uint32_t)r, [&](bool pass, uint32_t k, int i) { push(pass, k, i, (uint32_t)lb); });
        update(lb, c_start);
        return;
      }
    }
    ch.keys_full();
    process_keys(ch, lb, c_start);
  };

  // Every wave walks the same group-chunks, each taking its interleaved
  // quarter.  Group-chunks below n_full lie entirely inside the logical
  // vocabulary; at most the row's last one is partial.  The loop over whole
  // group-chunks always issues the next one's loads before processing the
  // current one -- the partial one after the last whole one, else a re-read
  // of the current one (a cache hit) -- and every issue is unconditional, so
  // the wait for the current one is an exact in-order count and the next
  // one's loads stay in flight meanwhile.  A row too short to hold one whole
  // vector reads its partial group-chunk with bounds-checked loads instead.
  const int64_t wave_off = (int64_t)(wave * 64 + lane) * VEC;
  const int32_t wave_off32 = (int32_t)wave_off;                       // vocab < 2^24
  const int n_full = (int)(valid_vocab / kGroupChunk);
  const int full_end = min(c_end, n_full);
  const bool clampable = valid_vocab >= VEC;
  const int32_t last_vec = clampable ? (int32_t)((valid_vocab / VEC - 1) * VEC) : 0;  // last whole vector
  const int pre_end = (c_end > n_full && clampable) ? full_end + 1 : full_end;       // chunks worth prefetching
  int c = c_begin;
  Chunk<TIO> tail;
  bool tail_loaded = false;
  if (c < full_end) {
    // two register buffers, roles alternating so that no chunk is copied:
    // while one chunk is processed the next one is in flight (three buffers
    // were measured slower).  Chunk indices past the prefetch end re-read its
    // last one (a cache hit).
    auto idx = [&](int k) { return k < pre_end ? k : pre_end - 1; };
    int tail_in = 0;                              // the buffer holding the prefetched partial chunk
    {
      Chunk<TIO> a, b;
      a.issue_clamped(rowp, c * kGroupChunk + wave_off32, last_vec);
      while (true) {
        b.issue_clamped(rowp, idx(c + 1) * kGroupChunk + wave_off32, last_vec);
        process_full(a, (int64_t)c * kGroupChunk + wave_off, (int64_t)c * kGroupChunk);
        if (++c >= full_end) { tail_in = 1; break; }
        a.issue_clamped(rowp, idx(c + 1) * kGroupChunk + wave_off32, last_vec);
        process_full(b, (int64_t)c * kGroupChunk + wave_off, (int64_t)c * kGroupChunk);
        if (++c >= full_end) { tail_in = 0; break; }
      }
      if (pre_end > full_end) {
#pragma unroll
        for (int j = 0; j < (int)(sizeof(tail.w) / sizeof(tail.w[0])); ++j) tail.w[j] = tail_in == 1 ? b.w[j] : a.w[j];
        tail_loaded = true;
      }
    }
  }
  if (c < c_end) {                               // the partial last group-chunk of the row
    const int64_t c_start = (int64_t)c * kGroupChunk;
    if (!tail_loaded) {
      if (clampable) tail.issue_clamped(rowp, (int32_t)c_start + wave_off32, last_vec);
      else tail.issue(rowp, c_start + wave_off, valid_vocab);
    }
    tail.make_keys(rowp, c_start + wave_off, valid_vocab);
    process_keys(tail, c_start + wave_off, c_start);
  }
  if (lane < nbest) wl.pool[lane] = hv;         // the sorted list, for the merge below
  if (lane == 0) wl.nbest = (uint32_t)nbest;
  __syncthreads();

  // ---- merge the sorted wave lists ----------------------------------------
  if (threadIdx.x < kWaves * K) {
    const int w = threadIdx.x / K, i = threadIdx.x % K;
    const int nw = (int)sh.wave[w].nbest;
    if (i < nw) {
      const uint64_t cval = sh.wave[w].pool[i];
      int rank = i;
      for (int o = 0; o < kWaves; ++o)
        if (o != w) rank += count_greater(sh.wave[o].pool, (int)sh.wave[o].nbest, cval);
      if (rank < K) {
        if (segs == 1) {
          ids_out[row * K + rank] = composite_id(cval);
          unary_out[row * K + rank] = unary_transform(Chunk<TIO>::value(composite_key(cval)), mult, cap);
        } else {
          parts[((size_t)row * segs + seg) * K + rank] = cval;
        }
      }
    }
  }
  if (segs > 1) {
    // a segment with fewer than K real values leaves empty slots
    int total = 0;
    for (int w = 0; w < kWaves; ++w) total += (int)sh.wave[w].nbest;
    for (int i = total + (int)threadIdx.x; i < K; i += kThreads) parts[((size_t)row * segs + seg) * K + i] = 0ull;
  }
}

// bf16: at most 128 VGPRs so that 4 waves share each SIMD.
__global__ __launch_bounds__(kThreads, 4) void topk_rows_bf16(const uint16_t* __restrict__ logits, int64_t row_stride,
                                                            int64_t valid_vocab, int32_t K, int32_t wchunks,
                                                            int32_t segs, int32_t wchunks_per_seg, float mult,
                                                            float cap, uint64_t* __restrict__ parts,
                                                            int64_t* __restrict__ ids_out,
                                                            float* __restrict__ unary_out) {
  topk_rows_body<uint16_t>((int)blockIdx.x, logits, row_stride, valid_vocab, K, wchunks, segs, wchunks_per_seg, mult, cap, parts,
                           ids_out, unary_out);
}
__global__ __launch_bounds__(kThreads) void topk_rows_f32(const float* __restrict__ logits, int64_t row_stride,
                                                          int64_t valid_vocab, int32_t K, int32_t wchunks,
                                                          int32_t segs, int32_t wchunks_per_seg, float mult,
                                                          float cap, uint64_t* __restrict__ parts,
                                                          int64_t* __restrict__ ids_out,
                                                          float* __restrict__ unary_out) {
  topk_rows_body<float>((int)blockIdx.x, logits, row_stride, valid_vocab, K, wchunks, segs, wchunks_per_seg, mult, cap, parts,
                        ids_out, unary_out);
}

// The propose step's first stage in one launch (bf16): workgroups that
// compute the top-K rows and groups_x * ksplit that compute the conv and the
// slot projection (conv_slot_proj.h).  Neither part reads what the other
// writes, so they run side by side without a second stream.
template <int TAPS, int RT, int U>
__global__ __launch_bounds__(kThreads, 2) void topk_conv_proj_bf16(
    const uint16_t* __restrict__ logits, int64_t row_stride, int64_t valid_vocab, int32_t K, int32_t wchunks,
    int32_t segs, int32_t wchunks_per_seg, float mult, float cap, uint64_t* __restrict__ parts,
    int64_t* __restrict__ ids_out, float* __restrict__ unary_out, SlotProjArgs sp) {
  const int b = (int)blockIdx.x;
  // Dispatch order: with two k-steps in flight the conv + projection chains
  // end well inside the top-K's time and the top-K rows go first; with one,
  // those chains are the longer ones and go first (measured both ways: 32
  // requests 43.8 vs 47.2 us per step, 64 requests of 10 tokens 56.1 vs 54.4).
  const int n_spw = sp.groups_x * sp.ksplit;
  const int n_tk = (int)gridDim.x - n_spw;
  const int sp_first = U == 1;
  if (sp_first ? b < n_spw : b >= n_tk) {
    const int g = sp_first ? b : b - n_tk;
    conv_slot_proj_group<TAPS, RT, U>(g % sp.groups_x, g / sp.groups_x, sp);
    return;
  }
  topk_rows_body<uint16_t>(sp_first ? b - n_spw : b, logits, row_stride, valid_vocab, K, wchunks, segs,
                           wchunks_per_seg, mult, cap, parts, ids_out, unary_out);
}

// Merge of the per-segment K best (rows split over several workgroups).
template <typename TIO>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const uint64_t* __restrict__ parts, int32_t K,
                                                                   int32_t segs, float mult, float cap,
                                                                   int64_t* __restrict__ ids_out,
                                                                   float* __restrict__ unary_out) {
  __shared__ uint64_t cand[kTopkMergeCap];
  const int64_t row = blockIdx.x;
  const int m = segs * K;
  const uint64_t* src = parts + (size_t)row * m;
  for (int i = threadIdx.x; i < m; i += kMergeThreads) cand[i] = src[i];
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += kMergeThreads) {
    const uint64_t c = cand[i];
    if (c == 0) continue;                      // empty slot of a short segment
    int rank = 0;
    for (int j = 0; j < m; ++j) rank += (cand[j] > c) ? 1 : 0;
    if (rank < K) {
      ids_out[row * K + rank] = composite_id(c);
      unary_out[row * K + rank] = unary_transform(Chunk<TIO>::value(composite_key(c)), mult, cap);
    }
  }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

TopkPlan plan_topk(int64_t n_rows, int64_t valid_vocab, int32_t top_k) {
  TopkPlan p{};
  p.n_rows = n_rows;
  p.valid_vocab = valid_vocab;
  p.top_k = top_k;
  p.chunks = (int32_t)((valid_vocab + kGroupChunk - 1) / kGroupChunk);   // group-chunks per row
  if (p.chunks < 1) p.chunks = 1;
  // One workgroup (4 waves) per row; only when rows are very few are they
  // split into segments (merged by a second kernel), since the merge launch
  // costs more than the extra parallelism gains for a few hundred rows.
  int segs = 1;
  if (n_rows > 0 && n_rows < 128) {
    segs = (int)((512 + n_rows - 1) / n_rows);
    if (segs > p.chunks) segs = p.chunks;                               // >= 1 group-chunk per segment
    if (segs * top_k > kTopkMergeCap) segs = kTopkMergeCap / top_k;
    if (segs < 1) segs = 1;
  }
  p.chunks_per_seg = (p.chunks + segs - 1) / segs;
  p.segs = (p.chunks + p.chunks_per_seg - 1) / p.chunks_per_seg;   // no empty segments
  p.parts_offset = 0;
  p.bytes = (p.segs > 1 && n_rows > 0) ? align256((size_t)n_rows * p.segs * top_k * sizeof(uint64_t)) : 0;
  return p;
}

hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t stream) {
  if (p.n_rows == 0) return hipSuccess;
  uint64_t* parts = reinterpret_cast<uint64_t*>(static_cast<char*>(a.workspace) + p.parts_offset);
  const dim3 grid((unsigned)(p.n_rows * p.segs));
  if (a.dtype == DFLASH_BF16)
    hipLaunchKernelGGL(topk_rows_bf16, grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a.logits), a.row_stride, a.valid_vocab, a.top_k, p.chunks,
                       p.segs, p.chunks_per_seg, a.multiplier, a.softcap, parts, a.ids_out, a.unary_out);
  else
    hipLaunchKernelGGL(topk_rows_f32, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(a.logits), a.row_stride, a.valid_vocab, a.top_k, p.chunks,
                       p.segs, p.chunks_per_seg, a.multiplier, a.softcap, parts, a.ids_out, a.unary_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.segs == 1) return e;
  if (a.dtype == DFLASH_BF16)
    hipLaunchKernelGGL(topk_merge_kernel<uint16_t>, dim3((unsigned)p.n_rows), dim3(kMergeThreads), 0, stream,
                       parts, a.top_k, p.segs, a.multiplier, a.softcap, a.ids_out, a.unary_out);
  else
    hipLaunchKernelGGL(topk_merge_kernel<float>, dim3((unsigned)p.n_rows), dim3(kMergeThreads), 0, stream,
                       parts, a.top_k, p.segs, a.multiplier, a.softcap, a.ids_out, a.unary_out);
  return hipGetLastError();
}

bool conv_slot_proj_fits(const ConvArgs& c, const SelectArgs& s, const ProjPlan& p) {
  return c.dtype == DFLASH_BF16 && s.dtype == DFLASH_BF16 && c.block_size >= 2 && c.block_size <= kSpBlock &&
         s.slots == c.block_size - 1 &&
         c.taps >= 1 && c.taps <= 8 && c.group_size % 8 == 0 && c.hidden % 8 == 0 && p.frags == 1 &&
         s.rank >= 1 && s.rank <= 128 && c.n_tokens % c.block_size == 0 && c.n_tokens / c.block_size == s.n_req;
}

hipError_t launch_topk_conv_proj(const TopkArgs& a, const TopkPlan& p, const ConvArgs& c, const SelectArgs& s,
                                 const ProjPlan& pp, hipStream_t stream) {
  SlotProjArgs sp{static_cast<const uint16_t*>(c.x), static_cast<const uint16_t*>(c.base),
                  static_cast<const uint16_t*>(c.delta), c.delta_row_stride, static_cast<uint16_t*>(c.out),
                  (int32_t)(c.n_tokens / c.block_size), c.block_size, c.hidden, c.group_size,
                  static_cast<const uint16_t*>(s.proj),
                  s.rank, s.slots, pp.kslice, pp.ksplit, s.u_parts, 0};
  sp.groups_x = (sp.n_blocks + 3) / 4;
  const int64_t n_sp = sp.n_blocks > 0 ? (int64_t)sp.groups_x * sp.ksplit : 0;
  if (n_sp == 0) sp.groups_x = 0;
  const int64_t n_tk = p.n_rows * p.segs;
  if (n_sp + n_tk == 0) return hipSuccess;
  uint64_t* parts = reinterpret_cast<uint64_t*>(static_cast<char*>(a.workspace) + p.parts_offset);
  const dim3 grid((unsigned)(n_sp + n_tk));
  const int tiles = s.rank > 64 ? 8 : 4;
#define DFLASH_TCP(TAPS, RT)                                                                                      \
  do {                                                                                                            \
    if (sp_two_in_flight_fits<TAPS, RT>() && n_sp + n_tk <= kSpThreeWaveSlots)                                   \
      hipLaunchKernelGGL((topk_conv_proj_bf16<TAPS, RT, sp_two_in_flight_fits<TAPS, RT>() ? 2 : 1>), grid,       \
                         dim3(kThreads), 0, stream, static_cast<const uint16_t*>(a.logits), a.row_stride,        \
                         a.valid_vocab, a.top_k, p.chunks, p.segs, p.chunks_per_seg, a.multiplier, a.softcap,    \
                         parts, a.ids_out, a.unary_out, sp);                                                     \
    else                                                                                                          \
      hipLaunchKernelGGL((topk_conv_proj_bf16<TAPS, RT, 1>), grid, dim3(kThreads), 0, stream,                    \
                         static_cast<const uint16_t*>(a.logits), a.row_stride, a.valid_vocab, a.top_k, p.chunks, \
                         p.segs, p.chunks_per_seg, a.multiplier, a.softcap, parts, a.ids_out, a.unary_out, sp);  \
  } while (0)
#define DFLASH_TCP_T(TAPS)                 \
  if (tiles == 4) DFLASH_TCP(TAPS, 4);     \
  else DFLASH_TCP(TAPS, 8);
  switch (c.taps) {
    case 1: DFLASH_TCP_T(1) break;
    case 2: DFLASH_TCP_T(2) break;
    case 3: DFLASH_TCP_T(3) break;
    case 4: DFLASH_TCP_T(4) break;
    case 5: DFLASH_TCP_T(5) break;
    case 6: DFLASH_TCP_T(6) break;
    case 7: DFLASH_TCP_T(7) break;
    case 8: DFLASH_TCP_T(8) break;
    default: return hipErrorInvalidValue;
  }
#undef DFLASH_TCP_T
#undef DFLASH_TCP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.segs == 1 || p.n_rows == 0) return e;
  hipLaunchKernelGGL(topk_merge_kernel<uint16_t>, dim3((unsigned)p.n_rows), dim3(kMergeThreads), 0, stream, parts,
                     a.top_k, p.segs, a.multiplier, a.softcap, a.ids_out, a.unary_out);
  return hipGetLastError();
}

}  // namespace dflash

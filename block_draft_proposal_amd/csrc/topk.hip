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
  __device__ void issue(const uint16_t* rowp, int64_t lb, int64_t valid) {
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
  __device__ void issue_clamped(const uint16_t* rowp, int32_t lb, int32_t last_vec) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int32_t e0 = min(lb + l * (int32_t)vec_stride<VEC>(), last_vec);
      const u32x4 rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + e0));   // streamed once
      const uint4 r = make_uint4(rv.x, rv.y, rv.z, rv.w);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  __device__ void keys_full() {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j] = bf16_key2(w[j]);
  }
  // Keys of a partial group-chunk (issue() read the vectors below the end).
  __device__ void make_keys(const uint16_t* rowp, int64_t lb, int64_t valid) {
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
  // Calls f(key, value index) for every key >= tau (1 <= tau < 0x10000).
  // Survivors are rare: the lane first tests the maxima of four groups of
  // eight registers, and only a group holding one is searched register by
  // register.
  template <class F> __device__ void for_each_ge(uint64_t tau, F&& f) const {
    const unsigned short t1 = (unsigned short)(tau - 1);
    const u16x2 t = {t1, t1};
    u16x2 gm[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      gm[g] = __builtin_bit_cast(u16x2, w[8 * g]);
#pragma unroll
      for (int j = 1; j < 8; ++j) gm[g] = __builtin_elementwise_max(gm[g], __builtin_bit_cast(u16x2, w[8 * g + j]));
    }
    const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(gm[0], gm[1]),
                                              __builtin_elementwise_max(gm[2], gm[3]));
    if (max(m.x, m.y) <= t1) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (max(gm[g].x, gm[g].y) <= t1) continue;
#pragma unroll
      for (int j = 8 * g; j < 8 * g + 8; ++j) {
        const u16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, w[j]), t);
        if (__builtin_bit_cast(uint32_t, d) != 0u) {
          if (d.x) f(w[j] & 0xffffu, 2 * j);
          if (d.y) f(w[j] >> 16, 2 * j + 1);
        }
      }
    }
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
  // On raw bits (before make_keys): calls f(key, value index) for every
  // positive value whose bits, read as int16, are >= r (1 <= r <= 0x7fff).
  // A positive value's key is bits | 0x8000, so this selects key >= r + 0x8000;
  // negative values (int16 < 0) never pass.  One packed signed max tests two
  // values.
  static constexpr bool kHasRawFilter = true;
  // Same group pre-test as for_each_ge.
  template <class F> __device__ void for_each_raw_ge(uint32_t r, F&& f) const {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const short r1 = (short)(r - 1);
    const s16x2 t = {r1, r1};
    const uint32_t t32 = __builtin_bit_cast(uint32_t, t);
    s16x2 gm[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      gm[g] = __builtin_bit_cast(s16x2, w[8 * g]);
#pragma unroll
      for (int j = 1; j < 8; ++j) gm[g] = __builtin_elementwise_max(gm[g], __builtin_bit_cast(s16x2, w[8 * g + j]));
    }
    const s16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(gm[0], gm[1]),
                                              __builtin_elementwise_max(gm[2], gm[3]));
    if (max(m.x, m.y) <= r1) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (max(gm[g].x, gm[g].y) <= r1) continue;
#pragma unroll
      for (int j = 8 * g; j < 8 * g + 8; ++j) {
        const s16x2 x = __builtin_bit_cast(s16x2, w[j]);
        const s16x2 mx = __builtin_elementwise_max(x, t);
        if (__builtin_bit_cast(uint32_t, mx) != t32) {
          if (x.x > r1) f((w[j] & 0xffffu) | 0x8000u, 2 * j);
          if (x.y > r1) f((w[j] >> 16) | 0x8000u, 2 * j + 1);
        }
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

  __device__ void issue(const float* rowp, int64_t lb, int64_t valid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = lb + l * vec_stride<VEC>();
      const uint4 r = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  __device__ void issue_clamped(const float* rowp, int32_t lb, int32_t last_vec) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int32_t e0 = min(lb + l * (int32_t)vec_stride<VEC>(), last_vec);
      const u32x4 rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + e0));   // streamed once
      const uint4 r = make_uint4(rv.x, rv.y, rv.z, rv.w);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
  }
  __device__ void keys_full() {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) w[j] = f32_key(w[j]);
  }
  __device__ void make_keys(const float* rowp, int64_t lb, int64_t valid) {
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
  // Group pre-test as in the bf16 chunk: eight groups of eight keys.
  template <class F> __device__ void for_each_ge(uint64_t tau, F&& f) const {
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
    if ((uint64_t)m < tau) return;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if ((uint64_t)gm[g] < tau) continue;
#pragma unroll
      for (int j = 8 * g; j < 8 * g + 8; ++j)
        if ((uint64_t)w[j] >= tau) f(w[j], j);
    }
  }
  static constexpr bool kHasRawFilter = false;
  __device__ int raw_max_i16() const { return 0; }
  template <class F> __device__ void for_each_raw_ge(uint32_t, F&&) const {}
  static constexpr uint64_t kKeyLimit = 0x100000000ull;
  static constexpr int kKeyBits = 32;
  __device__ static uint32_t key_at(const float* p) { return f32_key(__float_as_uint(*p)); }
  __device__ static float value(uint32_t k) { return f32_key_value(k); }
};

struct WaveLds {
  uint64_t pool[kMaxK + kWaveCap];   // [0, nbest): held best (sorted); then new candidates
  uint64_t tmp[kMaxK];
  uint32_t count;
  uint32_t nbest;
};

struct Shared {
  WaveLds wave[kWaves];
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


// Merge n new candidates pool[nb, nb + n) into the held sorted list
// pool[0, nb) and keep the best min(nb + n, K), sorted, in pool[0, ...).
// A held entry's new rank is its index plus the new candidates above it; a
// new candidate's rank is a binary search in the held list plus the new
// candidates above it (composites are unique, so ranks are distinct).
__device__ void keep_best(WaveLds& wl, int nb, int n, int K, int lane) {
  const uint64_t* held = wl.pool;
  const uint64_t* fresh = wl.pool + nb;
  for (int i = lane; i < nb; i += 64) {
    const uint64_t c = held[i];
    int rank = i;
    for (int j = 0; j < n; ++j) rank += (fresh[j] > c) ? 1 : 0;
    if (rank < K) wl.tmp[rank] = c;
  }
  for (int i = lane; i < n; i += 64) {
    const uint64_t c = fresh[i];
    int rank = count_greater(held, nb, c);
    for (int j = 0; j < n; ++j) rank += (fresh[j] > c) ? 1 : 0;
    if (rank < K) wl.tmp[rank] = c;
  }
  wave_sync();
  const int m = nb + n < K ? nb + n : K;
  for (int i = lane; i < m; i += 64) wl.pool[i] = wl.tmp[i];
  wave_sync();
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

template <typename TIO>
__device__ __forceinline__ void topk_rows_body(const TIO* __restrict__ logits, int64_t row_stride,
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
  const int64_t row = blockIdx.x / segs;
  const int seg = (int)(blockIdx.x % segs);
  const int c_begin = seg * wchunks_per_seg;
  const int c_end = min(wchunks, c_begin + wchunks_per_seg);
  const TIO* rowp = logits + row * row_stride;

  int nbest = 0;                                 // held best composites (wave-uniform)

  constexpr int VEC = Chunk<TIO>::VEC;
  // Appends a survivor (key, value index i of the lane's values) behind the held best.
  auto push = [&](uint32_t k, int i, uint32_t id_base) {
    const uint32_t pos = atomicAdd(&wl.count, 1u);
    // ids < 2^24: the 32-bit lane base plus the value's compile-time offset
    const uint32_t id = id_base + (uint32_t)((i / VEC) * vec_stride<VEC>() + i % VEC);
    if (pos < (uint32_t)kWaveCap) wl.pool[nbest + pos] = ((uint64_t)k << 24) | (uint64_t)(kIdMask - id);
  };
  // After the survivors of one chunk are in the pool: exact narrowing if they
  // overflowed, then keep the wave's K best.
  auto update = [&](int64_t lb, int64_t c_start) {
    wave_sync();
    uint32_t n = __builtin_amdgcn_readfirstlane(wl.count);
    if (n > (uint32_t)kWaveCap) n = narrow_exact<TIO>(rowp, lb, c_start, valid_vocab, lane, K, nbest, wl);
    if (n > 0) {
      keep_best(wl, nbest, (int)n, K, lane);
      nbest = min(K, nbest + (int)n);
    }
  };
  // General path: `ch` holds keys.  Threshold, compaction, update.
  auto process_keys = [&](const Chunk<TIO>& ch, int64_t lb, int64_t c_start) {
    uint64_t tau;
    if (nbest < K) {
      // K-th largest lane maximum: at least K values reach it (key 0 =
      // no real value; too few real lanes -> every real value)
      const uint32_t t = kth_largest_lane(ch.max_key(), K, Chunk<TIO>::kKeyBits);
      tau = t ? (uint64_t)t : 1u;
    } else {
      // a later value has a larger id than every held one: it must beat the
      // K-th key strictly
      tau = (uint64_t)composite_key(wl.pool[K - 1]) + 1;
    }
    if (lane == 0) wl.count = 0;
    wave_sync();
    if (tau < Chunk<TIO>::kKeyLimit) ch.for_each_ge(tau, [&](uint32_t k, int i) { push(k, i, (uint32_t)lb); });
    update(lb, c_start);
  };
  // One full chunk whose raw bits are in `ch`.  bf16: while the threshold is
  // a positive value the filter runs on raw bits (keys are built only for
  // survivors); otherwise the chunk goes through the key path.
  auto process_full = [&](Chunk<TIO>& ch, int64_t lb, int64_t c_start) {
    if (Chunk<TIO>::kHasRawFilter) {
      int r = 0;                                                 // raw int16 threshold, >= 1 when usable
      if (nbest == K) {
        const uint32_t tau = composite_key(wl.pool[K - 1]) + 1;   // strict, as above
        if (tau > 0x8000u && tau < 0x10000u) r = (int)(tau - 0x8000u);
      } else if (nbest == 0) {
        // first chunk: K-th largest positive raw lane maximum (a positive
        // int16 orders like its value); 0 when fewer than K lanes hold a
        // positive value
        r = (int)kth_largest_lane((uint32_t)max(ch.raw_max_i16(), 0), K, 15);
      }
      if (r >= 1) {
        if (lane == 0) wl.count = 0;
        wave_sync();
        ch.for_each_raw_ge((uint32_t)r, [&](uint32_t k, int i) { push(k, i, (uint32_t)lb); });
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
    // two buffers, alternating roles, so that no chunk is copied
    Chunk<TIO> a, b;
    bool in_b = false;                            // where the chunk prefetched past the loop sits
    a.issue_clamped(rowp, c * kGroupChunk + wave_off32, last_vec);
    while (true) {
      int cn = c + 1 < pre_end ? c + 1 : c;
      b.issue_clamped(rowp, cn * kGroupChunk + wave_off32, last_vec);
      process_full(a, (int64_t)c * kGroupChunk + wave_off, (int64_t)c * kGroupChunk);
      if (++c >= full_end) { in_b = true; break; }
      cn = c + 1 < pre_end ? c + 1 : c;
      a.issue_clamped(rowp, cn * kGroupChunk + wave_off32, last_vec);
      process_full(b, (int64_t)c * kGroupChunk + wave_off, (int64_t)c * kGroupChunk);
      if (++c >= full_end) break;
    }
    if (pre_end > full_end) {
#pragma unroll
      for (int j = 0; j < (int)(sizeof(tail.w) / sizeof(tail.w[0])); ++j) tail.w[j] = in_b ? b.w[j] : a.w[j];
      tail_loaded = true;
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
  topk_rows_body<uint16_t>(logits, row_stride, valid_vocab, K, wchunks, segs, wchunks_per_seg, mult, cap, parts,
                           ids_out, unary_out);
}
__global__ __launch_bounds__(kThreads) void topk_rows_f32(const float* __restrict__ logits, int64_t row_stride,
                                                          int64_t valid_vocab, int32_t K, int32_t wchunks,
                                                          int32_t segs, int32_t wchunks_per_seg, float mult,
                                                          float cap, uint64_t* __restrict__ parts,
                                                          int64_t* __restrict__ ids_out,
                                                          float* __restrict__ unary_out) {
  topk_rows_body<float>(logits, row_stride, valid_vocab, K, wchunks, segs, wchunks_per_seg, mult, cap, parts,
                        ids_out, unary_out);
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

}  // namespace dflash

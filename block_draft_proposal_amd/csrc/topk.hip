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
//  * Every value becomes an order-preserving unsigned key (-0 and +0 share a
//    key; a position outside the logical vocabulary has key 0, below every
//    real value), and every (key, id) pair a 56-bit composite
//    key << 24 | (2^24 - 1 - id) whose order is exactly (value desc, id asc)
//    and which is unique within a row.
//  * One 256-thread workgroup owns a row (or, when rows are too few to fill
//    the chip, a segment of a row; a small second kernel then merges the
//    segments).  It streams the row in chunks of 16384 values, 64 per thread
//    as eight 16-byte loads, so each wave load is one contiguous 1 KiB; the
//    next chunk's loads are issued before the current chunk is processed.
//    bf16 keys are built and kept two per register with packed 16-bit ops.
//  * The running K best composites live in LDS.  For the first chunk the
//    threshold is the minimum over P >= K thread groups of the group maxima
//    (at least K distinct values reach it); once K are held, a later value
//    must beat the K-th key strictly (its id is larger than every held id).
//    A packed saturating subtract tests two keys per instruction; the few
//    survivors are compacted into LDS and ranked exactly by counting.
//  * If a chunk yields more survivors than LDS holds (mass ties), an exact
//    bisection on the key, then on the id among the tied key, narrows the
//    chunk to exactly its K best; that path re-reads the chunk from cache.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 64;
constexpr int kChunk = kThreads * kPerThread;   // values per chunk
constexpr int kCap = kTopkMergeCap;             // LDS slots for new candidates
constexpr int kMaxK = DFLASH_MAX_TOP_K;
constexpr uint32_t kIdMask = 0xffffffu;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t composite(uint32_t key, int64_t id) {
  return ((uint64_t)key << 24) | (uint64_t)(kIdMask - (uint32_t)id);
}
__device__ __forceinline__ uint32_t composite_key(uint64_t c) { return (uint32_t)(c >> 24); }
__device__ __forceinline__ int64_t composite_id(uint64_t c) {
  return (int64_t)(kIdMask - (uint32_t)(c & kIdMask));
}

// bf16 bits -> key in [1, 0xffff]: negatives map to 0x10000 - bits (so -0
// joins +0 at 0x8000), non-negatives to bits | 0x8000.
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  return (b & 0x8000u) ? ((0x10000u - b) & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ float bf16_key_value(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : ((0x10000u - k) & 0xffffu);
  return __uint_as_float(b << 16);
}
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

// One thread's 64 values of a chunk.  Value i (0..63) sits at
// id = c_start + ((i / VEC) * 256 + tid) * VEC + i % VEC.
template <typename TIO> struct Chunk;

template <> struct Chunk<uint16_t> {
  static constexpr int VEC = 8, L = kPerThread / VEC, W = kPerThread / 2;
  uint4 raw[L];      // loaded bits
  uint32_t w[W];     // packed keys: word j = values 2j (low half), 2j+1 (high half)

  __device__ void issue(const uint16_t* rowp, int64_t c_start, int64_t valid, int tid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      raw[l] = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ void make_keys(const uint16_t* rowp, int64_t c_start, int64_t valid, int tid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      const uint32_t r4[4] = {raw[l].x, raw[l].y, raw[l].z, raw[l].w};
      if (e0 + VEC <= valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[l * 4 + q] = bf16_key2(r4[q]);
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
  // Calls f(key, value index) for every key >= tau (1 <= tau <= 0x10000).
  template <class F> __device__ void for_each_ge(uint64_t tau, F&& f) const {
    const unsigned short t1 = (unsigned short)(tau - 1);
    const u16x2 t = {t1, t1};
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const u16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, w[j]), t);
      if (__builtin_bit_cast(uint32_t, d) != 0u) {
        if (d.x) f(w[j] & 0xffffu, 2 * j);
        if (d.y) f(w[j] >> 16, 2 * j + 1);
      }
    }
  }
  static constexpr uint64_t kKeyLimit = 0x10000u;   // keys are < this
  __device__ static uint32_t key_at(const uint16_t* p) { return bf16_key(*p); }
  __device__ static float value(uint32_t k) { return bf16_key_value(k); }
};

template <> struct Chunk<float> {
  static constexpr int VEC = 4, L = kPerThread / VEC;
  uint4 raw[L];
  uint32_t w[kPerThread];

  __device__ void issue(const float* rowp, int64_t c_start, int64_t valid, int tid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      raw[l] = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ void make_keys(const float* rowp, int64_t c_start, int64_t valid, int tid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      const uint32_t r4[4] = {raw[l].x, raw[l].y, raw[l].z, raw[l].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[l * 4 + q] = (e0 + VEC <= valid) ? f32_key(r4[q])
                       : (e0 + q < valid) ? f32_key(__float_as_uint(rowp[e0 + q])) : 0u;
    }
  }
  __device__ uint32_t max_key() const {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) m = max(m, w[j]);
    return m;
  }
  template <class F> __device__ void for_each_ge(uint64_t tau, F&& f) const {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if ((uint64_t)w[j] >= tau) f(w[j], j);
  }
  static constexpr uint64_t kKeyLimit = 0x100000000ull;
  __device__ static uint32_t key_at(const float* p) { return f32_key(__float_as_uint(*p)); }
  __device__ static float value(uint32_t k) { return f32_key_value(k); }
};

struct Shared {
  uint64_t pool[kMaxK + kCap];   // [0, nbest): held best; then new candidates
  uint64_t best_tmp[kMaxK];
  uint32_t tmax[kThreads];
  uint32_t gmax[64];
  uint32_t red[kThreads / 64];
  uint32_t count;                // new candidates appended this chunk
  uint32_t tau_lo, tau_hi;       // threshold (64-bit, split)
};

__device__ __forceinline__ int64_t value_id(int64_t c_start, int i, int vec) {
  return c_start + ((int64_t)(i / vec) * kThreads + threadIdx.x) * vec + (i % vec);
}

// Workgroup-wide sum of one value per thread (all threads must call).
__device__ uint32_t block_sum(uint32_t v, Shared& sh) {
  v = wave_sum_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) s += sh.red[i];
  return s;
}

// Counts, over this thread's chunk values re-read from memory, those with
// key >= lo_key (mode 0), key > key_eq (mode 1), or key == key_eq and
// id < id_bound (mode 2); then sums over the workgroup.
template <typename TIO>
__device__ uint32_t count_pass(const TIO* rowp, int64_t c_start, int64_t valid, int mode, uint64_t lo_key,
                               uint32_t key_eq, int64_t id_bound, Shared& sh) {
  constexpr int VEC = Chunk<TIO>::VEC;
  uint32_t c = 0;
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t id = value_id(c_start, i, VEC);
    if (id >= valid) continue;
    const uint32_t k = Chunk<TIO>::key_at(rowp + id);
    if (mode == 0) c += ((uint64_t)k >= lo_key) ? 1u : 0u;
    else if (mode == 1) c += (k > key_eq) ? 1u : 0u;
    else c += (k == key_eq && id < id_bound) ? 1u : 0u;
  }
  return block_sum(c, sh);
}

// Exact narrowing when a chunk yields more than kCap candidates: replaces the
// new candidates (pool[nbest, ...)) by exactly the chunk's K best (or all its
// real values if fewer) and sets sh.count to their number.
template <typename TIO>
__device__ __noinline__ void narrow_exact(const TIO* rowp, int64_t c_start, int64_t valid, int K, int nbest,
                                          Shared& sh) {
  constexpr int VEC = Chunk<TIO>::VEC;
  const uint32_t n_real = count_pass(rowp, c_start, valid, 0, 1, 0, 0, sh);
  uint32_t kt = 1;                                     // take every real value when there are few
  int64_t id_bound = INT64_MAX;
  if (n_real > (uint32_t)K) {
    uint64_t lo = 1, hi = Chunk<TIO>::kKeyLimit;       // count(>= lo) >= K > count(>= hi)
    while (hi - lo > 1) {
      const uint64_t mid = lo + (hi - lo) / 2;
      if (count_pass(rowp, c_start, valid, 0, mid, 0, 0, sh) >= (uint32_t)K) lo = mid; else hi = mid;
    }
    kt = (uint32_t)lo;
    const uint32_t c_gt = count_pass(rowp, c_start, valid, 1, 0, kt, 0, sh);
    const uint32_t need = (uint32_t)K - c_gt;          // ties at kt to take, lowest ids first
    int64_t lo_i = c_start, hi_i = c_start + kChunk;   // count(id < lo_i) < need <= count(id < hi_i)
    while (hi_i - lo_i > 1) {
      const int64_t mid = lo_i + (hi_i - lo_i) / 2;
      if (count_pass(rowp, c_start, valid, 2, 0, kt, mid, sh) >= need) hi_i = mid; else lo_i = mid;
    }
    id_bound = hi_i;
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.count = 0;
  __syncthreads();
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t id = value_id(c_start, i, VEC);
    if (id >= valid) continue;
    const uint32_t k = Chunk<TIO>::key_at(rowp + id);
    if (k > kt || (k == kt && id < id_bound)) {
      const uint32_t pos = atomicAdd(&sh.count, 1u);
      if (pos < (uint32_t)kCap) sh.pool[nbest + pos] = composite(k, id);
    }
  }
  __syncthreads();
}

// Keep the K best of pool[0, n) in pool[0, min(n, K)) (sorted, best first).
__device__ void keep_best(Shared& sh, int n, int K) {
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const uint64_t c = sh.pool[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (sh.pool[j] > c) ? 1 : 0;
    if (rank < K) sh.best_tmp[rank] = c;
  }
  __syncthreads();
  const int m = n < K ? n : K;
  for (int i = threadIdx.x; i < m; i += kThreads) sh.pool[i] = sh.best_tmp[i];
  __syncthreads();
}

__device__ __forceinline__ float unary_transform(float z, float mult, float cap) {
  float y = mult * z;
  if (cap > 0.f) y = cap * tanhf(y / cap);
  return (z == -INFINITY) ? -INFINITY : y;     // masked entries stay masked
}

template <typename TIO>
__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const TIO* __restrict__ logits, int64_t row_stride,
                                                             int64_t valid_vocab, int32_t K, int32_t chunks,
                                                             int32_t segs, int32_t chunks_per_seg, float mult,
                                                             float cap, uint64_t* __restrict__ parts,
                                                             int64_t* __restrict__ ids_out,
                                                             float* __restrict__ unary_out) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / segs;
  const int seg = (int)(blockIdx.x % segs);
  const int c_begin = seg * chunks_per_seg;
  const int c_end = min(chunks, c_begin + chunks_per_seg);
  const TIO* rowp = logits + row * row_stride;
  int groups = 1;
  while (groups < K) groups <<= 1;               // P = next power of two >= K
  const int gsize = kThreads / groups;           // threads per group (>= 8)

  int nbest = 0;                                 // held best composites (uniform)
  Chunk<TIO> cur;
  if (c_begin < c_end) cur.issue(rowp, (int64_t)c_begin * kChunk, valid_vocab, tid);
  for (int c = c_begin; c < c_end; ++c) {
    const int64_t c_start = (int64_t)c * kChunk;
    Chunk<TIO> next;
    if (c + 1 < c_end) next.issue(rowp, c_start + kChunk, valid_vocab, tid);   // prefetch
    cur.make_keys(rowp, c_start, valid_vocab, tid);

    // ---- threshold --------------------------------------------------------
    if (nbest < K) {
      sh.tmax[tid] = cur.max_key();
      __syncthreads();
      if (tid < groups) {
        uint32_t g = 0;
        for (int i = 0; i < gsize; ++i) g = max(g, sh.tmax[tid * gsize + i]);
        sh.gmax[tid] = g;
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t tau = 0xffffffffu;
        int nonempty = 0;
        for (int g = 0; g < groups; ++g)
          if (sh.gmax[g] != 0) { ++nonempty; tau = min(tau, sh.gmax[g]); }
        const uint64_t t = (nonempty >= K) ? (uint64_t)tau : 1u;   // too few: every real value
        sh.tau_lo = (uint32_t)t;
        sh.tau_hi = (uint32_t)(t >> 32);
        sh.count = 0;
      }
    } else if (tid == 0) {
      // later values have larger ids than every held one: they must beat the
      // K-th key strictly
      const uint64_t t = (uint64_t)composite_key(sh.pool[K - 1]) + 1;
      sh.tau_lo = (uint32_t)t;
      sh.tau_hi = (uint32_t)(t >> 32);
      sh.count = 0;
    }
    __syncthreads();
    const uint64_t tau = ((uint64_t)sh.tau_hi << 32) | sh.tau_lo;

    // ---- compact the survivors behind the held best -----------------------
    if (tau < Chunk<TIO>::kKeyLimit) {
      cur.for_each_ge(tau, [&](uint32_t k, int i) {
        const uint32_t pos = atomicAdd(&sh.count, 1u);
        if (pos < (uint32_t)kCap) sh.pool[nbest + pos] = composite(k, value_id(c_start, i, Chunk<TIO>::VEC));
      });
    }
    __syncthreads();
    uint32_t n = sh.count;
    if (n > (uint32_t)kCap) {
      narrow_exact<TIO>(rowp, c_start, valid_vocab, K, nbest, sh);
      n = sh.count;
    }
    if (n > 0) {
      keep_best(sh, nbest + (int)n, K);
      nbest = min(K, nbest + (int)n);
    }
    if (c + 1 < c_end) cur = next;
  }

  // ---- output -----------------------------------------------------------
  if (segs == 1) {
    for (int i = tid; i < nbest; i += kThreads) {
      const uint64_t c = sh.pool[i];
      ids_out[row * K + i] = composite_id(c);
      unary_out[row * K + i] = unary_transform(Chunk<TIO>::value(composite_key(c)), mult, cap);
    }
  } else {
    uint64_t* dst = parts + ((size_t)row * segs + seg) * K;
    for (int i = tid; i < K; i += kThreads) dst[i] = i < nbest ? sh.pool[i] : 0ull;
  }
}

// Merge of the per-segment K best (rows split over several workgroups).
template <typename TIO>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const uint64_t* __restrict__ parts, int32_t K,
                                                              int32_t segs, float mult, float cap,
                                                              int64_t* __restrict__ ids_out,
                                                              float* __restrict__ unary_out) {
  __shared__ uint64_t cand[kCap];
  const int64_t row = blockIdx.x;
  const int m = segs * K;
  const uint64_t* src = parts + (size_t)row * m;
  for (int i = threadIdx.x; i < m; i += kThreads) cand[i] = src[i];
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += kThreads) {
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
  p.chunks = (int32_t)((valid_vocab + kChunk - 1) / kChunk);
  if (p.chunks < 1) p.chunks = 1;
  // One workgroup per row once rows cover the chip; otherwise split rows so
  // that about 512 workgroups stream, and merge the segments afterwards.
  int segs = 1;
  if (n_rows > 0 && n_rows < 256) {
    segs = (int)((512 + n_rows - 1) / n_rows);
    if (segs > p.chunks) segs = p.chunks;
    if (segs * top_k > kCap) segs = kCap / top_k;
    if (segs < 1) segs = 1;
  }
  p.segs = segs;
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
    hipLaunchKernelGGL(topk_rows_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a.logits), a.row_stride, a.valid_vocab, a.top_k, p.chunks,
                       p.segs, p.chunks_per_seg, a.multiplier, a.softcap, parts, a.ids_out, a.unary_out);
  else
    hipLaunchKernelGGL(topk_rows_kernel<float>, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(a.logits), a.row_stride, a.valid_vocab, a.top_k, p.chunks,
                       p.segs, p.chunks_per_seg, a.multiplier, a.softcap, parts, a.ids_out, a.unary_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.segs == 1) return e;
  if (a.dtype == DFLASH_BF16)
    hipLaunchKernelGGL(topk_merge_kernel<uint16_t>, dim3((unsigned)p.n_rows), dim3(kThreads), 0, stream, parts,
                       a.top_k, p.segs, a.multiplier, a.softcap, a.ids_out, a.unary_out);
  else
    hipLaunchKernelGGL(topk_merge_kernel<float>, dim3((unsigned)p.n_rows), dim3(kThreads), 0, stream, parts,
                       a.top_k, p.segs, a.multiplier, a.softcap, a.ids_out, a.unary_out);
  return hipGetLastError();
}

}  // namespace dflash

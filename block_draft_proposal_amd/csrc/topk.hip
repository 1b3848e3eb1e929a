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
// Design (HBM-bound stream, one pass over the logits):
//  * Every value becomes an order-preserving unsigned key (-0 and +0 share a
//    key; a position outside the logical vocabulary has key 0, below every
//    real value), and every (key, id) pair a 56-bit composite
//    key << 24 | (2^24 - 1 - id) whose order is exactly (value desc, id asc)
//    and which is unique within a row.
//  * A row is cut into chunks of 16384 values; one 256-thread workgroup reads
//    a chunk (64 values per thread, all 16-byte loads in flight at once, each
//    wave load one contiguous 1 KiB) and turns it into keys in registers
//    (bf16 keys packed two per register, built with packed 16-bit ops).
//  * Threshold: split the workgroup into P >= K thread groups; the minimum of
//    the groups' maxima is a key that at least K distinct values reach, so the
//    chunk's top-K all have keys >= it.  On random data only a few dozen
//    values pass; a packed saturating subtract tests two keys per instruction,
//    survivors are compacted into LDS and ranked exactly by counting.
//  * If too many pass (mass ties), an exact bisection on the key, then on the
//    id among the tied key, narrows the set to exactly K.  That path re-reads
//    the chunk (cache-resident) instead of holding extra registers.
//  * Each workgroup writes its chunk's K best composites; the last workgroup
//    of a row to finish (atomic ticket) ranks the row's chunks x K candidates,
//    decodes ids and values, applies the transform in fp32 and writes the row.
//  * Workgroups of one row are placed on one XCD (round-robin dispatch across
//    the 8 XCDs), so the merge reads partials from the same L2.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 64;
constexpr int kChunk = kThreads * kPerThread;   // values per workgroup
constexpr int kCap = kTopkMergeCap;             // LDS candidate slots
constexpr uint32_t kIdMask = 0xffffffu;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t composite(uint32_t key, int64_t id) {
  return ((uint64_t)key << 24) | (uint64_t)(kIdMask - (uint32_t)id);
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

// Keys of one thread's 64 chunk values.  Value i (0..63) sits at
// id = c_start + ((i / VEC) * 256 + tid) * VEC + i % VEC.
template <typename TIO> struct ChunkKeys;

template <> struct ChunkKeys<uint16_t> {
  static constexpr int VEC = 8, L = kPerThread / VEC, W = kPerThread / 2;
  uint32_t w[W];    // word j holds keys of values 2j (low half) and 2j+1 (high half)

  __device__ void load(const uint16_t* rowp, int64_t c_start, int64_t valid, int tid) {
    uint4 raw[L];
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      raw[l] = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
    }
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
  // Calls f(key, value index) for every key >= tau (tau >= 1).
  template <class F> __device__ void for_each_ge(uint32_t tau, F&& f) const {
    const u16x2 t = {(unsigned short)(tau - 1), (unsigned short)(tau - 1)};
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const u16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, w[j]), t);
      if (__builtin_bit_cast(uint32_t, d) != 0u) {
        if (d.x) f(w[j] & 0xffffu, 2 * j);
        if (d.y) f(w[j] >> 16, 2 * j + 1);
      }
    }
  }
  __device__ static uint32_t key_at(const uint16_t* p) { return bf16_key(*p); }
  __device__ static float value(uint32_t k) { return bf16_key_value(k); }
};

template <> struct ChunkKeys<float> {
  static constexpr int VEC = 4, L = kPerThread / VEC;
  uint32_t w[kPerThread];

  __device__ void load(const float* rowp, int64_t c_start, int64_t valid, int tid) {
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      uint4 r = (e0 + VEC <= valid) ? *reinterpret_cast<const uint4*>(rowp + e0) : make_uint4(0u, 0u, 0u, 0u);
      w[l * 4 + 0] = r.x; w[l * 4 + 1] = r.y; w[l * 4 + 2] = r.z; w[l * 4 + 3] = r.w;
    }
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const int64_t e0 = c_start + ((int64_t)l * kThreads + tid) * VEC;
      if (e0 + VEC <= valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[l * 4 + q] = f32_key(w[l * 4 + q]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[l * 4 + q] = (e0 + q < valid) ? f32_key(__float_as_uint(rowp[e0 + q])) : 0u;
      }
    }
  }
  __device__ uint32_t max_key() const {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) m = max(m, w[j]);
    return m;
  }
  template <class F> __device__ void for_each_ge(uint32_t tau, F&& f) const {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (w[j] >= tau) f(w[j], j);
  }
  __device__ static uint32_t key_at(const float* p) { return f32_key(__float_as_uint(*p)); }
  __device__ static float value(uint32_t k) { return f32_key_value(k); }
};

struct Shared {
  uint64_t cand[kCap];
  uint32_t tmax[kThreads];
  uint32_t gmax[64];
  uint32_t red[kThreads / 64];
  uint32_t count;
  uint32_t tau;
  uint32_t last;
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
  constexpr int VEC = ChunkKeys<TIO>::VEC;
  uint32_t c = 0;
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t id = value_id(c_start, i, VEC);
    if (id >= valid) continue;
    const uint32_t k = ChunkKeys<TIO>::key_at(rowp + id);
    if (mode == 0) c += ((uint64_t)k >= lo_key) ? 1u : 0u;
    else if (mode == 1) c += (k > key_eq) ? 1u : 0u;
    else c += (k == key_eq && id < id_bound) ? 1u : 0u;
  }
  return block_sum(c, sh);
}

// Exact narrowing when more than kCap values reach the first threshold:
// leaves exactly the chunk's top-K composites in sh.cand[0..K) and sets
// sh.count = K (or the number of real values, if fewer).
template <typename TIO>
__device__ __noinline__ void narrow_exact(const TIO* rowp, int64_t c_start, int64_t valid, int K, uint32_t tau,
                                          uint32_t top_key, Shared& sh) {
  constexpr int VEC = ChunkKeys<TIO>::VEC;
  uint64_t lo = tau, hi = (uint64_t)top_key + 1;      // count(>= lo) >= K > count(>= hi)
  while (hi - lo > 1) {
    const uint64_t mid = lo + (hi - lo) / 2;
    if (count_pass(rowp, c_start, valid, 0, mid, 0, 0, sh) >= (uint32_t)K) lo = mid; else hi = mid;
  }
  const uint32_t kt = (uint32_t)lo;
  const uint32_t c_ge = count_pass(rowp, c_start, valid, 0, kt, 0, 0, sh);
  int64_t id_bound = INT64_MAX;                       // ties at kt: only ids below this
  if (c_ge > (uint32_t)kCap) {
    const uint32_t c_gt = count_pass(rowp, c_start, valid, 1, 0, kt, 0, sh);
    const uint32_t need = (uint32_t)K - c_gt;
    int64_t lo_i = c_start, hi_i = c_start + kChunk;  // count(id < lo_i) < need <= count(id < hi_i)
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
    const uint32_t k = ChunkKeys<TIO>::key_at(rowp + id);
    if (k > kt || (k == kt && id < id_bound)) {
      const uint32_t pos = atomicAdd(&sh.count, 1u);
      if (pos < (uint32_t)kCap) sh.cand[pos] = composite(k, id);
    }
  }
  __syncthreads();
}

// Rank the first n LDS candidates (unique nonzero composites) and write the
// best k in order to dst[0..k); positions without a candidate get 0.
__device__ void rank_to_global(const Shared& sh, int n, int k, uint64_t* dst) {
  if (n > kCap) n = kCap;                 // cannot happen (see narrow_exact); keeps LDS reads in bounds
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const uint64_t c = sh.cand[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (sh.cand[j] > c) ? 1 : 0;
    if (rank < k) dst[rank] = c;
  }
  for (int r = n + (int)threadIdx.x; r < k; r += kThreads) dst[r] = 0;
}

template <typename TIO>
__global__ __launch_bounds__(kThreads) void topk_kernel(const TIO* __restrict__ logits,
                                                        int64_t row_stride, int64_t valid_vocab,
                                                        int64_t n_rows, int32_t K, int32_t chunks,
                                                        float mult, float cap,
                                                        uint64_t* __restrict__ parts,
                                                        uint32_t* __restrict__ counters,
                                                        int64_t* __restrict__ ids_out,
                                                        float* __restrict__ unary_out) {
  constexpr int VEC = ChunkKeys<TIO>::VEC;
  __shared__ Shared sh;
  const int tid = threadIdx.x;

  // XCD-aware placement: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of (row, chunk) work items so a row's chunks share an L2.
  const int64_t total = n_rows * chunks;
  const int64_t per_xcd = (int64_t)gridDim.x / 8;
  const int64_t vid = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (vid >= total) return;
  const int64_t row = vid / chunks;
  const int chunk = (int)(vid % chunks);
  const int64_t c_start = (int64_t)chunk * kChunk;
  const TIO* rowp = logits + row * row_stride;

  ChunkKeys<TIO> keys;
  keys.load(rowp, c_start, valid_vocab, tid);

  // ---- threshold from group maxima ---------------------------------------
  int groups = 1;
  while (groups < K) groups <<= 1;               // P = next power of two >= K
  const int gsize = kThreads / groups;           // threads per group (>= 8)
  sh.tmax[tid] = keys.max_key();
  if (tid == 0) sh.count = 0;
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
    for (int g = 0; g < groups; ++g) {
      if (sh.gmax[g] != 0) { ++nonempty; tau = min(tau, sh.gmax[g]); }
    }
    sh.tau = (nonempty >= K) ? tau : 1u;         // too few: every real value
  }
  __syncthreads();
  const uint32_t tau = sh.tau;

  // ---- compact the keys >= tau -------------------------------------------
  keys.for_each_ge(tau, [&](uint32_t k, int i) {
    const uint32_t pos = atomicAdd(&sh.count, 1u);
    if (pos < (uint32_t)kCap) sh.cand[pos] = composite(k, value_id(c_start, i, VEC));
  });
  __syncthreads();
  uint32_t n = sh.count;
  if (n > (uint32_t)kCap) {
    uint32_t top = 0;
    for (int g = 0; g < groups; ++g) top = max(top, sh.gmax[g]);
    narrow_exact<TIO>(rowp, c_start, valid_vocab, K, tau, top, sh);
    n = sh.count;
  }

  // ---- this chunk's K best -> partials ---------------------------------
  uint64_t* my_parts = parts + ((size_t)row * chunks + chunk) * K;
  rank_to_global(sh, (int)n, K, my_parts);

  // ---- last workgroup of the row merges ----------------------------------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t ticket = atomicAdd(&counters[row], 1u);
    sh.last = (ticket == (uint32_t)chunks - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!sh.last) return;
  __threadfence();
  const int m = chunks * K;
  const uint64_t* row_parts = parts + (size_t)row * chunks * K;
  for (int i = tid; i < m; i += kThreads) sh.cand[i] = row_parts[i];
  __syncthreads();
  for (int i = tid; i < m; i += kThreads) {
    const uint64_t c = sh.cand[i];
    if (c == 0) continue;                       // empty slot of a short chunk
    int rank = 0;
    for (int j = 0; j < m; ++j) rank += (sh.cand[j] > c) ? 1 : 0;
    if (rank < K) {
      const uint32_t key = (uint32_t)(c >> 24);
      const int64_t id = (int64_t)(kIdMask - (uint32_t)(c & kIdMask));
      const float z = ChunkKeys<TIO>::value(key);
      float y = mult * z;
      if (cap > 0.f) y = cap * tanhf(y / cap);
      if (z == -INFINITY) y = -INFINITY;      // masked entries stay masked
      ids_out[row * K + rank] = id;
      unary_out[row * K + rank] = y;
    }
  }
  if (tid == 0) counters[row] = 0u;           // leave the ticket cleared
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
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
  p.parts_offset = 0;
  p.counters_offset = align256((size_t)n_rows * p.chunks * top_k * sizeof(uint64_t));
  p.bytes = p.counters_offset + align256((size_t)n_rows * sizeof(uint32_t));
  if (n_rows == 0) p.bytes = 0;
  return p;
}

hipError_t launch_topk_zero(const TopkArgs& a, const TopkPlan& p, hipStream_t stream) {
  if (p.n_rows == 0) return hipSuccess;
  uint32_t* counters = reinterpret_cast<uint32_t*>(static_cast<char*>(a.workspace) + p.counters_offset);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((p.n_rows + 255) / 256)), dim3(256), 0, stream,
                     counters, p.n_rows);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t stream) {
  if (p.n_rows == 0) return hipSuccess;
  char* ws = static_cast<char*>(a.workspace);
  uint64_t* parts = reinterpret_cast<uint64_t*>(ws + p.parts_offset);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + p.counters_offset);
  const int64_t work = p.n_rows * p.chunks;
  const int64_t grid = (work + 7) / 8 * 8;     // whole rounds over the 8 XCDs
  if (a.dtype == DFLASH_BF16)
    hipLaunchKernelGGL(topk_kernel<uint16_t>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a.logits), a.row_stride, a.valid_vocab, p.n_rows,
                       a.top_k, p.chunks, a.multiplier, a.softcap, parts, counters, a.ids_out,
                       a.unary_out);
  else
    hipLaunchKernelGGL(topk_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       static_cast<const float*>(a.logits), a.row_stride, a.valid_vocab, p.n_rows,
                       a.top_k, p.chunks, a.multiplier, a.softcap, parts, counters, a.ids_out,
                       a.unary_out);
  return hipGetLastError();
}

}  // namespace dflash

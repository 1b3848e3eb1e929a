// Internal declarations of the DFlash2 HIP library: device helpers shared by
// the kernels and the host-side launchers called by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dflash {

// ---------------------------------------------------------------------------
// bfloat16 storage helpers (raw 16-bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {               // bf16 storage
  static constexpr int kVec = 8;                  // elements per 16-byte vector
  __device__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t nan_value() { return 0x7fc0u; }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load(const float* p) { return *p; }
  __device__ static float to_f32(float v) { return v; }
  __device__ static float nan_value() { return __builtin_nanf(""); }
};

// 16 bytes as a native 4 x u32 vector.  Register arrays of it, and selects
// between two of them, stay in registers (the HIP uint4 struct can be
// demoted to scratch memory by such a select).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ void unpack16(u32x4 v, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(v[i] << 16);
    o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(u32x4 v, float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
}

// Unpack one 16-byte vector into fp32 values.
__device__ __forceinline__ void unpack16(const uint4& v, float (&o)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& v, float (&o)[4]) {
  o[0] = __uint_as_float(v.x);
  o[1] = __uint_as_float(v.y);
  o[2] = __uint_as_float(v.z);
  o[3] = __uint_as_float(v.w);
}

// ---------------------------------------------------------------------------
// Top-K keys (shared by the streaming top-K and the fused head epilogue)
// ---------------------------------------------------------------------------
// Every value has an order-preserving unsigned key; every (key, id) pair a
// 56-bit composite key << 24 | (2^24 - 1 - id) whose order is exactly
// (value descending, id ascending) and which is unique within a row
// (ids < 2^24).  Composite 0 is below every real one.
constexpr uint32_t kIdMask = 0xffffffu;
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
// The unary transform of a selected logit: m z, then cap tanh(. / cap) when
// cap > 0; a masked (-inf) entry stays -inf.
__device__ __forceinline__ float unary_transform(float z, float mult, float cap) {
  float y = mult * z;
  if (cap > 0.f) y = cap * tanhf(y / cap);
  return (z == -INFINITY) ? -INFINITY : y;     // masked entries stay masked
}
// Number of entries of the sorted (descending) list l[0, n) greater than c.
__device__ __forceinline__ int count_greater(const uint64_t* l, int n, uint64_t c) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (l[mid] > c) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Wave (64-lane) reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
struct ConvArgs {
  const void* x;
  const void* base;
  const void* delta;
  int64_t delta_row_stride;
  void* out;
  int64_t n_tokens;
  int32_t hidden, group_size, taps, block_size;
  int32_t dtype;          // DFLASH_F32 / DFLASH_BF16
};
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);

struct TopkPlan {
  int64_t n_rows, valid_vocab;
  int32_t top_k;
  int32_t chunks;           // 16384-value chunks per row
  int32_t segs;             // workgroups per row (1: no merge kernel)
  int32_t chunks_per_seg;
  size_t parts_offset;      // byte offset of the per-segment partials in the workspace
  size_t bytes;             // total workspace bytes (0 when segs == 1)
};
TopkPlan plan_topk(int64_t n_rows, int64_t valid_vocab, int32_t top_k);
// LDS slots for one chunk's new candidates, and for a row merge.
constexpr int kTopkMergeCap = 2048;

struct TopkArgs {
  const void* logits;
  int64_t row_stride, n_rows, vocab, valid_vocab;
  int32_t top_k;
  float multiplier, softcap;
  int32_t dtype;
  int64_t* ids_out;
  float* unary_out;
  void* workspace;
};
hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t stream);

constexpr int kMaxTopK = 32;   // DFLASH_MAX_TOP_K

// Most slices the projection's contraction is split into (their partial
// sums are added by the consumer, in slice order).
constexpr int kMaxProjSplit = 32;
struct ProjPlan {
  int32_t n_rows, rank, hidden;
  int32_t row_tiles, ksplit, kslice;   // split of the contraction over workgroups
  int32_t frags;                       // row fragments of 16 per wave (bf16)
  size_t bytes;                        // fp32 partials [ksplit][n_rows][rank]
};
ProjPlan plan_proj(int32_t n_rows, int32_t rank, int32_t hidden, int32_t dtype);

struct SelectArgs {
  const int64_t* ids;
  const float* unary;
  const void* hidden;
  int64_t hidden_req_stride, hidden_slot_stride;
  const int64_t* anchor;
  const void* sel_a;
  const void* sel_b;
  const void* proj;
  int32_t n_req, slots, top_k, hidden_size, rank;
  int64_t vocab;
  int32_t dtype;
  float* u_parts;           // workspace: ProjPlan::bytes
  float* scores;            // [n_req, slots, K, K]
};
hipError_t launch_proj(const SelectArgs& a, const ProjPlan& p, hipStream_t stream);
hipError_t launch_lattice(const SelectArgs& a, const ProjPlan& p, hipStream_t stream);

struct WalkArgs {
  const float* scores;
  const int64_t* ids;
  const float* uniforms;
  const float* temperatures;
  const uint8_t* greedy;
  int32_t n_req, slots, top_k;
  int64_t* tokens;
  float* q;
};
hipError_t launch_walk(const WalkArgs& a, hipStream_t stream);

// Dense head: logits[n, v] = round_bf16(sum_k hidden[n, k] W[v, k]) (bf16).
struct LmHeadArgs {
  const void* hidden;
  int64_t hidden_row_stride;   // elements
  const void* weight;          // [vocab, hidden_size], rows contiguous
  int64_t n_rows;
  int32_t hidden_size;
  int64_t vocab;
  void* logits;
  int64_t logits_row_stride;   // elements
};
hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t stream);

// Fused head + top-K: per-row K best of each group of column tiles (sorted
// composites in the workspace [n_rows][n_grp][K]), then a merge per row.
constexpr int kLmMergeCand = 3072;  // merge candidates of one row held in LDS (24 KB)
struct LmTopkPlan {
  int32_t n_mb, n_nb, tiles_per_group, n_grp;
  size_t bytes;
};
LmTopkPlan plan_lm_head_topk(int64_t n_rows, int64_t vocab, int32_t top_k);
hipError_t launch_lm_head_topk(const LmHeadArgs& a, const LmTopkPlan& p, int64_t valid_vocab, int32_t top_k,
                               float mult, float cap, int64_t* ids_out, float* unary_out, void* workspace,
                               hipStream_t stream);

// Lattice and walk in one kernel (one workgroup per request) when the
// request's lattice and its staging fit in LDS; bit-identical to
// launch_lattice followed by launch_walk.  scores_out may be null.
// gfx950 lets one workgroup address 160 KB of LDS
constexpr size_t kLatticeWalkLdsMax = 160 * 1024;
constexpr size_t kWalkLdsMax = 160 * 1024;
size_t lattice_walk_lds_bytes(int slots, int top_k, int rank, int dtype);
bool lattice_walk_fits(const struct SelectArgs& a);   // LDS size, rank multiple of a vector, 16-byte tables
hipError_t launch_lattice_walk(const SelectArgs& a, const ProjPlan& p, const WalkArgs& w, float* scores_out,
                               hipStream_t stream);

}  // namespace dflash

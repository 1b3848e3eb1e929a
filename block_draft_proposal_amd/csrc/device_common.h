// Device helpers of the DFlash2 HIP kernels: bf16 storage, 16-byte vectors,
// the order-preserving top-K keys and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Buffer resources: word 3 of a raw dword buffer (32-bit data format, no
// swizzle).  A load through a buffer resource past num_records bytes returns
// zeros and reads no memory.
constexpr int kBufferFlags = 0x00020000;
// cache policy of a streaming (non-temporal) buffer load
constexpr int kBufferStream = 2;
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming (non-temporal) forms, for data read or written once: on this
// chip a stream of them runs well above the plain forms' rate (a 16-byte-lane
// copy: ~5.9 against ~5.0 TB/s).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }

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
// Workgroups of a launch are dealt to the chip's 8 XCDs in turn (workgroup
// w runs on XCD w % 8), each XCD with its own L2.  This renumbers them so
// that consecutive numbers share an XCD: XCD x takes the contiguous range
// starting at x * (n / 8) + min(x, n % 8).  Work that neighbouring numbers
// share (the same cache lines) is then fetched into one L2, not several.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t w, uint32_t n) {
  const uint32_t q = n >> 3, rem = n & 7, x = w & 7;
  return x * q + (x < rem ? x : rem) + (w >> 3);
}

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

}  // namespace dflash

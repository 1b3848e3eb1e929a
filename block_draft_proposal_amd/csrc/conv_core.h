// Per-vector arithmetic of the block-causal grouped dynamic depthwise
// convolution ("[Spec] DFlash2: local convolution + candidate selector", code
// excerpt of the grouped conv):
//   out[i,c] = sum_{t < T, t <= i mod B} (base[t,c] + delta[i,t,c/gs]) * x[i-t,c]
// shared by every kernel that produces conv outputs, so that they agree bit
// for bit: the coefficient is base + delta in fp32, the taps are taken in
// order 0, 1, ..., the first product is rounded on its own and every later
// one is fused into the sum, and the result is rounded once to the storage
// dtype (bf16: to nearest, ties to even).
#pragma once

#include "device_common.h"

namespace dflash {

// acc[e] for the VEC channels of one token at position j inside its block.
// coef_at(t, coef) gives tap t's coefficients, x_at(t, xv) the input row
// j - t; taps past the block start (t > j) are not taken.
template <int VEC, int TAPS, class Coef, class Xv>
__device__ __forceinline__ void conv_token(int j, Coef&& coef_at, Xv&& x_at, float (&acc)[VEC]) {
#pragma unroll
  for (int t = 0; t < TAPS; ++t) {
    if (t > j) break;
    float coef[VEC], xv[VEC];
    coef_at(t, coef);
    x_at(t, xv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = (t == 0) ? coef[e] * xv[e] : fmaf(coef[e], xv[e], acc[e]);
  }
}

// Coefficients of one tap for a vector lying in one group: base row + the
// group's dynamic scalar.
template <int VEC>
__device__ __forceinline__ void coef_one_group(const float (&bt)[VEC], float d, float (&coef)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) coef[e] = bt[e] + d;
}

// Eight fp32 conv outputs rounded to bf16 (nearest, ties to even), packed:
// v_cvt_pk_bf16_f32 rounds two values per instruction in the default
// round-to-nearest-even mode.
typedef __bf16 conv_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float conv_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const conv_f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, conv_bf16x2_t));
}
__device__ __forceinline__ uint4 pack_bf16x8(const float (&a)[8]) {
  uint4 v;
  v.x = pack_bf16x2(a[0], a[1]);
  v.y = pack_bf16x2(a[2], a[3]);
  v.z = pack_bf16x2(a[4], a[5]);
  v.w = pack_bf16x2(a[6], a[7]);
  return v;
}

}  // namespace dflash

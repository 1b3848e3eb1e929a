// Per-vector arithmetic of the block-causal grouped dynamic depthwise
// convolution ("[Spec] DFlash2: local convolution + candidate selector", code
// excerpt of the grouped conv):
//   out[i,c] = sum_{t < T, t <= i mod B} (base[t,c] + delta[i,t,c/gs]) * x[i-t,c]
// shared by every kernel that produces conv outputs, so that they agree bit
// for bit: the coefficient is base + delta in fp32, the taps are taken in
// order 0, 1, ..., the first product is rounded on its own and every later
// one is fused into the sum, and the result is rounded once to the storage
// dtype.
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

// Eight fp32 conv outputs rounded to bf16 (nearest, ties to even), packed.
__device__ __forceinline__ uint4 pack_bf16x8(const float (&a)[8]) {
  uint4 v;
  v.x = f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16);
  v.y = f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16);
  v.z = f32_to_bf16_rne(a[4]) | (f32_to_bf16_rne(a[5]) << 16);
  v.w = f32_to_bf16_rne(a[6]) | (f32_to_bf16_rne(a[7]) << 16);
  return v;
}

}  // namespace dflash

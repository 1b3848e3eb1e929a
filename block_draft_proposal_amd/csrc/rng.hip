// Counter-based uniforms for a captured draft step.
//
// The draft sampler of "[Spec] DFlash2: local convolution + candidate
// selector" (worker excerpt) draws the walk's uniforms inside its captured
// graph with a counter-based generator, so a replay draws fresh numbers from
// nothing but a staged counter.  Generator: Philox-4x32-10 as published by
// Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2,
// 3", SC 2011): ten rounds, each two 32 x 32 -> 64-bit products of the first
// and third words that scramble the other two with the key, the key stepping
// by the Weyl constants between rounds.
//
// Element i of the output is word i % 4 of block b = offset + i / 4 (the
// 64-bit block index in the first two counter words, the others zero; key =
// the seed's two 32-bit halves), keeping its top 24 bits: a float in [0, 1)
// that is a multiple of 2^-24.  seed and offset are read from device memory,
// so a captured launch picks up whatever the host staged before the replay.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

__global__ void philox_uniform_kernel(const uint64_t* __restrict__ seed_offset, int64_t n, float* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * b >= n) return;
  const uint64_t seed = seed_offset[0], c = seed_offset[1] + (uint64_t)b;
  uint32_t x0 = (uint32_t)c, x1 = (uint32_t)(c >> 32), x2 = 0u, x3 = 0u;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = kPhiloxM0 * x0, hi0 = __umulhi(kPhiloxM0, x0);
    const uint32_t lo1 = kPhiloxM1 * x2, hi1 = __umulhi(kPhiloxM1, x2);
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  const uint32_t w[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * b + j < n) out[4 * b + j] = (float)(w[j] >> 8) * 0x1p-24f;
}

}  // namespace

hipError_t launch_philox_uniforms(const uint64_t* seed_offset, int64_t n, float* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(philox_uniform_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, stream,
                     seed_offset, n, out);
  return hipGetLastError();
}

}  // namespace dflash

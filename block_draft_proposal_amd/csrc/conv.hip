// Block-causal grouped dynamic depthwise convolution on gfx950.
//
// Operation ("[Spec] DFlash2: local convolution + candidate selector", code
// excerpt of the grouped conv):
//   out[i,c] = sum_{t < T, t <= i mod B} (base[t,c] + delta[i,t,c/gs]) * x[i-t,c]
//
// HBM-bound stream: each input row is read once, each output row written once.
// A thread owns one 16-byte channel vector (8 bf16 / 4 fp32 channels) of one
// run of consecutive tokens inside one block and walks the run in token order,
// keeping the last T-1 input vectors in registers as the tap history, so that
// x is fetched from memory once per token (plus a T-1 token halo when a block
// is split into several runs to give small batches enough threads).  Lanes of
// a wave hold consecutive channel vectors of the same token, so every load and
// store of a wave is one contiguous 1 KiB (bf16) segment.  The static kernel
// base[t, c] is loaded once per thread and reused for the whole run.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;

template <typename TIO>
__device__ __forceinline__ void load_vec(const TIO* p, float (&o)[Elem<TIO>::kVec]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  unpack16(v, o);
}

__device__ __forceinline__ void store_vec(uint16_t* p, const float (&a)[8]) {
  uint4 v;
  v.x = f32_to_bf16_rne(a[0]) | (f32_to_bf16_rne(a[1]) << 16);
  v.y = f32_to_bf16_rne(a[2]) | (f32_to_bf16_rne(a[3]) << 16);
  v.z = f32_to_bf16_rne(a[4]) | (f32_to_bf16_rne(a[5]) << 16);
  v.w = f32_to_bf16_rne(a[6]) | (f32_to_bf16_rne(a[7]) << 16);
  *reinterpret_cast<uint4*>(p) = v;
}
__device__ __forceinline__ void store_vec(float* p, const float (&a)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(a[0], a[1], a[2], a[3]);
}

struct ConvGeom {
  int64_t units;          // threads with work: blocks * runs * vectors
  int64_t delta_row_stride;
  int32_t hidden, group_size, groups, block_size;
  int32_t run_len, runs_per_block, nvec, taps;
};

// Coefficient of tap t for the VEC channels starting at c0 of token row drow.
template <typename TIO, bool ONE_GROUP, int VEC>
__device__ __forceinline__ void add_delta(const TIO* drow, int t, int groups, int c0, int gs,
                                          const float (&bt)[VEC], float (&coef)[VEC]) {
  if (ONE_GROUP) {
    const float d = Elem<TIO>::load(drow + (int64_t)t * groups + c0 / gs);
#pragma unroll
    for (int e = 0; e < VEC; ++e) coef[e] = bt[e] + d;
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      coef[e] = bt[e] + Elem<TIO>::load(drow + (int64_t)t * groups + (c0 + e) / gs);
  }
}

// TAPS > 0: compile-time tap count with the register tap history.
template <typename TIO, int TAPS, bool ONE_GROUP>
__global__ __launch_bounds__(kThreads) void conv_kernel(const TIO* __restrict__ x,
                                                        const TIO* __restrict__ base,
                                                        const TIO* __restrict__ delta,
                                                        TIO* __restrict__ out, ConvGeom g) {
  constexpr int VEC = Elem<TIO>::kVec;
  const int64_t unit = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (unit >= g.units) return;

  const int v = (int)(unit % g.nvec);
  const int64_t rest = unit / g.nvec;
  const int run = (int)(rest % g.runs_per_block);
  const int64_t blk = rest / g.runs_per_block;
  const int c0 = v * VEC;
  const int H = g.hidden;
  const int j0 = run * g.run_len;
  const int j1 = min(j0 + g.run_len, g.block_size);
  const int64_t row0 = blk * g.block_size;

  float bt[TAPS][VEC];
#pragma unroll
  for (int t = 0; t < TAPS; ++t) load_vec<TIO>(base + (int64_t)t * H + c0, bt[t]);

  float hist[TAPS > 1 ? TAPS - 1 : 1][VEC];   // hist[t-1] = x[i - t]
#pragma unroll
  for (int t = 1; t < TAPS; ++t) {
    const int jj = j0 - t;
    if (jj >= 0) {
      load_vec<TIO>(x + (row0 + jj) * H + c0, hist[t - 1]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) hist[t - 1][e] = 0.f;
    }
  }

  for (int j = j0; j < j1; ++j) {
    const int64_t i = row0 + j;
    float xc[VEC];
    load_vec<TIO>(x + i * H + c0, xc);
    const TIO* drow = delta + i * g.delta_row_stride;
    float coef[VEC], acc[VEC];
    add_delta<TIO, ONE_GROUP, VEC>(drow, 0, g.groups, c0, g.group_size, bt[0], coef);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = coef[e] * xc[e];
#pragma unroll
    for (int t = 1; t < TAPS; ++t) {
      if (j >= t) {   // taps that reach before the block start are zero
        add_delta<TIO, ONE_GROUP, VEC>(drow, t, g.groups, c0, g.group_size, bt[t], coef);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(coef[e], hist[t - 1][e], acc[e]);
      }
    }
    store_vec(out + i * H + c0, acc);
#pragma unroll
    for (int t = TAPS - 2; t >= 1; --t) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) hist[t][e] = hist[t - 1][e];
    }
    if (TAPS > 1) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) hist[0][e] = xc[e];
    }
  }
}

// Any tap count: reloads x[i - t] per tap (cache hits) instead of a register history.
template <typename TIO>
__global__ __launch_bounds__(kThreads) void conv_kernel_any_taps(const TIO* __restrict__ x,
                                                                 const TIO* __restrict__ base,
                                                                 const TIO* __restrict__ delta,
                                                                 TIO* __restrict__ out, ConvGeom g) {
  constexpr int VEC = Elem<TIO>::kVec;
  const int64_t unit = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (unit >= g.units) return;
  const int v = (int)(unit % g.nvec);
  const int64_t rest = unit / g.nvec;
  const int run = (int)(rest % g.runs_per_block);
  const int64_t blk = rest / g.runs_per_block;
  const int c0 = v * VEC;
  const int H = g.hidden;
  const int j0 = run * g.run_len;
  const int j1 = min(j0 + g.run_len, g.block_size);
  const int64_t row0 = blk * g.block_size;
  for (int j = j0; j < j1; ++j) {
    const int64_t i = row0 + j;
    const TIO* drow = delta + i * g.delta_row_stride;
    float acc[VEC];
    for (int t = 0; t < g.taps && t <= j; ++t) {
      float bt[VEC], xv[VEC], coef[VEC];
      load_vec<TIO>(base + (int64_t)t * H + c0, bt);
      load_vec<TIO>(x + (i - t) * H + c0, xv);
      add_delta<TIO, false, VEC>(drow, t, g.groups, c0, g.group_size, bt, coef);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = (t == 0) ? coef[e] * xv[e] : fmaf(coef[e], xv[e], acc[e]);
    }
    store_vec(out + i * H + c0, acc);
  }
}

template <typename TIO, int TAPS>
hipError_t launch_t(const ConvArgs& a, const ConvGeom& g, hipStream_t s) {
  const dim3 grid((unsigned)((g.units + kThreads - 1) / kThreads));
  const bool one_group = (a.group_size % Elem<TIO>::kVec) == 0;
  const TIO* x = static_cast<const TIO*>(a.x);
  const TIO* b = static_cast<const TIO*>(a.base);
  const TIO* d = static_cast<const TIO*>(a.delta);
  TIO* o = static_cast<TIO*>(a.out);
  if (one_group)
    hipLaunchKernelGGL((conv_kernel<TIO, TAPS, true>), grid, dim3(kThreads), 0, s, x, b, d, o, g);
  else
    hipLaunchKernelGGL((conv_kernel<TIO, TAPS, false>), grid, dim3(kThreads), 0, s, x, b, d, o, g);
  return hipGetLastError();
}

template <typename TIO>
hipError_t launch_dtype(const ConvArgs& a, const ConvGeom& g, hipStream_t s) {
  switch (a.taps) {
    case 1: return launch_t<TIO, 1>(a, g, s);
    case 2: return launch_t<TIO, 2>(a, g, s);
    case 3: return launch_t<TIO, 3>(a, g, s);
    case 4: return launch_t<TIO, 4>(a, g, s);
    case 5: return launch_t<TIO, 5>(a, g, s);
    case 6: return launch_t<TIO, 6>(a, g, s);
    case 7: return launch_t<TIO, 7>(a, g, s);
    case 8: return launch_t<TIO, 8>(a, g, s);
    default: {
      const dim3 grid((unsigned)((g.units + kThreads - 1) / kThreads));
      hipLaunchKernelGGL((conv_kernel_any_taps<TIO>), grid, dim3(kThreads), 0, s,
                         static_cast<const TIO*>(a.x), static_cast<const TIO*>(a.base),
                         static_cast<const TIO*>(a.delta), static_cast<TIO*>(a.out), g);
      return hipGetLastError();
    }
  }
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
  const int vec = a.dtype == DFLASH_BF16 ? 8 : 4;
  ConvGeom g;
  g.hidden = a.hidden;
  g.group_size = a.group_size;
  g.groups = a.hidden / a.group_size;
  g.block_size = a.block_size;
  g.taps = a.taps;
  g.delta_row_stride = a.delta_row_stride;
  g.nvec = a.hidden / vec;
  const int64_t nblocks = a.n_tokens / a.block_size;
  // Split blocks into shorter token runs until the launch has enough threads
  // to cover the chip (each run re-reads a T-1 token halo from cache).
  int run = a.block_size;
  const int min_run = a.taps > 2 ? a.taps : 2;
  while (run > min_run &&
         nblocks * ((a.block_size + run - 1) / run) * (int64_t)g.nvec < (int64_t)256 * 1024)
    run = (run + 1) / 2;
  g.run_len = run;
  g.runs_per_block = (a.block_size + run - 1) / run;
  g.units = nblocks * g.runs_per_block * g.nvec;
  if (g.units == 0) return hipSuccess;
  return a.dtype == DFLASH_BF16 ? launch_dtype<uint16_t>(a, g, stream)
                                : launch_dtype<float>(a, g, stream);
}

}  // namespace dflash

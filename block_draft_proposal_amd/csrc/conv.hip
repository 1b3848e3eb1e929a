// Block-causal grouped dynamic depthwise convolution on gfx950.
//
// Operation ("[Spec] DFlash2: local convolution + candidate selector", code
// excerpt of the grouped conv):
//   out[i,c] = sum_{t < T, t <= i mod B} (base[t,c] + delta[i,t,c/gs]) * x[i-t,c]
//
// HBM-bound stream: each input row is read once from HBM, each output row
// written once.  A thread owns one 16-byte channel vector (8 bf16 / 4 fp32
// channels) of a short run of consecutive tokens inside one block.  It loads
// the run's input rows plus a T-1 token halo (cache hits: the neighbouring
// run's thread reads the same rows), the run's dynamic coefficients and the
// static kernel rows in one batch, then computes every token of the run from
// registers.  Lanes of a wave hold consecutive channel vectors of the same
// token, so every load and store of a wave is one contiguous 1 KiB (bf16)
// segment.
#include "conv_core.h"
#include "conv_walk.h"
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
// tokens per thread in the fixed-tap kernels: 4, or 8 once a launch has
// threads to spare (fewer halo rows per output, more loads in flight per
// thread; measured 22% faster on 15360 x 7168, slower on 480 x 4096)
constexpr int kRunSmall = 4, kRunLarge = 8;
constexpr int64_t kRunLargeMinThreads = (int64_t)1 << 20;   // threads the launch would have at kRunSmall

template <typename TIO>
__device__ __forceinline__ void load_vec(const TIO* p, float (&o)[Elem<TIO>::kVec]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  unpack16(v, o);
}

// outputs are written once and not read back by the conv: streaming stores
__device__ __forceinline__ void store_vec(uint16_t* p, const float (&a)[8]) {
  const uint4 v = pack_bf16x8(a);
  st16_nt(p, u32x4{v.x, v.y, v.z, v.w});
}
__device__ __forceinline__ void store_vec(float* p, const float (&a)[4]) {
  st16_nt(p, u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])});
}

__device__ __forceinline__ u32x4 pack_vec(const float (&a)[8]) {
  const uint4 v = pack_bf16x8(a);
  return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x4 pack_vec(const float (&a)[4]) {
  return u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])};
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

// TAPS <= 8: compile-time tap count.  A thread owns RUN consecutive tokens
// of one block (fewer at the block's end) for one channel vector.  Every load
// it needs -- the RUN + TAPS - 1 input rows of its window, the RUN x TAPS
// dynamic coefficients and the TAPS static rows -- is issued before the first
// multiply, with addresses clamped into the block, so a thread waits for one
// memory round trip instead of one per token.  Window rows before the block
// start or after its last token are loaded from a clamped address and never
// used: their taps are masked by the block-causal condition t <= i mod B.
template <typename TIO, int TAPS, bool ONE_GROUP, int RUN>
__global__ __launch_bounds__(kThreads) void conv_kernel(const TIO* __restrict__ x,
                                                        const TIO* __restrict__ base,
                                                        const TIO* __restrict__ delta,
                                                        TIO* __restrict__ out, ConvGeom g) {
  constexpr int VEC = Elem<TIO>::kVec;
  constexpr int W = RUN + TAPS - 1;             // window rows j0-TAPS+1 .. j0+RUN-1
  const int64_t unit = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (unit >= g.units) return;

  const int v = (int)(unit % g.nvec);
  const int64_t rest = unit / g.nvec;
  const int run = (int)(rest % g.runs_per_block);
  const int64_t blk = rest / g.runs_per_block;
  const int c0 = v * VEC;
  const int H = g.hidden;
  const int j0 = run * RUN;
  const int jlast = min(j0 + RUN, g.block_size) - 1;
  const int64_t row0 = blk * g.block_size;

  uint4 xw[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int jj = min(max(j0 - (TAPS - 1) + w, 0), jlast);
    xw[w] = *reinterpret_cast<const uint4*>(x + (row0 + jj) * H + c0);
  }
  uint4 bw[TAPS];
#pragma unroll
  for (int t = 0; t < TAPS; ++t) bw[t] = *reinterpret_cast<const uint4*>(base + (int64_t)t * H + c0);
  // One coefficient per (token, tap) when the vector lies in one group;
  // otherwise the per-channel coefficients are read where they are used.
  float dv[RUN][TAPS];
  if (ONE_GROUP) {
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const TIO* drow = delta + (row0 + min(j0 + u, jlast)) * g.delta_row_stride;
#pragma unroll
      for (int t = 0; t < TAPS; ++t) dv[u][t] = Elem<TIO>::load(drow + (int64_t)t * g.groups + c0 / g.group_size);
    }
  }

#pragma unroll
  for (int u = 0; u < RUN; ++u) {
    const int j = j0 + u;
    if (j > jlast) break;
    float acc[VEC];
    // taps that reach before the block start are zero (not taken)
    conv_token<VEC, TAPS>(
        j,
        [&](int t, float (&coef)[VEC]) {
          float bt[VEC];
          unpack16(bw[t], bt);
          if (ONE_GROUP) coef_one_group<VEC>(bt, dv[u][t], coef);
          else add_delta<TIO, false, VEC>(delta + (row0 + j) * g.delta_row_stride, t, g.groups, c0, g.group_size, bt,
                                          coef);
        },
        [&](int t, float (&xv)[VEC]) { unpack16(xw[u + TAPS - 1 - t], xv); }, acc);
    store_vec(out + (row0 + j) * H + c0, acc);
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

// ---------------------------------------------------------------------------
// Block walk (taps <= 8, blocks of <= 16 tokens, each 16-byte vector inside
// one group, whole groups per wave; conv_walk.h): each wave of a workgroup
// is an independent unit, one block x one chunk of 64 channel vectors.
// ---------------------------------------------------------------------------
constexpr int kWalkWaves = 4;                       // waves (independent units) per workgroup

struct WalkGeom {
  int64_t units;              // waves with work: blocks * slices
  int64_t delta_row_stride;   // elements
  int32_t hidden, groups, block_size, slices;
  int32_t vec_per_group;      // 16-byte vectors per group
};

template <typename TIO, int TAPS>
__global__ __launch_bounds__(kWalkWaves * 64) __attribute__((amdgpu_waves_per_eu(TAPS >= 8 ? 2 : 3, 8))) void conv_walk_kernel(const TIO* __restrict__ x,
                                                                    const TIO* __restrict__ base,
                                                                    const TIO* __restrict__ delta,
                                                                    TIO* __restrict__ out, WalkGeom g) {
  constexpr int VEC = Elem<TIO>::kVec;
  constexpr int E = (int)sizeof(TIO);
  extern __shared__ __align__(16) unsigned char cw_smem[];
  // the wave index as a scalar: the unit's block, slice and row addresses
  // are then computed once per wave in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // the slices of one token block read the same coefficient lines: keep
  // them on one XCD
  const int64_t unit_raw = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * kWalkWaves + wave;
  const bool active = unit_raw < g.units;
  const int64_t unit = active ? unit_raw : g.units - 1;   // a spare wave repeats the last unit, unstored
  const int slice = (int)(unit % g.slices);
  const int64_t blk = unit / g.slices;
  const int H = g.hidden, B = g.block_size;
  const int64_t row0 = blk * B;
  const int v = slice * 64 + lane;                  // this lane's vector (slices are full)
  const int c0 = v * VEC;
  const int gl = lane / g.vec_per_group;            // this lane's group within the slice
  TIO* s_d = reinterpret_cast<TIO*>(cw_smem) + (size_t)wave * (kWalkLdsPerWave / E);
  u32x4 xr[kWalkMaxBlock], br[TAPS];
  walk_load<TIO, TAPS>(x, base, delta, g.delta_row_stride, H, g.groups, B, row0, c0,
                       (int64_t)slice * kPieceGroups<TIO>, s_d, xr, br);
  __syncthreads();
  // outputs leave in one burst after the walk (a write burst per wave rather
  // than stores spread between the reads of other waves: measured faster)
  u32x4 ov[kWalkMaxBlock];
  walk_tokens<TIO, TAPS>(xr, br, s_d, B, gl, [&](int j, float (&acc)[VEC]) { ov[j] = pack_vec(acc); });
#pragma unroll
  for (int j = 0; j < kWalkMaxBlock; ++j)
    if (j < B && active) st16_nt(out + (row0 + j) * H + c0, ov[j]);
}

// The block walk's plan, or units == 0 when it does not apply: <= 8 taps,
// blocks of <= 16 tokens, whole 64-vector slices, each slice's groups one
// 16-byte piece of a coefficient row (64-channel groups), 16-byte aligned
// coefficient pieces.
WalkGeom plan_walk(const ConvArgs& a) {
  WalkGeom w{};
  const int vec = a.dtype == DFLASH_BF16 ? 8 : 4, e = a.dtype == DFLASH_BF16 ? 2 : 4;
  const int nvec = a.hidden / vec;
  const int G = a.hidden / a.group_size;
  if (a.taps > 8 || a.block_size > kWalkMaxBlock || nvec % 64) return w;
  if (64 * vec != (16 / e) * a.group_size) return w;
  if ((a.delta_row_stride * e) % 16 || ((int64_t)G * e) % 16 || (reinterpret_cast<uintptr_t>(a.delta) & 15)) return w;
  w.hidden = a.hidden;
  w.groups = G;
  w.block_size = a.block_size;
  w.slices = nvec / 64;
  w.vec_per_group = a.group_size / vec;
  w.delta_row_stride = a.delta_row_stride;
  w.units = (a.n_tokens / a.block_size) * w.slices;
  return w;
}

template <typename TIO, int TAPS>
hipError_t launch_walk_t(const ConvArgs& a, const WalkGeom& w, hipStream_t s) {
  const dim3 grid((unsigned)((w.units + kWalkWaves - 1) / kWalkWaves));
  hipLaunchKernelGGL((conv_walk_kernel<TIO, TAPS>), grid, dim3(kWalkWaves * 64), kWalkWaves * kWalkLdsPerWave, s,
                     static_cast<const TIO*>(a.x), static_cast<const TIO*>(a.base), static_cast<const TIO*>(a.delta),
                     static_cast<TIO*>(a.out), w);
  return hipGetLastError();
}

template <typename TIO, int TAPS>
hipError_t launch_t(const ConvArgs& a, const ConvGeom& g, hipStream_t s) {
  const WalkGeom w = plan_walk(a);
  if (w.units > 0) return launch_walk_t<TIO, TAPS>(a, w, s);
  const dim3 grid((unsigned)((g.units + kThreads - 1) / kThreads));
  const bool one_group = (a.group_size % Elem<TIO>::kVec) == 0;
  const TIO* x = static_cast<const TIO*>(a.x);
  const TIO* b = static_cast<const TIO*>(a.base);
  const TIO* d = static_cast<const TIO*>(a.delta);
  TIO* o = static_cast<TIO*>(a.out);
  if (g.run_len == kRunLarge) {
    if (one_group)
      hipLaunchKernelGGL((conv_kernel<TIO, TAPS, true, kRunLarge>), grid, dim3(kThreads), 0, s, x, b, d, o, g);
    else
      hipLaunchKernelGGL((conv_kernel<TIO, TAPS, false, kRunLarge>), grid, dim3(kThreads), 0, s, x, b, d, o, g);
  } else {
    if (one_group)
      hipLaunchKernelGGL((conv_kernel<TIO, TAPS, true, kRunSmall>), grid, dim3(kThreads), 0, s, x, b, d, o, g);
    else
      hipLaunchKernelGGL((conv_kernel<TIO, TAPS, false, kRunSmall>), grid, dim3(kThreads), 0, s, x, b, d, o, g);
  }
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
  if (a.taps <= 8) {
    const int64_t small = nblocks * ((a.block_size + kRunSmall - 1) / kRunSmall) * (int64_t)g.nvec;
    g.run_len = small >= kRunLargeMinThreads ? kRunLarge : kRunSmall;
  } else {
    // Any tap count: split blocks into shorter token runs until the launch
    // has enough threads to cover the chip.
    int run = a.block_size;
    while (run > 2 && nblocks * ((a.block_size + run - 1) / run) * (int64_t)g.nvec < (int64_t)256 * 1024)
      run = (run + 1) / 2;
    g.run_len = run;
  }
  g.runs_per_block = (a.block_size + g.run_len - 1) / g.run_len;
  g.units = nblocks * g.runs_per_block * g.nvec;
  if (g.units == 0) return hipSuccess;
  return a.dtype == DFLASH_BF16 ? launch_dtype<uint16_t>(a, g, stream)
                                : launch_dtype<float>(a, g, stream);
}

}  // namespace dflash

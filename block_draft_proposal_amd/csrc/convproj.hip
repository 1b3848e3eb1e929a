// The conv module's kernel projection and its prepare side.
//
// Operation ("[Spec] DFlash2: local convolution + candidate selector", code
// excerpt of the grouped conv module: one bias-free linear map of a token's
// input gives 2 * T * G coefficients, read as [input/output side, tap,
// group]; prepare convolves the input with side 0 of the base kernel plus
// side 0's coefficients and hands side 1's on, and finish convolves the
// sublayer output with side 1):
//   coeff[n, p] = round( sum_k x[n, k] * Wp[p, k] )      p < P = 2 * T * G
//   out = conv(x, base2[0], delta = coeff[:, 0:T*G])       (row stride P)
// rounded once to the storage dtype (the linear map's output dtype).
//
// Design (bf16): the tile product of gemm_tile.h with 128 x 128 tiles over 4
// waves and two 64-deep stages (64 KB of LDS, two workgroups per CU), or
// 64 x 64 tiles when there are too few of those to fill the chip.  The
// projection is skinny (a few hundred to a few thousand outputs), so when the
// tiles alone would leave the chip idle the contraction is split into slices
// of k blocks, one workgroup per (tile, slice), each writing fp32 partial
// sums; a second kernel adds the slices in slice order and rounds once.  With
// one slice the tile kernel rounds and writes the coefficients itself.  fp32
// inputs take a plain kernel (one thread per coefficient, fma in k order).
// The convolution is the existing conv kernel reading side 0 of the
// coefficients through the row stride P; finish is a plain dflash_conv with
// side 1 (base2[1], coeff + T * G, row stride P).
#include "dflash.h"
#include "dflash_internal.h"
#include "gemm_tile.h"

namespace dflash {
namespace {

// Large problems: 128 x 128 tiles over 4 waves of 64 x 64; small ones (too
// few 128 x 128 tiles to fill the chip): 64 x 64 tiles over 4 waves of
// 32 x 32, so fewer slices (less partial traffic) fill it.  Two 64-deep
// stages either way, three for the small tile (48 KB).
using ProjCfg = TileCfg<4, 4, 2, 2, 64, 2>;
using ProjCfgSmall = TileCfg<2, 2, 2, 2, 64, 3>;
constexpr int kProjTargetGroups = 256;   // workgroups the split aims for (one per CU at least)
constexpr int kProjMinBlocks = 8;        // k blocks per slice at least

// One (tile, slice) of the projection.  SPLIT: fp32 partial sums of slice
// blockIdx.y into parts[slice][n][p]; otherwise the whole contraction,
// rounded to bf16 into coeff[n][p].
template <class Cfg, bool SPLIT>
__global__ __launch_bounds__(Cfg::kThreads) void conv_proj_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int32_t N, int32_t H, int32_t P, int32_t n_mb,
    int32_t n_nb, int32_t kb_per_slice, float* __restrict__ parts, uint16_t* __restrict__ coeff) {
  extern __shared__ __align__(16) unsigned char cp_smem[];
  int mb, nb;
  tile_of(blockIdx.x, n_mb, mb, nb);
  if (nb >= n_nb) return;
  const int m0 = mb * Cfg::kBM, n0 = nb * Cfg::kBN;
  const int nk = (H + Cfg::kBK - 1) / Cfg::kBK;
  const int kb0 = (int)blockIdx.y * kb_per_slice;
  const int nkb = min(kb_per_slice, nk - kb0);
  f32x4_t acc[Cfg::kFragM][Cfg::kFragN];
  tile_product<Cfg>(x, H, w, H, N, P, H, m0, n0, kb0, nkb, cp_smem, acc);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = (wave / Cfg::kWavesN) * Cfg::kWM, wn = (wave % Cfg::kWavesN) * Cfg::kWN;
  float* part = parts + (int64_t)blockIdx.y * N * P;
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j) {
      const int col = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm + 16 * i + 4 * (lane >> 4) + v;
        if (row < N && col < P) {
          if (SPLIT) part[(int64_t)row * P + col] = acc[i][j][v];
          else coeff[(int64_t)row * P + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
        }
      }
    }
}

// coeff[e] = bf16(sum of the slices' partials of element e, in slice order).
__global__ void conv_proj_reduce_kernel(const float* __restrict__ parts, int32_t slices, int64_t count,
                                        uint16_t* __restrict__ coeff) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= count) return;
  float s = parts[e];
  for (int k = 1; k < slices; ++k) s += parts[(int64_t)k * count + e];
  coeff[e] = (uint16_t)f32_to_bf16_rne(s);
}

// fp32: one thread per coefficient, products fused into the sum in k order.
__global__ void conv_proj_f32_kernel(const float* __restrict__ x, const float* __restrict__ w, int32_t N,
                                     int32_t H, int32_t P, float* __restrict__ coeff) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)N * P) return;
  const int64_t n = e / P, p = e % P;
  const float* xr = x + n * H;
  const float* wr = w + p * H;
  float s = 0.f;
  for (int k = 0; k < H; ++k) s = fmaf(xr[k], wr[k], s);
  coeff[e] = s;
}

}  // namespace

ConvPrepPlan plan_conv_prepare(int64_t n_tokens, int32_t hidden, int32_t outputs, int32_t dtype) {
  ConvPrepPlan p{};
  if (dtype != DFLASH_BF16 || n_tokens <= 0 || outputs <= 0) return p;
  const int64_t big_tiles = ((n_tokens + ProjCfg::kBM - 1) / ProjCfg::kBM) *
                            ((outputs + ProjCfg::kBN - 1) / ProjCfg::kBN);
  p.small = big_tiles < kProjTargetGroups / 2;
  const int bm = p.small ? ProjCfgSmall::kBM : ProjCfg::kBM, bn = p.small ? ProjCfgSmall::kBN : ProjCfg::kBN;
  p.n_mb = (int32_t)((n_tokens + bm - 1) / bm);
  p.n_nb = (outputs + bn - 1) / bn;
  const int nk = (hidden + ProjCfg::kBK - 1) / ProjCfg::kBK;
  const int64_t tiles = (int64_t)p.n_mb * p.n_nb;
  int slices = (int)((kProjTargetGroups + tiles - 1) / tiles);
  const int max_slices = nk / kProjMinBlocks > 1 ? nk / kProjMinBlocks : 1;
  if (slices > max_slices) slices = max_slices;
  if (slices < 1) slices = 1;
  p.kb_per_slice = (nk + slices - 1) / slices;
  p.slices = (nk + p.kb_per_slice - 1) / p.kb_per_slice;       // no empty slice
  p.bytes = p.slices > 1 ? ((size_t)p.slices * n_tokens * outputs * sizeof(float) + 255) & ~(size_t)255 : 0;
  return p;
}

hipError_t launch_conv_prepare(const ConvPrepArgs& a, const ConvPrepPlan& p, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  const int32_t G = a.hidden / a.group_size;
  const int32_t P = 2 * a.taps * G;
  if (a.dtype == DFLASH_BF16) {
    const int64_t slots = (int64_t)((p.n_nb + 7) / 8) * p.n_mb;
    const dim3 grid((unsigned)(slots * 8), (unsigned)p.slices);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* w = static_cast<const uint16_t*>(a.proj_weight);
    uint16_t* coeff = static_cast<uint16_t*>(a.coeff_out);
    float* parts = static_cast<float*>(a.workspace);
    const bool split = p.slices > 1;
#define DFLASH_PROJ_TILE(CFG, SPLIT)                                                                        \
  hipLaunchKernelGGL((conv_proj_kernel<CFG, SPLIT>), grid, dim3(CFG::kThreads), CFG::kSmemBytes, stream, x, w, \
                     (int32_t)a.n_tokens, a.hidden, P, p.n_mb, p.n_nb, p.kb_per_slice, parts, coeff)
    if (p.small) {
      if (split) DFLASH_PROJ_TILE(ProjCfgSmall, true);
      else DFLASH_PROJ_TILE(ProjCfgSmall, false);
    } else {
      if (split) DFLASH_PROJ_TILE(ProjCfg, true);
      else DFLASH_PROJ_TILE(ProjCfg, false);
    }
#undef DFLASH_PROJ_TILE
    if (split) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t count = a.n_tokens * P;
      hipLaunchKernelGGL(conv_proj_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                         parts, p.slices, count, coeff);
    }
  } else {
    const int64_t count = a.n_tokens * P;
    hipLaunchKernelGGL(conv_proj_f32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(a.x), static_cast<const float*>(a.proj_weight),
                       (int32_t)a.n_tokens, a.hidden, P, static_cast<float*>(a.coeff_out));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // side 0: base2[0] and the first T * G coefficients of each row
  ConvArgs c{a.x, a.base2, a.coeff_out, P, a.out, a.n_tokens, a.hidden, a.group_size, a.taps, a.block_size,
             a.dtype};
  return launch_conv(c, stream);
}

}  // namespace dflash

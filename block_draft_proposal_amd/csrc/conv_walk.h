// The block walk of the block-causal grouped dynamic depthwise convolution
// ("[Spec] DFlash2: local convolution + candidate selector", code excerpt of
// the grouped conv): the loads and the per-token arithmetic of one wave's
// unit, kept apart from the kernel that schedules the units.
//
// Shape (taps <= 8, blocks of <= 16 tokens, each 16-byte vector inside one
// group, whole groups per chunk): a wave owns one block and a chunk of 64
// channel vectors (512 bf16 / 256 fp32 channels).  Lane l walks the block's
// tokens in order for its vector: every input row of the block is loaded once
// (no halo re-reads), the static rows once per block, and the last TAPS
// inputs stay in fp32 registers as the tap history.  The block's dynamic
// coefficients for the chunk's groups -- [token][tap][group] in memory -- are
// loaded as 16-byte pieces by the whole wave and transposed through the
// wave's LDS to [token][group][tap], so that each token's TAPS coefficients
// of a lane's group are one 16-byte (bf16) or two (fp32) LDS reads.
// Arithmetic: conv_core.h (shared with every conv producer).
#pragma once

#include "conv_core.h"

namespace dflash {

constexpr int kWalkMaxBlock = 16;
// Groups per chunk: one 16-byte piece of coefficients per (token, tap)
// (8 bf16 / 4 fp32 groups, i.e. 64-channel groups).
template <typename TIO> constexpr int kPieceGroups = 16 / (int)sizeof(TIO);
constexpr int kWalkMaxPieces = kWalkMaxBlock * 8 / 64;   // pieces per lane: tokens x taps / 64
// LDS per wave: [token][group][8 tap slots]
constexpr int kWalkLdsPerWave = kWalkMaxBlock * 16 * 8;   // bytes (bf16: 8 groups x 2 B; fp32: 4 x 4 B)

// Every load of the walk first: the block's input rows at the lane's channel
// vector c0 (xr), the static rows (br), and the chunk's coefficients (groups
// g0 .. g0 + kPieceGroups - 1 of every token and tap) transposed into s_d.
// The caller makes the LDS writes visible to the wave before walk_tokens.
template <typename TIO, int TAPS>
__device__ __forceinline__ void walk_load(const TIO* __restrict__ x, const TIO* __restrict__ base,
                                          const TIO* __restrict__ delta, int64_t delta_row_stride, int H,
                                          int groups, int B, int64_t row0, int c0, int64_t g0, TIO* s_d,
                                          u32x4 (&xr)[kWalkMaxBlock], u32x4 (&br)[TAPS]) {
  constexpr int E = (int)sizeof(TIO);
  constexpr int PV = 16 / E;                        // elements per 16-byte piece
  constexpr int TS = 8;                             // tap slots per (token, group) in LDS
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kWalkMaxBlock; ++j)
    if (j < B) xr[j] = ld16_nt(x + (row0 + j) * H + c0);   // each input row is read once
#pragma unroll
  for (int t = 0; t < TAPS; ++t) br[t] = ld16(base + (int64_t)t * H + c0);
  // one 16-byte piece per (token j, tap t), piece i = j * TAPS + t
  const int n_pieces = B * TAPS;
  u32x4 dr[kWalkMaxPieces];
#pragma unroll
  for (int p = 0; p < kWalkMaxPieces; ++p) {
    const int i = min(p * 64 + lane, n_pieces - 1);
    const int t = i % TAPS, j = i / TAPS;
    if (p * 64 < n_pieces) dr[p] = ld16(delta + (row0 + j) * delta_row_stride + (int64_t)t * groups + g0);
  }
  // transpose to [token][group][tap slot] (slots past TAPS are never read)
#pragma unroll
  for (int p = 0; p < kWalkMaxPieces; ++p) {
    const int i = p * 64 + lane;
    if (i < n_pieces) {
      const int t = i % TAPS, j = i / TAPS;
      TIO* dst = s_d + (size_t)j * kPieceGroups<TIO> * TS + t;
#pragma unroll
      for (int k = 0; k < PV; ++k) {
        if constexpr (E == 2) *reinterpret_cast<uint16_t*>(dst + k * TS) = (uint16_t)(dr[p][k >> 1] >> (16 * (k & 1)));
        else *reinterpret_cast<uint32_t*>(dst + k * TS) = dr[p][k];
      }
    }
  }
}

// The walk over tokens 0 .. B-1 of the block: emit(j, acc) receives token j's
// fp32 outputs for the lane's vector (gl: the lane's group within the chunk).
template <typename TIO, int TAPS, class Emit>
__device__ __forceinline__ void walk_tokens(const u32x4 (&xr)[kWalkMaxBlock], const u32x4 (&br)[TAPS],
                                            const TIO* s_d, int B, int gl, Emit&& emit) {
  constexpr int VEC = Elem<TIO>::kVec;
  constexpr int E = (int)sizeof(TIO);
  constexpr int TS = 8;
  float bt[TAPS][VEC];
#pragma unroll
  for (int t = 0; t < TAPS; ++t) unpack16(br[t], bt[t]);
  float hist[TAPS][VEC];                            // hist[t] = input row j - t
#pragma unroll
  for (int j = 0; j < kWalkMaxBlock; ++j) {
    // a constant trip count (guarded) keeps the loop unrolled, so xr and
    // hist stay in registers
    if (j < B) {
      // a compiler-only barrier: each token's LDS reads stay in its own
      // iteration (hoisting all of them ahead of the loop spills registers)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = TAPS - 1; t > 0; --t)
#pragma unroll
        for (int e = 0; e < VEC; ++e) hist[t][e] = hist[t - 1][e];
      unpack16(xr[j], hist[0]);
      // this token's coefficients of the lane's group, tap slots 0..TS-1
      const TIO* dj = s_d + ((size_t)j * kPieceGroups<TIO> + gl) * TS;
      float d[TS];
      if constexpr (E == 2) {
        unpack16(ld16(dj), d);
      } else {
        float lo[4], hi[4];
        unpack16(ld16(dj), lo);
        unpack16(ld16(dj + 4), hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) { d[k] = lo[k]; d[4 + k] = hi[k]; }
      }
      float acc[VEC];
      conv_token<VEC, TAPS>(
          j, [&](int t, float (&coef)[VEC]) { coef_one_group<VEC>(bt[t], d[t], coef); },
          [&](int t, float (&xv)[VEC]) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) xv[e] = hist[t][e];
          },
          acc);
      emit(j, acc);
    }
  }
}

}  // namespace dflash

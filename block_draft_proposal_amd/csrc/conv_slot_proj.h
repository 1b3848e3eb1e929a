// The propose step's convolution and the projection of its slot rows, as
// workgroups of the launch they share with the top-K (so that the step needs
// no second stream).
//
// Operation ("[Spec] DFlash2: local convolution + candidate selector": the
// conv output of the draft block feeds the selector's low-rank projection
// u = P h of each slot's hidden row, slot s being block position 1 + s):
//   conv_out = conv(x, base, delta)                     (every row)
//   u_parts[slice][slot row][k] = the projection's partial sum over one slice
//                                  of the channels     (slot rows only)
// with the slices of plan_proj, so that the result equals the chain
// conv -> projection bit for bit.
//
// Design (bf16, blocks of at most 16 tokens, at most 8 taps, one group per
// 16-byte channel vector, few rows): a wave owns one block -- its tokens are
// the first rows of a 16-row MFMA A tile, the rows past the block zeros --
// and one slice of the channels.  Per k-step each
// lane computes the conv output vector of its A-operand slot (token
// lane & 15, channels kc .. kc + 7 with kc = k + 8 (lane >> 4)) with the conv
// kernel's arithmetic (conv_core.h), stores it to conv_out, and feeds it to
// the MFMAs against P.  The input rows of earlier tokens come from the
// neighbouring lanes of the same 16-lane row (DPP row shifts; a lane below
// the shift does not use that tap), so a lane loads one input vector per
// k-step.  Token 0 of a block is no slot and enters the MFMA as zeros.  The
// per-slice MFMA chains are those of the projection kernel: each output is
// the chain over its slice's k-steps in order, whatever rows share the tile,
// and operands past the slice or the rank are zeroed after clamped loads.
#pragma once

#include "conv_core.h"
#include "dflash_internal.h"
#include "gemm_tile.h"

namespace dflash {

constexpr int kSpBlock = 16;      // most tokens per block = rows of an MFMA tile
// k-steps whose loads are issued together (U): a launch-time choice.  Every
// wave of a launch gets the register count of its largest part, and these
// workgroups share the top-K's launch.  Their k-steps are chains of dependent
// loads that wait in the queue the top-K's stream keeps full, so two in
// flight shorten the launch (32 requests at 4 taps x 4 column tiles: 38.5 ->
// 37.1 us) where the launch then still has a slot for every workgroup at
// three waves per SIMD (<= 168 VGPRs: 4 column tiles and up to 7 taps); when
// it has more workgroups than that, one in flight keeps four waves per SIMD
// and every workgroup resident (64 requests of 10 tokens: 60.0 -> 55.7 us
// per step).  Three in flight: 45 us; four, at 224 VGPRs: 12 us slower.
template <int TAPS, int RT> constexpr bool sp_two_in_flight_fits() { return RT == 4 && TAPS <= 7; }
constexpr int64_t kSpThreeWaveSlots = 256 * 3;    // resident workgroups of 4 waves at three waves per SIMD

// The 16-byte vector of lane (lane - t) of the same 16-lane row (row shift by
// t; t is a compile-time constant after unrolling).
template <int T>
__device__ __forceinline__ u32x4 row_shr(const u32x4& v) {
  if constexpr (T == 0) {
    return v;
  } else {
    u32x4 r;
    r.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, 0x110 + T, 0xf, 0xf, false);
    r.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, 0x110 + T, 0xf, 0xf, false);
    r.z = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, 0x110 + T, 0xf, 0xf, false);
    r.w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, 0x110 + T, 0xf, 0xf, false);
    return r;
  }
}

template <int TAPS>
__device__ __forceinline__ void shifted_inputs(const u32x4& own, u32x4 (&xs)[TAPS]) {
  xs[0] = own;
  if constexpr (TAPS > 1) xs[1] = row_shr<1>(own);
  if constexpr (TAPS > 2) xs[2] = row_shr<2>(own);
  if constexpr (TAPS > 3) xs[3] = row_shr<3>(own);
  if constexpr (TAPS > 4) xs[4] = row_shr<4>(own);
  if constexpr (TAPS > 5) xs[5] = row_shr<5>(own);
  if constexpr (TAPS > 6) xs[6] = row_shr<6>(own);
  if constexpr (TAPS > 7) xs[7] = row_shr<7>(own);
}

// Arguments of the conv + slot projection part of a launch.
struct SlotProjArgs {
  const uint16_t* x;
  const uint16_t* base;
  const uint16_t* delta;
  int64_t delta_row_stride;
  uint16_t* conv_out;
  int32_t n_blocks, block_size, H, group_size;
  const uint16_t* P;
  int32_t rank, slots, kslice, ksplit;
  float* u_parts;
  int32_t groups_x;   // workgroups per slice: ceil(n_blocks / 4)
};

// One workgroup (4 waves) of the conv + slot projection: blocks 4 gx ..
// 4 gx + 3, one per wave, channel slice `split`.
template <int TAPS, int RT, int U>
__device__ __forceinline__ void conv_slot_proj_group(int gx, int split, const SlotProjArgs& sp) {
  static_assert(TAPS >= 1 && TAPS <= 8, "taps");
  const uint16_t* __restrict__ x = sp.x;
  const uint16_t* __restrict__ base = sp.base;
  const uint16_t* __restrict__ delta = sp.delta;
  const int64_t delta_row_stride = sp.delta_row_stride;
  uint16_t* __restrict__ conv_out = sp.conv_out;
  const int32_t n_blocks = sp.n_blocks, B = sp.block_size, H = sp.H, group_size = sp.group_size;
  const uint16_t* __restrict__ P = sp.P;
  const int32_t rank = sp.rank, slots = sp.slots, kslice = sp.kslice;
  float* __restrict__ u_parts = sp.u_parts;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int blk = gx * 4 + wave;
  const bool blk_ok = blk < n_blocks;
  const int64_t row0 = (int64_t)(blk_ok ? blk : n_blocks - 1) * B;   // clamped for addressing
  const int pos = lane & 15;                        // token of this lane's A slot
  const bool tok_ok = blk_ok && pos < B;            // a token of the block (rows past it: zeros)
  const bool slot_ok = tok_ok && pos >= 1 && pos <= slots;
  const int k0 = split * kslice;
  const int k1 = min(H, k0 + kslice);
  const int kofs = 8 * (lane >> 4);
  const int G = H / group_size;
  // a lane past the block reads its block's last row (its results are never
  // used: a token's taps come from lanes pos - t of the same block)
  const int tok = pos < B ? pos : B - 1;
  const uint16_t* xrow = x + (row0 + tok) * H;
  const uint16_t* drow = delta + (row0 + tok) * delta_row_stride;
  uint16_t* orow = conv_out + (row0 + tok) * H;

  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int kk = k0; kk < k1; kk += 32 * U) {
    // every load of the round first: own input vector, static rows, the
    // group's dynamic scalars, P fragments (addresses clamped into the slice)
    u32x4 xv[U], bw[U][TAPS], pv[U][RT];
    float dv[U][TAPS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = min(kk + 32 * u + kofs, k1 - 8);
      xv[u] = ld16(xrow + kc);
#pragma unroll
      for (int t = 0; t < TAPS; ++t) bw[u][t] = ld16(base + (int64_t)t * H + kc);
#pragma unroll
      for (int t = 0; t < TAPS; ++t) dv[u][t] = Elem<uint16_t>::load(drow + (int64_t)t * G + kc / group_size);
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
        const int col = min(tt * 16 + (lane & 15), rank - 1);
        pv[u][tt] = ld16(P + (int64_t)col * H + kc);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = min(kk + 32 * u + kofs, k1 - 8);
      const bool k_ok = kk + 32 * u + kofs < k1;
      u32x4 xs[TAPS];
      shifted_inputs<TAPS>(xv[u], xs);
      float cv[8];
      conv_token<8, TAPS>(
          pos,
          [&](int t, float (&coef)[8]) {
            float bt[8];
            unpack16(bw[u][t], bt);
            coef_one_group<8>(bt, dv[u][t], coef);
          },
          [&](int t, float (&xf)[8]) { unpack16(xs[t], xf); }, cv);
      const uint4 packed = pack_bf16x8(cv);
      if (tok_ok && k_ok) *reinterpret_cast<uint4*>(orow + kc) = packed;
      const u32x4 pk = {packed.x, packed.y, packed.z, packed.w};
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (slot_ok && k_ok) ? pk : zero);
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
        const bool c_ok = tt * 16 + (lane & 15) < rank;
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, (c_ok && k_ok) ? pv[u][tt] : zero);
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[tt], 0, 0, 0);
      }
    }
  }
  // D layout: lane holds column (lane & 15) of each tile, tile rows (block
  // positions) 4 * (lane >> 4) + v.
  if (!blk_ok) return;
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) {
    const int col = tt * 16 + (lane & 15);
    if (col >= rank) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 4 * (lane >> 4) + v;
      if (p >= 1 && p <= slots) {
        const int64_t srow = (int64_t)blk * slots + (p - 1);
        u_parts[proj_part_index(split, (int64_t)n_blocks * slots, rank, srow, col)] = acc[tt][v];
      }
    }
  }
}

}  // namespace dflash

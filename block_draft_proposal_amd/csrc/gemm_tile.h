// Tiled bf16 x bf16 -> fp32 contraction on the matrix cores of gfx950, shared
// by the dense head and the conv's kernel projection:
//   C[m, n] = sum_k A[m, k] * B[n, k]
// A [M, K] and B [N, K], both with the contraction axis contiguous (A with a
// row stride, B with a row stride too).
//
// A workgroup computes one (16 FM WM) x (16 FN WN) tile of C over a range of
// 64- (or 32-) wide k blocks.  Each of its WM x WN waves holds a (16 FM) x
// (16 FN) block as FM x FN accumulators of v_mfma_f32_16x16x32_bf16; bf16 x
// bf16 products are exact in fp32.  Operands reach LDS by 16-byte direct
// global -> LDS loads, so no register staging is needed and the LDS rows are
// unpadded: each lane picks the global chunk that the XOR swizzle puts in its
// slot, and the 16 rows one MFMA fragment reads fall on distinct banks.  A
// ring of STAGES stages; each thread waits only for its own direct loads
// (vector-memory counter) before a bare barrier, so the stages already in
// flight keep flowing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace dflash {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

template <int FM, int FN, int WM, int WN, int BK, int STAGES>
struct TileCfg {
  static constexpr int kFragM = FM, kFragN = FN;            // MFMA fragments per wave
  static constexpr int kWavesM = WM, kWavesN = WN;          // waves along rows and columns
  static constexpr int kWM = 16 * FM, kWN = 16 * FN;        // a wave's block
  static constexpr int kBM = kWM * WM, kBN = kWN * WN;      // the tile
  static constexpr int kBK = BK;                            // contraction depth of one stage
  static constexpr int kStages = STAGES;                    // loads run STAGES - 1 stages ahead
  static constexpr int kChunks = BK / 8;                    // 16-byte chunks per stage row
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kBlockRows = 1024 / kRowBytes;       // rows per 1 KB block of direct loads
  static constexpr int kSwzShift = BK == 64 ? 1 : 2;        // log2 of the rows sharing a 256-byte bank window
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kStageBytes = (kBM + kBN) * kRowBytes;
  static constexpr int kBOff = kBM * kRowBytes;             // the B tile within a stage
  static constexpr int kLoadsPerStage = (kBM + kBN) / kBlockRows / kWaves;   // per thread
  static constexpr size_t kSmemBytes = (size_t)STAGES * kStageBytes;
  // the rounded output tile goes through LDS in passes of kOutCols columns
  static constexpr int kOutCols = kBN < 128 ? kBN : 128;
  static constexpr int kOutPasses = kBN / kOutCols;
  static constexpr int kCPad = kOutCols + 8;                // bf16 elements per LDS row of one pass
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(kBM % (kBlockRows * kWaves) == 0 && kBN % (kBlockRows * kWaves) == 0,
                "stage rows split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 5, "wait counts cover up to three stages ahead");
  static_assert(kOutCols % kWN == 0 && kBN % kOutCols == 0, "a wave's columns lie in one output pass");
  static_assert(sizeof(uint16_t) * kBM * kCPad <= kSmemBytes, "an output pass fits in the ring");
  // chunk c of stage row r sits in slot c ^ swz(r)
  __device__ static __forceinline__ int swz(int row) { return (row >> kSwzShift) & (kChunks - 1); }
};

// Workgroup -> (row block, column block).  Consecutive workgroups go to
// consecutive XCDs; the n_mb row blocks of one column block get ids that are
// equal modulo 8, so they share an XCD (and its L2).
__device__ __forceinline__ void tile_of(int id, int n_mb, int& mb, int& nb) {
  const int xcd = id & 7, slot = id >> 3;
  nb = (slot / n_mb) * 8 + xcd;
  mb = slot % n_mb;
}

// Row addresses of a [rows, H] operand whose rows sit at a fixed stride.
struct StridedRows {
  const uint16_t* base;
  int64_t stride;
  __device__ __forceinline__ const uint16_t* operator()(int r) const { return base + (int64_t)r * stride; }
};

// Issues the direct global -> LDS loads of one stage: rows [r0, r0 + ROWS)
// x k [k0, k0 + BK) of a [rows, H] matrix (row r at row_at(r)), in 1 KB
// blocks of kBlockRows rows dealt round the waves; lane l of a block fills
// slot l % kChunks of row l / kChunks with the chunk the swizzle puts there.
// Addresses are clamped into the matrix: rows past the end repeat the last
// row (their results are never used) and k past H is zeroed by zero_tail
// before use.
template <class Cfg, int ROWS, class RowAt>
__device__ __forceinline__ void issue_stage(const RowAt& row_at, int rows, int H, int r0, int k0,
                                            unsigned char* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < ROWS / Cfg::kBlockRows / Cfg::kWaves; ++q) {
    const int blk = q * Cfg::kWaves + wave, r = blk * Cfg::kBlockRows + lane / Cfg::kChunks;
    const int k = k0 + 8 * ((lane % Cfg::kChunks) ^ Cfg::swz(r));
    const uint16_t* src = row_at(min(r0 + r, rows - 1)) + min(k, H - 8);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + blk * 1024), 16, 0, 0);
  }
}
template <class Cfg, int ROWS>
__device__ __forceinline__ void issue_stage(const uint16_t* __restrict__ base, int64_t stride, int rows, int H,
                                            int r0, int k0, unsigned char* dst) {
  issue_stage<Cfg, ROWS>(StridedRows{base, stride}, rows, H, r0, k0, dst);
}

// After the stage has landed: zeroes this thread's chunks of it whose k is at
// or past H (only the last k block of a contraction that is not a multiple of
// BK has any).
template <class Cfg, int ROWS>
__device__ __forceinline__ void zero_tail(int H, int k0, unsigned char* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < ROWS / Cfg::kBlockRows / Cfg::kWaves; ++q) {
    const int blk = q * Cfg::kWaves + wave, r = blk * Cfg::kBlockRows + lane / Cfg::kChunks;
    if (k0 + 8 * ((lane % Cfg::kChunks) ^ Cfg::swz(r)) >= H) st16(dst + blk * 1024 + lane * 16, zero);
  }
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the stage ring.  __syncthreads() would also fence,
// which waits for every outstanding direct load, prefetched stages included;
// here each thread has already waited for its own loads of the stage about to
// be read (wait_vm) and for its own LDS accesses (lgkmcnt 0), and the empty
// asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));   // lgkmcnt(0) only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The kBM x kBN fp32 tile at (m0, n0) summed over k blocks [kb0, kb0 + nkb)
// of the H-long contraction (nk = ceil(H / BK) blocks in all), A's and B's
// rows addressed by row functors (row r -> pointer to its first element;
// StridedRows for a plain row stride); each wave
// holds its kWM x kWN block in kFragM x kFragN accumulators.  D layout of one
// 16 x 16 MFMA: lane l holds column l % 16 and rows 4 (l / 16) + v, v = 0..3.
// Stage t lives in ring slot t % kStages; each iteration waits for its own
// stage, passes one barrier (after which the slot computed last iteration is
// free) and refills that slot with stage t + kStages - 1 before computing.
// The k blocks are summed in increasing order.  Ends with a barrier, so the
// LDS may be reused.
template <class Cfg, class RowA, class RowB>
__device__ __forceinline__ void tile_product(const RowA& A, const RowB& B, int M, int N, int H, int m0, int n0,
                                             int kb0, int nkb, unsigned char* smem,
                                             f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  constexpr int S = Cfg::kStages;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave / Cfg::kWavesN) * Cfg::kWM, wn = (wave % Cfg::kWavesN) * Cfg::kWN;
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = (H + Cfg::kBK - 1) / Cfg::kBK;
  const bool ragged = (H % Cfg::kBK) != 0;
  auto stage = [&](int t) { return smem + (t % S) * Cfg::kStageBytes; };
#pragma unroll
  for (int t = 0; t < S - 1; ++t) {
    if (t < nkb) {
      issue_stage<Cfg, Cfg::kBM>(A, M, H, m0, (kb0 + t) * Cfg::kBK, stage(t));
      issue_stage<Cfg, Cfg::kBN>(B, N, H, n0, (kb0 + t) * Cfg::kBK, stage(t) + Cfg::kBOff);
    }
  }
  // fragment reads: row (lane & 15) of a 16-row group, chunk (lane >> 4) of a
  // 32-wide k slice (16-row groups start at multiples of 16, so the swizzle
  // of the row is that of lane & 15)
  const int frow = lane & 15, fsw = Cfg::swz(frow);
  for (int kt = 0; kt < nkb; ++kt) {
    unsigned char* cur = stage(kt);
    // this thread's loads of stage kt are done once at most the loads of
    // the later stages already issued are outstanding
    const int ahead = min(S - 2, nkb - 1 - kt);
    if (ahead >= 3) wait_vm<3 * Cfg::kLoadsPerStage>();
    else if (ahead == 2) wait_vm<2 * Cfg::kLoadsPerStage>();
    else if (ahead == 1) wait_vm<Cfg::kLoadsPerStage>();
    else wait_vm<0>();
    if (ragged && kb0 + kt == nk - 1) {
      zero_tail<Cfg, Cfg::kBM>(H, (kb0 + kt) * Cfg::kBK, cur);
      zero_tail<Cfg, Cfg::kBN>(H, (kb0 + kt) * Cfg::kBK, cur + Cfg::kBOff);
    }
    ring_barrier();
    if (kt + S - 1 < nkb) {
      unsigned char* nxt = stage(kt + S - 1);
      issue_stage<Cfg, Cfg::kBM>(A, M, H, m0, (kb0 + kt + S - 1) * Cfg::kBK, nxt);
      issue_stage<Cfg, Cfg::kBN>(B, N, H, n0, (kb0 + kt + S - 1) * Cfg::kBK, nxt + Cfg::kBOff);
    }
    const unsigned char* sa = cur;
    const unsigned char* sb = cur + Cfg::kBOff;
#pragma unroll
    for (int ks = 0; ks < Cfg::kChunks; ks += 4) {       // 32-wide k slices: chunks ks .. ks + 3
      const int slot = ((ks + (lane >> 4)) ^ fsw) * 16;
      bf16x8_t af[Cfg::kFragM], bfrag[Cfg::kFragN];
#pragma unroll
      for (int i = 0; i < Cfg::kFragM; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, ld16(sa + (wm + 16 * i + frow) * Cfg::kRowBytes + slot));
#pragma unroll
      for (int j = 0; j < Cfg::kFragN; ++j)
        bfrag[j] = __builtin_bit_cast(bf16x8_t, ld16(sb + (wn + 16 * j + frow) * Cfg::kRowBytes + slot));
#pragma unroll
      for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfrag[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();
}
template <class Cfg>
__device__ __forceinline__ void tile_product(const uint16_t* __restrict__ A, int64_t a_stride,
                                             const uint16_t* __restrict__ B, int64_t b_stride, int M, int N, int H,
                                             int m0, int n0, int kb0, int nkb, unsigned char* smem,
                                             f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  tile_product<Cfg>(StridedRows{A, a_stride}, StridedRows{B, b_stride}, M, N, H, m0, n0, kb0, nkb, smem, acc);
}

// The wave's accumulators rounded to bf16 (nearest, ties to even), two per
// register: pk[i][j][0] holds rows 4 (l / 16) + 0, 1 and pk[i][j][1] rows
// + 2, 3 of fragment (i, j), low half first.  Rounding once here frees the
// fp32 accumulators before an epilogue.
template <class Cfg>
__device__ __forceinline__ void pack_tile(const f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN],
                                          uint32_t (&pk)[Cfg::kFragM][Cfg::kFragN][2]) {
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pk[i][j][h] = f32_to_bf16_rne(acc[i][j][2 * h]) | (f32_to_bf16_rne(acc[i][j][2 * h + 1]) << 16);
}

// Writes into LDS ([kBM][kCPad] bf16) the rounded values of the waves whose
// columns lie in output pass `pass` (tile columns [pass kOutCols, (pass + 1)
// kOutCols)).
template <class Cfg>
__device__ __forceinline__ void tile_to_lds(const uint32_t (&pk)[Cfg::kFragM][Cfg::kFragN][2], uint16_t* cs,
                                            int pass) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave / Cfg::kWavesN) * Cfg::kWM, wn = (wave % Cfg::kWavesN) * Cfg::kWN - pass * Cfg::kOutCols;
  if (wn < 0 || wn >= Cfg::kOutCols) return;
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        cs[(wm + 16 * i + 4 * (lane >> 4) + v) * Cfg::kCPad + wn + 16 * j + (lane & 15)] =
            (uint16_t)((v & 1) ? (pk[i][j][v >> 1] >> 16) : (pk[i][j][v >> 1] & 0xffffu));
}

}  // namespace dflash

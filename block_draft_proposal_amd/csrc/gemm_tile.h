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
//
// With two 64-deep stages and large wave blocks the product is
// software-pipelined by 32-wide k slices: the fragments of the next slice are
// read from LDS into a second register set while the current slice's MFMAs
// run, so no MFMA waits on an LDS read, and one barrier per stage both
// publishes the next stage and frees the one just read for the direct loads
// of the stage after.  Strided operands are then loaded through buffer
// resources (one 32-bit offset per lane, zeros past the matrix).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Workgroup -> (row block, column block) for many row blocks.  XCD x (the
// workgroups with id % 8 == x) owns the column blocks nb % 8 == x and walks
// them in groups of GM row blocks: for each column block the group's row
// blocks, then the next column block.  The ~32 workgroups an XCD runs at once
// then cover about 32 / GM column blocks x GM row blocks, each operand tile
// fetched into its L2 once for several workgroups (with one row block per
// column block in flight, every workgroup fetched its own A rows).  Covers
// ids [0, 8 n_mb ceil(n_nb / 8)); nb >= n_nb marks an idle workgroup.
template <int GM>
__device__ __forceinline__ void tile_of_grouped(int id, int n_mb, int n_nb, int& mb, int& nb) {
  const int xcd = id & 7, slot = id >> 3;
  const int ncb = (n_nb + 7) >> 3;               // column blocks of this XCD
  const int g = slot / (GM * ncb), rem = slot - g * GM * ncb;
  const int gsz = min(GM, n_mb - g * GM);        // the last group may be smaller
  mb = g * GM + rem % gsz;
  nb = (rem / gsz) * 8 + xcd;
}
__host__ __device__ constexpr int64_t grouped_grid(int n_mb, int n_nb) {
  return (int64_t)8 * n_mb * ((n_nb + 7) / 8);
}

// Row addresses of a [rows, H] operand whose rows sit at a fixed stride.
struct StridedRows {
  const uint16_t* base;
  int64_t stride;
  __device__ __forceinline__ const uint16_t* operator()(int r) const { return base + (int64_t)r * stride; }
};

// Cache policy of an operand's direct loads: a row functor may declare
// kAux (kBufferStream for rows read once); 0 (default caching) otherwise.
template <class R, class = void> struct RowAux { static constexpr int value = 0; };
template <class R> struct RowAux<R, std::void_t<decltype(R::kAux)>> { static constexpr int value = R::kAux; };

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
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + blk * 1024), 16, 0, RowAux<RowAt>::value);
  }
}
template <class Cfg, int ROWS>
__device__ __forceinline__ void issue_stage(const uint16_t* __restrict__ base, int64_t stride, int rows, int H,
                                            int r0, int k0, unsigned char* dst) {
  issue_stage<Cfg, ROWS>(StridedRows{base, stride}, rows, H, r0, k0, dst);
}

// Direct-load sources of one tile's operand rows [r0, r0 + ROWS), each with
// issue(k0, dst): the stage at contraction offset k0 into LDS at dst, in the
// layout of issue_stage.
//
// BufRows, for rows at a fixed stride: a buffer resource based at row r0
// whose record count ends at the matrix's last element, so the hardware
// returns zeros for rows past the end (no clamping) and every address is one
// 32-bit offset: the lane's chunk in its first load plus uniform steps (the
// swizzle repeats every kWaves x kBlockRows rows, so a thread's later loads
// of a stage differ from its first by whole row blocks).  Row strides and
// contraction lengths stay below 2^22 elements, which keeps every offset of
// a 256-row tile within 32 bits.
template <class Cfg, int ROWS>
struct BufRows {
  static constexpr int kLoads = ROWS / Cfg::kBlockRows / Cfg::kWaves;
  static_assert(((Cfg::kWaves * Cfg::kBlockRows) >> Cfg::kSwzShift) % Cfg::kChunks == 0,
                "the swizzle repeats every row step of a thread's loads");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;                              // bytes, first load, k = 0
  uint32_t q_step;                                // bytes between a thread's loads
  __device__ __forceinline__ BufRows(const StridedRows& m, int rows, int H, int r0) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int valid = min(rows - r0, ROWS);      // >= 1: the tile starts inside the matrix
    const uint32_t bytes = (uint32_t)(((uint32_t)(valid - 1) * (uint32_t)m.stride + (uint32_t)H) * 2u);
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(m.base + (int64_t)r0 * m.stride), (short)0, (int)bytes,
                                             kBufferFlags);
    const int r = wave * Cfg::kBlockRows + lane / Cfg::kChunks;
    lane_off = ((uint32_t)r * (uint32_t)m.stride + 8u * (uint32_t)((lane % Cfg::kChunks) ^ Cfg::swz(r))) * 2u;
    q_step = (uint32_t)(Cfg::kWaves * Cfg::kBlockRows) * (uint32_t)m.stride * 2u;
  }
  __device__ __forceinline__ void issue(int k0, unsigned char* dst) const {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + (q * Cfg::kWaves + wave) * 1024), 16,
                                               lane_off + (uint32_t)k0 * 2u + (uint32_t)q * q_step, 0, 0, 0);
  }
};
// PtrRows, for rows addressed by a functor: issue_stage's clamped addresses.
template <class Cfg, int ROWS, class RowAt>
struct PtrRows {
  const RowAt& row_at;
  int rows, H, r0;
  __device__ __forceinline__ void issue(int k0, unsigned char* dst) const {
    issue_stage<Cfg, ROWS>(row_at, rows, H, r0, k0, dst);
  }
};
template <class Cfg, int ROWS, class RowAt>
__device__ __forceinline__ auto tile_rows(const RowAt& row_at, int rows, int H, int r0) {
  if constexpr (std::is_same<RowAt, StridedRows>::value) return BufRows<Cfg, ROWS>(row_at, rows, H, r0);
  else return PtrRows<Cfg, ROWS, RowAt>{row_at, rows, H, r0};
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
__device__ __forceinline__ void tile_product_ring(const RowA& A, const RowB& B, int M, int N, int H, int m0, int n0,
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

// The fragments of one 32-wide k slice (chunks ks .. ks + 3 of every stage
// row) of the wave's block: row (lane & 15) of a 16-row group, chunk
// (lane >> 4) of the slice (16-row groups start at multiples of 16, so the
// swizzle of the row is that of lane & 15).
template <class Cfg>
__device__ __forceinline__ void read_slice(const unsigned char* st, int ks, int wm, int wn,
                                           bf16x8_t (&af)[Cfg::kFragM], bf16x8_t (&bfr)[Cfg::kFragN]) {
  const int lane = threadIdx.x & 63, frow = lane & 15;
  const int slot = ((ks + (lane >> 4)) ^ Cfg::swz(frow)) * 16;
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
    af[i] = __builtin_bit_cast(bf16x8_t, ld16(st + (wm + 16 * i + frow) * Cfg::kRowBytes + slot));
#pragma unroll
  for (int j = 0; j < Cfg::kFragN; ++j)
    bfr[j] = __builtin_bit_cast(bf16x8_t, ld16(st + Cfg::kBOff + (wn + 16 * j + frow) * Cfg::kRowBytes + slot));
}

template <class Cfg>
__device__ __forceinline__ void mfma_slice(const bf16x8_t (&af)[Cfg::kFragM], const bf16x8_t (&bfr)[Cfg::kFragN],
                                           f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN]) {
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

// Scheduling groups (instruction classes of the AMDGPU scheduler: 0x008 MFMA,
// 0x020 vector-memory read, 0x100 LDS read) for one slice: the NL direct
// loads and NR fragment reads are spread between the slice's MFMAs instead
// of being issued as one burst.
template <int NM, int NR, int NL>
__device__ __forceinline__ void interleave_slice() {
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  constexpr int per_read = NL > 0 ? 1 : 2;        // MFMAs between two fragment reads
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, per_read, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  constexpr int rest = NM - NL - per_read * NR;
  if constexpr (rest > 0) __builtin_amdgcn_sched_group_barrier(0x008, rest, 0);
}

// One 64-deep stage kt of the two-stage product (stage t in ring slot t % 2).
// On entry slice 0 of stage kt is in (a0, b0).  Phase A computes it while
// reading slice 1 into (a1, b1).  Then this thread's loads of stage kt + 1
// (the only ones in flight) are waited for and one barrier publishes stage
// kt + 1 to every wave -- and, every wave's reads of stage kt being done,
// frees its slot.  Phase B computes slice 1 while issuing stage kt + 2 into
// that slot (LOAD) and reading slice 0 of stage kt + 1 into (a0, b0).
template <class Cfg, bool LOAD, class LA, class LB>
__device__ __forceinline__ void slice_stage(const LA& la, const LB& lb, int H, int kb0, int nkb, int kt,
                                            unsigned char* smem, int wm, int wn,
                                            bf16x8_t (&a0)[Cfg::kFragM], bf16x8_t (&b0)[Cfg::kFragN],
                                            bf16x8_t (&a1)[Cfg::kFragM], bf16x8_t (&b1)[Cfg::kFragN],
                                            f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  constexpr int NM = Cfg::kFragM * Cfg::kFragN, NR = Cfg::kFragM + Cfg::kFragN, NL = Cfg::kLoadsPerStage;
  auto stage = [&](int t) { return smem + (t & 1) * Cfg::kStageBytes; };
  read_slice<Cfg>(stage(kt), 4, wm, wn, a1, b1);
  mfma_slice<Cfg>(a0, b0, acc);
  interleave_slice<NM, NR, 0>();
  wait_vm<0>();
  const int nk = (H + Cfg::kBK - 1) / Cfg::kBK;
  if ((H % Cfg::kBK) != 0 && kt + 1 < nkb && kb0 + kt + 1 == nk - 1) {
    zero_tail<Cfg, Cfg::kBM>(H, (kb0 + kt + 1) * Cfg::kBK, stage(kt + 1));
    zero_tail<Cfg, Cfg::kBN>(H, (kb0 + kt + 1) * Cfg::kBK, stage(kt + 1) + Cfg::kBOff);
  }
  ring_barrier();
  if constexpr (LOAD) {
    la.issue((kb0 + kt + 2) * Cfg::kBK, stage(kt));
    lb.issue((kb0 + kt + 2) * Cfg::kBK, stage(kt) + Cfg::kBOff);
  }
  // past the last stage this reads a slot whose values are never used
  read_slice<Cfg>(stage(kt + 1), 0, wm, wn, a0, b0);
  mfma_slice<Cfg>(a1, b1, acc);
  interleave_slice<NM, NR, LOAD ? NL : 0>();
}

// The two-stage, 64-deep product pipelined by slices (same result as
// tile_product_ring: every accumulator takes the same MFMA chain over the
// 32-wide k slices in increasing order).  Stages 0 and 1 are issued up front;
// stage kt + 2 goes out in phase B of stage kt, one stage of compute ahead of
// its use; the last two stages issue nothing.
template <class Cfg, class RowA, class RowB>
__device__ __forceinline__ void tile_product_sliced(const RowA& A, const RowB& B, int M, int N, int H, int m0,
                                                    int n0, int kb0, int nkb, unsigned char* smem,
                                                    f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  static_assert(Cfg::kBK == 64 && Cfg::kStages == 2, "two 64-deep stages");
  const int wave = threadIdx.x >> 6;
  const int wm = (wave / Cfg::kWavesN) * Cfg::kWM, wn = (wave % Cfg::kWavesN) * Cfg::kWN;
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (nkb <= 0) return;
  auto stage = [&](int t) { return smem + (t & 1) * Cfg::kStageBytes; };
  const auto la = tile_rows<Cfg, Cfg::kBM>(A, M, H, m0);
  const auto lb = tile_rows<Cfg, Cfg::kBN>(B, N, H, n0);
  la.issue(kb0 * Cfg::kBK, stage(0));
  lb.issue(kb0 * Cfg::kBK, stage(0) + Cfg::kBOff);
  if (nkb > 1) {
    la.issue((kb0 + 1) * Cfg::kBK, stage(1));
    lb.issue((kb0 + 1) * Cfg::kBK, stage(1) + Cfg::kBOff);
    wait_vm<Cfg::kLoadsPerStage>();
  } else {
    wait_vm<0>();
  }
  const int nk = (H + Cfg::kBK - 1) / Cfg::kBK;
  if ((H % Cfg::kBK) != 0 && kb0 == nk - 1) {
    zero_tail<Cfg, Cfg::kBM>(H, kb0 * Cfg::kBK, stage(0));
    zero_tail<Cfg, Cfg::kBN>(H, kb0 * Cfg::kBK, stage(0) + Cfg::kBOff);
  }
  ring_barrier();
  bf16x8_t a0[Cfg::kFragM], b0[Cfg::kFragN], a1[Cfg::kFragM], b1[Cfg::kFragN];
  read_slice<Cfg>(stage(0), 0, wm, wn, a0, b0);
  int kt = 0;
  for (; kt + 2 < nkb; ++kt) slice_stage<Cfg, true>(la, lb, H, kb0, nkb, kt, smem, wm, wn, a0, b0, a1, b1, acc);
  for (; kt < nkb; ++kt) slice_stage<Cfg, false>(la, lb, H, kb0, nkb, kt, smem, wm, wn, a0, b0, a1, b1, acc);
  __syncthreads();
}

// The kBM x kBN fp32 tile at (m0, n0) over k blocks [kb0, kb0 + nkb): the
// sliced pipeline for two 64-deep stages and waves of >= 32 MFMAs per slice
// (where the matrix cores bound the product), the plain ring otherwise.
template <class Cfg, class RowA, class RowB>
__device__ __forceinline__ void tile_product(const RowA& A, const RowB& B, int M, int N, int H, int m0, int n0,
                                             int kb0, int nkb, unsigned char* smem,
                                             f32x4_t (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  if constexpr (Cfg::kBK == 64 && Cfg::kStages == 2 && Cfg::kFragM * Cfg::kFragN >= 32)
    tile_product_sliced<Cfg>(A, B, M, N, H, m0, n0, kb0, nkb, smem, acc);
  else
    tile_product_ring<Cfg>(A, B, M, N, H, m0, n0, kb0, nkb, smem, acc);
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

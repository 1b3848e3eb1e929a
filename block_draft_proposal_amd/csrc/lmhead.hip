// Dense lm_head on the matrix cores of gfx950 (bf16 in, fp32 accumulate).
//
// Operation ("[Spec] DFlash2: local convolution + candidate selector",
// implementation breakdown and risk notes: compute_candidates multiplies the
// slot hidden rows by the target lm_head weight as a dense matrix; the
// product is returned in the model's dtype):
//   logits[n, v] = round_bf16( sum_k h[n, k] * W[v, k] )
// h [M, H] (row stride given), W [V, H] (rows contiguous), both with the
// contraction axis contiguous.
//
// Design: one workgroup (4 waves) per 128 x 128 output tile.  The k axis is
// walked in stages of 64: each stage's A (hidden) and B (head) tiles are
// loaded to registers while the previous stage is multiplied out of LDS
// (double buffer, one barrier per stage).  Each wave owns a 64 x 64 sub-tile
// as 4 x 4 v_mfma_f32_16x16x32_bf16 accumulators; bf16 x bf16 products are
// exact in fp32.  LDS rows hold 64 + 8 elements (144 bytes), so the 16 rows
// of an MFMA fragment fall on distinct bank groups.  Workgroups are dealt to
// the 8 XCDs in turn; the mapping of workgroup to tile keeps the row blocks
// that share one head tile on the same XCD, so each head tile is fetched from
// HBM about once and re-read from that XCD's L2.  The fp32 tile is rounded
// to bf16 (nearest, ties to even) and written through LDS as 16-byte rows.
//
// Fused head + top-K (compute_candidates without the logits reaching HBM):
// a workgroup computes one column tile of its row block (a few when a row's
// lists would not fit the merge) with the same tile product; each rounded
// tile is put in LDS and two threads per row fold the row's values into
// sorted register lists of the K best composites (value descending, id
// ascending; ids grow along each thread's walk, so one strict comparison
// with the K-th decides), merged pairwise at the end.  The lists of all
// column groups are merged per row by a second kernel, which ranks the
// candidates that can still place by binary-searched counts in the other
// sorted lists.  Both paths rank the same bf16
// logits, so the fused result equals the head followed by the streaming
// top-K bit for bit.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Each wave computes a (16 kFragM) x (16 kFragN) block of the tile with
// kFragM x kFragN MFMAs of 16 x 16 x 32; the waves tile it kWavesM x kWavesN.
// The LDS bytes each MFMA needs fall as the wave's block grows.
constexpr int kFragM = 8, kFragN = 4;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kWM = 16 * kFragM, kWN = 16 * kFragN;
constexpr int kBM = kWM * kWavesM, kBN = kWN * kWavesN;
constexpr int kBK = 64;                     // contraction depth of one stage (32 or 64)
constexpr int kChunks = kBK / 8;            // 16-byte chunks per stage row
constexpr int kRowBytes = kBK * 2;
constexpr int kBlockRows = 1024 / kRowBytes;   // rows per 1 KB block of direct loads
constexpr int kSwzShift = kBK == 64 ? 1 : 2;   // log2 of the rows sharing a 256-byte bank window
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kLmThreads = 64 * kWaves;
constexpr int kStages = 2;                  // LDS ring depth: loads run kStages - 1 stages ahead
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;   // one stage of A and B
constexpr int kLoadsPerStage = (kBM + kBN) / kBlockRows / kWaves;   // direct loads per thread per stage
// The rounded output tile goes through LDS in passes of kOutCols columns.
constexpr int kOutCols = kBN < 128 ? kBN : 128;
constexpr int kOutPasses = kBN / kOutCols;
constexpr int kCPad = kOutCols + 8;         // bf16 elements per LDS row of one pass
static_assert(kBK == 32 || kBK == 64, "stage depth");
static_assert(kBM % (kBlockRows * kWaves) == 0 && kBN % (kBlockRows * kWaves) == 0,
              "stage rows split evenly over the waves");
static_assert(kStages >= 2 && kStages <= 5, "wait counts below cover up to three stages ahead");
static_assert(kOutCols % kWN == 0 && kBN % kOutCols == 0, "a wave's columns lie in one output pass");

// The LDS of one workgroup: a ring of kStages stages, each the A tile
// [kBM rows][kBK k] then the B tile [kBN rows][kBK k], rows of kRowBytes
// without padding.  Within a row the 16-byte k chunks are stored
// XOR-swizzled: chunk c of row r sits in slot c ^ swz(r), so the 16 rows one
// MFMA fragment reads, and the two chunks of neighbouring lane groups, fall
// on distinct banks.
struct LmSmem {
  unsigned char stage[kStages][kStageBytes];
};
static_assert(sizeof(uint16_t) * kBM * kCPad <= sizeof(LmSmem), "output tile fits in the ring");

typedef __attribute__((address_space(3))) void lds_void_t;

// Workgroup -> (row block, column block).  Consecutive workgroups go to
// consecutive XCDs; the n_mb row blocks of one column block get ids that
// are equal modulo 8, so they share an XCD (and its L2).
__device__ __forceinline__ void tile_of(int id, int n_mb, int& mb, int& nb) {
  const int xcd = id & 7, slot = id >> 3;
  nb = (slot / n_mb) * 8 + xcd;
  mb = slot % n_mb;
}

__device__ __forceinline__ int swz(int row) { return (row >> kSwzShift) & (kChunks - 1); }

// Issues the direct global -> LDS loads of one stage: rows [r0, r0 + ROWS)
// x k [k0, k0 + kBK) of a [rows, H] matrix, in 1 KB blocks of kBlockRows
// rows dealt round the waves; lane l of a block fills slot l % kChunks of
// row l / kChunks with the chunk the swizzle puts there.  Addresses are
// clamped into the matrix: rows past the end repeat the last row (their
// results are never used) and k past H is zeroed by zero_tail before use.
template <int ROWS>
__device__ __forceinline__ void issue_stage(const uint16_t* __restrict__ base, int64_t stride, int rows, int H,
                                            int r0, int k0, unsigned char* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < ROWS / kBlockRows / kWaves; ++q) {
    const int blk = q * kWaves + wave, r = blk * kBlockRows + lane / kChunks;
    const int k = k0 + 8 * ((lane % kChunks) ^ swz(r));
    const uint16_t* src = base + (int64_t)min(r0 + r, rows - 1) * stride + min(k, H - 8);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + blk * 1024), 16, 0, 0);
  }
}

// After the stage has landed: zeroes this thread's chunks of it whose k is
// at or past H (only the last stage of a hidden size that is not a multiple
// of kBK has any).
template <int ROWS>
__device__ __forceinline__ void zero_tail(int H, int k0, unsigned char* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < ROWS / kBlockRows / kWaves; ++q) {
    const int blk = q * kWaves + wave, r = blk * kBlockRows + lane / kChunks;
    if (k0 + 8 * ((lane % kChunks) ^ swz(r)) >= H) st16(dst + blk * 1024 + lane * 16, zero);
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

// The kBM x kBN fp32 tile of (mb, nb); each wave holds its kWM x kWN block
// in kFragM x kFragN accumulators.  D layout of one 16 x 16 MFMA: lane l holds column
// l % 16 and rows 4 (l / 16) + v, v = 0..3.  Stage t of the contraction
// lives in ring slot t % kStages; each iteration waits for its own stage,
// passes one barrier (after which the slot computed last iteration is free)
// and refills that slot with stage t + kStages - 1 before computing.  Ends
// with a barrier, so the ring may be reused.
__device__ __forceinline__ void tile_product(const uint16_t* __restrict__ h, int64_t h_stride,
                                             const uint16_t* __restrict__ W, int M, int H, int V, int m0, int n0,
                                             LmSmem& sm, f32x4_t (&acc)[kFragM][kFragN]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave / kWavesN) * kWM, wn = (wave % kWavesN) * kWN;
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = (H + kBK - 1) / kBK;
  const bool ragged = (H % kBK) != 0;
  constexpr int kBOff = kBM * kRowBytes;        // the B tile within a stage
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) {
    if (t < nk) {
      issue_stage<kBM>(h, h_stride, M, H, m0, t * kBK, sm.stage[t]);
      issue_stage<kBN>(W, H, V, H, n0, t * kBK, sm.stage[t] + kBOff);
    }
  }
  // fragment reads: row (lane & 15) of a 16-row group, chunk (lane >> 4) of a
  // 32-wide k slice (16-row groups start at multiples of 16, so the swizzle
  // of the row is that of lane & 15)
  const int frow = lane & 15, fsw = swz(frow);
  for (int kt = 0; kt < nk; ++kt) {
    unsigned char* cur = sm.stage[kt % kStages];
    // this thread's loads of stage kt are done once at most the loads of
    // the later stages already issued are outstanding
    const int ahead = min(kStages - 2, nk - 1 - kt);
    if (ahead >= 3) wait_vm<3 * kLoadsPerStage>();
    else if (ahead == 2) wait_vm<2 * kLoadsPerStage>();
    else if (ahead == 1) wait_vm<kLoadsPerStage>();
    else wait_vm<0>();
    if (ragged && kt == nk - 1) {
      zero_tail<kBM>(H, kt * kBK, cur);
      zero_tail<kBN>(H, kt * kBK, cur + kBOff);
    }
    ring_barrier();
    if (kt + kStages - 1 < nk) {
      unsigned char* nxt = sm.stage[(kt + kStages - 1) % kStages];
      issue_stage<kBM>(h, h_stride, M, H, m0, (kt + kStages - 1) * kBK, nxt);
      issue_stage<kBN>(W, H, V, H, n0, (kt + kStages - 1) * kBK, nxt + kBOff);
    }
    const unsigned char* sa = cur;
    const unsigned char* sb = cur + kBOff;
#pragma unroll
    for (int ks = 0; ks < kChunks; ks += 4) {        // 32-wide k slices: chunks ks .. ks + 3
      const int slot = ((ks + (lane >> 4)) ^ fsw) * 16;
      bf16x8_t af[kFragM], bfrag[kFragN];
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, ld16(sa + (wm + 16 * i + frow) * kRowBytes + slot));
#pragma unroll
      for (int j = 0; j < kFragN; ++j)
        bfrag[j] = __builtin_bit_cast(bf16x8_t, ld16(sb + (wn + 16 * j + frow) * kRowBytes + slot));
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfrag[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();
}

// The wave's accumulators rounded to bf16 (nearest, ties to even), two per
// register: pk[i][j][0] holds rows 4 (l / 16) + 0, 1 and pk[i][j][1] rows
// + 2, 3 of fragment (i, j), low half first.  Rounding once here frees the
// fp32 accumulators before the epilogue.
__device__ __forceinline__ void pack_tile(const f32x4_t (&acc)[kFragM][kFragN], uint32_t (&pk)[kFragM][kFragN][2]) {
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pk[i][j][h] = f32_to_bf16_rne(acc[i][j][2 * h]) | (f32_to_bf16_rne(acc[i][j][2 * h + 1]) << 16);
}

// Writes into LDS the rounded values of the waves whose columns lie in
// output pass `pass` (tile columns [pass kOutCols, (pass + 1) kOutCols)).
__device__ __forceinline__ void tile_to_lds(const uint32_t (&pk)[kFragM][kFragN][2], uint16_t* cs, int pass) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave / kWavesN) * kWM, wn = (wave % kWavesN) * kWN - pass * kOutCols;
  if (wn < 0 || wn >= kOutCols) return;
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        cs[(wm + 16 * i + 4 * (lane >> 4) + v) * kCPad + wn + 16 * j + (lane & 15)] =
            (uint16_t)((v & 1) ? (pk[i][j][v >> 1] >> 16) : (pk[i][j][v >> 1] & 0xffffu));
}

__global__ __launch_bounds__(kLmThreads) void lm_head_kernel(const uint16_t* __restrict__ h, int64_t h_stride,
                                                             const uint16_t* __restrict__ W, int32_t M, int32_t H,
                                                             int32_t V, uint16_t* __restrict__ logits,
                                                             int64_t l_stride, int32_t n_mb, int32_t n_nb) {
  extern __shared__ __align__(16) unsigned char lm_smem[];
  LmSmem& sm = *reinterpret_cast<LmSmem*>(lm_smem);
  int mb, nb;
  tile_of(blockIdx.x, n_mb, mb, nb);
  if (nb >= n_nb) return;
  const int m0 = mb * kBM, n0 = nb * kBN;
  uint32_t pk[kFragM][kFragN][2];
  {
    f32x4_t acc[kFragM][kFragN];
    tile_product(h, h_stride, W, M, H, V, m0, n0, sm, acc);
    pack_tile(acc, pk);
  }

  // per pass: the rounded values into LDS, then whole 16-byte row pieces out
  const int tid = threadIdx.x;
  uint16_t* cs = reinterpret_cast<uint16_t*>(sm.stage[0]);
  for (int pass = 0; pass < kOutPasses; ++pass) {
    tile_to_lds(pk, cs, pass);
    __syncthreads();
    const int c0 = n0 + pass * kOutCols;
#pragma unroll
    for (int q = 0; q < (kBM * kOutCols / 8) / kLmThreads; ++q) {
      const int c = tid + kLmThreads * q;
      const int row = c / (kOutCols / 8), col = 8 * (c % (kOutCols / 8));
      if (m0 + row >= M) continue;
      uint16_t* dst = logits + (int64_t)(m0 + row) * l_stride + c0 + col;
      const uint16_t* src = cs + row * kCPad + col;
      if (c0 + col + 8 <= V) {
        st16(dst, ld16(src));
      } else {
        for (int e = 0; e < 8 && c0 + col + e < V; ++e) dst[e] = src[e];
      }
    }
    __syncthreads();
  }
}

// KB: list slots (K rounded up to 8, 16 or 32).  The list holds KB - K
// sentinels (all ones, above every entry) ahead of the K real entries, so
// the threshold is always the last slot and no index depends on K.
template <int KB>
__device__ __forceinline__ void list_insert(uint64_t (&best)[KB], uint64_t c) {
#pragma unroll
  for (int i = 0; i < KB; ++i) {                 // keeps the list sorted descending
    if (c > best[i]) { const uint64_t t = best[i]; best[i] = c; c = t; }
  }
}
template <int KB>
__device__ __forceinline__ void list_insert(uint32_t (&best)[KB], uint32_t c) {
#pragma unroll
  for (int i = 0; i < KB; ++i) {                 // keeps the list sorted descending
    const uint32_t hi = max(best[i], c);
    c = min(best[i], c);
    best[i] = hi;
  }
}

// Within one tile a value's order is carried by a 32-bit key: its 16-bit
// value key above 255 - (column within the tile), so larger is better and
// equal values rank by column; 0 marks an empty slot.
static_assert(kBN <= 256, "tile columns fit the 8-bit column field");
__device__ __forceinline__ uint32_t tile_key(uint32_t key, int col_in_tile) {
  return (key << 8) | (uint32_t)(255 - col_in_tile);
}
__device__ __forceinline__ uint64_t tile_key_composite(uint32_t tk, int n0) {
  return composite(tk >> 8, n0 + 255 - (int)(tk & 255u));
}

constexpr int kRowThreads = kLmThreads / kBM;   // scan threads per tile row
constexpr int kScanCols = kOutCols / kRowThreads;   // columns each of them folds in per output pass
static_assert(kLmThreads % kBM == 0 && kScanCols % 8 == 0, "scan threads split the rows evenly");
static_assert(sizeof(uint32_t) * kBM * (kRowThreads - 1) * 32 <= sizeof(LmSmem), "list exchange fits the ring");

// kRowThreads threads per row: thread t takes row t / kRowThreads and, of
// every output pass of a tile, the kScanCols columns from p kScanCols on,
// p = t % kRowThreads, folding them into a sorted list of its own.  After
// the tile the lists of a row meet in LDS and the row's p = 0 thread merges
// them, with the group's list so far (from the workspace, for the second
// tile of a group on), and stores the group's list.  No list is live across
// a tile product.
//
// bound[r] is a lower bound on the key of row r's K-th best value: once a
// merged list holds K values the bound is raised (atomic max) to the key of
// its K-th, since K values of the row have at least that key.  Values with a
// smaller key cannot place and are skipped before any list work; the bound
// only grows, so a stale read filters less but never wrongly.
template <int KB>
__global__ __launch_bounds__(kLmThreads) void lm_head_topk_kernel(
    const uint16_t* __restrict__ h, int64_t h_stride, const uint16_t* __restrict__ W, int32_t M, int32_t H,
    int32_t V, int32_t valid, int32_t K, int32_t n_mb, int32_t n_nb, int32_t tiles_per_group, int32_t n_grp,
    uint64_t* __restrict__ parts, uint32_t* __restrict__ bound) {
  extern __shared__ __align__(16) unsigned char lm_smem[];
  LmSmem& sm = *reinterpret_cast<LmSmem*>(lm_smem);
  int mb, grp;
  tile_of(blockIdx.x, n_mb, mb, grp);
  if (grp >= n_grp) return;
  const int m0 = mb * kBM, tid = threadIdx.x;
  const int row = tid / kRowThreads, part = tid % kRowThreads;
  const bool row_ok = m0 + row < M;
  const int nb0 = grp * tiles_per_group, nb1 = min(n_nb, nb0 + tiles_per_group);
  uint16_t* cs = reinterpret_cast<uint16_t*>(sm.stage[0]);
  uint64_t* dst = parts + ((int64_t)(m0 + row) * n_grp + grp) * K;
  for (int nb = nb0; nb < nb1; ++nb) {
    const int n0 = nb * kBN;
    uint32_t pk[kFragM][kFragN][2];
    {
      f32x4_t acc[kFragM][kFragN];
      tile_product(h, h_stride, W, M, H, V, m0, n0, sm, acc);   // ends with a barrier
      pack_tile(acc, pk);
    }
    uint32_t lo = 0;
    if (row_ok) lo = __hip_atomic_load(bound + m0 + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t tl[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) tl[i] = (i < KB - K) ? ~0u : 0u;
    for (int pass = 0; pass < kOutPasses; ++pass) {
      tile_to_lds(pk, cs, pass);
      __syncthreads();
      const int t_lo = pass * kOutCols + kScanCols * part;   // first column within the tile
      if (row_ok && n0 + t_lo < valid) {
        const uint16_t* rowp = cs + row * kCPad + kScanCols * part;
#pragma unroll 2
        for (int c8 = 0; c8 < kScanCols; c8 += 8) {
          if (n0 + t_lo + c8 >= valid) break;
          const u32x4 v = ld16(rowp + c8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tc = t_lo + c8 + e;
            const uint32_t key = bf16_key((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu));
            if (key >= lo && n0 + tc < valid) {
              const uint32_t c = tile_key(key, tc);
              if (c > tl[KB - 1]) list_insert(tl, c);
            }
          }
        }
      }
      __syncthreads();                         // the pass's LDS is reused next
    }
    // row merge: the other threads' lists to LDS, the p = 0 thread folds them
    // in, widens its list to composites and adds the group's earlier tiles
    uint32_t* xch = reinterpret_cast<uint32_t*>(lm_smem);   // [kBM][kRowThreads - 1][KB]
    if (part > 0) {
#pragma unroll
      for (int i = 0; i < KB; ++i) xch[(row * (kRowThreads - 1) + part - 1) * KB + i] = tl[i];
    }
    __syncthreads();
    if (part == 0 && row_ok) {
      for (int o = 0; o < kRowThreads - 1; ++o) {
#pragma unroll
        for (int i = KB - 1; i >= 0; --i) {
          const uint32_t c = xch[(row * (kRowThreads - 1) + o) * KB + i];
          if (c != ~0u && c > tl[KB - 1]) list_insert(tl, c);
        }
      }
      uint64_t kth;                            // the group list's K-th entry
      if (nb == nb0) {
#pragma unroll
        for (int i = 0; i < KB; ++i)
          if (i >= KB - K) dst[i - (KB - K)] = tl[i] == 0u ? 0ull : tile_key_composite(tl[i], n0);
        kth = tl[KB - 1] == 0u ? 0ull : tile_key_composite(tl[KB - 1], n0);
      } else {                                 // with the group's earlier tiles (stored by this thread)
        uint64_t best[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i)
          best[i] = (i < KB - K) ? ~0ull : (tl[i] == 0u ? 0ull : tile_key_composite(tl[i], n0));
        for (int i = K - 1; i >= 0; --i) {
          const uint64_t c = dst[i];
          if (c > best[KB - 1]) list_insert(best, c);
        }
#pragma unroll
        for (int i = 0; i < KB; ++i)
          if (i >= KB - K) dst[i - (KB - K)] = best[i];
        kth = best[KB - 1];
      }
      if (kth != 0 && composite_key(kth) > lo)
        __hip_atomic_fetch_max(bound + m0 + row, composite_key(kth), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();                           // xch lies in the ring the next tile refills
  }
}

__global__ void clear_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Per row: the K best of n_grp sorted lists of K composites (0 = empty
// slot), all distinct.  Thread t takes lists t, t + 256, ... and the largest
// head among them; the K-th largest of these thread maxima (the floor) has K
// list heads at or above it, so nothing below it can place.  Only the K
// threads at or above the floor hold entries at or above it, at most
// ceil(n_grp / 256) lists of K each, so the candidates fit kLmMergeCand;
// every entry above a candidate is a candidate too, so its rank among the
// candidates is its rank in the row.
constexpr int kMergeThreadsLm = 256;
__global__ __launch_bounds__(kMergeThreadsLm) void merge_lists_kernel(const uint64_t* __restrict__ parts,
                                                                    int32_t n_grp, int32_t K, float mult, float cap,
                                                                    int64_t* __restrict__ ids_out,
                                                                    float* __restrict__ unary_out) {
  __shared__ uint64_t s_max[kMergeThreadsLm];
  __shared__ uint64_t s_cand[kLmMergeCand];
  __shared__ uint64_t s_floor;
  __shared__ int s_n;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint64_t* src = parts + row * (int64_t)n_grp * K;
  uint64_t mx = 0;
  for (int g = tid; g < n_grp; g += kMergeThreadsLm) mx = max(mx, src[(int64_t)g * K]);
  s_max[tid] = mx;
  if (tid == 0) { s_floor = 0; s_n = 0; }
  __syncthreads();
  int above = 0;
  for (int o = 0; o < kMergeThreadsLm; ++o) above += (s_max[o] > mx) ? 1 : 0;
  if (mx != 0 && above == K - 1) s_floor = mx;   // exactly one thread: the maxima are distinct
  __syncthreads();
  const uint64_t floor = s_floor;
  if (mx != 0 && mx >= floor) {
    for (int g = tid; g < n_grp; g += kMergeThreadsLm) {
      const uint64_t* list = src + (int64_t)g * K;
      for (int j = 0; j < K; ++j) {             // descending: stop at the first miss
        const uint64_t c = list[j];
        if (c == 0 || c < floor) break;
        s_cand[atomicAdd(&s_n, 1)] = c;
      }
    }
  }
  __syncthreads();
  const int n = s_n;
  for (int i = tid; i < n; i += kMergeThreadsLm) {
    const uint64_t c = s_cand[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (s_cand[j] > c) ? 1 : 0;
    if (rank < K) {
      ids_out[row * K + rank] = composite_id(c);
      unary_out[row * K + rank] = unary_transform(bf16_key_value(composite_key(c)), mult, cap);
    }
  }
}

}  // namespace

LmTopkPlan plan_lm_head_topk(int64_t n_rows, int64_t vocab, int32_t top_k) {
  LmTopkPlan p{};
  p.n_mb = (int32_t)((n_rows + kBM - 1) / kBM);
  p.n_nb = (int32_t)((vocab + kBN - 1) / kBN);
  // one tile per workgroup unless a row's merge candidates could overflow
  // (K threads of the merge, ceil(n_grp / 256) lists of K each)
  int t = 1;
  while ((int64_t)top_k * top_k * (((p.n_nb + t - 1) / t + 255) / 256) > kLmMergeCand) ++t;
  p.tiles_per_group = t;
  p.n_grp = (p.n_nb + t - 1) / t;
  const size_t lists = (size_t)n_rows * p.n_grp * top_k * sizeof(uint64_t);
  p.bound_offset = (lists + 255) & ~(size_t)255;
  p.bytes = (p.bound_offset + (size_t)n_rows * sizeof(uint32_t) + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_lm_head_topk(const LmHeadArgs& a, const LmTopkPlan& p, int64_t valid_vocab, int32_t top_k,
                               float mult, float cap, int64_t* ids_out, float* unary_out, void* workspace,
                               hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  uint64_t* parts = static_cast<uint64_t*>(workspace);
  uint32_t* bound = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) + p.bound_offset);
  hipLaunchKernelGGL(clear_u32_kernel, dim3((unsigned)((a.n_rows + 255) / 256)), dim3(256), 0, stream, bound,
                     a.n_rows);
  const int64_t slots = (int64_t)((p.n_grp + 7) / 8) * p.n_mb;
  const dim3 grid((unsigned)(slots * 8));
#define DFLASH_LMTK(KB)                                                                                    \
  hipLaunchKernelGGL((lm_head_topk_kernel<KB>), grid, dim3(kLmThreads), sizeof(LmSmem), stream,                \
                     static_cast<const uint16_t*>(a.hidden), a.hidden_row_stride,                          \
                     static_cast<const uint16_t*>(a.weight), (int32_t)a.n_rows, a.hidden_size,             \
                     (int32_t)a.vocab, (int32_t)valid_vocab, top_k, p.n_mb, p.n_nb, p.tiles_per_group,     \
                     p.n_grp, parts, bound)
  if (top_k <= 8) DFLASH_LMTK(8);
  else if (top_k <= 16) DFLASH_LMTK(16);
  else DFLASH_LMTK(32);
#undef DFLASH_LMTK
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_lists_kernel, dim3((unsigned)a.n_rows), dim3(kMergeThreadsLm), 0, stream, parts, p.n_grp, top_k, mult, cap, ids_out,
                     unary_out);
  return hipGetLastError();
}

hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t stream) {
  if (a.n_rows == 0 || a.vocab == 0) return hipSuccess;
  const int n_mb = (int)((a.n_rows + kBM - 1) / kBM);
  const int n_nb = (int)((a.vocab + kBN - 1) / kBN);
  const int64_t slots = (int64_t)((n_nb + 7) / 8) * n_mb;
  hipLaunchKernelGGL(lm_head_kernel, dim3((unsigned)(slots * 8)), dim3(kLmThreads), sizeof(LmSmem), stream,
                     static_cast<const uint16_t*>(a.hidden), a.hidden_row_stride,
                     static_cast<const uint16_t*>(a.weight), (int32_t)a.n_rows, a.hidden_size, (int32_t)a.vocab,
                     static_cast<uint16_t*>(a.logits), a.logits_row_stride, n_mb, n_nb);
  return hipGetLastError();
}

}  // namespace dflash

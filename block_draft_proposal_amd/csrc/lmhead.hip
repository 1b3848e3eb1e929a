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
// Design: one workgroup (8 waves) per 256 x 256 output tile, the tile
// product of gemm_tile.h (direct global -> LDS staging into a two-stage
// swizzled ring, 128 x 64 per wave, pipelined by 32-wide k slices).  Each
// XCD walks its column blocks in groups of 8 row blocks, so the workgroups
// it runs together share head tiles and hidden rows in its L2.  The fp32 tile is rounded to bf16 (nearest, ties to even) and
// written through LDS as 16-byte row pieces.
//
// Fused head + top-K (compute_candidates without the logits reaching HBM):
// each workgroup computes a group of consecutive column tiles of its row
// block with the same tile product and keeps each row's K best of the group
// in LDS.  Once a row has a threshold (its group list's K-th, or a per-row
// bound on the K-th best key that finished group lists publish), the
// rounded values are tested in registers and only the few that pass reach
// the lists; tiles without thresholds are staged in LDS and scanned.  After
// its last tile a group stores its K best composites (value descending, id
// ascending), and a second kernel merges the groups of each row.  Both
// paths rank the same bf16 logits, so the fused result equals the head
// followed by the streaming top-K bit for bit.
#include "dflash.h"
#include "dflash_internal.h"
#include "gemm_tile.h"

namespace dflash {
namespace {

// The head's tile: 256 x 256 over 8 waves of 128 x 64, two 64-deep stages
// (128 KB of LDS, one workgroup per CU, two waves per SIMD).
using LmCfg = TileCfg<8, 4, 2, 4, 64, 2>;
constexpr int kBM = LmCfg::kBM, kBN = LmCfg::kBN;
constexpr int kFragM = LmCfg::kFragM, kFragN = LmCfg::kFragN;
constexpr int kLmThreads = LmCfg::kThreads;
constexpr int kOutCols = LmCfg::kOutCols, kOutPasses = LmCfg::kOutPasses, kCPad = LmCfg::kCPad;
constexpr size_t kLmSmem = LmCfg::kSmemBytes;
// row blocks per group of the XCD-local tile order (tile_of_grouped)
constexpr int kGroupRows = 8;
typedef short i16x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kLmThreads) void lm_head_kernel(const uint16_t* __restrict__ h, int64_t h_stride,
                                                             const uint16_t* __restrict__ W, int32_t M, int32_t H,
                                                             int32_t V, uint16_t* __restrict__ logits,
                                                             int64_t l_stride, int32_t n_mb, int32_t n_nb) {
  extern __shared__ __align__(16) unsigned char lm_smem[];
  int mb, nb;
  tile_of_grouped<kGroupRows>(blockIdx.x, n_mb, n_nb, mb, nb);
  if (nb >= n_nb) return;
  const int m0 = mb * kBM, n0 = nb * kBN;
  uint32_t pk[kFragM][kFragN][2];
  {
    f32x4_t acc[kFragM][kFragN];
    tile_product<LmCfg>(h, h_stride, W, H, M, V, H, m0, n0, 0, (H + LmCfg::kBK - 1) / LmCfg::kBK, lm_smem, acc);
    pack_tile<LmCfg>(acc, pk);
  }

  // per pass: the rounded values into LDS, then whole 16-byte row pieces out
  const int tid = threadIdx.x;
  uint16_t* cs = reinterpret_cast<uint16_t*>(lm_smem);
  for (int pass = 0; pass < kOutPasses; ++pass) {
    tile_to_lds<LmCfg>(pk, cs, pass);
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

// Within a group of column tiles a value's order is carried by a 32-bit key:
// its 16-bit value key above 65535 - (column within the group), so larger is
// better and equal values rank by column; 0 marks an empty slot.  A group
// spans at most 65536 columns.
constexpr int kMaxGroupCols = 65536;
__device__ __forceinline__ uint32_t group_key(uint32_t key, int col_in_group) {
  return (key << 16) | (uint32_t)(0xFFFF - col_in_group);
}
__device__ __forceinline__ uint64_t group_key_composite(uint32_t gk, int g0) {
  return composite(gk >> 16, g0 + 0xFFFF - (int)(gk & 0xFFFFu));
}

constexpr int kRowThreads = kLmThreads / kBM;   // scan threads per tile row
constexpr int kScanCols = kOutCols / kRowThreads;   // columns each of them folds in per output pass
static_assert(kLmThreads % kBM == 0 && kScanCols % 8 == 0, "scan threads split the rows evenly");
static_assert(sizeof(uint32_t) * kBM * (kRowThreads - 1) * 32 <= kLmSmem, "list exchange fits the ring");
// the group lists ([kBM][KB] keys) sit in LDS past the tile ring
template <int KB> constexpr size_t lm_topk_smem() { return kLmSmem + sizeof(uint32_t) * kBM * KB; }
static_assert(lm_topk_smem<32>() <= 160 * 1024, "ring + group lists fit a workgroup's LDS");
// Each scan thread's pending candidates: kCandCap keys in the ring past the
// staged output pass (which the scan reads), inserted into its list when the
// buffer fills and at the end of each pass.
constexpr int kCandCap = 16;
constexpr size_t kCandOff = sizeof(uint16_t) * kBM * kCPad;
static_assert(kCandOff % 16 == 0 && kCandOff + sizeof(uint32_t) * kLmThreads * kCandCap <= kLmSmem,
              "candidate buffers fit the ring beside the staged pass");
// The filter from registers: per tile row a threshold and a buffer of up to
// kRowCap passing keys with its count, all in the ring after the tile
// product, then an overflow flag.
constexpr int kRowCap = 112;
constexpr size_t kThrOff = sizeof(uint32_t) * (kBM * kRowCap + kBM);
constexpr size_t kOverOff = kThrOff + sizeof(uint32_t) * kBM;
static_assert(kThrOff % 16 == 0 && kOverOff + 16 <= kLmSmem, "row buffers, counts and thresholds fit the ring");

// A workgroup walks a group of consecutive column tiles of its row block.
// kRowThreads threads per row: thread t takes row t / kRowThreads and, of
// every output pass of a tile, the kScanCols columns from p kScanCols on,
// p = t % kRowThreads, folding them into a sorted list of its own -- the p = 0
// thread starting from the row's group list (in LDS), the others empty; a
// value enters only above the group list's K-th entry.  A value that passes
// is first appended to the thread's candidate buffer (one store), and the
// buffer is inserted into the list when it fills or the pass ends: inserting
// on the spot would run the K-step insertion for every lane of the wave
// whenever any one lane had a value to insert.  After the tile the
// lists of a row meet in LDS and the p = 0 thread merges them and stores the
// group list back.  No list is live across a tile product.  After the
// group's last tile its K best go to the workspace as composites.
//
// bound[r] is a lower bound on the key of row r's K-th best value: once a
// group list holds K values the bound is raised (atomic max) to the key of
// its K-th, since K values of the row have at least that key.  Values with a
// smaller key cannot place and are skipped before any list work; the bound
// only grows, so a stale read filters less but never wrongly.
//
// Most tiles skip the staging: once every row of the tile has a threshold
// (its group list's K-th key, or the bound), each lane tests the 128
// rounded values it holds against their rows' thresholds and appends the
// few that pass to their row's buffer in LDS (an LDS atomic gives the
// slot); the p = 0 thread of each row then inserts its row's entries into
// the group list.  A tile where some row has no threshold yet (a group's
// first tiles) or a row's buffer overflows takes the staged scan instead.
// Both paths let exactly the values above the same thresholds reach the
// lists, so the result does not depend on which one a tile takes.
template <int KB>
__global__ __launch_bounds__(kLmThreads) void lm_head_topk_kernel(
    const uint16_t* __restrict__ h, int64_t h_stride, const uint16_t* __restrict__ W, int32_t M, int32_t H,
    int32_t V, int32_t valid, int32_t K, int32_t n_mb, int32_t n_nb, int32_t tiles_per_group, int32_t n_grp,
    uint64_t* __restrict__ parts, uint32_t* __restrict__ bound) {
  extern __shared__ __align__(16) unsigned char lm_smem[];
  int mb, grp;
  tile_of_grouped<kGroupRows>(blockIdx.x, n_mb, n_grp, mb, grp);
  if (grp >= n_grp) return;
  const int m0 = mb * kBM, tid = threadIdx.x;
  const int row = tid / kRowThreads, part = tid % kRowThreads;
  const bool row_ok = m0 + row < M;
  const int nb0 = grp * tiles_per_group, nb1 = min(n_nb, nb0 + tiles_per_group);
  uint16_t* cs = reinterpret_cast<uint16_t*>(lm_smem);
  uint32_t* glist = reinterpret_cast<uint32_t*>(lm_smem + kLmSmem) + row * KB;   // the row's group list
  // KB - K sentinels (above every entry) ahead of the K real slots, so the
  // K-th entry is always the last slot; visible after the tile product's
  // first barrier
  if (part == 0) {
#pragma unroll
    for (int i = 0; i < KB; ++i) glist[i] = (i < KB - K) ? ~0u : 0u;
  }
  for (int nb = nb0; nb < nb1; ++nb) {
    const int n0 = nb * kBN, cg0 = (nb - nb0) * kBN;   // the tile's first column, in the row and in the group
    uint32_t pk[kFragM][kFragN][2];
    {
      f32x4_t acc[kFragM][kFragN];
      tile_product<LmCfg>(h, h_stride, W, H, M, V, H, m0, n0, 0, (H + LmCfg::kBK - 1) / LmCfg::kBK, lm_smem,
                          acc);                  // ends with a barrier
      pack_tile<LmCfg>(acc, pk);
    }
    {
      // thresholds: a value passes iff its group key exceeds its row's
      // (the group list's K-th, and key >= bound); rows past M take none
      uint32_t* s_cnt = reinterpret_cast<uint32_t*>(lm_smem) + kBM * kRowCap;
      uint32_t* s_thr = reinterpret_cast<uint32_t*>(lm_smem + kThrOff);
      uint32_t* s_over = reinterpret_cast<uint32_t*>(lm_smem + kOverOff);
      if (tid == 0) *s_over = 0u;
      __syncthreads();
      if (tid < kBM) {
        uint32_t t = ~0u;
        if (m0 + tid < M) {
          const uint32_t b = __hip_atomic_load(bound + m0 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          t = max(reinterpret_cast<const uint32_t*>(lm_smem + kLmSmem)[tid * KB + KB - 1], b ? (b << 16) - 1u : 0u);
          if (t == 0u) *s_over = 1u;              // no threshold yet: stage the tile
        }
        s_thr[tid] = t;
        s_cnt[tid] = 0u;
      }
      __syncthreads();
      // the flag is one LDS word read by every thread after a barrier: uniform
      if (__builtin_amdgcn_readfirstlane(*s_over) == 0u) {
        // lane-dependent values are derived here from an opaque copy of the
        // thread index, so the compiler forms them per tile instead of
        // keeping them across the tile product (where they would spill)
        uint32_t tq = (uint32_t)tid;
        asm volatile("" : "+v"(tq));
        const int wave = tid >> 6, lane = (int)(tq & 63u);
        const int wm = (wave / LmCfg::kWavesN) * LmCfg::kWM, wn = (wave % LmCfg::kWavesN) * LmCfg::kWN;
        uint32_t* s_cand = reinterpret_cast<uint32_t*>(lm_smem);
        // A pre-filter over the packed values: pk[i][j][h] holds rows
        // r4 + 2h (low half) and r4 + 2h + 1 (high half) of fragment row i
        // at column j.  For a strictly positive threshold value a value can
        // only pass if its bf16 bits, read as a signed 16-bit integer, are
        // >= the threshold's (negative values are negative integers), so the
        // packed signed maximum over the four columns against the packed
        // thresholds flags the row pairs worth an exact look (ties included;
        // any other threshold flags its pair).
        u32x4 t4[kFragM];
#pragma unroll
        for (int i = 0; i < kFragM; ++i) t4[i] = ld16(s_thr + wm + 16 * i + 4 * (lane >> 4));
        uint32_t flags = 0u;                     // bit 2 i + h: row pair (i, h) has a candidate
#pragma unroll
        for (int i = 0; i < kFragM; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t ka = t4[i][2 * h] >> 16, kb = t4[i][2 * h + 1] >> 16;
            const i16x2 thm = {(short)((ka & 0x7fffu) - 1u), (short)((kb & 0x7fffu) - 1u)};
            i16x2 mx = __builtin_bit_cast(i16x2, pk[i][0][h]);
#pragma unroll
            for (int j = 1; j < kFragN; ++j) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(i16x2, pk[i][j][h]));
            const i16x2 m2 = __builtin_elementwise_max(mx, thm);
            const bool above = __builtin_bit_cast(uint32_t, m2) != __builtin_bit_cast(uint32_t, thm);
            flags |= ((ka > 0x8000u && kb > 0x8000u) ? above : true) ? (1u << (2 * i + h)) : 0u;
          }
        // the exact test for flagged pairs: group key against the row's
        // threshold, valid columns only, then an LDS slot in the row's buffer
#pragma unroll
        for (int i = 0; i < kFragM; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if ((flags >> (2 * i + h)) & 1u) {
              // opaque copies: keys and addresses are formed here, not
              // hoisted out of the tile loop and kept (or spilled)
              uint32_t lq = (uint32_t)tid, w[kFragN];
#pragma unroll
              for (int j = 0; j < kFragN; ++j) w[j] = pk[i][j][h];
              asm volatile("" : "+v"(lq), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
              const uint32_t l = lq & 63u, wv = lq >> 6;
              const uint32_t r0 = (wv / LmCfg::kWavesN) * LmCfg::kWM + (uint32_t)(16 * i + 2 * h) + 4u * (l >> 4);
#pragma unroll
              for (int j = 0; j < kFragN; ++j) {
                const uint32_t tc = (wv % LmCfg::kWavesN) * LmCfg::kWN + (uint32_t)(16 * j) + (l & 15u);
                const uint32_t ck = 0xFFFFu - ((uint32_t)cg0 + tc);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                  const uint32_t c = (bf16_key(e ? (w[j] >> 16) : (w[j] & 0xffffu)) << 16) | ck;
                  if (n0 + (int)tc < valid && c > t4[i][2 * h + e]) {
                    const uint32_t slot = atomicAdd(s_cnt + r0 + e, 1u);
                    if (slot < (uint32_t)kRowCap) s_cand[(r0 + e) * kRowCap + slot] = c;
                  }
                }
              }
            }
          }
        __syncthreads();
        if (tid < kBM && s_cnt[tid] > (uint32_t)kRowCap) *s_over = 1u;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(*s_over) == 0u) {
          if (part == 0 && row_ok) {
            uint32_t tl[KB];
#pragma unroll
            for (int i = 0; i < KB; ++i) tl[i] = glist[i];
            const uint32_t lo_r = __hip_atomic_load(bound + m0 + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int n = (int)s_cnt[row];
            for (int e = 0; e < n; ++e) {
              const uint32_t c = s_cand[row * kRowCap + e];
              if (c > tl[KB - 1]) list_insert(tl, c);
            }
#pragma unroll
            for (int i = 0; i < KB; ++i) glist[i] = tl[i];
            if (tl[KB - 1] != 0u && (tl[KB - 1] >> 16) > lo_r)
              __hip_atomic_fetch_max(bound + m0 + row, tl[KB - 1] >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __syncthreads();                       // the buffers lie in the ring the next tile refills
          continue;
        }
      }
    }
    uint32_t lo = 0;
    if (row_ok) lo = __hip_atomic_load(bound + m0 + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t gk = glist[KB - 1];           // the group list's K-th (0 until it holds K)
    uint32_t tl[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) tl[i] = part == 0 ? glist[i] : ((i < KB - K) ? ~0u : 0u);
    for (int pass = 0; pass < kOutPasses; ++pass) {
      tile_to_lds<LmCfg>(pk, cs, pass);
      __syncthreads();
      const int t_lo = pass * kOutCols + kScanCols * part;   // first column within the tile
      if (row_ok && n0 + t_lo < valid) {
        const uint16_t* rowp = cs + row * kCPad + kScanCols * part;
        uint32_t* cand = reinterpret_cast<uint32_t*>(lm_smem + kCandOff) + tid * kCandCap;
        int n_cand = 0;
        // a value is appended when its full key (value, then column) beats
        // the thread's list and the group list: stale between flushes, so
        // it lets more through, never fewer; bf16 values tie often, so the
        // column takes part in the test
        uint32_t thr = max(tl[KB - 1], gk);
        auto flush = [&]() {
          for (int i = 0; i < n_cand; ++i) {
            const uint32_t c = cand[i];
            if (c > tl[KB - 1]) list_insert(tl, c);
          }
          n_cand = 0;
          thr = max(tl[KB - 1], gk);
        };
#pragma unroll 2
        for (int c8 = 0; c8 < kScanCols; c8 += 8) {
          if (n0 + t_lo + c8 >= valid) break;
          const u32x4 v = ld16(rowp + c8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tc = t_lo + c8 + e;
            const uint32_t key = bf16_key((e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu));
            const uint32_t c = group_key(key, cg0 + tc);
            if (key >= lo && n0 + tc < valid && c > thr) cand[n_cand++] = c;
          }
          if (n_cand > kCandCap - 8) flush();       // room for the next 8 values
        }
        flush();
      }
      __syncthreads();                         // the pass's LDS is reused next
    }
    // row merge: the other threads' lists to LDS, the p = 0 thread folds them
    // into its list (the group list and this thread's values) and stores it
    uint32_t* xch = reinterpret_cast<uint32_t*>(lm_smem);   // [kBM][kRowThreads - 1][KB], in the ring
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
#pragma unroll
      for (int i = 0; i < KB; ++i) glist[i] = tl[i];
      if (tl[KB - 1] != 0u && (tl[KB - 1] >> 16) > lo)
        __hip_atomic_fetch_max(bound + m0 + row, tl[KB - 1] >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();                           // xch lies in the ring the next tile refills
  }
  if (part == 0 && row_ok) {
    uint64_t* dst = parts + ((int64_t)(m0 + row) * n_grp + grp) * K;
    for (int i = KB - K; i < KB; ++i) {
      const uint32_t c = glist[i];
      dst[i - (KB - K)] = c == 0u ? 0ull : group_key_composite(c, nb0 * kBN);
    }
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
  // groups of column tiles per workgroup: about 4096 workgroups (16 per CU,
  // one resident at a time), so that a group's later tiles are filtered by
  // its own list and the per-row bound; at least enough tiles that a row's
  // merge candidates fit (K threads of the merge, ceil(n_grp / 256) lists of
  // K each); a group spans at most 65536 columns
  int t = 1;
  while ((int64_t)top_k * top_k * (((p.n_nb + t - 1) / t + 255) / 256) > kLmMergeCand) ++t;
  const int64_t tiles = (int64_t)p.n_mb * p.n_nb;
  const int t_par = (int)(tiles / 4096);
  if (t_par > t) t = t_par;
  if (t > kMaxGroupCols / kBN) t = kMaxGroupCols / kBN;
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
  const dim3 grid((unsigned)grouped_grid(p.n_mb, p.n_grp));
#define DFLASH_LMTK(KB)                                                                                    \
  hipLaunchKernelGGL((lm_head_topk_kernel<KB>), grid, dim3(kLmThreads), lm_topk_smem<KB>(), stream,     \
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
  hipLaunchKernelGGL(lm_head_kernel, dim3((unsigned)grouped_grid(n_mb, n_nb)), dim3(kLmThreads), kLmSmem, stream,
                     static_cast<const uint16_t*>(a.hidden), a.hidden_row_stride,
                     static_cast<const uint16_t*>(a.weight), (int32_t)a.n_rows, a.hidden_size, (int32_t)a.vocab,
                     static_cast<uint16_t*>(a.logits), a.logits_row_stride, n_mb, n_nb);
  return hipGetLastError();
}

}  // namespace dflash

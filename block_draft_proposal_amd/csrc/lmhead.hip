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

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLmThreads = 256;
constexpr int kRowPad = kBK + 8;            // bf16 elements per LDS row of a stage
constexpr int kCPad = kBN + 8;              // bf16 elements per LDS row of the output tile

struct LmSmem {
  uint16_t a[2][kBM * kRowPad];
  uint16_t b[2][kBN * kRowPad];
};
static_assert(sizeof(uint16_t) * kBM * kCPad <= sizeof(uint16_t) * 2 * kBM * kRowPad, "output tile fits in A");

// Workgroup -> (row block, column block).  Consecutive workgroups go to
// consecutive XCDs; the n_mb row blocks of one column block get ids that
// are equal modulo 8, so they share an XCD (and its L2).
__device__ __forceinline__ void tile_of(int id, int n_mb, int& mb, int& nb) {
  const int xcd = id & 7, slot = id >> 3;
  nb = (slot / n_mb) * 8 + xcd;
  mb = slot % n_mb;
}

// Stage loads: rows [r0, r0 + 128) x k [k0, k0 + 64) of a [rows, H] matrix,
// as 1024 16-byte chunks, 4 per thread (chunk c: row c / 8, k offset 8 (c % 8)).
// Loads are unconditional at clamped addresses; chunks outside the matrix
// become zero afterwards.
__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ base, int64_t stride, int rows, int H,
                                           int r0, int k0, int tid, u32x4 (&v)[4]) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + kLmThreads * q;
    const int row = r0 + (c >> 3), k = k0 + 8 * (c & 7);
    const u32x4 x = ld16(base + (int64_t)min(row, rows - 1) * stride + min(k, H - 8));
    v[q] = (row < rows && k < H) ? x : zero;
  }
}

__device__ __forceinline__ void store_stage(uint16_t* __restrict__ s, int tid, const u32x4 (&v)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + kLmThreads * q;
    st16(s + (c >> 3) * kRowPad + 8 * (c & 7), v[q]);
  }
}

// The 128 x 128 fp32 tile of (mb, nb), in the wave's 4 x 4 accumulators.
// D layout of one 16 x 16 MFMA: lane l holds column l % 16 and rows
// 4 (l / 16) + v, v = 0..3.
__device__ __forceinline__ void tile_product(const uint16_t* __restrict__ h, int64_t h_stride,
                                             const uint16_t* __restrict__ W, int M, int H, int V, int m0, int n0,
                                             LmSmem& sm, f32x4_t (&acc)[4][4]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk = (H + kBK - 1) / kBK;
  u32x4 ra[4], rb[4];
  load_stage(h, h_stride, M, H, m0, 0, tid, ra);
  load_stage(W, H, V, H, n0, 0, tid, rb);
  store_stage(sm.a[0], tid, ra);
  store_stage(sm.b[0], tid, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_stage(h, h_stride, M, H, m0, (kt + 1) * kBK, tid, ra);
      load_stage(W, H, V, H, n0, (kt + 1) * kBK, tid, rb);
    }
    const uint16_t* sa = sm.a[cur];
    const uint16_t* sb = sm.b[cur];
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 32) {
      bf16x8_t af[4], bfrag[4];
      const int kofs = ks + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, ld16(sa + (wm + 16 * i + (lane & 15)) * kRowPad + kofs));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfrag[j] = __builtin_bit_cast(bf16x8_t, ld16(sb + (wn + 16 * j + (lane & 15)) * kRowPad + kofs));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfrag[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_stage(sm.a[cur ^ 1], tid, ra);
      store_stage(sm.b[cur ^ 1], tid, rb);
    }
    __syncthreads();
  }
}

// Rounds the wave's accumulators to bf16 into the output tile in LDS.
__device__ __forceinline__ void tile_to_lds(const f32x4_t (&acc)[4][4], uint16_t* cs) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        cs[(wm + 16 * i + 4 * (lane >> 4) + v) * kCPad + wn + 16 * j + (lane & 15)] =
            (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
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
  f32x4_t acc[4][4];
  tile_product(h, h_stride, W, M, H, V, m0, n0, sm, acc);

  // round to bf16 into LDS, then write whole 16-byte row pieces
  const int tid = threadIdx.x;
  uint16_t* cs = sm.a[0];
  tile_to_lds(acc, cs);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < (kBM * kBN / 8) / kLmThreads; ++q) {
    const int c = tid + kLmThreads * q;
    const int row = c >> 4, col = 8 * (c & 15);
    if (m0 + row >= M) continue;
    uint16_t* dst = logits + (int64_t)(m0 + row) * l_stride + n0 + col;
    const uint16_t* src = cs + row * kCPad + col;
    if (n0 + col + 8 <= V) {
      st16(dst, ld16(src));
    } else {
      for (int e = 0; e < 8 && n0 + col + e < V; ++e) dst[e] = src[e];
    }
  }
}

// KB: list slots (K rounded up to 8, 16 or 32).  The list holds KB - K
// sentinels (all ones, above every composite) ahead of the K real entries,
// so the threshold is always the last slot and no index depends on K.
template <int KB>
__device__ __forceinline__ void list_insert(uint64_t (&best)[KB], uint64_t c) {
#pragma unroll
  for (int i = 0; i < KB; ++i) {                 // keeps the list sorted descending
    if (c > best[i]) { const uint64_t t = best[i]; best[i] = c; c = t; }
  }
}

static_assert(sizeof(uint64_t) * kBM * 32 <= sizeof(LmSmem), "pair exchange fits the stage buffers");

// Two threads per row: thread t takes row t / 2 and the 64 columns of half
// t % 2 of every tile of its group, keeping its own sorted list; at the end
// the pair's lists meet in LDS and the even thread writes their merge.
template <int KB>
__global__ __launch_bounds__(kLmThreads) void lm_head_topk_kernel(
    const uint16_t* __restrict__ h, int64_t h_stride, const uint16_t* __restrict__ W, int32_t M, int32_t H,
    int32_t V, int32_t valid, int32_t K, int32_t n_mb, int32_t n_nb, int32_t tiles_per_group, int32_t n_grp,
    uint64_t* __restrict__ parts) {
  extern __shared__ __align__(16) unsigned char lm_smem[];
  LmSmem& sm = *reinterpret_cast<LmSmem*>(lm_smem);
  int mb, grp;
  tile_of(blockIdx.x, n_mb, mb, grp);
  if (grp >= n_grp) return;
  const int m0 = mb * kBM, tid = threadIdx.x;
  const int row = tid >> 1, half = tid & 1;
  const bool row_ok = m0 + row < M;
  uint64_t best[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i) best[i] = (i < KB - K) ? ~0ull : 0ull;
  const int nb0 = grp * tiles_per_group, nb1 = min(n_nb, nb0 + tiles_per_group);
  uint16_t* cs = sm.a[0];
  for (int nb = nb0; nb < nb1; ++nb) {
    const int n0 = nb * kBN;
    f32x4_t acc[4][4];
    tile_product(h, h_stride, W, M, H, V, m0, n0, sm, acc);   // ends with a barrier
    tile_to_lds(acc, cs);
    __syncthreads();
    if (row_ok) {
      const uint16_t* rowp = cs + row * kCPad + 64 * half;
      const int c_lo = n0 + 64 * half;
#pragma unroll 2
      for (int c8 = 0; c8 < 64; c8 += 8) {
        if (c_lo + c8 >= valid) break;
        const u32x4 v = ld16(rowp + c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = c_lo + c8 + e;
          const uint32_t bits = (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
          const uint64_t c = composite(bf16_key(bits), col);
          if (col < valid && c > best[KB - 1]) list_insert(best, c);
        }
      }
    }
    __syncthreads();                           // the tile's LDS is reused by the next stage
  }
  // pair merge: the odd thread's list to LDS, the even thread folds it in
  uint64_t* xch = reinterpret_cast<uint64_t*>(lm_smem);      // [128 rows][KB], after the last barrier
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < KB; ++i) xch[row * KB + i] = best[i];
  }
  __syncthreads();
  if (half == 0 && row_ok) {
#pragma unroll
    for (int i = KB - 1; i >= 0; --i) {
      const uint64_t c = xch[row * KB + i];
      if (c != ~0ull && c > best[KB - 1]) list_insert(best, c);
    }
    uint64_t* dst = parts + ((int64_t)(m0 + row) * n_grp + grp) * K;
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (i >= KB - K) dst[i - (KB - K)] = best[i];
  }
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
  p.bytes = (size_t)n_rows * p.n_grp * top_k * sizeof(uint64_t);
  p.bytes = (p.bytes + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_lm_head_topk(const LmHeadArgs& a, const LmTopkPlan& p, int64_t valid_vocab, int32_t top_k,
                               float mult, float cap, int64_t* ids_out, float* unary_out, void* workspace,
                               hipStream_t stream) {
  if (a.n_rows == 0) return hipSuccess;
  uint64_t* parts = static_cast<uint64_t*>(workspace);
  const int64_t slots = (int64_t)((p.n_grp + 7) / 8) * p.n_mb;
  const dim3 grid((unsigned)(slots * 8));
#define DFLASH_LMTK(KB)                                                                                    \
  hipLaunchKernelGGL((lm_head_topk_kernel<KB>), grid, dim3(kLmThreads), sizeof(LmSmem), stream,                \
                     static_cast<const uint16_t*>(a.hidden), a.hidden_row_stride,                          \
                     static_cast<const uint16_t*>(a.weight), (int32_t)a.n_rows, a.hidden_size,             \
                     (int32_t)a.vocab, (int32_t)valid_vocab, top_k, p.n_mb, p.n_nb, p.tiles_per_group,     \
                     p.n_grp, parts)
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

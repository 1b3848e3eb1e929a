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
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  uint16_t* cs = sm.a[0];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        cs[(wm + 16 * i + 4 * (lane >> 4) + v) * kCPad + wn + 16 * j + (lane & 15)] =
            (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
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

}  // namespace

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

// Candidate selector on gfx950: rank-r projection, lattice and walk.
//
// Operations ("[Spec] DFlash2: local convolution + candidate selector"):
//   executive summary -- edge(p -> c) = <A[p] (.) project(h), B[c]> + unary[c]
//   scored over adjacent slots, slot 0's predecessor being the verified anchor
//   (draft-sampler excerpt: block position 0 is the anchor);
//   walk-kernel excerpt -- one program per request, a serial loop over slots
//   starting from row 0: greedy rows take the argmax (lowest index among ties)
//   and emit a one-hot q, sampled rows draw by inverse CDF from a supplied
//   uniform and emit the softmax q they drew from.
//
// Kernels
//  * Projection u = P h for every slot row, the one dense contraction on the
//    path, on the matrix cores (v_mfma_f32_16x16x32_bf16; bf16 x bf16
//    products are exact in fp32), split over slices of the hidden axis whose
//    partials the consumer adds in a fixed order (deterministic):
//    proj_mfma_kernel (few rows: a wave owns 16 rows x all rank columns of one
//    slice) and proj_tile_kernel (2048 slot rows or more: LDS-staged 128 x 128
//    tiles of the shared tile product, gemm_tile.h).  Each output is the same
//    MFMA chain over its slice's 32-wide k steps whatever the grouping, so the
//    two agree with the propose step's fused projection bit for bit.
//    proj_f32_kernel is the fp32-storage path (VALU fma chain).
//  * The lattice block of one slot on one wave's matrix cores (tile_mfma):
//    w = A[p] (.) u in fp32, then against B[c] -- fp32 tables by fp32 MFMA
//    steps, bf16 tables by two bf16 MFMA steps per 8 k values (w split into a
//    bf16 hi and lo part), every term within 2^-18 of A u B.  Kernels:
//    lattice_mfma_kernel (standalone: one wave per slot row),
//    lattice_walk_kernel (one workgroup per request, the lattice in LDS, then
//    every row decided in parallel and the path found by pointer jumping),
//    lattice_walk_wave_kernel (one wave per request for large batches: only
//    the walked rows are decided, slot by slot, pipelined).
//  * walk_kernel / walk_lds_kernel: the standalone walk over given scores.
// Every lattice and walk evaluation runs the same arithmetic, so the fused
// kernels equal dflash_lattice followed by dflash_walk bit for bit.
#include "dflash.h"
#include "dflash_internal.h"
#include "conv_core.h"
#include "gemm_tile.h"

namespace dflash {
namespace {


constexpr int kThreads = 256;
constexpr int kRowsPerWG = 64;       // 4 waves x 16 rows
constexpr int kProjUnroll = 4;       // projection k-steps whose loads are issued together

// Exact n / d for 0 <= n, d < 2^16 (d >= 1) by one multiply-high:
// q = (n * ceil(2^32 / d)) >> 32.  The error n * (M d - 2^32) / (d 2^32) is
// below 1/d, so the floor is exact.
struct FastDiv {
  uint64_t m;   // ceil(2^32 / d) = floor((2^32 - 1) / d) + 1, by a 32-bit division
  __device__ explicit FastDiv(int d) : m((uint64_t)(0xFFFFFFFFu / (uint32_t)d) + 1) {}
  __device__ int quot(int n) const { return (int)(((uint64_t)(uint32_t)n * m) >> 32); }
};

__device__ __forceinline__ const void* hidden_row(const void* hidden, int64_t req_stride,
                                                  int64_t slot_stride, int32_t slots, int row,
                                                  int elem_bytes) {
  const int req = row / slots, s = row % slots;
  return static_cast<const char*>(hidden) + ((int64_t)req * req_stride + (int64_t)s * slot_stride) * elem_bytes;
}

// RT = column tiles of 16 per wave (rank <= 16 * RT); FR = row fragments of
// 16 per wave, so that each wave reuses every P fragment it loads for FR
// MFMAs (P is read from cache once per 16 * FR rows instead of per 16).  A
// workgroup covers 64 * FR rows, all rank columns and one slice of H.
template <int RT, int FR>
__global__ __launch_bounds__(kThreads) void proj_mfma_kernel(const uint16_t* __restrict__ hidden,
                                                             int64_t req_stride, int64_t slot_stride,
                                                             int32_t slots, const uint16_t* __restrict__ P,
                                                             int32_t n_rows, int32_t rank, int32_t H,
                                                             int32_t kslice, float* __restrict__ u_parts) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_base = (blockIdx.x * 4 + wave) * 16 * FR;
  const int split = blockIdx.y;
  const int k0 = split * kslice;
  const int k1 = min(H, k0 + kslice);
  const int kofs = 8 * (lane >> 4);
  const uint16_t* hrow[FR];
  bool arow_ok[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int arow = row_base + 16 * f + (lane & 15);
    arow_ok[f] = arow < n_rows;
    hrow[f] = arow_ok[f] ? static_cast<const uint16_t*>(hidden_row(hidden, req_stride, slot_stride, slots, arow, 2))
                         : hidden;
  }
  f32x4_t acc[FR][RT];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // kProjUnroll k-steps per round: every load of the round is issued (at an
  // address clamped into the slice and the table) before the first MFMA;
  // operands past the slice, the rows or the rank are zeroed afterwards, so
  // each output is the same MFMA chain over the slice's k-steps in order,
  // whatever FR is.
  constexpr int U = FR > 1 ? 2 : kProjUnroll;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int kk = k0; kk < k1; kk += 32 * U) {
    u32x4 av[U][FR], bv[U][RT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = min(kk + 32 * u + kofs, k1 - 8);
#pragma unroll
      for (int f = 0; f < FR; ++f) av[u][f] = ld16(hrow[f] + kc);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int col = min(t * 16 + (lane & 15), rank - 1);
        bv[u][t] = ld16(P + (int64_t)col * H + kc);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool k_ok = kk + 32 * u + kofs < k1;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bool c_ok = t * 16 + (lane & 15) < rank;
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, (c_ok && k_ok) ? bv[u][t] : zero);
#pragma unroll
        for (int f = 0; f < FR; ++f) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (arow_ok[f] && k_ok) ? av[u][f] : zero);
          acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[f][t], 0, 0, 0);
        }
      }
    }
  }
  // D layout: lane holds column (lane & 15), rows 4 * (lane >> 4) + v.
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int col = t * 16 + (lane & 15);
    if (col >= rank) continue;
#pragma unroll
    for (int f = 0; f < FR; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row_base + 16 * f + 4 * (lane >> 4) + v;
        if (row < n_rows) u_parts[proj_part_index(split, n_rows, rank, row, col)] = acc[f][t][v];
      }
  }
}


// Large batches: the projection as 128 x 128 output tiles of the shared
// tile product (gemm_tile.h: direct global -> LDS stages, 64-deep k blocks,
// v_mfma_f32_16x16x32_bf16 with operand lane groups at k + 8 (lane >> 4),
// k-steps in order), over one slice of the contraction per workgroup.  Each
// output is the MFMA chain over its slice's k-steps from zero, exactly as in
// proj_mfma_kernel and the conv + slot projection, so every producer of the
// partials agrees bit for bit.  Rank columns past `rank` repeat the last P
// row and are not stored.
using ProjTileCfg = TileCfg<4, 4, 2, 2, 64, 2>;

// Slot row n of a request-major [R][S] view with strides in elements.
struct SlotRows {
  static constexpr int kAux = kBufferStream;        // each slot row is read once: streaming loads
  const uint16_t* h;
  int64_t req_stride, slot_stride;
  int32_t slots;
  __device__ __forceinline__ const uint16_t* operator()(int n) const {
    const int req = n / slots, s = n - req * slots;
    return h + (int64_t)req * req_stride + (int64_t)s * slot_stride;
  }
};

__global__ __launch_bounds__(ProjTileCfg::kThreads) void proj_tile_kernel(
    const uint16_t* __restrict__ hidden, int64_t req_stride, int64_t slot_stride, int32_t slots,
    const uint16_t* __restrict__ P, int32_t n_rows, int32_t rank, int32_t H, int32_t kb_per_slice,
    float* __restrict__ u_parts) {
  typedef ProjTileCfg Cfg;
  extern __shared__ __align__(16) unsigned char pt_smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.y;
  const int nk = (H + Cfg::kBK - 1) / Cfg::kBK;
  const int kb0 = split * kb_per_slice;
  const int nkb = min(kb_per_slice, nk - kb0);
  const int m0 = blockIdx.x * Cfg::kBM;
  f32x4_t acc[Cfg::kFragM][Cfg::kFragN];
  tile_product<Cfg>(SlotRows{hidden, req_stride, slot_stride, slots}, StridedRows{P, H}, n_rows, rank, H, m0, 0,
                    kb0, nkb, pt_smem, acc);
  const int wm = (wave / Cfg::kWavesN) * Cfg::kWM, wn = (wave % Cfg::kWavesN) * Cfg::kWN;
#pragma unroll
  for (int j = 0; j < Cfg::kFragN; ++j) {
    const int col = wn + 16 * j + (lane & 15);
    if (col >= rank) continue;
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm + 16 * i + 4 * (lane >> 4) + v;
        if (row < n_rows) u_parts[proj_part_index(split, n_rows, rank, row, col)] = acc[i][j][v];
      }
  }
}

__global__ __launch_bounds__(kThreads) void proj_f32_kernel(const float* __restrict__ hidden,
                                                            int64_t req_stride, int64_t slot_stride,
                                                            int32_t slots, const float* __restrict__ P,
                                                            int32_t n_rows, int32_t rank, int32_t H,
                                                            float* __restrict__ u_parts) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (int64_t)n_rows * rank) return;
  const int row = (int)(t / rank), col = (int)(t % rank);
  const float* h = static_cast<const float*>(hidden_row(hidden, req_stride, slot_stride, slots, row, 4));
  const float* p = P + (int64_t)col * H;
  float acc = 0.f;
  for (int k = 0; k < H; ++k) acc = fmaf(h[k], p[k], acc);
  u_parts[t] = acc;                                    // one slice: [0][row][col]
}

// u[n][k] = sum over the projection slices sp = 0..ksplit-1 of the partial
// u_parts[sp][n][k] (slice-major, n_rows slot rows per slice), added in slice
// order.  load_proj_slices issues every load of the value before
// add_proj_slices uses the first, so callers can put other loads between the
// two and pay one memory round trip for all.
__device__ __forceinline__ void load_proj_slices(const float* __restrict__ u_parts, int ksplit, int64_t n_rows,
                                                 int r, int64_t n, int k, float (&v)[kMaxProjSplit]) {
  const float* base = u_parts + n * r + k;
  const int64_t slice = n_rows * r;
  // every load unconditional (a slot past the last slice re-reads it), so
  // none waits for another
#pragma unroll
  for (int q = 0; q < kMaxProjSplit; ++q) v[q] = base[(q < ksplit ? q : ksplit - 1) * slice];
}

__device__ __forceinline__ float add_proj_slices(const float (&v)[kMaxProjSplit], int ksplit) {
  float u = v[0];
#pragma unroll
  for (int q = 1; q < kMaxProjSplit; ++q)
    if (q < ksplit) u += v[q];
  return u;
}

__device__ __forceinline__ float sum_proj_slices(const float* __restrict__ u_parts, int ksplit, int64_t n_rows,
                                                 int r, int64_t n, int k) {
  float v[kMaxProjSplit];
  load_proj_slices(u_parts, ksplit, n_rows, r, n, k, v);
  return add_proj_slices(v, ksplit);
}


// ---------------------------------------------------------------------------
// The K x K lattice block of one slot as one fp32 matrix-core tile.
//
// scores[j][c] = sum_k w[j][k] B[c][k] + unary[c],  w[j] = A[pred_j] (.) u
// is a (K x r) by (r x K) product: one v_mfma_f32_16x16x4_f32 tile for
// K <= 16, one v_mfma_f32_32x32x2_f32 tile for K <= 32.  Lane l serves row /
// column e = l % MT (predecessor row j of the A operand, candidate c of the B
// operand) and k-group g = l / MT of G = 64 / MT groups; group g owns the
// contiguous range k in [g L, g L + L) (L a multiple of the 16-byte vector,
// G L >= r; k >= r enters as zero), so each lane gathers one contiguous
// piece of its two table rows with 16-byte loads.  MFMA step kk takes
// k = g L + kk from every group.  Operands are fp32 (A * u rounded once to
// fp32, B exact), never bf16: rounding A (.) u to bf16 would blur near-ties.
// Every lattice evaluation (standalone or fused with the walk) runs this same
// sequence, so they agree bit for bit.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int MT> struct LatTile;
template <> struct LatTile<16> {
  typedef f32x4_t acc_t;
  static constexpr int kAcc = 4;
  __device__ static acc_t mfma(float a, float b, acc_t c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
  __device__ static acc_t mfma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // row of accumulator i in this lane (its column is lane % 16)
  __device__ static int row(int lane, int i) { return 4 * (lane >> 4) + i; }
};
template <> struct LatTile<32> {
  typedef f32x16_t acc_t;
  static constexpr int kAcc = 16;
  __device__ static acc_t mfma(float a, float b, acc_t c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
  __device__ static acc_t mfma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int row(int lane, int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
};

// Tile size and k-range length per lane group for K candidates, rank r and
// `vec` elements per 16-byte vector (the shape every kernel and the host use).
__host__ __device__ inline int lattice_mt(int K) { return K <= 16 ? 16 : 32; }
__host__ __device__ inline int lattice_group_len(int K, int r, int vec) {
  const int G = 64 / lattice_mt(K);
  return (r + G * vec - 1) / (G * vec) * vec;
}
// k extent of the padded u row (G L floats, zeros past r).
__host__ __device__ inline int lattice_kpad(int K, int r, int vec) {
  return (64 / lattice_mt(K)) * lattice_group_len(K, r, vec);
}

// Table rows are gathered with 16-byte loads when every row and the tables
// are 16-byte aligned; otherwise element by element into the same packed
// vectors (odd ranks), with the same arithmetic afterwards.
template <typename TIO>
__device__ __forceinline__ u32x4 gather_piece(const TIO* __restrict__ row, int k, int r, bool vload) {
  constexpr int VEC = Elem<TIO>::kVec;
  if (vload) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    return k < r ? ld16(row + k) : zero;          // a vector lies wholly inside or past r
  }
  TIO e[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) e[i] = (k + i < r) ? row[k + i] : TIO(0);
  return *reinterpret_cast<const u32x4*>(e);
}

// The two table rows a lane gathers for one slot: A[pred] and B[cand]
// (row 0 for an id outside [0, vocab), whose products become NaN).
template <typename TIO>
struct TileRows {
  const TIO* arow;
  const TIO* brow;
  bool pok, cok;
};
template <typename TIO>
__device__ __forceinline__ TileRows<TIO> tile_rows(const TIO* __restrict__ A, const TIO* __restrict__ B,
                                                   int64_t vocab, int r, int64_t pred, int64_t cand) {
  TileRows<TIO> t;
  t.pok = pred >= 0 && pred < vocab;
  t.cok = cand >= 0 && cand < vocab;
  t.arow = A + (t.pok ? pred : 0) * (int64_t)r;
  t.brow = B + (t.cok ? cand : 0) * (int64_t)r;
  return t;
}

// Gathers pieces v0 .. v0 + NB - 1 (those below nv) of the lane's k-range
// (starting at kg) of both rows.
template <typename TIO, int NB>
__device__ __forceinline__ void tile_gather(const TileRows<TIO>& t, int kg, int v0, int nv, int r, bool vload,
                                            u32x4 (&av)[NB], u32x4 (&bv)[NB]) {
  constexpr int VEC = Elem<TIO>::kVec;
#pragma unroll
  for (int v = 0; v < NB; ++v) {
    if (v0 + v < nv) {
      av[v] = gather_piece(t.arow, kg + (v0 + v) * VEC, r, vload);
      bv[v] = gather_piece(t.brow, kg + (v0 + v) * VEC, r, vload);
    }
  }
}

// The MFMA steps of those pieces.  fp32 tables: one v_mfma_f32_*_f32 step
// per k = kg + (v0 + v) VEC + e, in order, with w = A * u rounded to fp32
// (NaN for an out-of-range predecessor) against B (NaN for an out-of-range
// candidate).  bf16 tables: w (the same fp32 product) is split as
// hi = bf16(w), lo = bf16(w - hi) (w - hi is exact in fp32), and each 16-byte
// piece of 8 k values takes two bf16 MFMA steps, hi x B then lo x B: bf16 x
// bf16 products are exact in fp32 and hi + lo carries w to within
// 2^-18 |w|, so every term is within 2^-18 of A u B (a single bf16 rounding
// of w would be 2^-9).  The 8 k values of a piece sit in the instruction's k
// positions 8 g .. 8 g + 7 of lane group g, in order.
template <typename TIO, int MT, int NB>
__device__ __forceinline__ void tile_mfma(typename LatTile<MT>::acc_t& acc, const u32x4 (&av)[NB],
                                          const u32x4 (&bv)[NB], bool pok, bool cok, int kg, int v0, int nv,
                                          const float* s_u) {
  constexpr int VEC = Elem<TIO>::kVec;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int v = 0; v < NB; ++v) {
    if (v0 + v < nv) {
      float a[VEC];
      unpack16(av[v], a);
      const float* u = s_u + kg + (v0 + v) * VEC;
      float w[VEC];
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const float4 u4 = *reinterpret_cast<const float4*>(u + e);
        w[e] = a[e] * u4.x;                                         // A[p] (.) project(h)
        w[e + 1] = a[e + 1] * u4.y;
        w[e + 2] = a[e + 2] * u4.z;
        w[e + 3] = a[e + 3] * u4.w;
      }
      if constexpr (sizeof(TIO) == 2) {
        u32x4 hi, lo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hi[q] = pack_bf16x2(w[2 * q], w[2 * q + 1]);
          const float r0 = w[2 * q] - __uint_as_float(hi[q] << 16);
          const float r1 = w[2 * q + 1] - __uint_as_float(hi[q] & 0xffff0000u);
          lo[q] = pack_bf16x2(r0, r1);
        }
        const u32x4 qnan = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, cok ? bv[v] : qnan);
        acc = LatTile<MT>::mfma(__builtin_bit_cast(bf16x8_t, pok ? hi : qnan), b, acc);
        acc = LatTile<MT>::mfma(__builtin_bit_cast(bf16x8_t, pok ? lo : qnan), b, acc);
      } else {
        float b[VEC];
        unpack16(bv[v], b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = LatTile<MT>::mfma(pok ? w[e] : nan, cok ? b[e] : nan, acc);
      }
    }
  }
}

// One slot's tile on one wave.  pred / cand: this lane's predecessor and
// candidate token ids (lanes past K pass any in-range id; their rows and
// columns are not used); s_u: the slot's u, G L floats (zeros past r), in LDS.
// An id outside [0, vocab) turns its whole row (pred) or column (cand) NaN.
// NB: 16-byte pieces of each table row gathered per round (register budget
// only: the MFMA sequence is the same for every NB).
template <typename TIO, int MT, int NB>
__device__ __forceinline__ typename LatTile<MT>::acc_t lattice_slot_tile(
    const TIO* __restrict__ A, const TIO* __restrict__ B, int64_t vocab, int r, int L, bool vload, int64_t pred,
    int64_t cand, const float* s_u) {
  constexpr int VEC = Elem<TIO>::kVec;
  const int lane = threadIdx.x & 63;
  const int kg = (lane / MT) * L;
  const TileRows<TIO> t = tile_rows(A, B, vocab, r, pred, cand);
  typename LatTile<MT>::acc_t acc = {};
  const int nv = L / VEC;
  for (int v0 = 0; v0 < nv; v0 += NB) {
    u32x4 av[NB], bv[NB];
    tile_gather<TIO, NB>(t, kg, v0, nv, r, vload, av, bv);
    tile_mfma<TIO, MT, NB>(acc, av, bv, t.pok, t.cok, kg, v0, nv, s_u);
  }
  return acc;
}

// Stores one slot's tile plus unary: row j, column c of the block goes to
// dst[j * row_stride + c] (global or LDS); rows and columns past K are not
// stored.  un: the slot's unary [K] (global).
template <int MT>
__device__ __forceinline__ void lattice_store(const typename LatTile<MT>::acc_t& acc, const float* __restrict__ un,
                                              int K, float* dst, int row_stride) {
  const int lane = threadIdx.x & 63;
  const int c = lane % MT;
  if (c >= K) return;
  const float uc = un[c];
#pragma unroll
  for (int i = 0; i < LatTile<MT>::kAcc; ++i) {
    const int j = LatTile<MT>::row(lane, i);
    if (j < K) dst[j * row_stride + c] = acc[i] + uc;
  }
}

// Standalone lattice: one wave per slot row, four per workgroup.  LDS: each
// wave's u row (G L floats).
constexpr int kLatWaves = 4;

template <typename TIO, int MT>
__global__ __launch_bounds__(kLatWaves * 64) void lattice_mfma_kernel(
    const int64_t* __restrict__ ids, const float* __restrict__ unary, const int64_t* __restrict__ anchor,
    const TIO* __restrict__ A, const TIO* __restrict__ B, const float* __restrict__ u_parts, int32_t ksplit,
    int32_t slots, int32_t K, int32_t r, int32_t L, int32_t vload, int64_t vocab, int32_t n_rows,
    float* __restrict__ scores) {
  extern __shared__ __align__(16) float lat_smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kpad = (64 / MT) * L;
  float* s_u = lat_smem + wave * kpad;
  const int n_raw = blockIdx.x * kLatWaves + wave;
  const bool row_ok = n_raw < n_rows;
  const int n = row_ok ? n_raw : n_rows - 1;        // a wave past the rows repeats the last one, unstored
  const int req = n / slots, s = n - req * slots;
  for (int k = lane; k < kpad; k += 64) s_u[k] = k < r ? sum_proj_slices(u_parts, ksplit, n_rows, r, n, k) : 0.f;
  const int e = lane % MT;
  const int ec = e < K ? e : 0;
  const int64_t pred = (s == 0) ? anchor[req] : ids[((int64_t)n - 1) * K + ec];
  const int64_t cand = ids[(int64_t)n * K + ec];
  __syncthreads();
  const typename LatTile<MT>::acc_t acc =
      lattice_slot_tile<TIO, MT, 8>(A, B, vocab, r, L, vload != 0, pred, cand, s_u);
  if (row_ok) lattice_store<MT>(acc, unary + (int64_t)n * K, K, scores + (int64_t)n * K * K, K);
}

// Lane j's value of v, as a wave-uniform value.
__device__ __forceinline__ float lane_value(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// One walk decision on a wave: lane j (< K) holds row[j].  Returns the chosen
// index (wave-uniform) and sets q (this lane's probability).  Maxima are
// exact in any order (tree); the normalising sum and the CDF run left to
// right over the candidates, as the definition is evaluated.
__device__ __forceinline__ int walk_decide(float v, int lane, int K, bool greedy, float temp, float u,
                                           float& q) {
  const bool on = lane < K;
  if (greedy) {
    // first maximum in candidate order = lowest index among ties
    float best = lane_value(v, 0);
    int idx = 0;
    for (int j = 1; j < K; ++j) {
      const float x = lane_value(v, j);
      if (x > best) { best = x; idx = j; }
    }
    q = (lane == idx) ? 1.f : 0.f;
    return idx;
  }
  const float t = fmaxf(temp, 1e-5f);
  const float xs = v / t;
  float mx = lane_value(xs, 0);
  for (int j = 1; j < K; ++j) mx = fmaxf(mx, lane_value(xs, j));
  // exp rounded once to fp32 (from the fp64 exponential)
  const float e = on ? (float)exp((double)(xs - mx)) : 0.f;
  float total = 0.f;
  for (int j = 0; j < K; ++j) total += lane_value(e, j);          // left to right
  const float p = e / total;
  float cdf = 0.f;
  int cnt = 0;
  for (int j = 0; j < K; ++j) {                                     // C_j left to right
    cdf += lane_value(p, j);
    cnt += (u >= cdf) ? 1 : 0;
  }
  q = on ? p : 0.f;
  return cnt < K - 1 ? cnt : K - 1;
}

constexpr int kWalkLdsBytes = 64 * 1024;   // scores + ids + uniforms of a request, staged when they fit

__device__ __forceinline__ size_t walk_stage_bytes(int slots, int K) {
  return (size_t)slots * K * K * sizeof(float) + (size_t)slots * K * sizeof(int64_t) + (size_t)slots * sizeof(float);
}

__global__ __launch_bounds__(kThreads) void walk_kernel(const float* __restrict__ scores,
                                                        const int64_t* __restrict__ ids,
                                                        const float* __restrict__ uniforms,
                                                        const float* __restrict__ temperatures,
                                                        const uint8_t* __restrict__ greedy_mask,
                                                        int32_t slots, int32_t K,
                                                        int64_t* __restrict__ tokens,
                                                        float* __restrict__ q_out) {
  extern __shared__ __align__(16) unsigned char walk_smem[];
  const int req = blockIdx.x;
  const int64_t per_req = (int64_t)slots * K * K;
  const float* src = scores + (int64_t)req * per_req;
  const int64_t* ids_r = ids + (int64_t)req * slots * K;
  const float* uni_r = uniforms + (int64_t)req * slots;
  // layout: ids (8-byte) first, then scores, then uniforms
  int64_t* s_ids = reinterpret_cast<int64_t*>(walk_smem);
  float* s_sc = reinterpret_cast<float*>(s_ids + (int64_t)slots * K);
  float* s_u = s_sc + per_req;
  const bool staged = walk_stage_bytes(slots, K) <= (size_t)kWalkLdsBytes;
  if (staged) {
    for (int64_t i = threadIdx.x; i < per_req; i += kThreads) s_sc[i] = src[i];
    for (int i = threadIdx.x; i < slots * K; i += kThreads) s_ids[i] = ids_r[i];
    for (int i = threadIdx.x; i < slots; i += kThreads) s_u[i] = uni_r[i];
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const bool greedy = greedy_mask[req] != 0;
  const float temp = temperatures[req];
  const float* sc = staged ? s_sc : src;
  const int64_t* id = staged ? s_ids : ids_r;
  const float* un = staged ? s_u : uni_r;
  int prev = 0;
  for (int s = 0; s < slots; ++s) {
    const int64_t row_off = ((int64_t)s * K + prev) * K;
    const float v = lane < K ? sc[row_off + lane] : 0.f;
    float q;
    const int idx = walk_decide(v, lane, K, greedy, temp, un[s], q);
    const int64_t n = (int64_t)req * slots + s;
    if (lane < K) q_out[n * K + lane] = q;
    if (lane == 0) tokens[n] = id[s * K + idx];
    prev = idx;
  }
}

// Every row's walk decision, then the walked path, for one request whose
// S x K x K scores sit in LDS (sc, overwritten: exponentials, then q).  A
// row's decision does not depend on the path, so all S*K rows are decided in
// parallel (row maxima, sums and CDFs sequential per row, as walk_decide
// runs them; the fp64 exponentials spread over entries, in place).  The
// path is then found by pointer jumping: with f_s the choice map of slot s
// (row j -> index chosen in row (s, j)), the index chosen at slot s is
// (f_s o ... o f_0)(0), an inclusive scan in ceil(log2 S) rounds; the row
// walked at slot s is the index chosen at slot s - 1 (row 0 at slot 0).
// Row sj of sc starts at sc + sj * (K + 1): the odd stride keeps the per-row
// threads, which walk their rows in step, on distinct LDS banks.
// mx, nxt, galt: [S*K] LDS scratch; un: the request's uniforms (LDS);
// cand: the request's candidate ids [S][K] (LDS or global).  Every thread of
// the workgroup calls; ends with the outputs written.
template <int NT>
__device__ void decide_and_walk(float* sc, float* mx, int* nxt, int* galt, const float* un, int S, int K,
                                bool greedy, float temp, const FastDiv& div_k, int64_t row0,
                                const int64_t* cand, int64_t* __restrict__ tokens, float* __restrict__ q_out) {
  const int tid = threadIdx.x;
  const int n_entries = S * K * K;
  const int ks = K + 1;
  if (greedy) {
    for (int sj = tid; sj < S * K; sj += NT) {
      float* row = sc + sj * ks;
      // first maximum in candidate order = lowest index among ties
      float best = row[0];
      int idx = 0;
      for (int c = 1; c < K; ++c) {
        const float x = row[c];
        if (x > best) { best = x; idx = c; }
      }
      for (int c = 0; c < K; ++c) row[c] = (c == idx) ? 1.f : 0.f;
      nxt[sj] = idx;
    }
  } else {
    const float t = fmaxf(temp, 1e-5f);
    for (int sj = tid; sj < S * K; sj += NT) {
      const float* row = sc + sj * ks;
      float m = row[0] / t;
      for (int c = 1; c < K; ++c) m = fmaxf(m, row[c] / t);
      mx[sj] = m;
    }
    __syncthreads();
    // exp rounded once to fp32 (from the fp64 exponential), over the score
    for (int e = tid; e < n_entries; e += NT) {
      const int sj = div_k.quot(e);
      float* x = sc + sj * ks + (e - sj * K);
      *x = (float)exp((double)(*x / t - mx[sj]));
    }
    __syncthreads();
    for (int sj = tid; sj < S * K; sj += NT) {
      float* row = sc + sj * ks;
      float total = 0.f;
      for (int c = 0; c < K; ++c) total += row[c];                 // left to right
      const float u = un[div_k.quot(sj)];
      float cdf = 0.f;
      int cnt = 0;
      for (int c = 0; c < K; ++c) {
        const float p = row[c] / total;
        row[c] = p;
        cdf += p;                                                   // C_c left to right
        cnt += (u >= cdf) ? 1 : 0;
      }
      nxt[sj] = cnt < K - 1 ? cnt : K - 1;
    }
  }
  __syncthreads();
  int* g_cur = nxt;
  int* g_alt = galt;
  for (int d = 1; d < S; d <<= 1) {
    for (int i = tid; i < S * K; i += NT) {
      const int s = div_k.quot(i);
      g_alt[i] = (s >= d) ? g_cur[s * K + g_cur[i - d * K]] : g_cur[i];
    }
    __syncthreads();
    int* tmp = g_cur; g_cur = g_alt; g_alt = tmp;
  }
  for (int i = tid; i < S * K; i += NT) {
    const int s = div_k.quot(i), c = i - s * K;
    const int prev = (s == 0) ? 0 : g_cur[(s - 1) * K];   // row walked at slot s
    const int64_t n = row0 + s;
    q_out[n * K + c] = sc[(s * K + prev) * ks + c];
    if (c == 0) tokens[n] = cand[s * K + g_cur[s * K]];
  }
}

// Walk for one request in one workgroup of 1024 threads when its scores fit
// in LDS: the scores, staged with batched coalesced loads, then
// decide_and_walk.  Same arithmetic as walk_kernel (bit-identical tokens and
// q).  LDS: scores [S][K][K+1], row maxima, choice maps, scan buffer [S][K],
// uniforms [S].
constexpr int kWalkThreads = 1024;
__host__ __device__ inline size_t walk_lds_bytes(int S, int K) {
  return (size_t)S * K * (K + 1) * 4 + 3 * (size_t)S * K * 4 + (size_t)S * 4;
}

__global__ __launch_bounds__(kWalkThreads) void walk_lds_kernel(const float* __restrict__ scores,
                                                                const int64_t* __restrict__ ids,
                                                                const float* __restrict__ uniforms,
                                                                const float* __restrict__ temperatures,
                                                                const uint8_t* __restrict__ greedy_mask,
                                                                int32_t slots, int32_t K,
                                                                int64_t* __restrict__ tokens,
                                                                float* __restrict__ q_out) {
  extern __shared__ __align__(16) float wk_smem[];
  const int S = slots;
  const int req = blockIdx.x, tid = threadIdx.x;
  float* sc = wk_smem;
  float* mx = sc + S * K * (K + 1);
  int* nxt = reinterpret_cast<int*>(mx + S * K);
  int* galt = nxt + S * K;
  float* un = reinterpret_cast<float*>(galt + S * K);
  const int64_t row0 = (int64_t)req * S;
  const int n_e = S * K * K;
  const float* src = scores + row0 * K * K;
  const FastDiv div_k(K);                           // indices < S*K*K <= 40960 (LDS bound)
  constexpr int kBatch = 16;                        // loads issued before the first store
  for (int base = 0; base < n_e; base += kWalkThreads * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = __builtin_nontemporal_load(src + min(base + q * kWalkThreads + tid, n_e - 1));
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = base + q * kWalkThreads + tid;
      if (i < n_e) {
        const int sj = div_k.quot(i);
        sc[sj * (K + 1) + i - sj * K] = v[q];
      }
    }
  }
  for (int i = tid; i < S; i += kWalkThreads) un[i] = uniforms[row0 + i];
  __syncthreads();
  decide_and_walk<kWalkThreads>(sc, mx, nxt, galt, un, S, K, greedy_mask[req] != 0, temperatures[req], div_k,
                                row0, ids + row0 * K, tokens, q_out);
}


// Lattice + walk for one request in one workgroup of 1024 threads (16
// waves).  The lattice is lattice_slot_tile's (bit-identical to
// lattice_mfma_kernel) and the decisions decide_and_walk's (bit-identical to
// the walk kernels), so the result equals dflash_lattice followed by
// dflash_walk.  Phases:
//   1. candidate ids of every slot, uniforms, and u of every slot (the
//      projection slices summed in order, zero past r) -> LDS, one round of
//      loads;
//   2. wave w evaluates slots w, w + 16, ...: its table gathers, the fp32
//      matrix-core tile, + unary -> the score rows in LDS (and scores_out);
//   3, 4. decide_and_walk: every row's decision in parallel, then the walked
//      path by pointer jumping, q rows and tokens written in parallel.
// LDS: candidate ids [S][K] (int64), u [S][G L] (the scan's second buffer
// afterwards), scores [S][K][K+1], row maxima [S][K], uniforms [S], chosen
// index per row [S][K].
constexpr int kLWThreads = 1024;

struct LatticeWalkLds {
  size_t cand, u, sc, mx, un, next, bytes;
};

__host__ __device__ inline LatticeWalkLds lattice_walk_layout(int S, int K, int kpad) {
  LatticeWalkLds L;
  const size_t u_floats = (size_t)S * (kpad > K ? kpad : K);
  size_t o = 0;
  L.cand = o; o += (size_t)S * K * 8;
  L.u = o;    o += (u_floats * 4 + 15) & ~(size_t)15;
  L.sc = o;   o += (size_t)S * K * (K + 1) * 4;
  L.mx = o;   o += (size_t)S * K * 4;
  L.next = o; o += (size_t)S * K * 4;
  L.un = o;   o += (size_t)S * 4;
  L.bytes = o;
  return L;
}

template <typename TIO, int MT>
__global__ __launch_bounds__(kLWThreads) void lattice_walk_kernel(
    const int64_t* __restrict__ ids, const float* __restrict__ unary, const int64_t* __restrict__ anchor,
    const TIO* __restrict__ A, const TIO* __restrict__ B, const float* __restrict__ u_parts, int32_t ksplit,
    int32_t slots, int32_t K, int32_t r, int32_t L, int32_t vload, int64_t vocab,
    const float* __restrict__ uniforms, const float* __restrict__ temperatures,
    const uint8_t* __restrict__ greedy_mask, float* __restrict__ scores_out, int64_t* __restrict__ tokens,
    float* __restrict__ q_out) {
  extern __shared__ __align__(16) unsigned char lw_smem[];
  const int req = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int S = slots;
  const int kpad = (64 / MT) * L;
  const LatticeWalkLds Ly = lattice_walk_layout(S, K, kpad);
  int64_t* s_cand = reinterpret_cast<int64_t*>(lw_smem + Ly.cand);
  float* s_u = reinterpret_cast<float*>(lw_smem + Ly.u);
  float* s_sc = reinterpret_cast<float*>(lw_smem + Ly.sc);
  float* s_mx = reinterpret_cast<float*>(lw_smem + Ly.mx);
  float* s_un = reinterpret_cast<float*>(lw_smem + Ly.un);
  int* s_next = reinterpret_cast<int*>(lw_smem + Ly.next);
  const int64_t row0 = (int64_t)req * S;            // first slot row of this request
  const FastDiv div_k(K), div_kp(kpad);             // every index below is < 2^16 (LDS bound)

  // ---- 1. candidate ids, uniforms, u -----------------------------------
  // Each pass issues every load of its items before the first LDS write or
  // add, so the phase costs one memory round trip per pass (one pass
  // whenever S * max(K, G L) <= 1024).
  {
    const int n_e = S * K, n_u = S * kpad;
    const int n_all = max(max(n_e, n_u), S);
    for (int i = tid; i < n_all; i += kLWThreads) {
      const bool has_e = i < n_e, has_s = i < S;
      bool has_u = i < n_u;
      float uni = 0.f;
      int64_t cand = 0;
      float v[kMaxProjSplit];
      int s_u_row = 0, k = 0;
      if (has_s) uni = uniforms[row0 + i];
      if (has_e) cand = ids[row0 * K + i];
      if (has_u) {
        s_u_row = div_kp.quot(i);
        k = i - s_u_row * kpad;
        if (k < r) load_proj_slices(u_parts, ksplit, (int64_t)gridDim.x * S, r, row0 + s_u_row, k, v);
      }
      // keep the compiler from sinking the slice loads below the LDS writes
      // (which would start a second round trip after the first one drained)
      asm volatile("" ::: "memory");
      if (has_s) s_un[i] = uni;
      if (has_e) s_cand[i] = cand;
      if (has_u) s_u[i] = k < r ? add_proj_slices(v, ksplit) : 0.f;
    }
  }
  __syncthreads();

  // ---- 2. one slot per wave: gathers, matrix-core tile, + unary ---------
  {
    const int e = lane % MT;
    const int ec = e < K ? e : 0;
    const int64_t anc = anchor[req];
    for (int s = wave; s < S; s += kLWThreads / 64) {
      const int64_t pred = (s == 0) ? anc : s_cand[(s - 1) * K + ec];
      const int64_t cand = s_cand[s * K + ec];
      const typename LatTile<MT>::acc_t acc =
          lattice_slot_tile<TIO, MT, 4>(A, B, vocab, r, L, vload != 0, pred, cand, s_u + s * kpad);
      const float* un = unary + (row0 + s) * K;
      lattice_store<MT>(acc, un, K, s_sc + s * K * (K + 1), K + 1);
      if (scores_out) lattice_store<MT>(acc, un, K, scores_out + (row0 + s) * K * K, K);
    }
  }
  __syncthreads();

  // ---- 3, 4. every row's decision, then the walked path -----------------
  decide_and_walk<kLWThreads>(s_sc, s_mx, s_next, reinterpret_cast<int*>(s_u), s_un, S, K,
                              greedy_mask[req] != 0, temperatures[req], div_k, row0, s_cand, tokens, q_out);
}

// walk_decide's arithmetic (the same operations in the same order, so the
// same bits) with short dependency chains, for one wave whose lanes 0..K-1
// hold the row and whose other lanes hold -inf (they add 0 to every sum and
// never win; a count past K - 1 is capped as before).  The values summed in
// order are read into uniform registers all at once before each ordered sum,
// and the row maximum is a wave reduction (fmaxf is exact in any order).
template <int MT>
__device__ __forceinline__ int walk_decide_wave(float v, int lane, int K, bool greedy, float temp, float u,
                                                float& q) {
  constexpr int BT = 8;                             // lanes read per batch
  const bool on = lane < K;
  if (greedy) {
    // first maximum in candidate order = lowest index among ties
    float best = lane_value(v, 0);
    int idx = 0;
#pragma unroll
    for (int j0 = 0; j0 < MT; j0 += BT) {
      float r[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) r[b] = lane_value(v, j0 + b);
#pragma unroll
      for (int b = 0; b < BT; ++b)
        if (j0 + b > 0 && r[b] > best) { best = r[b]; idx = j0 + b; }
    }
    q = (lane == idx) ? 1.f : 0.f;
    return idx;
  }
  const float t = fmaxf(temp, 1e-5f);
  const float xs = v / t;
  const float mx = wave_max_f32(xs);
  // exp rounded once to fp32 (from the fp64 exponential)
  const float e = on ? (float)exp((double)(xs - mx)) : 0.f;
  float total = 0.f;
#pragma unroll
  for (int j0 = 0; j0 < MT; j0 += BT) {
    float r[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) r[b] = lane_value(e, j0 + b);
#pragma unroll
    for (int b = 0; b < BT; ++b) total += r[b];                    // left to right
  }
  const float p = e / total;
  float cdf = 0.f;
  int cnt = 0;
#pragma unroll
  for (int j0 = 0; j0 < MT; j0 += BT) {
    float r[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) r[b] = lane_value(p, j0 + b);
#pragma unroll
    for (int b = 0; b < BT; ++b) {                                 // C_j left to right
      cdf += r[b];
      cnt += (u >= cdf) ? 1 : 0;
    }
  }
  q = on ? p : 0.f;
  return cnt < K - 1 ? cnt : K - 1;
}

// Lattice + walk with one wave per request, for batches with requests
// enough to occupy every SIMD.  Slot by slot the wave evaluates the slot's
// tile on the matrix cores (tile_mfma: the sequence every lattice kernel
// runs), takes the walked row -- the one chosen at the previous slot --
// straight from the accumulators (one lane shuffle), and decides it with
// walk_decide's arithmetic.  Only the S walked rows are decided, not all
// S x K.  Pipelining: every small per-slot input (candidate ids, unary,
// uniforms) is staged in LDS up front, so inside the loop the wave issues
// only the next slot's u and table loads -- the vector-memory counter
// retires in order, so waiting for a later small load would wait for those
// prefetches too; slot s + 1's loads are in flight while slot s is decided,
// and slot s + 1's MFMA chain is issued in the same stretch of code as slot
// s's decision.  The two register sets for table pieces alternate roles
// (two slots per loop turn), so nothing is copied.  Bit-identical to
// dflash_lattice followed by dflash_walk.  Needs S <= 16, bf16 or fp32
// tables with 16-byte aligned rows, rank a multiple of the tile's k-groups
// (G VEC) so that every gathered piece lies inside the row, NV = L / VEC
// pieces per lane (1, 2, 4 or 8) and G L <= 128.  LDS per wave: two u rows,
// the candidate ids [S][MT] (int64), unary [S][MT] and uniforms [S].
constexpr int kLWWaves = 4;          // requests (waves) per workgroup
constexpr int kWaveMaxSlots = 16;

template <typename TIO, int MT, int NV>
__global__ __launch_bounds__(kLWWaves * 64) void lattice_walk_wave_kernel(
    const int64_t* __restrict__ ids, const float* __restrict__ unary, const int64_t* __restrict__ anchor,
    const TIO* __restrict__ A, const TIO* __restrict__ B, const float* __restrict__ u_parts, int32_t ksplit,
    int32_t slots, int32_t K, int32_t r, int64_t vocab, int32_t n_req, const float* __restrict__ uniforms,
    const float* __restrict__ temperatures, const uint8_t* __restrict__ greedy_mask,
    float* __restrict__ scores_out, int64_t* __restrict__ tokens, float* __restrict__ q_out) {
  constexpr int VEC = Elem<TIO>::kVec;
  constexpr int L = NV * VEC;
  constexpr int KPAD = (64 / MT) * L;
  typedef LatTile<MT> Tile;
  extern __shared__ __align__(16) float lww_smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int req = blockIdx.x * kLWWaves + wave;
  if (req >= n_req) return;                          // waves are independent: no workgroup barrier
  const int S = slots;
  float* s_u2 = lww_smem + wave * 2 * KPAD;          // u rows of two slots (alternating)
  const int64_t row0 = (int64_t)req * S;
  const bool greedy = greedy_mask[req] != 0;
  const float temp = temperatures[req];
  const int e = lane % MT;
  const int kg = (lane / MT) * L;

  // Every small per-slot input to the wave's LDS up front: candidate ids (as
  // given), unary, uniforms.
  int64_t* s_id = reinterpret_cast<int64_t*>(lww_smem + kLWWaves * 2 * KPAD) + wave * kWaveMaxSlots * MT;
  float* s_un = reinterpret_cast<float*>(reinterpret_cast<int64_t*>(lww_smem + kLWWaves * 2 * KPAD) +
                                         kLWWaves * kWaveMaxSlots * MT) + wave * (kWaveMaxSlots * MT + kWaveMaxSlots);
  float* s_uni = s_un + kWaveMaxSlots * MT;
  for (int i = lane; i < S * MT; i += 64) {
    const int si = i / MT, ei = i - si * MT;
    const int64_t src = (row0 + si) * K + (ei < K ? ei : 0);
    s_id[i] = ids[src];
    s_un[i] = unary[src];
  }
  if (lane < S) s_uni[lane] = uniforms[row0 + lane];
  const int64_t anc = anchor[req];
  asm volatile("" ::: "memory");
  // slot s's predecessor / candidate id of this lane's row / column index
  // (an id outside [0, vocab) is out of range for tile_rows as it is)
  auto pred_of = [&](int s) -> int64_t { return s == 0 ? anc : s_id[(s - 1) * MT + e]; };
  auto cand_of = [&](int s) -> int64_t { return s_id[s * MT + e]; };
  auto load_u = [&](int s, float (&uv)[2][kMaxProjSplit]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = lane + 64 * h;
      if (k < KPAD) load_proj_slices(u_parts, ksplit, (int64_t)n_req * S, r, row0 + s, k, uv[h]);
    }
  };
  auto store_u = [&](const float (&uv)[2][kMaxProjSplit], float* dst) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = lane + 64 * h;
      if (k < KPAD) dst[k] = add_proj_slices(uv[h], ksplit);
    }
    asm volatile("" ::: "memory");
  };
  // the table pieces of slot s (rank is a multiple of G VEC: every piece lies
  // inside its row, so the loads are unconditional)
  auto gather = [&](int s, u32x4 (&ga)[NV], u32x4 (&gb)[NV]) -> TileRows<TIO> {
    const TileRows<TIO> t = tile_rows(A, B, vocab, r, pred_of(s), cand_of(s));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      ga[v] = ld16(t.arow + kg + v * VEC);
      gb[v] = ld16(t.brow + kg + v * VEC);
    }
    return t;
  };

  // slot 0: u to LDS and its tile; slot 1's operands in flight
  float uv[2][kMaxProjSplit];
  load_u(0, uv);
  u32x4 a0[NV], b0[NV], a1[NV], b1[NV];
  TileRows<TIO> t0 = gather(0, a0, b0);
  store_u(uv, s_u2);
  load_u(S > 1 ? 1 : 0, uv);
  TileRows<TIO> t1 = gather(S > 1 ? 1 : 0, a1, b1);
  typename Tile::acc_t acc = {};
  tile_mfma<TIO, MT, NV>(acc, a0, b0, t0.pok, t0.cok, kg, 0, NV, s_u2);

  int prev = 0;
  // One slot: (xa, xb, tx) hold slot s + 1's pieces, (ya, yb, ty) receive slot
  // s + 2's.  Slots past S - 1 are clamped (their results are not used).
  auto step = [&](int s, u32x4 (&xa)[NV], u32x4 (&xb)[NV], const TileRows<TIO>& tx, u32x4 (&ya)[NV],
                  u32x4 (&yb)[NV], TileRows<TIO>& ty) {
    const int64_t n = row0 + s;
    const int sa = min(s + 2, S - 1);
    float* un_lds = s_u2 + ((s + 1) & 1) * KPAD;
    store_u(uv, un_lds);
    load_u(sa, uv);
    ty = gather(sa, ya, yb);
    // slot s + 1's MFMA chain and slot s's decision, in one stretch of code
    typename Tile::acc_t acc_n = {};
    tile_mfma<TIO, MT, NV>(acc_n, xa, xb, tx.pok, tx.cok, kg, 0, NV, un_lds);
    const float* un = s_un + s * MT;
    if (scores_out) lattice_store<MT>(acc, un, K, scores_out + n * K * K, K);
    // row prev of slot s's tile: its column c sits in lane (prev's lane
    // group) * MT + c, accumulator i(prev); + unary[c] as lattice_store adds it
    int src_grp, ai;
    if (MT == 32) { src_grp = (prev >> 2) & 1; ai = 4 * (prev >> 3) + (prev & 3); }
    else          { src_grp = prev >> 2;       ai = prev & 3; }
    float x = acc[0];
#pragma unroll
    for (int i = 1; i < Tile::kAcc; ++i) x = (ai == i) ? acc[i] : x;
    const float row_v = __shfl(x, src_grp * MT + e, 64);
    const float v = lane < K ? row_v + un[e] : -INFINITY;
    float q;
    const int idx = walk_decide_wave<MT>(v, lane, K, greedy, temp, s_uni[s], q);
    if (lane < K) q_out[n * K + lane] = q;
    if (lane == 0) tokens[n] = s_id[s * MT + idx];   // the chosen candidate's id as given
    prev = idx;
    acc = acc_n;
  };
  for (int s = 0; s < S; s += 2) {
    step(s, a1, b1, t1, a0, b0, t0);
    if (s + 1 < S) step(s + 1, a0, b0, t0, a1, b1, t1);
  }
}

}  // namespace

ProjPlan plan_proj(int32_t n_rows, int32_t rank, int32_t hidden, int32_t dtype) {
  ProjPlan p{};
  p.n_rows = n_rows;
  p.rank = rank;
  p.hidden = hidden;
  if (dtype == DFLASH_BF16 && n_rows >= kProjTileMinRows && rank <= ProjTileCfg::kBN) {
    // 128-row tiles; the contraction split so that ~480 workgroups exist,
    // a split above 4 rounded up to a multiple of 4 (at 15360 slot rows x
    // 7168 channels: 4 slices 53 us, 2 slices 64, 5 slices 69, 8 slices 63)
    p.tiled = 1;
    p.row_tiles = (n_rows + ProjTileCfg::kBM - 1) / ProjTileCfg::kBM;
    const int nk = (hidden + ProjTileCfg::kBK - 1) / ProjTileCfg::kBK;
    int ks = (480 + p.row_tiles - 1) / p.row_tiles;
    if (ks > 4) ks = (ks + 3) & ~3;
    if (ks > kMaxProjSplit) ks = kMaxProjSplit;
    if (ks > nk) ks = nk;
    if (ks < 1) ks = 1;
    const int kb = (nk + ks - 1) / ks;
    p.kslice = kb * ProjTileCfg::kBK;
    p.ksplit = (nk + kb - 1) / kb;
  } else if (dtype == DFLASH_BF16) {
    p.frags = 1;
    p.row_tiles = (n_rows + kRowsPerWG - 1) / kRowsPerWG;
    int ks = p.row_tiles > 0 ? (512 + p.row_tiles - 1) / p.row_tiles : 1;
    const int max_ks = hidden / 256 > 1 ? hidden / 256 : 1;   // slices of >= 8 k-steps
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
    if (ks > kMaxProjSplit) ks = kMaxProjSplit;
    int slice = (hidden + ks - 1) / ks;
    slice = (slice + 31) / 32 * 32;
    p.kslice = slice;
    p.ksplit = (hidden + slice - 1) / slice;
  } else {
    p.row_tiles = 0;
    p.kslice = hidden;
    p.ksplit = 1;
  }
  p.bytes = (size_t)p.ksplit * n_rows * rank * sizeof(float);
  p.bytes = (p.bytes + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_proj(const SelectArgs& a, const ProjPlan& p, hipStream_t stream) {
  const int n_rows = a.n_req * a.slots;
  if (n_rows == 0 || a.rank == 0) return hipSuccess;
  if (a.dtype == DFLASH_BF16 && p.tiled) {
    hipLaunchKernelGGL(proj_tile_kernel, dim3(p.row_tiles, p.ksplit), dim3(ProjTileCfg::kThreads),
                       ProjTileCfg::kSmemBytes, stream, static_cast<const uint16_t*>(a.hidden), a.hidden_req_stride,
                       a.hidden_slot_stride, a.slots, static_cast<const uint16_t*>(a.proj), n_rows, a.rank,
                       a.hidden_size, p.kslice / ProjTileCfg::kBK, a.u_parts);
    return hipGetLastError();
  }
  if (a.dtype == DFLASH_BF16) {
    const dim3 grid(p.row_tiles, p.ksplit);
    const uint16_t* h = static_cast<const uint16_t*>(a.hidden);
    const uint16_t* P = static_cast<const uint16_t*>(a.proj);
    const int tiles = (a.rank + 15) / 16;
#define DFLASH_PROJ(RT, FR)                                                                        \
  hipLaunchKernelGGL((proj_mfma_kernel<RT, FR>), grid, dim3(kThreads), 0, stream, h, a.hidden_req_stride, \
                     a.hidden_slot_stride, a.slots, P, n_rows, a.rank, a.hidden_size, p.kslice,          \
                     a.u_parts)
#define DFLASH_PROJ_RT(FR)                  \
  if (tiles <= 1) DFLASH_PROJ(1, FR);       \
  else if (tiles <= 2) DFLASH_PROJ(2, FR);  \
  else if (tiles <= 4) DFLASH_PROJ(4, FR);  \
  else if (tiles <= 8) DFLASH_PROJ(8, FR);  \
  else return hipErrorInvalidValue;   /* rank > 128 is rejected by the API layer */
    DFLASH_PROJ_RT(1)
#undef DFLASH_PROJ_RT
#undef DFLASH_PROJ
  } else {
    const int64_t n = (int64_t)n_rows * a.rank;
    hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, static_cast<const float*>(a.hidden), a.hidden_req_stride,
                       a.hidden_slot_stride, a.slots, static_cast<const float*>(a.proj), n_rows, a.rank,
                       a.hidden_size, a.u_parts);
  }
  return hipGetLastError();
}


namespace {
// 16-byte gathers of the table rows need 16-byte aligned rows and tables.
bool lattice_vload(const SelectArgs& a) {
  const int e = a.dtype == DFLASH_BF16 ? 2 : 4;
  return ((int64_t)a.rank * e) % 16 == 0 && (reinterpret_cast<uintptr_t>(a.sel_a) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(a.sel_b) & 15) == 0;
}
int lattice_vec(int32_t dtype) { return dtype == DFLASH_BF16 ? 8 : 4; }
}  // namespace

int lattice_kpad_floats(int32_t top_k, int32_t rank, int32_t dtype) {
  return lattice_kpad(top_k, rank, lattice_vec(dtype));
}

hipError_t launch_lattice(const SelectArgs& a, const ProjPlan& p, hipStream_t stream) {
  const int n_rows = a.n_req * a.slots;
  if (n_rows == 0) return hipSuccess;
  const int MT = lattice_mt(a.top_k);
  const int L = lattice_group_len(a.top_k, a.rank, lattice_vec(a.dtype));
  const size_t lds = (size_t)kLatWaves * (64 / MT) * L * sizeof(float);
  const int vload = lattice_vload(a) ? 1 : 0;
  const dim3 grid((n_rows + kLatWaves - 1) / kLatWaves);
#define DFLASH_LAT(TIO, MTV)                                                                                   \
  hipLaunchKernelGGL((lattice_mfma_kernel<TIO, MTV>), grid, dim3(kLatWaves * 64), lds, stream, a.ids, a.unary, \
                     a.anchor, static_cast<const TIO*>(a.sel_a), static_cast<const TIO*>(a.sel_b), a.u_parts,   \
                     p.ksplit, a.slots, a.top_k, a.rank, L, vload, a.vocab, n_rows, a.scores)
  if (a.dtype == DFLASH_BF16) {
    if (MT == 16) DFLASH_LAT(uint16_t, 16); else DFLASH_LAT(uint16_t, 32);
  } else {
    if (MT == 16) DFLASH_LAT(float, 16); else DFLASH_LAT(float, 32);
  }
#undef DFLASH_LAT
  return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, hipStream_t stream) {
  if (a.n_req == 0 || a.slots == 0) return hipSuccess;
  const size_t wl = walk_lds_bytes(a.slots, a.top_k);
  if (wl <= kWalkLdsMax) {
    hipLaunchKernelGGL(walk_lds_kernel, dim3(a.n_req), dim3(kWalkThreads), wl, stream, a.scores, a.ids, a.uniforms,
                       a.temperatures, a.greedy, a.slots, a.top_k, a.tokens, a.q);
    return hipGetLastError();
  }
  const size_t need = (size_t)a.slots * a.top_k * a.top_k * sizeof(float) +
                      (size_t)a.slots * a.top_k * sizeof(int64_t) + (size_t)a.slots * sizeof(float);
  const size_t lds = need <= (size_t)kWalkLdsBytes ? need : 0;
  hipLaunchKernelGGL(walk_kernel, dim3(a.n_req), dim3(kThreads), lds, stream, a.scores, a.ids, a.uniforms,
                     a.temperatures, a.greedy, a.slots, a.top_k, a.tokens, a.q);
  return hipGetLastError();
}


size_t lattice_walk_lds_bytes(int slots, int K, int r, int dtype) {
  return lattice_walk_layout(slots, K, lattice_kpad(K, r, lattice_vec(dtype))).bytes;
}

bool lattice_walk_fits(const SelectArgs& a) {
  return lattice_walk_per_wave(a) || lattice_walk_lds_bytes(a.slots, a.top_k, a.rank, a.dtype) <= kLatticeWalkLdsMax;
}

// One wave per request once the batch has a request for every SIMD (the
// serial decisions then hide behind each other); the tile's k-range must be
// whole 16-byte pieces inside the rank, one gather round and two u values
// per lane.
bool lattice_walk_per_wave(const SelectArgs& a) {
  const int vec = lattice_vec(a.dtype);
  const int MT = lattice_mt(a.top_k);
  const int L = lattice_group_len(a.top_k, a.rank, vec);
  const int nv = L / vec;
  return a.n_req >= kLatticeWalkWaveMinReq && a.slots <= kWaveMaxSlots && lattice_vload(a) &&
         a.rank % ((64 / MT) * vec) == 0 && (nv == 1 || nv == 2 || nv == 4 || nv == 8) &&
         lattice_kpad(a.top_k, a.rank, vec) <= 128;
}

hipError_t launch_lattice_walk(const SelectArgs& a, const ProjPlan& p, const WalkArgs& w, float* scores_out,
                               hipStream_t stream) {
  if (a.n_req == 0 || a.slots == 0) return hipSuccess;
  if (lattice_walk_per_wave(a)) {
    const int MT = lattice_mt(a.top_k);
    const int vec = lattice_vec(a.dtype);
    const int L = lattice_group_len(a.top_k, a.rank, vec);
    const int nv = L / vec;
    const size_t lds = (size_t)kLWWaves * (2 * (64 / MT) * L * sizeof(float) + kWaveMaxSlots * MT * sizeof(int64_t) +
                                           (kWaveMaxSlots * MT + kWaveMaxSlots) * sizeof(float));
    const dim3 grid((a.n_req + kLWWaves - 1) / kLWWaves);
#define DFLASH_LWW(TIO, MTV, NVV)                                                                                 \
  hipLaunchKernelGGL((lattice_walk_wave_kernel<TIO, MTV, NVV>), grid, dim3(kLWWaves * 64), lds, stream, a.ids,      \
                     a.unary, a.anchor, static_cast<const TIO*>(a.sel_a), static_cast<const TIO*>(a.sel_b),         \
                     a.u_parts, p.ksplit, a.slots, a.top_k, a.rank, a.vocab, a.n_req, w.uniforms, w.temperatures,   \
                     w.greedy, scores_out, w.tokens, w.q)
#define DFLASH_LWW_NV(TIO, MTV)                                     \
  if (nv == 1) DFLASH_LWW(TIO, MTV, 1);                             \
  else if (nv == 2) DFLASH_LWW(TIO, MTV, 2);                        \
  else if (nv == 4) DFLASH_LWW(TIO, MTV, 4);                        \
  else DFLASH_LWW(TIO, MTV, 8);
    if (a.dtype == DFLASH_BF16) {
      if (MT == 16) { DFLASH_LWW_NV(uint16_t, 16) } else { DFLASH_LWW_NV(uint16_t, 32) }
    } else {
      if (MT == 16) { DFLASH_LWW_NV(float, 16) } else { DFLASH_LWW_NV(float, 32) }
    }
#undef DFLASH_LWW_NV
#undef DFLASH_LWW
    return hipGetLastError();
  }
  if (!lattice_walk_fits(a)) return hipErrorInvalidValue;
  const size_t lds = lattice_walk_lds_bytes(a.slots, a.top_k, a.rank, a.dtype);
  const int MT = lattice_mt(a.top_k);
  const int L = lattice_group_len(a.top_k, a.rank, lattice_vec(a.dtype));
  const int vload = lattice_vload(a) ? 1 : 0;
#define DFLASH_LW(TIO, MTV)                                                                                      \
  hipLaunchKernelGGL((lattice_walk_kernel<TIO, MTV>), dim3(a.n_req), dim3(kLWThreads), lds, stream, a.ids, a.unary, \
                     a.anchor, static_cast<const TIO*>(a.sel_a), static_cast<const TIO*>(a.sel_b), a.u_parts,      \
                     p.ksplit, a.slots, a.top_k, a.rank, L, vload, a.vocab, w.uniforms, w.temperatures, w.greedy,  \
                     scores_out, w.tokens, w.q)
  if (a.dtype == DFLASH_BF16) {
    if (MT == 16) DFLASH_LW(uint16_t, 16); else DFLASH_LW(uint16_t, 32);
  } else {
    if (MT == 16) DFLASH_LW(float, 16); else DFLASH_LW(float, 32);
  }
#undef DFLASH_LW
  return hipGetLastError();
}

}  // namespace dflash

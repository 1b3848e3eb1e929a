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
//  * proj_mfma_kernel: u = P h for every slot row, the one dense contraction
//    on the path, on the matrix cores (v_mfma_f32_16x16x32_bf16; bf16 x bf16
//    products are exact in fp32).  A workgroup owns 64 slot rows x all rank
//    columns and one slice of the hidden axis; slices are summed later in a
//    fixed order, so the result is deterministic.  proj_f32_kernel is the
//    fp32-storage path (VALU fma chain).
//  * lattice_kernel: one workgroup per (request, slot); stages w = A[p] * u
//    and B[c] in LDS as fp32 and evaluates the K x K block as fp32 fma chains
//    in fixed k order (never bf16: rounding A * u to bf16 would blur
//    near-ties).
//  * walk_kernel: one workgroup per request; the request's S x K x K scores
//    are staged in LDS with coalesced loads, then one wave walks the slots
//    (lane j = candidate j) with wave reductions; the serial chain only
//    touches LDS.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
  const int kstride = proj_slice_stride((int)gridDim.y);   // gridDim.y = ksplit
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
        if (row < n_rows) {
          float* dst = u_parts + ((int64_t)row * rank + col) * kstride;
          dst[split] = acc[f][t][v];
          if (split == (int)gridDim.y - 1)
            for (int sp = split + 1; sp < kstride; ++sp) dst[sp] = 0.f;   // pad slots: +0
        }
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
  float* dst = u_parts + t * proj_slice_stride(1);   // one slice, slice-minor layout
  dst[0] = acc;
  dst[1] = dst[2] = dst[3] = 0.f;                      // pad slots: +0
}

// u[n][k] = sum over the projection slices sp = 0..ksplit-1 of the partial
// u_parts[n][k][sp] (slice-minor, stride proj_slice_stride(ksplit)), added in
// slice order.  load_proj_slices issues every load of the value (16-byte
// vectors of 4 slices) before add_proj_slices uses the first, so callers can
// put other loads between the two and pay one memory round trip for all.
__device__ __forceinline__ void load_proj_slices(const float* __restrict__ u_parts, int ksplit, int r, int64_t n,
                                                 int k, float (&v)[kMaxProjSplit]) {
  constexpr int NV = kMaxProjSplit / 4;
  const int nv = proj_slice_stride(ksplit) / 4;   // 16-byte vectors holding slices
  const float4* base = reinterpret_cast<const float4*>(u_parts + (n * r + k) * (int64_t)(4 * nv));
  // every load unconditional (a vector past the last re-reads it), so none
  // waits for another
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const float4 a = base[q < nv ? q : nv - 1];
    v[4 * q] = a.x;
    v[4 * q + 1] = a.y;
    v[4 * q + 2] = a.z;
    v[4 * q + 3] = a.w;
  }
}

// Adds whole 16-byte vectors of slices in order: the writers fill the slots
// past the last slice with +0, which leaves every sum unchanged (a -0 sum
// becomes +0, which no output depends on) and spares a test per slice.
__device__ __forceinline__ float add_proj_slices(const float (&v)[kMaxProjSplit], int ksplit) {
  const int nv = proj_slice_stride(ksplit) / 4;
  float u = v[0];
  u += v[1];
  u += v[2];
  u += v[3];
#pragma unroll
  for (int q = 1; q < kMaxProjSplit / 4; ++q) {
    if (q < nv) {
      u += v[4 * q];
      u += v[4 * q + 1];
      u += v[4 * q + 2];
      u += v[4 * q + 3];
    }
  }
  return u;
}

__device__ __forceinline__ float sum_proj_slices(const float* __restrict__ u_parts, int ksplit, int r, int64_t n,
                                                 int k) {
  float v[kMaxProjSplit];
  load_proj_slices(u_parts, ksplit, r, n, k, v);
  return add_proj_slices(v, ksplit);
}

template <typename TIO>
__device__ __forceinline__ float load_f32(const TIO* p, int64_t i) { return Elem<TIO>::to_f32(p[i]); }

// One lattice block (K x K) for slot row n = req * slots + s, evaluated into
// `dst` (global or LDS) with row stride K.  All threads of the workgroup call.
template <typename TIO>
__device__ void lattice_block(const int64_t* __restrict__ ids, const float* __restrict__ unary,
                              const int64_t* __restrict__ anchor, const TIO* __restrict__ A,
                              const TIO* __restrict__ B, const float* __restrict__ u_parts,
                              int ksplit, int n_rows, int req, int s, int slots, int K, int r,
                              int64_t vocab, float* s_u, float* s_w, float* s_bt, int64_t* s_pred,
                              int64_t* s_cand, float* dst) {
  const int tid = threadIdx.x;
  const int n = req * slots + s;
  const int wstride = r + 1;                         // padded row of w (LDS banks)
  for (int k = tid; k < r; k += kThreads) s_u[k] = sum_proj_slices(u_parts, ksplit, r, n, k);
  for (int j = tid; j < K; j += kThreads) {
    s_pred[j] = (s == 0) ? anchor[req] : ids[((int64_t)req * slots + s - 1) * K + j];
    s_cand[j] = ids[(int64_t)n * K + j];
  }
  __syncthreads();
  for (int i = tid; i < K * r; i += kThreads) {
    const int j = i / r, k = i % r;
    const int64_t p = s_pred[j], c = s_cand[j];
    const float a = (p >= 0 && p < vocab) ? load_f32(A, p * r + k) : __builtin_nanf("");
    const float b = (c >= 0 && c < vocab) ? load_f32(B, c * r + k) : __builtin_nanf("");
    s_w[j * wstride + k] = a * s_u[k];               // A[p] (.) project(h)
    s_bt[k * K + j] = b;
  }
  __syncthreads();
  for (int e = tid; e < K * K; e += kThreads) {
    const int j = e / K, c = e % K;
    const float* w = s_w + j * wstride;
    float acc = 0.f;
    for (int k = 0; k < r; ++k) acc = fmaf(w[k], s_bt[k * K + c], acc);
    dst[j * K + c] = acc + unary[(int64_t)n * K + c];
  }
  __syncthreads();
}

template <typename TIO>
__global__ __launch_bounds__(kThreads) void lattice_kernel(const int64_t* __restrict__ ids,
                                                           const float* __restrict__ unary,
                                                           const int64_t* __restrict__ anchor,
                                                           const TIO* __restrict__ A,
                                                           const TIO* __restrict__ B,
                                                           const float* __restrict__ u_parts,
                                                           int32_t ksplit, int32_t slots, int32_t K,
                                                           int32_t r, int64_t vocab, int32_t n_rows,
                                                           float* __restrict__ scores) {
  extern __shared__ float smem[];
  float* s_u = smem;                                     // r
  float* s_w = s_u + r;                                  // K * (r + 1)
  float* s_bt = s_w + K * (r + 1);                       // r * K
  const int used = r + K * (r + 1) + r * K;
  int64_t* s_ids = reinterpret_cast<int64_t*>(smem + ((used + 1) & ~1));  // 2K, 8-byte aligned
  const int n = blockIdx.x;
  const int req = n / slots, s = n % slots;
  lattice_block<TIO>(ids, unary, anchor, A, B, u_parts, ksplit, n_rows, req, s, slots, K, r, vocab,
                     s_u, s_w, s_bt, s_ids, s_ids + K, scores + (int64_t)n * K * K);
}

// The same lattice block for the common case (rank a multiple of the 16-byte
// vector, 16-byte aligned tables): 16-byte gathers of the A and B rows, B
// kept one row per candidate in LDS, and each thread evaluates a TJ x TC
// tile of entries, so that every LDS read feeds TJ or TC chains.  Every
// entry is still one fma chain over k from 0 with w = A * u, so the result
// equals lattice_block's bit for bit.
// LDS: pred, cand [K] (int64), u [r], w [K][r+4] (fp32), B rows [K][r + 16 B].
struct LatticeTileLds {
  size_t pred, cand, u, w, b, bytes;
  int wstride, bstride;
};
__host__ __device__ inline LatticeTileLds lattice_tile_layout(int K, int r, int elem) {
  LatticeTileLds L;
  L.wstride = r + 4;
  L.bstride = r + 16 / elem;
  size_t o = 0;
  L.pred = o; o += (size_t)K * 8;
  L.cand = o; o += (size_t)K * 8;
  L.u = o;    o += (((size_t)r * 4) + 15) & ~(size_t)15;
  L.w = o;    o += (size_t)K * L.wstride * 4;
  L.b = o;    o += (size_t)K * L.bstride * elem;
  L.bytes = o;
  return L;
}

template <typename TIO, int TJ, int TC>
__global__ __launch_bounds__(kThreads) void lattice_tiled_kernel(
    const int64_t* __restrict__ ids, const float* __restrict__ unary, const int64_t* __restrict__ anchor,
    const TIO* __restrict__ A, const TIO* __restrict__ B, const float* __restrict__ u_parts, int32_t ksplit,
    int32_t slots, int32_t K, int32_t r, int64_t vocab, int32_t n_rows, float* __restrict__ scores) {
  constexpr int VEC = Elem<TIO>::kVec;
  extern __shared__ __align__(16) unsigned char lt_smem[];
  const LatticeTileLds L = lattice_tile_layout(K, r, (int)sizeof(TIO));
  int64_t* s_pred = reinterpret_cast<int64_t*>(lt_smem + L.pred);
  int64_t* s_cand = reinterpret_cast<int64_t*>(lt_smem + L.cand);
  float* s_u = reinterpret_cast<float*>(lt_smem + L.u);
  float* s_w = reinterpret_cast<float*>(lt_smem + L.w);
  TIO* s_b = reinterpret_cast<TIO*>(lt_smem + L.b);
  const int tid = threadIdx.x;
  const int n = blockIdx.x;
  const int req = n / slots, s = n % slots;

  for (int k = tid; k < r; k += kThreads) s_u[k] = sum_proj_slices(u_parts, ksplit, r, n, k);
  for (int j = tid; j < K; j += kThreads) {
    s_pred[j] = (s == 0) ? anchor[req] : ids[((int64_t)req * slots + s - 1) * K + j];
    s_cand[j] = ids[(int64_t)n * K + j];
  }
  __syncthreads();

  // gather: 16-byte pieces, unconditional loads (ids clamped into range),
  // out-of-range ids become NaN afterwards
  {
    constexpr int kPer = 4;
    const int ppr = r / VEC;
    const int n_pieces = K * ppr;                   // per table
    const int total = 2 * n_pieces;
    for (int base = 0; base < total; base += kThreads * kPer) {
      u32x4 raw[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = min(base + q * kThreads + tid, total - 1);
        const bool is_b = i >= n_pieces;
        const int ii = is_b ? i - n_pieces : i;
        const int j = ii / ppr, v = ii - j * ppr;
        const int64_t t = is_b ? s_cand[j] : s_pred[j];
        const int64_t tc = (t >= 0 && t < vocab) ? t : 0;
        raw[q] = ld16((is_b ? B : A) + tc * r + v * VEC);
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = base + q * kThreads + tid;
        if (i >= total) continue;
        const bool is_b = i >= n_pieces;
        const int ii = is_b ? i - n_pieces : i;
        const int j = ii / ppr, v = ii - j * ppr;
        const int64_t t = is_b ? s_cand[j] : s_pred[j];
        const bool ok = t >= 0 && t < vocab;
        if (is_b) {
          TIO nanrow[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) nanrow[e] = Elem<TIO>::nan_value();
          st16(s_b + (size_t)j * L.bstride + v * VEC, ok ? raw[q] : ld16(nanrow));
        } else {
          float a[VEC];
          unpack16(raw[q], a);
#pragma unroll
          for (int e = 0; e < VEC; e += 4)
            *reinterpret_cast<float4*>(s_w + j * L.wstride + v * VEC + e) =
                make_float4((ok ? a[e] : __builtin_nanf("")) * s_u[v * VEC + e],
                            (ok ? a[e + 1] : __builtin_nanf("")) * s_u[v * VEC + e + 1],
                            (ok ? a[e + 2] : __builtin_nanf("")) * s_u[v * VEC + e + 2],
                            (ok ? a[e + 3] : __builtin_nanf("")) * s_u[v * VEC + e + 3]);
        }
      }
    }
  }
  __syncthreads();

  // TJ x TC tiles of the K x K block; rows and columns past K are clamped
  // (computed, not stored)
  const int ntc = (K + TC - 1) / TC, ntiles = ((K + TJ - 1) / TJ) * ntc;
  for (int t = tid; t < ntiles; t += kThreads) {
    const int j0 = (t / ntc) * TJ, c0 = (t % ntc) * TC;
    const float* w[TJ];
    const TIO* b[TC];
#pragma unroll
    for (int a = 0; a < TJ; ++a) w[a] = s_w + min(j0 + a, K - 1) * L.wstride;
#pragma unroll
    for (int c = 0; c < TC; ++c) b[c] = s_b + (size_t)min(c0 + c, K - 1) * L.bstride;
    float acc[TJ][TC];
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
      for (int c = 0; c < TC; ++c) acc[a][c] = 0.f;
    for (int k0 = 0; k0 < r; k0 += VEC) {
      float bv[TC][VEC];
#pragma unroll
      for (int c = 0; c < TC; ++c) unpack16(ld16(b[c] + k0), bv[c]);
#pragma unroll
      for (int a = 0; a < TJ; ++a) {
#pragma unroll
        for (int e4 = 0; e4 < VEC; e4 += 4) {
          const float4 wv = *reinterpret_cast<const float4*>(w[a] + k0 + e4);
#pragma unroll
          for (int c = 0; c < TC; ++c) {
            acc[a][c] = fmaf(wv.x, bv[c][e4 + 0], acc[a][c]);
            acc[a][c] = fmaf(wv.y, bv[c][e4 + 1], acc[a][c]);
            acc[a][c] = fmaf(wv.z, bv[c][e4 + 2], acc[a][c]);
            acc[a][c] = fmaf(wv.w, bv[c][e4 + 3], acc[a][c]);
          }
        }
      }
    }
    float* dst = scores + (int64_t)n * K * K;
#pragma unroll
    for (int a = 0; a < TJ; ++a)
#pragma unroll
      for (int c = 0; c < TC; ++c)
        if (j0 + a < K && c0 + c < K) dst[(j0 + a) * K + c0 + c] = acc[a][c] + unary[(int64_t)n * K + c0 + c];
  }
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

// Lattice + walk for one request in one workgroup of 1024 threads, when the
// request's whole lattice and its staging fit in LDS.  Same per-entry
// arithmetic as lattice_block (u summed over the projection slices in order,
// w = A * u, fma chain over k from 0, + unary) and the same decision
// arithmetic as walk_decide, so the result is bit-identical to lattice_kernel
// followed by walk_kernel.  Phases, each one round of global loads or pure
// LDS work:
//   1. ids of every slot and its predecessor, u, unary, uniforms -> LDS
//   2. w = A[pred] (.) u (fp32) and the B[cand] rows -> LDS
//   3. one thread per lattice entry: its fma chain over k
//   4, 5. decide_and_walk: every row's decision in parallel, then the walked
//      path by pointer jumping, q rows and tokens written in parallel.
// LDS layout: pred ids [S][K], cand ids [S][K] (int64), w [S][K][r+4] (fp32;
// rows 16-byte aligned and 4 banks apart), B rows [S][K][r + 16 bytes]
// (storage dtype, one row per candidate), unary [S][K], scores [S][K][K+1]
// (then exponentials, then q), u [S][r] during the gather (the scan's
// second buffer during the walk), row maxima [S][K], uniforms [S], chosen
// index per row [S][K].
constexpr int kLWThreads = 1024;

struct LatticeWalkLds {
  size_t pred, cand, w, b, unary, sc, e, mx, un, next, bytes;
  int wstride, bstride;   // row strides of w (floats) and B rows (elements)
};

__host__ __device__ inline LatticeWalkLds lattice_walk_layout(int S, int K, int r, int elem) {
  LatticeWalkLds L;
  L.wstride = r + 4;
  L.bstride = r + 16 / elem;
  const size_t u_bytes = (size_t)S * r * 4, g_bytes = (size_t)S * K * 4;
  size_t o = 0;
  L.pred = o;  o += (size_t)S * K * 8;
  L.cand = o;  o += (size_t)S * K * 8;
  L.w = o;     o += (size_t)S * K * L.wstride * 4;
  L.b = o;     o += (size_t)S * K * L.bstride * elem;
  L.unary = o; o += (size_t)S * K * 4;
  L.sc = o;    o += (size_t)S * K * (K + 1) * 4;
  L.e = o;     o += u_bytes > g_bytes ? u_bytes : g_bytes;
  L.mx = o;    o += (size_t)S * K * 4;
  L.un = o;    o += (size_t)S * 4;
  L.next = o;  o += (size_t)S * K * 4;
  L.bytes = o;
  return L;
}

template <typename TIO>
__global__ __launch_bounds__(kLWThreads) void lattice_walk_kernel(
    const int64_t* __restrict__ ids, const float* __restrict__ unary, const int64_t* __restrict__ anchor,
    const TIO* __restrict__ A, const TIO* __restrict__ B, const float* __restrict__ u_parts, int32_t ksplit,
    int32_t slots, int32_t K, int32_t r, int64_t vocab, int32_t n_rows, const float* __restrict__ uniforms,
    const float* __restrict__ temperatures, const uint8_t* __restrict__ greedy_mask,
    float* __restrict__ scores_out, int64_t* __restrict__ tokens, float* __restrict__ q_out) {
  extern __shared__ __align__(16) unsigned char lw_smem[];
  const int req = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = slots;
  const LatticeWalkLds L = lattice_walk_layout(S, K, r, (int)sizeof(TIO));
  int64_t* s_pred = reinterpret_cast<int64_t*>(lw_smem + L.pred);
  int64_t* s_cand = reinterpret_cast<int64_t*>(lw_smem + L.cand);
  float* s_u = reinterpret_cast<float*>(lw_smem + L.e);      // u during the gather, the scan buffer afterwards
  float* s_w = reinterpret_cast<float*>(lw_smem + L.w);
  TIO* s_b = reinterpret_cast<TIO*>(lw_smem + L.b);
  float* s_unary = reinterpret_cast<float*>(lw_smem + L.unary);
  float* s_sc = reinterpret_cast<float*>(lw_smem + L.sc);
  float* s_mx = reinterpret_cast<float*>(lw_smem + L.mx);
  float* s_un = reinterpret_cast<float*>(lw_smem + L.un);
  int* s_next = reinterpret_cast<int*>(lw_smem + L.next);
  const int64_t row0 = (int64_t)req * S;            // first slot row of this request
  const int wstride = L.wstride, bstride = L.bstride;
  const FastDiv div_k(K), div_r(r);                 // every index below is < 2^16 (LDS bound)

  // ---- 1. ids, u (projection slices summed in order), unary, uniforms ----
  // Each pass issues every load of its items (uniform, ids, unary, all u
  // slices) before the first LDS write or add, so the phase costs one memory
  // round trip per pass (one pass whenever S * max(K, r) <= 1024).
  {
    const int n_e = S * K, n_u = S * r;
    const int n_all = max(max(n_e, n_u), S);
    for (int i = tid; i < n_all; i += kLWThreads) {
      const bool has_e = i < n_e, has_u = i < n_u, has_s = i < S;
      float uni = 0.f, un = 0.f;
      int64_t pred = 0, cand = 0;
      float v[kMaxProjSplit];
      if (has_s) uni = uniforms[row0 + i];
      if (has_e) {
        const int s = div_k.quot(i), j = i - s * K;
        pred = (s == 0) ? anchor[req] : ids[(row0 + s - 1) * K + j];
        cand = ids[row0 * K + i];
        un = unary[row0 * K + i];
      }
      if (has_u) {
        const int s = div_r.quot(i);
        load_proj_slices(u_parts, ksplit, r, row0 + s, i - s * r, v);
      }
      // keep the compiler from sinking the slice loads below the LDS writes
      // (which would start a second round trip after the first one drained)
      asm volatile("" ::: "memory");
      if (has_s) s_un[i] = uni;
      if (has_e) {
        s_pred[i] = pred;
        s_cand[i] = cand;
        s_unary[i] = un;
      }
      if (has_u) s_u[i] = add_proj_slices(v, ksplit);
    }
  }
  __syncthreads();

  // ---- 2. gather: w = A[pred] (.) u (fp32), B[cand] rows ------------------
  // 16-byte pieces of the table rows (r is a multiple of VEC, rows 16-byte
  // aligned).  Loads are unconditional (indices clamped into range) so that
  // every thread issues all of its loads before the first use; out-of-range
  // ids become NaN afterwards.
  {
    constexpr int VEC = Elem<TIO>::kVec;
    constexpr int kPer = 2;                          // pieces per thread per pass
    const int pieces_per_row = r / VEC;
    const int n_pieces = S * K * pieces_per_row;     // per table
    const int total = 2 * n_pieces;
    const FastDiv div_ppr(pieces_per_row);
    for (int base = 0; base < total; base += kLWThreads * kPer) {
      u32x4 raw[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = min(base + q * kLWThreads + tid, total - 1);
        const bool is_b = i >= n_pieces;
        const int ii = is_b ? i - n_pieces : i;
        const int sj = div_ppr.quot(ii), v = ii - sj * pieces_per_row;
        const int64_t t = is_b ? s_cand[sj] : s_pred[sj];
        const int64_t tc = (t >= 0 && t < vocab) ? t : 0;
        raw[q] = ld16((is_b ? B : A) + tc * r + v * VEC);
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = base + q * kLWThreads + tid;
        if (i >= total) continue;
        const bool is_b = i >= n_pieces;
        const int ii = is_b ? i - n_pieces : i;
        const int sj = div_ppr.quot(ii), v = ii - sj * pieces_per_row;
        const int s = div_k.quot(sj);
        const int64_t t = is_b ? s_cand[sj] : s_pred[sj];
        const bool ok = t >= 0 && t < vocab;
        if (is_b) {
          // the candidate's row piece as it is (NaN for an out-of-range id)
          TIO nanrow[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) nanrow[e] = Elem<TIO>::nan_value();
          st16(s_b + (size_t)sj * bstride + v * VEC, ok ? raw[q] : ld16(nanrow));
        } else {
          float a[VEC];
          unpack16(raw[q], a);
          float wv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            wv[e] = (ok ? a[e] : __builtin_nanf("")) * s_u[s * r + v * VEC + e];   // A[p] (.) project(h)
#pragma unroll
          for (int e = 0; e < VEC; e += 4)
            *reinterpret_cast<float4*>(s_w + sj * wstride + v * VEC + e) = make_float4(wv[e], wv[e + 1], wv[e + 2], wv[e + 3]);
        }
      }
    }
  }
  __syncthreads();

  // ---- 3. one thread per entry (s, j, c): fma chain over k from 0 ---------
  const int n_entries = S * K * K;
  for (int e = tid; e < n_entries; e += kLWThreads) {
    constexpr int VEC = Elem<TIO>::kVec;
    const int sj = div_k.quot(e), c = e - sj * K;
    const int s = div_k.quot(sj);
    const float* w = s_w + sj * wstride;
    const TIO* b = s_b + (size_t)(s * K + c) * bstride;
    float acc = 0.f;
    for (int k0 = 0; k0 < r; k0 += VEC) {
      float bv[VEC];
      unpack16(ld16(b + k0), bv);
#pragma unroll
      for (int e4 = 0; e4 < VEC; e4 += 4) {
        const float4 wv = *reinterpret_cast<const float4*>(w + k0 + e4);
        acc = fmaf(wv.x, bv[e4 + 0], acc);
        acc = fmaf(wv.y, bv[e4 + 1], acc);
        acc = fmaf(wv.z, bv[e4 + 2], acc);
        acc = fmaf(wv.w, bv[e4 + 3], acc);
      }
    }
    const float v = acc + s_unary[s * K + c];
    s_sc[sj * (K + 1) + c] = v;
    if (scores_out) scores_out[row0 * K * K + e] = v;
  }
  __syncthreads();

  // ---- 4, 5. every row's decision, then the walked path --------------------
  decide_and_walk<kLWThreads>(s_sc, s_mx, s_next, reinterpret_cast<int*>(lw_smem + L.e), s_un, S, K,
                              greedy_mask[req] != 0, temperatures[req], div_k, row0, s_cand, tokens, q_out);
}

}  // namespace

ProjPlan plan_proj(int32_t n_rows, int32_t rank, int32_t hidden, int32_t dtype) {
  ProjPlan p{};
  p.n_rows = n_rows;
  p.rank = rank;
  p.hidden = hidden;
  if (dtype == DFLASH_BF16) {
    // four row fragments per wave once there are rows enough to fill the chip
    p.frags = n_rows >= 4096 ? 4 : 1;
    p.row_tiles = (n_rows + kRowsPerWG * p.frags - 1) / (kRowsPerWG * p.frags);
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
  p.bytes = (size_t)proj_slice_stride(p.ksplit) * n_rows * rank * sizeof(float);
  p.bytes = (p.bytes + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_proj(const SelectArgs& a, const ProjPlan& p, hipStream_t stream) {
  const int n_rows = a.n_req * a.slots;
  if (n_rows == 0 || a.rank == 0) return hipSuccess;
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
    if (p.frags == 4) {
      DFLASH_PROJ_RT(4)
    } else {
      DFLASH_PROJ_RT(1)
    }
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

size_t lattice_lds_bytes(int K, int r) {
  const size_t used = (size_t)(r + K * (r + 1) + r * K);
  return ((used + 1) & ~(size_t)1) * sizeof(float) + 2 * (size_t)K * sizeof(int64_t);
}

hipError_t launch_lattice(const SelectArgs& a, const ProjPlan& p, hipStream_t stream) {
  const int n_rows = a.n_req * a.slots;
  if (n_rows == 0) return hipSuccess;
  const int vec = a.dtype == DFLASH_BF16 ? 8 : 4;
  if (a.rank % vec == 0 && (reinterpret_cast<uintptr_t>(a.sel_a) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(a.sel_b) & 15) == 0) {
    const size_t lds = lattice_tile_layout(a.top_k, a.rank, a.dtype == DFLASH_BF16 ? 2 : 4).bytes;
    // 2 x 2 tiles once the block has enough entries to keep the threads busy
    const bool big = a.top_k >= 16;
#define DFLASH_LT(TIO, TJ, TC)                                                                                    \
  hipLaunchKernelGGL((lattice_tiled_kernel<TIO, TJ, TC>), dim3(n_rows), dim3(kThreads), lds, stream, a.ids, a.unary, \
                     a.anchor, static_cast<const TIO*>(a.sel_a), static_cast<const TIO*>(a.sel_b), a.u_parts,       \
                     p.ksplit, a.slots, a.top_k, a.rank, a.vocab, n_rows, a.scores)
    if (a.dtype == DFLASH_BF16) {
      if (big) DFLASH_LT(uint16_t, 2, 2); else DFLASH_LT(uint16_t, 1, 1);
    } else {
      if (big) DFLASH_LT(float, 2, 2); else DFLASH_LT(float, 1, 1);
    }
#undef DFLASH_LT
    return hipGetLastError();
  }
  const size_t lds = lattice_lds_bytes(a.top_k, a.rank);
  if (a.dtype == DFLASH_BF16)
    hipLaunchKernelGGL(lattice_kernel<uint16_t>, dim3(n_rows), dim3(kThreads), lds, stream, a.ids, a.unary,
                       a.anchor, static_cast<const uint16_t*>(a.sel_a), static_cast<const uint16_t*>(a.sel_b),
                       a.u_parts, p.ksplit, a.slots, a.top_k, a.rank, a.vocab, n_rows, a.scores);
  else
    hipLaunchKernelGGL(lattice_kernel<float>, dim3(n_rows), dim3(kThreads), lds, stream, a.ids, a.unary,
                       a.anchor, static_cast<const float*>(a.sel_a), static_cast<const float*>(a.sel_b),
                       a.u_parts, p.ksplit, a.slots, a.top_k, a.rank, a.vocab, n_rows, a.scores);
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
  return lattice_walk_layout(slots, K, r, dtype == DFLASH_BF16 ? 2 : 4).bytes;
}

bool lattice_walk_fits(const SelectArgs& a) {
  const int vec = a.dtype == DFLASH_BF16 ? 8 : 4;
  return lattice_walk_lds_bytes(a.slots, a.top_k, a.rank, a.dtype) <= kLatticeWalkLdsMax && a.rank % vec == 0 &&
         (reinterpret_cast<uintptr_t>(a.sel_a) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.sel_b) & 15) == 0;
}

hipError_t launch_lattice_walk(const SelectArgs& a, const ProjPlan& p, const WalkArgs& w, float* scores_out,
                               hipStream_t stream) {
  if (a.n_req == 0 || a.slots == 0) return hipSuccess;
  if (!lattice_walk_fits(a)) return hipErrorInvalidValue;
  const size_t lds = lattice_walk_lds_bytes(a.slots, a.top_k, a.rank, a.dtype);
  const int n_rows = a.n_req * a.slots;
  if (a.dtype == DFLASH_BF16)
    hipLaunchKernelGGL((lattice_walk_kernel<uint16_t>), dim3(a.n_req), dim3(kLWThreads), lds, stream, a.ids, a.unary,
                       a.anchor, static_cast<const uint16_t*>(a.sel_a), static_cast<const uint16_t*>(a.sel_b),
                       a.u_parts, p.ksplit, a.slots, a.top_k, a.rank, a.vocab, n_rows, w.uniforms, w.temperatures,
                       w.greedy, scores_out, w.tokens, w.q);
  else
    hipLaunchKernelGGL((lattice_walk_kernel<float>), dim3(a.n_req), dim3(kLWThreads), lds, stream, a.ids, a.unary,
                       a.anchor, static_cast<const float*>(a.sel_a), static_cast<const float*>(a.sel_b), a.u_parts,
                       p.ksplit, a.slots, a.top_k, a.rank, a.vocab, n_rows, w.uniforms, w.temperatures, w.greedy,
                       scores_out, w.tokens, w.q);
  return hipGetLastError();
}

}  // namespace dflash

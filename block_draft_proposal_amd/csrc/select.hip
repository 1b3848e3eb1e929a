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

__device__ __forceinline__ const void* hidden_row(const void* hidden, int64_t req_stride,
                                                  int64_t slot_stride, int32_t slots, int row,
                                                  int elem_bytes) {
  const int req = row / slots, s = row % slots;
  return static_cast<const char*>(hidden) + ((int64_t)req * req_stride + (int64_t)s * slot_stride) * elem_bytes;
}

// RT = column tiles of 16 per wave (rank <= 16 * RT).
template <int RT>
__global__ __launch_bounds__(kThreads) void proj_mfma_kernel(const uint16_t* __restrict__ hidden,
                                                             int64_t req_stride, int64_t slot_stride,
                                                             int32_t slots, const uint16_t* __restrict__ P,
                                                             int32_t n_rows, int32_t rank, int32_t H,
                                                             int32_t kslice, float* __restrict__ u_parts) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_base = blockIdx.x * kRowsPerWG + wave * 16;
  const int split = blockIdx.y;
  const int k0 = split * kslice;
  const int k1 = min(H, k0 + kslice);
  const int arow = row_base + (lane & 15);
  const bool arow_ok = arow < n_rows;
  const uint16_t* hrow = arow_ok ? static_cast<const uint16_t*>(hidden_row(hidden, req_stride, slot_stride,
                                                                         slots, arow, 2))
                                 : hidden;
  const int kofs = 8 * (lane >> 4);
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kk = k0; kk < k1; kk += 32) {
    const int k = kk + kofs;
    const bool k_ok = k < k1;
    uint4 av = make_uint4(0u, 0u, 0u, 0u);
    if (arow_ok && k_ok) av = *reinterpret_cast<const uint4*>(hrow + k);
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int col = t * 16 + (lane & 15);
      uint4 bv = make_uint4(0u, 0u, 0u, 0u);
      if (col < rank && k_ok) bv = *reinterpret_cast<const uint4*>(P + (int64_t)col * H + k);
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[t], 0, 0, 0);
    }
  }
  // D layout: lane holds column (lane & 15), rows 4 * (lane >> 4) + v.
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int col = t * 16 + (lane & 15);
    if (col >= rank) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row_base + 4 * (lane >> 4) + v;
      if (row < n_rows) u_parts[((int64_t)split * n_rows + row) * rank + col] = acc[t][v];
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
  u_parts[t] = acc;
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
  for (int k = tid; k < r; k += kThreads) {
    float u = u_parts[(int64_t)n * r + k];
    for (int sp = 1; sp < ksplit; ++sp) u += u_parts[((int64_t)sp * n_rows + n) * r + k];
    s_u[k] = u;
  }
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

// One walk decision on a wave: lane j (< K) holds row[j].  Returns the chosen
// index (same on every lane) and sets q (this lane's probability).
__device__ __forceinline__ int walk_decide(float v, int lane, int K, bool greedy, float temp,
                                           float u, float& q) {
  const bool on = lane < K;
  if (greedy) {
    const float best = wave_max_f32(on ? v : -INFINITY);
    int idx = wave_min_i32((on && v == best) ? lane : K);
    if (idx > K - 1) idx = 0;             // all-NaN row: no maximum; stay in range
    q = (lane == idx) ? 1.f : 0.f;
    return idx;
  }
  const float t = fmaxf(temp, 1e-5f);
  const float xs = v / t;
  const float mx = wave_max_f32(on ? xs : -INFINITY);
  // exp rounded once to fp32 (from the fp64 exponential)
  const float e = on ? (float)exp((double)(xs - mx)) : 0.f;
  float total = 0.f;
  for (int j = 0; j < K; ++j) total += __shfl(e, j, 64);        // left to right
  const float p = e / total;
  float cdf = 0.f;
  for (int j = 0; j < K; ++j) {
    const float pj = __shfl(p, j, 64);
    if (j <= lane) cdf += pj;                                     // C_lane, left to right
  }
  const unsigned long long hit = __ballot(on && u >= cdf);
  const int cnt = __popcll(hit);
  q = on ? p : 0.f;
  return cnt < K - 1 ? cnt : K - 1;
}

constexpr int kWalkLdsFloats = 16384;   // 64 KiB: S * K * K staged when it fits

__global__ __launch_bounds__(kThreads) void walk_kernel(const float* __restrict__ scores,
                                                        const int64_t* __restrict__ ids,
                                                        const float* __restrict__ uniforms,
                                                        const float* __restrict__ temperatures,
                                                        const uint8_t* __restrict__ greedy_mask,
                                                        int32_t slots, int32_t K,
                                                        int64_t* __restrict__ tokens,
                                                        float* __restrict__ q_out) {
  extern __shared__ float s_sc[];
  const int req = blockIdx.x;
  const int64_t per_req = (int64_t)slots * K * K;
  const float* src = scores + (int64_t)req * per_req;
  const bool staged = per_req <= kWalkLdsFloats;
  if (staged) {
    for (int64_t i = threadIdx.x; i < per_req; i += kThreads) s_sc[i] = src[i];
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const bool greedy = greedy_mask[req] != 0;
  const float temp = temperatures[req];
  int prev = 0;
  for (int s = 0; s < slots; ++s) {
    const int64_t row_off = ((int64_t)s * K + prev) * K;
    const float v = lane < K ? (staged ? s_sc[row_off + lane] : src[row_off + lane]) : 0.f;
    const float u = uniforms[(int64_t)req * slots + s];
    float q;
    const int idx = walk_decide(v, lane, K, greedy, temp, u, q);
    const int64_t n = (int64_t)req * slots + s;
    if (lane < K) q_out[n * K + lane] = q;
    if (lane == 0) tokens[n] = ids[n * K + idx];
    prev = idx;
  }
}

}  // namespace

ProjPlan plan_proj(int32_t n_rows, int32_t rank, int32_t hidden, int32_t dtype) {
  ProjPlan p{};
  p.n_rows = n_rows;
  p.rank = rank;
  p.hidden = hidden;
  if (dtype == DFLASH_BF16) {
    p.row_tiles = (n_rows + kRowsPerWG - 1) / kRowsPerWG;
    int ks = p.row_tiles > 0 ? (512 + p.row_tiles - 1) / p.row_tiles : 1;
    const int max_ks = hidden / 256 > 1 ? hidden / 256 : 1;
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
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
  if (a.dtype == DFLASH_BF16) {
    const dim3 grid(p.row_tiles, p.ksplit);
    const uint16_t* h = static_cast<const uint16_t*>(a.hidden);
    const uint16_t* P = static_cast<const uint16_t*>(a.proj);
    const int tiles = (a.rank + 15) / 16;
#define DFLASH_PROJ(RT)                                                                        \
  hipLaunchKernelGGL(proj_mfma_kernel<RT>, grid, dim3(kThreads), 0, stream, h, a.hidden_req_stride, \
                     a.hidden_slot_stride, a.slots, P, n_rows, a.rank, a.hidden_size, p.kslice,    \
                     a.u_parts)
    if (tiles <= 1) DFLASH_PROJ(1);
    else if (tiles <= 2) DFLASH_PROJ(2);
    else if (tiles <= 4) DFLASH_PROJ(4);
    else if (tiles <= 8) DFLASH_PROJ(8);
    else return hipErrorInvalidValue;   // rank > 128 is rejected by the API layer
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
  const int64_t per_req = (int64_t)a.slots * a.top_k * a.top_k;
  const size_t lds = per_req <= kWalkLdsFloats ? (size_t)per_req * sizeof(float) : 0;
  hipLaunchKernelGGL(walk_kernel, dim3(a.n_req), dim3(kThreads), lds, stream, a.scores, a.ids, a.uniforms,
                     a.temperatures, a.greedy, a.slots, a.top_k, a.tokens, a.q);
  return hipGetLastError();
}

}  // namespace dflash

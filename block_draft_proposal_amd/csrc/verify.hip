// Verify and commit of a drafted block.
//
// Contract ("[Spec] DFlash2: local convolution + candidate selector",
// executive summary and walk-kernel excerpt): verify checks the drafted
// tokens against the distribution the walk actually drew them from (a point
// mass on greedy rows, the softmax over the candidates otherwise), which is
// what makes the draft lossless; the worker then commits the accepted tokens
// and places the bonus token after them.  Rule (the standard rejection rule
// of speculative sampling; the pages do not print it): for s = 0, 1, ... keep
// drafted token x while u_accept[s] * q(x) < p_s(x); at the first rejection
// commit one token drawn from max(0, p_s - q_s) renormalised; after S kept
// tokens commit one drawn from p_S.  p_s = softmax(z_s / T) over the valid
// ids (T clamped to >= 1e-5), or the point mass on the lowest-id maximum for
// a greedy request.  Draws are inverse CDFs in id order with u_residual.
//
// Design: row statistics first, one workgroup per target row (all R (S+1)
// rows in parallel, so the logits stream through once): maximum, its lowest
// id, and the softmax normaliser sum_v exp((z_v - zmax) / T) in fp64 (one
// online pass, rescaled when the running maximum grows).  Then one workgroup
// per request: one thread takes the accept decisions in slot order (fp64:
// u q(x) is exact, p(x) from one logit and the row's statistics), and all
// threads draw the committed token: each sums the weights of a contiguous
// range of ids in fp64, the range sums are scanned in order, and the thread
// whose range holds the crossing walks it again to find the id.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kVerifyThreads = 256;
constexpr int kCommitThreads = 1024;

template <typename TIO>
__device__ __forceinline__ double logit_at(const TIO* z, int64_t v);
template <>
__device__ __forceinline__ double logit_at<uint16_t>(const uint16_t* z, int64_t v) {
  return (double)bf16_to_f32(z[v]);
}
template <>
__device__ __forceinline__ double logit_at<float>(const float* z, int64_t v) {
  return (double)z[v];
}

__device__ __forceinline__ double clamp_temperature(float t) { return fmax((double)t, 1e-5); }

// Statistics of one segment of one target row: the segment's maximum, its
// lowest id, and (sampled requests) sum exp((z - m) / T) over the segment,
// relative to the segment's own maximum.  Pass 1 finds the maximum with
// branch-free selects (each thread walks its ids in increasing order, so a
// strict comparison keeps the lowest id); pass 2 sums against that fixed
// maximum.  Loads are issued kUnroll vectors at a time.
constexpr int kUnroll = 4;

template <typename TIO>
__global__ __launch_bounds__(kVerifyThreads) void verify_stats_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t rows_per_req, int64_t valid,
    const float* __restrict__ temperatures, const uint8_t* __restrict__ greedy_mask, VerifyRowStats* __restrict__ stats) {
  __shared__ float s_m[kVerifyThreads];
  __shared__ int64_t s_a[kVerifyThreads];
  __shared__ double s_s[kVerifyThreads];
  const int64_t row = blockIdx.x / kVerifySegs;
  const int seg = (int)(blockIdx.x % kVerifySegs);
  const int r = (int)(row / rows_per_req);
  const int tid = threadIdx.x;
  const TIO* z = logits + row * row_stride;
  constexpr int VEC = Elem<TIO>::kVec;
  // the row as: `head` single elements up to the first 16-byte boundary,
  // nvec whole vectors, then single elements; segment `seg` takes its share
  // of the vectors, the first segment the head and the last the tail
  int64_t head = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(z) & 15u)) & 15u) / sizeof(TIO));
  if (head > valid) head = valid;
  const int64_t nvec = (valid - head) / VEC;
  const int64_t vlo = nvec * seg / kVerifySegs, vhi = nvec * (seg + 1) / kVerifySegs;
  const int64_t slo = 0, shi = seg == 0 ? head : 0;           // singles before the vectors
  const int64_t tlo = seg == kVerifySegs - 1 ? head + nvec * VEC : valid, thi = valid;   // singles after

  // pass 1: maximum and its lowest id
  float m = -INFINITY;
  int64_t arg = -1;
  auto see = [&](float v, int64_t id) {
    const bool up = v > m;                      // -inf and NaN never raise it
    m = up ? v : m;
    arg = up ? id : arg;
  };
  for (int64_t v = slo + tid; v < shi; v += kVerifyThreads) see(Elem<TIO>::to_f32(z[v]), v);
  for (int64_t i0 = vlo + tid; i0 < vhi; i0 += kVerifyThreads * kUnroll) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kVerifyThreads;
      raw[u] = ld16(z + head + (i < vhi ? i : vlo) * VEC);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kVerifyThreads;
      if (i >= vhi) break;
      float f[VEC];
      unpack16(raw[u], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) see(f[e], head + i * VEC + e);
    }
  }
  for (int64_t v = tlo + tid; v < thi; v += kVerifyThreads) see(Elem<TIO>::to_f32(z[v]), v);
  s_m[tid] = m;
  s_a[tid] = arg;
  __syncthreads();
  for (int w = kVerifyThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const float mb = s_m[tid + w];
      const int64_t ab = s_a[tid + w];
      if (mb > s_m[tid] || (mb == s_m[tid] && ab >= 0 && (s_a[tid] < 0 || ab < s_a[tid]))) {
        s_m[tid] = mb;
        s_a[tid] = ab;
      }
    }
    __syncthreads();
  }
  const float mseg = s_m[0];
  const int64_t aseg = s_a[0];

  // pass 2 (sampled requests): sum exp((z - mseg) / T) in fp64
  double sum = 0.0;
  if (greedy_mask[r] == 0 && mseg > -INFINITY) {
    const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
    const double mm = (double)mseg;
    auto add = [&](float v) {
      if (v > -INFINITY) sum += exp(((double)v - mm) * inv_t);
    };
    for (int64_t v = slo + tid; v < shi; v += kVerifyThreads) add(Elem<TIO>::to_f32(z[v]));
    for (int64_t i0 = vlo + tid; i0 < vhi; i0 += kVerifyThreads * kUnroll) {
      u32x4 raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kVerifyThreads;
        raw[u] = ld16(z + head + (i < vhi ? i : vlo) * VEC);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kVerifyThreads;
        if (i >= vhi) break;
        float f[VEC];
        unpack16(raw[u], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) add(f[e]);
      }
    }
    for (int64_t v = tlo + tid; v < thi; v += kVerifyThreads) add(Elem<TIO>::to_f32(z[v]));
  }
  s_s[tid] = sum;
  __syncthreads();
  for (int w = kVerifyThreads / 2; w > 0; w >>= 1) {      // fixed tree: the same order every launch
    if (tid < w) s_s[tid] += s_s[tid + w];
    __syncthreads();
  }
  if (tid == 0) stats[blockIdx.x] = VerifyRowStats{(double)mseg, s_s[0], aseg};
}

// The row's statistics from its segments, in segment (id) order: the maximum,
// its lowest id (the first segment that holds it), and the normaliser
// sum_k s_k exp((m_k - m) / T).
__device__ __forceinline__ VerifyRowStats merge_segments(const VerifyRowStats* st, double inv_t) {
  VerifyRowStats o{-INFINITY, 0.0, 0};
  for (int k = 0; k < kVerifySegs; ++k)
    if (st[k].m > o.m) {
      o.m = st[k].m;
      o.arg = st[k].arg;
    }
  if (o.m > -INFINITY)
    for (int k = 0; k < kVerifySegs; ++k)
      if (st[k].m > -INFINITY) o.s += st[k].s * exp((st[k].m - o.m) * inv_t);
  return o;
}

template <typename TIO>
__global__ __launch_bounds__(kCommitThreads) void verify_commit_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t S, int32_t K, int64_t valid,
    const int64_t* __restrict__ cand_ids, const float* __restrict__ q, const int64_t* __restrict__ tokens,
    const float* __restrict__ u_accept, const float* __restrict__ u_residual, const float* __restrict__ temperatures,
    const uint8_t* __restrict__ greedy_mask, const VerifyRowStats* __restrict__ stats, int32_t* __restrict__ accepted,
    int64_t* __restrict__ committed) {
  __shared__ int s_n;
  __shared__ int s_nc;
  __shared__ int64_t s_cid[kMaxTopK];
  __shared__ double s_cq[kMaxTopK];
  __shared__ double s_sum[kCommitThreads];
  __shared__ int s_chunk;
  __shared__ double s_base;
  __shared__ int64_t s_tok;
  const int r = blockIdx.x, tid = threadIdx.x;
  const bool greedy = greedy_mask[r] != 0;
  const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
  if (tid == 0) {
    int n = 0;
    for (; n < S; ++n) {
      const int64_t x = tokens[(int64_t)r * S + n];
      const VerifyRowStats st = merge_segments(stats + ((int64_t)r * (S + 1) + n) * kVerifySegs, inv_t);
      bool keep;
      if (greedy) {
        keep = x == st.arg;
      } else {
        double qx = 0.0;                                     // a token outside the candidates has q = 0
        for (int j = 0; j < K; ++j)
          if (cand_ids[((int64_t)r * S + n) * K + j] == x) qx = (double)q[((int64_t)r * S + n) * K + j];
        const TIO* z = logits + ((int64_t)r * (S + 1) + n) * row_stride;
        const double px = (x >= 0 && x < valid && st.m > -INFINITY)
                              ? exp((logit_at(z, x) - st.m) * inv_t) / st.s : 0.0;
        keep = (double)u_accept[(int64_t)r * S + n] * qx < px;
      }
      if (!keep) break;
    }
    s_n = n;
    // the rejected slot's candidates, by id, for the residual max(0, p - q)
    int nc = 0;
    if (n < S && !greedy) {
      for (int j = 0; j < K; ++j) {
        const int64_t id = cand_ids[((int64_t)r * S + n) * K + j];
        if (id < 0 || id >= valid) continue;
        int at = nc++;
        while (at > 0 && s_cid[at - 1] > id) {
          s_cid[at] = s_cid[at - 1];
          s_cq[at] = s_cq[at - 1];
          --at;
        }
        s_cid[at] = id;
        s_cq[at] = (double)q[((int64_t)r * S + n) * K + j];
      }
    }
    s_nc = nc;
  }
  __syncthreads();
  const int n = s_n;
  const int64_t row = (int64_t)r * (S + 1) + n;
  const VerifyRowStats st = merge_segments(stats + row * kVerifySegs, inv_t);
  int64_t tok;
  if (greedy || !(st.m > -INFINITY)) {
    tok = st.arg;
  } else {
    // weights w(v) = p(v) (bonus) or max(0, p(v) - q(v)) (after a rejection),
    // summed per contiguous id range in id order
    const TIO* z = logits + row * row_stride;
    const int nc = s_nc;
    const int64_t chunk = (valid + kCommitThreads - 1) / kCommitThreads;
    const int64_t v0 = (int64_t)tid * chunk, v1 = v0 + chunk < valid ? v0 + chunk : valid;
    auto weight = [&](int64_t v, int& ci) {
      double w = exp((logit_at(z, v) - st.m) * inv_t) / st.s;
      if (ci < nc && s_cid[ci] == v) {
        w = w - s_cq[ci] > 0.0 ? w - s_cq[ci] : 0.0;
        ++ci;
      }
      return w;
    };
    int ci0 = 0;
    while (ci0 < nc && s_cid[ci0] < v0) ++ci0;
    double sum = 0.0;
    {
      int ci = ci0;
      for (int64_t v = v0; v < v1; ++v) sum += weight(v, ci);
    }
    s_sum[tid] = sum;
    __syncthreads();
    if (tid == 0) {
      double total = 0.0;
      for (int t = 0; t < kCommitThreads; ++t) total += s_sum[t];
      const double target = (double)u_residual[r] * total;
      double base = 0.0;
      int c = -1, last = -1;
      for (int t = 0; t < kCommitThreads; ++t) {
        if (s_sum[t] > 0.0) last = t;
        if (c < 0 && base + s_sum[t] > target && s_sum[t] > 0.0) {
          c = t;
          break;
        }
        base += s_sum[t];
      }
      if (c < 0) {                                         // rounding left the target at the very end
        c = last;
        base = 0.0;
        for (int t = 0; t < c; ++t) base += s_sum[t];
      }
      s_chunk = c;
      s_base = base;
    }
    __syncthreads();
    if (tid == s_chunk) {
      double total = 0.0;                                  // the same sum, in the same order, as above
      for (int t = 0; t < kCommitThreads; ++t) total += s_sum[t];
      const double goal = (double)u_residual[r] * total;
      double acc = s_base;
      int ci = ci0;
      int64_t pick = -1, lastpos = -1;
      for (int64_t v = v0; v < v1; ++v) {
        const double w = weight(v, ci);
        if (w > 0.0) lastpos = v;
        acc += w;
        if (acc > goal && w > 0.0) {
          pick = v;
          break;
        }
      }
      s_tok = pick >= 0 ? pick : lastpos;
    }
    __syncthreads();
    tok = s_tok;
  }
  if (tid == 0) accepted[r] = n;
  for (int s = tid; s <= S; s += kCommitThreads) {
    int64_t c = -1;
    if (s < n) c = tokens[(int64_t)r * S + s];
    else if (s == n) c = tok;
    committed[(int64_t)r * (S + 1) + s] = c;
  }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  if (a.n_req == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.n_req * (a.slots + 1);
  VerifyRowStats* stats = static_cast<VerifyRowStats*>(a.workspace);   // [rows][kVerifySegs]
#define DFLASH_VERIFY(TIO)                                                                                   \
  hipLaunchKernelGGL(verify_stats_kernel<TIO>, dim3((unsigned)(rows * kVerifySegs)), dim3(kVerifyThreads), 0,    \
                     stream,                                                                                  \
                     static_cast<const TIO*>(a.logits), a.row_stride, a.slots + 1, a.valid_vocab,             \
                     a.temperatures, a.greedy_mask, stats);                                                   \
  {                                                                                                          \
    hipError_t e = hipGetLastError();                                                                        \
    if (e != hipSuccess) return e;                                                                           \
  }                                                                                                          \
  hipLaunchKernelGGL(verify_commit_kernel<TIO>, dim3((unsigned)a.n_req), dim3(kCommitThreads), 0, stream,      \
                     static_cast<const TIO*>(a.logits), a.row_stride, a.slots, a.top_k, a.valid_vocab,        \
                     a.cand_ids, a.q, a.tokens, a.u_accept, a.u_residual, a.temperatures, a.greedy_mask,      \
                     stats, a.accepted_out, a.committed_out)
  if (a.dtype == DFLASH_BF16) {
    DFLASH_VERIFY(uint16_t);
  } else {
    DFLASH_VERIFY(float);
  }
#undef DFLASH_VERIFY
  return hipGetLastError();
}

}  // namespace dflash

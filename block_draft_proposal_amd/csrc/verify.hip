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

// Running (max, lowest id of the max, normaliser relative to the max).
struct Online {
  double m, s;
  int64_t arg;
};

__device__ __forceinline__ void online_add(Online& o, double z, int64_t v, double inv_t, bool sum) {
  if (!(z > -INFINITY)) return;                          // -inf (and NaN) weigh nothing
  if (z > o.m) {
    if (sum) o.s = (o.m > -INFINITY ? o.s * exp((o.m - z) * inv_t) : 0.0) + 1.0;
    o.m = z;
    o.arg = v;
  } else {
    if (sum) o.s += exp((z - o.m) * inv_t);
    if (z == o.m && v < o.arg) o.arg = v;
  }
}

__device__ __forceinline__ Online online_merge(Online a, Online b, double inv_t, bool sum) {
  if (!(b.m > -INFINITY)) return a;
  if (!(a.m > -INFINITY)) return b;
  Online o;
  o.m = a.m > b.m ? a.m : b.m;
  o.arg = a.m > b.m ? a.arg : (b.m > a.m ? b.arg : (a.arg < b.arg ? a.arg : b.arg));
  o.s = sum ? a.s * exp((a.m - o.m) * inv_t) + b.s * exp((b.m - o.m) * inv_t) : 0.0;
  return o;
}

template <typename TIO>
__global__ __launch_bounds__(kVerifyThreads) void verify_stats_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t rows_per_req, int64_t valid,
    const float* __restrict__ temperatures, const uint8_t* __restrict__ greedy_mask, VerifyRowStats* __restrict__ stats) {
  __shared__ double s_m[kVerifyThreads], s_s[kVerifyThreads];
  __shared__ int64_t s_a[kVerifyThreads];
  const int64_t row = blockIdx.x;
  const int r = (int)(row / rows_per_req);
  const int tid = threadIdx.x;
  const TIO* z = logits + row * row_stride;
  const bool sum = greedy_mask[r] == 0;
  const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
  Online o{-INFINITY, 0.0, 0};
  constexpr int VEC = Elem<TIO>::kVec;
  // rows need not be 16-byte aligned: the elements before the first aligned
  // 16 bytes and after the last whole vector are read one by one
  int64_t head = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(z) & 15u)) & 15u) / sizeof(TIO));
  if (head > valid) head = valid;
  const int64_t nvec = (valid - head) / VEC;
  for (int64_t v = tid; v < head; v += kVerifyThreads) online_add(o, logit_at(z, v), v, inv_t, sum);
  for (int64_t i = tid; i < nvec; i += kVerifyThreads) {
    float f[VEC];
    unpack16(ld16(z + head + i * VEC), f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) online_add(o, (double)f[e], head + i * VEC + e, inv_t, sum);
  }
  for (int64_t v = head + nvec * VEC + tid; v < valid; v += kVerifyThreads)
    online_add(o, logit_at(z, v), v, inv_t, sum);
  s_m[tid] = o.m;
  s_s[tid] = o.s;
  s_a[tid] = o.arg;
  __syncthreads();
  for (int w = kVerifyThreads / 2; w > 0; w >>= 1) {      // tree merge: same order every launch
    if (tid < w) {
      const Online a{s_m[tid], s_s[tid], s_a[tid]}, b{s_m[tid + w], s_s[tid + w], s_a[tid + w]};
      const Online c = online_merge(a, b, inv_t, sum);
      s_m[tid] = c.m;
      s_s[tid] = c.s;
      s_a[tid] = c.arg;
    }
    __syncthreads();
  }
  if (tid == 0) stats[row] = VerifyRowStats{s_m[0], s_s[0], s_a[0]};
}

template <typename TIO>
__global__ __launch_bounds__(kVerifyThreads) void verify_commit_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t S, int32_t K, int64_t valid,
    const int64_t* __restrict__ cand_ids, const float* __restrict__ q, const int64_t* __restrict__ tokens,
    const float* __restrict__ u_accept, const float* __restrict__ u_residual, const float* __restrict__ temperatures,
    const uint8_t* __restrict__ greedy_mask, const VerifyRowStats* __restrict__ stats, int32_t* __restrict__ accepted,
    int64_t* __restrict__ committed) {
  __shared__ int s_n;
  __shared__ int s_nc;
  __shared__ int64_t s_cid[kMaxTopK];
  __shared__ double s_cq[kMaxTopK];
  __shared__ double s_sum[kVerifyThreads];
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
      const VerifyRowStats st = stats[(int64_t)r * (S + 1) + n];
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
  const VerifyRowStats st = stats[row];
  int64_t tok;
  if (greedy || !(st.m > -INFINITY)) {
    tok = st.arg;
  } else {
    // weights w(v) = p(v) (bonus) or max(0, p(v) - q(v)) (after a rejection),
    // summed per contiguous id range in id order
    const TIO* z = logits + row * row_stride;
    const int nc = s_nc;
    const int64_t chunk = (valid + kVerifyThreads - 1) / kVerifyThreads;
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
      for (int t = 0; t < kVerifyThreads; ++t) total += s_sum[t];
      const double target = (double)u_residual[r] * total;
      double base = 0.0;
      int c = -1, last = -1;
      for (int t = 0; t < kVerifyThreads; ++t) {
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
      for (int t = 0; t < kVerifyThreads; ++t) total += s_sum[t];
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
  for (int s = tid; s <= S; s += kVerifyThreads) {
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
  VerifyRowStats* stats = static_cast<VerifyRowStats*>(a.workspace);
#define DFLASH_VERIFY(TIO)                                                                                   \
  hipLaunchKernelGGL(verify_stats_kernel<TIO>, dim3((unsigned)rows), dim3(kVerifyThreads), 0, stream,          \
                     static_cast<const TIO*>(a.logits), a.row_stride, a.slots + 1, a.valid_vocab,             \
                     a.temperatures, a.greedy_mask, stats);                                                   \
  {                                                                                                          \
    hipError_t e = hipGetLastError();                                                                        \
    if (e != hipSuccess) return e;                                                                           \
  }                                                                                                          \
  hipLaunchKernelGGL(verify_commit_kernel<TIO>, dim3((unsigned)a.n_req), dim3(kVerifyThreads), 0, stream,      \
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

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
// Design: row statistics first, kVerifySegs workgroups per target row (all
// R (S+1) rows in parallel, so the logits stream through once).  Each wave
// owns a contiguous quarter of its segment and reads it in coalesced 16-byte
// vectors.  Pass 1: the maximum (fp32 max; NaN and -inf never raise it), then
// its lowest id from the few threads that hold it.  Pass 2 (sampled
// requests): exp((z - m) / T) in fp64 summed per chunk of 64 vectors (one per
// lane), the chunk sums stored in id order; the segment's sum is the sum of
// its chunks.  Then one workgroup per request: one thread takes the accept
// decisions in slot order (fp64: u q(x) is exact, p(x) from one logit and the
// row's statistics), and the committed token is drawn from the stored chunk
// sums of its row: the chunks (corrected at the candidate ids for a residual
// draw) are scanned in id order to find the one holding the crossing, and
// only that chunk's ids are evaluated one by one.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kVerifyThreads = 256;   // 4 waves per (row, segment)
constexpr int kVerifyWaves = kVerifyThreads / 64;
constexpr int kCommitThreads = 1024;
constexpr int kRowsLds = 64;          // target rows of a request whose statistics the commit keeps in LDS
constexpr int kChunkVecs = 64;        // vectors of one chunk: one per lane of a wave
constexpr int kBatch = 4;             // chunks whose per-lane sums a wave reduces together
constexpr int kUnroll = 4;            // vectors per lane in flight (sums)
constexpr int kUnrollMax = 8;         // vectors per lane in flight (maximum)

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

// e^x for x <= 0 in fp64 (every exponent here is (z - m) / T with m the
// maximum).  Cody and Waite's reduction x = k ln2 + r, |r| <= ln2 / 2, with
// ln2 split into a high part of 32 significant bits (so k * hi is exact) and
// the remainder; e^r by its Taylor series to degree 13 (truncation below
// 2^-57 there), by Horner's rule; then scaled by 2^k.  Below -745.2 (and for
// -inf or NaN) the result is 0.
__device__ __forceinline__ double exp_nonpos(double x) {
  if (!(x > -745.2)) return 0.0;
  const double k = rint(x * 0x1.71547652b82fep+0);                 // x / ln2
  double r = fma(-k, 0x1.62e42ffp-1, x);                            // ln2, high 32 bits
  r = fma(-k, -0x1.718432a1b0e26p-35, r);                           // ln2 - high part
  double p = 0x1.6124613a86d09p-33;                                 // 1/13!
  p = fma(p, r, 0x1.1eed8eff8d898p-29);                             // 1/12!
  p = fma(p, r, 0x1.ae64567f544e4p-26);                             // 1/11!
  p = fma(p, r, 0x1.27e4fb7789f5cp-22);                             // 1/10!
  p = fma(p, r, 0x1.71de3a556c734p-19);                             // 1/9!
  p = fma(p, r, 0x1.a01a01a01a01ap-16);                             // 1/8!
  p = fma(p, r, 0x1.a01a01a01a01ap-13);                             // 1/7!
  p = fma(p, r, 0x1.6c16c16c16c17p-10);                             // 1/6!
  p = fma(p, r, 0x1.1111111111111p-7);                              // 1/5!
  p = fma(p, r, 0x1.5555555555555p-5);                              // 1/4!
  p = fma(p, r, 0x1.5555555555555p-3);                              // 1/3!
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)k);
}

// e^x for x <= 0, table-driven (Tang's method), here with a 256-entry table:
// x = (k / 256) ln2 + r with |r| <= ln2 / 512, so e^x = 2^(k >> 8)
// 2^((k & 255) / 256) e^r.  The powers 2^(j/256) sit in an LDS table
// (exp_table_fill), e^r is its Taylor series to degree 4 (truncation below
// 2^-54 on that range; 32- and 64-entry tables with degrees 6 and 5 measured
// the same); k (/ 256) ln2
// is subtracted in the same two parts as in exp_nonpos.  About 3 ulp; zero
// below -745.2 and for -inf or NaN, like exp_nonpos.
constexpr int kExpBits = 8;                 // table of 2^(j / 2^kExpBits)
constexpr int kExpTable = 1 << kExpBits;
// Taylor degree for |r| <= ln2 / 2^(kExpBits+1): truncation below 2^-54
constexpr int kExpDegree = kExpBits >= 8 ? 4 : kExpBits >= 6 ? 5 : kExpBits == 5 ? 6 : 7;

__device__ __forceinline__ void exp_table_fill(double* t) {
  for (int j = threadIdx.x; j < kExpTable; j += blockDim.x)   // 2^(j/256) = 2 e^((j - 256) ln2 / 256)
    t[j] = 2.0 * exp_nonpos((double)(j - kExpTable) * (0x1.62e42fefa39efp-1 / kExpTable));
}

// exp_tab in two steps, so that a caller can issue several table reads
// before it needs them: the reduction (k, r) and the table index, then the
// polynomial and the scaling.  x is first clamped to -745.2, where the
// result rounds to 0 (so do -inf and NaN, which the clamp maps there); k is
// rounded by adding 1.5 * 2^52, which leaves it in the low bits of the sum.
struct ExpReduced {
  double r;
  int k;
};

__device__ __forceinline__ ExpReduced exp_tab_reduce(double x) {
  x = fmax(x, -745.2);
  const double t = fma(x, 0x1.71547652b82fep+0 * kExpTable, 0x1.8p52);    // 1.5 * 2^52 + k
  const double k = t - 0x1.8p52;
  double r = fma(-k, 0x1.62e42ffp-1 / kExpTable, x);
  ExpReduced o;
  o.r = fma(-k, -0x1.718432a1b0e26p-35 / kExpTable, r);
  o.k = (int)(uint32_t)__double_as_longlong(t);
  return o;
}

__device__ __forceinline__ double exp_tab_finish(const ExpReduced& a, double table_value) {
  // 1/d! for d = 0..7, rounded to double
  constexpr double c[8] = {1.0, 1.0, 0.5, 0x1.5555555555555p-3, 0x1.5555555555555p-5, 0x1.1111111111111p-7,
                           0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13};
  double p = fma(a.r, c[kExpDegree], c[kExpDegree - 1]);
#pragma unroll
  for (int d = kExpDegree - 2; d >= 0; --d) p = fma(p, a.r, c[d]);
  return ldexp(table_value * p, a.k >> kExpBits);
}

__device__ __forceinline__ double exp_tab(double x, const double* t) {
  const ExpReduced a = exp_tab_reduce(x);
  return exp_tab_finish(a, t[a.k & (kExpTable - 1)]);
}

// sum_e exp_tab(f[e] inv_t - m_scaled) in order e = 0, 1, ..., with all
// table reads issued together (m_scaled = m inv_t: the exponent of a logit z
// against the maximum m is always formed as fma(z, inv_t, -m inv_t))
template <int VEC>
__device__ __forceinline__ double exp_tab_sum(const float (&f)[VEC], double m_scaled, double inv_t, const double* t) {
  ExpReduced a[VEC];
  double tv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) a[e] = exp_tab_reduce(fma((double)f[e], inv_t, -m_scaled));
#pragma unroll
  for (int e = 0; e < VEC; ++e) tv[e] = t[a[e].k & (kExpTable - 1)];
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) s += exp_tab_finish(a[e], tv[e]);
  return s;
}

// kBatch per-lane values v[0..kBatch) summed over the 64 lanes of a wave,
// the sums scattered: halving steps across the high lane bits (each lane
// keeps the half its bit selects and adds the partner's copy of it), then
// full steps across the low kLaneGroup bits.  Lane l ends with the sum of
// value l / kLaneGroup in v[0]; the order of the additions is fixed.
constexpr int kLaneGroup = 64 / kBatch;   // lanes that end with the same sum
__device__ __forceinline__ void reduce_scatter(double (&v)[kBatch], int lane) {
#pragma unroll
  for (int m = 32, h = kBatch / 2; h >= 1; m >>= 1, h >>= 1) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const double keep = up ? v[h + i] : v[i];
      const double send = up ? v[i] : v[h + i];
      v[i] = keep + __shfl_xor(send, m, 64);
    }
  }
#pragma unroll
  for (int m = 1; m < kLaneGroup; m <<= 1) v[0] += __shfl_xor(v[0], m, 64);
}

// The logits are streamed: non-temporal 16-byte loads do not allocate in the
// caches, so they neither evict what other work keeps there nor force the
// write-back of dirty lines (measured: the all-greedy 480-row call after a
// 1 GiB write drops from 68 to 37 us, and is 2 us faster otherwise).  A
// sampled row is read twice; its second read then misses the caches, which
// costs ~8% on a batch of 16384 sampled rows, less than a cached first read
// costs the greedy rows (a per-row choice of load kind was merged away by
// the compiler).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Geometry of one target row: `head` single elements up to the first 16-byte
// boundary, nvec whole vectors, then single elements to `valid`; segment seg
// takes its share of the vectors, wave w of it a contiguous quarter, read in
// chunks of kChunkVecs vectors.
struct RowGeom {
  int64_t head, nvec;
  __device__ void wave_range(int seg, int w, int64_t& lo, int64_t& hi) const {
    const int64_t slo = nvec * seg / kVerifySegs, shi = nvec * (seg + 1) / kVerifySegs;
    lo = slo + (shi - slo) * w / kVerifyWaves;
    hi = slo + (shi - slo) * (w + 1) / kVerifyWaves;
  }
};

template <typename TIO>
__device__ __forceinline__ RowGeom row_geom(const TIO* z, int64_t valid) {
  constexpr int VEC = Elem<TIO>::kVec;
  RowGeom g;
  g.head = (int64_t)(((16u - (reinterpret_cast<uintptr_t>(z) & 15u)) & 15u) / sizeof(TIO));
  if (g.head > valid) g.head = valid;
  g.nvec = (valid - g.head) / VEC;
  return g;
}

// Statistics of one segment of one target row: its maximum, the maximum's
// lowest id, and (sampled requests) the fp64 sums of exp((z - m) / T) per
// chunk, stored in id order, and over the segment.
template <typename TIO>
__global__ __launch_bounds__(kVerifyThreads) void verify_stats_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t rows_per_req, int64_t valid,
    const float* __restrict__ temperatures, const uint8_t* __restrict__ greedy_mask, VerifyRowStats* __restrict__ stats,
    double* __restrict__ chunk_sums, int32_t nch_bound) {
  __shared__ double s_exp[kExpTable];
  __shared__ float s_wm[kVerifyWaves];
  __shared__ uint32_t s_arg;
  __shared__ double s_wsum[kVerifyWaves];
  __shared__ double s_single;
  constexpr int VEC = Elem<TIO>::kVec;
  const int64_t row = blockIdx.x / kVerifySegs;
  const int seg = (int)(blockIdx.x % kVerifySegs);
  const int r = (int)(row / rows_per_req);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const TIO* z = logits + row * row_stride;
  const RowGeom g = row_geom(z, valid);
  int64_t wlo, whi;
  g.wave_range(seg, wave, wlo, whi);
  // singles: the head belongs to the first segment, the tail to the last;
  // wave 0 reads them
  const int64_t shi = (seg == 0 && wave == 0) ? g.head : 0;
  const int64_t tlo = (seg == kVerifySegs - 1 && wave == 0) ? g.head + g.nvec * VEC : valid;
  const TIO* zv = z + g.head;                           // 16-byte aligned vectors

  exp_table_fill(s_exp);                               // visible after the barrier below
  // pass 1: the maximum, and where each lane first met its own maximum (an
  // id for a single element, a vector index for a vector)
  float m = -INFINITY;
  int64_t at = -1;
  bool at_vec = false;
  for (int64_t v = lane; v < shi; v += 64) {
    const float f = Elem<TIO>::to_f32(z[v]);
    if (f > m) {
      m = f;
      at = v;
    }
  }
#pragma unroll 1
  for (int64_t i0 = wlo + lane; i0 < whi; i0 += 64 * kUnrollMax) {
    u32x4 raw[kUnrollMax];
#pragma unroll
    for (int u = 0; u < kUnrollMax; ++u) {
      const int64_t i = i0 + (int64_t)u * 64;
      raw[u] = ld16_stream(zv + (i < whi ? i : wlo) * VEC);
    }
#pragma unroll
    for (int u = 0; u < kUnrollMax; ++u) {             // branch-free: a vector past the end counts as -inf
      const int64_t i = i0 + (int64_t)u * 64;
      float f[VEC];
      unpack16(raw[u], f);
      float vm = f[0];
#pragma unroll
      for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, f[e]);
      vm = i < whi ? vm : -INFINITY;
      const bool up = vm > m;                          // NaN never raises it
      m = up ? vm : m;
      at = up ? i : at;
      at_vec = up ? true : at_vec;
    }
  }
  for (int64_t v = tlo + lane; v < valid; v += 64) {
    const float f = Elem<TIO>::to_f32(z[v]);
    if (f > m) {
      m = f;
      at = v;
      at_vec = false;
    }
  }
  const float wm = wave_max_f32(m);
  if (lane == 0) s_wm[wave] = wm;
  if (tid == 0) s_arg = 0xffffffffu;
  __syncthreads();
  float mseg = s_wm[0];
#pragma unroll
  for (int w = 1; w < kVerifyWaves; ++w) mseg = fmaxf(mseg, s_wm[w]);
  // its lowest id: each lane holding it found its own first occurrence
  if (mseg > -INFINITY && m == mseg) {
    uint32_t found = (uint32_t)at;
    if (at_vec) {
      float f[VEC];
      unpack16(ld16(zv + at * VEC), f);
      found = 0xffffffffu;
#pragma unroll
      for (int e = VEC - 1; e >= 0; --e)
        if (f[e] == mseg) found = (uint32_t)(g.head + at * VEC + e);
    }
    atomicMin(&s_arg, found);
  }

  // pass 2 (sampled requests): chunk sums of exp((z - mseg) / T) in fp64
  double lacc = 0.0;                                   // lane l: its chunks (l / kLaneGroup of each batch)
  double single = 0.0;                                 // head and tail singles (wave 0)
  const bool sampled = greedy_mask[r] == 0 && mseg > -INFINITY;
  if (sampled) {
    const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
    const double ms = (double)mseg * inv_t;
    double* cs = chunk_sums + (((int64_t)row * kVerifySegs + seg) * kVerifyWaves + wave) * nch_bound;
    const int64_t nch = (whi - wlo + kChunkVecs - 1) / kChunkVecs;
    for (int64_t b0 = 0; b0 < nch; b0 += kBatch) {
      double part[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; jj += kUnroll) {
        u32x4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int64_t i = wlo + (b0 + jj + u) * kChunkVecs + lane;
          raw[u] = ld16_stream(zv + (i < whi ? i : wlo) * VEC);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int64_t i = wlo + (b0 + jj + u) * kChunkVecs + lane;
          double s = 0.0;
          if (b0 + jj + u < nch) {                     // chunk-uniform; the last chunk's tail is masked
            float f[VEC];
            unpack16(raw[u], f);
            s = exp_tab_sum(f, ms, inv_t, s_exp);
            s = i < whi ? s : 0.0;
          }
          part[jj + u] = s;
        }
      }
      // the batch's chunk sums over the wave's lanes (a fixed butterfly:
      // lane l ends with chunk l / kLaneGroup)
      reduce_scatter(part, lane);
      const int nb = (int)(nch - b0 < kBatch ? nch - b0 : kBatch);
      const int c = lane / kLaneGroup;
      if (lane % kLaneGroup == 0 && c < nb) cs[b0 + c] = part[0];
      if (c < nb) lacc += part[0];
    }
    if (wave == 0) {
      double h = 0.0;
      for (int64_t v = lane; v < shi; v += 64) h += exp_tab(fma(logit_at(z, v), inv_t, -ms), s_exp);
      double t = 0.0;
      for (int64_t v = tlo + lane; v < valid; v += 64) t += exp_tab(fma(logit_at(z, v), inv_t, -ms), s_exp);
      for (int o = 32; o > 0; o >>= 1) {               // the same tree for every launch
        h += __shfl_xor(h, o, 64);
        t += __shfl_xor(t, o, 64);
      }
      single = h + t;
    }
  }
  // the wave's total: the kBatch chunk positions of the lanes l = kLaneGroup c
#pragma unroll
  for (int m = kLaneGroup; m < 64; m <<= 1) lacc += __shfl_xor(lacc, m, 64);
  if (lane == 0) s_wsum[wave] = lacc;
  if (tid == 0) s_single = single;
  __syncthreads();
  if (tid == 0) {
    double s = s_single;
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) s += s_wsum[w];
    const uint32_t a = s_arg;
    stats[blockIdx.x] = VerifyRowStats{(double)mseg, s, a == 0xffffffffu ? (int64_t)-1 : (int64_t)a};
  }
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
      if (st[k].m > -INFINITY) o.s += st[k].s * exp_nonpos((st[k].m - o.m) * inv_t);
  return o;
}

// Inclusive scan of one double per thread over the workgroup, in thread
// order: doubling steps within each wave (shuffles), then the totals of the
// preceding waves added in wave order.  Returns this thread's prefix and the
// workgroup's total; wtot holds kCommitThreads / 64 doubles.  Starts with a
// barrier (so wtot may be reused right after a previous scan) and ends with
// one.
__device__ __forceinline__ double block_scan(double v, double* wtot, double& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  __syncthreads();
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  double before = 0.0, all = 0.0;
  for (int w = 0; w < kCommitThreads / 64; ++w) {
    if (w == wave) before = all;
    all += wtot[w];
  }
  total = all;
  __syncthreads();
  return before + v;
}

template <typename TIO>
__global__ __launch_bounds__(kCommitThreads) void verify_commit_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t S, int32_t K, int64_t valid,
    const int64_t* __restrict__ cand_ids, const float* __restrict__ q, const int64_t* __restrict__ tokens,
    const float* __restrict__ u_accept, const float* __restrict__ u_residual, const float* __restrict__ temperatures,
    const uint8_t* __restrict__ greedy_mask, const VerifyRowStats* __restrict__ stats,
    const double* __restrict__ chunk_sums, int32_t nch_bound, int32_t* __restrict__ accepted,
    int64_t* __restrict__ committed) {
  __shared__ double s_exp[kExpTable];
  __shared__ int s_n;
  __shared__ int s_nc;
  __shared__ int64_t s_cid[kMaxTopK], s_rid[kMaxTopK];
  __shared__ double s_cq[kMaxTopK], s_cz[kMaxTopK];
  __shared__ VerifyRowStats s_rows[kRowsLds];
  __shared__ double s_rscale[kRowsLds][kVerifySegs];
  __shared__ double s_wtot[kCommitThreads / 64];
  __shared__ VerifyRowStats s_st;
  __shared__ double s_scale[kVerifySegs];
  __shared__ int s_block, s_lastblock;
  __shared__ double s_base;
  __shared__ int64_t s_ra, s_rb;
  __shared__ unsigned long long s_tok, s_lastid;
  constexpr int VEC = Elem<TIO>::kVec;
  const int r = blockIdx.x, tid = threadIdx.x;
  const bool greedy = greedy_mask[r] != 0;
  const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
  exp_table_fill(s_exp);
  // Loads that do not wait for the decisions are all issued here: each of
  // the first S K threads holds one candidate (id, q and its logit) of its
  // slot, and thread t <= S merges row t's segment records (kept in LDS for
  // the first kRowsLds rows, with the chunk scales of the sampled draw).
  const int pslot = tid / K, pj = tid - pslot * K;
  const bool pre = !greedy && (int64_t)S * K > tid;
  int64_t pid = -1;
  double pq = 0.0, pz = 0.0;
  if (pre) {
    pid = cand_ids[((int64_t)r * S + pslot) * K + pj];
    pq = (double)q[((int64_t)r * S + pslot) * K + pj];
    if (pid < 0 || pid >= valid) pid = -1;
    else pz = logit_at(logits + ((int64_t)r * (S + 1) + pslot) * row_stride, pid);
  }
  // the accept decisions of all slots at once; n = the first rejection
  if (tid == 0) s_n = S;
  __syncthreads();
  for (int n = tid; n <= S; n += kCommitThreads) {
    const VerifyRowStats* rs = stats + ((int64_t)r * (S + 1) + n) * kVerifySegs;
    const VerifyRowStats st = merge_segments(rs, inv_t);
    if (n < kRowsLds) {
      s_rows[n] = st;
      // a chunk sum against its segment's maximum -> probability mass
      for (int k = 0; k < kVerifySegs; ++k)
        s_rscale[n][k] = (!greedy && st.m > -INFINITY && rs[k].m > -INFINITY)
                             ? exp_nonpos((rs[k].m - st.m) * inv_t) / st.s : 0.0;
    }
    if (n == S) continue;
    const int64_t x = tokens[(int64_t)r * S + n];
    bool keep;
    if (greedy) {
      keep = x == st.arg;
    } else {
      double qx = 0.0;                                       // a token outside the candidates has q = 0
      for (int j = K - 1; j >= 0; --j)                       // the first candidate holding x
        if (cand_ids[((int64_t)r * S + n) * K + j] == x) qx = (double)q[((int64_t)r * S + n) * K + j];
      const TIO* z = logits + ((int64_t)r * (S + 1) + n) * row_stride;
      const double px = (x >= 0 && x < valid && st.m > -INFINITY)
                            ? exp_tab(fma(logit_at(z, x), inv_t, -st.m * inv_t), s_exp) / st.s : 0.0;
      keep = (double)u_accept[(int64_t)r * S + n] * qx < px;
    }
    if (!keep) atomicMin(&s_n, n);
  }
  __syncthreads();
  // the rejected slot's candidates in id order (equal ids keep their order),
  // for the residual max(0, p - q), with their logits
  {
    const int n = s_n;
    const bool held = n < S && (int64_t)(n + 1) * K <= kCommitThreads;   // preloaded above
    const int t0 = held ? n * K : 0;
    const bool ranker = n < S && !greedy && tid >= t0 && tid < t0 + K;
    const int j = tid - t0;
    int64_t id = pid;
    double qj = pq, zj = pz;
    if (ranker && !held) {
      id = cand_ids[((int64_t)r * S + n) * K + j];
      qj = (double)q[((int64_t)r * S + n) * K + j];
      if (id < 0 || id >= valid) id = -1;
      else zj = logit_at(logits + ((int64_t)r * (S + 1) + n) * row_stride, id);
    }
    if (ranker) s_rid[j] = id;
    if (n < kRowsLds) {
      if (tid == kCommitThreads - 1) s_st = s_rows[n];
      if (tid < kVerifySegs) s_scale[tid] = s_rscale[n][tid];
    } else if (tid == kCommitThreads - 1) {         // the committed row's statistics
      const VerifyRowStats* rs = stats + ((int64_t)r * (S + 1) + n) * kVerifySegs;
      const VerifyRowStats st = merge_segments(rs, inv_t);
      s_st = st;
      for (int k = 0; k < kVerifySegs; ++k)
        s_scale[k] = (!greedy && st.m > -INFINITY && rs[k].m > -INFINITY)
                         ? exp_nonpos((rs[k].m - st.m) * inv_t) / st.s : 0.0;
    }
    __syncthreads();
    if (ranker) {
      int rank = 0, nc = 0;
      for (int i = 0; i < K; ++i) {
        const int64_t o = s_rid[i];
        if (o < 0) continue;
        ++nc;
        if (id >= 0 && (o < id || (o == id && i < j))) ++rank;
      }
      if (id >= 0) {
        s_cid[rank] = id;
        s_cq[rank] = qj;
        s_cz[rank] = zj;
      }
      if (j == 0) s_nc = nc;
    } else if (tid == kCommitThreads - 1 && !(n < S && !greedy)) {
      s_nc = 0;
    }
  }
  __syncthreads();
  const int n = s_n;
  const int64_t row = (int64_t)r * (S + 1) + n;
  const VerifyRowStats st = s_st;
  int64_t tok;
  if (greedy || !(st.m > -INFINITY)) {
    tok = st.arg;
  } else {
    // weights w(v) = p(v) (bonus) or max(0, p(v) - q(v)) (after a rejection);
    // when no residual weight is positive (q covers p) the draw is from p
    const TIO* z = logits + row * row_stride;
    const RowGeom g = row_geom(z, valid);
    const double u = (double)u_residual[r];
    const double ms = st.m * inv_t;
    auto p_of = [&](int64_t v) { return exp_tab(fma(logit_at(z, v), inv_t, -ms), s_exp) / st.s; };
    // Regions in id order: 0 = head singles, then the chunks of segment
    // seg, wave w, chunk j at 1 + (seg * waves + w) * nch_bound + j (empty
    // past a wave's last chunk), last = tail singles.  Each thread sums a
    // contiguous block of regions; the blocks are scanned.
    const int64_t n_regions = 2 + (int64_t)kVerifySegs * kVerifyWaves * nch_bound;
    const int64_t per = (n_regions + kCommitThreads - 1) / kCommitThreads;
    const int64_t r0 = (int64_t)tid * per, r1 = r0 + per < n_regions ? r0 + per : n_regions;
    tok = -1;
    for (int attempt = 0; attempt < 2 && tok < 0; ++attempt) {
      const int nc = attempt == 0 ? s_nc : 0;
      auto weight_from = [&](int64_t v, double w) {       // w = p(v)
        for (int c = 0; c < nc; ++c)
          if (s_cid[c] == v) w = w - s_cq[c] > 0.0 ? w - s_cq[c] : 0.0;
        return w;
      };
      auto weight = [&](int64_t v) { return weight_from(v, p_of(v)); };
      auto region = [&](int64_t rg, int64_t& a, int64_t& b) -> double {
        if (rg == 0 || rg == n_regions - 1) {
          a = rg == 0 ? 0 : g.head + g.nvec * VEC;
          b = rg == 0 ? g.head : valid;
          double s = 0.0;
          for (int64_t v = a; v < b; ++v) s += weight(v);
          return s;
        }
        const int64_t k = rg - 1;
        const int seg = (int)(k / ((int64_t)kVerifyWaves * nch_bound));
        const int w = (int)((k / nch_bound) % kVerifyWaves);
        const int64_t j = k % nch_bound;
        int64_t wlo, whi;
        g.wave_range(seg, w, wlo, whi);
        const int64_t i0 = wlo + j * kChunkVecs;
        a = b = 0;
        if (i0 >= whi || !(s_scale[seg] > 0.0)) return 0.0;
        const int64_t i1 = i0 + kChunkVecs < whi ? i0 + kChunkVecs : whi;
        a = g.head + i0 * VEC;
        b = g.head + i1 * VEC;
        double s = chunk_sums[((row * kVerifySegs + seg) * kVerifyWaves + w) * nch_bound + j] * s_scale[seg];
        for (int c = 0; c < nc; ++c)                        // the residual at the candidate ids
          if (s_cid[c] >= a && s_cid[c] < b && (c == 0 || s_cid[c - 1] != s_cid[c])) {
            const double pc = exp_tab(fma(s_cz[c], inv_t, -ms), s_exp) / st.s;   // p of that id
            s -= pc - weight_from(s_cid[c], pc);
          }
        return s > 0.0 ? s : 0.0;
      };
      double bsum = 0.0;
      int64_t a0 = 0, b0 = 0;                              // this thread's first region
      for (int64_t rg = r0; rg < r1; ++rg) {
        int64_t a, b;
        bsum += region(rg, a, b);
        if (rg == r0) {
          a0 = a;
          b0 = b;
        }
      }
      if (tid == 0) {
        s_block = kCommitThreads;
        s_lastblock = -1;
      }
      double total;
      const double incl = block_scan(bsum, s_wtot, total);  // starts and ends with a barrier
      const double target = u * total;
      // the first block whose cumulative weight passes the target; rounding
      // can leave the target at the very end: then the last block with weight
      if (bsum > 0.0) {
        atomicMax(&s_lastblock, tid);
        if (incl > target) atomicMin(&s_block, tid);
      }
      __syncthreads();
      const int blk = s_block < kCommitThreads ? s_block : s_lastblock;
      if (blk < 0) {                                         // no weight at all
        __syncthreads();
        continue;
      }
      // the block's owner finds the region the same way
      if (tid == blk) {
        double acc = incl - bsum;
        int64_t ra = a0, rb = b0;                          // a block of one region: that one
        double rbase = acc;
        for (int64_t rg = r0; per > 1 && rg < r1; ++rg) {
          int64_t a, b;
          const double w = region(rg, a, b);
          if (w > 0.0) {
            ra = a;
            rb = b;
            rbase = acc;
            if (acc + w > target) break;
          }
          acc += w;
        }
        s_ra = ra;
        s_rb = rb;
        s_base = rbase;
        s_tok = ~0ull;
        s_lastid = 0;
      }
      __syncthreads();
      const int64_t ra = s_ra, rb = s_rb;
      const double base = s_base;
      // the region's ids (at most kChunkVecs * VEC): weights in parallel,
      // scanned in id order; the first whose cumulative weight passes the
      // target, else the last with weight
      const double wv = (ra + tid < rb) ? weight(ra + tid) : 0.0;
      double vtotal;
      const double vincl = block_scan(wv, s_wtot, vtotal) + base;
      if (wv > 0.0) {
        atomicMax(&s_lastid, (unsigned long long)(ra + tid + 1));
        if (vincl > target) atomicMin(&s_tok, (unsigned long long)(ra + tid));
      }
      __syncthreads();
      tok = s_tok != ~0ull ? (int64_t)s_tok : s_lastid > 0 ? (int64_t)(s_lastid - 1) : st.arg;
      __syncthreads();
    }
    if (tok < 0) tok = st.arg;
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

int32_t verify_chunks_bound(int64_t valid_vocab) {
  // vectors of 4 elements at the least (fp32); a segment's and a wave's share
  // rounded up, in chunks of kChunkVecs vectors
  const int64_t nvec = (valid_vocab + 3) / 4;
  const int64_t per_seg = (nvec + kVerifySegs - 1) / kVerifySegs + 1;
  const int64_t per_wave = (per_seg + kVerifyWaves - 1) / kVerifyWaves + 1;
  return (int32_t)((per_wave + kChunkVecs - 1) / kChunkVecs);
}

size_t verify_workspace_bytes(int32_t n_req, int32_t slots, int64_t valid_vocab) {
  const size_t rows = (size_t)n_req * (slots + 1);
  const size_t stats = rows * kVerifySegs * sizeof(VerifyRowStats);
  const size_t chunks = rows * kVerifySegs * kVerifyWaves * (size_t)verify_chunks_bound(valid_vocab) * sizeof(double);
  return stats + chunks;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  if (a.n_req == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.n_req * (a.slots + 1);
  VerifyRowStats* stats = static_cast<VerifyRowStats*>(a.workspace);   // [rows][kVerifySegs]
  double* chunk_sums = reinterpret_cast<double*>(stats + rows * kVerifySegs);
  const int32_t nch_bound = verify_chunks_bound(a.valid_vocab);
#define DFLASH_VERIFY(TIO)                                                                                   \
  hipLaunchKernelGGL(verify_stats_kernel<TIO>, dim3((unsigned)(rows * kVerifySegs)), dim3(kVerifyThreads), 0,    \
                     stream,                                                                                  \
                     static_cast<const TIO*>(a.logits), a.row_stride, a.slots + 1, a.valid_vocab,             \
                     a.temperatures, a.greedy_mask, stats, chunk_sums, nch_bound);                            \
  {                                                                                                          \
    hipError_t e = hipGetLastError();                                                                        \
    if (e != hipSuccess) return e;                                                                           \
  }                                                                                                          \
  hipLaunchKernelGGL(verify_commit_kernel<TIO>, dim3((unsigned)a.n_req), dim3(kCommitThreads), 0, stream,      \
                     static_cast<const TIO*>(a.logits), a.row_stride, a.slots, a.top_k, a.valid_vocab,        \
                     a.cand_ids, a.q, a.tokens, a.u_accept, a.u_residual, a.temperatures, a.greedy_mask,      \
                     stats, chunk_sums, nch_bound, a.accepted_out, a.committed_out)
  if (a.dtype == DFLASH_BF16) {
    DFLASH_VERIFY(uint16_t);
  } else {
    DFLASH_VERIFY(float);
  }
#undef DFLASH_VERIFY
  return hipGetLastError();
}

}  // namespace dflash

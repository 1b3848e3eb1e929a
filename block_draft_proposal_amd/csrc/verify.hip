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
// owns a contiguous quarter of its segment and reads it once, a chunk of
// kChunkVecs 16-byte vectors at a time (kChunkLoads coalesced vectors per
// lane, the next chunk in flight): the maximum and where each lane first met
// it, and (sampled requests) the sum of exp((z - M) / T) of each chunk
// against the wave's running maximum M (raised only when some lane's chunk
// exceeds it), stored with that M.  These sums use the hardware 2^x in fp32
// and carry a rigorous bound on their error.  Then one workgroup per
// request: the accept decisions (p(x) from one logit in fp64) and the
// committed draw (the chunks scanned in id order to find the one holding the
// crossing, whose ids are then weighed one by one) are taken with the
// approximate sums only where the bound cannot change them.  An undecided
// decision recomputes its row's sums in fp64 in the same workgroup; an
// undecided draw lists its request, and two more kernels compute that row's
// fp64 sums and take the draw again.
#include "dflash.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int kVerifyThreads = 256;   // 4 waves per (row, segment)
constexpr int kVerifyWaves = kVerifyThreads / 64;
constexpr int kCommitThreads = 256;   // 4 waves per request: four requests per CU at once
constexpr int kRowsLds = 64;          // target rows of a request whose statistics the commit keeps in LDS
constexpr int kChunkLoads = 4;        // vectors per lane of one chunk
constexpr int kChunkVecs = 64 * kChunkLoads;   // vectors of one chunk, contiguous in the row
constexpr int kUnrollMax = 8;         // vectors per lane in flight (maximum only)

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

// The sum of one double per lane over the wave, in every lane (a fixed
// butterfly, so the order of the additions is the same on every launch).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
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

// exp((f - M) / T) = 2^x, x = (f - M) c with c = log2(e) / T rounded to
// fp32, summed over a 16-byte vector in fp32 with the hardware 2^x, and a
// bound on the sum's error in units of 2^-24.  Error of one term against the
// exact value: 2^x is within 1.43 ulp (2^-24 relative units) of the exact
// power of two for every fp32 x in [-126, 0] (checked exhaustively on the
// device against fp64 exp2); x carries at most 3 roundings (f - M, c, the
// product), so 2^x is off by at most 2.08 |x| 2^-24 relative more; the
// pairwise sum of the vector's terms adds at most 3 2^-24 of the sum.  So
// |sum - exact| <= 2^-24 sum_t t (4.43 + 2.08 |x|) <= 2^-24 (4.5 s - 2.1 e)
// with e = sum_t t x <= 0, which is added to `e` (the slack in the constants
// covers the rounding of s and of e's own fp32 sums over up to 64 terms).
// Below 2^-126 a term is at most 2^-125 off.  A NaN logit makes the sum NaN
// and a -inf logit the bound (0 times -inf): no decision or draw trusts a NaN
// sum or bound, so such a row is decided from its exact sums (where NaN and
// -inf give zero terms).
template <int VEC>
__device__ __forceinline__ void exp2_sum(const float (&f)[VEC], float M, float c, float& s, float& e) {
  static_assert(VEC == 4 || VEC == 8, "pairwise sum of 4 or 8 terms");
  float t[VEC], ee = e;
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    const float x = (f[k] - M) * c;
    t[k] = __builtin_amdgcn_exp2f(x);
    ee = fmaf(t[k], x, ee);
  }
  float a = (t[0] + t[1]) + (t[2] + t[3]);
  if constexpr (VEC == 8) a = a + ((t[4] + t[5]) + (t[6] + t[7]));
  s = a;
  e = ee;
}

// Statistics of one segment of one target row in one read: its maximum, the
// maximum's lowest id, and (sampled requests) the sums of exp((z - M) / T)
// per chunk, stored in id order with the M each was taken against, and over
// the segment against the segment's maximum, with the bound on their error.
template <typename TIO>
__global__ __launch_bounds__(kVerifyThreads) __attribute__((amdgpu_waves_per_eu(4))) void verify_stats_kernel(
    const TIO* __restrict__ logits, int64_t row_stride, int32_t rows_per_req, int64_t valid,
    const float* __restrict__ temperatures, const uint8_t* __restrict__ greedy_mask, VerifyRowStats* __restrict__ stats,
    double* __restrict__ chunk_sums, float* __restrict__ chunk_ref, int32_t nch_bound,
    uint32_t* __restrict__ pending_count) {
  __shared__ float s_wm[kVerifyWaves], s_wM[kVerifyWaves];
  __shared__ uint32_t s_arg;
  __shared__ double s_wsum[kVerifyWaves], s_wbnd[kVerifyWaves];
  constexpr int VEC = Elem<TIO>::kVec;
  const int64_t row = blockIdx.x / kVerifySegs;
  const int seg = (int)(blockIdx.x % kVerifySegs);
  const int r = (int)(row / rows_per_req);
  // the wave index as a scalar: the buffer resource of the wave's range stays uniform
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const TIO* z = logits + row * row_stride;
  const RowGeom g = row_geom(z, valid);
  int64_t wlo, whi;
  g.wave_range(seg, wave, wlo, whi);
  // singles: the head belongs to the first segment, the tail to the last;
  // wave 0 reads them
  const int64_t shi = (seg == 0 && wave == 0) ? g.head : 0;
  const int64_t tlo = (seg == kVerifySegs - 1 && wave == 0) ? g.head + g.nvec * VEC : valid;
  const TIO* zv = z + g.head;                           // 16-byte aligned vectors
  const bool sampled = greedy_mask[r] == 0;
  const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
  const float c = (float)(inv_t * 0x1.71547652b82fep+0);
  if (blockIdx.x == 0 && tid == 0) *pending_count = 0u;   // the commit pass lists undecided draws

  // the lane's maximum and where it first met it (an id for a single
  // element, a vector index for a vector)
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
  float M = -INFINITY;                                 // the wave's running maximum over its vectors
  // lane: the sums of the wave's chunks so far (the same in every lane) and
  // its own bound terms sum t x, both against M
  double lacc = 0.0, pe = 0.0;
  const int64_t base = ((int64_t)row * kVerifySegs + seg) * kVerifyWaves + wave;
  double* cs = chunk_sums + base * nch_bound;
  float* cr = chunk_ref + base * nch_bound;
  // offsets within the wave's range fit 32 bits (a row has under 2^24 ids)
  const int32_t nw = (int32_t)(whi - wlo);
  const int32_t nch = (nw + kChunkVecs - 1) / kChunkVecs;
  const TIO* zw = zv + wlo * VEC;
  int32_t atw = -1;                                    // the lane's maximum in a vector: its offset in the range
  if (!sampled) {
    // greedy requests need only the maximum: kUnrollMax vectors per lane in
    // flight, branch-free
#pragma unroll 1
    for (int32_t i0 = lane; i0 < nw; i0 += 64 * kUnrollMax) {
      u32x4 rv[kUnrollMax];
#pragma unroll
      for (int u = 0; u < kUnrollMax; ++u) {
        const int32_t io = i0 + u * 64;
        rv[u] = ld16_stream(zw + (io < nw ? io : 0) * VEC);
      }
#pragma unroll
      for (int u = 0; u < kUnrollMax; ++u) {
        const int32_t io = i0 + u * 64;
        float f[VEC];
        unpack16(rv[u], f);
        float vm = f[0];
#pragma unroll
        for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, f[e]);
        vm = io < nw ? vm : -INFINITY;
        const bool up = vm > m;                        // NaN never raises it
        m = up ? vm : m;
        atw = up ? io : atw;
        at_vec = up ? true : at_vec;
      }
    }
  }
  // sampled rows: every load through a buffer resource over the wave's range,
  // so a vector past its end reads as zeros without memory traffic and the
  // next chunk's loads need no condition
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<TIO*>(zw), 0, nw * 16, kBufferFlags);
  auto load_chunk = [&](int32_t j, u32x4 (&dst)[kChunkLoads]) {
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u)
      dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (j * kChunkVecs + u * 64 + lane) * 16, 0, kBufferStream);
  };
  // lane l holds the sum and reference of chunk jb + l of the current block
  // of 64 chunks until the block is stored
  double my_cs = 0.0;
  float my_cr = 0.f;
  // chunk j from cur, with chunk j + 1 loaded into nxt first
  auto chunk_step = [&](int32_t j, const u32x4 (&cur)[kChunkLoads], u32x4 (&nxt)[kChunkLoads]) {
    load_chunk(j + 1, nxt);
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u) {            // branch-free: a vector past the end counts as -inf
      const int32_t io = j * kChunkVecs + u * 64 + lane;
      float f[VEC];
      unpack16(cur[u], f);
      float vm = f[0];
#pragma unroll
      for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, f[e]);
      vm = io < nw ? vm : -INFINITY;
      const bool up = vm > m;                          // NaN never raises it
      m = up ? vm : m;
      atw = up ? io : atw;
      at_vec = up ? true : at_vec;
      bm = fmaxf(bm, vm);
    }
    // the wave's maximum only when some lane's chunk passes M (uniform)
    if (__builtin_amdgcn_ballot_w64(bm > M) != 0ull) {
      bm = wave_max_f32(bm);
      if (M > -INFINITY) {
        const double sc = exp_nonpos(((double)M - (double)bm) * inv_t);
        lacc *= sc;
        pe *= sc;
      }
      M = bm;
    }
    double ps = 0.0;
    float ee = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int u = 0; u < kChunkLoads; ++u) {
        float ss = 0.f;
        if (j * kChunkVecs + u * 64 + lane < nw) {     // skipped by a wave wholly past the end
          float f[VEC];
          unpack16(cur[u], f);
          exp2_sum(f, M, c, ss, ee);
        }
        ps += (double)ss;
      }
    }
    pe += (double)ee;
    ps = wave_sum_f64(ps);                             // the chunk's sum, in every lane
    const bool mine = lane == (j & 63);
    my_cs = mine ? ps : my_cs;
    my_cr = mine ? M : my_cr;
    lacc += ps;
  };
  if (sampled && nch > 0) {
    u32x4 ra[kChunkLoads], rb[kChunkLoads];            // two buffers in turn: no copies between chunks
    load_chunk(0, ra);
    for (int32_t jb = 0; jb < nch; jb += 64) {         // blocks of 64 chunks (even: ra stays first)
      const int32_t je = jb + 64 < nch ? jb + 64 : nch;
      int32_t j = jb;
#pragma unroll 1
      for (; j + 1 < je; j += 2) {
        chunk_step(j, ra, rb);
        chunk_step(j + 1, rb, ra);
      }
      if (j < je) chunk_step(j, ra, rb);
      if (jb + lane < je) {
        cs[jb + lane] = my_cs;
        cr[jb + lane] = my_cr;
      }
    }
  }
  if (at_vec) at = wlo + atw;                          // a vector index (the head singles set ids)
  for (int64_t v = tlo + lane; v < valid; v += 64) {
    const float f = Elem<TIO>::to_f32(z[v]);
    if (f > m) {
      m = f;
      at = v;
      at_vec = false;
    }
  }
  // the wave's bound terms (lacc already holds the wave's sums)
  pe = wave_sum_f64(pe);
  const float wm = wave_max_f32(m);
  if (lane == 0) {
    s_wm[wave] = wm;
    s_wM[wave] = M;
    s_wsum[wave] = lacc;
    s_wbnd[wave] = pe;
  }
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
  // the head and tail singles against the segment maximum, in fp64 (wave 0)
  double single = 0.0;
  if (sampled && mseg > -INFINITY && wave == 0) {
    const double ms = (double)mseg * inv_t;
    double h = 0.0, t = 0.0;
    for (int64_t v = lane; v < shi; v += 64) h += exp_nonpos(fma(logit_at(z, v), inv_t, -ms));
    for (int64_t v = tlo + lane; v < valid; v += 64) t += exp_nonpos(fma(logit_at(z, v), inv_t, -ms));
    for (int o = 32; o > 0; o >>= 1) {               // the same tree for every launch
      h += __shfl_xor(h, o, 64);
      t += __shfl_xor(t, o, 64);
    }
    single = h + t;
  }
  __syncthreads();
  if (tid == 0) {
    double s = 0.0, b = 0.0;
    if (sampled && mseg > -INFINITY) {
      for (int w = 0; w < kVerifyWaves; ++w) {
        if (!(s_wM[w] > -INFINITY)) continue;
        const double sc = exp_nonpos(((double)s_wM[w] - (double)mseg) * inv_t);
        s += s_wsum[w] * sc;
        b += 0x1p-24 * (4.5 * s_wsum[w] - 2.1 * s_wbnd[w]) * sc;
      }
      s += single;
      b += 0x1p-100 + 0x1p-50 * s;                     // terms below 2^-126; the fp64 sums and scalings
    }
    const uint32_t a = s_arg;
    stats[blockIdx.x] = VerifyRowStats{(double)mseg, s, b, a == 0xffffffffu ? (int64_t)-1 : (int64_t)a};
  }
}

// The row's statistics from its segments, in segment (id) order: the maximum,
// its lowest id (the first segment that holds it), the normaliser
// sum_k s_k exp((m_k - m) / T) and its error bound.
__device__ __forceinline__ VerifyRowStats merge_segments(const VerifyRowStats* st, double inv_t) {
  VerifyRowStats o{-INFINITY, 0.0, 0.0, 0};
  for (int k = 0; k < kVerifySegs; ++k)
    if (st[k].m > o.m) {
      o.m = st[k].m;
      o.arg = st[k].arg;
    }
  if (o.m > -INFINITY) {
    for (int k = 0; k < kVerifySegs; ++k)
      if (st[k].m > -INFINITY) {
        const double sc = exp_nonpos((st[k].m - o.m) * inv_t);
        o.s += st[k].s * sc;
        o.b += st[k].b * sc;
      }
    o.b += 0x1p-50 * o.s;
  }
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

// The exact (fp64) sum of exp((z - m) / T) over chunk j of a (segment, wave)
// range [wlo, whi) of vectors, by one wave, in every lane.
template <typename TIO>
__device__ __forceinline__ double exact_chunk_sum(const TIO* zv, int64_t wlo, int64_t whi, int64_t j, double ms,
                                                  double inv_t, const double* s_exp) {
  constexpr int VEC = Elem<TIO>::kVec;
  const int lane = threadIdx.x & 63;
  u32x4 raw[kChunkLoads];
#pragma unroll
  for (int u = 0; u < kChunkLoads; ++u) {
    const int64_t i = wlo + j * kChunkVecs + u * 64 + lane;
    raw[u] = ld16_stream(zv + (i < whi ? i : wlo) * VEC);
  }
  double ps = 0.0;
#pragma unroll
  for (int u = 0; u < kChunkLoads; ++u) {
    const int64_t i = wlo + j * kChunkVecs + u * 64 + lane;
    if (i < whi) {
      float f[VEC];
      unpack16(raw[u], f);
      ps += exp_tab_sum(f, ms, inv_t, s_exp);
    }
  }
  return wave_sum_f64(ps);
}

// The exact sum of the head and/or tail singles of a row (ids before the
// first whole vector, after the last) against m, by one wave, in every lane.
template <typename TIO>
__device__ __forceinline__ double exact_singles(const TIO* z, const RowGeom& g, int64_t valid, double ms, double inv_t,
                                                const double* s_exp, bool head, bool tail) {
  constexpr int VEC = Elem<TIO>::kVec;
  const int lane = threadIdx.x & 63;
  double h = 0.0, t = 0.0;
  for (int64_t v = lane; head && v < g.head; v += 64) h += exp_tab(fma(logit_at(z, v), inv_t, -ms), s_exp);
  for (int64_t v = g.head + g.nvec * VEC + lane; tail && v < valid; v += 64)
    t += exp_tab(fma(logit_at(z, v), inv_t, -ms), s_exp);
  return wave_sum_f64(h) + wave_sum_f64(t);
}

// The exact (fp64) sums of one target row against its maximum m, by the
// whole commit workgroup: every chunk's sum is overwritten with its fp64
// value and its reference with m, and the row's total (chunks and singles)
// is returned to every thread.  Wave w of the workgroup takes the row's
// (segment, wave) ranges w, w + waves, ...
template <typename TIO>
__device__ double exact_row_sums(const TIO* z, int64_t valid, double m, double inv_t, const double* s_exp,
                                 double* cs_row, float* cr_row, int32_t nch_bound, double* red) {
  const RowGeom g = row_geom(z, valid);
  const TIO* zv = z + g.head;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const double ms = m * inv_t;
  double lacc = 0.0;
  for (int part = wv; part < kVerifySegs * kVerifyWaves; part += kCommitThreads / 64) {
    int64_t wlo, whi;
    g.wave_range(part / kVerifyWaves, part % kVerifyWaves, wlo, whi);
    const int64_t nch = (whi - wlo + kChunkVecs - 1) / kChunkVecs;
    double* cs = cs_row + (int64_t)part * nch_bound;
    float* cr = cr_row + (int64_t)part * nch_bound;
    for (int64_t j = 0; j < nch; ++j) {
      const double cj = exact_chunk_sum(zv, wlo, whi, j, ms, inv_t, s_exp);
      if (lane == 0) {
        cs[j] = cj;
        cr[j] = (float)m;
      }
      lacc += cj;
    }
  }
  if (wv == 0) lacc += exact_singles(z, g, valid, ms, inv_t, s_exp, true, true);
  __syncthreads();                                        // red is free
  if (lane == 0) red[wv] = lacc;
  __syncthreads();
  double all = 0.0;
  for (int w = 0; w < kCommitThreads / 64; ++w) all += red[w];
  __syncthreads();
  return all;
}

// Accept decision of slot n of a sampled request from approximate
// statistics: +1 keep, 0 reject, -1 undecided (the bound on the normaliser
// straddles u q(x) S = e(x)).  Keep iff u q(x) < p(x) = e(x) / S with
// e(x) = exp((z_x - m) / T) in fp64.
__device__ __forceinline__ int certain_keep(double uq, double ex, const VerifyRowStats& st) {
  if (uq * (st.s + st.b) < ex) return 1;
  if (uq * (st.s - st.b) >= ex) return 0;
  return -1;
}

constexpr int kParts = kVerifySegs * kVerifyWaves;   // (segment, wave) ranges of a row
// Arguments of the commit passes.
template <typename TIO>
struct CommitArgs {
  const TIO* logits;
  int64_t row_stride;
  int32_t S, K;
  int64_t valid;
  const int64_t* cand_ids;
  const float* q;
  const int64_t* tokens;
  const float *u_accept, *u_residual, *temperatures;
  const uint8_t* greedy_mask;
  const VerifyRowStats* stats;
  double* chunk_sums;
  float* chunk_ref;
  int32_t nch_bound;
  int32_t* pending;                  // [n_req]: the row whose draw is left to the exact pass, else -1
  int32_t* list;                     // [n_req]: the requests with a pending draw ...
  uint32_t* count;                   // ... and their number (cleared by the statistics pass)
  double* partials;                  // [n_req][kParts]: the exact range totals
  int32_t* accepted;
  int64_t* committed;
};

// The commit of request r by a workgroup of kCommitThreads threads.  First
// pass (FIXUP false): the decisions, and the draw where the approximate sums
// decide it; a draw they cannot decide leaves its row in pending[r] (else
// -1) and its token unwritten.  Second pass (FIXUP true, from the fix-up
// kernel once the row's exact sums are in): the draw again from them.
template <typename TIO, bool FIXUP>
__device__ void commit_body(const CommitArgs<TIO>& ca, const int r) {
  const TIO* __restrict__ logits = ca.logits;
  const int64_t row_stride = ca.row_stride;
  const int32_t S = ca.S, K = ca.K;
  const int64_t valid = ca.valid;
  const int64_t* __restrict__ cand_ids = ca.cand_ids;
  const float* __restrict__ q = ca.q;
  const int64_t* __restrict__ tokens = ca.tokens;
  const float* __restrict__ u_accept = ca.u_accept;
  const float* __restrict__ u_residual = ca.u_residual;
  const float* __restrict__ temperatures = ca.temperatures;
  const uint8_t* __restrict__ greedy_mask = ca.greedy_mask;
  const VerifyRowStats* __restrict__ stats = ca.stats;
  double* __restrict__ chunk_sums = ca.chunk_sums;
  float* __restrict__ chunk_ref = ca.chunk_ref;
  const int32_t nch_bound = ca.nch_bound;
  int32_t* __restrict__ pending = ca.pending;
  const double* __restrict__ partials = ca.partials;
  int32_t* __restrict__ accepted = ca.accepted;
  int64_t* __restrict__ committed = ca.committed;
  __shared__ double s_exp[kExpTable];
  __shared__ int s_n, s_unc, s_exact_row;
  __shared__ int s_nc;
  __shared__ int64_t s_cid[kMaxTopK], s_rid[kMaxTopK];
  __shared__ double s_cq[kMaxTopK], s_cz[kMaxTopK];
  __shared__ VerifyRowStats s_rows[kRowsLds];
  __shared__ double s_wtot[kCommitThreads / 64];
  __shared__ VerifyRowStats s_st, s_exact_st;
  __shared__ int s_block, s_lastblock, s_sure;
  __shared__ int s_qj[kRowsLds];                           // per slot: the first candidate holding its token
  __shared__ double s_qx[kRowsLds];                        // ... and its q
  __shared__ double s_base;
  __shared__ int64_t s_ra, s_rb;
  __shared__ unsigned long long s_tok, s_lastid;
  constexpr int VEC = Elem<TIO>::kVec;
  const int tid = threadIdx.x;
  const int fix_n = FIXUP ? pending[r] : -1;
  const bool greedy = greedy_mask[r] != 0;
  const double inv_t = 1.0 / clamp_temperature(temperatures[r]);
  const int64_t row_sums = (int64_t)kVerifySegs * kVerifyWaves;   // chunk records per target row: x nch / nbt bound
  exp_table_fill(s_exp);
  // Loads that do not wait for the decisions are all issued here: each of
  // the first S K threads holds one candidate (id, q and its logit) of its
  // slot, and thread t <= S merges row t's segment records (kept in LDS for
  // the first kRowsLds rows).
  const int pslot = tid / K, pj = tid - pslot * K;
  const bool pre = !greedy && (int64_t)S * K > tid;
  int64_t pid = -1;
  double pq = 0.0, pz = 0.0;
  // q(x) of slot n's token x from these (slots whose candidates are all
  // held, n < kRowsLds): the lowest j with id x, found by an LDS minimum
  const int n_qlds = min(min(S, kRowsLds), kCommitThreads / max(K, 1));
  if (tid < n_qlds) s_qj[tid] = K;
  int64_t ptok = -1;
  if (pre) {
    pid = cand_ids[((int64_t)r * S + pslot) * K + pj];
    pq = (double)q[((int64_t)r * S + pslot) * K + pj];
    if (pslot < n_qlds) ptok = tokens[(int64_t)r * S + pslot];
    if (pid < 0 || pid >= valid) pid = -1;
    else pz = logit_at(logits + ((int64_t)r * (S + 1) + pslot) * row_stride, pid);
  }
  __syncthreads();
  if (pre && pslot < n_qlds && pid >= 0 && pid == ptok) atomicMin(&s_qj[pslot], pj);
  __syncthreads();
  if (pre && pslot < n_qlds && pid >= 0 && pid == ptok && s_qj[pslot] == pj) s_qx[pslot] = pq;
  // slot n's u q(x) and e(x) (sampled requests)
  auto slot_terms = [&](int n, const VerifyRowStats& st, double& uq, double& ex) {
    const int64_t x = tokens[(int64_t)r * S + n];
    double qx = 0.0;                                       // a token outside the candidates has q = 0
    if (n < n_qlds) {
      // a valid x: the held lowest match; an invalid x has e(x) = 0 and is
      // rejected whatever q(x) is
      if (s_qj[n] < K) qx = s_qx[n];
    } else {
      for (int j = K - 1; j >= 0; --j)                     // the first candidate holding x
        if (cand_ids[((int64_t)r * S + n) * K + j] == x) qx = (double)q[((int64_t)r * S + n) * K + j];
    }
    const TIO* z = logits + ((int64_t)r * (S + 1) + n) * row_stride;
    ex = (x >= 0 && x < valid && st.m > -INFINITY) ? exp_tab(fma(logit_at(z, x), inv_t, -st.m * inv_t), s_exp) : 0.0;
    uq = (double)u_accept[(int64_t)r * S + n] * qx;
  };
  auto row_stats = [&](int n) {
    return n < kRowsLds ? s_rows[n] : merge_segments(stats + ((int64_t)r * (S + 1) + n) * kVerifySegs, inv_t);
  };
  // the accept decisions of all slots at once: n = the first certain
  // rejection, u = the first undecided slot
  if (tid == 0) {
    s_n = FIXUP ? fix_n : S;
    s_unc = S;
    s_exact_row = -1;
  }
  __syncthreads();
  for (int n = tid; !FIXUP && n <= S; n += kCommitThreads) {
    const VerifyRowStats st = merge_segments(stats + ((int64_t)r * (S + 1) + n) * kVerifySegs, inv_t);
    if (n < kRowsLds) s_rows[n] = st;
    if (n == S) continue;
    int keep;
    if (greedy) {
      keep = tokens[(int64_t)r * S + n] == st.arg ? 1 : 0;
    } else {
      double uq, ex;
      slot_terms(n, st, uq, ex);
      keep = certain_keep(uq, ex, st);
    }
    if (keep == 0) atomicMin(&s_n, n);
    if (keep < 0) atomicMin(&s_unc, n);
  }
  __syncthreads();
  // undecided slots before the first rejection, in slot order: the row's
  // sums in fp64, then the decision as the exact rule takes it
  for (; !FIXUP;) {
    const int nu = s_unc, nr = s_n;                       // LDS words read by all after a barrier: uniform
    if (nu >= nr) break;
    const int64_t row = (int64_t)r * (S + 1) + nu;
    VerifyRowStats st = row_stats(nu);
    st.s = exact_row_sums(logits + row * row_stride, valid, st.m, inv_t, s_exp, chunk_sums + row * row_sums * nch_bound,
                          chunk_ref + row * row_sums * nch_bound, nch_bound, s_wtot);
    st.b = 0.0;
    if (tid == 0) {
      double uq, ex;
      slot_terms(nu, st, uq, ex);
      if (!(uq < ex / st.s)) s_n = nu;
      s_exact_row = nu;
      s_exact_st = st;
      s_unc = S;
    }
    __syncthreads();
    for (int n = nu + 1 + tid; n < s_n; n += kCommitThreads) {   // the next undecided slot
      const VerifyRowStats sn = row_stats(n);
      double uq, ex;
      slot_terms(n, sn, uq, ex);
      if (certain_keep(uq, ex, sn) < 0) atomicMin(&s_unc, n);
    }
    __syncthreads();
  }
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
    if (tid == kCommitThreads - 1) {
      if (FIXUP) {                                       // the exact sums of the pending row
        VerifyRowStats e = merge_segments(stats + ((int64_t)r * (S + 1) + n) * kVerifySegs, inv_t);
        double t = 0.0;
        for (int k = 0; k < kParts; ++k) t += partials[(int64_t)r * kParts + k];
        e.s = t;
        e.b = 0.0;
        s_st = e;
      } else {
        s_st = (s_exact_row == n) ? s_exact_st : row_stats(n);
      }
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
  VerifyRowStats st = s_st;
  int64_t tok;
  if (greedy || !(st.m > -INFINITY)) {
    tok = st.arg;
  } else {
    // weights w(v) = p(v) (bonus) or max(0, p(v) - q(v)) (after a rejection);
    // when no residual weight is positive (q covers p) the draw is from p
    const TIO* z = logits + row * row_stride;
    const RowGeom g = row_geom(z, valid);
    const double u = (double)u_residual[r];
    double* cs_row = chunk_sums + row * row_sums * nch_bound;
    float* cr_row = chunk_ref + row * row_sums * nch_bound;
    // Regions in id order: 0 = head singles, then the chunks of segment
    // seg, wave w, chunk j at 1 + (seg * waves + w) * nch_bound + j (empty
    // past a wave's last chunk), last = tail singles.  Each thread sums a
    // contiguous block of regions; the blocks are scanned.
    const int64_t n_regions = 2 + row_sums * nch_bound;
    const int64_t per = (n_regions + kCommitThreads - 1) / kCommitThreads;
    const int64_t r0 = (int64_t)tid * per, r1 = r0 + per < n_regions ? r0 + per : n_regions;
    tok = -1;
    // With approximate sums the draw stands where the bound cannot move it:
    // every cumulative weight is within 2 b / S of its exact value (the chunk
    // sums' errors add up to at most b / S, and the normaliser's error moves
    // every p, hence every weight max(0, p - q), by at most b / S of p), and
    // so is the target u * total; the drawn id stands when the target lies
    // more than 4 b / S (plus rounding) inside its cumulative interval.
    // Otherwise the row's sums are recomputed in fp64 and the draw taken
    // again.
    bool undecided = false;
    for (int exact = (FIXUP || st.b == 0.0) ? 1 : 0; exact < 2 && tok < 0; ++exact) {
      if (exact && !FIXUP && st.b != 0.0) {                 // left to the exact pass
        undecided = true;
        break;
      }
      const double ms = st.m * inv_t;
      const double margin = 4.0 * st.b / st.s + 0x1p-40;
      auto p_of = [&](int64_t v) { return exp_tab(fma(logit_at(z, v), inv_t, -ms), s_exp) / st.s; };
      for (int attempt = 0; attempt < 2 && tok < 0; ++attempt) {
        const int nc = attempt == 0 ? s_nc : 0;
        // the candidates are in id order: the first at or after v by
        // bisection, then q of each entry holding v taken off in turn
        auto lower = [&](int64_t v) {
          int lo = 0, hi = nc;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_cid[mid] < v) lo = mid + 1;
            else hi = mid;
          }
          return lo;
        };
        auto weight_at = [&](int64_t v, double w, int c) {  // w = p(v), c = lower(v)
          for (; c < nc && s_cid[c] == v; ++c) w = w - s_cq[c] > 0.0 ? w - s_cq[c] : 0.0;
          return w;
        };
        auto weight = [&](int64_t v) { return weight_at(v, p_of(v), lower(v)); };
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
          if (i0 >= whi) return 0.0;
          const float ref = cr_row[k];                       // the chunk's reference maximum
          const double sc = ref > -INFINITY ? exp_nonpos(((double)ref - st.m) * inv_t) / st.s : 0.0;
          if (!(sc > 0.0)) return 0.0;
          const int64_t i1 = i0 + kChunkVecs < whi ? i0 + kChunkVecs : whi;
          a = g.head + i0 * VEC;
          b = g.head + i1 * VEC;
          double s = cs_row[k] * sc;
          for (int c = lower(a); c < nc && s_cid[c] < b; ++c)   // the residual at the candidate ids
            if (c == 0 || s_cid[c - 1] != s_cid[c]) {
              const double pc = exp_tab(fma(s_cz[c], inv_t, -ms), s_exp) / st.s;   // p of that id
              s -= pc - weight_at(s_cid[c], pc, c);
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
          s_sure = 1;
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
        // no weight, or a total within the bound of none: exact sums decide
        if (!exact && total <= 4.0 * margin) break;
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
        // the region's ids (at most kChunkVecs * VEC, kIdsPer consecutive ids
        // per thread): weights in parallel, scanned in id order; the first
        // whose cumulative weight passes the target, else the last with weight
        constexpr int kIdsPer = (kChunkVecs * VEC + kCommitThreads - 1) / kCommitThreads;
        const int64_t v0 = ra + (int64_t)tid * kIdsPer;
        double wl[kIdsPer], wv = 0.0;
        int cl = v0 < rb ? lower(v0) : nc;
#pragma unroll
        for (int i = 0; i < kIdsPer; ++i) {
          wl[i] = 0.0;
          if (v0 + i < rb) {
            while (cl < nc && s_cid[cl] < v0 + i) ++cl;
            wl[i] = weight_at(v0 + i, p_of(v0 + i), cl);
          }
          wv += wl[i];
        }
        double vtotal;
        const double vincl = block_scan(wv, s_wtot, vtotal) + base;
        int64_t hit = -1, last = -1;
        double hlo = 0.0, hhi = 0.0, cum = vincl - wv;
#pragma unroll
        for (int i = 0; i < kIdsPer; ++i) {
          if (wl[i] > 0.0) {
            last = v0 + i;
            if (hit < 0 && cum + wl[i] > target) {
              hit = v0 + i;
              hlo = cum;
              hhi = cum + wl[i];
            }
          }
          cum += wl[i];
        }
        if (last >= 0) atomicMax(&s_lastid, (unsigned long long)(last + 1));
        if (hit >= 0) atomicMin(&s_tok, (unsigned long long)hit);
        __syncthreads();
        // the drawn id stands if the target is well inside its interval
        if (!exact) {
          if (s_tok == ~0ull || s_block >= kCommitThreads) {
            if (tid == 0) s_sure = 0;
          } else if (hit == (int64_t)s_tok && !(hhi - target > margin && target - hlo > margin)) {
            s_sure = 0;
          }
          __syncthreads();
        }
        const bool sure = exact || s_sure != 0;
        if (sure) tok = s_tok != ~0ull ? (int64_t)s_tok : s_lastid > 0 ? (int64_t)(s_lastid - 1) : st.arg;
        __syncthreads();
        if (!sure) break;
      }
    }
    if (undecided) {
      if (tid == 0) {
        pending[r] = n;
        ca.list[atomicAdd(ca.count, 1u)] = r;
      }
      tok = -2;                                              // written by the exact pass
    } else if (tok < 0) {
      tok = st.arg;
    }
  }
  if (FIXUP) {
    if (tid == 0) committed[(int64_t)r * (S + 1) + n] = tok;
    return;
  }
  if (tid == 0) {
    accepted[r] = n;
    if (tok != -2) pending[r] = -1;
  }
  for (int s = tid; s <= S; s += kCommitThreads) {
    int64_t c = -1;
    if (s < n) c = tokens[(int64_t)r * S + s];
    else if (s == n) c = tok;
    if (s != n || tok != -2) committed[(int64_t)r * (S + 1) + s] = c;
  }
}

template <typename TIO>
// (capped at 4 waves per SIMD, 128 registers: four requests per CU at once,
// a few spills on the rare paths; 166 registers let three in and ran 1.5x
// slower on 1024 requests)
__global__ __launch_bounds__(kCommitThreads) __attribute__((amdgpu_waves_per_eu(4))) void verify_commit_kernel(CommitArgs<TIO> ca) {
  commit_body<TIO, false>(ca, blockIdx.x);
}

// The exact (fp64) sums of the rows whose draw the first pass left pending
// (the requests in list[0 .. count)), by (request, segment, wave range)
// items dealt over a fixed grid of kExactGroups workgroups: each item's
// chunk sums against the row maximum (references set to it) and its total.
// With nothing pending every workgroup exits at once.  (One workgroup per
// item: a kernel that also redrew a request in the workgroup finishing its
// last item chained redraws behind later items, 2.5-4x slower.)
constexpr int kExactGroups = 512;
template <typename TIO>
__global__ __launch_bounds__(kVerifyThreads) void verify_exact_kernel(CommitArgs<TIO> ca) {
  const uint32_t items = *ca.count * (uint32_t)kParts;
  if (blockIdx.x >= items) return;                       // uniform over the workgroup
  __shared__ double s_exp[kExpTable];
  __shared__ double s_red[kVerifyWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  exp_table_fill(s_exp);
  for (uint32_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int r = ca.list[item / kParts], part = (int)(item % kParts);
    const int n = ca.pending[r];
    const int64_t row = (int64_t)r * (ca.S + 1) + n;
    const double inv_t = 1.0 / clamp_temperature(ca.temperatures[r]);
    const double m = merge_segments(ca.stats + row * kVerifySegs, inv_t).m;
    const double ms = m * inv_t;
    const TIO* z = ca.logits + row * ca.row_stride;
    const RowGeom g = row_geom(z, ca.valid);
    int64_t wlo, whi;
    g.wave_range(part / kVerifyWaves, part % kVerifyWaves, wlo, whi);
    const int64_t nch = (whi - wlo + kChunkVecs - 1) / kChunkVecs;
    double* cs = ca.chunk_sums + (row * kParts + part) * ca.nch_bound;
    float* cr = ca.chunk_ref + (row * kParts + part) * ca.nch_bound;
    __syncthreads();                                     // the table; s_red of the previous item read
    double lacc = 0.0;
    for (int64_t j = wave; j < nch; j += kVerifyWaves) {
      const double cj = exact_chunk_sum(z + g.head, wlo, whi, j, ms, inv_t, s_exp);
      if (lane == 0) {
        cs[j] = cj;
        cr[j] = (float)m;
      }
      lacc += cj;
    }
    // the head singles with the first range, the tail singles with the last
    if (wave == 0 && (part == 0 || part == kParts - 1))
      lacc += exact_singles(z, g, ca.valid, ms, inv_t, s_exp, part == 0, part == kParts - 1);
    if (lane == 0) s_red[wave] = lacc;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < kVerifyWaves; ++w) t += s_red[w];
      ca.partials[(int64_t)r * kParts + part] = t;
    }
  }
}

// The draws left pending, taken again from the exact sums: one workgroup
// per listed request, over a fixed grid of kFixupGroups workgroups.
constexpr int kFixupGroups = 256;
template <typename TIO>
__global__ __launch_bounds__(kCommitThreads) void verify_fixup_kernel(CommitArgs<TIO> ca) {
  const uint32_t cnt = *ca.count;
  for (uint32_t i = blockIdx.x; i < cnt; i += gridDim.x) {
    __syncthreads();                                     // LDS of the previous request read
    commit_body<TIO, true>(ca, ca.list[i]);
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

// Workspace: VerifyRowStats [rows][kVerifySegs], chunk sums (double) and
// their reference maxima (float), each [rows][kParts][nch_bound], then per
// request the pending row (int32), the list of requests with a pending draw
// (int32) and its length, and the exact range totals (double)
// [n_req][kParts].
struct VerifyLayout {
  size_t chunks, refs, pending, list, count, partials, bytes;
};
VerifyLayout verify_layout(int32_t n_req, int32_t slots, int64_t valid_vocab) {
  const size_t rows = (size_t)n_req * (slots + 1);
  const size_t per_row = (size_t)kParts * verify_chunks_bound(valid_vocab);
  VerifyLayout l;
  l.chunks = rows * kVerifySegs * sizeof(VerifyRowStats);
  l.refs = l.chunks + rows * per_row * sizeof(double);
  l.pending = (l.refs + rows * per_row * sizeof(float) + 7) & ~(size_t)7;
  l.list = l.pending + (size_t)n_req * sizeof(int32_t);
  l.count = l.list + (size_t)n_req * sizeof(int32_t);
  l.partials = (l.count + sizeof(uint32_t) + 7) & ~(size_t)7;
  l.bytes = l.partials + (size_t)n_req * kParts * sizeof(double);
  return l;
}

size_t verify_workspace_bytes(int32_t n_req, int32_t slots, int64_t valid_vocab) {
  return verify_layout(n_req, slots, valid_vocab).bytes;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  if (a.n_req == 0) return hipSuccess;
  const int64_t rows = (int64_t)a.n_req * (a.slots + 1);
  const VerifyLayout l = verify_layout(a.n_req, a.slots, a.valid_vocab);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  VerifyRowStats* stats = reinterpret_cast<VerifyRowStats*>(ws);   // [rows][kVerifySegs]
  double* chunk_sums = reinterpret_cast<double*>(ws + l.chunks);
  float* chunk_ref = reinterpret_cast<float*>(ws + l.refs);
  int32_t* pending = reinterpret_cast<int32_t*>(ws + l.pending);
  double* partials = reinterpret_cast<double*>(ws + l.partials);
  const int32_t nch_bound = verify_chunks_bound(a.valid_vocab);
  int32_t* list = reinterpret_cast<int32_t*>(ws + l.list);
  uint32_t* count = reinterpret_cast<uint32_t*>(ws + l.count);
#define DFLASH_VERIFY(TIO)                                                                                   \
  {                                                                                                          \
    hipLaunchKernelGGL(verify_stats_kernel<TIO>, dim3((unsigned)(rows * kVerifySegs)), dim3(kVerifyThreads), 0,  \
                       stream, static_cast<const TIO*>(a.logits), a.row_stride, a.slots + 1, a.valid_vocab,   \
                       a.temperatures, a.greedy_mask, stats, chunk_sums, chunk_ref, nch_bound,                \
                       count);                                                                               \
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;                                         \
    const CommitArgs<TIO> ca{static_cast<const TIO*>(a.logits), a.row_stride, a.slots, a.top_k, a.valid_vocab, \
                             a.cand_ids, a.q, a.tokens, a.u_accept, a.u_residual, a.temperatures,             \
                             a.greedy_mask, stats, chunk_sums, chunk_ref, nch_bound, pending, list, count,   \
                             partials, a.accepted_out, a.committed_out};                                       \
    hipLaunchKernelGGL(verify_commit_kernel<TIO>, dim3((unsigned)a.n_req), dim3(kCommitThreads), 0, stream, ca); \
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;                                         \
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;                                         \
    hipLaunchKernelGGL(verify_exact_kernel<TIO>, dim3(kExactGroups), dim3(kVerifyThreads), 0, stream, ca);     \
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;                                         \
    hipLaunchKernelGGL(verify_fixup_kernel<TIO>, dim3(kFixupGroups), dim3(kCommitThreads), 0, stream, ca);     \
  }
  if (a.dtype == DFLASH_BF16) {
    DFLASH_VERIFY(uint16_t);
  } else {
    DFLASH_VERIFY(float);
  }
#undef DFLASH_VERIFY
  return hipGetLastError();
}

}  // namespace dflash

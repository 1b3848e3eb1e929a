// C ABI of the DFlash2 draft-block library: host-side validation and launch
// sequencing.  Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "dflash.h"
#include "dflash_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DFLASH_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int elem_bytes(int32_t dtype) { return dtype == DFLASH_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dtype) { return dtype == DFLASH_F32 || dtype == DFLASH_BF16; }
hipStream_t as_hip(dflash_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return DFLASH_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr int64_t kMaxVocab = (int64_t)1 << 24;
// the dense head addresses a 256-row tile of either operand with 32-bit byte
// offsets: row strides (the weight's is hidden_size) stay below 2^22 elements
constexpr int64_t kMaxHeadStride = (int64_t)1 << 22;

// ---------------------------------------------------------------------------
int check_conv(const void* x, const void* base, const void* delta, int64_t delta_row_stride,
               const void* out, int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps,
               int32_t block_size, int32_t dtype) {
  if (!dtype_ok(dtype)) return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: unknown dtype %d", dtype);
  if (n_tokens < 0) return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: n_tokens < 0");
  if (hidden <= 0 || group_size <= 0 || taps <= 0 || block_size <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: hidden, group_size, taps, block_size must be > 0");
  if (hidden % group_size)
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: conv_group_size=%d must divide hidden_size=%d",
                group_size, hidden);
  const int vec = dtype == DFLASH_BF16 ? 8 : 4;
  if (hidden % vec)
    return fail(DFLASH_ERR_UNSUPPORTED, "dflash_conv: hidden must be a multiple of %d", vec);
  if (n_tokens % block_size)
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: n_tokens=%lld is not a whole number of blocks of %d",
                (long long)n_tokens, block_size);
  const int64_t groups = hidden / group_size;
  if (delta_row_stride < (int64_t)taps * groups)
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: delta_row_stride < taps * groups");
  if (n_tokens == 0) return DFLASH_OK;
  if (!x || !base || !delta || !out) return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: null pointer");
  if (!aligned16(x) || !aligned16(base) || !aligned16(out))
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: x, base and out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(delta) % elem_bytes(dtype))
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: delta misaligned");
  const size_t bytes = (size_t)n_tokens * hidden * elem_bytes(dtype);
  if (overlaps(x, bytes, out, bytes)) return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv: out overlaps x");
  return DFLASH_OK;
}

int check_topk(const void* logits, int64_t row_stride, int64_t n_rows, int64_t vocab, int64_t valid_vocab,
               int32_t top_k, float mult, float cap, int32_t dtype, const void* ids_out,
               const void* unary_out, const dflash::TopkPlan& plan, const void* ws, size_t ws_bytes,
               const char* who) {
  if (!dtype_ok(dtype)) return fail(DFLASH_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (n_rows < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_rows < 0", who);
  if (top_k < 1) return fail(DFLASH_ERR_INVALID_ARG, "%s: top_k must be >= 1", who);
  if (top_k > DFLASH_MAX_TOP_K) return fail(DFLASH_ERR_UNSUPPORTED, "%s: top_k > %d", who, DFLASH_MAX_TOP_K);
  if (!(valid_vocab >= top_k && valid_vocab <= vocab && vocab <= row_stride))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: need top_k <= valid_vocab <= vocab <= row_stride", who);
  if (vocab >= kMaxVocab) return fail(DFLASH_ERR_UNSUPPORTED, "%s: vocab must be < 2^24", who);
  if (!(std::isfinite(mult) && mult > 0.f))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: output_multiplier must be finite and > 0", who);
  if (!(std::isfinite(cap) && cap >= 0.f))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: final_logit_softcapping must be finite and >= 0", who);
  if (n_rows == 0) return DFLASH_OK;
  if (!logits || !ids_out || !unary_out) return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(logits) || (row_stride * elem_bytes(dtype)) % 16)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: logits rows must be 16-byte aligned", who);
  if ((reinterpret_cast<uintptr_t>(ids_out) & 7) || (reinterpret_cast<uintptr_t>(unary_out) & 3))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: misaligned output", who);
  if (ws_bytes < plan.bytes || (plan.bytes && !ws))
    return fail(DFLASH_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes, plan.bytes);
  if (plan.bytes && (reinterpret_cast<uintptr_t>(ws) & 255))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", who);
  return DFLASH_OK;
}

int check_select(const int64_t* ids, const float* unary, const void* hidden, int64_t req_stride,
                 int64_t slot_stride, const int64_t* anchor, const void* sel_a, const void* sel_b,
                 const void* proj, int32_t n_req, int32_t slots, int32_t top_k, int32_t hidden_size,
                 int32_t rank, int64_t vocab, int32_t dtype, const char* who) {
  if (!dtype_ok(dtype)) return fail(DFLASH_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (n_req < 0 || slots < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_req and slots must be >= 0", who);
  if (top_k < 1) return fail(DFLASH_ERR_INVALID_ARG, "%s: top_k must be >= 1", who);
  if (top_k > DFLASH_MAX_TOP_K) return fail(DFLASH_ERR_UNSUPPORTED, "%s: top_k > %d", who, DFLASH_MAX_TOP_K);
  if (rank < 1 || hidden_size < 1 || vocab < 1)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: rank, hidden_size and vocab must be >= 1", who);
  const int vec = dtype == DFLASH_BF16 ? 8 : 4;
  if (hidden_size % vec) return fail(DFLASH_ERR_UNSUPPORTED, "%s: hidden_size must be a multiple of %d", who, vec);
  if (dtype == DFLASH_BF16 && rank > 128) return fail(DFLASH_ERR_UNSUPPORTED, "%s: bf16 rank > 128", who);
  if (rank > dflash::kMaxLatticeKpad || dflash::lattice_kpad_floats(top_k, rank, dtype) > dflash::kMaxLatticeKpad)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: rank too large for the lattice kernels", who);
  if (vocab >= ((int64_t)1 << 31)) return fail(DFLASH_ERR_UNSUPPORTED, "%s: vocab must be < 2^31", who);
  if (req_stride < 0 || slot_stride < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: negative stride", who);
  if ((int64_t)n_req * slots == 0) return DFLASH_OK;
  if (!ids || !unary || !hidden || !anchor || !sel_a || !sel_b || !proj)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  const int e = elem_bytes(dtype);
  if (!aligned16(hidden) || (req_stride * e) % 16 || (slot_stride * e) % 16 || !aligned16(proj))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: hidden rows and proj must be 16-byte aligned", who);
  if ((reinterpret_cast<uintptr_t>(sel_a) % e) || (reinterpret_cast<uintptr_t>(sel_b) % e))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: selector tables misaligned", who);
  return DFLASH_OK;
}

int check_walk(const float* scores, const int64_t* ids, const float* uniforms, const float* temperatures,
               const uint8_t* greedy, int32_t n_req, int32_t slots, int32_t top_k, const int64_t* tokens,
               const float* q, const char* who) {
  if (n_req < 0 || slots < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_req and slots must be >= 0", who);
  if (top_k < 1) return fail(DFLASH_ERR_INVALID_ARG, "%s: top_k must be >= 1", who);
  if (top_k > DFLASH_MAX_TOP_K) return fail(DFLASH_ERR_UNSUPPORTED, "%s: top_k > %d", who, DFLASH_MAX_TOP_K);
  if ((int64_t)n_req * slots == 0) return DFLASH_OK;
  if (!scores || !ids || !uniforms || !temperatures || !greedy || !tokens || !q)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  return DFLASH_OK;
}

int record(void* const* events, int idx, hipStream_t s) {
  if (!events || !events[idx]) return DFLASH_OK;
  const hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(events[idx]), s);
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "stage event record failed: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

// The conv -> projection chain of a draft block does not depend on the
// top-K, so it runs on an auxiliary stream of the library beside it: one per
// host thread and device, created on first use with default priority and
// held until the process ends (as are its two events).
struct ForkJoin {
  hipStream_t aux;
  hipEvent_t fork, join;
};
constexpr int kMaxDevices = 64;
// The two events only order work between two streams of one device: no
// timing, and no system-scope fence (nothing on the host waits for them;
// the device-side ordering and the kernel-boundary cache maintenance still
// hold).  The system-scope fence would cost a cache write-back per call.
constexpr unsigned kOrderFlags = hipEventDisableTiming | hipEventDisableSystemFence;

int fork_join(ForkJoin** out, const char* who) {
  thread_local ForkJoin per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_ERR_UNSUPPORTED, "%s: device index %d", who, dev);
  ForkJoin& f = per_device[dev];
  if (!f.aux) {
    ForkJoin n{};
    e = hipStreamCreateWithFlags(&n.aux, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, kOrderFlags);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, kOrderFlags);
    if (e != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);   // best effort: the set-up error is the one reported
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.aux) (void)hipStreamDestroy(n.aux);
      return fail(DFLASH_ERR_LAUNCH, "%s: auxiliary stream set-up failed: %s", who, hipGetErrorString(e));
    }
    f = n;
  }
  *out = &f;
  return DFLASH_OK;
}

int stream_op(hipError_t e, const char* who) {
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "%s: stream ordering failed: %s", who, hipGetErrorString(e));
  return DFLASH_OK;
}

struct BlockLayout {
  dflash::TopkPlan topk;
  dflash::ProjPlan proj;
  size_t proj_off, scores_off, bytes;
};

BlockLayout block_layout(const dflash_draft_config* cfg, int32_t n_req, int64_t valid_vocab) {
  BlockLayout L{};
  const int32_t slots = cfg->block_size - 1;
  const int64_t rows = (int64_t)n_req * slots;
  const int32_t K = cfg->selector_top_k, r = cfg->selector_rank;
  L.topk = dflash::plan_topk(rows, valid_vocab, K);
  // dtype only changes the projection split; size for the larger plan
  const dflash::ProjPlan pb = dflash::plan_proj((int32_t)rows, r, cfg->hidden_size, DFLASH_BF16);
  const dflash::ProjPlan pf = dflash::plan_proj((int32_t)rows, r, cfg->hidden_size, DFLASH_F32);
  L.proj_off = align256(L.topk.bytes);
  L.scores_off = L.proj_off + align256(pb.bytes > pf.bytes ? pb.bytes : pf.bytes);
  // the scores need workspace only when no lattice + walk kernel keeps a
  // request's scores on chip (its LDS need, for the larger dtype)
  const size_t lw = std::max(dflash::lattice_walk_lds_bytes(slots, K, r, DFLASH_BF16),
                             dflash::lattice_walk_lds_bytes(slots, K, r, DFLASH_F32));
  const bool scores_in_ws = lw > dflash::kLatticeWalkLdsMax;
  L.bytes = L.scores_off + (scores_in_ws ? align256((size_t)rows * K * K * sizeof(float)) : 0);
  return L;
}

// Scratch of dflash_propose_block_noalloc: device storage of the library
// itself (each GPU holds its own copy from the library's first use on it
// until the process ends).  In host code `scratch` names a host-side stand-in,
// not device memory: the device address comes from hipGetSymbolAddress, once
// per device (scratch_ptr), and only that address is ever handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) static unsigned char scratch[kNoAllocScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

int scratch_ptr(void** out, const char* who) {
  static DeviceScratch per_device[kMaxDevices];
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DFLASH_ERR_LAUNCH, "%s: hipGetDevice failed: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_ERR_UNSUPPORTED, "%s: device index %d", who, dev);
  DeviceScratch& d = per_device[dev];
  // with device `dev` current: its copy of the array
  std::call_once(d.once, [&] { d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
  if (d.err != hipSuccess || !d.ptr)
    return fail(DFLASH_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed: %s", who, hipGetErrorString(d.err));
  *out = d.ptr;
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_abi_version(void) { return DFLASH_ABI_VERSION; }

const char* dflash_last_error(void) { return g_last_error.c_str(); }

int dflash_validate_config(const dflash_draft_config* c) {
  if (!c) return fail(DFLASH_ERR_INVALID_ARG, "dflash_validate_config: null config");
  if (c->conv_kernel_size < 0 || c->conv_group_size < 0 || c->selector_rank < 0 || c->selector_top_k < 0)
    return fail(DFLASH_ERR_INVALID_ARG, "draft config: negative field");
  if ((c->conv_kernel_size > 0) != (c->conv_group_size > 0))
    return fail(DFLASH_ERR_INVALID_ARG, "draft config: conv_kernel_size and conv_group_size must be set together");
  if ((c->selector_rank > 0) != (c->selector_top_k > 0))
    return fail(DFLASH_ERR_INVALID_ARG, "draft config: selector_rank and selector_top_k must be set together");
  if (!(std::isfinite(c->output_multiplier) && c->output_multiplier > 0.f))
    return fail(DFLASH_ERR_INVALID_ARG, "draft config: output_multiplier must be finite and > 0");
  if (!(std::isfinite(c->final_logit_softcapping) && c->final_logit_softcapping >= 0.f))
    return fail(DFLASH_ERR_INVALID_ARG, "draft config: final_logit_softcapping must be finite and >= 0");
  if (c->block_size < 1) return fail(DFLASH_ERR_INVALID_ARG, "draft config: block_size must be >= 1");
  if (c->hidden_size < 1) return fail(DFLASH_ERR_INVALID_ARG, "draft config: hidden_size must be >= 1");
  if (c->conv_group_size > 0 && c->hidden_size % c->conv_group_size)
    return fail(DFLASH_ERR_INVALID_ARG, "draft config: conv_group_size=%d must divide hidden_size=%d",
                c->conv_group_size, c->hidden_size);
  if (c->selector_top_k > DFLASH_MAX_TOP_K)
    return fail(DFLASH_ERR_UNSUPPORTED, "draft config: selector_top_k > %d", DFLASH_MAX_TOP_K);
  return ok();
}

int dflash_conv(const void* x, const void* base, const void* delta, int64_t delta_row_stride, void* out,
                int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps, int32_t block_size,
                int32_t dtype, dflash_stream_t stream) {
  int st = check_conv(x, base, delta, delta_row_stride, out, n_tokens, hidden, group_size, taps, block_size,
                      dtype);
  if (st != DFLASH_OK) return st;
  if (n_tokens == 0) return ok();
  dflash::ConvArgs a{x, base, delta, delta_row_stride, out, n_tokens, hidden, group_size, taps, block_size,
                     dtype};
  st = launch_status(dflash::launch_conv(a, as_hip(stream)), "dflash_conv");
  return st == DFLASH_OK ? ok() : st;
}

size_t dflash_conv_prepare_workspace_size(int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps,
                                          int32_t dtype) {
  if (n_tokens <= 0 || hidden <= 0 || group_size <= 0 || taps <= 0 || hidden % group_size) return 0;
  const int64_t outputs = 2LL * taps * (hidden / group_size);
  if (outputs > INT32_MAX) return 0;
  return dflash::plan_conv_prepare(n_tokens, hidden, (int32_t)outputs, dtype).bytes;
}

int dflash_conv_prepare(const void* x, const void* proj_weight, const void* base2, void* out, void* coeff_out,
                        int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps, int32_t block_size,
                        int32_t dtype, void* workspace, size_t workspace_bytes, dflash_stream_t stream) {
  if (hidden > 0 && group_size > 0 && taps > 0 && hidden % group_size == 0 &&
      2LL * taps * (hidden / group_size) > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "dflash_conv_prepare: 2*taps*groups too large");
  const int64_t P = (hidden > 0 && group_size > 0) ? 2LL * (taps > 0 ? taps : 1) * (hidden / group_size) : 1;
  int st = check_conv(x, base2, coeff_out, P, out, n_tokens, hidden, group_size, taps, block_size, dtype);
  if (st != DFLASH_OK) return st;
  if (n_tokens == 0) return ok();
  if (!proj_weight) return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv_prepare: null proj_weight");
  if (!aligned16(proj_weight) || !aligned16(coeff_out))
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv_prepare: proj_weight and coeff_out must be 16-byte aligned");
  const size_t e = elem_bytes(dtype);
  const size_t xb = (size_t)n_tokens * hidden * e, cb = (size_t)n_tokens * P * e;
  if (overlaps(coeff_out, cb, x, xb) || overlaps(coeff_out, cb, out, xb) ||
      overlaps(coeff_out, cb, proj_weight, (size_t)P * hidden * e) ||
      overlaps(coeff_out, cb, base2, 2 * (size_t)taps * hidden * e) ||
      overlaps(out, xb, proj_weight, (size_t)P * hidden * e) || overlaps(out, xb, base2, 2 * (size_t)taps * hidden * e))
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv_prepare: an output overlaps another buffer");
  const dflash::ConvPrepPlan plan = dflash::plan_conv_prepare(n_tokens, hidden, (int32_t)P, dtype);
  if (plan.bytes > 0) {
    if (!workspace || workspace_bytes < plan.bytes)
      return fail(DFLASH_ERR_WORKSPACE, "dflash_conv_prepare: workspace needs %zu bytes", plan.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(DFLASH_ERR_INVALID_ARG, "dflash_conv_prepare: workspace must be 256-byte aligned");
  }
  dflash::ConvPrepArgs a{x, proj_weight, base2, out, coeff_out, n_tokens, hidden, group_size, taps, block_size,
                         dtype, workspace};
  st = launch_status(dflash::launch_conv_prepare(a, plan, as_hip(stream)), "dflash_conv_prepare");
  return st == DFLASH_OK ? ok() : st;
}

int dflash_philox_uniforms(const uint64_t* seed_offset, int64_t n, float* out, dflash_stream_t stream) {
  const char* who = "dflash_philox_uniforms";
  if (n < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n < 0", who);
  if (n == 0) return ok();
  if (!seed_offset || !out) return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  if (reinterpret_cast<uintptr_t>(seed_offset) % 8 || reinterpret_cast<uintptr_t>(out) % 4)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (overlaps(seed_offset, 16, out, (size_t)n * 4))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: out overlaps seed_offset", who);
  const int st = launch_status(dflash::launch_philox_uniforms(seed_offset, n, out, as_hip(stream)), who);
  return st == DFLASH_OK ? ok() : st;
}

int dflash_hbm_ceiling(int32_t kind, const void* src, void* dst, int64_t bytes, dflash_stream_t stream) {
  const char* who = "dflash_hbm_ceiling";
  if (kind != DFLASH_CEILING_READ && kind != DFLASH_CEILING_COPY)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: unknown kind %d", who, kind);
  if (bytes < 0 || bytes % 16) return fail(DFLASH_ERR_INVALID_ARG, "%s: bytes must be >= 0 and a multiple of 16", who);
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(src) || (kind == DFLASH_CEILING_COPY ? !aligned16(dst) : reinterpret_cast<uintptr_t>(dst) % 4))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: misaligned pointer", who);
  if (overlaps(src, (size_t)bytes, dst, kind == DFLASH_CEILING_COPY ? (size_t)bytes : 4))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: dst overlaps src", who);
  const int st = launch_status(dflash::launch_hbm_ceiling(kind, src, dst, bytes, as_hip(stream)), who);
  return st == DFLASH_OK ? ok() : st;
}

size_t dflash_verify_workspace_size(int32_t n_req, int32_t slots, int64_t valid_vocab) {
  if (n_req <= 0 || slots < 0 || valid_vocab <= 0) return 0;
  return dflash::verify_workspace_bytes(n_req, slots, valid_vocab);
}

int dflash_verify(const void* target_logits, int64_t row_stride, int32_t n_req, int32_t slots, int64_t vocab,
                  int64_t valid_vocab, int32_t top_k, const int64_t* cand_ids, const float* q, const int64_t* tokens,
                  const float* u_accept, const float* u_residual, const float* temperatures,
                  const uint8_t* greedy_mask, int32_t dtype, int32_t* accepted_out, int64_t* committed_out,
                  void* workspace, size_t workspace_bytes, dflash_stream_t stream) {
  const char* who = "dflash_verify";
  if (!dtype_ok(dtype)) return fail(DFLASH_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (n_req < 0 || slots < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_req and slots must be >= 0", who);
  if (top_k < 1) return fail(DFLASH_ERR_INVALID_ARG, "%s: top_k must be >= 1", who);
  if (top_k > DFLASH_MAX_TOP_K) return fail(DFLASH_ERR_UNSUPPORTED, "%s: top_k > %d", who, DFLASH_MAX_TOP_K);
  if (!(valid_vocab >= 1 && valid_vocab <= vocab && vocab <= row_stride))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: need 1 <= valid_vocab <= vocab <= row_stride", who);
  if (n_req == 0) return ok();
  if (!target_logits || !u_residual || !temperatures || !greedy_mask || !accepted_out || !committed_out ||
      (slots > 0 && (!cand_ids || !q || !tokens || !u_accept)))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  if (reinterpret_cast<uintptr_t>(target_logits) % elem_bytes(dtype))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: target_logits misaligned", who);
  const size_t need = dflash_verify_workspace_size(n_req, slots, valid_vocab);
  if (!workspace || workspace_bytes < need)
    return fail(DFLASH_ERR_WORKSPACE, "%s: workspace needs %zu bytes", who, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 8)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: workspace must be 8-byte aligned", who);
  dflash::VerifyArgs a{target_logits, row_stride, vocab, valid_vocab, n_req, slots, top_k, cand_ids, q, tokens,
                       u_accept, u_residual, temperatures, greedy_mask, dtype, accepted_out, committed_out, workspace};
  const int st = launch_status(dflash::launch_verify(a, as_hip(stream)), who);
  return st == DFLASH_OK ? ok() : st;
}

size_t dflash_topk_workspace_size(int64_t n_rows, int64_t valid_vocab, int32_t top_k) {
  if (n_rows <= 0 || valid_vocab <= 0 || top_k <= 0) return 0;
  return dflash::plan_topk(n_rows, valid_vocab, top_k).bytes;
}

int dflash_topk(const void* logits, int64_t row_stride, int64_t n_rows, int64_t vocab, int64_t valid_vocab,
                int32_t top_k, float output_multiplier, float softcap, int32_t dtype, int64_t* ids_out,
                float* unary_out, void* workspace, size_t workspace_bytes, dflash_stream_t stream) {
  const dflash::TopkPlan plan = dflash::plan_topk(n_rows > 0 ? n_rows : 0, valid_vocab > 0 ? valid_vocab : 1,
                                                  top_k > 0 ? top_k : 1);
  int st = check_topk(logits, row_stride, n_rows, vocab, valid_vocab, top_k, output_multiplier, softcap, dtype,
                      ids_out, unary_out, plan, workspace, workspace_bytes, "dflash_topk");
  if (st != DFLASH_OK) return st;
  if (n_rows == 0) return ok();
  dflash::TopkArgs a{logits, row_stride, n_rows, vocab, valid_vocab, top_k, output_multiplier, softcap,
                     dtype, ids_out, unary_out, workspace};
  st = launch_status(dflash::launch_topk(a, plan, as_hip(stream)), "dflash_topk");
  return st == DFLASH_OK ? ok() : st;
}

size_t dflash_lattice_workspace_size(int32_t n_req, int32_t slots, int32_t rank, int32_t hidden_size) {
  if (n_req <= 0 || slots <= 0 || rank <= 0 || hidden_size <= 0) return 0;
  const dflash::ProjPlan pb = dflash::plan_proj(n_req * slots, rank, hidden_size, DFLASH_BF16);
  const dflash::ProjPlan pf = dflash::plan_proj(n_req * slots, rank, hidden_size, DFLASH_F32);
  return pb.bytes > pf.bytes ? pb.bytes : pf.bytes;
}

int dflash_lattice(const int64_t* ids, const float* unary, const void* hidden, int64_t hidden_req_stride,
                   int64_t hidden_slot_stride, const int64_t* anchor_ids, const void* sel_a, const void* sel_b,
                   const void* proj, int32_t n_req, int32_t slots, int32_t top_k, int32_t hidden_size,
                   int32_t rank, int64_t vocab, int32_t dtype, float* scores_out, void* workspace,
                   size_t workspace_bytes, dflash_stream_t stream) {
  int st = check_select(ids, unary, hidden, hidden_req_stride, hidden_slot_stride, anchor_ids, sel_a, sel_b,
                        proj, n_req, slots, top_k, hidden_size, rank, vocab, dtype, "dflash_lattice");
  if (st != DFLASH_OK) return st;
  if ((int64_t)n_req * slots == 0) return ok();
  if (!scores_out) return fail(DFLASH_ERR_INVALID_ARG, "dflash_lattice: null scores_out");
  const dflash::ProjPlan plan = dflash::plan_proj(n_req * slots, rank, hidden_size, dtype);
  if (workspace_bytes < plan.bytes || !workspace)
    return fail(DFLASH_ERR_WORKSPACE, "dflash_lattice: workspace of %zu bytes < %zu needed", workspace_bytes,
                plan.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(DFLASH_ERR_INVALID_ARG, "dflash_lattice: workspace must be 256-byte aligned");
  dflash::SelectArgs a{ids, unary, hidden, hidden_req_stride, hidden_slot_stride, anchor_ids, sel_a, sel_b,
                       proj, n_req, slots, top_k, hidden_size, rank, vocab, dtype,
                       static_cast<float*>(workspace), scores_out};
  st = launch_status(dflash::launch_proj(a, plan, as_hip(stream)), "dflash_lattice(projection)");
  if (st != DFLASH_OK) return st;
  st = launch_status(dflash::launch_lattice(a, plan, as_hip(stream)), "dflash_lattice");
  return st == DFLASH_OK ? ok() : st;
}

int dflash_walk(const float* scores, const int64_t* ids, const float* uniforms, const float* temperatures,
                const uint8_t* greedy_mask, int32_t n_req, int32_t slots, int32_t top_k, int64_t* tokens_out,
                float* q_out, dflash_stream_t stream) {
  int st = check_walk(scores, ids, uniforms, temperatures, greedy_mask, n_req, slots, top_k, tokens_out, q_out,
                      "dflash_walk");
  if (st != DFLASH_OK) return st;
  if ((int64_t)n_req * slots == 0) return ok();
  dflash::WalkArgs a{scores, ids, uniforms, temperatures, greedy_mask, n_req, slots, top_k, tokens_out, q_out};
  st = launch_status(dflash::launch_walk(a, as_hip(stream)), "dflash_walk");
  return st == DFLASH_OK ? ok() : st;
}

int dflash_lm_head(const void* hidden, int64_t hidden_row_stride, const void* weight, int64_t n_rows,
                   int32_t hidden_size, int64_t vocab, void* logits_out, int64_t logits_row_stride, int32_t dtype,
                   dflash_stream_t stream) {
  const char* who = "dflash_lm_head";
  if (!dtype_ok(dtype)) return fail(DFLASH_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (dtype != DFLASH_BF16) return fail(DFLASH_ERR_UNSUPPORTED, "%s: bf16 only", who);
  if (n_rows < 0 || vocab < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_rows and vocab must be >= 0", who);
  if (n_rows >= ((int64_t)1 << 31) || vocab >= ((int64_t)1 << 31))
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: n_rows and vocab must be < 2^31", who);
  if (hidden_size < 8 || hidden_size % 8)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: hidden_size must be a positive multiple of 8", who);
  if (hidden_row_stride < hidden_size || logits_row_stride < vocab)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: row strides shorter than the rows", who);
  if (hidden_row_stride % 8 || logits_row_stride % 8)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: row strides must be multiples of 8 elements", who);
  if (hidden_row_stride >= kMaxHeadStride)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: hidden_row_stride and hidden_size must be < 2^22", who);
  if (n_rows == 0 || vocab == 0) return ok();
  if (!hidden || !weight || !logits_out) return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(logits_out))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: hidden, weight and logits_out must be 16-byte aligned", who);
  const size_t lb = ((size_t)(n_rows - 1) * logits_row_stride + vocab) * 2;
  if (overlaps(logits_out, lb, hidden, ((size_t)(n_rows - 1) * hidden_row_stride + hidden_size) * 2) ||
      overlaps(logits_out, lb, weight, (size_t)vocab * hidden_size * 2))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: logits_out overlaps an input", who);
  dflash::LmHeadArgs a{hidden, hidden_row_stride, weight, n_rows, hidden_size, vocab, logits_out, logits_row_stride};
  const int st = launch_status(dflash::launch_lm_head(a, as_hip(stream)), who);
  return st == DFLASH_OK ? ok() : st;
}

size_t dflash_lm_head_topk_workspace_size(int64_t n_rows, int64_t vocab, int32_t top_k) {
  if (n_rows <= 0 || vocab <= 0 || top_k <= 0 || top_k > DFLASH_MAX_TOP_K) return 0;
  return dflash::plan_lm_head_topk(n_rows, vocab, top_k).bytes;
}

int dflash_lm_head_topk(const void* hidden, int64_t hidden_row_stride, const void* weight, int64_t n_rows,
                        int32_t hidden_size, int64_t vocab, int64_t valid_vocab, int32_t top_k,
                        float output_multiplier, float final_logit_softcapping, int32_t dtype, int64_t* ids_out,
                        float* unary_out, void* workspace, size_t workspace_bytes, dflash_stream_t stream) {
  const char* who = "dflash_lm_head_topk";
  if (!dtype_ok(dtype)) return fail(DFLASH_ERR_INVALID_ARG, "%s: unknown dtype %d", who, dtype);
  if (dtype != DFLASH_BF16) return fail(DFLASH_ERR_UNSUPPORTED, "%s: bf16 only", who);
  if (n_rows < 0 || vocab < 1) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_rows >= 0 and vocab >= 1 needed", who);
  if (n_rows >= ((int64_t)1 << 31) || vocab >= kMaxVocab)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: n_rows < 2^31 and vocab < 2^24 needed", who);
  if (valid_vocab < 1 || valid_vocab > vocab)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: need 1 <= valid_vocab <= vocab", who);
  if (top_k < 1 || top_k > valid_vocab) return fail(DFLASH_ERR_INVALID_ARG, "%s: need 1 <= top_k <= valid_vocab", who);
  if (top_k > DFLASH_MAX_TOP_K) return fail(DFLASH_ERR_UNSUPPORTED, "%s: top_k > %d", who, DFLASH_MAX_TOP_K);
  if (!std::isfinite(output_multiplier) || output_multiplier <= 0.f || !std::isfinite(final_logit_softcapping) ||
      final_logit_softcapping < 0.f)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: multiplier must be finite and > 0, softcap finite and >= 0", who);
  if (hidden_size < 8 || hidden_size % 8)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: hidden_size must be a positive multiple of 8", who);
  if (hidden_row_stride < hidden_size || hidden_row_stride % 8)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: hidden_row_stride must be >= hidden_size and a multiple of 8", who);
  if (hidden_row_stride >= kMaxHeadStride)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: hidden_row_stride and hidden_size must be < 2^22", who);
  if (n_rows == 0) return ok();
  if (!hidden || !weight || !ids_out || !unary_out) return fail(DFLASH_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(hidden) || !aligned16(weight))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: hidden and weight must be 16-byte aligned", who);
  const dflash::LmTopkPlan p = dflash::plan_lm_head_topk(n_rows, vocab, top_k);
  if (workspace_bytes < p.bytes || !workspace)
    return fail(DFLASH_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who, workspace_bytes, p.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", who);
  dflash::LmHeadArgs a{hidden, hidden_row_stride, weight, n_rows, hidden_size, vocab, nullptr, 0};
  const int st = launch_status(dflash::launch_lm_head_topk(a, p, valid_vocab, top_k, output_multiplier,
                                                           final_logit_softcapping, ids_out, unary_out, workspace,
                                                           as_hip(stream)),
                               who);
  return st == DFLASH_OK ? ok() : st;
}

size_t dflash_propose_block_workspace_size(const dflash_draft_config* cfg, int32_t n_req, int64_t valid_vocab) {
  if (!cfg || n_req <= 0 || valid_vocab <= 0 || cfg->block_size < 2 || cfg->selector_top_k <= 0 ||
      cfg->selector_rank <= 0 || cfg->hidden_size <= 0)
    return 0;
  return block_layout(cfg, n_req, valid_vocab).bytes;
}

int dflash_propose_block_schedule(const dflash_draft_config* cfg, int32_t n_req, int32_t dtype) {
  if (dflash_validate_config(cfg) != DFLASH_OK) return 0;
  if (cfg->conv_kernel_size == 0 || cfg->selector_top_k == 0 || cfg->block_size < 2 || n_req < 1 ||
      (dtype != DFLASH_F32 && dtype != DFLASH_BF16))
    return 0;
  // the shape fields propose_impl hands to the same decision
  const int32_t B = cfg->block_size, S = B - 1, H = cfg->hidden_size;
  const dflash::ConvArgs ca{nullptr, nullptr, nullptr, 0, nullptr, (int64_t)n_req * B, H,
                            cfg->conv_group_size, cfg->conv_kernel_size, B, dtype};
  const dflash::SelectArgs sa{nullptr, nullptr, nullptr, (int64_t)B * H, (int64_t)H, nullptr, nullptr, nullptr,
                              nullptr, n_req, S, cfg->selector_top_k, H, cfg->selector_rank, 0, dtype,
                              nullptr, nullptr};
  const dflash::ProjPlan pp = dflash::plan_proj(n_req * S, cfg->selector_rank, H, dtype);
  return dflash::conv_slot_proj_fits(ca, sa, pp) ? DFLASH_SCHEDULE_ONE_LAUNCH : DFLASH_SCHEDULE_AUX_STREAM;
}

}  // extern "C"

namespace {

// Stages 0 and 2 on `st`: the conv, then the projection of the slot rows of
// its output.
int conv_and_proj(const dflash::ConvArgs& ca, const dflash::SelectArgs& sa, const dflash::ProjPlan& pp,
                  void* const* ev, hipStream_t st, const char* who) {
  int rc;
  if ((rc = record(ev, 0, st)) != DFLASH_OK) return rc;
  if ((rc = launch_status(dflash::launch_conv(ca, st), who)) != DFLASH_OK) return rc;
  if ((rc = record(ev, 1, st)) != DFLASH_OK) return rc;
  if ((rc = record(ev, 4, st)) != DFLASH_OK) return rc;
  if ((rc = launch_status(dflash::launch_proj(sa, pp, st), who)) != DFLASH_OK) return rc;
  return record(ev, 5, st);
}

// The draft block on `stream` with workspace [ws, ws + ws_bytes).  aux_ok:
// the conv and the projection may run on the library's auxiliary stream
// beside the top-K (created on first use); otherwise every stage runs on
// `stream`, in the order conv, projection, top-K, lattice + walk.
int propose_impl(const dflash_draft_config* cfg, const dflash_block_args* a, dflash_stream_t stream, void* ws_ptr,
                 size_t ws_bytes, bool aux_ok, const char* who) {
  if (!a) return fail(DFLASH_ERR_INVALID_ARG, "%s: null args", who);
  int st = dflash_validate_config(cfg);
  if (st != DFLASH_OK) return st;
  if (cfg->conv_kernel_size == 0 || cfg->selector_top_k == 0)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: needs both the conv and the selector enabled", who);
  if (cfg->block_size < 2) return fail(DFLASH_ERR_INVALID_ARG, "%s: block_size must be >= 2", who);
  if (a->n_req < 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: n_req < 0", who);
  const int32_t B = cfg->block_size, S = B - 1, H = cfg->hidden_size, K = cfg->selector_top_k;
  const int32_t r = cfg->selector_rank, T = cfg->conv_kernel_size, gs = cfg->conv_group_size;
  const int64_t N = (int64_t)a->n_req * B, rows = (int64_t)a->n_req * S;
  if (rows >= ((int64_t)1 << 31)) return fail(DFLASH_ERR_UNSUPPORTED, "%s: too many slot rows", who);
  st = check_conv(a->x, a->conv_base, a->conv_delta, a->delta_row_stride, a->conv_out, N, H, gs, T, B, a->dtype);
  if (st != DFLASH_OK) return st;
  const BlockLayout L = block_layout(cfg, a->n_req > 0 ? a->n_req : 1, a->valid_vocab > 0 ? a->valid_vocab : 1);
  st = check_topk(a->logits, a->logits_row_stride, rows, a->vocab, a->valid_vocab, K, cfg->output_multiplier,
                  cfg->final_logit_softcapping, a->dtype, a->ids_out, a->unary_out, L.topk, ws_ptr, ws_bytes, who);
  if (st != DFLASH_OK) return st;
  st = check_select(a->ids_out, a->unary_out, a->conv_out, (int64_t)B * H, H, a->anchor_ids, a->sel_a, a->sel_b,
                    a->proj, a->n_req, S, K, H, r, a->vocab, a->dtype, who);
  if (st != DFLASH_OK) return st;
  st = check_walk(a->scores_out ? a->scores_out : reinterpret_cast<const float*>(16), a->ids_out, a->uniforms,
                  a->temperatures, a->greedy_mask, a->n_req, S, K, a->tokens_out, a->q_out, who);
  if (st != DFLASH_OK) return st;
  if (a->n_req == 0) return ok();
  if (ws_bytes < L.bytes || (L.bytes && !ws_ptr))
    return fail(DFLASH_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes, L.bytes);
  if (reinterpret_cast<uintptr_t>(ws_ptr) & 255)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", who);

  hipStream_t s = as_hip(stream);
  char* ws = static_cast<char*>(ws_ptr);
  float* scores = a->scores_out ? a->scores_out : reinterpret_cast<float*>(ws + L.scores_off);
  void* const* ev = a->stage_events;
  dflash::TopkArgs ta{a->logits, a->logits_row_stride, rows, a->vocab, a->valid_vocab, K, cfg->output_multiplier,
                      cfg->final_logit_softcapping, a->dtype, a->ids_out, a->unary_out, ws_ptr};
  dflash::ConvArgs ca{a->x, a->conv_base, a->conv_delta, a->delta_row_stride, a->conv_out, N, H, gs, T, B,
                      a->dtype};
  const dflash::ProjPlan pp = dflash::plan_proj((int32_t)rows, r, H, a->dtype);
  const void* hidden = static_cast<const char*>(a->conv_out) + (size_t)H * (a->dtype == DFLASH_BF16 ? 2 : 4);
  dflash::SelectArgs sa{a->ids_out, a->unary_out, hidden, (int64_t)B * H, (int64_t)H, a->anchor_ids, a->sel_a,
                        a->sel_b, a->proj, a->n_req, S, K, H, r, a->vocab, a->dtype,
                        reinterpret_cast<float*>(ws + L.proj_off), scores};
  if (dflash::conv_slot_proj_fits(ca, sa, pp)) {
    // stages 0-2 in one launch on `stream`: the conv and the slot projection
    // as workgroups beside the top-K's (their stage events bracket it)
    if ((st = record(ev, 0, s)) != DFLASH_OK) return st;
    if ((st = record(ev, 2, s)) != DFLASH_OK) return st;
    if ((st = launch_status(dflash::launch_topk_conv_proj(ta, L.topk, ca, sa, pp, s), who)) != DFLASH_OK) return st;
    if ((st = record(ev, 1, s)) != DFLASH_OK) return st;
    if ((st = record(ev, 3, s)) != DFLASH_OK) return st;
    if ((st = record(ev, 4, s)) != DFLASH_OK) return st;
    if ((st = record(ev, 5, s)) != DFLASH_OK) return st;
  } else if (!aux_ok) {
    // every stage on `stream`: conv, projection, then the top-K
    if ((st = conv_and_proj(ca, sa, pp, ev, s, who)) != DFLASH_OK) return st;
    if ((st = record(ev, 2, s)) != DFLASH_OK) return st;
    if ((st = launch_status(dflash::launch_topk(ta, L.topk, s), who)) != DFLASH_OK) return st;
    if ((st = record(ev, 3, s)) != DFLASH_OK) return st;
  } else {
    ForkJoin* fj = nullptr;
    if ((st = fork_join(&fj, who)) != DFLASH_OK) return st;
    hipStream_t aux = fj->aux;
    // fork: the auxiliary stream starts after the work already on `stream`
    if ((st = stream_op(hipEventRecord(fj->fork, s), who)) != DFLASH_OK) return st;
    // stage 1 on `stream`: transform + top-K
    if ((st = record(ev, 2, s)) != DFLASH_OK) return st;
    if ((st = launch_status(dflash::launch_topk(ta, L.topk, s), who)) != DFLASH_OK) return st;
    if ((st = record(ev, 3, s)) != DFLASH_OK) return st;
    // stages 0 and 2 on the auxiliary stream: conv, then the projection of
    // the slot rows of its output
    if ((st = stream_op(hipStreamWaitEvent(aux, fj->fork, 0), who)) != DFLASH_OK) return st;
    if ((st = conv_and_proj(ca, sa, pp, ev, aux, who)) != DFLASH_OK) return st;
    // join: `stream` waits for the auxiliary chain
    if ((st = stream_op(hipEventRecord(fj->join, aux), who)) != DFLASH_OK) return st;
    if ((st = stream_op(hipStreamWaitEvent(s, fj->join, 0), who)) != DFLASH_OK) return st;
  }
  // stage 3 on `stream`: lattice + walk (one kernel when a request's lattice fits in LDS)
  if ((st = record(ev, 6, s)) != DFLASH_OK) return st;
  dflash::WalkArgs wa{scores, a->ids_out, a->uniforms, a->temperatures, a->greedy_mask, a->n_req, S, K,
                      a->tokens_out, a->q_out};
  if (dflash::lattice_walk_fits(sa)) {
    if ((st = launch_status(dflash::launch_lattice_walk(sa, pp, wa, a->scores_out, s), who)) != DFLASH_OK) return st;
  } else {
    if ((st = launch_status(dflash::launch_lattice(sa, pp, s), who)) != DFLASH_OK) return st;
    if ((st = launch_status(dflash::launch_walk(wa, s), who)) != DFLASH_OK) return st;
  }
  if ((st = record(ev, 7, s)) != DFLASH_OK) return st;
  return ok();
}


}  // namespace

extern "C" {

int dflash_propose_block(const dflash_draft_config* cfg, const dflash_block_args* a, dflash_stream_t stream) {
  if (!a) return fail(DFLASH_ERR_INVALID_ARG, "dflash_propose_block: null args");
  return propose_impl(cfg, a, stream, a->workspace, a->workspace_bytes, true, "dflash_propose_block");
}

int dflash_propose_block_noalloc(const dflash_draft_config* cfg, const dflash_block_args* a,
                                 dflash_stream_t stream) {
  const char* who = "dflash_propose_block_noalloc";
  if (!a) return fail(DFLASH_ERR_INVALID_ARG, "%s: null args", who);
  if (!cfg) return fail(DFLASH_ERR_INVALID_ARG, "%s: null config", who);
  if (cfg->block_size >= 2 && cfg->selector_top_k > 0 && cfg->selector_rank > 0 && cfg->hidden_size > 0 &&
      a->n_req > 0 && a->valid_vocab > 0) {
    const size_t need = block_layout(cfg, a->n_req, a->valid_vocab).bytes;
    if (need > kNoAllocScratchBytes)
      return fail(DFLASH_ERR_WORKSPACE, "%s: needs %zu bytes of scratch, more than the %zu-byte static scratch", who,
                  need, kNoAllocScratchBytes);
  }
  void* ptr = nullptr;
  int st = scratch_ptr(&ptr, who);
  if (st != DFLASH_OK) return st;
  return propose_impl(cfg, a, stream, ptr, kNoAllocScratchBytes, false, who);
}

}  // extern "C"

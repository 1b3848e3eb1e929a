/*
 * dflash.h -- C ABI of the DFlash2 draft-block hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * The operations are those of "[Spec] DFlash2: local convolution + candidate
 * selector" (sglang PR 35371):
 *   - the block-causal grouped dynamic depthwise convolution (code excerpt of
 *     the grouped conv and of the conv module),
 *   - the unary logit transform and per-slot top-K (implementation breakdown:
 *     output_multiplier / final_logit_softcapping and the deterministic top-k),
 *   - the candidate-selector lattice (executive summary: the edge formula),
 *   - the per-request greedy / inverse-CDF walk (walk-kernel excerpt and the
 *     lossless-q contract of the executive summary),
 *   - the whole draft block fused in one call (draft-sampler excerpt).
 * Padded vocabulary handling follows "DSpark padded-vocab d2t fix" (vllm PR
 * 55133): ids at or beyond the logical vocabulary are never selected.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  Tensors are
 *     row-major and contiguous unless a stride (in ELEMENTS) is given.
 *   - The caller owns every buffer.  Inputs are never written; outputs are
 *     fully overwritten.  The library never allocates device memory: scratch
 *     comes from a caller-provided workspace whose size is returned by the
 *     matching *_workspace_size() query (0 is a valid size; pass any pointer,
 *     including NULL, then).  A workspace must not be shared by two calls that
 *     may overlap in time.
 *   - Every call enqueues its kernels on `stream` and returns without a host
 *     synchronisation.  Arguments are validated on the host before anything is
 *     enqueued: on any status other than DFLASH_OK nothing was enqueued, except
 *     DFLASH_ERR_LAUNCH (a launch failed; work enqueued before it stays
 *     enqueued).  dflash_last_error() then describes the failure.
 *   - Float storage dtype: DFLASH_BF16 (raw bfloat16 bits) or DFLASH_F32.
 *     One dtype applies to all float inputs of a call that take it; computed
 *     floats (unary, scores, q) are always fp32.
 *   - Vector loads need 16-byte alignment of the tensors and row strides named
 *     in each entry point; a violation is DFLASH_ERR_INVALID_ARG.
 *   - Thread safety: the error string is per thread.  The library's mutable
 *     state is set up on first use and kept until the process ends: the
 *     auxiliary stream and two ordering events of dflash_propose_block (one
 *     set per host thread and device) and the device address of the
 *     no-allocation scratch (one per device); calls from several threads are
 *     safe as long as they share no workspace or output buffers.
 *   - Sizes: 1 <= top_k <= 32; vocab < 2^24; everything else bounded by int64.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dflash_stream_t; /* a hipStream_t (NULL = default stream) */

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = -1, /* argument breaks the contract (the pages' ValueError) */
  DFLASH_ERR_UNSUPPORTED = -2, /* valid but outside what this library implements */
  DFLASH_ERR_WORKSPACE = -3,   /* workspace smaller than the size query returns */
  DFLASH_ERR_LAUNCH = -4       /* a HIP launch reported an error */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

#define DFLASH_ABI_VERSION 1
#define DFLASH_MAX_TOP_K 32

/* Mirrors the six DFlash draft-config fields of the implementation breakdown
 * plus the runtime block size (set_block_size) and the hidden width.
 * Fields of a pair are both 0 (feature off) or both > 0. */
typedef struct {
  int32_t conv_kernel_size;        /* T: taps            } a pair            */
  int32_t conv_group_size;         /* gs: channels/group }                   */
  int32_t selector_rank;           /* r                  } a pair            */
  int32_t selector_top_k;          /* K                  }                   */
  float output_multiplier;         /* m, default 1.0; finite and > 0         */
  float final_logit_softcapping;   /* cap, default 0 (off); finite and >= 0  */
  int32_t block_size;              /* B >= 1, runtime override of the block  */
  int32_t hidden_size;             /* H; H % gs == 0 when the conv is on     */
} dflash_draft_config;

/* Library ABI version (DFLASH_ABI_VERSION). */
int dflash_abi_version(void);

/* Check a draft config (host pointer) against the pages' contract: the conv
 * pair and the selector pair are each both-zero or both-positive, the group
 * size divides the hidden width (grouped-conv module constructor), the
 * multiplier is finite and > 0, the softcap finite and >= 0, block_size >= 1,
 * top_k <= DFLASH_MAX_TOP_K.  Returns DFLASH_OK or DFLASH_ERR_INVALID_ARG
 * (DFLASH_ERR_UNSUPPORTED for top_k beyond the maximum). */
int dflash_validate_config(const dflash_draft_config* cfg);

/* Message of the last failure on the calling thread ("" if none). */
const char* dflash_last_error(void);

/* ---------------------------------------------------------------------------
 * dflash_conv -- block-causal grouped dynamic depthwise convolution.
 *   out[i,c] = sum_{t=0}^{T-1} [i mod B >= t] * (base[t,c] + delta[i,t,c/gs]) * x[i-t,c]
 * (code excerpt of the grouped conv: the coefficient belongs to the OUTPUT
 * token i and tap t; taps that reach before the token's block are zero; the
 * block size may be any value >= 1, power of two or not.)
 *   x      [n_tokens, hidden]              dtype; 16-byte aligned
 *   base   [taps, hidden]                  dtype; 16-byte aligned (one side of
 *                                          the module's [2, taps, hidden] kernel)
 *   delta  row i at delta + i*delta_row_stride, holding [taps, hidden/group_size]
 *                                          dtype; delta_row_stride >= taps*G
 *                                          (2*taps*G when it is one side of the
 *                                          packed [N, 2, taps, G] projection)
 *   out    [n_tokens, hidden]              dtype; 16-byte aligned; may not alias x
 * Arithmetic: fp32 (coefficient = base + delta, then a fused multiply-add per
 * tap, tap 0 first), rounded once to the output dtype (round to nearest even).
 * Requires n_tokens % block_size == 0, hidden % group_size == 0 and hidden a
 * multiple of 8 (bf16) / 4 (fp32).  n_tokens == 0 is a no-op. */
int dflash_conv(const void* x, const void* base, const void* delta, int64_t delta_row_stride,
                void* out, int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps,
                int32_t block_size, int32_t dtype, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_conv_prepare -- the prepare side of the grouped conv module ("[Spec]
 * DFlash2", code excerpt of the conv module: one bias-free projection of the
 * input gives both sides' coefficients, read as [2, taps, G]; prepare
 * convolves the input with side 0 and returns side 1's coefficients):
 *   coeff[n, p] = round( sum_k x[n, k] * proj_weight[p, k] ),  p < 2*taps*G,
 *                 p = side*taps*G + tap*G + group
 *   out         = dflash_conv(x, base2[0], delta = coeff (row stride 2*taps*G))
 *   x           [n_tokens, hidden]            dtype; 16-byte aligned
 *   proj_weight [2*taps*G, hidden]            dtype; 16-byte aligned (the
 *                                             linear map's [out, in] layout)
 *   base2       [2, taps, hidden]             dtype; 16-byte aligned
 *   out         [n_tokens, hidden]            dtype; 16-byte aligned
 *   coeff_out   [n_tokens, 2, taps, G]        dtype; 16-byte aligned; both
 *                                             sides, rounded once (bf16: to
 *                                             nearest even; fp32 sums in fp32)
 * finish is dflash_conv(y, base2 + taps*hidden, coeff_out + taps*G,
 * 2*taps*G, ...).  Conv requirements as for dflash_conv.  bf16 needs
 * dflash_conv_prepare_workspace_size() bytes of scratch (256-byte aligned;
 * may be 0), fp32 none.  n_tokens == 0 is a no-op. */
size_t dflash_conv_prepare_workspace_size(int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps,
                                          int32_t dtype);
int dflash_conv_prepare(const void* x, const void* proj_weight, const void* base2, void* out, void* coeff_out,
                        int64_t n_tokens, int32_t hidden, int32_t group_size, int32_t taps, int32_t block_size,
                        int32_t dtype, void* workspace, size_t workspace_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_topk -- per-row top-K over transformed unary logits.
 * For each row n: the K ids v < valid_vocab with the largest transformed
 * value y = T(z[n,v]), ordered by (y descending, id ascending).  T(z) = m*z,
 * then cap*tanh(T/cap) when cap > 0; -inf stays -inf.  T is strictly
 * increasing, so ranks are taken exactly on the raw logits (-0 == +0).
 * Ids >= valid_vocab are never read or selected (DSpark padded vocab).
 *   logits    row n at logits + n*row_stride, length >= vocab; dtype; the
 *             pointer and row_stride*elem_size 16-byte aligned
 *   ids_out   [n_rows, top_k] int64
 *   unary_out [n_rows, top_k] fp32, T(z) of each selected id
 * Preconditions (not checked on the device): no NaN among the first
 * valid_vocab logits of a row.  Requires 1 <= top_k <= min(32, valid_vocab),
 * valid_vocab <= vocab <= row_stride, vocab < 2^24. */
size_t dflash_topk_workspace_size(int64_t n_rows, int64_t valid_vocab, int32_t top_k);
int dflash_topk(const void* logits, int64_t row_stride, int64_t n_rows, int64_t vocab,
                int64_t valid_vocab, int32_t top_k, float output_multiplier, float softcap,
                int32_t dtype, int64_t* ids_out, float* unary_out, void* workspace,
                size_t workspace_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_lattice -- candidate-selector lattice over adjacent slots.
 *   u[r,s,:]        = P h[r,s,:]                        (rank-r projection)
 *   scores[r,s,j,c] = sum_k A[p,k] * u[r,s,k] * B[ids[r,s,c],k] + unary[r,s,c]
 * with p = anchor[r] for s = 0 (every row j of slot 0 is the same) and
 * p = ids[r,s-1,j] otherwise (executive summary: edge(p -> c) =
 * <A[p] (.) project(h), B[c]> + unary[c]).
 *   ids, unary   [n_req, slots, top_k] int64 / fp32 (dflash_topk's outputs)
 *   hidden       row (r,s) at hidden + r*hidden_req_stride + s*hidden_slot_stride,
 *                hidden_size values; dtype; 16-byte aligned rows
 *   anchor_ids   [n_req] int64
 *   sel_a, sel_b [vocab, rank] dtype;  proj [rank, hidden_size] dtype
 *   scores_out   [n_req, slots, top_k, top_k] fp32
 * Arithmetic: u is a bf16 x bf16 (exact products) fp32-accumulated contraction
 * on the matrix cores (fp32 VALU for DFLASH_F32); each score is the fp32 chain
 * w_k = A[p,k]*u_k, acc = fma(w_k, B[c,k], acc) over k = 0..rank-1, then
 * + unary.  A token id outside [0, vocab) yields NaN scores for the entries
 * that would read it (no out-of-bounds access). */
size_t dflash_lattice_workspace_size(int32_t n_req, int32_t slots, int32_t rank, int32_t hidden_size);
int dflash_lattice(const int64_t* ids, const float* unary, const void* hidden,
                   int64_t hidden_req_stride, int64_t hidden_slot_stride,
                   const int64_t* anchor_ids, const void* sel_a, const void* sel_b,
                   const void* proj, int32_t n_req, int32_t slots, int32_t top_k,
                   int32_t hidden_size, int32_t rank, int64_t vocab, int32_t dtype,
                   float* scores_out, void* workspace, size_t workspace_bytes,
                   dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_walk -- per-request walk over the lattice (walk-kernel excerpt).
 * prev = 0; for each slot s: row = scores[r,s,prev,:].
 *   greedy_mask[r] != 0: idx = lowest index of the row maximum; q = one-hot.
 *   otherwise (fp32, left-to-right sums): t = max(temperatures[r], 1e-5);
 *     x = row / t; e_j = exp(x_j - max x) rounded to fp32; p = e / sum(e);
 *     C_j = p_0 + ... + p_j; idx = min(#{j : C_j <= uniforms[r,s]}, K-1); q = p.
 *   tokens[r,s] = ids[r,s,idx]; q_out[r,s,:] = q; prev = idx.
 *   scores [n_req, slots, top_k, top_k] fp32;  ids [n_req, slots, top_k] int64
 *   uniforms [n_req, slots] fp32 in [0,1);  temperatures [n_req] fp32
 *   greedy_mask [n_req] uint8;  tokens_out [n_req, slots] int64
 *   q_out [n_req, slots, top_k] fp32 */
int dflash_walk(const float* scores, const int64_t* ids, const float* uniforms,
                const float* temperatures, const uint8_t* greedy_mask, int32_t n_req,
                int32_t slots, int32_t top_k, int64_t* tokens_out, float* q_out,
                dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_lm_head -- the dense head of compute_candidates ("[Spec] DFlash2",
 * implementation breakdown and risk notes: the slot hidden rows times the
 * target lm_head weight taken as a dense matrix; the product comes back in
 * the model's dtype):
 *   logits[n, v] = round_bf16( sum_k hidden[n, k] * weight[v, k] )
 *   hidden       row n at hidden + n*hidden_row_stride, hidden_size elements
 *   weight       [vocab, hidden_size], rows contiguous (the head's layout)
 *   logits_out   row n at logits_out + n*logits_row_stride, vocab elements
 * bf16 only (DFLASH_ERR_UNSUPPORTED otherwise).  The products are exact in
 * fp32 and summed in fp32 on the matrix cores; each sum is rounded once to
 * bf16 (nearest, ties to even).  hidden_size must be a multiple of 8;
 * hidden, weight, logits_out and both row strides 16-byte aligned;
 * logits_out must not overlap the inputs; n_rows and vocab below 2^31;
 * hidden_row_stride (hence hidden_size) below 2^22 elements
 * (DFLASH_ERR_UNSUPPORTED otherwise). */
int dflash_lm_head(const void* hidden, int64_t hidden_row_stride, const void* weight, int64_t n_rows,
                   int32_t hidden_size, int64_t vocab, void* logits_out, int64_t logits_row_stride,
                   int32_t dtype, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_lm_head_topk -- compute_candidates from the hidden rows ("[Spec]
 * DFlash2", implementation breakdown: the dense head, the unary transform
 * and the deterministic top-k) without the logits reaching memory:
 *   ids_out[n, 0..K)   = dflash_topk over the rows of dflash_lm_head(hidden)
 *   unary_out[n, 0..K) = their transformed logits
 * bit for bit equal to dflash_lm_head followed by dflash_topk with the same
 * arguments.  Arguments as for those two calls (bf16 only; valid_vocab <=
 * vocab; 1 <= top_k <= DFLASH_MAX_TOP_K, top_k <= valid_vocab).  Scratch:
 * dflash_lm_head_topk_workspace_size(n_rows, vocab, top_k) bytes, 256-byte
 * aligned (per row, the K best of every group of consecutive 256-column
 * tiles, plus a per-row bound). */
size_t dflash_lm_head_topk_workspace_size(int64_t n_rows, int64_t vocab, int32_t top_k);
int dflash_lm_head_topk(const void* hidden, int64_t hidden_row_stride, const void* weight, int64_t n_rows,
                        int32_t hidden_size, int64_t vocab, int64_t valid_vocab, int32_t top_k,
                        float output_multiplier, float final_logit_softcapping, int32_t dtype,
                        int64_t* ids_out, float* unary_out, void* workspace, size_t workspace_bytes,
                        dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_philox_uniforms -- counter-based uniforms for a captured draft step
 * ("[Spec] DFlash2", worker excerpt: the sampler draws its uniforms inside
 * the captured graph).  Philox-4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011):
 *   out[i] = (word i%4 of Philox(counter = {lo, hi of offset + i/4, 0, 0},
 *             key = {lo, hi of seed})) >> 8, times 2^-24      in [0, 1)
 *   seed_offset  device uint64 [2] = {seed, offset}, 8-byte aligned; read by
 *                the kernel, so a captured launch uses what the host staged
 *                before the replay (advance offset by ceil(n/4) per draw)
 *   out          device fp32 [n], 4-byte aligned
 * n == 0 is a no-op. */
int dflash_philox_uniforms(const uint64_t* seed_offset, int64_t n, float* out, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_hbm_ceiling -- measurement support, not a step of the method: the
 * bandwidth this chip sustains for a plain stream of a given size, in the
 * load and store forms the path's streaming kernels use (16-byte lanes,
 * non-temporal), so that a kernel's achieved bandwidth can be read against
 * a stream of the same byte count.
 *   kind   DFLASH_CEILING_READ: reads `bytes` from src (dst: a device word
 *          that receives a value only for one bit pattern of the data);
 *          DFLASH_CEILING_COPY: copies `bytes` from src to dst
 *   src    device, 16-byte aligned; dst 16-byte (copy) or 4-byte (read)
 *          aligned, not overlapping src
 *   bytes  a multiple of 16 (0 is a no-op) */
enum { DFLASH_CEILING_READ = 0, DFLASH_CEILING_COPY = 1 };
int dflash_hbm_ceiling(int32_t kind, const void* src, void* dst, int64_t bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_verify -- verify and commit of a drafted block ("[Spec] DFlash2",
 * executive summary and walk-kernel excerpt: verify checks the drafted tokens
 * against the distribution the walk drew them from -- a point mass on greedy
 * rows -- which is what keeps the draft lossless; the worker then commits the
 * kept tokens and places the bonus token after them).  Rule (the standard
 * rejection rule of speculative sampling):
 *   for s = 0 .. slots-1: keep tokens[r,s] = x while u_accept[r,s]*q(x) < p_s(x),
 *     q(x) = q[r,s,j] for cand_ids[r,s,j] == x (0 if x is not a candidate);
 *   at the first rejection commit a draw from max(0, p_s - q_s) renormalised,
 *   after slots kept tokens commit a draw from p_slots.
 * p_s = softmax(z_s / max(T, 1e-5)) over ids < valid_vocab, or the point mass
 * on the lowest-id maximum for a greedy request; draws are inverse CDFs in id
 * order with u_residual[r] (fp64 sums).
 *   target_logits  rows r*(slots+1) + s, s = 0..slots, row_stride elements
 *                  (row s: the target's logits for slot s given the block
 *                  before it; row slots: after the whole block); dtype
 *   cand_ids, q    [n_req, slots, top_k] int64 / fp32 (the walk's candidates
 *                  and q); tokens [n_req, slots] int64
 *   u_accept       [n_req, slots] fp32 in [0,1); u_residual [n_req] fp32
 *   temperatures   [n_req] fp32; greedy_mask [n_req] u8
 *   accepted_out   [n_req] int32: drafted tokens kept
 *   committed_out  [n_req, slots+1] int64: the kept tokens, then the
 *                  correction or bonus token, then -1
 * The sums behind p are first taken in fp32 with a bound on their error; a
 * decision or draw that the bound cannot settle is taken again from the
 * row's fp64 sums, so results are those of the fp64 rule either way.
 * Scratch: dflash_verify_workspace_size(n_req, slots, valid_vocab) bytes,
 * 8-byte aligned, owned by the caller (per-row statistics, per-chunk sums and
 * their reference maxima for the sampled rows -- about valid_vocab / 80 bytes
 * per target row -- and a list of the requests whose draw needs the fp64
 * sums); calls that share it must be ordered on one stream.  0 when any
 * argument is <= 0.  n_req == 0 is a no-op. */
size_t dflash_verify_workspace_size(int32_t n_req, int32_t slots, int64_t valid_vocab);
int dflash_verify(const void* target_logits, int64_t row_stride, int32_t n_req, int32_t slots, int64_t vocab,
                  int64_t valid_vocab, int32_t top_k, const int64_t* cand_ids, const float* q, const int64_t* tokens,
                  const float* u_accept, const float* u_residual, const float* temperatures,
                  const uint8_t* greedy_mask, int32_t dtype, int32_t* accepted_out, int64_t* committed_out,
                  void* workspace, size_t workspace_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_propose_block -- one whole draft block (draft-sampler excerpt):
 *   conv (side given by the caller's base/delta pointers) ->
 *   transform + top-K over the slot logits ->
 *   projection of each slot's hidden = conv-output row r*B + 1 + s (block
 *   position 0 is the verified anchor) -> lattice -> walk,
 * ordered on `stream` as one unit.  The conv and the projection do not
 * depend on the top-K.  In bf16 with blocks of 2 to 16 tokens, at most 8 taps, a
 * group size that is a multiple of 8, rank <= 128 and fewer than 2048 slot
 * rows, they run as workgroups of the top-K's launch on `stream` (no second
 * stream).  Otherwise they run beside the top-K on an auxiliary stream of the
 * library (one per host thread and device, created on the first such call
 * with default priority and kept until the process ends) that waits for the
 * work already on `stream` and that `stream` waits for before the lattice.
 * Either way the call's outputs are ready for work enqueued on `stream`
 * after it.  Results
 * equal the chain dflash_conv -> dflash_topk -> dflash_lattice -> dflash_walk
 * on the same inputs bit for bit.
 * cfg: conv and selector must both be enabled; cfg->hidden_size = H. */
typedef struct {
  const void* x;              /* [n_req*B, H] dtype */
  const void* conv_base;      /* [T, H] dtype */
  const void* conv_delta;     /* row i at conv_delta + i*delta_row_stride: [T, G] dtype */
  int64_t delta_row_stride;   /* elements, >= T*G */
  const void* logits;         /* row (r*(B-1)+s) at logits + row*logits_row_stride */
  int64_t logits_row_stride;  /* elements, >= vocab */
  int64_t vocab;              /* physical vocab: logits row length and rows of sel_a/sel_b */
  int64_t valid_vocab;        /* logical vocab: ids >= it are never selected */
  const int64_t* anchor_ids;  /* [n_req] */
  const void* sel_a;          /* [vocab, r] dtype */
  const void* sel_b;          /* [vocab, r] dtype */
  const void* proj;           /* [r, H] dtype */
  const float* uniforms;      /* [n_req, B-1] */
  const float* temperatures;  /* [n_req] */
  const uint8_t* greedy_mask; /* [n_req] */
  void* conv_out;             /* [n_req*B, H] dtype (output) */
  int64_t* ids_out;           /* [n_req, B-1, K] (output) */
  float* unary_out;           /* [n_req, B-1, K] (output) */
  int64_t* tokens_out;        /* [n_req, B-1] (output) */
  float* q_out;               /* [n_req, B-1, K] (output) */
  float* scores_out;          /* [n_req, B-1, K, K] (output) or NULL: kept in the workspace */
  void* workspace;
  size_t workspace_bytes;
  /* NULL, or 8 hipEvent_t handles (host array): events[2*k] is recorded before
   * and events[2*k+1] after stage k on the stream that runs it; stages:
   * 0 conv and 2 projection (auxiliary stream), 1 top-K and 3 lattice + walk
   * (`stream`).  When the conv and the projection share the top-K's launch,
   * stages 0 and 1 both bracket that launch and stage 2 brackets nothing.  A
   * NULL entry skips that record.  For timing only. */
  void* const* stage_events;
  int32_t n_req;
  int32_t dtype;
} dflash_block_args;

size_t dflash_propose_block_workspace_size(const dflash_draft_config* cfg, int32_t n_req,
                                           int64_t valid_vocab);

/* Which schedule dflash_propose_block takes for this config, batch size and
 * dtype, decided on the host from these alone (no GPU work, no allocation):
 *   DFLASH_SCHEDULE_ONE_LAUNCH: conv and projection are workgroups of the
 *     top-K's launch on `stream`;
 *   DFLASH_SCHEDULE_AUX_STREAM: conv then projection on the auxiliary stream,
 *     beside the top-K on `stream`.
 * dflash_propose_block_noalloc runs the auxiliary-stream work on `stream`
 * before the top-K instead.  Returns 0 for a config or size
 * dflash_propose_block would reject on shape alone (invalid config, conv or
 * selector disabled, block_size < 2, n_req < 1, unknown dtype). */
typedef enum { DFLASH_SCHEDULE_ONE_LAUNCH = 1, DFLASH_SCHEDULE_AUX_STREAM = 2 } dflash_schedule;
int dflash_propose_block_schedule(const dflash_draft_config* cfg, int32_t n_req, int32_t dtype);
int dflash_propose_block(const dflash_draft_config* cfg, const dflash_block_args* args,
                         dflash_stream_t stream);

/*
 * dflash_propose_block_noalloc -- dflash_propose_block for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same computation and
 * results, with no hipMalloc, hipFree or other allocating call inside.
 *   - Scratch: a 64 MiB array of device storage inside the library (each GPU
 *     the library runs on holds its own copy from the first use on it until
 *     the process ends); args->workspace and args->workspace_bytes are
 *     ignored.  A batch whose workspace (dflash_propose_block_workspace_size)
 *     exceeds 64 MiB is rejected with DFLASH_ERR_WORKSPACE, nothing enqueued.
 *   - Every stage runs on `stream` (conv, projection, top-K, lattice + walk),
 *     never on the auxiliary stream; stage events as for dflash_propose_block.
 *   - The scratch is shared by every call on a GPU and keeps whatever the
 *     last call left (no call relies on its contents): two calls that may
 *     overlap in time on the same GPU race.  Serialise them (one stream, or
 *     events).
 */
int dflash_propose_block_noalloc(const dflash_draft_config* cfg, const dflash_block_args* args,
                                 dflash_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */

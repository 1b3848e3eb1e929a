// Internal declarations of the DFlash2 HIP library: the host-side launchers
// called by the C ABI layer and the plans they share with it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "device_common.h"

namespace dflash {

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
struct ConvArgs {
  const void* x;
  const void* base;
  const void* delta;
  int64_t delta_row_stride;
  void* out;
  int64_t n_tokens;
  int32_t hidden, group_size, taps, block_size;
  int32_t dtype;          // DFLASH_F32 / DFLASH_BF16
};
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);

struct TopkPlan {
  int64_t n_rows, valid_vocab;
  int32_t top_k;
  int32_t chunks;           // 16384-value chunks per row
  int32_t segs;             // workgroups per row (1: no merge kernel)
  int32_t chunks_per_seg;
  size_t parts_offset;      // byte offset of the per-segment partials in the workspace
  size_t bytes;             // total workspace bytes (0 when segs == 1)
};
TopkPlan plan_topk(int64_t n_rows, int64_t valid_vocab, int32_t top_k);
// LDS slots for one chunk's new candidates, and for a row merge.
constexpr int kTopkMergeCap = 2048;

struct TopkArgs {
  const void* logits;
  int64_t row_stride, n_rows, vocab, valid_vocab;
  int32_t top_k;
  float multiplier, softcap;
  int32_t dtype;
  int64_t* ids_out;
  float* unary_out;
  void* workspace;
};
hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t stream);

constexpr int kMaxTopK = 32;   // DFLASH_MAX_TOP_K

// Most slices the projection's contraction is split into (their partial
// sums are added by the consumer, in slice order).  Few: the consumer loads
// and adds every slice of each value it needs, and the projection runs beside
// the top-K, off the critical path, so more workgroups would not pay.
constexpr int kMaxProjSplit = 16;
// The partials are stored slice-major, [ksplit][n_rows][rank]: a workgroup's
// partials of its output tile are whole contiguous rows of one slice, written
// once (no segment shared with another workgroup's slice, so no partial-line
// writes), and a reader of one value takes its slices from ksplit places.
__host__ __device__ inline int64_t proj_part_index(int split, int64_t n_rows, int rank, int64_t row, int col) {
  return ((int64_t)split * n_rows + row) * rank + col;
}
struct ProjPlan {
  int32_t n_rows, rank, hidden;
  int32_t row_tiles, ksplit, kslice;   // split of the contraction over workgroups
  int32_t frags;                       // row fragments of 16 per wave (bf16, per-wave kernel)
  int32_t tiled;                       // 128 x 128 tiles of the shared tile product (bf16, large batches)
  size_t bytes;                        // fp32 partials [ksplit][n_rows][rank]
};
// Slot rows from which the bf16 projection runs as LDS-staged 128 x 128 tiles.
constexpr int kProjTileMinRows = 2048;
ProjPlan plan_proj(int32_t n_rows, int32_t rank, int32_t hidden, int32_t dtype);

struct SelectArgs {
  const int64_t* ids;
  const float* unary;
  const void* hidden;
  int64_t hidden_req_stride, hidden_slot_stride;
  const int64_t* anchor;
  const void* sel_a;
  const void* sel_b;
  const void* proj;
  int32_t n_req, slots, top_k, hidden_size, rank;
  int64_t vocab;
  int32_t dtype;
  float* u_parts;           // workspace: ProjPlan::bytes
  float* scores;            // [n_req, slots, K, K]
};
hipError_t launch_proj(const SelectArgs& a, const ProjPlan& p, hipStream_t stream);
// The propose step's conv and slot-row projection as workgroups of one
// launch (bf16, blocks of 16, <= 8 taps, one group per vector, few rows);
// the same conv_out and projection partials as launch_conv followed by
// launch_proj ...
bool conv_slot_proj_fits(const ConvArgs& c, const SelectArgs& s, const ProjPlan& p);
// ... in the top-K's launch: one kernel for the propose step's first stage.
hipError_t launch_topk_conv_proj(const TopkArgs& a, const TopkPlan& p, const ConvArgs& c, const SelectArgs& s,
                                 const ProjPlan& pp, hipStream_t stream);
hipError_t launch_lattice(const SelectArgs& a, const ProjPlan& p, hipStream_t stream);

struct WalkArgs {
  const float* scores;
  const int64_t* ids;
  const float* uniforms;
  const float* temperatures;
  const uint8_t* greedy;
  int32_t n_req, slots, top_k;
  int64_t* tokens;
  float* q;
};
hipError_t launch_walk(const WalkArgs& a, hipStream_t stream);

// Dense head: logits[n, v] = round_bf16(sum_k hidden[n, k] W[v, k]) (bf16).
struct LmHeadArgs {
  const void* hidden;
  int64_t hidden_row_stride;   // elements
  const void* weight;          // [vocab, hidden_size], rows contiguous
  int64_t n_rows;
  int32_t hidden_size;
  int64_t vocab;
  void* logits;
  int64_t logits_row_stride;   // elements
};
hipError_t launch_lm_head(const LmHeadArgs& a, hipStream_t stream);

// Fused head + top-K: per-row K best of each group of column tiles (sorted
// composites in the workspace [n_rows][n_grp][K]), then a merge per row.
constexpr int kLmMergeCand = 3072;  // merge candidates of one row held in LDS (24 KB)
struct LmTopkPlan {
  int32_t n_mb, n_nb, tiles_per_group, n_grp;
  size_t bound_offset;      // byte offset of the per-row key bounds (uint32 [n_rows])
  size_t bytes;             // total workspace bytes: group lists, then the bounds
};
LmTopkPlan plan_lm_head_topk(int64_t n_rows, int64_t vocab, int32_t top_k);
hipError_t launch_lm_head_topk(const LmHeadArgs& a, const LmTopkPlan& p, int64_t valid_vocab, int32_t top_k,
                               float mult, float cap, int64_t* ids_out, float* unary_out, void* workspace,
                               hipStream_t stream);

// The conv module's prepare side: kernel projection of x (all 2 * T * G
// coefficients of each token, in the storage dtype), then the conv of x with
// side 0.
struct ConvPrepArgs {
  const void* x;            // [n_tokens, hidden]
  const void* proj_weight;  // [2 * taps * G, hidden]
  const void* base2;        // [2, taps, hidden]; side 0 is used
  void* out;                // [n_tokens, hidden]
  void* coeff_out;          // [n_tokens, 2, taps, G]
  int64_t n_tokens;
  int32_t hidden, group_size, taps, block_size;
  int32_t dtype;
  void* workspace;          // fp32 partial sums when the contraction is split
};
struct ConvPrepPlan {
  bool small;               // 64 x 64 tiles instead of 128 x 128
  int32_t n_mb, n_nb;       // tiles over (tokens, coefficients)
  int32_t slices, kb_per_slice;   // split of the contraction (bf16); slices == 1: none
  size_t bytes;             // workspace bytes (0 without a split)
};
ConvPrepPlan plan_conv_prepare(int64_t n_tokens, int32_t hidden, int32_t outputs, int32_t dtype);
hipError_t launch_conv_prepare(const ConvPrepArgs& a, const ConvPrepPlan& p, hipStream_t stream);

// Philox-4x32-10 uniforms: seed_offset = {seed, offset} in device memory.
hipError_t launch_philox_uniforms(const uint64_t* seed_offset, int64_t n, float* out, hipStream_t stream);
// HBM ceilings (ceiling.hip): kind 0 reads bytes from src (dst: a 4-byte
// sink), kind 1 copies them to dst; bytes a multiple of 16.
hipError_t launch_hbm_ceiling(int kind, const void* src, void* dst, int64_t bytes, hipStream_t stream);

// Verify and commit of a drafted block.
struct VerifyRowStats {
  double m;                 // maximum logit of the row (valid ids), -inf if none is finite
  double s;                 // sum_v exp((z_v - m) / T) (sampled requests), approximate
  double b;                 // bound on |s - the exact sum|
  int64_t arg;              // lowest id of the maximum
};
struct VerifyArgs {
  const void* logits;       // [n_req * (slots + 1)] rows of row_stride elements
  int64_t row_stride, vocab, valid_vocab;
  int32_t n_req, slots, top_k;
  const int64_t* cand_ids;  // [n_req, slots, top_k]
  const float* q;           // [n_req, slots, top_k]
  const int64_t* tokens;    // [n_req, slots]
  const float* u_accept;    // [n_req, slots]
  const float* u_residual;  // [n_req]
  const float* temperatures;
  const uint8_t* greedy_mask;
  int32_t dtype;
  int32_t* accepted_out;    // [n_req]
  int64_t* committed_out;   // [n_req, slots + 1]
  void* workspace;          // VerifyRowStats [rows][kVerifySegs], then the chunk sums
};
constexpr int kVerifySegs = 4;   // workgroups (and statistics records) per target row
// chunks per wave of a row segment at most, and the workspace for them
int32_t verify_chunks_bound(int64_t valid_vocab);
size_t verify_workspace_bytes(int32_t n_req, int32_t slots, int64_t valid_vocab);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

// Lattice and walk in one kernel (one workgroup per request) when the
// request's scores and staging fit in LDS; bit-identical to launch_lattice
// followed by launch_walk.  scores_out may be null.
// gfx950 lets one workgroup address 160 KB of LDS
constexpr size_t kLatticeWalkLdsMax = 160 * 1024;
constexpr size_t kWalkLdsMax = 160 * 1024;
size_t lattice_walk_lds_bytes(int slots, int top_k, int rank, int dtype);
bool lattice_walk_fits(const struct SelectArgs& a);   // one kernel can take the request (see below)
// Requests at which the fused lattice + walk switches from one workgroup per
// request (every row decided in parallel) to one wave per request (only the
// walked rows decided, requests overlapping each other).
constexpr int kLatticeWalkWaveMinReq = 512;
bool lattice_walk_per_wave(const struct SelectArgs& a);
// Floats of one slot's zero-padded u row in the lattice kernels (the fp32
// matrix-core tile's k extent for top_k candidates and this rank).
int lattice_kpad_floats(int32_t top_k, int32_t rank, int32_t dtype);
constexpr int kMaxLatticeKpad = 4096;   // keeps the standalone lattice's LDS (4 waves' u rows) at 64 KB
hipError_t launch_lattice_walk(const SelectArgs& a, const ProjPlan& p, const WalkArgs& w, float* scores_out,
                               hipStream_t stream);

}  // namespace dflash

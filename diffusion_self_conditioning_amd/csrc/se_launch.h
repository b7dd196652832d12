// se_launch.h -- internal interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/softembed.h"

namespace se {

// ---- launch markers (se_set_launch_events) ----------------------------------------------
// Hands out the calling thread's next two armed events, for the start and the end of the
// kernel about to be launched; false (and nulls) when fewer than two remain.  The .hip
// files launch every kernel through SE_LAUNCH (se_dispatch.h), which passes them to the
// dispatch.
bool next_launch_events(hipEvent_t* start, hipEvent_t* end);
// The status of the launch just made on `stream`.
inline hipError_t launched(hipStream_t) { return hipGetLastError(); }

// ---- work decomposition of the slice contraction (pure host logic) -------------
// The output [M, N] is cut into BM x BN tiles; the contracted (vocab) axis into
// blocks of kSplitQuantum positions, and the blocks of each tile into `splits`
// contiguous ranges (split-K over the vocabulary axis, the in-GPU form of the
// partition identity on calvarado04.com, "The fix").  Every tile uses the same
// split boundaries, and logical workgroup b takes tile b % tiles, split b / tiles,
// so the workgroups that read the same probability columns run side by side.
// Both contraction kernels use the same boundaries and add their MFMA products in
// the same order, so fused and unfused results are bitwise identical.
constexpr int kBM = 256;
constexpr int kBN = 256;
#ifndef SE_WAVES
#define SE_WAVES 8          // waves per contraction workgroup: 4 (2 x 2 grid) or 8 (2 x 4)
#endif
constexpr int kGemmThreads = 64 * SE_WAVES;
constexpr int kSplitQuantum = 128;        // vocab positions per split block
constexpr int kSuperStep = 128;           // vocab positions per super-step of the contraction
constexpr int kMinBlocksPerSplit = 2;     // at least 256 vocab positions per split
constexpr int kTargetCUs = 256;           // MI355X compute units: the count used without a device
constexpr int64_t kTileFloats = (int64_t)kBM * kBN;

struct GemmPlan {
  int64_t tiles_m, tiles_n, tiles, kblocks, splits, grid;
  size_t ws_bytes;
};

// Splits fill the current device's compute units: tiles x splits ~ CU count.
int device_cu_count();
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);

// Positions one wave of the sweep holds in registers: 12 16-byte groups per lane, or 16
// (the wide form, taken only where it lets 4 waves hold a range that would take 8).
constexpr int kSweepPiece = 64 * 4 * 12;
constexpr int kSweepPieceWide = 64 * 4 * 16;

// Waves per range (1, 2, 4 or 8; 0 when the ranges are too long) and 16-byte groups per
// lane (12 or 16) of the register sweep over the split ranges of `g`.
struct SweepShape {
  int waves, groups;
};
SweepShape sweep_shape(const GemmPlan& g, int64_t K);

struct OnepassLayout {
  GemmPlan g;
  int64_t rows_pad;
  SweepShape sweep;
  size_t off_probs, off_parts, off_stats, off_arg, off_fac, total;
};

OnepassLayout onepass_layout(int64_t n_rows, int64_t K, int64_t d);

// workspace of the staged call: tiled bf16 probabilities, then the split partials
struct StagedLayout {
  GemmPlan g;
  size_t off_probs, off_parts, total;
};

StagedLayout staged_layout(int64_t n_rows, int64_t K, int64_t d);

struct GemmParams {
  const void* a;          // fused: fp32 logits; unfused: bf16 probabilities
  int64_t lda;            // elements
  int64_t a_ss;           // bytes from one super-step of a row to the next: kSuperStep *
                          // element size (row-major), or rows * kSuperStep * 2 for the
                          // super-step-tiled bf16 layout [super-step][row][kSuperStep]
  const float* lse;       // fused only: per-row log-sum-exp
  int64_t col0;           // vocab_start: column of `a` holding slice position 0
  const void* w;          // shard, row 0 = slice position 0: bf16, or e4m3 codes
  const float* wscale;    // e4m3 table only: power-of-two scale of each shard row
  bool w8_direct;         // e4m3 codes read as they are: the probabilities arrive multiplied
                          // by the row scales (staged, super-step-tiled); wscale unused
  int64_t ldw;            // elements (bytes for e4m3 codes)
  int64_t M, N, K;
  float gamma;
  float* out;
  int64_t ldo;
  float* ws;              // split partials [splits][tiles][kTileFloats]
  int tiles_n, tiles, splits, kblocks;
  // one-pass: partials are written even for one split and left for
  // launch_onepass_reduce, which reads the per-(split, row) statistics
  // stats[s * rows_pad + row] = {reference, Z, S1 (nats), max}, stat_arg = the max's
  // slice position
  bool keep_partials;
  const float* stats;
  const int32_t* stat_arg;
  int64_t rows_pad;
  // The one-read calls' range merge (merge_ranges_row), run by the contraction itself when
  // merge_rows: each workgroup of a split shorter than the longest (whose main loop ends a
  // block earlier) merges kWaves rows after its partial store, one per wave, with the
  // statistics of merge_ranges ranges at merge_stats (row stride M) and the slice's split
  // ranges from merge_r0.  Only for a launch of one wave of workgroups.
  bool merge_rows;
  int merge_ranges, merge_r0;
  float* factors;
  float* row_max;
  float* row_lse;
  float* row_entropy;
  int32_t* row_argmax;
};

// Whether the contraction of plan `g` for m rows can carry the range merge: one wave of
// workgroups (at most one per CU) and enough workgroups of short splits for 8 rows each.
bool contraction_can_merge(const GemmPlan& g, int64_t m_rows);

// The host-side checks of se_soft_embed_step (and its e4m3 form, w8) short of the workspace.
se_status check_step(const float* logits, int64_t ld_logits, int64_t n_rows, int64_t vocab,
                     int64_t vocab_start, int64_t vocab_end, const void* w_shard,
                     const float* w_scale, int64_t w_rows, int64_t ld_w, int64_t d,
                     const float* out, int64_t ld_out, const float* row_max,
                     const float* row_lse, const float* row_entropy, const int32_t* row_argmax,
                     bool w8);

hipError_t launch_row_stats(const float* logits, int64_t ld, int64_t n_rows, int vocab,
                            float* row_max, float* row_lse, float* row_entropy,
                            int32_t* row_argmax, hipStream_t stream);

// se_row_stats, and in the same pass the bf16 probabilities of slice [col0, col0 + K)
// in the super-step-tiled layout (see launch_probs_bf16_tiled); pscale (optional, 16-byte
// aligned, one power of two per slice position): the probabilities are stored times pscale[k]
hipError_t launch_row_stats_probs(const float* logits, int64_t ld, int64_t n_rows, int vocab,
                                  float* row_max, float* row_lse, float* row_entropy,
                                  int32_t* row_argmax, int64_t col0, int64_t K,
                                  uint16_t* probs, const float* pscale, hipStream_t stream);

hipError_t launch_probs_bf16(const float* logits, int64_t ld, const float* row_lse,
                             int64_t n_rows, int64_t col0, int64_t K, uint16_t* probs,
                             int64_t ldp, hipStream_t stream);

// the same probabilities of slice positions [0, K) in the super-step-tiled layout:
// position k of row i at probs[(k / kSuperStep) * n_rows * kSuperStep + i * kSuperStep +
// k % kSuperStep]
hipError_t launch_probs_bf16_tiled(const float* logits, int64_t ld, const float* row_lse,
                                   int64_t n_rows, int64_t col0, int64_t K, uint16_t* probs,
                                   hipStream_t stream);

// fused: `a` holds fp32 logits (else bf16 probabilities); w8: `w` holds e4m3 codes
// with per-row scales (else bf16)
hipError_t launch_soft_embed(const GemmParams& p, bool fused, bool w8, hipStream_t stream);

// one-pass sweep: per (row, split range) maximum, Z, S1 and argmax, and the bf16
// probabilities against the range maximum, in the super-step-tiled layout
hipError_t launch_split_sweep(const float* logits, int64_t ld, int64_t col0, int64_t K,
                              int64_t n_rows, int splits, int kblocks, uint16_t* probs,
                              float* stats, int32_t* stat_arg, int64_t rows_pad,
                              hipStream_t stream);

hipError_t launch_onepass_reduce(const GemmParams& p, float* row_max, float* row_lse,
                                 float* row_entropy, int32_t* row_argmax, int64_t col0,
                                 hipStream_t stream);

// Whole-step sweep.  The ranges of one row, in column order (r = 0 .. n_ranges - 1):
// [0, s) cut every `chunk` positions; the contraction's split ranges of the slice
// [s, e); then [e, vocab) cut at e0 + j chunk, e0 = e rounded down to a multiple of 4.
struct StepRanges {
  int64_t s, e, vocab, chunk;
  int n_pre, splits, n_post, kblocks;
};

// One read of every logit: per (row, range) maximum, first argmax (a vocabulary id),
// Z and S1 against the range maximum (stats[r * n_rows + row] = {m, Z, S1 nats, m},
// stat_arg likewise), and for the slice's split ranges the bf16 probabilities against
// the range maximum in the super-step-tiled layout.  sw.waves (1, 2, 4 or 8) wavefronts
// share a range of at most waves * 256 * sw.groups positions (sw.groups 16 only with 4
// waves).  pscale (optional, 16-byte aligned, one power of two per slice position): the
// probabilities are stored times pscale[j].
hipError_t launch_step_sweep(const float* logits, int64_t ld, int64_t n_rows,
                             const StepRanges& g, SweepShape sw, uint16_t* probs, float* stats,
                             int32_t* stat_arg, const float* pscale, hipStream_t stream);

// Merge of each row's range statistics: row max / lse / entropy / argmax, and the
// factor gamma e^(m_r - lse) of every split range r0 + j (factors[j * n_rows + row]).
hipError_t launch_merge_ranges(const float* stats, const int32_t* stat_arg, int64_t n_rows,
                               int n_ranges, int r0, int splits, float gamma, float* factors,
                               float* row_max, float* row_lse, float* row_entropy,
                               int32_t* row_argmax, hipStream_t stream);

// out = sum_s factors[s * p.rows_pad + row] * partial_s, splits in order (partials as
// the contraction left them with keep_partials).
hipError_t launch_scaled_reduce(const GemmParams& p, const float* factors, hipStream_t stream);

hipError_t launch_merge_slices(const float* outs, int64_t n_parts, int64_t part_stride,
                               int64_t n_rows, int64_t d, int64_t ld_part,
                               const float* part_max, const float* part_lse,
                               const float* part_entropy, const int32_t* part_argmax,
                               float* out, int64_t ld_out, float* row_max, float* row_lse,
                               float* row_entropy, int32_t* row_argmax, hipStream_t stream);

hipError_t launch_quantize_fp8(const uint16_t* w, int64_t ldw, int64_t rows, int64_t d,
                               uint8_t* codes, int64_t ldq, float* row_scale, hipStream_t stream);

hipError_t launch_accept_converge(const float* row_entropy, const int32_t* row_argmax,
                                  int64_t n_canvas, int len, double budget, int stable_steps,
                                  double tau, int step_limit, uint8_t* accepted,
                                  int32_t* prev_argmax, int32_t* stable_count,
                                  int32_t* step_count, uint8_t* newly, uint8_t* converged,
                                  hipStream_t stream);

hipError_t launch_reduce_parts(const float* parts, int64_t n_parts, int64_t part_stride,
                               int64_t n_rows, int64_t d, int64_t ld_part, float* out,
                               int64_t ld_out, uint16_t* out_bf16, int64_t ld_bf16,
                               hipStream_t stream);

hipError_t launch_zero_rows(float* out, int64_t ldo, int64_t M, int64_t N, hipStream_t stream);

}  // namespace se

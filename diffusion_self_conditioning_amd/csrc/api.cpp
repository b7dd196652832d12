// api.cpp -- the C ABI of libsoftembed: argument checks, work decomposition,
// launches.  Every check runs on the host before anything is enqueued, so a
// rejected call launches nothing and touches no output.  The one runtime
// condition the pages document as a failure -- a contraction whose two sides
// disagree in length (calvarado04.com, "The symptom": the [65536, 2816] shard
// against full-width probabilities) -- is SE_ERR_SLICE here.
#include "../../include/softembed.h"
#include "se_launch.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <mutex>

namespace se {

namespace {
constexpr int kMaxCachedDevices = 64;
std::once_flag cu_once[kMaxCachedDevices];
int cu_count[kMaxCachedDevices];

int query_cu_count(int dev) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1)
    return kTargetCUs;
  return n;
}
}  // namespace

// Compute units of the calling thread's current device, read once per device and
// kept for the life of the process (the library's only global state).  Without a
// usable device (a host with no GPU asking for a workspace size) the MI355X count.
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return kTargetCUs;
  }
  if (dev >= kMaxCachedDevices) return query_cu_count(dev);
  std::call_once(cu_once[dev], [dev] { cu_count[dev] = query_cu_count(dev); });
  return cu_count[dev];
}

// ---- launch markers ------------------------------------------------------------------
// Per-thread list of caller-created HIP events armed by se_set_launch_events; each kernel
// launch the thread makes afterwards takes the next two, stamped by the dispatch with the
// kernel's start and end.
namespace {
struct LaunchMarkers {
  void* const* events = nullptr;
  int32_t n = 0;
  int32_t used = 0;
};
thread_local LaunchMarkers t_markers;
}  // namespace

bool next_launch_events(hipEvent_t* start, hipEvent_t* end) {
  LaunchMarkers& m = t_markers;
  *start = *end = nullptr;
  if (m.events == nullptr || m.n - m.used < 2) return false;
  *start = static_cast<hipEvent_t>(m.events[m.used]);
  *end = static_cast<hipEvent_t>(m.events[m.used + 1]);
  m.used += 2;
  return true;
}

// The split count minimises a makespan model of the contraction:
//   waves(s) * (ceil(kblocks / s) * t_block + t_start) + s * M * N * 8 bytes / partial_rate,
// where waves(s) = ceil(tiles * s / CUs).  Each workgroup streams one 128-position block of
// its tile per t_block, a launch with more workgroups than CUs runs in waves, each wave
// pays a start-up (its first probability tile and table stages), and every split writes
// and reads back an fp32 partial of the output (the last term, only for s > 1).  The
// constants are MI355X measurements: about 4 us per block at the one-rank shape, 2 us of
// start-up, and 5 TB/s for the partials' round trip (a plain copy's rate).
constexpr double kBlockUs = 4.0, kStartUs = 2.0, kPartialBytesPerUs = 5.0e6;
constexpr int64_t kMaxSplits = 64;

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan g{};
  g.tiles_m = (M + kBM - 1) / kBM;
  g.tiles_n = (N + kBN - 1) / kBN;
  g.tiles = g.tiles_m * g.tiles_n;
  g.kblocks = (K + kSplitQuantum - 1) / kSplitQuantum;
  g.splits = 1;
  const int64_t cus = device_cu_count();
  if (g.tiles > 0 && g.kblocks > 0) {
    const int64_t cap = std::max<int64_t>(1, std::min(kMaxSplits, g.kblocks / kMinBlocksPerSplit));
    double best = 0.0;
    for (int64_t sp = 1; sp <= cap; ++sp) {
      const double waves = (double)((g.tiles * sp + cus - 1) / cus);
      const double blocks = (double)((g.kblocks + sp - 1) / sp);
      double t = waves * (blocks * kBlockUs + kStartUs);
      if (sp > 1) t += (double)sp * (double)M * (double)N * 8.0 / kPartialBytesPerUs;
      if (sp == 1 || t < best) { best = t; g.splits = sp; }
    }
  }
  g.grid = g.tiles * g.splits;
  g.ws_bytes = g.splits > 1 ? (size_t)(g.splits * g.tiles * kTileFloats) * sizeof(float) : 0;
  return g;
}

namespace {
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
// bf16 probabilities of K slice positions in the super-step-tiled layout
size_t tiled_probs_bytes(int64_t n_rows, int64_t K) {
  return (size_t)((K + kSuperStep - 1) / kSuperStep) * (size_t)n_rows * kSuperStep * 2;
}
}  // namespace

bool contraction_can_merge(const GemmPlan& g, int64_t m_rows) {
  if (g.grid > device_cu_count() || g.splits < 2) return false;
  const int64_t longest = (g.kblocks + g.splits - 1) / g.splits;
  int64_t short_splits = 0;
  for (int64_t s = 0; s < g.splits; ++s)
    short_splits += (((s + 1) * g.kblocks) / g.splits - (s * g.kblocks) / g.splits) < longest;
  return short_splits * g.tiles * (kGemmThreads / 64) >= m_rows;
}

SweepShape sweep_shape(const GemmPlan& g, int64_t K) {
  if (K <= 0) return {0, 0};
  const int64_t longest = std::min(((g.kblocks + g.splits - 1) / g.splits) * kSplitQuantum, K);
  for (int w : {1, 2, 4})
    if (longest <= kSweepPiece * (int64_t)w) return {w, 12};
  // ranges of 12,289 .. 16,384 positions (the 2,048-row whole vocabulary): 4 waves of 16
  // groups sweep them faster than 8 waves of 12 (measured 811 -> 590 us there)
  if (longest <= 4 * (int64_t)kSweepPieceWide) return {4, 16};
  if (longest <= 8 * (int64_t)kSweepPiece) return {8, 12};
  return {0, 0};
}

// Workspace of the one-pass call: tiled bf16 probabilities of the slice, the split
// partials (kept even for one split), per-(split, row) statistics, and per-(split, row)
// factors.
OnepassLayout onepass_layout(int64_t n_rows, int64_t K, int64_t d) {
  auto up = up256;
  OnepassLayout o{};
  o.g = plan_gemm(n_rows, d, K);
  o.rows_pad = o.g.tiles_m * kBM;
  o.sweep = sweep_shape(o.g, K);
  o.off_probs = 0;
  o.off_parts = up(tiled_probs_bytes(n_rows, K));
  o.off_stats = o.off_parts + up((size_t)(o.g.splits * o.g.tiles * kTileFloats) * 4);
  o.off_arg = o.off_stats + up((size_t)(o.g.splits * o.rows_pad) * 16);
  o.off_fac = o.off_arg + up((size_t)(o.g.splits * o.rows_pad) * 4);
  o.total = o.off_fac + up((size_t)(o.g.splits * o.rows_pad) * 4);
  return o;
}

// Workspace of the one-read step: tiled bf16 probabilities of the slice, the split
// partials (kept even for one split), per-(range, row) statistics and argmax, and the
// per-(split, row) factors.  sweep.waves = 0 when the slice is empty or a split range
// is longer than 8 waves hold in registers (8 * kSweepPiece positions); the call is then
// the two-pass step and the workspace is that call's.
struct StepOnepassLayout {
  GemmPlan g;
  StepRanges rg;
  SweepShape sweep;
  int n_ranges;
  size_t off_probs, off_parts, off_stats, off_arg, off_fac, total;
};

StagedLayout staged_layout(int64_t n_rows, int64_t K, int64_t d);

StepOnepassLayout step_onepass_layout(int64_t n_rows, int64_t vocab, int64_t s, int64_t e,
                                      int64_t d) {
  StepOnepassLayout o{};
  const int64_t K = e - s;
  o.g = plan_gemm(n_rows, d, K);
  o.sweep = sweep_shape(o.g, K);
  if (o.sweep.waves == 0) {
    o.total = staged_layout(n_rows, K, d).total;
    return o;
  }
  StepRanges& r = o.rg;
  r.s = s;
  r.e = e;
  r.vocab = vocab;
  r.chunk = 256 * (int64_t)o.sweep.groups * o.sweep.waves;
  r.n_pre = (int)((s + r.chunk - 1) / r.chunk);
  r.splits = (int)o.g.splits;
  r.kblocks = (int)o.g.kblocks;
  r.n_post = e < vocab ? (int)((vocab - (e & ~(int64_t)3) + r.chunk - 1) / r.chunk) : 0;
  o.n_ranges = r.n_pre + r.splits + r.n_post;
  o.off_probs = 0;
  o.off_parts = up256(tiled_probs_bytes(n_rows, K));
  o.off_stats = o.off_parts + up256((size_t)(o.g.splits * o.g.tiles * kTileFloats) * 4);
  o.off_arg = o.off_stats + up256((size_t)o.n_ranges * (size_t)n_rows * 16);
  o.off_fac = o.off_arg + up256((size_t)o.n_ranges * (size_t)n_rows * 4);
  o.total = o.off_fac + up256((size_t)o.g.splits * (size_t)n_rows * 4);
  return o;
}

StagedLayout staged_layout(int64_t n_rows, int64_t K, int64_t d) {
  StagedLayout o{};
  o.g = plan_gemm(n_rows, d, K);
  o.off_probs = 0;
  o.off_parts = up256(tiled_probs_bytes(n_rows, K));
  o.total = o.off_parts + o.g.ws_bytes;
  return o;
}

}  // namespace se

namespace {

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }
inline bool aligned4(const void* ptr) { return ((uintptr_t)ptr & 3u) == 0; }

// Rows of the helper kernels go in grid.y, which is limited to 65535.
constexpr int64_t kMaxGridY = 65535;

se_status from_hip(hipError_t e) { return e == hipSuccess ? SE_OK : SE_ERR_HIP; }

// Shape and slice checks (no pointers involved).
se_status check_slice_shape(int64_t n_rows, int64_t vocab, int64_t s, int64_t e, int64_t w_rows,
                            int64_t d, int64_t ld_w, int64_t ld_out) {
  if (n_rows < 0 || vocab < 1 || d < 1 || w_rows < 0) return SE_ERR_SHAPE;
  if (vocab > INT32_MAX || d > INT32_MAX || n_rows > INT32_MAX) return SE_ERR_SHAPE;
  if (ld_w < d || ld_out < d) return SE_ERR_SHAPE;
  if (s < 0 || e < s || e > vocab || e - s > w_rows) return SE_ERR_SLICE;
  return SE_OK;
}

se_status check_slice_layout(int64_t s, int64_t d, int64_t ld_w, int64_t ld_out, const void* w,
                             const void* out) {
  if (!aligned16(w) || !aligned16(out)) return SE_ERR_ALIGN;
  if ((s % 8) != 0 || (d % 8) != 0 || (ld_w % 8) != 0 || (ld_out % 4) != 0) return SE_ERR_ALIGN;
  return SE_OK;
}

// The e4m3 table's extra checks: codes in 16-byte pieces of 16 columns, one fp32
// scale per shard row.
se_status check_fp8_layout(int64_t d, int64_t ld_w, const float* w_scale) {
  if (!w_scale) return SE_ERR_NULL;
  if (!aligned4(w_scale) || (d % 16) != 0 || (ld_w % 16) != 0) return SE_ERR_ALIGN;
  return SE_OK;
}

se_status run_soft_embed(bool fused, const void* a, int64_t lda, const float* lse, int64_t n_rows,
                         int64_t s, int64_t e, const void* w, const float* w_scale, int64_t ldw,
                         int64_t d, float gamma, float* out, int64_t ld_out, void* ws,
                         size_t ws_bytes, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (e == s) {
    for (int64_t r0 = 0; r0 < n_rows; r0 += kMaxGridY) {
      const int64_t nr = (n_rows - r0) < kMaxGridY ? (n_rows - r0) : kMaxGridY;
      se_status rc = from_hip(se::launch_zero_rows(out + r0 * ld_out, ld_out, nr, d, st));
      if (rc != SE_OK) return rc;
    }
    return SE_OK;
  }
  const se::GemmPlan g = se::plan_gemm(n_rows, d, e - s);
  if (g.grid > INT32_MAX) return SE_ERR_SHAPE;
  // the kernels address one tile's rows of `a` and a split's rows of the shard with
  // 32-bit byte offsets
  const int64_t esz = fused ? 4 : 2;
  const int64_t wsz = w_scale ? 1 : 2;
  if ((int64_t)(se::kBM - 1) * lda * esz + (e - s) * esz > (int64_t)UINT32_MAX ||
      (e - s) * ldw * wsz > (int64_t)UINT32_MAX)
    return SE_ERR_SHAPE;
  if (ws_bytes < g.ws_bytes) return SE_ERR_WORKSPACE;
  if (g.ws_bytes > 0 && (ws == nullptr)) return SE_ERR_NULL;
  if (g.ws_bytes > 0 && !aligned16(ws)) return SE_ERR_ALIGN;
  se::GemmParams p{};
  p.a = a;
  p.lda = lda;
  p.a_ss = (int64_t)se::kSuperStep * esz;
  p.lse = lse;
  p.col0 = s;
  p.w = w;
  p.wscale = w_scale;
  p.ldw = ldw;
  p.M = n_rows;
  p.N = d;
  p.K = e - s;
  p.gamma = gamma;
  p.out = out;
  p.ldo = ld_out;
  p.ws = static_cast<float*>(ws);
  p.tiles_n = (int)g.tiles_n;
  p.tiles = (int)g.tiles;
  p.splits = (int)g.splits;
  p.kblocks = (int)g.kblocks;
  p.keep_partials = false;
  return from_hip(se::launch_soft_embed(p, fused, w_scale != nullptr, st));
}

// The contraction of super-step-tiled bf16 probabilities ([K / 128][n_rows][128], slice
// position 0 first) in the workspace of a staged call.
se_status run_staged_gemm(const se::StagedLayout& o, const uint16_t* probs, int64_t n_rows,
                          int64_t K, const void* w_shard, const float* w_scale, bool w8_direct,
                          int64_t ld_w, int64_t d, float gamma, float* out, int64_t ld_out,
                          unsigned char* ws, hipStream_t st) {
  se::GemmParams p{};
  p.w8_direct = w8_direct;           // e4m3 codes read as they are: the scales are in probs
  p.a = probs;
  p.lda = se::kSuperStep;
  p.a_ss = n_rows * se::kSuperStep * 2;
  p.col0 = 0;
  p.w = w_shard;
  p.wscale = w_scale;
  p.ldw = ld_w;
  p.M = n_rows;
  p.N = d;
  p.K = K;
  p.gamma = gamma;
  p.out = out;
  p.ldo = ld_out;
  p.ws = reinterpret_cast<float*>(ws + o.off_parts);
  p.tiles_n = (int)o.g.tiles_n;
  p.tiles = (int)o.g.tiles;
  p.splits = (int)o.g.splits;
  p.kblocks = (int)o.g.kblocks;
  return from_hip(se::launch_soft_embed(p, false, w_scale != nullptr, st));
}

}  // namespace

extern "C" {

const char* se_status_string(se_status s) {
  switch (s) {
    case SE_OK: return "SE_OK";
    case SE_ERR_NULL: return "SE_ERR_NULL: a required pointer is NULL";
    case SE_ERR_SHAPE: return "SE_ERR_SHAPE: invalid size or leading dimension";
    case SE_ERR_SLICE: return "SE_ERR_SLICE: vocab slice out of range or longer than the shard";
    case SE_ERR_ALIGN: return "SE_ERR_ALIGN: pointer, pitch, vocab_start or d misaligned";
    case SE_ERR_WORKSPACE: return "SE_ERR_WORKSPACE: workspace too small";
    case SE_ERR_HIP: return "SE_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown se_status";
}

const char* se_version(void) {
  return "libsoftembed 0.4 gfx950 (row_stats, probs_bf16, soft_embed bf16-mfma split-K, fused, accept_converge, reduce_partials, e4m3 table, one-pass, staged, step, one-read step)";
}

se_status se_set_launch_events(void* const* events, int32_t n_events) {
  if (n_events < 0) return SE_ERR_SHAPE;
  if (n_events > 0 && events == nullptr) return SE_ERR_NULL;
  se::LaunchMarkers& m = se::t_markers;
  m.events = n_events > 0 ? events : nullptr;
  m.n = n_events;
  m.used = 0;
  return SE_OK;
}

int32_t se_launch_events_used(void) { return se::t_markers.used; }

se_status se_row_stats(const float* logits, int64_t ld_logits, int64_t n_rows, int64_t vocab,
                       float* row_max, float* row_lse, float* row_entropy, int32_t* row_argmax,
                       void* stream) {
  if (n_rows < 0 || vocab < 1 || vocab > INT32_MAX || n_rows > INT32_MAX) return SE_ERR_SHAPE;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !row_max || !row_lse || !row_entropy || !row_argmax) return SE_ERR_NULL;
  if (!aligned16(logits) || (ld_logits % 4) != 0) return SE_ERR_ALIGN;
  if (!aligned4(row_max) || !aligned4(row_lse) || !aligned4(row_entropy) || !aligned4(row_argmax))
    return SE_ERR_ALIGN;
  return from_hip(se::launch_row_stats(logits, ld_logits, n_rows, (int)vocab, row_max, row_lse,
                                       row_entropy, row_argmax,
                                       static_cast<hipStream_t>(stream)));
}

se_status se_probs_bf16(const float* logits, int64_t ld_logits, const float* row_lse,
                        int64_t n_rows, int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                        uint16_t* probs, int64_t ld_probs, void* stream) {
  if (n_rows < 0 || vocab < 1 || vocab > INT32_MAX || n_rows > INT32_MAX) return SE_ERR_SHAPE;
  if (ld_logits < vocab || ld_probs < vocab) return SE_ERR_SHAPE;
  if (vocab_start < 0 || vocab_end < vocab_start || vocab_end > vocab) return SE_ERR_SLICE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !row_lse || !probs) return SE_ERR_NULL;
  if (!aligned16(logits) || !aligned16(probs) || !aligned4(row_lse)) return SE_ERR_ALIGN;
  if ((ld_logits % 4) != 0 || (ld_probs % 8) != 0 || (vocab_start % 8) != 0) return SE_ERR_ALIGN;
  const int64_t K = vocab_end - vocab_start;
  if (K == 0) return SE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < n_rows; r0 += kMaxGridY) {
    const int64_t nr = (n_rows - r0) < kMaxGridY ? (n_rows - r0) : kMaxGridY;
    se_status rc = from_hip(se::launch_probs_bf16(logits + r0 * ld_logits, ld_logits,
                                                  row_lse + r0, nr, vocab_start, K,
                                                  probs + r0 * ld_probs, ld_probs, st));
    if (rc != SE_OK) return rc;
  }
  return SE_OK;
}

size_t se_soft_embed_workspace_bytes(int64_t n_rows, int64_t vocab_start, int64_t vocab_end,
                                     int64_t d) {
  if (n_rows < 0 || d < 1 || vocab_start < 0 || vocab_end < vocab_start) return 0;
  if (n_rows > INT32_MAX || d > INT32_MAX || vocab_end > INT32_MAX) return 0;
  if (n_rows == 0 || vocab_end == vocab_start) return 0;
  return se::plan_gemm(n_rows, d, vocab_end - vocab_start).ws_bytes;
}

int64_t se_soft_embed_splits(int64_t n_rows, int64_t vocab_start, int64_t vocab_end, int64_t d) {
  if (n_rows < 1 || d < 1 || vocab_start < 0 || vocab_end <= vocab_start) return 0;
  if (n_rows > INT32_MAX || d > INT32_MAX || vocab_end > INT32_MAX) return 0;
  return se::plan_gemm(n_rows, d, vocab_end - vocab_start).splits;
}

se_status se_soft_embed(const uint16_t* probs, int64_t ld_probs, int64_t n_rows, int64_t vocab,
                        int64_t vocab_start, int64_t vocab_end, const uint16_t* w_shard,
                        int64_t w_rows, int64_t ld_w, int64_t d, float gamma, float* out,
                        int64_t ld_out, void* workspace, size_t workspace_bytes, void* stream) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_probs < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!probs || !w_shard || !out) return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_shard, out);
  if (rc != SE_OK) return rc;
  if (!aligned16(probs) || (ld_probs % 8) != 0) return SE_ERR_ALIGN;
  return run_soft_embed(false, probs, ld_probs, nullptr, n_rows, vocab_start, vocab_end, w_shard,
                        nullptr, ld_w, d, gamma, out, ld_out, workspace, workspace_bytes, stream);
}

se_status se_soft_embed_fused(const float* logits, int64_t ld_logits, const float* row_lse,
                              int64_t n_rows, int64_t vocab, int64_t vocab_start,
                              int64_t vocab_end, const uint16_t* w_shard, int64_t w_rows,
                              int64_t ld_w, int64_t d, float gamma, float* out, int64_t ld_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !row_lse || !w_shard || !out) return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_shard, out);
  if (rc != SE_OK) return rc;
  if (!aligned16(logits) || (ld_logits % 4) != 0 || !aligned4(row_lse)) return SE_ERR_ALIGN;
  return run_soft_embed(true, logits, ld_logits, row_lse, n_rows, vocab_start, vocab_end, w_shard,
                        nullptr, ld_w, d, gamma, out, ld_out, workspace, workspace_bytes, stream);
}

size_t se_soft_embed_staged_workspace_bytes(int64_t n_rows, int64_t vocab_start,
                                            int64_t vocab_end, int64_t d) {
  if (n_rows < 1 || d < 1 || vocab_start < 0 || vocab_end <= vocab_start) return 0;
  if (n_rows > INT32_MAX || d > INT32_MAX || vocab_end > INT32_MAX) return 0;
  return se::staged_layout(n_rows, vocab_end - vocab_start, d).total;
}

se_status se_soft_embed_staged(const float* logits, int64_t ld_logits, const float* row_lse,
                               int64_t n_rows, int64_t vocab, int64_t vocab_start,
                               int64_t vocab_end, const uint16_t* w_shard, int64_t w_rows,
                               int64_t ld_w, int64_t d, float gamma, float* out, int64_t ld_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !row_lse || !w_shard || !out) return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_shard, out);
  if (rc != SE_OK) return rc;
  if (!aligned16(logits) || (ld_logits % 4) != 0 || !aligned4(row_lse)) return SE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t K = vocab_end - vocab_start;
  if (K == 0) return run_soft_embed(true, logits, ld_logits, row_lse, n_rows, vocab_start,
                                    vocab_end, w_shard, nullptr, ld_w, d, gamma, out, ld_out,
                                    workspace, workspace_bytes, stream);   // writes zeros
  const se::StagedLayout o = se::staged_layout(n_rows, K, d);
  if (o.g.grid > INT32_MAX) return SE_ERR_SHAPE;
  if ((int64_t)se::tiled_probs_bytes(n_rows, K) > (int64_t)UINT32_MAX ||
      K * ld_w * 2 > (int64_t)UINT32_MAX)
    return SE_ERR_SHAPE;
  if (workspace_bytes < o.total) return SE_ERR_WORKSPACE;
  if (!workspace) return SE_ERR_NULL;
  if (!aligned16(workspace)) return SE_ERR_ALIGN;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* probs = reinterpret_cast<uint16_t*>(ws + o.off_probs);
  rc = from_hip(se::launch_probs_bf16_tiled(logits, ld_logits, row_lse, n_rows, vocab_start, K,
                                            probs, st));
  if (rc != SE_OK) return rc;
  return run_staged_gemm(o, probs, n_rows, K, w_shard, nullptr, false, ld_w, d, gamma, out, ld_out,
                         ws, st);
}

}  // extern "C"

namespace se {
// Every check of the whole step that needs neither the workspace nor the device: sizes,
// the slice, pointers, alignment and the 32-bit offset limits.  SE_OK for n_rows == 0
// once the sizes are valid.
se_status check_step(const float* logits, int64_t ld_logits, int64_t n_rows, int64_t vocab,
                     int64_t vocab_start, int64_t vocab_end, const void* w_shard,
                     const float* w_scale, int64_t w_rows, int64_t ld_w, int64_t d,
                     const float* out, int64_t ld_out, const float* row_max,
                     const float* row_lse, const float* row_entropy, const int32_t* row_argmax,
                     bool w8) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !w_shard || !out || !row_max || !row_lse || !row_entropy || !row_argmax)
    return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_shard, out);
  if (rc != SE_OK) return rc;
  if (w8) {
    rc = check_fp8_layout(d, ld_w, w_scale);
    if (rc != SE_OK) return rc;
  }
  if (!aligned16(logits) || (ld_logits % 4) != 0) return SE_ERR_ALIGN;
  if (!aligned4(row_max) || !aligned4(row_lse) || !aligned4(row_entropy) || !aligned4(row_argmax))
    return SE_ERR_ALIGN;
  const int64_t K = vocab_end - vocab_start;
  if (K == 0) return SE_OK;
  const se::StagedLayout o = se::staged_layout(n_rows, K, d);
  if (o.g.grid > INT32_MAX) return SE_ERR_SHAPE;
  if ((int64_t)se::tiled_probs_bytes(n_rows, K) > (int64_t)UINT32_MAX ||
      K * ld_w * (w8 ? 1 : 2) > (int64_t)UINT32_MAX)
    return SE_ERR_SHAPE;
  return SE_OK;
}
}  // namespace se

namespace {
// The whole step: statistics (with the slice's staged probabilities), then the
// contraction of the staged probabilities against a bf16 table, or an e4m3 table with
// per-row scales when w_scale is given.
se_status run_step(const float* logits, int64_t ld_logits, int64_t n_rows, int64_t vocab,
                   int64_t vocab_start, int64_t vocab_end, const void* w_shard,
                   const float* w_scale, int64_t w_rows, int64_t ld_w, int64_t d, float gamma,
                   float* out, int64_t ld_out, float* row_max, float* row_lse,
                   float* row_entropy, int32_t* row_argmax, void* workspace,
                   size_t workspace_bytes, void* stream, bool w8) {
  se_status rc = se::check_step(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end,
                                w_shard, w_scale, w_rows, ld_w, d, out, ld_out, row_max, row_lse,
                                row_entropy, row_argmax, w8);
  if (rc != SE_OK || n_rows == 0) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t K = vocab_end - vocab_start;
  if (K == 0) {                       // statistics, and zeros for the empty slice
    rc = from_hip(se::launch_row_stats(logits, ld_logits, n_rows, (int)vocab, row_max, row_lse,
                                       row_entropy, row_argmax, st));
    if (rc != SE_OK) return rc;
    return run_soft_embed(true, logits, ld_logits, row_lse, n_rows, vocab_start, vocab_end,
                          w_shard, w8 ? w_scale : nullptr, ld_w, d, gamma, out, ld_out,
                          workspace, workspace_bytes, stream);
  }
  const se::StagedLayout o = se::staged_layout(n_rows, K, d);
  if (workspace_bytes < o.total) return SE_ERR_WORKSPACE;
  if (!workspace) return SE_ERR_NULL;
  if (!aligned16(workspace)) return SE_ERR_ALIGN;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* probs = reinterpret_cast<uint16_t*>(ws + o.off_probs);
  // e4m3 table with 16-byte aligned scales: the statistics pass stores the probabilities times
  // their rows' scales and the contraction reads the codes as they are
  const bool direct = w8 && aligned16(w_scale);
  rc = from_hip(se::launch_row_stats_probs(logits, ld_logits, n_rows, (int)vocab, row_max,
                                           row_lse, row_entropy, row_argmax, vocab_start, K,
                                           probs, direct ? w_scale : nullptr, st));
  if (rc != SE_OK) return rc;
  return run_staged_gemm(o, probs, n_rows, K, w_shard, w8 ? w_scale : nullptr, direct, ld_w, d,
                         gamma, out, ld_out, ws, st);
}
}  // namespace

extern "C" {

se_status se_soft_embed_step(const float* logits, int64_t ld_logits, int64_t n_rows,
                             int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                             const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
                             float gamma, float* out, int64_t ld_out, float* row_max,
                             float* row_lse, float* row_entropy, int32_t* row_argmax,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return run_step(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end, w_shard, nullptr,
                  w_rows, ld_w, d, gamma, out, ld_out, row_max, row_lse, row_entropy,
                  row_argmax, workspace, workspace_bytes, stream, false);
}

se_status se_soft_embed_step_fp8(const float* logits, int64_t ld_logits, int64_t n_rows,
                                 int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                 const uint8_t* w_codes, const float* w_scale, int64_t w_rows,
                                 int64_t ld_w, int64_t d, float gamma, float* out,
                                 int64_t ld_out, float* row_max, float* row_lse,
                                 float* row_entropy, int32_t* row_argmax, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return run_step(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end, w_codes, w_scale,
                  w_rows, ld_w, d, gamma, out, ld_out, row_max, row_lse, row_entropy,
                  row_argmax, workspace, workspace_bytes, stream, true);
}

size_t se_soft_embed_step_onepass_workspace_bytes(int64_t n_rows, int64_t vocab,
                                                  int64_t vocab_start, int64_t vocab_end,
                                                  int64_t d) {
  if (n_rows < 0 || d < 1 || vocab_start < 0 || vocab_end < vocab_start || vocab < vocab_end)
    return 0;
  if (n_rows > INT32_MAX || d > INT32_MAX || vocab > INT32_MAX) return 0;
  if (n_rows == 0) return 0;
  return se::step_onepass_layout(n_rows, vocab, vocab_start, vocab_end, d).total;
}

}  // extern "C"

namespace {
// The one-read step: one sweep over the logits (per-range statistics, the slice's staged
// probabilities), the contraction with the range merge, and the factor-scaled split
// reduction.  w8: the table is e4m3 codes with per-row power-of-two scales; the sweep
// stores each probability times its row's scale and the contraction reads the codes as
// they are.  Shapes the sweep cannot take run as the two-pass step, in the same workspace.
se_status run_step_onepass(const float* logits, int64_t ld_logits, int64_t n_rows,
                           int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                           const void* w_shard, const float* w_scale, int64_t w_rows,
                           int64_t ld_w, int64_t d, float gamma, float* out, int64_t ld_out,
                           float* row_max, float* row_lse, float* row_entropy,
                           int32_t* row_argmax, void* workspace, size_t workspace_bytes,
                           void* stream, bool w8) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  // the sweep reads 4 scales at a time; the same rule whichever pass runs
  if (w8 && w_scale && !aligned16(w_scale)) return SE_ERR_ALIGN;
  const se::StepOnepassLayout o =
      se::step_onepass_layout(n_rows, vocab, vocab_start, vocab_end, d);
  if (o.sweep.waves == 0)          // empty slice, or split ranges too long: two passes
    return run_step(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end, w_shard,
                    w8 ? w_scale : nullptr, w_rows, ld_w, d, gamma, out, ld_out, row_max,
                    row_lse, row_entropy, row_argmax, workspace, workspace_bytes, stream, w8);
  if (!logits || !w_shard || !out || !row_max || !row_lse || !row_entropy || !row_argmax)
    return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_shard, out);
  if (rc != SE_OK) return rc;
  if (w8) {
    rc = check_fp8_layout(d, ld_w, w_scale);
    if (rc != SE_OK) return rc;
  }
  if (!aligned16(logits) || (ld_logits % 4) != 0) return SE_ERR_ALIGN;
  if (!aligned4(row_max) || !aligned4(row_lse) || !aligned4(row_entropy) || !aligned4(row_argmax))
    return SE_ERR_ALIGN;
  const int64_t K = vocab_end - vocab_start;
  if (o.g.grid > INT32_MAX || n_rows * o.n_ranges > INT32_MAX) return SE_ERR_SHAPE;
  if ((int64_t)se::tiled_probs_bytes(n_rows, K) > (int64_t)UINT32_MAX ||
      K * ld_w * (w8 ? 1 : 2) > (int64_t)UINT32_MAX)
    return SE_ERR_SHAPE;
  if (workspace_bytes < o.total) return SE_ERR_WORKSPACE;
  if (!workspace) return SE_ERR_NULL;
  if (!aligned16(workspace)) return SE_ERR_ALIGN;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* probs = reinterpret_cast<uint16_t*>(ws + o.off_probs);
  float* stats = reinterpret_cast<float*>(ws + o.off_stats);
  int32_t* stat_arg = reinterpret_cast<int32_t*>(ws + o.off_arg);
  float* factors = reinterpret_cast<float*>(ws + o.off_fac);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = from_hip(se::launch_step_sweep(logits, ld_logits, n_rows, o.rg, o.sweep, probs, stats,
                                      stat_arg, w8 ? w_scale : nullptr, st));
  if (rc != SE_OK) return rc;
  se::GemmParams p{};
  p.a = probs;                       // super-step-tiled: [K / 128][n_rows][128]
  p.lda = se::kSuperStep;
  p.a_ss = n_rows * se::kSuperStep * 2;
  p.col0 = 0;
  p.w = w_shard;
  p.wscale = w8 ? w_scale : nullptr;
  p.w8_direct = w8;                  // the scales are in the probabilities
  p.ldw = ld_w;
  p.M = n_rows;
  p.N = d;
  p.K = K;
  p.gamma = gamma;
  p.out = out;
  p.ldo = ld_out;
  p.ws = reinterpret_cast<float*>(ws + o.off_parts);
  p.tiles_n = (int)o.g.tiles_n;
  p.tiles = (int)o.g.tiles;
  p.splits = (int)o.g.splits;
  p.kblocks = (int)o.g.kblocks;
  p.keep_partials = true;
  p.rows_pad = n_rows;
  // the range merge rides in the contraction's short-split workgroups when it can
  p.merge_rows = se::contraction_can_merge(o.g, n_rows);
  p.stats = stats;
  p.stat_arg = stat_arg;
  p.merge_ranges = o.n_ranges;
  p.merge_r0 = o.rg.n_pre;
  p.factors = factors;
  p.row_max = row_max;
  p.row_lse = row_lse;
  p.row_entropy = row_entropy;
  p.row_argmax = row_argmax;
  rc = from_hip(se::launch_soft_embed(p, false, w8, st));
  if (rc != SE_OK) return rc;
  if (!p.merge_rows) {
    rc = from_hip(se::launch_merge_ranges(stats, stat_arg, n_rows, o.n_ranges, o.rg.n_pre,
                                          (int)o.g.splits, gamma, factors, row_max, row_lse,
                                          row_entropy, row_argmax, st));
    if (rc != SE_OK) return rc;
  }
  return from_hip(se::launch_scaled_reduce(p, factors, st));
}
}  // namespace

extern "C" {

se_status se_soft_embed_step_onepass(const float* logits, int64_t ld_logits, int64_t n_rows,
                                     int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                     const uint16_t* w_shard, int64_t w_rows, int64_t ld_w,
                                     int64_t d, float gamma, float* out, int64_t ld_out,
                                     float* row_max, float* row_lse, float* row_entropy,
                                     int32_t* row_argmax, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return run_step_onepass(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end, w_shard,
                          nullptr, w_rows, ld_w, d, gamma, out, ld_out, row_max, row_lse,
                          row_entropy, row_argmax, workspace, workspace_bytes, stream, false);
}

se_status se_soft_embed_step_onepass_fp8(const float* logits, int64_t ld_logits,
                                         int64_t n_rows, int64_t vocab, int64_t vocab_start,
                                         int64_t vocab_end, const uint8_t* w_codes,
                                         const float* w_scale, int64_t w_rows, int64_t ld_w,
                                         int64_t d, float gamma, float* out, int64_t ld_out,
                                         float* row_max, float* row_lse, float* row_entropy,
                                         int32_t* row_argmax, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return run_step_onepass(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end, w_codes,
                          w_scale, w_rows, ld_w, d, gamma, out, ld_out, row_max, row_lse,
                          row_entropy, row_argmax, workspace, workspace_bytes, stream, true);
}

se_status se_quantize_table_fp8(const uint16_t* w, int64_t ld_w, int64_t rows, int64_t d,
                                uint8_t* codes, int64_t ld_codes, float* row_scale,
                                void* stream) {
  if (rows < 0 || d < 1 || d > INT32_MAX || ld_w < d || ld_codes < d) return SE_ERR_SHAPE;
  if (rows / 4 >= (int64_t)INT32_MAX) return SE_ERR_SHAPE;
  if (rows == 0) return SE_OK;
  if (!w || !codes || !row_scale) return SE_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned4(row_scale)) return SE_ERR_ALIGN;
  if ((d % 16) != 0 || (ld_w % 8) != 0 || (ld_codes % 16) != 0) return SE_ERR_ALIGN;
  return from_hip(se::launch_quantize_fp8(w, ld_w, rows, d, codes, ld_codes, row_scale,
                                          static_cast<hipStream_t>(stream)));
}

se_status se_soft_embed_fp8(const uint16_t* probs, int64_t ld_probs, int64_t n_rows, int64_t vocab,
                            int64_t vocab_start, int64_t vocab_end, const uint8_t* w_codes,
                            const float* w_scale, int64_t w_rows, int64_t ld_w, int64_t d,
                            float gamma, float* out, int64_t ld_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_probs < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!probs || !w_codes || !out) return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_codes, out);
  if (rc != SE_OK) return rc;
  rc = check_fp8_layout(d, ld_w, w_scale);
  if (rc != SE_OK) return rc;
  if (!aligned16(probs) || (ld_probs % 8) != 0) return SE_ERR_ALIGN;
  return run_soft_embed(false, probs, ld_probs, nullptr, n_rows, vocab_start, vocab_end, w_codes,
                        w_scale, ld_w, d, gamma, out, ld_out, workspace, workspace_bytes, stream);
}

se_status se_soft_embed_fp8_fused(const float* logits, int64_t ld_logits, const float* row_lse,
                                  int64_t n_rows, int64_t vocab, int64_t vocab_start,
                                  int64_t vocab_end, const uint8_t* w_codes, const float* w_scale,
                                  int64_t w_rows, int64_t ld_w, int64_t d, float gamma,
                                  float* out, int64_t ld_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !row_lse || !w_codes || !out) return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_codes, out);
  if (rc != SE_OK) return rc;
  rc = check_fp8_layout(d, ld_w, w_scale);
  if (rc != SE_OK) return rc;
  if (!aligned16(logits) || (ld_logits % 4) != 0 || !aligned4(row_lse)) return SE_ERR_ALIGN;
  return run_soft_embed(true, logits, ld_logits, row_lse, n_rows, vocab_start, vocab_end, w_codes,
                        w_scale, ld_w, d, gamma, out, ld_out, workspace, workspace_bytes, stream);
}

size_t se_soft_embed_onepass_workspace_bytes(int64_t n_rows, int64_t vocab_start,
                                             int64_t vocab_end, int64_t d) {
  if (n_rows < 1 || d < 1 || vocab_start < 0 || vocab_end <= vocab_start) return 0;
  if (n_rows > INT32_MAX || d > INT32_MAX || vocab_end > INT32_MAX) return 0;
  return se::onepass_layout(n_rows, vocab_end - vocab_start, d).total;
}

se_status se_soft_embed_onepass(const float* logits, int64_t ld_logits, int64_t n_rows,
                                int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
                                float gamma, float* out, int64_t ld_out, float* row_max,
                                float* row_lse, float* row_entropy, int32_t* row_argmax,
                                void* workspace, size_t workspace_bytes, void* stream) {
  se_status rc = check_slice_shape(n_rows, vocab, vocab_start, vocab_end, w_rows, d, ld_w, ld_out);
  if (rc != SE_OK) return rc;
  if (ld_logits < vocab) return SE_ERR_SHAPE;
  if (vocab_end == vocab_start) return SE_ERR_SLICE;   // a softmax over no positions
  if (n_rows == 0) return SE_OK;   // nothing to read or write: buffers may be NULL
  if (!logits || !w_shard || !out || !row_max || !row_lse || !row_entropy || !row_argmax)
    return SE_ERR_NULL;
  rc = check_slice_layout(vocab_start, d, ld_w, ld_out, w_shard, out);
  if (rc != SE_OK) return rc;
  if (!aligned16(logits) || (ld_logits % 4) != 0) return SE_ERR_ALIGN;
  if (!aligned4(row_max) || !aligned4(row_lse) || !aligned4(row_entropy) || !aligned4(row_argmax))
    return SE_ERR_ALIGN;
  const int64_t K = vocab_end - vocab_start;
  const se::OnepassLayout o = se::onepass_layout(n_rows, K, d);
  if (o.g.grid > INT32_MAX || n_rows * o.g.splits > INT32_MAX) return SE_ERR_SHAPE;
  // 32-bit byte offsets: a tile's rows of the probabilities, a split's table rows, and a
  // row's range of logits in the sweep
  if ((int64_t)se::tiled_probs_bytes(n_rows, K) > (int64_t)UINT32_MAX ||
      K * ld_w * 2 > (int64_t)UINT32_MAX || K * 4 > (int64_t)UINT32_MAX)
    return SE_ERR_SHAPE;
  if (workspace_bytes < o.total) return SE_ERR_WORKSPACE;
  if (!workspace) return SE_ERR_NULL;
  if (!aligned16(workspace)) return SE_ERR_ALIGN;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* probs = reinterpret_cast<uint16_t*>(ws + o.off_probs);
  float* stats = reinterpret_cast<float*>(ws + o.off_stats);
  int32_t* stat_arg = reinterpret_cast<int32_t*>(ws + o.off_arg);
  float* factors = reinterpret_cast<float*>(ws + o.off_fac);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // split ranges that fit the wave-per-range sweep: that sweep (its ranges are exactly
  // the splits), the range merge and the factor-scaled split reduction; longer ranges:
  // the workgroup-per-range sweep and the one-pass reduction
  se::StepRanges rg{};
  rg.s = vocab_start;
  rg.e = vocab_end;
  rg.vocab = vocab_end;
  rg.chunk = 256 * (int64_t)o.sweep.groups * o.sweep.waves;
  rg.splits = (int)o.g.splits;
  rg.kblocks = (int)o.g.kblocks;
  if (o.sweep.waves > 0)
    rc = from_hip(se::launch_step_sweep(logits, ld_logits, n_rows, rg, o.sweep, probs, stats,
                                        stat_arg, nullptr, st));
  else
    rc = from_hip(se::launch_split_sweep(logits, ld_logits, vocab_start, K, n_rows,
                                         (int)o.g.splits, (int)o.g.kblocks, probs, stats,
                                         stat_arg, o.rows_pad, st));
  if (rc != SE_OK) return rc;
  se::GemmParams p{};
  p.a = probs;                       // super-step-tiled: [K / 128][n_rows][128]
  p.lda = se::kSuperStep;
  p.a_ss = n_rows * se::kSuperStep * 2;
  p.col0 = 0;
  p.w = w_shard;
  p.ldw = ld_w;
  p.M = n_rows;
  p.N = d;
  p.K = K;
  p.gamma = gamma;
  p.out = out;
  p.ldo = ld_out;
  p.ws = reinterpret_cast<float*>(ws + o.off_parts);
  p.tiles_n = (int)o.g.tiles_n;
  p.tiles = (int)o.g.tiles;
  p.splits = (int)o.g.splits;
  p.kblocks = (int)o.g.kblocks;
  p.keep_partials = true;
  p.stats = stats;
  p.stat_arg = stat_arg;
  p.rows_pad = o.rows_pad;
  if (o.sweep.waves == 0) {
    rc = from_hip(se::launch_soft_embed(p, false, false, st));
    if (rc != SE_OK) return rc;
    return from_hip(se::launch_onepass_reduce(p, row_max, row_lse, row_entropy, row_argmax,
                                              vocab_start, st));
  }
  // the sweep wrote statistics and factors with row stride n_rows; the range merge rides in
  // the contraction's short-split workgroups when it can
  p.rows_pad = n_rows;
  p.merge_rows = se::contraction_can_merge(o.g, n_rows);
  p.merge_ranges = (int)o.g.splits;
  p.merge_r0 = 0;
  p.factors = factors;
  p.row_max = row_max;
  p.row_lse = row_lse;
  p.row_entropy = row_entropy;
  p.row_argmax = row_argmax;
  rc = from_hip(se::launch_soft_embed(p, false, false, st));
  if (rc != SE_OK) return rc;
  if (!p.merge_rows) {
    rc = from_hip(se::launch_merge_ranges(stats, stat_arg, n_rows, (int)o.g.splits, 0,
                                          (int)o.g.splits, gamma, factors, row_max, row_lse,
                                          row_entropy, row_argmax, st));
    if (rc != SE_OK) return rc;
  }
  return from_hip(se::launch_scaled_reduce(p, factors, st));
}

se_status se_merge_slices(const float* outs, int64_t n_parts, int64_t part_stride,
                          int64_t n_rows, int64_t d, int64_t ld_part, const float* part_max,
                          const float* part_lse, const float* part_entropy,
                          const int32_t* part_argmax, float* out, int64_t ld_out,
                          float* row_max, float* row_lse, float* row_entropy,
                          int32_t* row_argmax, void* stream) {
  if (n_parts < 1 || n_parts > INT32_MAX || n_rows < 0 || d < 1 || ld_part < d || ld_out < d)
    return SE_ERR_SHAPE;
  if (n_rows > kMaxGridY || d > INT32_MAX) return SE_ERR_SHAPE;
  if (n_parts > 1 && part_stride < n_rows * ld_part) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;
  if (!outs || !part_max || !part_lse || !part_entropy || !part_argmax || !out || !row_max ||
      !row_lse || !row_entropy || !row_argmax)
    return SE_ERR_NULL;
  if ((d % 4) != 0 || (ld_part % 4) != 0 || (ld_out % 4) != 0 ||
      (n_parts > 1 && (part_stride % 4) != 0))
    return SE_ERR_ALIGN;
  if (!aligned16(outs) || !aligned16(out)) return SE_ERR_ALIGN;
  if (!aligned4(part_max) || !aligned4(part_lse) || !aligned4(part_entropy) ||
      !aligned4(part_argmax) || !aligned4(row_max) || !aligned4(row_lse) ||
      !aligned4(row_entropy) || !aligned4(row_argmax))
    return SE_ERR_ALIGN;
  return from_hip(se::launch_merge_slices(outs, n_parts, part_stride, n_rows, d, ld_part,
                                          part_max, part_lse, part_entropy, part_argmax, out,
                                          ld_out, row_max, row_lse, row_entropy, row_argmax,
                                          static_cast<hipStream_t>(stream)));
}

se_status se_accept_converge(const float* row_entropy, const int32_t* row_argmax,
                             int64_t n_canvas, int64_t canvas_len, double entropy_budget,
                             int32_t stable_steps, double entropy_tau, int32_t step_limit,
                             uint8_t* accepted, int32_t* prev_argmax, int32_t* stable_count,
                             int32_t* step_count, uint8_t* newly_accepted, uint8_t* converged,
                             void* stream) {
  if (n_canvas < 0 || n_canvas > INT32_MAX || canvas_len < 1 || canvas_len > 1024) return SE_ERR_SHAPE;
  if (stable_steps < 1 || step_limit < 1) return SE_ERR_SHAPE;
  if (entropy_budget != entropy_budget || entropy_tau != entropy_tau) return SE_ERR_SHAPE;
  if (n_canvas == 0) return SE_OK;
  if (!row_entropy || !row_argmax || !accepted || !prev_argmax || !stable_count || !step_count ||
      !newly_accepted || !converged)
    return SE_ERR_NULL;
  if (!aligned4(row_entropy) || !aligned4(row_argmax) || !aligned4(prev_argmax) ||
      !aligned4(stable_count) || !aligned4(step_count))
    return SE_ERR_ALIGN;
  return from_hip(se::launch_accept_converge(row_entropy, row_argmax, n_canvas, (int)canvas_len,
                                             entropy_budget, stable_steps, entropy_tau,
                                             step_limit, accepted, prev_argmax, stable_count,
                                             step_count, newly_accepted, converged,
                                             static_cast<hipStream_t>(stream)));
}

se_status se_reduce_partials(const float* parts, int64_t n_parts, int64_t part_stride,
                             int64_t n_rows, int64_t d, int64_t ld_part, float* out,
                             int64_t ld_out, uint16_t* out_bf16, int64_t ld_bf16, void* stream) {
  if (n_parts < 1 || n_rows < 0 || d < 1 || ld_part < d) return SE_ERR_SHAPE;
  if (n_rows > kMaxGridY || d > INT32_MAX) return SE_ERR_SHAPE;
  if (out && ld_out < d) return SE_ERR_SHAPE;
  if (out_bf16 && ld_bf16 < d) return SE_ERR_SHAPE;
  if (n_parts > 1 && part_stride < n_rows * ld_part) return SE_ERR_SHAPE;
  if (n_rows == 0) return SE_OK;
  if (!parts || (!out && !out_bf16)) return SE_ERR_NULL;
  if ((d % 4) != 0 || (ld_part % 4) != 0 || (n_parts > 1 && (part_stride % 4) != 0))
    return SE_ERR_ALIGN;
  if (!aligned16(parts) || (out && (!aligned16(out) || (ld_out % 4) != 0))) return SE_ERR_ALIGN;
  if (out_bf16 && ((((uintptr_t)out_bf16) & 7u) != 0 || (ld_bf16 % 4) != 0)) return SE_ERR_ALIGN;
  return from_hip(se::launch_reduce_parts(parts, n_parts, part_stride, n_rows, d, ld_part, out,
                                          ld_out, out_bf16, ld_bf16,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"

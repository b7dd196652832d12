// onepass.hip -- the single sweep over the logits of the one-pass soft embedding.
//
// The expected token embedding needs softmax(logits) (calvarado04.com, "Where the
// shapes stop agreeing"), and the sampler needs each row's max, log-sum-exp, entropy
// and argmax (agentlenshq overview of DiffusionGemma in vLLM, sampling loop).  The
// two-pass path reads the full-width logits once for those statistics and again for
// the probabilities.  Here the vocabulary slice is cut into the contraction's split-K
// ranges, and each range is normalised against its own maximum m_s:
//     P[i, k] = bf16_rne(e^(l[i, k] - m_s)),  Z_s = sum e^(l - m_s),
//     S1_s = sum e^(l - m_s) (l - m_s),  argmax_s = first position of m_s,
// so the probabilities can be written before any other range has been seen.  The
// contraction of P runs unchanged per split, and the split reduction rescales every
// split by e^(m_s - M), M = max_s m_s, and divides by Z = sum_s e^(m_s - M) Z_s: the
// merge rule of the partition identity ("The fix") written for softmax numerators.
//
// One workgroup per (row, split range), for split ranges longer than the register sweep
// below holds: a first pass reads the range and finds its maximum and first position; a
// second pass reads it again, forms the probabilities, writes them as bf16 and sums Z_s
// and S1_s in fp32.
#include <type_traits>

#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kSweepThreads = 512;                  // one workgroup per (row, split range)
constexpr int kSweepWaves = kSweepThreads / 64;

// Pass 1 reads the range (16-byte buffer loads, eight in flight per lane) and finds the
// first maximum; pass 2 reads it again, forms the probabilities against that maximum,
// writes them as bf16 and sums Z and S1.  Cross-wave reductions go through a small LDS
// array in wave order, so the sums are independent of scheduling.
__global__ void __launch_bounds__(kSweepThreads)
split_sweep_kernel(const float* __restrict__ logits, int64_t ld, int64_t col0, int64_t K,
                   int64_t n_rows, int splits, int kblocks, uint16_t* __restrict__ probs,
                   float4* __restrict__ stats, int32_t* __restrict__ stat_arg,
                   int64_t rows_pad) {
  __shared__ float red_v[kSweepWaves], red_w[kSweepWaves];
  __shared__ int red_i[kSweepWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x % n_rows;
  const int s = (int)(blockIdx.x / n_rows);
  // the contraction's split boundaries (positions of the slice)
  const int64_t k_lo = (((int64_t)s * kblocks) / splits) * kSplitQuantum;
  const int64_t k_hi = min((((int64_t)(s + 1) * kblocks) / splits) * kSplitQuantum, K);
  const int n = (int)(k_hi - k_lo);
  const int n4 = n / 4;                               // whole 16-byte groups
  const float* __restrict__ x = logits + row * ld + col0 + k_lo;
  // probabilities in the super-step-tiled layout: range position j (k_lo + j, k_lo a
  // multiple of kSuperStep) of this row at blk[(j / kSuperStep) * n_rows * kSuperStep +
  // j % kSuperStep]
  uint16_t* __restrict__ blk = probs + (k_lo / kSuperStep) * n_rows * kSuperStep + row * kSuperStep;
  auto pidx = [&](int j) -> int64_t {
    return (int64_t)(j / kSuperStep) * n_rows * kSuperStep + j % kSuperStep;
  };

  // pass 1
  float mv = -INFINITY;
  int mi = 0;
  auto max4 = [&](const float4& v, int k) {
    argmax_step(mv, mi, v.x, k);
    argmax_step(mv, mi, v.y, k + 1);
    argmax_step(mv, mi, v.z, k + 2);
    argmax_step(mv, mi, v.w, k + 3);
  };
  // eight 16-byte loads in flight per lane; the buffer resource bounds them to the range
  // (out-of-range lanes read zeros, which the mask below discards)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)n4 * 16u);
  for (int base = 0; base < n4; base += 8 * kSweepThreads) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = buffer_load_f4(xr, (uint32_t)(base + u * kSweepThreads + tid) * 16u, 0u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = base + u * kSweepThreads + tid;
      if (g < n4) max4(v[u], 4 * g);
    }
  }
  for (int j = 4 * n4 + tid; j < n; j += kSweepThreads) argmax_step(mv, mi, x[j], j);
  wave_argmax(mv, mi);
  if (lane == 0) { red_v[wave] = mv; red_i[wave] = mi; }
  __syncthreads();
  mv = red_v[0];
  mi = red_i[0];
  for (int w = 1; w < kSweepWaves; ++w) argmax_step(mv, mi, red_v[w], red_i[w]);
  const float nl = neg_lse_log2(mv);

  // pass 2
  float z = 0.f, s1 = 0.f;
  for (int g = tid; g < n4; g += kSweepThreads) {
    const float4 v = reinterpret_cast<const float4*>(x)[g];
    const float t0 = __builtin_fmaf(v.x, kLog2e, nl), t1 = __builtin_fmaf(v.y, kLog2e, nl);
    const float t2 = __builtin_fmaf(v.z, kLog2e, nl), t3 = __builtin_fmaf(v.w, kLog2e, nl);
    const float q0 = exp2_hw(t0), q1 = exp2_hw(t1), q2 = exp2_hw(t2), q3 = exp2_hw(t3);
    z += (q0 + q1) + (q2 + q3);
    s1 = __builtin_fmaf(q0, t0, __builtin_fmaf(q1, t1, __builtin_fmaf(q2, t2, __builtin_fmaf(q3, t3, s1))));
    store_stream_u2(blk + pidx(4 * g), pack_bf16x2(q0, q1), pack_bf16x2(q2, q3));
  }
  for (int j = 4 * n4 + tid; j < n; j += kSweepThreads) {
    const float t = __builtin_fmaf(x[j], kLog2e, nl);
    const float q = exp2_hw(t);
    z += q;
    s1 = __builtin_fmaf(q, t, s1);
    store_stream_u16(blk + pidx(j), __builtin_bit_cast(uint16_t, (__bf16)q));
  }
  z = wave_sum(z);
  s1 = wave_sum(s1);
  __syncthreads();                                    // red_v / red_i reads are done
  if (lane == 0) { red_v[wave] = z; red_w[wave] = s1; }
  __syncthreads();
  if (tid == 0) {
    float zt = 0.f, st = 0.f;
    for (int w = 0; w < kSweepWaves; ++w) { zt += red_v[w]; st += red_w[w]; }
    stats[(int64_t)s * rows_pad + row] = make_float4(mv, zt, st * kLn2, mv);
    stat_arg[(int64_t)s * rows_pad + row] = (int32_t)(k_lo + mi);
  }
}

// ---- the whole step in one read -------------------------------------------------------
// The statistics of a row need every logit of it; the probabilities of the slice need
// the row's lse.  Cutting the whole row into ranges and normalising each slice range
// against its own maximum (as in the one-pass call) lets one sweep produce both: the
// range statistics merge into the row's, and the split reduction rescales split r by
// e^(m_r - lse).  One wavefront owns one (row, range): its values stay in registers
// between the maximum and the sums, and its reductions are the fixed DPP butterflies of
// a single wave, so no workgroup barrier is involved.

// A workgroup holds 256 threads (four (row, range) items of 1 wave, two of 2 waves, one of
// 4), or 512 threads for one item of 8 waves.
constexpr int sweep_threads(int W) { return W <= 4 ? 256 : 64 * W; }
#ifndef SE_SWEEP_LOAD
#define SE_SWEEP_LOAD buffer_load_f4_nt               // the logits are read once
#endif

__device__ __forceinline__ void step_range(const StepRanges& g, int r, int64_t& c0,
                                           int64_t& c1) {
  if (r < g.n_pre) {
    c0 = (int64_t)r * g.chunk;
    c1 = min(c0 + g.chunk, g.s);
    return;
  }
  r -= g.n_pre;
  if (r < g.splits) {
    const int64_t K = g.e - g.s;
    c0 = g.s + (((int64_t)r * g.kblocks) / g.splits) * kSplitQuantum;
    c1 = g.s + min((((int64_t)(r + 1) * g.kblocks) / g.splits) * kSplitQuantum, K);
    return;
  }
  r -= g.splits;
  const int64_t e0 = g.e & ~(int64_t)3;
  c0 = max(g.e, e0 + (int64_t)r * g.chunk);
  c1 = min(g.vocab, e0 + (int64_t)(r + 1) * g.chunk);
}

// W wavefronts (1, 2, 4 or 8) of a workgroup share one (row, range); wave k of the group
// takes the k-th of W near-equal, 4-aligned pieces, at most 64 NF4 positions (NF4 = 12 or
// 16 16-byte groups per lane, held in registers between the maximum and the sums).  The
// group combines its maxima and then its sums through LDS in wave order.
static_assert(kSweepPiece == 64 * 4 * 12 && kSweepPieceWide == 64 * 4 * 16, "sweep pieces");

// SCALED: slice position j's probability is stored times pscale[j] (a power of two, so the
// bf16 value is the unscaled one times pscale[j] exactly); the statistics stay unscaled.
template <int W, int NF4, bool SCALED>
__global__ void __launch_bounds__(sweep_threads(W))
step_sweep_kernel(const float* __restrict__ logits, int64_t ld, int64_t n_rows, StepRanges g,
                  int n_ranges, uint16_t* __restrict__ probs, float4* __restrict__ stats,
                  int32_t* __restrict__ stat_arg, const float* __restrict__ pscale) {
  constexpr int kWaves = sweep_threads(W) / 64;
  __shared__ float grp_v[kWaves], grp_z[kWaves], grp_s[kWaves];
  __shared__ int grp_i[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k = wave % W;
  const int64_t item = (int64_t)blockIdx.x * (kWaves / W) + wave / W;
  const bool active = item < n_rows * n_ranges;
  if (W == 1 && !active) return;                      // whole wavefronts; no barrier below
  // Unscaled: items in range-major order, so that workgroups launched together take one
  // range of neighbouring rows, whose staged probabilities are neighbouring 256-byte runs of
  // one super-step (measured: sweep 78 -> 76 us at the whole vocabulary; row-major order
  // spreads the stores over all super-steps).  Scaled: row-major order, so that workgroups
  // launched together read the scales of different ranges (all reading one range's scales
  // at once, the sweep measured 86 -> 92 us).
  const int64_t row = active ? (SCALED ? item / n_ranges : item % n_rows) : 0;
  const int r = active ? (int)(SCALED ? item % n_ranges : item / n_rows) : 0;
  int64_t c0 = 0, c1 = 0;
  if (active) step_range(g, r, c0, c1);
  const bool in_slice = r >= g.n_pre && r < g.n_pre + g.splits;
  // this wave's piece [p0, p1) of the range
  const int64_t piece = (((c1 - c0) + W - 1) / W + 3) & ~(int64_t)3;
  const int64_t p0 = min(c0 + k * piece, c1), p1 = min(p0 + piece, c1);
  const float* __restrict__ x = logits + row * ld;
  // 16-byte groups [a0, a1) (row starts are 16-byte aligned); at most 3 positions
  // before a0 and 3 after a1, one per lane (lanes 0-2 and 4-6)
  const int64_t a0 = min((p0 + 3) & ~(int64_t)3, p1);
  const int64_t a1 = max(p1 & ~(int64_t)3, a0);
  const int ng = (int)((a1 - a0) >> 2);
  const int base = (int)(a0 - c0);                      // range position of group 0
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + a0, (uint32_t)ng * 16u);
  float4 v[NF4];
#pragma unroll
  for (int u = 0; u < NF4; ++u) v[u] = SE_SWEEP_LOAD(xr, (uint32_t)(u * 64 + lane) * 16u, 0u);
  int rs = -1;                                          // range position of the scalar
  if (lane < (int)(a0 - p0)) rs = (int)(p0 - c0) + lane;
  else if (lane >= 4 && lane < 4 + (int)(p1 - a1)) rs = (int)(a1 - c0) + lane - 4;
  const float xs = rs >= 0 ? x[c0 + rs] : 0.f;
  // the scales of the same positions (slice positions js + base + 4 gi ..; 16-byte aligned),
  // each loaded where it is used (held for the whole loop they would cost occupancy)
  float ss = 1.f;
  __amdgpu_buffer_rsrc_t sr = make_rsrc(pscale, 0u);
  if constexpr (SCALED) {
    if (active && in_slice) {
      sr = make_rsrc(pscale + (c0 - g.s) + base, (uint32_t)ng * 16u);
      if (rs >= 0) ss = pscale[c0 - g.s + rs];
    }
  }

  float mv = -INFINITY;
  int mi = INT_MAX;
#pragma unroll
  for (int u = 0; u < NF4; ++u) {
    const int gi = u * 64 + lane;
    if (gi < ng) {
      const int kk = base + 4 * gi;
      argmax_step(mv, mi, v[u].x, kk);
      argmax_step(mv, mi, v[u].y, kk + 1);
      argmax_step(mv, mi, v[u].z, kk + 2);
      argmax_step(mv, mi, v[u].w, kk + 3);
    }
  }
  if (rs >= 0) argmax_step(mv, mi, xs, rs);
  wave_argmax(mv, mi);
  if constexpr (W > 1) {
    if (lane == 0) { grp_v[wave] = mv; grp_i[wave] = mi; }
    __syncthreads();
    const int w0 = wave - k;
    mv = grp_v[w0];
    mi = grp_i[w0];
    for (int q = 1; q < W; ++q) argmax_step(mv, mi, grp_v[w0 + q], grp_i[w0 + q]);
  }
  const float nl = neg_lse_log2(mv);

  // probabilities of slice position j of this row at
  // probs[(j / kSuperStep) * n_rows * kSuperStep + row * kSuperStep + j % kSuperStep]
  uint16_t* __restrict__ prow = probs + row * kSuperStep;
  const int64_t js = c0 - g.s;                          // slice position of range position 0
  auto tiled = [&](int64_t j) -> int64_t {
    return (j / kSuperStep) * n_rows * kSuperStep + j % kSuperStep;
  };
  float z = 0.f, s1 = 0.f;
#pragma unroll
  for (int u = 0; u < NF4; ++u) {
    const int gi = u * 64 + lane;
    if (gi < ng) {
      const float t0 = __builtin_fmaf(v[u].x, kLog2e, nl), t1 = __builtin_fmaf(v[u].y, kLog2e, nl);
      const float t2 = __builtin_fmaf(v[u].z, kLog2e, nl), t3 = __builtin_fmaf(v[u].w, kLog2e, nl);
      const float q0 = exp2_hw(t0), q1 = exp2_hw(t1), q2 = exp2_hw(t2), q3 = exp2_hw(t3);
      z += (q0 + q1) + (q2 + q3);
      s1 = __builtin_fmaf(q0, t0, __builtin_fmaf(q1, t1, __builtin_fmaf(q2, t2, __builtin_fmaf(q3, t3, s1))));
      if (active && in_slice) {                         // 4 positions in one super-step
        if constexpr (SCALED) {
          const float4 sc = buffer_load_f4(sr, (uint32_t)gi * 16u, 0u);
          store_stream_u2(prow + tiled(js + base + 4 * gi), pack_bf16x2(q0 * sc.x, q1 * sc.y),
                          pack_bf16x2(q2 * sc.z, q3 * sc.w));
        } else {
          store_stream_u2(prow + tiled(js + base + 4 * gi), pack_bf16x2(q0, q1), pack_bf16x2(q2, q3));
        }
      }
    }
  }
  if (rs >= 0) {
    const float t = __builtin_fmaf(xs, kLog2e, nl);
    const float q = exp2_hw(t);
    z += q;
    s1 = __builtin_fmaf(q, t, s1);
    if (active && in_slice) store_stream_u16(prow + tiled(js + rs), __builtin_bit_cast(uint16_t, (__bf16)(q * ss)));
  }
  z = wave_sum(z);
  s1 = wave_sum(s1);
  if constexpr (W > 1) {
    if (lane == 0) { grp_z[wave] = z; grp_s[wave] = s1; }
    __syncthreads();
    const int w0 = wave - k;
    z = grp_z[w0];
    s1 = grp_s[w0];
    for (int q = 1; q < W; ++q) { z += grp_z[w0 + q]; s1 += grp_s[w0 + q]; }
  }
  if (active && k == 0 && lane == 0) {
    stats[(int64_t)r * n_rows + row] = make_float4(mv, z, s1 * kLn2, mv);
    stat_arg[(int64_t)r * n_rows + row] = (int32_t)(c0 + mi);
  }
}

// The range merge as a kernel of its own: one wavefront per row (merge_ranges_row).
constexpr int kMergeRangesThreads = 256;

__global__ void __launch_bounds__(kMergeRangesThreads)
merge_ranges_kernel(const float4* __restrict__ stats, const int32_t* __restrict__ stat_arg,
                    int64_t n_rows, int n_ranges, int r0, int splits, float gamma,
                    float* __restrict__ factors, float* __restrict__ row_max,
                    float* __restrict__ row_lse, float* __restrict__ row_entropy,
                    int32_t* __restrict__ row_argmax) {
  const int64_t row = (int64_t)blockIdx.x * (kMergeRangesThreads / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;                           // whole wavefronts only
  merge_ranges_row(stats, stat_arg, n_rows, n_ranges, r0, splits, gamma, factors, row_max,
                   row_lse, row_entropy, row_argmax, row);
}

// Merge of T slice results (one-pass calls on disjoint vocabulary slices, in vocabulary
// order) into the result over their union.  With lse = ln sum_r e^(lse_r), slice r
// carries probability mass pi_r = e^(lse_r - lse):
//   out = sum_r pi_r out_r,   H = sum_r pi_r (H_r - ln pi_r),
//   max = max_r max_r, argmax = the first slice's argmax among those reaching max.
// Each thread produces 4 consecutive columns of one row; slices are added in order.
constexpr int kMergeThreads = 256;

__global__ void __launch_bounds__(kMergeThreads)
merge_slices_kernel(const float* __restrict__ outs, int n_parts, int64_t part_stride,
                    int64_t n_rows, int64_t d, int64_t ld_part, const float* __restrict__ pmax,
                    const float* __restrict__ plse, const float* __restrict__ pent,
                    const int32_t* __restrict__ parg, float* __restrict__ out, int64_t ld_out,
                    float* __restrict__ row_max, float* __restrict__ row_lse,
                    float* __restrict__ row_entropy, int32_t* __restrict__ row_argmax) {
  const int64_t row = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * kMergeThreads + threadIdx.x) * 4;
  if (c >= d) return;
  float top = -INFINITY;
  for (int r = 0; r < n_parts; ++r) top = fmaxf(top, plse[r * n_rows + row]);
  float zs = 0.f;
  for (int r = 0; r < n_parts; ++r) zs += exp2_hw((plse[r * n_rows + row] - top) * kLog2e);
  const float lse = top + logf(zs);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float h = 0.f;
  for (int r = 0; r < n_parts; ++r) {
    const float lp = plse[r * n_rows + row] - lse;          // ln pi_r
    const float pi = exp2_hw(lp * kLog2e);
    const float4 v = *reinterpret_cast<const float4*>(outs + r * part_stride + row * ld_part + c);
    a.x = __builtin_fmaf(pi, v.x, a.x);
    a.y = __builtin_fmaf(pi, v.y, a.y);
    a.z = __builtin_fmaf(pi, v.z, a.z);
    a.w = __builtin_fmaf(pi, v.w, a.w);
    h = __builtin_fmaf(pi, pent[r * n_rows + row] - lp, h);
  }
  *reinterpret_cast<float4*>(out + row * ld_out + c) = a;
  if (c == 0) {
    float mx = -INFINITY;
    int32_t am = 0;
    for (int r = 0; r < n_parts; ++r) {
      const float m = pmax[r * n_rows + row];
      if (m > mx) { mx = m; am = parg[r * n_rows + row]; }
    }
    row_max[row] = mx;
    row_lse[row] = lse;
    row_entropy[row] = h;
    row_argmax[row] = am;
  }
}

}  // namespace

hipError_t launch_merge_slices(const float* outs, int64_t n_parts, int64_t part_stride,
                               int64_t n_rows, int64_t d, int64_t ld_part,
                               const float* part_max, const float* part_lse,
                               const float* part_entropy, const int32_t* part_argmax,
                               float* out, int64_t ld_out, float* row_max, float* row_lse,
                               float* row_entropy, int32_t* row_argmax, hipStream_t stream) {
  const int64_t groups = (d + 3) / 4;
  const dim3 grid((unsigned)((groups + kMergeThreads - 1) / kMergeThreads), (unsigned)n_rows);
  SE_LAUNCH(merge_slices_kernel, grid, dim3(kMergeThreads), 0, stream, outs,
                     (int)n_parts, part_stride, n_rows, d, ld_part, part_max, part_lse,
                     part_entropy, part_argmax, out, ld_out, row_max, row_lse, row_entropy,
                     row_argmax);
  return launched(stream);
}

hipError_t launch_step_sweep(const float* logits, int64_t ld, int64_t n_rows,
                             const StepRanges& g, SweepShape sw, uint16_t* probs, float* stats,
                             int32_t* stat_arg, const float* pscale, hipStream_t stream) {
  const int n_ranges = g.n_pre + g.splits + g.n_post;
  float4* st = reinterpret_cast<float4*>(stats);
  auto go = [&](auto kernel, int w) {
    const int per_block = (sweep_threads(w) / 64) / w;          // (row, range) items
    const dim3 grid((unsigned)((n_rows * n_ranges + per_block - 1) / per_block));
    SE_LAUNCH(kernel, grid, dim3(sweep_threads(w)), 0, stream, logits, ld, n_rows, g,
                       n_ranges, probs, st, stat_arg, pscale);
    return launched(stream);
  };
  auto pick = [&](auto scaled) -> hipError_t {
    constexpr bool S = decltype(scaled)::value;
    if (sw.groups == 16) {
      if (sw.waves == 4) return go(step_sweep_kernel<4, 16, S>, 4);
      return hipErrorInvalidValue;
    }
    if (sw.groups != 12) return hipErrorInvalidValue;
    switch (sw.waves) {
      case 1: return go(step_sweep_kernel<1, 12, S>, 1);
      case 2: return go(step_sweep_kernel<2, 12, S>, 2);
      case 4: return go(step_sweep_kernel<4, 12, S>, 4);
      case 8: return go(step_sweep_kernel<8, 12, S>, 8);
      default: return hipErrorInvalidValue;
    }
  };
  return pscale ? pick(std::true_type{}) : pick(std::false_type{});
}

hipError_t launch_merge_ranges(const float* stats, const int32_t* stat_arg, int64_t n_rows,
                               int n_ranges, int r0, int splits, float gamma, float* factors,
                               float* row_max, float* row_lse, float* row_entropy,
                               int32_t* row_argmax, hipStream_t stream) {
  const int per_block = kMergeRangesThreads / 64;
  const dim3 grid((unsigned)((n_rows + per_block - 1) / per_block));
  SE_LAUNCH(merge_ranges_kernel, grid, dim3(kMergeRangesThreads), 0, stream,
                     reinterpret_cast<const float4*>(stats), stat_arg, n_rows, n_ranges, r0,
                     splits, gamma, factors, row_max, row_lse, row_entropy, row_argmax);
  return launched(stream);
}

hipError_t launch_split_sweep(const float* logits, int64_t ld, int64_t col0, int64_t K,
                              int64_t n_rows, int splits, int kblocks, uint16_t* probs,
                              float* stats, int32_t* stat_arg, int64_t rows_pad,
                              hipStream_t stream) {
  const dim3 grid((unsigned)(n_rows * splits));
  SE_LAUNCH(split_sweep_kernel, grid, dim3(kSweepThreads), 0, stream, logits, ld, col0,
                     K, n_rows, splits, kblocks, probs, reinterpret_cast<float4*>(stats),
                     stat_arg, rows_pad);
  return launched(stream);
}

}  // namespace se

// row_stats.hip -- one streaming pass over each full-width fp32 logits row:
// running max, sum of 2^(t), sum of 2^(t) * t with t = (l - m) * log2(e), and
// the first index of the maximum.  These give the log-sum-exp and the entropy
// of the row's softmax:
//     lse = m + ln Z,     H = ln Z - S1 / Z,   Z = sum e^(l-m),  S1 = sum e^(l-m)(l-m)
// (H = -sum p ln p rewritten with ln p = (l - m) - ln Z; no 0*log 0 and no
// cancellation between two large numbers).  The softmax is over the whole
// vocabulary as on calvarado04.com, "Where the shapes stop agreeing" (the
// sampler runs on gathered, full-width logits); entropy and argmax are what the
// DiffusionGemma sampler's acceptance and convergence tests consume (agentlenshq
// overview, "sampling loop and entropy-bound denoising").
//
// Partial states are merged with the online-normaliser rule (Milakov &
// Gimelshein, "Online normalizer calculation for softmax", 2018), extended to
// carry S1 and the argmax.  One workgroup of 1024 threads owns one row; each
// thread streams 16-byte loads, 4 in flight, then wavefront shuffles and LDS
// combine the 16 wave states in a fixed order.
//
// PROBS (the whole-step entry point): once the row's lse is known, the same
// workgroup reads the vocabulary slice [col0, col0 + K) of its row again -- moments
// after streaming it, so mostly from cache -- and writes the slice's bf16
// probabilities, exactly as probs.hip forms them, in the super-step-tiled layout the
// contraction streams: position k of row i at
// probs[(k / kSuperStep) * n_rows * kSuperStep + i * kSuperStep + k % kSuperStep].
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

#include <climits>

namespace se {

namespace {

struct RowState {
  float m;    // running max (natural units)
  float z;    // sum 2^(t_v), t_v = (l_v - m) * log2e
  float s1;   // sum 2^(t_v) * t_v   (log2 units)
  int idx;    // first index of m
};

#ifndef SE_ROW_THREADS
#define SE_ROW_THREADS 1024
#endif
#ifndef SE_ROW_UNROLL
#define SE_ROW_UNROLL 4
#endif
constexpr int kRowThreads = SE_ROW_THREADS;
constexpr int kUnroll = SE_ROW_UNROLL;

__device__ __forceinline__ void merge(RowState& a, RowState b) {
  const bool take_b = (b.m > a.m) || (b.m == a.m && b.idx < a.idx);
  if (take_b) { RowState t = a; a = b; b = t; }
  if (b.z > 0.f) {                     // b holds at least one element
    const float dm = (b.m - a.m) * kLog2e;   // <= 0
    const float f = exp2_hw(dm);
    a.z = __builtin_fmaf(f, b.z, a.z);
    a.s1 = __builtin_fmaf(f, __builtin_fmaf(dm, b.z, b.s1), a.s1);
  }
}

// Rescale the state to a new, larger maximum `nm`.
__device__ __forceinline__ void raise_max(RowState& st, float nm, int nidx) {
  if (st.z > 0.f) {
    const float dm = (st.m - nm) * kLog2e;
    const float f = exp2_hw(dm);
    st.s1 = f * __builtin_fmaf(dm, st.z, st.s1);
    st.z = f * st.z;
  }
  st.m = nm;
  st.idx = nidx;
}

__device__ __forceinline__ void accum(RowState& st, float v, float nml) {
  const float t = __builtin_fmaf(v, kLog2e, nml);
  const float e = exp2_hw(t);
  st.z += e;
  st.s1 = __builtin_fmaf(e, t, st.s1);
}

__device__ __forceinline__ RowState shfl_xor_state(const RowState& s, int mask) {
  RowState o;
  o.m = __shfl_xor(s.m, mask);
  o.z = __shfl_xor(s.z, mask);
  o.s1 = __shfl_xor(s.s1, mask);
  o.idx = __shfl_xor(s.idx, mask);
  return o;
}

// A group: the kUnroll chunks c, c + kRowThreads, ... of every thread, kUnroll * kRowThreads
// float4s (16,384 positions at 1024 threads and 4 chunks) of the row; the main loop takes
// one group per iteration.
constexpr int kGroupF4 = kUnroll * kRowThreads;
// HOLD (with PROBS): the slice's first groups [hg0, hg0 + hn), hn <= HOLD, inside the main
// loop's range, are met in the same order as always and kept in registers; the slice's
// probabilities there are written from registers once the row's lse is known, and the rest
// of the slice (if it is longer) is read again.  The groups read earliest are the ones held:
// they are the likeliest to have left the caches.
constexpr int kHoldGroups = 16 / kUnroll;        // 16 float4 (64 VGPRs) per thread
static_assert(kHoldGroups >= 1, "at most 16 chunks per group");

// SCALED (with PROBS): slice position k's probability is stored times pscale[k] (a power of
// two, so the bf16 value is the unscaled one times pscale[k] exactly; 16-byte aligned).
template <bool PROBS, int HOLD, bool SCALED>
__global__ void __launch_bounds__(kRowThreads)
row_stats_kernel(const float* __restrict__ logits, int64_t ld, int vocab,
                 float* __restrict__ row_max, float* __restrict__ row_lse,
                 float* __restrict__ row_entropy, int32_t* __restrict__ row_argmax,
                 int64_t col0, int64_t K, uint16_t* __restrict__ probs, int64_t n_rows,
                 const float* __restrict__ pscale) {
  const int64_t row = blockIdx.x;
  const float* __restrict__ x = logits + row * ld;
  const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x);
  const int tid = threadIdx.x;
  const int n4 = vocab >> 2;

  RowState st{-INFINITY, 0.f, 0.f, INT_MAX};
  int c = tid;
  // Each thread visits its chunks in increasing index order, so a strict ">"
  // keeps the first occurrence of the maximum.
  auto group = [&](int c, const float4 (&v)[kUnroll]) {
    float cm = v[0].x;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      cm = fmaxf(fmaxf(fmaxf(cm, v[u].x), fmaxf(v[u].y, v[u].z)), v[u].w);
    if (cm > st.m) {
      int idx = 0;
#pragma unroll
      for (int u = kUnroll - 1; u >= 0; --u) {
        const int b = 4 * (c + u * kRowThreads);
        idx = (v[u].w == cm) ? b + 3 : idx;
        idx = (v[u].z == cm) ? b + 2 : idx;
        idx = (v[u].y == cm) ? b + 1 : idx;
        idx = (v[u].x == cm) ? b : idx;
      }
      raise_max(st, cm, idx);
    }
    const float nml = -(st.m * kLog2e);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      accum(st, v[u].x, nml);
      accum(st, v[u].y, nml);
      accum(st, v[u].z, nml);
      accum(st, v[u].w, nml);
    }
  };
  float4 held[HOLD > 0 ? HOLD : 1][kUnroll];
  int hg0 = 0, hn = 0;
  if constexpr (HOLD > 0) {
    hg0 = (int)(col0 / (4 * kGroupF4));
    hn = min((int)((col0 + K + 4 * kGroupF4 - 1) / (4 * kGroupF4)) - hg0, HOLD);
    for (; c < tid + hg0 * kGroupF4; c += kGroupF4) {
      float4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = load_stream_f4(x4 + c + u * kRowThreads);
      group(c, v);
    }
#pragma unroll
    for (int h = 0; h < HOLD; ++h) {
      if (h < hn) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) held[h][u] = load_stream_f4(x4 + c + u * kRowThreads);
        group(c, held[h]);
        c += kGroupF4;
      }
    }
  }
  for (; c + (kUnroll - 1) * kRowThreads < n4; c += kGroupF4) {
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_stream_f4(x4 + c + u * kRowThreads);
    group(c, v);
  }
  for (; c < n4; c += kRowThreads) {
    const float4 v = load_stream_f4(x4 + c);
    const float cm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (cm > st.m) {
      const int b = 4 * c;
      const int idx = (v.x == cm) ? b : (v.y == cm) ? b + 1 : (v.z == cm) ? b + 2 : b + 3;
      raise_max(st, cm, idx);
    }
    const float nml = -(st.m * kLog2e);
    accum(st, v.x, nml);
    accum(st, v.y, nml);
    accum(st, v.z, nml);
    accum(st, v.w, nml);
  }
  if (tid == 0) {
    // the last vocab % 4 columns, after every chunk this thread has seen
    for (int j = 4 * n4; j < vocab; ++j) {
      const float v = x[j];
      if (v > st.m) raise_max(st, v, j);
      accum(st, v, -(st.m * kLog2e));
    }
  }

  // wavefront reduction (fixed butterfly order)
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) merge(st, shfl_xor_state(st, mask));

  __shared__ RowState partial[kRowThreads / 64];
  __shared__ float row_lse_s;
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) partial[wave] = st;
  __syncthreads();
  if (wave == 0) {
    RowState r = (lane < kRowThreads / 64) ? partial[lane]
                                           : RowState{-INFINITY, 0.f, 0.f, INT_MAX};
#pragma unroll
    for (int mask = 8; mask >= 1; mask >>= 1) merge(r, shfl_xor_state(r, mask));
    if (lane == 0) {
      const float lnz = logf(r.z);
      row_max[row] = r.m;
      row_argmax[row] = r.idx;
      row_lse[row] = r.m + lnz;
      row_entropy[row] = lnz - (r.s1 * kLn2) / r.z;
      row_lse_s = r.m + lnz;
    }
  }
  if constexpr (PROBS) {
    __syncthreads();
    const float nl = neg_lse_log2(row_lse_s);
    const float* __restrict__ xs = x + col0;
    uint16_t* __restrict__ prow = probs + row * kSuperStep;
    // the slice's positions [k_begin, K) read again (k_begin a multiple of 8)
    // the scales of slice positions k .. k + 3 (k a multiple of 4), or of position k alone
    auto scale4 = [&](int64_t k) -> float4 {
      if constexpr (SCALED) return reinterpret_cast<const float4*>(pscale + k)[0];
      else return make_float4(1.f, 1.f, 1.f, 1.f);
    };
    auto scale1 = [&](int64_t k) -> float {
      if constexpr (SCALED) return pscale[k];
      else return 1.f;
    };
    auto reread = [&](int64_t k_begin) {
      auto put8 = [&](int64_t k, const float4& a, const float4& b) {
        uint4 o;
        if constexpr (SCALED) {
          const float4 sa = scale4(k), sb = scale4(k + 4);
          o.x = pack_bf16x2(prob_from_logit(a.x, nl) * sa.x, prob_from_logit(a.y, nl) * sa.y);
          o.y = pack_bf16x2(prob_from_logit(a.z, nl) * sa.z, prob_from_logit(a.w, nl) * sa.w);
          o.z = pack_bf16x2(prob_from_logit(b.x, nl) * sb.x, prob_from_logit(b.y, nl) * sb.y);
          o.w = pack_bf16x2(prob_from_logit(b.z, nl) * sb.z, prob_from_logit(b.w, nl) * sb.w);
        } else {
          o.x = pack_bf16x2(prob_from_logit(a.x, nl), prob_from_logit(a.y, nl));
          o.y = pack_bf16x2(prob_from_logit(a.z, nl), prob_from_logit(a.w, nl));
          o.z = pack_bf16x2(prob_from_logit(b.x, nl), prob_from_logit(b.y, nl));
          o.w = pack_bf16x2(prob_from_logit(b.z, nl), prob_from_logit(b.w, nl));
        }
        store_stream_u4(prow + (k / kSuperStep) * n_rows * kSuperStep + k % kSuperStep, o);
      };
      // four 8-position groups per thread in flight, then the remaining groups one by one
      constexpr int64_t kStride = 8 * (int64_t)kRowThreads;
      int64_t k = k_begin + 8 * (int64_t)tid;
      for (; k + 3 * kStride + 8 <= K; k += 4 * kStride) {
        float4 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = reinterpret_cast<const float4*>(xs + k + u * kStride)[0];
          b[u] = reinterpret_cast<const float4*>(xs + k + u * kStride)[1];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) put8(k + u * kStride, a[u], b[u]);
      }
      for (; k < K; k += kStride) {
        if (k + 8 <= K) {
          put8(k, reinterpret_cast<const float4*>(xs + k)[0], reinterpret_cast<const float4*>(xs + k)[1]);
        } else {
          uint16_t* __restrict__ pp = prow + (k / kSuperStep) * n_rows * kSuperStep + k % kSuperStep;
          for (int64_t j = 0; j < K - k; ++j)
            store_stream_u16(pp + j, __builtin_bit_cast(
                                         uint16_t, (__bf16)(prob_from_logit(xs[k + j], nl) * scale1(k + j))));
        }
      }
    };
    if constexpr (HOLD > 0) {
      // chunk c of the row holds positions 4 c .. 4 c + 3 (one super-step, as 4 c % 128 <=
      // 124); slice position k = 4 c - col0.  col0 is a multiple of 8, so no chunk straddles
      // it; a chunk straddling the slice's end is written element by element.
#pragma unroll
      for (int h = 0; h < HOLD; ++h) {
        if (h < hn) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int64_t k = 4 * (int64_t)(tid + (hg0 + h) * kGroupF4 + u * kRowThreads) - col0;
            if (k < 0 || k >= K) continue;
            uint16_t* dst = prow + (k / kSuperStep) * n_rows * kSuperStep + k % kSuperStep;
            const float4 v = held[h][u];
            if (k + 4 <= K) {
              if constexpr (SCALED) {
                const float4 sv = scale4(k);
                store_stream_u2(dst, pack_bf16x2(prob_from_logit(v.x, nl) * sv.x, prob_from_logit(v.y, nl) * sv.y),
                                pack_bf16x2(prob_from_logit(v.z, nl) * sv.z, prob_from_logit(v.w, nl) * sv.w));
              } else {
                store_stream_u2(dst, pack_bf16x2(prob_from_logit(v.x, nl), prob_from_logit(v.y, nl)),
                                pack_bf16x2(prob_from_logit(v.z, nl), prob_from_logit(v.w, nl)));
              }
            } else {
              const float e4[4] = {v.x, v.y, v.z, v.w};
              for (int j = 0; j < (int)(K - k); ++j)
                store_stream_u16(dst + j, __builtin_bit_cast(
                                              uint16_t, (__bf16)(prob_from_logit(e4[j], nl) * scale1(k + j))));
            }
          }
        }
      }
      // a slice longer than the held groups: the rest is read again
      const int64_t k_rest = (int64_t)(hg0 + hn) * 4 * kGroupF4 - col0;
      if (k_rest < K) reread(k_rest);
    } else {
      reread(0);
    }
  }
}

}  // namespace

hipError_t launch_row_stats(const float* logits, int64_t ld, int64_t n_rows, int vocab,
                            float* row_max, float* row_lse, float* row_entropy,
                            int32_t* row_argmax, hipStream_t stream) {
  SE_LAUNCH((row_stats_kernel<false, 0, false>), dim3((unsigned)n_rows), dim3(kRowThreads), 0,
                     stream, logits, ld, vocab, row_max, row_lse, row_entropy, row_argmax,
                     (int64_t)0, (int64_t)0, nullptr, n_rows, nullptr);
  return launched(stream);
}

hipError_t launch_row_stats_probs(const float* logits, int64_t ld, int64_t n_rows, int vocab,
                                  float* row_max, float* row_lse, float* row_entropy,
                                  int32_t* row_argmax, int64_t col0, int64_t K,
                                  uint16_t* probs, const float* pscale, hipStream_t stream) {
  // the slice's first kHoldGroups groups, when they lie inside the main loop's range: kept
  // in registers (the rest of a longer slice is read again); otherwise all read again
  const int64_t gpos = 4 * (int64_t)kGroupF4;
  const int64_t g0 = col0 / gpos;
  const int64_t g_held = min((col0 + K + gpos - 1) / gpos, g0 + kHoldGroups);
  const bool hold = K > 0 && g_held <= (vocab / 4) / kGroupF4;
  auto go = [&](auto kernel) {
    SE_LAUNCH(kernel, dim3((unsigned)n_rows), dim3(kRowThreads), 0, stream, logits, ld, vocab,
              row_max, row_lse, row_entropy, row_argmax, col0, K, probs, n_rows, pscale);
    return launched(stream);
  };
  if (pscale)
    return hold ? go(row_stats_kernel<true, kHoldGroups, true>) : go(row_stats_kernel<true, 0, true>);
  return hold ? go(row_stats_kernel<true, kHoldGroups, false>) : go(row_stats_kernel<true, 0, false>);
}

}  // namespace se

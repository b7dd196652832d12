// accept.hip -- entropy-bound acceptance and the convergence test of the
// diffusion sampler, run on the per-position statistics of se_row_stats.
//
// The rule (agentlenshq overview of DiffusionGemma in vLLM, section on the
// sampling loop and entropy-bound denoising): candidate tokens are accepted from
// the most confident to the least confident until the cumulative entropy exceeds
// a fixed budget; a canvas has converged when its argmax prediction has been
// stable for several steps and its mean per-token entropy is below a threshold,
// or when a step limit is reached.
//
// One workgroup per canvas: one thread per position, the workgroup size the power of
// two at or above canvas_len (64 .. 1024):
//   1. stability: any position whose argmax differs from the previous step's;
//   2. entropies become exact fixed-point integers q = rint(H * 2^32), so the
//      cumulative and the mean sums are exact and independent of summation order;
//   3. the positions not yet accepted are sorted by (entropy, index) -- a bitonic
//      sort of 64-bit keys in LDS -- and an inclusive scan of q in that order
//      gives the cumulative entropies;
//   4. the accepted prefix ends before the first cumulative value above the
//      budget, but holds at least one position when any is left;
//   5. per canvas: stable-step counter, step counter, converged flag.
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kAcceptThreads = 1024;
constexpr double kFix = 4294967296.0;            // 2^32 fixed-point scale of entropies

// fp32 -> uint32 whose unsigned order is the float order (-0 folded onto +0)
__device__ __forceinline__ uint32_t sortable(float h) {
  uint32_t u = __builtin_bit_cast(uint32_t, h);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void __launch_bounds__(kAcceptThreads)
accept_converge_kernel(const float* __restrict__ row_entropy,
                       const int32_t* __restrict__ row_argmax, int len, double budget,
                       int stable_steps, double tau, int step_limit,
                       uint8_t* __restrict__ accepted, int32_t* __restrict__ prev_argmax,
                       int32_t* __restrict__ stable_count, int32_t* __restrict__ step_count,
                       uint8_t* __restrict__ newly, uint8_t* __restrict__ converged) {
  __shared__ unsigned long long key[kAcceptThreads];
  __shared__ long long q[kAcceptThreads];
  __shared__ long long scan[kAcceptThreads];
  __shared__ uint8_t take[kAcceptThreads];
  __shared__ int first_over;
  __shared__ int n_elig;

  const int c = blockIdx.x;
  const int i = threadIdx.x;
  const int nt = blockDim.x;                       // power of two >= len
  const int64_t base = (int64_t)c * len;
  const bool in = i < len;

  float h = 0.f;
  int am = 0, pam = 0, acc = 1;
  if (in) {
    h = row_entropy[base + i];
    am = row_argmax[base + i];
    pam = prev_argmax[base + i];
    acc = accepted[base + i];
  }
  if (i == 0) { first_over = nt; n_elig = 0; }

  // 1. stability of the argmax prediction
  const int changed = __syncthreads_or(in && am != pam);

  // 2. exact fixed-point entropies
  const long long qi = in ? __double2ll_rn((double)h * kFix) : 0ll;
  q[i] = qi;
  const bool elig = in && acc == 0;
  key[i] = elig ? ((unsigned long long)sortable(h) << 32) | (unsigned)i : ~0ull;
  if (elig) atomicAdd(&n_elig, 1);
  __syncthreads();

  // 3. bitonic sort of the keys, ascending: (entropy, index) of eligible positions
  for (int k = 2; k <= nt; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int ixj = i ^ j;
      if (ixj > i) {
        const unsigned long long a = key[i], b = key[ixj];
        const bool up = (i & k) == 0;
        if ((a > b) == up) { key[i] = b; key[ixj] = a; }
      }
      __syncthreads();
    }
  }
  // inclusive scan of q in sorted order (Hillis-Steele, exact integer adds)
  const unsigned long long ks = key[i];
  const bool s_elig = ks != ~0ull;
  long long v = s_elig ? q[(int)(ks & 0xffffffffu)] : 0ll;
  scan[i] = v;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const long long add = i >= off ? scan[i - off] : 0ll;
    __syncthreads();
    v += add;
    scan[i] = v;
    __syncthreads();
  }
  // 4. the accepted prefix: positions before the first cumulative value above the
  //    budget, at least one
  if (s_elig && (double)v > budget * kFix) atomicMin(&first_over, i);
  __syncthreads();
  const int n_acc = n_elig > 0 ? max(min(first_over, n_elig), 1) : 0;
  take[i] = 0;
  __syncthreads();
  if (i < n_acc) take[(int)(ks & 0xffffffffu)] = 1;

  // 5. per-canvas state; the mean entropy is the exact sum of q over the canvas
  //    (reused from the scan array: reduce q in index order)
  __syncthreads();
  scan[i] = qi;
  __syncthreads();
  for (int off = nt / 2; off > 0; off >>= 1) {
    if (i < off) scan[i] += scan[i + off];
    __syncthreads();
  }
  __syncthreads();
  if (in) {
    newly[base + i] = take[i];
    if (take[i]) accepted[base + i] = 1;
    prev_argmax[base + i] = am;
  }
  if (i == 0) {
    const int st = changed ? 0 : stable_count[c] + 1;
    const int steps = step_count[c] + 1;
    stable_count[c] = st;
    step_count[c] = steps;
    const bool calm = (double)scan[0] < tau * (double)len * kFix;
    converged[c] = (uint8_t)((st >= stable_steps && calm) || steps >= step_limit);
  }
}

}  // namespace

hipError_t launch_accept_converge(const float* row_entropy, const int32_t* row_argmax,
                                  int64_t n_canvas, int len, double budget, int stable_steps,
                                  double tau, int step_limit, uint8_t* accepted,
                                  int32_t* prev_argmax, int32_t* stable_count,
                                  int32_t* step_count, uint8_t* newly, uint8_t* converged,
                                  hipStream_t stream) {
  int nt = 64;
  while (nt < len) nt <<= 1;
  SE_LAUNCH(accept_converge_kernel, dim3((unsigned)n_canvas), dim3(nt), 0,
                     stream, row_entropy, row_argmax, len, budget, stable_steps, tau, step_limit,
                     accepted, prev_argmax, stable_count, step_count, newly, converged);
  return launched(stream);
}

}  // namespace se

// probs.hip -- materialise bf16 probabilities of a vocab slice (unfused path).
//     probs[i, s + k] = bf16_rne( e^(l[i, s + k] - lse_i) ),  0 <= k < K
// The cast of the probability slice to the embedding dtype is the first line
// of the fix on calvarado04.com ("The fix"); rounding is nearest-even.
// Each thread converts 8 consecutive columns: two 16-byte loads, one 16-byte
// store.  Grid: x over column groups, y over rows.
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kProbThreads = 256;

// TILED: position k of row i goes to probs[(k / kSuperStep) * n_rows * kSuperStep +
// i * kSuperStep + k % kSuperStep] (8 positions never straddle a super-step).
template <bool TILED>
__global__ void __launch_bounds__(kProbThreads)
probs_bf16_kernel(const float* __restrict__ logits, int64_t ld, const float* __restrict__ lse,
                  int64_t col0, int64_t K, uint16_t* __restrict__ probs, int64_t ldp,
                  int64_t n_rows, int64_t row0) {
  const int64_t row = row0 + blockIdx.y;
  const int64_t k = ((int64_t)blockIdx.x * kProbThreads + threadIdx.x) * 8;
  if (k >= K) return;
  const float nl = neg_lse_log2(lse[row]);
  const float* __restrict__ x = logits + row * ld + col0 + k;
  uint16_t* __restrict__ p =
      TILED ? probs + (k / kSuperStep) * n_rows * kSuperStep + row * kSuperStep + k % kSuperStep
            : probs + row * ldp + col0 + k;
  if (k + 8 <= K) {
    const float4 a = reinterpret_cast<const float4*>(x)[0];
    const float4 b = reinterpret_cast<const float4*>(x)[1];
    uint4 o;
    o.x = pack_bf16x2(prob_from_logit(a.x, nl), prob_from_logit(a.y, nl));
    o.y = pack_bf16x2(prob_from_logit(a.z, nl), prob_from_logit(a.w, nl));
    o.z = pack_bf16x2(prob_from_logit(b.x, nl), prob_from_logit(b.y, nl));
    o.w = pack_bf16x2(prob_from_logit(b.z, nl), prob_from_logit(b.w, nl));
    store_stream_u4(p, o);
  } else {
    for (int64_t j = 0; j < K - k; ++j)
      store_stream_u16(p + j, __builtin_bit_cast(uint16_t, (__bf16)prob_from_logit(x[j], nl)));
  }
}

}  // namespace

hipError_t launch_probs_bf16(const float* logits, int64_t ld, const float* row_lse,
                             int64_t n_rows, int64_t col0, int64_t K, uint16_t* probs,
                             int64_t ldp, hipStream_t stream) {
  const int64_t groups = (K + 7) / 8;
  const dim3 grid((unsigned)((groups + kProbThreads - 1) / kProbThreads), (unsigned)n_rows);
  SE_LAUNCH(probs_bf16_kernel<false>, grid, dim3(kProbThreads), 0, stream, logits, ld,
                     row_lse, col0, K, probs, ldp, n_rows, (int64_t)0);
  return launched(stream);
}

hipError_t launch_probs_bf16_tiled(const float* logits, int64_t ld, const float* row_lse,
                                   int64_t n_rows, int64_t col0, int64_t K, uint16_t* probs,
                                   hipStream_t stream) {
  const int64_t groups = (K + 7) / 8;
  constexpr int64_t kMaxRows = 65535;                 // grid.y per launch
  for (int64_t r0 = 0; r0 < n_rows; r0 += kMaxRows) {
    const int64_t nr = n_rows - r0 < kMaxRows ? n_rows - r0 : kMaxRows;
    const dim3 grid((unsigned)((groups + kProbThreads - 1) / kProbThreads), (unsigned)nr);
    SE_LAUNCH(probs_bf16_kernel<true>, grid, dim3(kProbThreads), 0, stream, logits, ld,
                       row_lse, col0, K, probs, (int64_t)0, n_rows, r0);
    const hipError_t e = launched(stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace se

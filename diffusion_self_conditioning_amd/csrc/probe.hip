// probe.hip -- the achievable bf16 MFMA rate of the device, the measured ceiling that the
// contraction's roofline is read against beside the nominal peak (2.5 PFLOP/s dense bf16
// at the 2.4 GHz peak clock).  Every wave runs chains of v_mfma_f32_32x32x16_bf16 on
// register operands, back to back; nothing is read from memory, and one value per lane is
// stored at the end so the work stays live.  With operands all equal to u, every
// accumulator element ends at 16 u^2 per MFMA of its chain, so the stored sums are exact
// for small counts and the probe doubles as a check of the instruction's arithmetic.
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kLoopThreads = 256;   // 4 waves per workgroup
constexpr int kLoopChains = 8;      // independent accumulator chains per wave
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(kLoopThreads)
mfma_loop_kernel(float* __restrict__ out, int iters, float unit) {
  const unsigned short ub = (unsigned short)(__float_as_uint(unit) >> 16);
  const u16x8_t ui = {ub, ub, ub, ub, ub, ub, ub, ub};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ui);
  f32x16 acc[kLoopChains];
#pragma unroll
  for (int c = 0; c < kLoopChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kLoopChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kLoopChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * kLoopThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace se

// The entry point (include/softembed.h): host checks first, then one launch.
extern "C" se_status se_mfma_loop(float* out, int64_t blocks, int64_t iters, float unit,
                                  void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > ((int64_t)1 << 24)) return SE_ERR_SHAPE;
  if (!out) return SE_ERR_NULL;
  if (((uintptr_t)out & 3u) != 0) return SE_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  SE_LAUNCH(se::mfma_loop_kernel, dim3((unsigned)blocks), dim3(se::kLoopThreads), 0, st, out,
            (int)iters, unit);
  return se::launched(st) == hipSuccess ? SE_OK : SE_ERR_HIP;
}

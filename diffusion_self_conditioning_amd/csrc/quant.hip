// quant.hip -- the e4m3 (OCP FP8) form of the embedding table: one power-of-two
// scale per vocabulary row and one e4m3 code per element.
//
// The pages serve the model with FP8 weights (agentlenshq overview of DiffusionGemma
// in vLLM, section on performance and quantization: quantized checkpoints hold FP8
// weights with fully dynamic activations).  For the soft embedding the table is the
// operand streamed from HBM, so its e4m3 form halves the bytes of the contraction's
// dominant stream.  The scale of row v is 2^k_v with k_v the smallest integer
// (at least -126) such that max_j |W[v, j]| <= 448 * 2^k_v -- 448 is the largest
// finite e4m3 value -- and the code of W[v, j] is e4m3_rne(W[v, j] * 2^-k_v).  With
// a power-of-two scale the product code * scale is exactly a bf16 value, so the
// dequantized table is exact in bf16 and the e4m3 contraction equals the bf16
// contraction of the dequantized table.
//
// One wave per table row: a pass for the row's absolute maximum (integer compare of
// the bf16 magnitude bits, exact), then a pass that scales and converts (hardware
// round-to-nearest-even conversion to e4m3).
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kQuantThreads = 256;                 // 4 rows per workgroup
constexpr int kQuantRows = kQuantThreads / 64;

__device__ __forceinline__ uint32_t mag_max8(uint4 v) {
  const uint32_t a = max(v.x & 0x7fffu, (v.x >> 16) & 0x7fffu);
  const uint32_t b = max(v.y & 0x7fffu, (v.y >> 16) & 0x7fffu);
  const uint32_t c = max(v.z & 0x7fffu, (v.z >> 16) & 0x7fffu);
  const uint32_t d = max(v.w & 0x7fffu, (v.w >> 16) & 0x7fffu);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// four fp32 -> four e4m3 codes (bytes 0..3), round to nearest even
__device__ __forceinline__ uint32_t to_fp8x4(float a, float b, float c, float d) {
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__global__ void __launch_bounds__(kQuantThreads)
quantize_fp8_kernel(const uint16_t* __restrict__ w, int64_t ldw, int64_t rows, int d,
                    uint8_t* __restrict__ codes, int64_t ldq, float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kQuantRows + (threadIdx.x >> 6);
  if (row >= rows) return;                         // uniform per wave
  const uint16_t* src = w + row * ldw;

  uint32_t amax = 0;
  for (int c = 8 * lane; c < d; c += 512)
    amax = max(amax, mag_max8(*reinterpret_cast<const uint4*>(src + c)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o));

  // smallest k with a <= 448 2^k: a = f 2^e with f in [0.5, 1) and 448 = 0.875 2^9
  int k = 0;
  if (amax != 0) {
    int e;
    const float f = __builtin_frexpf(bf16_lo(amax), &e);
    k = f <= 0.875f ? e - 9 : e - 8;
    k = max(k, -126);
  }
  const float inv = __builtin_ldexpf(1.f, -k);     // exact: -k <= 126
  if (lane == 0) row_scale[row] = __builtin_ldexpf(1.f, k);

  uint8_t* dst = codes + row * ldq;
  for (int c = 8 * lane; c < d; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + c);
    uint2 o;
    o.x = to_fp8x4(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
    o.y = to_fp8x4(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
    *reinterpret_cast<uint2*>(dst + c) = o;
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* w, int64_t ldw, int64_t rows, int64_t d,
                               uint8_t* codes, int64_t ldq, float* row_scale,
                               hipStream_t stream) {
  const int64_t blocks = (rows + kQuantRows - 1) / kQuantRows;
  SE_LAUNCH(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                     w, ldw, rows, (int)d, codes, ldq, row_scale);
  return launched(stream);
}

}  // namespace se

// reduce.hip -- sum of per-rank partial soft embeddings on one GPU, in a fixed order.
//
// The fix on calvarado04.com ("The fix") forms E^sc = gamma * sum_r S^(r) with one
// all-reduce over the tensor-parallel ranks and leaves the result in the embedding
// dtype.  This kernel is the on-device form of that sum for partials that sit on one
// GPU (T slice calls of se_soft_embed[_fused], gamma already applied): parts are
// added in the order r = 0, 1, ..., T-1 in fp32, and the sum is written as fp32
// and / or rounded to bf16 (nearest even), the pages' output dtype.
#include "se_device.h"
#include "se_dispatch.h"
#include "se_launch.h"

namespace se {
namespace {

constexpr int kReduceThreads = 256;

__global__ void __launch_bounds__(kReduceThreads)
reduce_parts_kernel(const float* __restrict__ parts, int64_t n_parts, int64_t part_stride,
                    int64_t d, int64_t ld_part, float* __restrict__ out, int64_t ld_out,
                    uint16_t* __restrict__ out_bf16, int64_t ld_bf16) {
  const int64_t row = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x) * 4;
  if (c >= d) return;
  const float* src = parts + row * ld_part + c;
  float4 a = *reinterpret_cast<const float4*>(src);
  for (int64_t r = 1; r < n_parts; ++r) {
    const float4 v = *reinterpret_cast<const float4*>(src + r * part_stride);
    a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
  }
  if (out) *reinterpret_cast<float4*>(out + row * ld_out + c) = a;
  if (out_bf16) {
    uint2 o;
    o.x = pack_bf16x2(a.x, a.y);
    o.y = pack_bf16x2(a.z, a.w);
    *reinterpret_cast<uint2*>(out_bf16 + row * ld_bf16 + c) = o;
  }
}

}  // namespace

hipError_t launch_reduce_parts(const float* parts, int64_t n_parts, int64_t part_stride,
                               int64_t n_rows, int64_t d, int64_t ld_part, float* out,
                               int64_t ld_out, uint16_t* out_bf16, int64_t ld_bf16,
                               hipStream_t stream) {
  const dim3 grid((unsigned)((d / 4 + kReduceThreads - 1) / kReduceThreads), (unsigned)n_rows);
  SE_LAUNCH(reduce_parts_kernel, grid, dim3(kReduceThreads), 0, stream, parts, n_parts,
                     part_stride, d, ld_part, out, ld_out, out_bf16, ld_bf16);
  return launched(stream);
}

}  // namespace se

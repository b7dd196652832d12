// Host-only stand-ins for the HIP runtime calls and the kernel launchers that api.cpp
// reaches, so that the C ABI's host code (argument checks, work decomposition, workspace
// layouts, launch markers) can be built with AddressSanitizer and UndefinedBehaviorSanitizer
// and driven on a machine without a GPU.  Each launcher records that it was reached and,
// like the real ones, takes the next two armed launch events; none touches the pointers it
// is given.
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "../../diffusion_self_conditioning_amd/csrc/se_launch.h"

int g_launches = 0;
int g_event_records = 0;
int g_marked_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  ++g_event_records;
  return hipSuccess;
}
}

namespace se {
namespace {
hipError_t launched_stub(hipStream_t) {
  ++g_launches;
  hipEvent_t start, end;
  if (next_launch_events(&start, &end)) ++g_marked_launches;
  return hipSuccess;
}
}  // namespace

hipError_t launch_row_stats(const float*, int64_t, int64_t, int, float*, float*, float*,
                            int32_t*, hipStream_t s) { return launched_stub(s); }
hipError_t launch_row_stats_probs(const float*, int64_t, int64_t, int, float*, float*, float*,
                                  int32_t*, int64_t, int64_t, uint16_t*, const float*,
                                  hipStream_t s) {
  return launched_stub(s);
}
hipError_t launch_probs_bf16(const float*, int64_t, const float*, int64_t, int64_t, int64_t,
                             uint16_t*, int64_t, hipStream_t s) { return launched_stub(s); }
hipError_t launch_probs_bf16_tiled(const float*, int64_t, const float*, int64_t, int64_t,
                                   int64_t, uint16_t*, hipStream_t s) { return launched_stub(s); }
hipError_t launch_soft_embed(const GemmParams& p, bool, bool, hipStream_t s) {
  // the contraction, then the split reduction unless the partials are kept or there is one
  launched_stub(s);
  if (p.splits > 1 && !p.keep_partials) launched_stub(s);
  return hipSuccess;
}
hipError_t launch_split_sweep(const float*, int64_t, int64_t, int64_t, int64_t, int, int,
                              uint16_t*, float*, int32_t*, int64_t, hipStream_t s) {
  return launched_stub(s);
}
hipError_t launch_onepass_reduce(const GemmParams&, float*, float*, float*, int32_t*, int64_t,
                                 hipStream_t s) { return launched_stub(s); }
hipError_t launch_step_sweep(const float*, int64_t, int64_t, const StepRanges&, SweepShape sw,
                             uint16_t*, float*, int32_t*, const float*, hipStream_t s) {
  const bool narrow = sw.groups == 12 && (sw.waves == 1 || sw.waves == 2 || sw.waves == 4 ||
                                          sw.waves == 8);
  if (!narrow && !(sw.groups == 16 && sw.waves == 4)) return hipErrorInvalidValue;
  return launched_stub(s);
}
hipError_t launch_merge_ranges(const float*, const int32_t*, int64_t, int, int, int, float,
                               float*, float*, float*, float*, int32_t*, hipStream_t s) {
  return launched_stub(s);
}
hipError_t launch_scaled_reduce(const GemmParams&, const float*, hipStream_t s) {
  return launched_stub(s);
}
hipError_t launch_merge_slices(const float*, int64_t, int64_t, int64_t, int64_t, int64_t,
                               const float*, const float*, const float*, const int32_t*, float*,
                               int64_t, float*, float*, float*, int32_t*, hipStream_t s) {
  return launched_stub(s);
}
hipError_t launch_quantize_fp8(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t,
                               float*, hipStream_t s) { return launched_stub(s); }
hipError_t launch_accept_converge(const float*, const int32_t*, int64_t, int, double, int,
                                  double, int, uint8_t*, int32_t*, int32_t*, int32_t*, uint8_t*,
                                  uint8_t*, hipStream_t s) { return launched_stub(s); }
hipError_t launch_reduce_parts(const float*, int64_t, int64_t, int64_t, int64_t, int64_t, float*,
                               int64_t, uint16_t*, int64_t, hipStream_t s) {
  return launched_stub(s);
}
hipError_t launch_zero_rows(float*, int64_t, int64_t, int64_t, hipStream_t s) {
  return launched_stub(s);
}
}  // namespace se

// scratch.hip -- se_soft_embed_step_noalloc: the whole step with its workspace in a
// library-owned device array, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object: every GPU the library runs on holds its
// own copy (kScratchBytes) from the moment the code object is loaded until the process
// ends.  On the host, `scratch` names a host-side stand-in, not device memory, so its
// device address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever handed to kernels.
#include "../../include/softembed.h"
#include "se_launch.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace se {
namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::once_flag scratch_once[kMaxScratchDevices];
void* scratch_addr[kMaxScratchDevices];
hipError_t scratch_err[kMaxScratchDevices];

// The device address of the calling thread's current device's copy of `scratch`.
hipError_t scratch_ptr(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_addr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = scratch_addr[dev];
  return scratch_err[dev];
}

}  // namespace
}  // namespace se

extern "C" size_t se_soft_embed_step_noalloc_max_bytes(void) { return se::kScratchBytes; }

extern "C" se_status se_soft_embed_step_noalloc(
    const float* logits, int64_t ld_logits, int64_t n_rows, int64_t vocab, int64_t vocab_start,
    int64_t vocab_end, const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
    float gamma, float* out, int64_t ld_out, float* row_max, float* row_lse, float* row_entropy,
    int32_t* row_argmax, void* stream) {
  // every check of se_soft_embed_step first, then the size of the array, so that nothing
  // touches the device for a call that will be rejected
  se_status rc = se::check_step(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end,
                                w_shard, nullptr, w_rows, ld_w, d, out, ld_out, row_max, row_lse,
                                row_entropy, row_argmax, false);
  if (rc != SE_OK || n_rows == 0) return rc;
  const size_t need = se_soft_embed_staged_workspace_bytes(n_rows, vocab_start, vocab_end, d);
  if (need > se::kScratchBytes) return SE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && se::scratch_ptr(&ws) != hipSuccess) return SE_ERR_HIP;
  return se_soft_embed_step(logits, ld_logits, n_rows, vocab, vocab_start, vocab_end, w_shard,
                            w_rows, ld_w, d, gamma, out, ld_out, row_max, row_lse, row_entropy,
                            row_argmax, ws, need > 0 ? se::kScratchBytes : 0, stream);
}

// se_dispatch.h -- the kernel launch of every .hip translation unit.  Internal; not part
// of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "se_launch.h"

// Launches `kernel` on `stream`.  With launch markers armed on the calling thread
// (se_set_launch_events), the dispatch itself stamps the kernel's start and end into the
// next two armed events (hipExtLaunchKernel): no command is added to the stream, so the
// markers time the kernel alone and change nothing around it.  Otherwise a plain launch.
#define SE_LAUNCH(kernel, grid, block, shmem, stream, ...)                                     \
  do {                                                                                      \
    hipEvent_t se_start_ = nullptr, se_end_ = nullptr;                                      \
    if (se::next_launch_events(&se_start_, &se_end_))                                       \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, se_start_, se_end_, 0u,      \
                            __VA_ARGS__);                                                   \
    else                                                                                    \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                  \
  } while (0)

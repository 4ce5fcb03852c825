// Kernel launches with optional timing, for the HIP sources only (the C-ABI
// layer never launches a kernel itself).
//
// CA_LAUNCH(kernel_id, kernel, grid, block, shared_bytes, stream, args...)
// launches like hipLaunchKernelGGL. While launch profiling is on and selects
// kernel_id, it launches through hipExtLaunchKernelGGL with a start/stop
// event pair that the dispatch itself stamps with the kernel's start and end:
// no marker packets go into the stream between kernels (a marker around each
// launch costs several microseconds of idle device time per kernel), and the
// elapsed time is the kernel's own.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "launch.h"

#define CA_LAUNCH(kid, kern, grid, block, shmem, st, ...)                                          \
  do {                                                                                              \
    const ::ca::ProfPair ca_pp_ = ::ca::prof_launch(kid);                                           \
    if (ca_pp_.a) {                                                                                 \
      hipExtLaunchKernelGGL(kern, grid, block, shmem, st, ca_pp_.a, ca_pp_.b, 0u, __VA_ARGS__);     \
    } else {                                                                                        \
      hipLaunchKernelGGL(kern, grid, block, shmem, st, __VA_ARGS__);                                \
    }                                                                                               \
  } while (0)

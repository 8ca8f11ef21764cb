// Kernel launch helper shared by the .hip files: a plain launch, or, when the
// caller armed profiling events with qmm_profile_next(), a launch whose start
// and stop events are stamped by the dispatch itself (hipExtLaunchKernelGGL),
// so their interval is the kernel's own execution time.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "qmm_internal.h"

namespace qmm {

template <typename K, typename... Args>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  ProfileEvents pe = take_profile_events();
  if (pe.start || pe.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<hipEvent_t>(pe.start),
                          static_cast<hipEvent_t>(pe.stop), 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

template <typename K, typename... Args>
inline void launch_kernel_lds(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                              Args... args) {
  ProfileEvents pe = take_profile_events();
  if (pe.start || pe.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(lds), s, static_cast<hipEvent_t>(pe.start),
                          static_cast<hipEvent_t>(pe.stop), 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

}  // namespace qmm

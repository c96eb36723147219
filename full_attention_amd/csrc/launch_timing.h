// Kernel launch with the optional timing hook (pakv_set_timing_events): when a
// pair of caller events is due for this kernel kind, the launch goes through
// hipExtLaunchKernelGGL, which has the dispatch itself record the start and
// stop events, so the elapsed time is the kernel's alone (no host gaps).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pakv_internal.h"

namespace pakv {

template <typename Kernel, typename... Args>
inline void launch(int kind, Kernel kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                   Args... args) {
    const int slot = timing_slot(kind);
    if (slot >= 0) {
        void* const* ev = timing_events();
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, static_cast<hipEvent_t>(ev[2 * slot]),
                              static_cast<hipEvent_t>(ev[2 * slot + 1]), 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
    }
}

}  // namespace pakv

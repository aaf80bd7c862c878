// Host-side kernel launch that reports the status of this launch only.
//
// hipLaunchKernel returns the error of the launch it makes; reading
// hipGetLastError after a <<<>>> launch would instead report (and clear) an
// error left by any earlier, unrelated HIP call of the thread.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

template <typename... KArgs>
hipError_t launch_exact(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, KArgs... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}

// Converts each argument to the kernel's parameter type first.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count differs from the kernel's");
  return launch_exact<KArgs...>(kernel, grid, block, stream, static_cast<KArgs>(args)...);
}

}  // namespace attn

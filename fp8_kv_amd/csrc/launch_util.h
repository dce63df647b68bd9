// Kernel launch helper shared by the libpgqa kernels.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace pgqa_launch {

// Launches `kernel` on `stream` and returns the status of this launch alone:
// hipLaunchKernel reports its own result, whereas hipGetLastError after a
// triple-chevron launch would also return (and clear) an error left behind by
// an unrelated earlier call on the same thread.  Every argument is converted
// to the kernel's parameter type before its address is taken.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                  Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<std::decay_t<KArgs>...> vals(
      static_cast<std::decay_t<KArgs>>(std::forward<Args>(args))...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {};
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
}

}  // namespace pgqa_launch

// hipLaunchKernel with an argument array built from the kernel's own
// parameter types: a wrong number of arguments, or one that does not convert
// to its parameter's type, does not compile; the launch's own status is
// returned (nothing else's error state is read or cleared).
#ifndef ATTN_LAUNCH_H
#define ATTN_LAUNCH_H

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace attn_launch {

template <typename... P, typename... A, size_t... I>
hipError_t launch_impl(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t stream, std::index_sequence<I...>,
                       A... a) {
  std::tuple<P...> vals(a...);
  void* args[] = {(void*)&std::get<I>(vals)...};
  return hipLaunchKernel((const void*)kern, grid, block, args, 0, stream);
}

template <typename... P, typename... A>
hipError_t launch(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t stream, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  return launch_impl(kern, grid, block, stream, std::index_sequence_for<P...>{}, a...);
}

}  // namespace attn_launch

#endif  // ATTN_LAUNCH_H

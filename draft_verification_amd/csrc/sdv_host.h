// Host-side launch helper: hipLaunchKernel returns the launch status directly,
// so a stale error left by unrelated code is never misreported as ours.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace sdv {

template <typename... KArgs, typename Tuple, size_t... I>
static hipError_t launch_impl(void (*k)(KArgs...), dim3 g, dim3 b, size_t shmem, hipStream_t s,
                              Tuple& t, std::index_sequence<I...>) {
  void* argv[sizeof...(KArgs) + 1] = {(void*)&std::get<I>(t)..., nullptr};
  return hipLaunchKernel((const void*)k, g, b, argv, shmem, s);
}

// launch(kernel, grid, block, shmem, stream, args...): arguments are converted
// to the kernel's exact parameter types before their addresses are taken.
template <typename... KArgs, typename... Args>
static hipError_t launch(void (*k)(KArgs...), dim3 g, dim3 b, size_t shmem, hipStream_t s,
                         Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> t(std::forward<Args>(args)...);
  return launch_impl(k, g, b, shmem, s, t, std::index_sequence_for<KArgs...>{});
}

}  // namespace sdv

#define SDV_TRY_LAUNCH(expr)                   \
  do {                                         \
    if ((expr) != hipSuccess) return SD_ELAUNCH; \
  } while (0)

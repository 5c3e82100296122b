// Instantiates the N-node kernels (Map, closure, fallback) for one episode
// size N, with window capacities K = 1, 2, 4.  The build compiles this file
// once per N in 1..EP_MAX_NODES with -DEP_N=<N>, so the per-N units compile in
// parallel and every kernel has N fixed at compile time (all register arrays
// are indexed statically).
#include "ep_device.hpp"

#ifndef EP_N
#error "compile with -DEP_N=<episode size>"
#endif

namespace epk {
namespace {

template <int K>
hipError_t launch_map_k(const MapArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((map_kernel<EP_N, K>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_map(const MapArgs& a, int K, dim3 grid, hipStream_t s) {
  switch (K) {
    case 1: return launch_map_k<1>(a, grid, s);
    case 2: return launch_map_k<2>(a, grid, s);
    case 4: return launch_map_k<4>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int K>
hipError_t launch_closure_k(const ClosureArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((closure_kernel<EP_N, K>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_closure(const ClosureArgs& a, int K, dim3 grid, hipStream_t s) {
  switch (K) {
    case 1: return launch_closure_k<1>(a, grid, s);
    case 2: return launch_closure_k<2>(a, grid, s);
    case 4: return launch_closure_k<4>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int K>
hipError_t launch_fallback_k(const FallbackArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((fallback_kernel<EP_N, K>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fallback(const FallbackArgs& a, int K, dim3 grid, hipStream_t s) {
  switch (K) {
    case 1: return launch_fallback_k<1>(a, grid, s);
    case 2: return launch_fallback_k<2>(a, grid, s);
    case 4: return launch_fallback_k<4>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t map_occupancy(int K, int* blocks) {
  switch (K) {
    case 1: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, map_kernel<EP_N, 1>, kBlock, 0);
    case 2: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, map_kernel<EP_N, 2>, kBlock, 0);
    case 4: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, map_kernel<EP_N, 4>, kBlock, 0);
    default: return hipErrorInvalidValue;
  }
}

const Launchers kLaunchers = {launch_map, launch_closure, launch_fallback, map_occupancy};

}  // namespace

#define EPK_CAT2(a, b) a##b
#define EPK_CAT(a, b) EPK_CAT2(a, b)
const Launchers* EPK_CAT(launchers_n, EP_N)() { return &kLaunchers; }

}  // namespace epk

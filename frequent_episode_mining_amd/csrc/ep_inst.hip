// Instantiates the N-node kernels (Map, closure, finish) for one episode
// size N and every window kind.  The build compiles this file once per N in
// 1..EP_MAX_NODES with -DEP_N=<N>, so the per-N units compile in parallel and
// every kernel has N fixed at compile time (register arrays are indexed
// statically).
#include "ep_device.hpp"

#ifndef EP_N
#error "compile with -DEP_N=<episode size>"
#endif

namespace epk {
namespace {

// One lane holding all N machines of a (segment, episode) is built up to N = 8.
constexpr int kMaxClassNodes = 8;
constexpr int kClassMch = EP_N <= kMaxClassNodes ? EP_N : 1;

template <class Mach>
hipError_t launch_scan_m(const MapArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((map_scan_kernel<EP_N, Mach>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan(const MapArgs& a, int win, dim3 grid, dim3 block, hipStream_t s) {
  switch (win) {
    case kRuns1: return launch_scan_m<RunMachine<EP_N, 1>>(a, grid, block, s);
    case kRuns2: return launch_scan_m<RunMachine<EP_N, 2>>(a, grid, block, s);
    case kRuns4: return launch_scan_m<RunMachine<EP_N, 4>>(a, grid, block, s);
    case kRing: return launch_scan_m<RingMachine<EP_N>>(a, grid, block, s);
    default: return hipErrorInvalidValue;
  }
}

template <int W, int MCH>
hipError_t launch_bits_wm(const MapArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((map_bits_kernel<EP_N, W, MCH>), grid, block, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_bits(const MapArgs& a, int win, bool all_machines, dim3 grid, dim3 block,
                       size_t lds, hipStream_t s) {
  if (all_machines && EP_N > kMaxClassNodes) return hipErrorInvalidValue;
  if (win == kBits32)
    return all_machines ? launch_bits_wm<32, kClassMch>(a, grid, block, lds, s)
                        : launch_bits_wm<32, 1>(a, grid, block, lds, s);
  if (win == kBits64)
    return all_machines ? launch_bits_wm<64, kClassMch>(a, grid, block, lds, s)
                        : launch_bits_wm<64, 1>(a, grid, block, lds, s);
  return hipErrorInvalidValue;
}

template <int W, int MCH>
hipError_t launch_list_wm(const MapArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  if (a.lazy)
    hipLaunchKernelGGL((map_list_kernel<EP_N, W, MCH, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((map_list_kernel<EP_N, W, MCH, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_list(const MapArgs& a, int win, bool all_machines, dim3 grid, dim3 block,
                       hipStream_t s) {
  if (all_machines && EP_N > kMaxClassNodes) return hipErrorInvalidValue;
  if (win == kBits32)
    return all_machines ? launch_list_wm<32, kClassMch>(a, grid, block, s)
                        : launch_list_wm<32, 1>(a, grid, block, s);
  if (win == kBits64)
    return all_machines ? launch_list_wm<64, kClassMch>(a, grid, block, s)
                        : launch_list_wm<64, 1>(a, grid, block, s);
  return hipErrorInvalidValue;
}

hipError_t launch_ticks(const MapArgs& a, bool all_machines, dim3 grid, dim3 block, size_t lds,
                        hipStream_t s) {
  if (all_machines && EP_N > kMaxClassNodes) return hipErrorInvalidValue;
  if (all_machines)
    hipLaunchKernelGGL((map_ticks_kernel<EP_N, kClassMch>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((map_ticks_kernel<EP_N, 1>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <class Mach>
hipError_t launch_closure_m(const ClosureArgs& a, dim3 grid, hipStream_t s) {
  if (a.queue_cap > 0)
    hipLaunchKernelGGL((closure_kernel<EP_N, Mach, false>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((closure_kernel<EP_N, Mach, true>), grid, dim3(kBlock), 0, s, a);
  if (a.queue_cap > 0)  // the queued repairs, pulled one per wave
    hipLaunchKernelGGL((repair_kernel<EP_N, Mach>), dim3((unsigned)a.repair_blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_closure(const ClosureArgs& a, int win, dim3 grid, hipStream_t s) {
  switch (win) {
    case kRuns1: return launch_closure_m<RunMachine<EP_N, 1>>(a, grid, s);
    case kRuns2: return launch_closure_m<RunMachine<EP_N, 2>>(a, grid, s);
    case kRuns4: return launch_closure_m<RunMachine<EP_N, 4>>(a, grid, s);
    case kBits32: return launch_closure_m<BitMachine<EP_N, 32>>(a, grid, s);
    case kBits64: return launch_closure_m<BitMachine<EP_N, 64>>(a, grid, s);
    case kRing: return launch_closure_m<RingMachine<EP_N>>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <class Mach>
hipError_t launch_finish_m(const FallbackArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((finish_kernel<Mach>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finish(const FallbackArgs& a, int win, dim3 grid, hipStream_t s) {
  switch (win) {
    case kRuns1: return launch_finish_m<RunMachine<EP_N, 1>>(a, grid, s);
    case kRuns2: return launch_finish_m<RunMachine<EP_N, 2>>(a, grid, s);
    case kRuns4: return launch_finish_m<RunMachine<EP_N, 4>>(a, grid, s);
    case kBits32: return launch_finish_m<BitMachine<EP_N, 32>>(a, grid, s);
    case kBits64: return launch_finish_m<BitMachine<EP_N, 64>>(a, grid, s);
    case kRing: return launch_finish_m<RingMachine<EP_N>>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <class Mach>
hipError_t launch_reduce_m(const ReduceArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((reduce_kernel<EP_N, Mach>), grid, block, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int win, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  switch (win) {
    case kRuns1: return launch_reduce_m<RunMachine<EP_N, 1>>(a, grid, block, lds, s);
    case kRuns2: return launch_reduce_m<RunMachine<EP_N, 2>>(a, grid, block, lds, s);
    case kRuns4: return launch_reduce_m<RunMachine<EP_N, 4>>(a, grid, block, lds, s);
    case kBits32: return launch_reduce_m<BitMachine<EP_N, 32>>(a, grid, block, lds, s);
    case kBits64: return launch_reduce_m<BitMachine<EP_N, 64>>(a, grid, block, lds, s);
    case kRing: return launch_reduce_m<RingMachine<EP_N>>(a, grid, block, lds, s);
    default: return hipErrorInvalidValue;
  }
}

template <class Mach>
hipError_t launch_stream_m(const StreamArgs& a, bool tail, dim3 grid, hipStream_t s) {
  if (tail)
    hipLaunchKernelGGL((stream_tail_kernel<EP_N, Mach>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((stream_entry_kernel<EP_N, Mach>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamArgs& a, int win, bool tail, dim3 grid, hipStream_t s) {
  switch (win) {
    case kRuns1: return launch_stream_m<RunMachine<EP_N, 1>>(a, tail, grid, s);
    case kRuns2: return launch_stream_m<RunMachine<EP_N, 2>>(a, tail, grid, s);
    case kRuns4: return launch_stream_m<RunMachine<EP_N, 4>>(a, tail, grid, s);
    case kBits32: return launch_stream_m<BitMachine<EP_N, 32>>(a, tail, grid, s);
    case kBits64: return launch_stream_m<BitMachine<EP_N, 64>>(a, tail, grid, s);
    case kRing: return launch_stream_m<RingMachine<EP_N>>(a, tail, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_entry(const StreamArgs& a, int win, dim3 grid, hipStream_t s) {
  return launch_stream(a, win, false, grid, s);
}

hipError_t launch_stream_tail(const StreamArgs& a, int win, dim3 grid, hipStream_t s) {
  return launch_stream(a, win, true, grid, s);
}

template <class F>
hipError_t occ(F f, int block, size_t lds, int* out) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, f, block, lds);
}

hipError_t occupancy(int win, bool all_machines, int block, size_t lds, int* out) {
  if (all_machines && EP_N > kMaxClassNodes) return hipErrorInvalidValue;
  switch (win) {
    case kRuns1: return occ(map_scan_kernel<EP_N, RunMachine<EP_N, 1>>, block, 0, out);
    case kRuns2: return occ(map_scan_kernel<EP_N, RunMachine<EP_N, 2>>, block, 0, out);
    case kRuns4: return occ(map_scan_kernel<EP_N, RunMachine<EP_N, 4>>, block, 0, out);
    case kRing: return occ(map_scan_kernel<EP_N, RingMachine<EP_N>>, block, 0, out);
    case kBits32:
      return all_machines ? occ(map_bits_kernel<EP_N, 32, kClassMch>, block, lds, out)
                          : occ(map_bits_kernel<EP_N, 32, 1>, block, lds, out);
    case kBits64:
      return all_machines ? occ(map_bits_kernel<EP_N, 64, kClassMch>, block, lds, out)
                          : occ(map_bits_kernel<EP_N, 64, 1>, block, lds, out);
    default: return hipErrorInvalidValue;
  }
}

hipError_t occupancy_ticks(bool all_machines, int block, size_t lds, int* out) {
  if (all_machines && EP_N > kMaxClassNodes) return hipErrorInvalidValue;
  return all_machines ? occ(map_ticks_kernel<EP_N, kClassMch>, block, lds, out)
                      : occ(map_ticks_kernel<EP_N, 1>, block, lds, out);
}

const Launchers kLaunchers = {launch_scan,         launch_bits,        launch_ticks,
                              launch_list,         launch_closure,     launch_finish,
                              launch_reduce,       launch_stream_entry, launch_stream_tail,
                              occupancy,           occupancy_ticks};

}  // namespace

#define EPK_CAT2(a, b) a##b
#define EPK_CAT(a, b) EPK_CAT2(a, b)
const Launchers* EPK_CAT(launchers_n, EP_N)() { return &kLaunchers; }

}  // namespace epk

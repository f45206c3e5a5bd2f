// Device-resident Philox state for calls that run inside a captured HIP graph.
//
// The PyTorch PR "REDO of dropout support for mem eff" (Summary) changes how
// the RNG state passes from forward to backward in order to allow CUDA-graph
// capture.  Here a call may keep {seed, offset} in device memory instead of
// the library's host state: a one-thread kernel ahead of the forward copies
// the state into the call's own {seed, offset} buffer (which the forward, and
// later the backward, read) and advances the state's offset, all in stream
// order, so every replay of a captured graph draws fresh bits.
#include "kernels.h"

namespace sdpa14 {
namespace {

__global__ __launch_bounds__(64) void rng_step_kernel(uint64_t* state, uint64_t* used,
                                                      uint64_t advance) {
  if (threadIdx.x != 0) return;
  const uint64_t seed = state[0], offset = state[1];
  used[0] = seed;
  used[1] = offset;
  state[1] = offset + advance;
}

}  // namespace

hipError_t launch_rng_step(uint64_t* state, uint64_t* used, uint64_t advance,
                           hipStream_t stream) {
  hipLaunchKernelGGL(rng_step_kernel, dim3(1), dim3(64), 0, stream, state, used, advance);
  return hipGetLastError();
}

}  // namespace sdpa14

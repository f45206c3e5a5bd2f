// The backward main kernel at head dim 128 (kernels in bwd_kernels.h).
//
// A translation unit of its own so that it can be compiled with the
// iterative-ILP instruction scheduler: at head dim 128 the kernel holds one
// wave per SIMD (its registers and LDS allow no more), and that schedule,
// which trades registers for instruction-level parallelism, measured 10%
// faster there (2070 against 2306 us at b1 h32 q4096 k8192 d128, outputs
// bitwise the same), while at head dim 64, where two waves share a SIMD, the
// default schedule is faster.
#include "bwd_kernels.h"

namespace sdpa14 {

hipError_t launch_bwd_main_e128(const BwdParams& p, bool causal, bool dropout, bool f16,
                                const TileChoice& tiles, hipStream_t stream) {
  return f16 ? launch_main_t<128, true>(p, causal, dropout, tiles, stream)
             : launch_main_t<128, false>(p, causal, dropout, tiles, stream);
}

}  // namespace sdpa14

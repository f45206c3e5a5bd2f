// Backward launchers.  The kernels are in bwd_kernels.h; the head-dim-128
// main kernel is instantiated in bwd_e128.hip.
#include "bwd_kernels.h"

namespace sdpa14 {

size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t Sq) {
  const size_t raw = (size_t)B * (size_t)H * (size_t)Sq * 8u;
  return (raw + 255u) & ~(size_t)255u;
}

hipError_t launch_bwd_rows(const BwdParams& p, bool f16, hipStream_t stream) {
  const int E = tile_head_dim(p.E);
  if (f16) return E == 64 ? launch_rows_t<64, true>(p, stream) : launch_rows_t<128, true>(p, stream);
  return E == 64 ? launch_rows_t<64, false>(p, stream) : launch_rows_t<128, false>(p, stream);
}

hipError_t launch_bwd_main(const BwdParams& p, bool causal, bool dropout, bool f16,
                           const TileChoice& tiles, hipStream_t stream) {
  const int E = tile_head_dim(p.E);
  if (E == 128) return launch_bwd_main_e128(p, causal, dropout, f16, tiles, stream);
  return f16 ? launch_main_t<64, true>(p, causal, dropout, tiles, stream)
             : launch_main_t<64, false>(p, causal, dropout, tiles, stream);
}

}  // namespace sdpa14

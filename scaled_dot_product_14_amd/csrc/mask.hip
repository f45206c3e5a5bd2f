// Writes the dropout keep mask as bytes, through the same device Philox code
// and counter arithmetic the attention kernels use.  For tests of the mask
// contract only; the attention kernels never read this buffer.
#include "kernels.h"

namespace sdpa14 {
namespace {

__global__ __launch_bounds__(256) void mask_kernel(MaskParams p) {
  const int sk4 = (p.Sk + 3) >> 2;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.H * p.Sq * sk4;
  if (t >= total) return;
  const int64_t row = t / sk4;  // (b*H + h)*Sq + i
  const int grp = (int)(t - row * sk4);
  const int bh = (int)(row / p.Sq);
  const int i = (int)(row - (int64_t)bh * p.Sq);
  const uint64_t ctr = philox_row_base(p.drop, bh, p.Sq, i, sk4) + (uint32_t)grp;
  const PhiloxOut w = philox4x32_10(ctr, p.drop.seed_lo, p.drop.seed_hi);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = 4 * grp + u;
    if (j < p.Sk) p.mask[row * p.Sk + j] = (w.w[u] >= p.drop.threshold) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_mask(const MaskParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.B * p.H * p.Sq * ((p.Sk + 3) / 4);
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(mask_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sdpa14

// Philox-4x32-10 on the device, and the dropout keep test built on it.
//
// Generator: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3" (SC'11).  Each round forms the two 32x32->64-bit products of
// counter words 0 and 2 with fixed odd multipliers; the new counter is
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).  The key words advance by two Weyl
// constants between rounds.
//
// Use for dropout: the PyTorch PR "REDO of dropout support for mem eff"
// (Summary) hands the RNG state from forward to backward and indexes the
// stream by the absolute position of each score element.  Here one call
// covers four consecutive keys j = 4c..4c+3 of query row i of head (b, h):
// counter = offset + ((b*H + h)*Sq + i) * ceil(Sk/4) + c, key = seed, and key
// j takes output word j % 4.  For a call on a slice of the heads, H is the
// head count of the whole problem and h the global head index, the sharded
// dropout the nvFuser PR "DID loop split for SDPA" leaves open (its test keeps
// p = 0 pending sharded dropout support).  An element is kept iff its word is >= the
// threshold floor(p * 2^32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa14 {

struct PhiloxOut {
  uint32_t w[4];
};

// a ^ b ^ k in one VALU instruction (three-input bitwise op, truth table 0x96);
// k is wave-uniform (a key word).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

__device__ __forceinline__ PhiloxOut philox4x32_10(uint64_t counter, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
  uint32_t c0 = static_cast<uint32_t>(counter);
  uint32_t c1 = static_cast<uint32_t>(counter >> 32);
  uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    // Each 32x32 -> 64-bit product is one v_mad_u64_u32 (high and low words at once).
    const uint64_t p0 = static_cast<uint64_t>(kM0) * c0, p1 = static_cast<uint64_t>(kM1) * c2;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    const uint32_t n0 = xor3(hi1, c1, k0);
    const uint32_t n2 = xor3(hi0, c3, k1);
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  PhiloxOut o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// Dropout parameters shared by the kernels.
struct DropoutParams {
  uint64_t offset;        // Philox offset of this forward call
  uint32_t seed_lo;       // key word 0
  uint32_t seed_hi;       // key word 1
  uint32_t threshold;     // floor(p * 2^32); keep iff word >= threshold
  float keep_scale;       // 1 / (1 - p), rounded to fp32 on the host
  int32_t heads_total;    // heads of the unsharded problem (the call's H when not sharded)
  int32_t head_offset;    // global index of the call's head 0
  const uint64_t* state;  // device {seed, offset} of the call, or null: the fields above
};

// Global index, in the random stream, of the call's head h of batch b.  A call
// on a slice of the heads then draws the mask the whole problem would.
__device__ __forceinline__ int dropout_head(const DropoutParams& d, int b, int h) {
  return b * d.heads_total + d.head_offset + h;
}

// Takes seed and offset from device memory when the call keeps them there
// (a captured graph then draws fresh bits on every replay).
__device__ __forceinline__ void load_dropout_state(DropoutParams& d) {
  if (d.state != nullptr) {
    const uint64_t seed = d.state[0], offset = d.state[1];
    d.seed_lo = static_cast<uint32_t>(seed);
    d.seed_hi = static_cast<uint32_t>(seed >> 32);
    d.offset = offset;
  }
}

// Counter of query row `row` of global head `bhg` (dropout_head) for key group
// 0; key group c adds c.
__device__ __forceinline__ uint64_t philox_row_base(const DropoutParams& d, int bhg, int Sq,
                                                    int row, int sk4) {
  return d.offset + (static_cast<uint64_t>(bhg) * static_cast<uint64_t>(Sq) +
                     static_cast<uint64_t>(row)) * static_cast<uint64_t>(sk4);
}

}  // namespace sdpa14

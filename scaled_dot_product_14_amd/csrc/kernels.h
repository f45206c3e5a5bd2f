// Kernel parameter blocks and launchers shared by the C ABI layer and the
// kernel translation units.  Host-visible; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "philox.h"

namespace sdpa14 {

// Element strides of a logical [B, H, S, E] tensor (E has unit stride).
struct Strides {
  int64_t b, h, s;
};

struct FwdParams {
  const uint16_t* q;  // bf16 bits
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // contiguous [B, H, Sq], or null (inference: not written)
  Strides sq, sk, sv, so;
  int B, H, Sq, Sk;
  int E;             // head dim of the tensors, at most the kernel's tile head dim;
                     // columns past it read as zeros and are never stored
  float scale_log2;  // scale * log2(e)
  DropoutParams drop;
  const uint16_t* bias;  // additive bias [B, H, Sq, Sk] (bf16 bits, unit key stride), or null
  Strides sbias;         // its strides (0 for a broadcast dimension)
  uint32_t* keep;        // dropout keep bits [B, H, Sq, keep_w] words to write, or null
  int keep_w;            // words per row: ceil(Sk / 32) rounded up to a multiple of 4
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const float* lse;  // contiguous [B, H, Sq]
  float* dl;         // workspace: -D_i plane then LSE_i*log2(e) - log2(scale) plane, each [B, H, Sq]
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int B, H, Sq, Sk;
  int E;             // head dim of the tensors (as in FwdParams)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  DropoutParams drop;
  const uint16_t* bias;  // as in FwdParams
  Strides sbias;
  const uint32_t* keep;  // keep bits written by the forward, or null: regenerate
  int keep_w;
  uint16_t* dbias;       // bias gradient [B, H, Sq, Sk] (needs bias), or null: not computed
  Strides sdbias;
};

struct MaskParams {
  uint8_t* mask;  // [B, H, Sq, Sk] bytes
  int B, H, Sq, Sk;
  DropoutParams drop;
};

// Tile choices the launchers take; 0 lets the launcher decide.
struct TileChoice {
  int fwd_shape;  // forward workgroup: 1 = 4 query sub-tiles, 2 = 2 sub-tiles x 2 key
                  // shares, 3 = 1 sub-tile x 4 key shares (32 query rows per sub-tile),
                  // 4 = causal split launch (kinds 3 with 32-key tiles and 2, head dim 64)
  int bwd_roles;  // backward main pass: 1 = both roles in one launch, 2 = dK/dV and dQ
                  // blocks as two launches (no dropout, no bias; else one launch)
  int bwd_order;  // backward dispatch order: 1 = the arithmetic order that problems past
                  // the order table's size use, whatever the size
  int fwd_order;  // split forward: 1 = the default workgroup order, no dispatch table
};

// Tile head dim of the kernels that run head dim E (a multiple of 8, at most 128).
inline int tile_head_dim(int E) { return E <= 64 ? 64 : 128; }
// f16: the 16-bit tensors are IEEE half instead of bfloat16.  p.E is the head
// dim; the kernels run at tile_head_dim(p.E).
hipError_t launch_fwd(const FwdParams& p, bool causal, bool dropout, bool f16,
                      const TileChoice& tiles, hipStream_t stream);
// Backward: the row pass filling p.dl (which must hold bwd_workspace_bytes(B,
// H, Sq) bytes), then the main kernel, launched in that order on one stream.
hipError_t launch_bwd_rows(const BwdParams& p, bool f16, hipStream_t stream);
hipError_t launch_bwd_main(const BwdParams& p, bool causal, bool dropout, bool f16,
                           const TileChoice& tiles, hipStream_t stream);
// The main kernel at tile head dim 128 (its own translation unit).
hipError_t launch_bwd_main_e128(const BwdParams& p, bool causal, bool dropout, bool f16,
                                const TileChoice& tiles, hipStream_t stream);
size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t Sq);
// Words per row of the keep-bit cache: bit j % 32 of word j / 32 is key j's bit.
inline int keep_words(int64_t Sk) { return (int)(((Sk + 31) / 32 + 3) / 4 * 4); }
hipError_t launch_mask(const MaskParams& p, hipStream_t stream);
// One thread: used[0..1] = state[0..1], then state[1] += advance.
hipError_t launch_rng_step(uint64_t* state, uint64_t* used, uint64_t advance,
                           hipStream_t stream);

}  // namespace sdpa14

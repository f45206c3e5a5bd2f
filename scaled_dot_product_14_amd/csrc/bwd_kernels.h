// Fused attention backward for gfx950, recomputing the probabilities from the
// stashed log-sum-exp (nvFuser issue 2278: what the forward stashes is chosen
// by what the backward needs; here O and LSE are stashed and P is recomputed).
// The backward statement follows sdpfa_bwd of the nvFuser PR "DID loop split
// for SDPA"; dropout regenerates the forward's mask from (seed, offset) and the
// absolute element index (PyTorch PR "REDO of dropout support for mem eff").
//
// Two launches, no atomics:
//
//   prep        one pass over the rows: D_i = rowsum(dO * O) and the row's
//               LSE*log2(e) - log2(scale), stored as a float pair per row in
//               the caller's workspace.
//   main        two workgroup roles.
//     dK/dV role  a 64-key block: waves (sb, qs), sb = 32-key sub-block, qs =
//                 which of the two 32-row query tiles of an iteration.  Each
//                 wave keeps its sub-block's K and V fragments and its dK^T,
//                 dV^T accumulators in registers.  Per query tile:
//                   S = Q K^T, dPd = dO V^T          (lane = key, registers = rows)
//                   Ps = scale * exp(S*scale - LSE)  (masked; dropout kept/scaled)
//                   dS' = Ps * (dP - D)
//                   dV^T += dO^T Pd, dK^T += Q^T dS' (dO^T, Q^T read transposed)
//                 With a bias gradient asked for, the role also stores
//                 dS = Ps * (dP - D) / scale for its block: it meets every
//                 (row, key) of the block exactly once, and writes zeros for
//                 the rows a causal mask hides from all of the block's keys.
//     dQ role     a 64-row block: waves (qsb, ks), qsb = 32-row sub-block, ks =
//                 which of the two 32-key tiles of an iteration.  Each wave
//                 keeps its rows' Q and dO fragments, D and LSE in registers.
//                 Per key tile: S^T = K Q^T, dP^T = V dO^T (lane = row), dS'^T
//                 as above, dQ^T += K^T dS'^T with K^T read transposed.
//               The tiles a workgroup streams (Q and dO, or K and V) go straight
//               from memory to LDS (buffer loads with the LDS destination), into
//               a ring of three stages filled two iterations ahead, so neither
//               registers nor VALU work are spent on staging and the memory
//               latency is covered by two iterations of math.  The two waves of
//               a sub-block are summed through LDS at the end; each finalizes
//               half of the outputs.
//
// The kernels and their launch templates live in this header; bwd.hip
// instantiates them for head dim 64 and the row pass, bwd_e128.hip the main
// kernel for head dim 128 (compiled with its own instruction scheduler).
//
// Both roles recompute S and dP, so the backward does 7 products of 2*E flops
// per visible score element (5 are counted).  In exchange dQ needs neither
// fp32 atomics nor a zeroed accumulator nor a conversion pass, and every output
// is bitwise reproducible.
#pragma once

#include <algorithm>
#include <vector>

#include "device_common.h"
#include "kernels.h"
#include "lds_ring.h"
#include "occupancy.h"

namespace sdpa14 {
namespace {

// Bytes of one (batch, head) slice of the bias, rounded up to whole 8-byte
// granules: a partially valid dword would otherwise read as zero under the
// buffer range check.  The rounding stays inside the granule holding the last
// element, so it never reaches another page.
template <typename P>
__device__ __forceinline__ uint32_t bias_bytes(const P& p) {
  const int64_t b = ((int64_t)(p.Sq - 1) * p.sbias.s + p.Sk) * 2;
  return (uint32_t)((b + 7) & ~int64_t(7));
}

// Bytes of one (batch, head) slice of the bias gradient.
template <typename P>
__device__ __forceinline__ uint32_t dbias_bytes(const P& p) {
  return (uint32_t)(((int64_t)(p.Sq - 1) * p.sdbias.s + p.Sk) * 2);
}

constexpr float kLog2e = 1.44269504088896340736f;

template <int E, bool BIAS, bool KEEP>
struct BwdCfg {
  static constexpr int NES = E / 16;  // 16-wide contraction steps over E
  static constexpr int NEB = E / 32;  // 32-wide output blocks over E
  static constexpr int CPR = E / 8;   // 16-byte chunks per row
  static constexpr int ROW_B = 2 * E;
  static constexpr int TILE_B = 32 * ROW_B;
  static constexpr int NLD = TILE_B / (256 * 16);  // LDS-DMA loads per thread per tile
  static_assert(NLD == E / 64, "tile loads");
  static constexpr int DL_B = 64 * 8;              // -D and L of the pair's 64 rows
  // With a bias, each stage also holds the 64 x 64 block of it that the step
  // needs (rows of 128 bytes, laid out like a head-dim-64 tile), 2 loads per thread.
  static constexpr int BIAS_B = BIAS ? 64 * 128 : 0;
  static constexpr int NBL = BIAS ? 2 : 0;
  // With the forward's keep bits, each stage holds 16 bytes (four 32-key words)
  // of each of its 64 rows, one load by 16 lanes of each wave.
  static constexpr int KEEP_B = KEEP ? 64 * 16 : 0;
  static constexpr int NKL = KEEP ? 1 : 0;
  static constexpr int STAGE_A = 4 * TILE_B + DL_B + BIAS_B + KEEP_B;  // Q, Q', dO, dO', -D, L, bias, bits
  static constexpr int STAGE_B = 4 * TILE_B + BIAS_B + KEEP_B;         // K, K', V, V', bias, bits
  static constexpr int NSTAGE = 3;
  static constexpr int NPAIR_A = 4 * NLD + 1 + NBL + NKL;  // loads per thread per stage, dK/dV role
  static constexpr int NPAIR_B = 4 * NLD + NBL + NKL;      // loads per thread per stage, dQ role
  static constexpr int RED_B = 4 * NEB * 16 * 64 * 4;  // end-of-block exchange
  static constexpr int LDS_B = NSTAGE * STAGE_A;
  // The dQ role's stage 2 also takes the block's (D, L) in the prologue.
  static_assert(STAGE_A >= STAGE_B + DL_B && LDS_B >= RED_B, "LDS budget");
};

// Loads rows row0 .. row0+63 of x and of y, two 32-row tiles each, into a
// stage laid out [x rows 0-31][x rows 32-63][y rows 0-31][y rows 32-63].  ox,
// oy are the thread's dma_src_offset values; x_row, y_row the row strides in bytes.
template <int E>
__device__ __forceinline__ void issue_tiles(unsigned char* st, int wave, uint32_t row0,
                                            __amdgpu_buffer_rsrc_t rx, uint32_t x_row,
                                            const uint32_t (&ox)[E / 64],
                                            __amdgpu_buffer_rsrc_t ry, uint32_t y_row,
                                            const uint32_t (&oy)[E / 64]) {
  constexpr int TILE_B = 64 * E, NLD = E / 64;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t r = row0 + 32u * half;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      dma16(rx, st + half * TILE_B + k * 4096 + wave * 1024, r * x_row + ox[k]);
      dma16(ry, st + (2 + half) * TILE_B + k * 4096 + wave * 1024, r * y_row + oy[k]);
    }
  }
}

// Dropout keep bits for the dK/dV role (bhg: the global head, dropout_head).
// The lane holds key `key` (key % 4 ==
// lane % 4) and, for register group c, the four rows row0 + u, u = 0..3.  Lane t
// of each quad evaluates the Philox call of row row0 + t for the key group of
// the quad (four words: keys 4*(key/4) + 0..3), packs the four keep bits, and
// every lane collects its own key's bit from the four lanes of its quad.
// Returns bit u = keep(row0 + u, key).
__device__ __forceinline__ uint32_t keep_bits_for_key(const DropoutParams& d, int bhg, int Sq,
                                                      int sk4, int row0, int key, int lane) {
  const int t = lane & 3;
  const uint64_t ctr = philox_row_base(d, bhg, Sq, row0 + t, sk4) + (uint32_t)(key >> 2);
  const PhiloxOut w = philox4x32_10(ctr, d.seed_lo, d.seed_hi);
  const int nib = (w.w[0] >= d.threshold ? 1 : 0) | (w.w[1] >= d.threshold ? 2 : 0) |
                  (w.w[2] >= d.threshold ? 4 : 0) | (w.w[3] >= d.threshold ? 8 : 0);
  const int n0 = __builtin_amdgcn_mov_dpp(nib, 0x00, 0xF, 0xF, false);  // quad lane 0
  const int n1 = __builtin_amdgcn_mov_dpp(nib, 0x55, 0xF, 0xF, false);  // quad lane 1
  const int n2 = __builtin_amdgcn_mov_dpp(nib, 0xAA, 0xF, 0xF, false);  // quad lane 2
  const int n3 = __builtin_amdgcn_mov_dpp(nib, 0xFF, 0xF, 0xF, false);  // quad lane 3
  return ((n0 >> t) & 1) | (((n1 >> t) & 1) << 1) | (((n2 >> t) & 1) << 2) |
         (((n3 >> t) & 1) << 3);
}

// End-of-block exchange between the two waves of a sub-block.  Each wave
// holds NEB accumulator blocks (C layout: lane = output row row0 + l32,
// register r of block eb = column 32*eb + 8*(r/4) + 4*g + r%4).  The wave with
// `upper` set finalizes blocks NEB/2 .. NEB-1, the other blocks 0 .. NEB/2-1.
// exchange_put writes the half the partner finalizes into this wave's slot;
// after a barrier, exchange_finish adds the partner's slot, scales by mul and
// stores bf16 rows below `limit`.
template <int E>
__device__ __forceinline__ void exchange_put(const f32x16 (&acc)[E / 32], float* red, int slot,
                                             bool upper, int lane) {
  constexpr int HALF = E / 64;
  f32x4* buf = reinterpret_cast<f32x4*>(red + slot * (HALF * 16 * 64));
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const int eb = upper ? i : HALF + i;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      f32x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = acc[eb][4 * cg + t];
      buf[(i * 4 + cg) * 64 + lane] = v;
    }
  }
}

template <int E, bool F16>
__device__ __forceinline__ void exchange_finish(const f32x16 (&acc)[E / 32], float mul,
                                                uint16_t* dst, int64_t stride, int row0,
                                                int limit, int e_real, const float* red,
                                                int partner_slot, bool upper, int lane) {
  constexpr int HALF = E / 64;
  const f32x4* buf = reinterpret_cast<const f32x4*>(red + partner_slot * (HALF * 16 * 64));
  const int row = row0 + (lane & 31);
  const int g = lane >> 5;
  if (row >= limit) return;
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const int eb = upper ? HALF + i : i;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      const f32x4 o = buf[(i * 4 + cg) * 64 + lane];
      const int e = eb * 32 + 8 * cg + 4 * g;
      if (e >= e_real) continue;  // a column past the tensors' head dim
      *reinterpret_cast<uint2*>(dst + (int64_t)row * stride + e) =
          pack16x4<F16>((acc[eb][4 * cg + 0] + o[0]) * mul, (acc[eb][4 * cg + 1] + o[1]) * mul,
                      (acc[eb][4 * cg + 2] + o[2]) * mul, (acc[eb][4 * cg + 3] + o[3]) * mul);
    }
  }
}

// ---------------------------------------------------------------------------
template <int E, bool CAUSAL, bool DROPOUT, bool BIAS, bool F16, bool KEEP, bool DBIAS>
__device__ __forceinline__ void role_dkdv(const BwdParams& p, int bh, int kblk,
                                          unsigned char* lds) {
  using C = BwdCfg<E, BIAS, KEEP>;
  constexpr int NES = C::NES, NEB = C::NEB, NLD = C::NLD, TILE_B = C::TILE_B;
  constexpr int ST_Q = 0, ST_DO = 2 * TILE_B, ST_DL = 4 * TILE_B, ST_BIAS = ST_DL + C::DL_B;
  constexpr int ST_KEEP = ST_BIAS + C::BIAS_B;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int sb = wave & 1, qs = wave >> 1;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int kb0 = kblk * 64;
  const int kbs = kb0 + 32 * sb;  // first key of this wave's sub-block
  const int key = kbs + l32;
  const float c = p.scale_log2;
  DropoutParams drop = p.drop;
  if (DROPOUT) load_dropout_state(drop);
  const int bhg = dropout_head(drop, b, h);

  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(p.q + b * p.sq.b + h * p.sq.h, p.Sq, p.sq.s, p.E);
  const __amdgpu_buffer_rsrc_t rdo =
      rows_rsrc(p.dout + b * p.sdo.b + h * p.sdo.h, p.Sq, p.sdo.s, p.E);
  // Waves 0, 1 stage rows of -D, waves 2, 3 rows of L (workspace planes).
  const __amdgpu_buffer_rsrc_t rdl = make_rsrc(
      p.dl + (wave >> 1) * ((int64_t)p.B * p.H * p.Sq) + (int64_t)bh * p.Sq, (uint32_t)p.Sq * 4u);
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(p.k + b * p.sk.b + h * p.sk.h, p.Sk, p.sk.s, p.E);
  const __amdgpu_buffer_rsrc_t rvv = rows_rsrc(p.v + b * p.sv.b + h * p.sv.h, p.Sk, p.sv.s, p.E);

  f32x16 dva[NEB], dka[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    dva[eb] = zero16();
    dka[eb] = zero16();
  }

  const int nqt = (p.Sq + 31) / 32;
  const int t0 = CAUSAL ? min(kb0 / 32, nqt) : 0;
  const int n_it = (nqt - t0 + 1) / 2;

  // Keep bits from the forward: stage it holds, for each of its 64 rows, the
  // 16-byte chunk of words that contains this workgroup's two 32-key words.
  __amdgpu_buffer_rsrc_t rkeep = make_rsrc(p.q, 0u);
  uint32_t okeep = 0u;
  if (KEEP) {
    rkeep = make_rsrc(p.keep + (int64_t)bh * p.Sq * p.keep_w, (uint32_t)(p.Sq * p.keep_w * 4));
    okeep = (uint32_t)((wave * 16 + (lane & 15)) * p.keep_w * 4 + (kblk >> 1) * 16);
  }
  // Additive bias: stage it also holds the bias block of its 64 query rows x
  // this workgroup's 64 keys; a lane reads its key's values for rows
  // 8*cg + 4*g + 0..3 with one transposed read per register group.
  __amdgpu_buffer_rsrc_t br = make_rsrc(p.q, 0u);
  uint32_t obias[2] = {0u, 0u};
  if (BIAS) {
    br = make_rsrc(p.bias + b * p.sbias.b + h * p.sbias.h, bias_bytes(p));
#pragma unroll
    for (int k = 0; k < 2; ++k) obias[k] = dma_src_offset<64>(k, tid, p.sbias.s) + (uint32_t)kb0 * 2u;
  }
  // Bias gradient: element (row, key) goes to byte offset 2 * (row * sdb + key)
  // of the head's slice.  A lane's register r holds row q0 + 8*(r/4) + 4*g +
  // r%4 of its key: the lane part (4*g rows, the key) is a vector offset, the
  // rest a wave-uniform scalar offset per store.
  __amdgpu_buffer_rsrc_t rdb = make_rsrc(p.q, 0u);
  uint32_t odb = 0u, sdb2 = 0u;
  const float inv_scale = 1.f / p.scale;
  if (DBIAS) {
    rdb = make_rsrc(p.dbias + b * p.sdbias.b + h * p.sdbias.h, dbias_bytes(p));
    sdb2 = (uint32_t)p.sdbias.s * 2u;
    odb = (uint32_t)(4 * g) * sdb2 + (uint32_t)key * 2u;
  }

  // Stage it % 3 of the ring holds query tiles t0 + 2*it and t0 + 2*it + 1.
  uint32_t oq[NLD], odo[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    oq[k] = dma_src_offset_e<E>(k, tid, p.sq.s, p.E);
    odo[k] = dma_src_offset_e<E>(k, tid, p.sdo.s, p.E);
  }
  // Load idx (0 .. NPAIR_A-1) of stage it: (half, tensor, k) for the Q and dO
  // tiles, then -D (waves 0, 1) and L (waves 2, 3) of the pair's 64 rows, then
  // the two loads of the bias block.
  auto issue_one = [&](int it, int idx, float after) {
    unsigned char* st = lds + ring_offset<C::STAGE_A>(it);
    const uint32_t row0 = (uint32_t)((t0 + 2 * it) * 32);
    if (idx < 4 * NLD) {
      const int half = idx / (2 * NLD), tensor = (idx / NLD) & 1, k = idx % NLD;
      const uint32_t r = row0 + 32u * half;
      unsigned char* dst = st + (tensor ? ST_DO : ST_Q) + half * TILE_B + k * 4096 + wave * 1024;
      if (tensor)
        dma16_after(rdo, dst, r * (uint32_t)(p.sdo.s * 2) + odo[k], after);
      else
        dma16_after(rq, dst, r * (uint32_t)(p.sq.s * 2) + oq[k], after);
    } else if (idx == 4 * NLD) {
      if (lane < 8)
        dma16_after(rdl, st + ST_DL + wave * 128,
                    row0 * 4u + (uint32_t)((wave & 1) * 128 + lane * 16), after);
    } else if (BIAS && idx < 4 * NLD + 1 + C::NBL) {
      const int k = idx - 4 * NLD - 1;
      dma16_after(br, st + ST_BIAS + k * 4096 + wave * 1024,
                  row0 * (uint32_t)(p.sbias.s * 2) + obias[k], after);
    } else if (lane < 16) {
      dma16_after(rkeep, st + ST_KEEP + wave * 256, row0 * (uint32_t)(p.keep_w * 4) + okeep, after);
    }
  };
  // The loads of a stage are spread over the step in NSLOT groups, each placed
  // after a value of the step's math, so the vector-memory queue drains while
  // the wave computes (a burst of them stalls the issuing wave).
  constexpr int NSLOT = 5;
  auto issue_slot = [&](int it, int slot, float after) {
#pragma unroll
    for (int idx = slot * C::NPAIR_A / NSLOT; idx < (slot + 1) * C::NPAIR_A / NSLOT; ++idx)
      issue_one(it, idx, after);
  };
  auto issue = [&](int it) {
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) issue_slot(it, slot, 0.f);
  };

  // Per-lane LDS offsets within a tile.  S and dPd read row l32 (the A operand:
  // lane = row, 8 consecutive e per lane); the transposed reads of dO^T and Q^T
  // map contraction slot (g, i) to tile row 8*(i/4) + 4*g + i%4, the
  // C-register order of S.
  int aoff[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es) aoff[es] = chunk_off<E>(l32, 2 * es + g);
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int troff[2][NEB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) troff[t][eb] = tr_off<E>(8 * t + tr_row, 32 * eb + tr_col);
  const int sk4 = (p.Sk + 3) >> 2;

  // K and V of the block pass through stage 2 (first refilled by iteration 0)
  // together with the first two stages; each wave then takes its sub-block's
  // fragments, the B operands of S = Q K^T and dPd = dO V^T: lane = key,
  // e = 16*es + 8*g + 0..7 (keys past Sk read as zeros).
  {
    uint32_t okv[NLD], ovv[NLD];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      okv[k] = dma_src_offset_e<E>(k, tid, p.sk.s, p.E);
      ovv[k] = dma_src_offset_e<E>(k, tid, p.sv.s, p.E);
    }
    issue_tiles<E>(lds + 2 * C::STAGE_A, wave, (uint32_t)kb0, rk, (uint32_t)(p.sk.s * 2), okv, rvv,
                   (uint32_t)(p.sv.s * 2), ovv);
  }
  if (n_it > 0) issue(0);
  // The block's own tiles first; stage 1 goes out once they are in.
  if (n_it > 0)
    ring_barrier<C::NPAIR_A>();
  else
    ring_barrier<0>();
  bf16x8 kf[NES], vf[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es) {
    kf[es] = lds_at<bf16x8>(lds + 2 * C::STAGE_A + sb * TILE_B, aoff[es]);
    vf[es] = lds_at<bf16x8>(lds + 2 * C::STAGE_A + (2 + sb) * TILE_B, aoff[es]);
  }
  if (n_it > 1) issue(1);
  if (n_it > 1)
    ring_barrier<C::NPAIR_A>();
  else
    ring_barrier<0>();

  for (int it = 0; it < n_it; ++it) {
    const int q0 = (t0 + 2 * it + qs) * 32;
    // Skip tiles past Sq and, when causal, tiles whose rows all precede the keys.
    const bool active = !(q0 >= p.Sq || (CAUSAL && q0 + 31 < kbs));
    // Every step issues the loads of stage it+2, also past the last stage (those
    // rows lie past Sq and read as zeros into a stage nobody reads again), so
    // the issue points need no branch and every barrier waits the same count.
    if (!active) {
      issue(it + 2);
      // A causal tile whose rows all precede this sub-block's keys: its bias
      // gradient is zero.  Lanes g = 0, 1 take rows q0 .. q0+15, q0+16 .. q0+31.
      if (DBIAS && q0 < p.Sq && key < p.Sk) {
#pragma unroll 4
        for (int r = 0; r < 16; ++r)
          if (q0 + 16 * g + r < p.Sq)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rdb,
                                                  (uint32_t)(16 * g) * sdb2 + (uint32_t)key * 2u,
                                                  (uint32_t)(q0 + r) * sdb2, 0);
      }
    }
    if (active) {
      // At head dim 128 (one wave per SIMD) LLVM's exponential-interleaving
      // instruction-group strategy measured 3% faster; it changes only the
      // instruction order.
      if constexpr (E == 128) __builtin_amdgcn_iglp_opt(2);
      const unsigned char* st = lds + ring_offset<C::STAGE_A>(it);
      const unsigned char* tq = st + ST_Q + qs * TILE_B;
      const unsigned char* tdo = st + ST_DO + qs * TILE_B;
      const unsigned char* dl = st + ST_DL + qs * 128;

      // -D and L of rows 8*cg + 4*g + u sit in register order: -D seeds dPd's
      // accumulator, so the products yield dPd - D directly (without dropout).
      f32x4 nd4[4], l4[4];
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        nd4[cg] = lds_at<f32x4>(dl, (8 * cg + 4 * g) * 4);
        l4[cg] = lds_at<f32x4>(dl, 256 + (8 * cg + 4 * g) * 4);
      }
      // A bias enters as L - log2(e) * bias, per element.
      if (BIAS) {
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          const bf16x4 bv = lds_tr4(reinterpret_cast<const uint16_t*>(
              st + ST_BIAS + tr_off<64>(qs * 32 + 8 * cg + tr_row, sb * 32 + tr_col)));
          const uint2 w = __builtin_bit_cast(uint2, bv);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            l4[cg][u] = fmaf(from16<F16>((u & 1) ? ((u < 2 ? w.x : w.y) >> 16) : (u < 2 ? w.x : w.y)),
                             -kLog2e, l4[cg][u]);
        }
      }
      f32x16 sacc = zero16(), dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) dpacc[r] = DROPOUT ? 0.f : nd4[r >> 2][r & 3];
#pragma unroll
      for (int es = 0; es < NES; ++es) {
        sacc = mfma16<F16>(lds_at<bf16x8>(tq, aoff[es]), kf[es], sacc);
        dpacc = mfma16<F16>(lds_at<bf16x8>(tdo, aoff[es]), vf[es], dpacc);
      }
      issue_slot(it + 2, 0, 0.f);

      // C layout: lane = key, register r = row q0 + 8*(r/4) + 4*g + r%4.  Only
      // diagonal and ragged tiles take the masked variant.
      const bool need_mask = (CAUSAL && q0 == kbs) || (q0 + 31 >= p.Sq) || (kbs + 31 >= p.Sk);
      bf16x8 pb[2], dsb[2];
      auto elementwise = [&](auto mask_flag) {
        constexpr bool MASK = decltype(mask_flag)::value;
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          uint32_t kbits = 0xF;
          if (DROPOUT && KEEP) {
            // Rows 8*cg + 4*g + u of the tile, this workgroup's word of this sub-block.
            const unsigned char* kw = st + ST_KEEP + (qs * 32 + 8 * cg + 4 * g) * 16 + (kblk & 1) * 8 + sb * 4;
            kbits = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) kbits |= ((lds_at<uint32_t>(kw, u * 16) >> l32) & 1u) << u;
          } else if (DROPOUT) {
            kbits = keep_bits_for_key(drop, bhg, p.Sq, sk4, q0 + 8 * cg + 4 * g, key, lane);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * cg + u;
            float x = fmaf(sacc[r], c, -l4[cg][u]);
            if (MASK) {
              const int qrow = q0 + 8 * cg + 4 * g + u;
              const bool ok = (qrow < p.Sq) & (key < p.Sk) & (!CAUSAL | (key <= qrow));
              x = ok ? x : -INFINITY;
            }
            const float ps = fast_exp2(x);
            float dp = dpacc[r], pd = ps;  // dp = dPd - D without dropout
            if (DROPOUT) {
              const bool keep = (kbits >> u) & 1;
              pd = keep ? ps * drop.keep_scale : 0.f;
              dp = (keep ? dp * drop.keep_scale : 0.f) + nd4[cg][u];
            }
            pb[r >> 3][r & 7] = to16<F16>(pd);
            dsb[r >> 3][r & 7] = to16<F16>(ps * dp);
            if (DBIAS) {
              // ps carries the scale: dS = ps * (dP - D) / scale.  Causally
              // hidden elements store ps = 0; only rows past Sq and keys past
              // Sk (ragged tiles) are skipped.
              bool in = true;
              if (MASK) in = (q0 + 8 * cg + 4 * g + u < p.Sq) & (key < p.Sk);
              if (in)
                __builtin_amdgcn_raw_buffer_store_b16(
                    __builtin_bit_cast(uint16_t, to16<F16>(ps * dp * inv_scale)), rdb, odb,
                    (uint32_t)(q0 + 8 * cg + u) * sdb2, 0);
            }
            if (u == 3 && (cg == 1 || cg == 3)) issue_slot(it + 2, 1 + cg / 2, ps);
          }
        }
      };
      if (need_mask)
        elementwise(Flag<true>{});
      else
        elementwise(Flag<false>{});
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int o0 = troff[0][eb] + hf * 16 * C::ROW_B, o1 = troff[1][eb] + hf * 16 * C::ROW_B;
          dva[eb] = mfma16<F16>(tr_pair(tdo, o0, o1), pb[hf], dva[eb]);
          dka[eb] = mfma16<F16>(tr_pair(tq, o0, o1), dsb[hf], dka[eb]);
          if (hf == 1 && (eb == 0 || eb == NEB - 1)) issue_slot(it + 2, eb == 0 ? 3 : 4, 0.f);
        }
    }
    // Stage it+1 must have landed; stage it is free once every wave is past here.
    ring_barrier<C::NPAIR_A>();
  }
  ring_barrier<0>();  // the trailing loads have landed before the stages are reused

  // dV = (1/scale) * sum(Pd^T dO) since Pd carries the scale; dK carries it already.
  // Wave qs = 0 finalizes the first half of the columns of dV and dK, qs = 1 the rest.
  float* red = reinterpret_cast<float*>(lds);
  const bool upper = qs == 1;
  exchange_put<E>(dva, red, 4 * sb + 2 * qs + 0, upper, lane);
  exchange_put<E>(dka, red, 4 * sb + 2 * qs + 1, upper, lane);
  ring_barrier<0>();
  uint16_t* dvp = p.dv + b * p.sdv.b + h * p.sdv.h;
  uint16_t* dkp = p.dk + b * p.sdk.b + h * p.sdk.h;
  const int partner = 4 * sb + 2 * (1 - qs);
  exchange_finish<E, F16>(dva, 1.f / p.scale, dvp, p.sdv.s, kbs, p.Sk, p.E, red, partner + 0, upper,
                          lane);
  exchange_finish<E, F16>(dka, 1.f, dkp, p.sdk.s, kbs, p.Sk, p.E, red, partner + 1, upper, lane);

  // Rows before the first tile this block visits (causal: every key of the
  // block is hidden from them) get a zero bias gradient: 8 lanes per row, 16
  // bytes (8 keys) each, the rows dealt over the workgroup.
  if (DBIAS && CAUSAL) {
    const int rows = min(t0 * 32, p.Sq);
    const int k8 = kb0 + 8 * (tid & 7);
    if (k8 < p.Sk) {
      for (int r = tid >> 3; r < rows; r += 32) {
        const uint32_t off = (uint32_t)r * sdb2 + (uint32_t)k8 * 2u;
        if (k8 + 8 <= p.Sk) {
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, rdb, off, 0u, 0);
        } else {
          for (int j = 0; j < p.Sk - k8; ++j)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rdb, off + 2u * (uint32_t)j, 0u, 0);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NST: stages in the ring.  Three (the default) keep the loads two steps
// ahead and take the block's Q, dO, -D and L through a third stage; two leave
// room for a second workgroup per CU at head dim 128, load those straight
// into registers and keep the loads one step ahead.
template <int E, bool CAUSAL, bool DROPOUT, bool BIAS, bool F16, bool KEEP, int NST = 3>
__device__ __forceinline__ void role_dq(const BwdParams& p, int bh, int qblk, unsigned char* lds) {
  static_assert(NST == 2 || NST == 3, "ring depth");
  using C = BwdCfg<E, BIAS, KEEP>;
  constexpr int NES = C::NES, NEB = C::NEB, NLD = C::NLD, TILE_B = C::TILE_B;
  constexpr int ST_K = 0, ST_V = 2 * TILE_B, ST_BIAS = 4 * TILE_B, ST_KEEP = ST_BIAS + C::BIAS_B;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int qsb = wave & 1, ks = wave >> 1;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0b = qblk * 64;
  const int q0 = q0b + 32 * qsb;
  const int qrow = q0 + l32;
  const float c = p.scale_log2;

  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(p.q + b * p.sq.b + h * p.sq.h, p.Sq, p.sq.s, p.E);
  const __amdgpu_buffer_rsrc_t rdo =
      rows_rsrc(p.dout + b * p.sdo.b + h * p.sdo.h, p.Sq, p.sdo.s, p.E);
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(p.k + b * p.sk.b + h * p.sk.h, p.Sk, p.sk.s, p.E);
  const __amdgpu_buffer_rsrc_t rvv = rows_rsrc(p.v + b * p.sv.b + h * p.sv.h, p.Sk, p.sv.s, p.E);

  // Waves 0, 1 stage rows of -D, waves 2, 3 rows of L (workspace planes).
  const __amdgpu_buffer_rsrc_t rdl = make_rsrc(
      p.dl + (wave >> 1) * ((int64_t)p.B * p.H * p.Sq) + (int64_t)bh * p.Sq, (uint32_t)p.Sq * 4u);

  f32x16 dqa[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) dqa[eb] = zero16();

  const int nkt = (p.Sk + 31) / 32;
  const int kt_end = CAUSAL ? min(nkt, min(q0b + 63, p.Sq - 1) / 32 + 1) : nkt;
  const int n_it = (kt_end + 1) / 2;

  // Keep bits from the forward: stage it holds, for each of this workgroup's 64
  // rows, the 16-byte chunk of words that contains the stage's two 32-key words.
  __amdgpu_buffer_rsrc_t rkeep = make_rsrc(p.q, 0u);
  uint32_t okeep = 0u;
  if (KEEP) {
    rkeep = make_rsrc(p.keep + (int64_t)bh * p.Sq * p.keep_w, (uint32_t)(p.Sq * p.keep_w * 4));
    okeep = (uint32_t)((q0b + wave * 16 + (lane & 15)) * p.keep_w * 4);
  }
  // Additive bias: stage it also holds the bias block of this workgroup's 64
  // rows x the stage's 64 keys; a lane reads keys 8*cg + 4*g + 0..3 of its
  // row (8 bytes) for register group cg.
  __amdgpu_buffer_rsrc_t br = make_rsrc(p.q, 0u);
  uint32_t obias[2] = {0u, 0u};
  if (BIAS) {
    br = make_rsrc(p.bias + b * p.sbias.b + h * p.sbias.h, bias_bytes(p));
#pragma unroll
    for (int k = 0; k < 2; ++k)
      obias[k] = dma_src_offset<64>(k, tid, p.sbias.s) + (uint32_t)q0b * (uint32_t)(p.sbias.s * 2);
  }

  // Stage it % 3 of the ring holds key tiles 2*it and 2*it + 1.
  uint32_t okk[NLD], ov[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    okk[k] = dma_src_offset_e<E>(k, tid, p.sk.s, p.E);
    ov[k] = dma_src_offset_e<E>(k, tid, p.sv.s, p.E);
  }
  // Load idx (0 .. NPAIR_B-1) of stage it: (half, tensor, k) for the K and V
  // tiles, then the two loads of the bias block.
  auto issue_one = [&](int it, int idx, float after) {
    unsigned char* st = lds + ring_offset<C::STAGE_B, NST>(it);
    if (BIAS && idx >= 4 * NLD && idx < 4 * NLD + C::NBL) {
      const int k = idx - 4 * NLD;
      dma16_after(br, st + ST_BIAS + k * 4096 + wave * 1024, (uint32_t)(128 * it) + obias[k],
                  after);
      return;
    }
    if (idx >= 4 * NLD) {
      if (lane < 16)
        dma16_after(rkeep, st + ST_KEEP + wave * 256, (uint32_t)((it >> 1) * 16) + okeep, after);
      return;
    }
    const int half = idx / (2 * NLD), tensor = (idx / NLD) & 1, k = idx % NLD;
    const uint32_t r = (uint32_t)(64 * it) + 32u * half;
    unsigned char* dst = st + (tensor ? ST_V : ST_K) + half * TILE_B + k * 4096 + wave * 1024;
    if (tensor)
      dma16_after(rvv, dst, r * (uint32_t)(p.sv.s * 2) + ov[k], after);
    else
      dma16_after(rk, dst, r * (uint32_t)(p.sk.s * 2) + okk[k], after);
  };
  // The loads of a stage are spread over the step in NSLOT groups.
  constexpr int NSLOT = 4;
  auto issue_slot = [&](int it, int slot, float after) {
#pragma unroll
    for (int idx = slot * C::NPAIR_B / NSLOT; idx < (slot + 1) * C::NPAIR_B / NSLOT; ++idx)
      issue_one(it, idx, after);
  };
  auto issue = [&](int it) {
#pragma unroll
    for (int slot = 0; slot < NSLOT; ++slot) issue_slot(it, slot, 0.f);
  };

  int aoff[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es) aoff[es] = chunk_off<E>(l32, 2 * es + g);
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int troff[2][NEB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) troff[t][eb] = tr_off<E>(8 * t + tr_row, 32 * eb + tr_col);
  const int key_limit = CAUSAL ? min(qrow, p.Sk - 1) : p.Sk - 1;
  const int sk4 = (p.Sk + 3) >> 2;
  uint64_t drow = 0;
  DropoutParams drop = p.drop;
  if (DROPOUT) {
    load_dropout_state(drop);
    drow = philox_row_base(drop, dropout_head(drop, b, h), p.Sq, qrow, sk4);
  }

  // The B operands of S^T = K Q^T and dP^T = V dO^T: each wave's rows of Q and
  // dO, lane = row, e = 16*es + 8*g + 0..7; and the row's -D and L.
  bf16x8 qf[NES], dof[NES];
  float ndsum, lse2;
  if constexpr (NST == 2) {
    // Straight from memory into registers; rows past Sq and columns past the
    // head dim read as zeros through the buffer range check.
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      const uint32_t col = (uint32_t)(16 * es + 8 * g);
      const uint32_t oob = (int)col < p.E ? 0u : 0x80000000u;
      qf[es] = __builtin_bit_cast(
          bf16x8, buffer_load16(rq, ((uint32_t)qrow * (uint32_t)(p.sq.s * 2) + 2u * col) | oob));
      dof[es] = __builtin_bit_cast(
          bf16x8, buffer_load16(rdo, ((uint32_t)qrow * (uint32_t)(p.sdo.s * 2) + 2u * col) | oob));
    }
    const int64_t row = (int64_t)bh * p.Sq + min(qrow, p.Sq - 1);
    ndsum = p.dl[row];
    lse2 = p.dl[(int64_t)p.B * p.H * p.Sq + row];
    if (n_it > 0) issue(0);
    ring_barrier<0>();
  } else {
  // Q and dO of the block pass through stage 2 (first refilled by iteration 0)
  // together with the first two stages; each wave then takes its rows'
  // fragments.
  {
    uint32_t oqq[NLD], odd[NLD];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      oqq[k] = dma_src_offset_e<E>(k, tid, p.sq.s, p.E);
      odd[k] = dma_src_offset_e<E>(k, tid, p.sdo.s, p.E);
    }
    issue_tiles<E>(lds + 2 * C::STAGE_B, wave, (uint32_t)q0b, rq, (uint32_t)(p.sq.s * 2), oqq, rdo,
                   (uint32_t)(p.sdo.s * 2), odd);
    // -D (waves 0, 1) and L (waves 2, 3) of the block's 64 rows, 4 rows per lane.
    if (lane < 8)
      dma16(rdl, lds + 2 * C::STAGE_B + 4 * TILE_B + wave * 128,
            (uint32_t)q0b * 4u + (uint32_t)((wave & 1) * 128 + lane * 16));
  }
  if (n_it > 0) issue(0);
  // The block's own tiles first; stage 1 goes out once they are in.
  if (n_it > 0)
    ring_barrier<C::NPAIR_B>();
  else
    ring_barrier<0>();
#pragma unroll
  for (int es = 0; es < NES; ++es) {
    qf[es] = lds_at<bf16x8>(lds + 2 * C::STAGE_B + qsb * TILE_B, aoff[es]);
    dof[es] = lds_at<bf16x8>(lds + 2 * C::STAGE_B + (2 + qsb) * TILE_B, aoff[es]);
  }
  ndsum = lds_at<float>(lds + 2 * C::STAGE_B + 4 * TILE_B, (qsb * 32 + l32) * 4);
  lse2 = lds_at<float>(lds + 2 * C::STAGE_B + 4 * TILE_B + 256, (qsb * 32 + l32) * 4);
  if (n_it > 1) issue(1);
  if (n_it > 1)
    ring_barrier<C::NPAIR_B>();
  else
    ring_barrier<0>();
  }
  // -D seeds dP's accumulator (without dropout).
  f32x16 dinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) dinit[r] = DROPOUT ? 0.f : ndsum;

  for (int it = 0; it < n_it; ++it) {
    const int j = 2 * it + ks;
    const int k0 = j * 32;
    const bool active = !(j >= kt_end || (CAUSAL && k0 > q0 + 31));
    // Loads of stage it+NST-1 on every step, as in the dK/dV role (past the
    // last stage they fetch rows nobody reads).
    if (!active) issue(it + NST - 1);
    if (active) {
      if constexpr (E == 128) __builtin_amdgcn_iglp_opt(2);  // as in the dK/dV role
      const unsigned char* st = lds + ring_offset<C::STAGE_B, NST>(it);
      const unsigned char* tk = st + ST_K + ks * TILE_B;
      const unsigned char* tv = st + ST_V + ks * TILE_B;

      // L of the row, minus log2(e) * bias per element when there is a bias.
      float lb[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) lb[r] = lse2;
      if (BIAS) {
        const int brow = qsb * 32 + l32;
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          const uint2 w = lds_at<uint2>(
              st, ST_BIAS + brow * 128 + (((4 * ks + cg) ^ tile_swz<64>(brow)) << 4) + 8 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t x = u < 2 ? w.x : w.y;
            lb[4 * cg + u] = fmaf(from16<F16>((u & 1) ? (x >> 16) : x), -kLog2e, lse2);
          }
        }
      }
      // S^T, dP^T: lane = row, register r = key k0 + 8*(r/4) + 4*g + r%4.
      f32x16 sacc = zero16(), dpacc = dinit;
#pragma unroll
      for (int es = 0; es < NES; ++es) {
        sacc = mfma16<F16>(lds_at<bf16x8>(tk, aoff[es]), qf[es], sacc);
        dpacc = mfma16<F16>(lds_at<bf16x8>(tv, aoff[es]), dof[es], dpacc);
      }
      issue_slot(it + NST - 1, 0, 0.f);

      // Only tiles that reach the diagonal or past Sk take the masked variant.
      const bool need_mask = (k0 + 31 > (CAUSAL ? min(q0, p.Sk - 1) : p.Sk - 1));
      const int lim = key_limit - k0 - 4 * g;
      bf16x8 dsb[2];
      auto elementwise = [&](auto mask_flag) {
        constexpr bool MASK = decltype(mask_flag)::value;
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          uint32_t kbits = 0xF;
          if (DROPOUT && KEEP) {
            kbits = (lds_at<uint32_t>(st, ST_KEEP + (qsb * 32 + l32) * 16 + (it & 1) * 8 + ks * 4) >>
                     (8 * cg + 4 * g)) & 0xFu;
          } else if (DROPOUT) {
            const PhiloxOut w = philox4x32_10(drow + (uint32_t)(k0 >> 2) + 2 * cg + g,
                                              drop.seed_lo, drop.seed_hi);
            kbits = (w.w[0] >= drop.threshold ? 1u : 0u) |
                    (w.w[1] >= drop.threshold ? 2u : 0u) |
                    (w.w[2] >= drop.threshold ? 4u : 0u) |
                    (w.w[3] >= drop.threshold ? 8u : 0u);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * cg + u;
            float x = fmaf(sacc[r], c, -lb[r]);
            if (MASK) x = (8 * cg + u <= lim) ? x : -INFINITY;
            const float ps = fast_exp2(x);
            float dp = dpacc[r];  // dP - D without dropout
            if (DROPOUT) dp = (((kbits >> u) & 1) ? dp * drop.keep_scale : 0.f) + ndsum;
            dsb[r >> 3][r & 7] = to16<F16>(ps * dp);
            if (u == 3 && (cg == 1 || cg == 3)) issue_slot(it + NST - 1, 1 + cg / 2, ps);
          }
        }
      };
      if (need_mask)
        elementwise(Flag<true>{});
      else
        elementwise(Flag<false>{});
      // dQ^T += K^T dS'^T: A = K^T read transposed from the tile, B = dS'^T from registers.
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int o0 = troff[0][eb] + hf * 16 * C::ROW_B, o1 = troff[1][eb] + hf * 16 * C::ROW_B;
          dqa[eb] = mfma16<F16>(tr_pair(tk, o0, o1), dsb[hf], dqa[eb]);
          if (hf == 1 && eb == 0) issue_slot(it + NST - 1, 3, 0.f);
        }
    }
    // Stage it+1 must have landed (with two stages it went out in this step).
    if constexpr (NST == 3)
      ring_barrier<C::NPAIR_B>();
    else
      ring_barrier<0>();
  }
  ring_barrier<0>();  // the trailing loads have landed before the stages are reused

  // Wave ks = 0 finalizes the first half of dQ's columns, ks = 1 the rest.
  float* red = reinterpret_cast<float*>(lds);
  const bool upper = ks == 1;
  exchange_put<E>(dqa, red, 2 * qsb + ks, upper, lane);
  ring_barrier<0>();
  uint16_t* dqp = p.dq + b * p.sdq.b + h * p.sdq.h;
  exchange_finish<E, F16>(dqa, 1.f, dqp, p.sdq.s, q0, p.Sq, p.E, red, 2 * qsb + (1 - ks), upper,
                          lane);
}

// Order in which a head's dK/dV and dQ blocks are dealt out: longest estimated
// run first, so the short blocks fill in at the end (longest-processing-time
// first).  Entry s: bit 15 set for a dQ block, low bits the block's rank.
constexpr int kMaxOrder = 1024;
struct BwdOrder {
  uint32_t word[kMaxOrder / 2];  // two entries a word, entry 2*i in the low half
  void set(int s, uint16_t v) {
    uint32_t& w = word[s >> 1];
    w = (w & (0xFFFF0000u >> (16 * (s & 1)))) | ((uint32_t)v << (16 * (s & 1)));
  }
  // Read as a whole word: a scalar load, where a 16-bit read is a vector one.
  __device__ int get(int s) const { return (int)(word[s >> 1] >> (16 * (s & 1))) & 0xFFFF; }
};

// Workgroup order: per head, blocks in BwdOrder order (or, past kMaxOrder
// blocks, dK/dV and dQ alternating, heaviest causal blocks first); all blocks
// of a head sit on one XCD when the head count allows.
// ROLES: 3 compiles both workgroup roles, 2 only the dQ role with a two-stage
// ring (so that two of its workgroups share a CU at head dim 128).  `order`
// says how a workgroup finds its block: 1 from the table `ord`, 0 dK/dV and dQ
// blocks alternating (past kMaxOrder blocks), 2 every block a dK/dV block and
// 3 every block a dQ block, rank = slot (launches of one role, past
// kMaxOrder blocks).
template <int E, bool BIAS, bool KEEP, int ROLES>
constexpr int bwd_lds_bytes() {
  using C = BwdCfg<E, BIAS, KEEP>;
  return ROLES == 2 ? (2 * C::STAGE_B > C::RED_B / 2 ? 2 * C::STAGE_B : C::RED_B / 2) : C::LDS_B;
}

template <int E, bool CAUSAL, bool DROPOUT, bool BIAS, bool F16, bool KEEP, bool DBIAS,
          int ROLES = 3>
__global__ __launch_bounds__(256) void bwd_kernel(BwdParams p, int nkb, int nqb, int order,
                                                  BwdOrder ord) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[bwd_lds_bytes<E, BIAS, KEEP, ROLES>()];
  // The parameters, the launch's ints and the table's first entries.
  warm_kernargs<8 * 64>();
  const int bh_count = p.B * p.H;
  int bh, slot;
  if ((bh_count & 7) == 0) {
    const int per_xcd = bh_count >> 3;
    const int xcd = blockIdx.x & 7, sx = blockIdx.x >> 3;
    slot = sx / per_xcd;
    bh = xcd * per_xcd + (sx - slot * per_xcd);
  } else {
    slot = blockIdx.x / bh_count;
    bh = blockIdx.x - slot * bh_count;
  }
  bool dkdv;
  int rank;
  if (order == 1) {
    const int e = ord.get(slot);
    dkdv = (e & 0x8000) == 0;
    rank = e & 0x7FFF;
  } else if (order >= 2) {
    dkdv = order == 2;
    rank = slot;
  } else {
    const int m = min(nkb, nqb);
    if (slot < 2 * m) {
      dkdv = (slot & 1) == 0;
      rank = slot >> 1;
    } else {
      dkdv = nkb > nqb;
      rank = slot - m;
    }
  }
  if constexpr (ROLES == 3) {
    if (dkdv) {
      role_dkdv<E, CAUSAL, DROPOUT, BIAS, F16, KEEP, DBIAS>(p, bh, rank, lds);
      return;
    }
  }
  role_dq<E, CAUSAL, DROPOUT, BIAS, F16, KEEP, ROLES == 2 ? 2 : 3>(
      p, bh, CAUSAL ? nqb - 1 - rank : rank, lds);
}

// -D_i = -rowsum(dO * O) and L_i = LSE_i * log2(e) - log2(scale) for every
// row, in two planes of B*H*Sq floats.  A block covers RPB rows of one head
// (block v of `total` is row block v % nblk of head v / nblk, so all index
// arithmetic is 32-bit and uniform); CPR lanes share a row and each loads one
// 16-byte chunk of dO and of O.
template <int E, bool F16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, uint32_t nblk,
                                                        uint32_t total) {
  constexpr int CPR = E / 8, RPB = 256 / CPR;
  warm_kernargs<sizeof(BwdParams) + 2 * sizeof(uint32_t)>();
  const int tid = threadIdx.x;
  const int col = tid % CPR;
  const float log2_scale = __log2f(p.scale);
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  for (uint64_t vv = blockIdx.x; vv < total; vv += gridDim.x) {
    const uint32_t v = (uint32_t)vv;
    const uint32_t bh = v / nblk;
    const int i = (int)(v - bh * nblk) * RPB + tid / CPR;
    const uint32_t b = bh / (uint32_t)p.H, h = bh - b * (uint32_t)p.H;
    float d = 0.f;
    if (i < p.Sq && col * 8 < p.E) {
      const bf16x8 x = load_bf16x8(p.dout + b * p.sdo.b + h * p.sdo.h + i * p.sdo.s + col * 8);
      const bf16x8 y = load_bf16x8(p.o + b * p.so.b + h * p.so.h + i * p.so.s + col * 8);
      d = dot8_16<F16>(x, y, 0.f);
    }
    d = group_sum<CPR>(d);
    if (i < p.Sq && col == 0) {
      const int64_t row = (int64_t)bh * p.Sq + i;
      p.dl[row] = -d;
      p.dl[rows + row] = p.lse[row] * kLog2e - log2_scale;
    }
  }
}

template <int E, bool F16>
hipError_t launch_rows_t(const BwdParams& p, hipStream_t stream) {
  constexpr int RPB = 256 / (E / 8);
  // B*H*nblk < 2^32: B*H*ceil(Sq/32) is below 2^31 and RPB >= 16.
  const uint32_t nblk = (uint32_t)((p.Sq + RPB - 1) / RPB);
  const uint32_t total = (uint32_t)((int64_t)p.B * p.H * nblk);
  hipLaunchKernelGGL((bwd_prep_kernel<E, F16>), dim3(std::min(total, 1u << 20)), dim3(256), 0,
                     stream, p, nblk, total);
  return hipGetLastError();
}

// Large problems without dropout or a bias run the two roles as two
// launches: the dK/dV blocks (the two-role kernel given only dK/dV blocks,
// whose code for that role measured faster than a one-role build) and then
// the dQ blocks with a two-stage ring, which leaves room for more dQ
// workgroups per CU: two instead of one at head dim 128, three instead of two
// at 64.  The second launch starts only when the first has drained, so this
// pays off only once each role fills the chip for several rounds: measured,
// from 2 rounds of the one-launch kernel's slots at head dim 128 (1932 vs
// 2062 us at b1 h32 q4096 k8192; 56 vs 50 us at b2 h12 s1024) and from 8 at
// head dim 64 (298 vs 328 us at 8x16x2048^2 causal, no change at 4 rounds).
// Dropout's registers and a bias's LDS would leave the dQ launch no more
// workgroups per CU, so those variants keep one launch.
template <int E, bool DROPOUT, bool BIAS>
constexpr bool bwd_can_split() {
  return !DROPOUT && !BIAS;
}

template <int E, bool F16>
hipError_t launch_main_t(const BwdParams& p, bool causal, bool dropout, const TileChoice& tiles,
                         hipStream_t stream) {
  const int nkb = (p.Sk + 63) / 64, nqb = (p.Sq + 63) / 64;
  const unsigned bhn = (unsigned)(p.B * p.H);
  bool split = false;
  if (!dropout && p.bias == nullptr) {
    if (tiles.bwd_roles == 1 || tiles.bwd_roles == 2) {
      split = tiles.bwd_roles == 2;
    } else {
      const long slots = (long)device_cus() * (E == 64 ? 2 : 1);  // one-launch residency
      split = slots > 0 && (long)std::min(nkb, nqb) * bhn >= (E == 64 ? 8 : 2) * slots;
    }
  }
  BwdOrder ord{}, ordk{}, ordq{};
  // Past kMaxOrder blocks (or when asked to) the blocks go out in an order the
  // kernel computes from the block index instead of the table.
  const bool table = tiles.bwd_order != 1;
  const int use_order = table && !split && nkb + nqb <= kMaxOrder ? 1 : 0;
  const int use_k = table && split && nkb <= kMaxOrder ? 1 : 0;
  const int use_q = table && split && nqb <= kMaxOrder ? 1 : 0;
  if (use_order || use_k || use_q) {
    // Estimated run of a block: steps times a measured per-step cost plus a
    // fixed prologue/epilogue (dK/dV: ~1.5 us per step + ~4 us; dQ: ~1.1 us +
    // ~3.3 us, at b2 h12 s1024 d64), in units of 0.1 us.
    const int nqt = (p.Sq + 31) / 32, nkt = (p.Sk + 31) / 32;
    struct Item {
      int cost, key;
    };
    std::vector<Item> items;
    items.reserve(nkb + nqb);
    for (int r = 0; r < nkb; ++r) {
      const int t0 = causal ? std::min(2 * r, nqt) : 0;
      items.push_back({15 * ((nqt - t0 + 1) / 2) + 40, r});
    }
    for (int r = 0; r < nqb; ++r) {
      const int qblk = causal ? nqb - 1 - r : r;
      const int kt_end = causal ? std::min(nkt, std::min(64 * qblk + 63, p.Sq - 1) / 32 + 1) : nkt;
      items.push_back({11 * ((kt_end + 1) / 2) + 33, 0x8000 | r});
    }
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& a, const Item& b) { return a.cost > b.cost; });
    int n = 0, nk = 0, nq = 0;
    for (const Item& it : items) {
      if (use_order) ord.set(n++, (uint16_t)it.key);
      if (use_k && (it.key & 0x8000) == 0) ordk.set(nk++, (uint16_t)it.key);
      if (use_q && (it.key & 0x8000) != 0) ordq.set(nq++, (uint16_t)it.key);
    }
  }
  auto go3 = [&](auto c, auto d, auto bias, auto keep, auto db) {
    constexpr bool Cf = decltype(c)::value, Df = decltype(d)::value, Bf = decltype(bias)::value;
    constexpr bool Kf = decltype(keep)::value, DBf = decltype(db)::value;
    if constexpr (bwd_can_split<E, Df, Bf>()) {
      if (split) {
        hipLaunchKernelGGL((bwd_kernel<E, Cf, Df, Bf, F16, Kf, DBf, 3>), dim3((unsigned)nkb * bhn),
                           dim3(256), 0, stream, p, nkb, nqb, use_k ? 1 : 2, ordk);
        hipLaunchKernelGGL((bwd_kernel<E, Cf, Df, Bf, F16, Kf, DBf, 2>), dim3((unsigned)nqb * bhn),
                           dim3(256), 0, stream, p, nkb, nqb, use_q ? 1 : 3, ordq);
        return;
      }
    }
    hipLaunchKernelGGL((bwd_kernel<E, Cf, Df, Bf, F16, Kf, DBf, 3>),
                       dim3((unsigned)(nkb + nqb) * bhn), dim3(256), 0, stream, p, nkb, nqb,
                       use_order, ord);
  };
  auto go2 = [&](auto c, auto d, auto bias, auto keep) {
    if constexpr (decltype(bias)::value) {
      if (p.dbias != nullptr) {
        go3(c, d, bias, keep, Flag<true>{});
        return;
      }
    }
    go3(c, d, bias, keep, Flag<false>{});
  };
  auto go = [&](auto c, auto d, auto bias) {
    if constexpr (decltype(d)::value) {
      if (p.keep != nullptr) {
        go2(c, d, bias, Flag<true>{});
        return;
      }
    }
    go2(c, d, bias, Flag<false>{});
  };
  auto with_bias = [&](auto c, auto d) {
    if (p.bias != nullptr)
      go(c, d, Flag<true>{});
    else
      go(c, d, Flag<false>{});
  };
  auto with_dropout = [&](auto c) {
    if (dropout)
      with_bias(c, Flag<true>{});
    else
      with_bias(c, Flag<false>{});
  };
  if (causal)
    with_dropout(Flag<true>{});
  else
    with_dropout(Flag<false>{});
  return hipGetLastError();
}

}  // namespace

}  // namespace sdpa14

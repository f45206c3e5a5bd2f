// Fused attention backward for gfx950, recomputing the probabilities from the
// stashed log-sum-exp (nvFuser issue 2278: what the forward stashes is chosen
// by what the backward needs; here O and LSE are stashed and P is recomputed).
// The backward statement follows sdpfa_bwd of the nvFuser PR "DID loop split
// for SDPA"; dropout regenerates the forward's mask from (seed, offset) and the
// absolute element index (PyTorch PR "REDO of dropout support for mem eff").
//
// One launch, two workgroup roles, no atomics and no workspace.  Each
// workgroup stages the tiles it streams in LDS with row-contiguous loads (every
// 8 lanes read one 128-byte row), and two waves share every staged tile; the
// vector-memory path, not the matrix cores, is what limits this pass.
//
//   dK/dV role  a 64-key block: waves (sb, qs), sb = 32-key sub-block,
//               qs = which of the two 32-row query tiles of an iteration.
//               Each wave keeps its sub-block's K and V fragments and its dK^T,
//               dV^T accumulators in registers.  Per query tile:
//                 S = Q K^T, dPd = dO V^T          (lane = key, registers = rows)
//                 Ps = scale * exp(S*scale - LSE)  (masked; dropout kept/scaled)
//                 dS' = Ps * (dP - D),  D_i = rowsum(dO * O) from the staged tiles
//                 dV^T += dO^T Pd, dK^T += Q^T dS' (dO^T, Q^T read transposed)
//               The two query-tile waves of a sub-block are summed at the end.
//   dQ role     a 64-row block: waves (qsb, ks), qsb = 32-row sub-block, ks =
//               which of the two 32-key tiles of an iteration.  Each wave keeps
//               its rows' Q and dO fragments, D and LSE in registers.  Per key
//               tile: S^T = K Q^T, dP^T = V dO^T (lane = row), dS'^T as above,
//               dQ^T += K^T dS'^T with K^T read transposed.  The two key-tile
//               waves of a sub-block are summed at the end.
//
// Both roles recompute S and dP, so the backward does 7 products of 2*E flops
// per visible score element (5 are counted).  In exchange dQ needs neither
// fp32 atomics nor a zeroed accumulator nor a conversion pass, and every output
// is bitwise reproducible.
#include "device_common.h"
#include "kernels.h"

namespace sdpa14 {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

template <int E>
struct BwdCfg {
  static constexpr int TP = E + 8;               // staged tile pitch (elements)
  static constexpr int TILE = 32 * TP;            // elements per staged 32-row tile
  static constexpr int CPR = E / 8;               // 16-byte chunks per row
  static constexpr int CPT = 32 * CPR / 256;      // chunks per thread per tile (256 threads)
  static constexpr int NEB = E / 32;
  static constexpr int NES = E / 16;
  // dK/dV role: 6 tiles (Q, dO, O for two query tiles) + per-wave D/LSE rows.
  static constexpr int A_BYTES = 6 * TILE * 2 + 4 * 64 * 4;
  // End-of-block reduction: two fp32 accumulator sets (dK^T, dV^T) per sub-block.
  static constexpr int RED_BYTES = 2 * 2 * NEB * 16 * 64 * 4;
  static constexpr int TOTAL = (A_BYTES > RED_BYTES ? A_BYTES : RED_BYTES);
};

// Adds, for each sub-block, the accumulator of the wave with `second` set into
// the wave without it, then that wave stores bf16 rows (C layout: lane = output
// row row0 + l32, register r = column 32*eb + 8*(r/4) + 4*g + r%4).
template <int E>
__device__ __forceinline__ void pair_reduce_store(const f32x16 (&acc)[E / 32], float mul,
                                                  uint16_t* dst, int64_t stride, int row0,
                                                  int limit, float* red, int slot, bool second,
                                                  int lane) {
  constexpr int NEB = E / 32;
  float* buf = red + slot * (NEB * 16 * 64);
  if (second) {
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) buf[(eb * 16 + r) * 64 + lane] = acc[eb][r];
  }
  __syncthreads();
  if (!second) {
    const int row = row0 + (lane & 31);
    const int g = lane >> 5;
    if (row < limit) {
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v[t] = (acc[eb][4 * cg + t] + buf[(eb * 16 + 4 * cg + t) * 64 + lane]) * mul;
          *reinterpret_cast<uint2*>(dst + (int64_t)row * stride + eb * 32 + 8 * cg + 4 * g) =
              pack_bf16x4(v[0], v[1], v[2], v[3]);
        }
    }
  }
}

// Dropout keep bits for the dK/dV role.  The lane holds key `key` (key % 4 ==
// lane % 4) and, for register group c, the four rows row0 + u, u = 0..3.  Lane t
// of each quad evaluates the Philox call of row row0 + t for the key group of
// the quad (four words: keys 4*(key/4) + 0..3), packs the four keep bits, and
// every lane collects its own key's bit from the four lanes of its quad.
// Returns bit u = keep(row0 + u, key).
__device__ __forceinline__ uint32_t keep_bits_for_key(const DropoutParams& d, int bh, int Sq,
                                                      int sk4, int row0, int key, int lane) {
  const int t = lane & 3;
  const uint64_t ctr = philox_row_base(d, bh, Sq, row0 + t, sk4) + (uint32_t)(key >> 2);
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int rows,
                                                            int64_t stride, int E) {
  return make_rsrc(base, rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * stride + E) * 2) : 0u);
}

// ---------------------------------------------------------------------------
template <int E, bool CAUSAL, bool DROPOUT>
__device__ __forceinline__ void role_dkdv(const BwdParams& p, int bh, int kblk,
                                          unsigned char* lds) {
  using C = BwdCfg<E>;
  constexpr int NES = C::NES, NEB = C::NEB, TP = C::TP, CPR = C::CPR, CPT = C::CPT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int sb = wave & 1, qs = wave >> 1;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int kb0 = kblk * 64;
  const int kbs = kb0 + 32 * sb;  // first key of this wave's sub-block
  const int key = kbs + l32;
  const float c = p.scale_log2;
  const float lsc = __log2f(p.scale);

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
  const uint16_t* op = p.o + b * p.so.b + h * p.so.h;
  const float* lsep = p.lse + (int64_t)bh * p.Sq;
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qp, p.Sq, p.sq.s, E);
  const __amdgpu_buffer_rsrc_t rdo = rows_rsrc(dop, p.Sq, p.sdo.s, E);
  const __amdgpu_buffer_rsrc_t ro = rows_rsrc(op, p.Sq, p.so.s, E);
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(p.k + b * p.sk.b + h * p.sk.h, p.Sk, p.sk.s, E);
  const __amdgpu_buffer_rsrc_t rvv = rows_rsrc(p.v + b * p.sv.b + h * p.sv.h, p.Sk, p.sv.s, E);

  // K, V of the sub-block as B operands of S = Q K^T and dPd = dO V^T: lane = key,
  // e = 16*es + 8*g + 0..7.  Keys past Sk read as zeros.
  bf16x8 kf[NES], vf[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es) {
    const uint32_t off16 = (uint32_t)(es * 16 + 8 * g) * 2u;
    kf[es] = __builtin_bit_cast(bf16x8, buffer_load16(rk, (uint32_t)key * (uint32_t)(p.sk.s * 2) + off16));
    vf[es] = __builtin_bit_cast(bf16x8, buffer_load16(rvv, (uint32_t)key * (uint32_t)(p.sv.s * 2) + off16));
  }
  f32x16 dva[NEB], dka[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    dva[eb] = zero16();
    dka[eb] = zero16();
  }

  const int nqt = (p.Sq + 31) / 32;
  const int t0 = CAUSAL ? min(kb0 / 32, nqt) : 0;
  const int n_it = (nqt - t0 + 1) / 2;
  uint16_t* tiles = reinterpret_cast<uint16_t*>(lds);  // [query tile slot][Q, dO, O]
  float* rv = reinterpret_cast<float*>(lds + 6 * C::TILE * 2) + wave * 64;  // D[32], LSE2[32]

  // Row-contiguous staging: thread tid moves chunks tid + 256*k of each tile.
  uint4 stg[6][CPT];
  auto load_pair = [&](int it) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row0 = (t0 + 2 * it + half) * 32;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int cidx = tid + 256 * k;
        const uint32_t row = (uint32_t)(row0 + cidx / CPR), col16 = (uint32_t)(cidx % CPR) * 16u;
        stg[3 * half + 0][k] = buffer_load16(rq, row * (uint32_t)(p.sq.s * 2) + col16);
        stg[3 * half + 1][k] = buffer_load16(rdo, row * (uint32_t)(p.sdo.s * 2) + col16);
        stg[3 * half + 2][k] = buffer_load16(ro, row * (uint32_t)(p.so.s * 2) + col16);
      }
    }
  };
  auto store_pair = [&]() {
#pragma unroll
    for (int s = 0; s < 6; ++s)
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int cidx = tid + 256 * k;
        *reinterpret_cast<uint4*>(tiles + s * C::TILE + (cidx / CPR) * TP + (cidx % CPR) * 8) =
            stg[s][k];
      }
  };

  // Transposed-read addressing: contraction slot (g, i) <-> tile row
  // 8*(i/4) + 4*g + i%4 (the C-register order of S); see device_common.h.
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sk4 = (p.Sk + 3) >> 2;

  if (n_it > 0) load_pair(0);
  for (int it = 0; it < n_it; ++it) {
    __syncthreads();  // previous iteration is done with the tiles
    store_pair();
    __syncthreads();
    if (it + 1 < n_it) load_pair(it + 1);
    const int q0 = (t0 + 2 * it + qs) * 32;
    // Skip tiles past Sq and, when causal, tiles whose rows all precede the keys.
    if (q0 >= p.Sq || (CAUSAL && q0 + 31 < kbs)) continue;
    const uint16_t* tq = tiles + (3 * qs + 0) * C::TILE;
    const uint16_t* tdo = tiles + (3 * qs + 1) * C::TILE;
    const uint16_t* to = tiles + (3 * qs + 2) * C::TILE;

    // D for row q0 + l32 (this lane's half of the columns), and LSE.
    float dpart = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPR / 2; ++cc) {
      const int col = (g * (CPR / 2) + cc) * 8;
      dpart = dot8_bf16(lds_bf16x8(tdo + l32 * TP + col), lds_bf16x8(to + l32 * TP + col), dpart);
    }
    const float dsum = pair_sum(dpart);
    const int qr = q0 + l32;
    const float lse_v = (qr < p.Sq) ? lsep[qr] : 0.f;
    if (g == 0) {
      rv[l32] = dsum;
      rv[32 + l32] = lse_v * kLog2e - lsc;  // exp2(S*c - this) = scale * P
    }

    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      sacc = mfma32x32x16(lds_bf16x8(tq + l32 * TP + es * 16 + 8 * g), kf[es], sacc);
      dpacc = mfma32x32x16(lds_bf16x8(tdo + l32 * TP + es * 16 + 8 * g), vf[es], dpacc);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float4 dv4[4], lv4[4];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      dv4[cg] = *reinterpret_cast<const float4*>(rv + 8 * cg + 4 * g);
      lv4[cg] = *reinterpret_cast<const float4*>(rv + 32 + 8 * cg + 4 * g);
    }

    // C layout: lane = key, register r = row q0 + 8*(r/4) + 4*g + r%4.
    const bool need_mask = (CAUSAL && q0 == kbs) || (q0 + 31 >= p.Sq) || (kbs + 31 >= p.Sk);
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      const float dvals[4] = {dv4[cg].x, dv4[cg].y, dv4[cg].z, dv4[cg].w};
      const float lvals[4] = {lv4[cg].x, lv4[cg].y, lv4[cg].z, lv4[cg].w};
      uint32_t kbits = 0xF;
      if (DROPOUT) kbits = keep_bits_for_key(p.drop, bh, p.Sq, sk4, q0 + 8 * cg + 4 * g, key, lane);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * cg + u;
        float x = fmaf(sacc[r], c, -lvals[u]);
        if (need_mask) {
          const int qrow = q0 + 8 * cg + 4 * g + u;
          const bool ok = (qrow < p.Sq) & (key < p.Sk) & (!CAUSAL | (key <= qrow));
          x = ok ? x : -INFINITY;
        }
        const float ps = fast_exp2(x);
        float dp = dpacc[r], pd = ps;
        if (DROPOUT) {
          const bool keep = (kbits >> u) & 1;
          pd = keep ? ps * p.drop.keep_scale : 0.f;
          dp = keep ? dp * p.drop.keep_scale : 0.f;
        }
        pb[r >> 3][r & 7] = (__bf16)pd;
        dsb[r >> 3][r & 7] = (__bf16)(ps * (dp - dvals[u]));
      }
    }
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int off = (16 * hf + tr_row) * TP + eb * 32 + tr_col;
        dva[eb] = mfma32x32x16(concat(lds_tr4(tdo + off), lds_tr4(tdo + off + 8 * TP)), pb[hf],
                               dva[eb]);
        dka[eb] = mfma32x32x16(concat(lds_tr4(tq + off), lds_tr4(tq + off + 8 * TP)), dsb[hf],
                               dka[eb]);
      }
  }

  // dV = (1/scale) * sum(Pd^T dO) since Pd carries the scale; dK carries it already.
  __syncthreads();  // the tiles are no longer read: reuse the LDS for the reduction
  float* red = reinterpret_cast<float*>(lds);
  uint16_t* dvp = p.dv + b * p.sdv.b + h * p.sdv.h;
  uint16_t* dkp = p.dk + b * p.sdk.b + h * p.sdk.h;
  pair_reduce_store<E>(dva, 1.f / p.scale, dvp, p.sdv.s, kbs, p.Sk, red, 2 * sb, qs == 1, lane);
  pair_reduce_store<E>(dka, 1.f, dkp, p.sdk.s, kbs, p.Sk, red, 2 * sb + 1, qs == 1, lane);
}

// ---------------------------------------------------------------------------
template <int E, bool CAUSAL, bool DROPOUT>
__device__ __forceinline__ void role_dq(const BwdParams& p, int bh, int qblk, unsigned char* lds) {
  using C = BwdCfg<E>;
  constexpr int NES = C::NES, NEB = C::NEB, TP = C::TP, CPR = C::CPR, CPT = C::CPT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int qsb = wave & 1, ks = wave >> 1;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0b = qblk * 64;
  const int q0 = q0b + 32 * qsb;
  const int qrow = q0 + l32;
  const float c = p.scale_log2;

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
  const uint16_t* op = p.o + b * p.so.b + h * p.so.h;
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qp, p.Sq, p.sq.s, E);
  const __amdgpu_buffer_rsrc_t rdo = rows_rsrc(dop, p.Sq, p.sdo.s, E);
  const __amdgpu_buffer_rsrc_t ro = rows_rsrc(op, p.Sq, p.so.s, E);
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(p.k + b * p.sk.b + h * p.sk.h, p.Sk, p.sk.s, E);
  const __amdgpu_buffer_rsrc_t rvv = rows_rsrc(p.v + b * p.sv.b + h * p.sv.h, p.Sk, p.sv.s, E);

  // Q, dO of this row as B operands of S^T = K Q^T and dP^T = V dO^T; D and LSE of the row.
  bf16x8 qf[NES], dof[NES];
  float dpart = 0.f;
#pragma unroll
  for (int es = 0; es < NES; ++es) {
    const uint32_t off16 = (uint32_t)(es * 16 + 8 * g) * 2u;
    qf[es] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)qrow * (uint32_t)(p.sq.s * 2) + off16));
    dof[es] = __builtin_bit_cast(bf16x8, buffer_load16(rdo, (uint32_t)qrow * (uint32_t)(p.sdo.s * 2) + off16));
    const bf16x8 o8 = __builtin_bit_cast(bf16x8, buffer_load16(ro, (uint32_t)qrow * (uint32_t)(p.so.s * 2) + off16));
    dpart = dot8_bf16(dof[es], o8, dpart);
  }
  const float dsum = pair_sum(dpart);
  const float lse2 =
      ((qrow < p.Sq) ? p.lse[(int64_t)bh * p.Sq + qrow] * kLog2e : 0.f) - __log2f(p.scale);

  f32x16 dqa[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) dqa[eb] = zero16();

  const int nkt = (p.Sk + 31) / 32;
  const int kt_end = CAUSAL ? min(nkt, min(q0b + 63, p.Sq - 1) / 32 + 1) : nkt;
  const int n_it = (kt_end + 1) / 2;
  uint16_t* tiles = reinterpret_cast<uint16_t*>(lds);  // [key tile slot][K, V]

  uint4 stg[4][CPT];
  auto load_pair = [&](int it) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row0 = (2 * it + half) * 32;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int cidx = tid + 256 * k;
        const uint32_t row = (uint32_t)(row0 + cidx / CPR), col16 = (uint32_t)(cidx % CPR) * 16u;
        stg[2 * half + 0][k] = buffer_load16(rk, row * (uint32_t)(p.sk.s * 2) + col16);
        stg[2 * half + 1][k] = buffer_load16(rvv, row * (uint32_t)(p.sv.s * 2) + col16);
      }
    }
  };
  auto store_pair = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int cidx = tid + 256 * k;
        *reinterpret_cast<uint4*>(tiles + s * C::TILE + (cidx / CPR) * TP + (cidx % CPR) * 8) =
            stg[s][k];
      }
  };

  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int key_limit = CAUSAL ? min(qrow, p.Sk - 1) : p.Sk - 1;
  const int sk4 = (p.Sk + 3) >> 2;
  uint64_t drow = 0;
  if (DROPOUT) drow = philox_row_base(p.drop, bh, p.Sq, qrow, sk4);

  if (n_it > 0) load_pair(0);
  for (int it = 0; it < n_it; ++it) {
    __syncthreads();
    store_pair();
    __syncthreads();
    if (it + 1 < n_it) load_pair(it + 1);
    const int j = 2 * it + ks;
    const int k0 = j * 32;
    if (j >= kt_end || (CAUSAL && k0 > q0 + 31)) continue;
    const uint16_t* tk = tiles + (2 * ks + 0) * C::TILE;
    const uint16_t* tv = tiles + (2 * ks + 1) * C::TILE;

    // S^T, dP^T: lane = row, register r = key k0 + 8*(r/4) + 4*g + r%4.
    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      sacc = mfma32x32x16(lds_bf16x8(tk + l32 * TP + es * 16 + 8 * g), qf[es], sacc);
      dpacc = mfma32x32x16(lds_bf16x8(tv + l32 * TP + es * 16 + 8 * g), dof[es], dpacc);
    }

    const bool need_mask = (k0 + 31 > (CAUSAL ? min(q0, p.Sk - 1) : p.Sk - 1));
    const int lim = key_limit - k0 - 4 * g;
    bf16x8 dsb[2];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      uint32_t kbits = 0xF;
      if (DROPOUT) {
        const PhiloxOut w = philox4x32_10(drow + (uint32_t)(k0 >> 2) + 2 * cg + g, p.drop.seed_lo,
                                          p.drop.seed_hi);
        kbits = (w.w[0] >= p.drop.threshold ? 1u : 0u) | (w.w[1] >= p.drop.threshold ? 2u : 0u) |
                (w.w[2] >= p.drop.threshold ? 4u : 0u) | (w.w[3] >= p.drop.threshold ? 8u : 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * cg + u;
        float x = fmaf(sacc[r], c, -lse2);
        if (need_mask) x = (8 * cg + u <= lim) ? x : -INFINITY;
        const float ps = fast_exp2(x);
        float dp = dpacc[r];
        if (DROPOUT) dp = ((kbits >> u) & 1) ? dp * p.drop.keep_scale : 0.f;
        dsb[r >> 3][r & 7] = (__bf16)(ps * (dp - dsum));
      }
    }
    // dQ^T += K^T dS'^T: A = K^T read transposed from the tile, B = dS'^T from registers.
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint16_t* ak = tk + (16 * hf + tr_row) * TP + eb * 32 + tr_col;
        dqa[eb] = mfma32x32x16(concat(lds_tr4(ak), lds_tr4(ak + 8 * TP)), dsb[hf], dqa[eb]);
      }
  }

  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
  uint16_t* dqp = p.dq + b * p.sdq.b + h * p.sdq.h;
  pair_reduce_store<E>(dqa, 1.f, dqp, p.sdq.s, q0, p.Sq, red, qsb, ks == 1, lane);
}

// Workgroup order: per head, dK/dV and dQ blocks alternate, heaviest causal
// blocks first; all blocks of a head sit on one XCD when the head count allows.
template <int E, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(256) void bwd_kernel(BwdParams p, int nkb, int nqb) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[BwdCfg<E>::TOTAL];
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
  const int m = min(nkb, nqb);
  bool dkdv;
  int rank;
  if (slot < 2 * m) {
    dkdv = (slot & 1) == 0;
    rank = slot >> 1;
  } else {
    dkdv = nkb > nqb;
    rank = slot - m;
  }
  if (dkdv)
    role_dkdv<E, CAUSAL, DROPOUT>(p, bh, rank, lds);
  else
    role_dq<E, CAUSAL, DROPOUT>(p, bh, CAUSAL ? nqb - 1 - rank : rank, lds);
}

template <int E>
hipError_t launch_bwd_t(const BwdParams& p, bool causal, bool dropout, hipStream_t stream) {
  const int nkb = (p.Sk + 63) / 64, nqb = (p.Sq + 63) / 64;
  const dim3 grid((unsigned)(nkb + nqb) * (unsigned)(p.B * p.H));
  if (causal) {
    if (dropout)
      hipLaunchKernelGGL((bwd_kernel<E, true, true>), grid, dim3(256), 0, stream, p, nkb, nqb);
    else
      hipLaunchKernelGGL((bwd_kernel<E, true, false>), grid, dim3(256), 0, stream, p, nkb, nqb);
  } else {
    if (dropout)
      hipLaunchKernelGGL((bwd_kernel<E, false, true>), grid, dim3(256), 0, stream, p, nkb, nqb);
    else
      hipLaunchKernelGGL((bwd_kernel<E, false, false>), grid, dim3(256), 0, stream, p, nkb, nqb);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int E, bool causal, bool dropout, hipStream_t stream) {
  return E == 64 ? launch_bwd_t<64>(p, causal, dropout, stream)
                 : launch_bwd_t<128>(p, causal, dropout, stream);
}

}  // namespace sdpa14

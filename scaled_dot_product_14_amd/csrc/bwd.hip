// Fused attention backward for gfx950, recomputing the probabilities from the
// stashed log-sum-exp (nvFuser issue 2278: what the forward stashes is chosen
// by what the backward needs; here O and LSE are stashed and P is recomputed).
// The backward statement follows sdpfa_bwd of the nvFuser PR "DID loop split
// for SDPA"; dropout regenerates the forward's mask from (seed, offset) and the
// absolute element index (PyTorch PR "REDO of dropout support for mem eff").
//
// One launch, two workgroup roles, no atomics and no workspace:
//
//   dK/dV role  a 32-key block.  Each of the 4 waves keeps the block's K and V
//               fragments and its own dK^T, dV^T accumulators in registers and
//               walks every 4th 32-row query tile that can see the block:
//                 S   = Q K^T, dPd = dO V^T        (lane = key, registers = rows)
//                 Ps  = scale * exp(S*scale - LSE) (masked; dropout kept/scaled)
//                 dS' = Ps * (dP - D)              (= scale * dS)
//                 dV^T += dO^T Pd,  dK^T += Q^T dS'
//               Q and dO rows arrive in registers already in the A-operand
//               layout of S and dPd; a copy goes to a wave-private LDS tile for
//               the transposed reads of dO^T and Q^T (ds_read_b64_tr_b16).
//               D_i = rowsum(dO * O) is formed from O rows on the fly.  The
//               four partial dK, dV are summed through LDS at the end.
//   dQ role     a 32-row query block.  Each wave keeps the block's Q and dO
//               fragments, D and LSE in registers and walks every 4th 32-key
//               tile:  S^T = K Q^T, dP^T = V dO^T (lane = row), dS'^T as above,
//               dQ^T += K^T dS'^T with K^T read transposed from a wave-private
//               LDS copy of the tile and dS'^T taken straight from registers.
//               The four partial dQ are summed through LDS at the end.
//
// Both roles recompute S and dP, so the backward does 7 products of 2*E flops
// per visible score element (5 are counted).  In exchange dQ needs neither
// fp32 atomics nor a zeroed accumulator nor a conversion pass, every output is
// bitwise reproducible, and a small causal problem gets twice as many
// independent workgroups.
#include "device_common.h"
#include "kernels.h"

namespace sdpa14 {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// Per-wave LDS footprint (bytes) of both roles, and of the final reduction.
template <int E>
struct BwdLds {
  static constexpr int TP = E + 32;  // tile pitch (elements): conflict-free transposed reads
  static constexpr int TILE = 32 * TP * 2;
  static constexpr int WAVE = 2 * TILE + 64 * 4;   // dK/dV role: Q, dO tiles, D and LSE rows
  static constexpr int RED = 4 * (E / 32) * 16 * 64 * 4;  // one fp32 accumulator per wave
  static constexpr int TOTAL = (4 * WAVE > RED) ? 4 * WAVE : RED;
};

// Sums the four waves' accumulators acc[E/32] (C layout: lane = output row
// row0 + l32, register r = column 32*eb + 8*(r/4) + 4*g + r%4), scales by mul and
// stores bf16 rows below `limit`.  Wave w stores every 4th group of 4 columns.
template <int E>
__device__ __forceinline__ void reduce_store(const f32x16 (&acc)[E / 32], float mul,
                                             uint16_t* dst, int64_t stride, int row0, int limit,
                                             unsigned char* lds, int wave, int lane) {
  constexpr int NEB = E / 32;
  float* red = reinterpret_cast<float*>(lds);
  __syncthreads();  // every wave is done with the LDS it used before
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave * NEB + eb) * 16 + r) * 64 + lane] = acc[eb][r];
  __syncthreads();
  const int row = row0 + (lane & 31);
  const int g = lane >> 5;
#pragma unroll
  for (int gi = wave; gi < NEB * 4; gi += 4) {
    const int eb = gi >> 2, cg = gi & 3;
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) s += red[((w * NEB + eb) * 16 + 4 * cg + t) * 64 + lane];
      v[t] = s * mul;
    }
    if (row < limit)
      *reinterpret_cast<uint2*>(dst + (int64_t)row * stride + eb * 32 + 8 * cg + 4 * g) =
          pack_bf16x4(v[0], v[1], v[2], v[3]);
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

// ---------------------------------------------------------------------------
template <int E, bool CAUSAL, bool DROPOUT>
__device__ __forceinline__ void role_dkdv(const BwdParams& p, int bh, int kblk,
                                          unsigned char* lds) {
  constexpr int NES = E / 16, NEB = E / 32;
  using L = BwdLds<E>;
  constexpr int TP = L::TP;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int kb0 = kblk * 32;
  const int key = kb0 + l32;
  const float c = p.scale_log2;
  const float lsc = __log2f(p.scale);

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
  const uint16_t* op = p.o + b * p.so.b + h * p.so.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;
  const float* lsep = p.lse + (int64_t)bh * p.Sq;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp, (uint32_t)(((int64_t)(p.Sq - 1) * p.sq.s + E) * 2));
  const __amdgpu_buffer_rsrc_t dor = make_rsrc(dop, (uint32_t)(((int64_t)(p.Sq - 1) * p.sdo.s + E) * 2));
  const __amdgpu_buffer_rsrc_t orr = make_rsrc(op, (uint32_t)(((int64_t)(p.Sq - 1) * p.so.s + E) * 2));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp, (uint32_t)(((int64_t)(p.Sk - 1) * p.sk.s + E) * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp, (uint32_t)(((int64_t)(p.Sk - 1) * p.sv.s + E) * 2));

  // K, V of the block as B operands of S = Q K^T and dPd = dO V^T: lane = key,
  // e = 16*es + 8*g + 0..7.  Keys past Sk read as zeros.
  bf16x8 kf[NES], vf[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es) {
    const uint32_t off16 = (uint32_t)(es * 16 + 8 * g) * 2u;
    kf[es] = __builtin_bit_cast(bf16x8, buffer_load16(kr, (uint32_t)key * (uint32_t)(p.sk.s * 2) + off16));
    vf[es] = __builtin_bit_cast(bf16x8, buffer_load16(vr, (uint32_t)key * (uint32_t)(p.sv.s * 2) + off16));
  }

  f32x16 dva[NEB], dka[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    dva[eb] = zero16();
    dka[eb] = zero16();
  }

  const int nqt = (p.Sq + 31) / 32;
  const int t0 = CAUSAL ? ((kb0 < p.Sq) ? kb0 / 32 : nqt) : 0;
  uint16_t* ql = reinterpret_cast<uint16_t*>(lds + wave * L::WAVE);
  uint16_t* dol = ql + 32 * TP;
  float* rv = reinterpret_cast<float*>(dol + 32 * TP);  // D[32], LSE2[32]
  // Transposed-read addressing: contraction slot (g, i) <-> tile row
  // 8*(i/4) + 4*g + i%4 (the C-register order of S); see device_common.h.
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t qs2 = (uint32_t)(p.sq.s * 2), dos2 = (uint32_t)(p.sdo.s * 2),
                 os2 = (uint32_t)(p.so.s * 2);
  const int sk4 = (p.Sk + 3) >> 2;

  bf16x8 qa[NES], doa[NES], oa[NES];
  float lse_v = 0.f;
  auto load_tile = [&](int t, bf16x8 (&q_)[NES], bf16x8 (&d_)[NES], bf16x8 (&o_)[NES], float& l_) {
    const uint32_t row = (uint32_t)(t * 32 + l32);
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      const uint32_t off16 = (uint32_t)(es * 16 + 8 * g) * 2u;
      q_[es] = __builtin_bit_cast(bf16x8, buffer_load16(qr, row * qs2 + off16));
      d_[es] = __builtin_bit_cast(bf16x8, buffer_load16(dor, row * dos2 + off16));
      o_[es] = __builtin_bit_cast(bf16x8, buffer_load16(orr, row * os2 + off16));
    }
    l_ = ((int)row < p.Sq) ? lsep[row] : 0.f;
  };

  int t = t0 + wave;
  if (t < nqt) load_tile(t, qa, doa, oa, lse_v);
  for (; t < nqt; t += 4) {
    const int q0 = t * 32;
    // Stage the rows for the transposed reads, and the per-row D and LSE.
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      *reinterpret_cast<bf16x8*>(ql + l32 * TP + es * 16 + 8 * g) = qa[es];
      *reinterpret_cast<bf16x8*>(dol + l32 * TP + es * 16 + 8 * g) = doa[es];
    }
    float dpart = 0.f;
#pragma unroll
    for (int es = 0; es < NES; ++es)
#pragma unroll
      for (int i = 0; i < 8; ++i) dpart = fmaf((float)doa[es][i], (float)oa[es][i], dpart);
    const float dsum = pair_sum(dpart);
    if (g == 0) {
      rv[l32] = dsum;
      rv[32 + l32] = lse_v * kLog2e - lsc;  // exp2(S*c - this) = scale * P
    }

    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      sacc = mfma32x32x16(qa[es], kf[es], sacc);
      dpacc = mfma32x32x16(doa[es], vf[es], dpacc);
    }
    bf16x8 qn[NES], don[NES], on[NES];
    float lsen = 0.f;
    if (t + 4 < nqt) load_tile(t + 4, qn, don, on, lsen);
    __builtin_amdgcn_wave_barrier();

    // C layout: lane = key, register r = row q0 + 8*(r/4) + 4*g + r%4.
    const bool need_mask = (CAUSAL && q0 == kb0) || (q0 + 31 >= p.Sq) || (kb0 + 31 >= p.Sk);
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      const float4 dv4 = *reinterpret_cast<const float4*>(rv + 8 * cg + 4 * g);
      const float4 lv4 = *reinterpret_cast<const float4*>(rv + 32 + 8 * cg + 4 * g);
      const float dvals[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
      const float lvals[4] = {lv4.x, lv4.y, lv4.z, lv4.w};
      uint32_t kbits = 0xF;
      if (DROPOUT) kbits = keep_bits_for_key(p.drop, bh, p.Sq, sk4, q0 + 8 * cg + 4 * g, key, lane);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * cg + u;
        const int qrow = q0 + 8 * cg + 4 * g + u;
        bool ok = true;
        if (need_mask) ok = (qrow < p.Sq) && (key < p.Sk) && (!CAUSAL || key <= qrow);
        const float ps = ok ? fast_exp2(fmaf(sacc[r], c, -lvals[u])) : 0.f;
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
        const uint16_t* ad = dol + (16 * hf + tr_row) * TP + eb * 32 + tr_col;
        dva[eb] = mfma32x32x16(concat(lds_tr4(ad), lds_tr4(ad + 8 * TP)), pb[hf], dva[eb]);
        const uint16_t* aq = ql + (16 * hf + tr_row) * TP + eb * 32 + tr_col;
        dka[eb] = mfma32x32x16(concat(lds_tr4(aq), lds_tr4(aq + 8 * TP)), dsb[hf], dka[eb]);
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      qa[es] = qn[es];
      doa[es] = don[es];
      oa[es] = on[es];
    }
    lse_v = lsen;
  }

  // dV = (1/scale) * sum(Pd^T dO) since Pd carries the scale; dK carries it already.
  uint16_t* dvp = p.dv + b * p.sdv.b + h * p.sdv.h;
  uint16_t* dkp = p.dk + b * p.sdk.b + h * p.sdk.h;
  reduce_store<E>(dva, 1.f / p.scale, dvp, p.sdv.s, kb0, p.Sk, lds, wave, lane);
  reduce_store<E>(dka, 1.f, dkp, p.sdk.s, kb0, p.Sk, lds, wave, lane);
}

// ---------------------------------------------------------------------------
template <int E, bool CAUSAL, bool DROPOUT>
__device__ __forceinline__ void role_dq(const BwdParams& p, int bh, int qblk, unsigned char* lds) {
  constexpr int NES = E / 16, NEB = E / 32;
  using L = BwdLds<E>;
  constexpr int TP = L::TP;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0 = qblk * 32;
  const int qrow = q0 + l32;
  const float c = p.scale_log2;

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
  const uint16_t* op = p.o + b * p.so.b + h * p.so.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp, (uint32_t)(((int64_t)(p.Sq - 1) * p.sq.s + E) * 2));
  const __amdgpu_buffer_rsrc_t dor = make_rsrc(dop, (uint32_t)(((int64_t)(p.Sq - 1) * p.sdo.s + E) * 2));
  const __amdgpu_buffer_rsrc_t orr = make_rsrc(op, (uint32_t)(((int64_t)(p.Sq - 1) * p.so.s + E) * 2));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp, (uint32_t)(((int64_t)(p.Sk - 1) * p.sk.s + E) * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp, (uint32_t)(((int64_t)(p.Sk - 1) * p.sv.s + E) * 2));

  // Q, dO of this row as B operands of S^T = K Q^T and dP^T = V dO^T; D and LSE of the row.
  bf16x8 qf[NES], dof[NES];
  float dpart = 0.f;
#pragma unroll
  for (int es = 0; es < NES; ++es) {
    const uint32_t off16 = (uint32_t)(es * 16 + 8 * g) * 2u;
    qf[es] = __builtin_bit_cast(bf16x8, buffer_load16(qr, (uint32_t)qrow * (uint32_t)(p.sq.s * 2) + off16));
    dof[es] = __builtin_bit_cast(bf16x8, buffer_load16(dor, (uint32_t)qrow * (uint32_t)(p.sdo.s * 2) + off16));
    const bf16x8 o8 = __builtin_bit_cast(bf16x8, buffer_load16(orr, (uint32_t)qrow * (uint32_t)(p.so.s * 2) + off16));
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart = fmaf((float)dof[es][i], (float)o8[i], dpart);
  }
  const float dsum = pair_sum(dpart);
  const float lse2 =
      ((qrow < p.Sq) ? p.lse[(int64_t)bh * p.Sq + qrow] * kLog2e : 0.f) - __log2f(p.scale);

  f32x16 dqa[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) dqa[eb] = zero16();

  const int nkt = (p.Sk + 31) / 32;
  const int kt_end = CAUSAL ? min(nkt, min(q0 + 31, p.Sq - 1) / 32 + 1) : nkt;
  uint16_t* kl = reinterpret_cast<uint16_t*>(lds + wave * L::WAVE);
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t ks2 = (uint32_t)(p.sk.s * 2), vs2 = (uint32_t)(p.sv.s * 2);
  const int key_limit = CAUSAL ? min(qrow, p.Sk - 1) : p.Sk - 1;
  const int sk4 = (p.Sk + 3) >> 2;
  uint64_t drow = 0;
  if (DROPOUT) drow = philox_row_base(p.drop, bh, p.Sq, qrow, sk4);

  bf16x8 ka[NES], va[NES];
  auto load_tile = [&](int j, bf16x8 (&k_)[NES], bf16x8 (&v_)[NES]) {
    const uint32_t row = (uint32_t)(j * 32 + l32);
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      const uint32_t off16 = (uint32_t)(es * 16 + 8 * g) * 2u;
      k_[es] = __builtin_bit_cast(bf16x8, buffer_load16(kr, row * ks2 + off16));
      v_[es] = __builtin_bit_cast(bf16x8, buffer_load16(vr, row * vs2 + off16));
    }
  };

  int j = wave;
  if (j < kt_end) load_tile(j, ka, va);
  for (; j < kt_end; j += 4) {
    const int k0 = j * 32;
#pragma unroll
    for (int es = 0; es < NES; ++es)
      *reinterpret_cast<bf16x8*>(kl + l32 * TP + es * 16 + 8 * g) = ka[es];

    // S^T, dP^T: lane = row, register r = key k0 + 8*(r/4) + 4*g + r%4.
    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      sacc = mfma32x32x16(ka[es], qf[es], sacc);
      dpacc = mfma32x32x16(va[es], dof[es], dpacc);
    }
    bf16x8 kn[NES], vn[NES];
    if (j + 4 < kt_end) load_tile(j + 4, kn, vn);
    __builtin_amdgcn_wave_barrier();

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
        const bool ok = !need_mask || (8 * cg + u <= lim);
        const float ps = ok ? fast_exp2(fmaf(sacc[r], c, -lse2)) : 0.f;
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
        const uint16_t* ak = kl + (16 * hf + tr_row) * TP + eb * 32 + tr_col;
        dqa[eb] = mfma32x32x16(concat(lds_tr4(ak), lds_tr4(ak + 8 * TP)), dsb[hf], dqa[eb]);
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      ka[es] = kn[es];
      va[es] = vn[es];
    }
  }

  uint16_t* dqp = p.dq + b * p.sdq.b + h * p.sdq.h;
  reduce_store<E>(dqa, 1.f, dqp, p.sdq.s, q0, p.Sq, lds, wave, lane);
}

// Workgroup order: per head, the dK/dV and dQ blocks alternate, heaviest causal
// blocks first; all blocks of a head sit on one XCD when the head count allows.
template <int E, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(256) void bwd_kernel(BwdParams p, int nkb, int nqb) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[BwdLds<E>::TOTAL];
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
  const int nkb = (p.Sk + 31) / 32, nqb = (p.Sq + 31) / 32;
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

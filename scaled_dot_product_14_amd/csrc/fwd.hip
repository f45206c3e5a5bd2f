// Fused attention forward for gfx950: O = dropout(softmax(scale * Q K^T + mask)) V
// and the per-row log-sum-exp, in one pass over the keys (flash-style tiling:
// the score matrix is never written to memory; the softmax is kept online with
// a running row maximum and row sum).
//
// What is computed follows the forward statement of the nvFuser PR "DID loop
// split for SDPA" (sdpfa_fwd returns attn, log_sumexp, seed, offset) and the
// dropout of the PyTorch PR "REDO of dropout support for mem eff" (absolute
// index for the RNG stream).  The tiling is this file's own design for CDNA4.
//
// Workgroup: NW waves, each owning 32 query rows (BM = 32*NW rows per
// workgroup).  Key/value tiles of BN rows are staged in LDS, shared by the
// waves, with the next tile's global loads in flight while the current one is
// consumed.
//
// Per wave and key tile:
//   S^T = K_tile Q^T       v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                          B = Q fragments held in registers for the whole loop.
//                          Result layout: lane = query (l%32), registers run
//                          over keys, four consecutive keys per register group.
//   online softmax         every lane owns one query row; row statistics need
//                          one exchange with lane l^32 (permlane32_swap).
//   dropout                the four consecutive keys of a register group are
//                          exactly one Philox call.
//   O^T += V^T P^T         A = V^T read transposed from the row-major V tile
//                          (ds_read_b64_tr_b16), B = P taken straight from the
//                          S^T registers (converted to bf16): no LDS round trip
//                          for P.  The contraction index is permuted
//                          consistently on both operands.
// The O^T accumulator keeps lane = query, so the rescale by exp(m_old - m_new)
// is a per-lane multiply.
#include "device_common.h"
#include "kernels.h"

namespace sdpa14 {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;

template <int E, int NW, int BN, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdParams p, int n_qtiles) {
  static_assert(E % 32 == 0 && BN % 32 == 0, "tile shape");
  constexpr int BM = NW * 32;
  constexpr int KP = E + 8;   // K tile pitch (elements): conflict-free 16-byte row reads
  constexpr int VP = E + 32;  // V tile pitch: conflict-free transposed reads
  constexpr int NT = NW * 64;
  constexpr int CPR = E / 8;  // 16-byte chunks per row
  constexpr int CHUNKS = BN * CPR;
  constexpr int PER = (CHUNKS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vs[BN * VP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh_count = p.B * p.H;
  const int rank = blockIdx.x / bh_count;
  const int bh = blockIdx.x - rank * bh_count;
  // Causal tiles with more keys go first.
  const int qt = CAUSAL ? (n_qtiles - 1 - rank) : rank;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int q0 = qt * BM + wave * 32;  // first query row of this wave
  const int qrow = q0 + l32;           // query row of this lane

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;

  // Q as the B operand of S^T = K Q^T: lane holds its row, e = 16*es + 8*g + 0..7.
  bf16x8 qf[E / 16];
#pragma unroll
  for (int es = 0; es < E / 16; ++es)
    qf[es] = (qrow < p.Sq) ? load_bf16x8(qp + (int64_t)qrow * p.sq.s + es * 16 + 8 * g)
                           : zero_bf16x8();

  int kend = p.Sk;
  if (CAUSAL) kend = min(kend, min(p.Sq, (qt + 1) * BM));  // keys <= last row of the tile
  const int n_kt = (kend + BN - 1) / BN;

  uint4 kreg[PER], vreg[PER];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, col = c - (c / CPR) * CPR;
      const int key = k0 + row;
      if (c < CHUNKS && key < p.Sk) {
        kreg[i] = *reinterpret_cast<const uint4*>(kp + (int64_t)key * p.sk.s + col * 8);
        vreg[i] = *reinterpret_cast<const uint4*>(vp + (int64_t)key * p.sv.s + col * 8);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      if (c < CHUNKS) {
        const int row = c / CPR, col = c - (c / CPR) * CPR;
        *reinterpret_cast<uint4*>(ks + row * KP + col * 8) = kreg[i];
        *reinterpret_cast<uint4*>(vs + row * VP + col * 8) = vreg[i];
      }
    }
  };

  // Transposed-read addressing for the V^T operand (see device_common.h): lane
  // reads rows 4*g + (lane%16)/4 (+8), columns 16*((lane/16)%2) + 4*(lane%4).
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 oacc[E / 32];
#pragma unroll
  for (int eb = 0; eb < E / 32; ++eb) oacc[eb] = zero16();
  float m_run = -INFINITY;  // running max of scale*log2(e)*S for this row
  float l_run = 0.f;        // this lane's share of the running row sum
  const float c = p.scale_log2;

  const int sk4 = (p.Sk + 3) >> 2;
  uint64_t drow = 0;
  if (DROPOUT) drow = philox_row_base(p.drop, bh, p.Sq, qrow, sk4);

  if (n_kt > 0) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(k0 + BN);
    if (CAUSAL && k0 > q0 + 31) continue;  // tile lies above the diagonal for this wave

    // S^T for BN keys x 32 queries.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int es = 0; es < E / 16; ++es) {
        const bf16x8 a = lds_bf16x8(ks + (kb * 32 + l32) * KP + es * 16 + 8 * g);
        s[kb] = mfma32x32x16(a, qf[es], s[kb]);
      }
    }

    const bool need_mask = (CAUSAL && (k0 + BN - 1 > q0)) || (k0 + BN > p.Sk);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool ok = (key < p.Sk) && (!CAUSAL || key <= qrow);
          if (!ok) s[kb][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(s[kb][r], c, -m_new));
        s[kb][r] = pv;
        rs += pv;
      }
    l_run = l_run * alpha + rs;

    if (DROPOUT) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          // keys k0 + 32*kb + 8*cg + 4*g + 0..3: one Philox group
          const uint32_t grp = (uint32_t)(k0 >> 2) + kb * 8 + cg * 2 + g;
          const PhiloxOut w = philox4x32_10(drow + grp, p.drop.seed_lo, p.drop.seed_hi);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (w.w[t] < p.drop.threshold) s[kb][4 * cg + t] = 0.f;
        }
    }

#pragma unroll
    for (int eb = 0; eb < E / 32; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[eb][r] *= alpha;

    // P as the B operand: 16-key step ks takes registers 8*(ks%2)..+7 of block ks/2,
    // i.e. keys 16*ks + 8*(i/4) + 4*g + i%4 for element i.
    bf16x8 pb[BN / 16];
#pragma unroll
    for (int ksx = 0; ksx < BN / 16; ++ksx)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[ksx][i] = (__bf16)s[ksx >> 1][8 * (ksx & 1) + i];

#pragma unroll
    for (int eb = 0; eb < E / 32; ++eb)
#pragma unroll
      for (int ksx = 0; ksx < BN / 16; ++ksx) {
        const uint16_t* base = vs + (ksx * 16 + tr_row) * VP + eb * 32 + tr_col;
        const bf16x8 a = concat(lds_tr4(base), lds_tr4(base + 8 * VP));
        oacc[eb] = mfma32x32x16(a, pb[ksx], oacc[eb]);
      }
  }

  const float l_tot = pair_sum(l_run);
  const float inv = (DROPOUT ? p.drop.keep_scale : 1.f) / l_tot;
  if (qrow < p.Sq) {
    uint16_t* op = p.o + b * p.so.b + h * p.so.h + (int64_t)qrow * p.so.s;
#pragma unroll
    for (int eb = 0; eb < E / 32; ++eb)
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const int e = eb * 32 + 8 * cg + 4 * g;
        *reinterpret_cast<uint2*>(op + e) =
            pack_bf16x4(oacc[eb][4 * cg + 0] * inv, oacc[eb][4 * cg + 1] * inv,
                        oacc[eb][4 * cg + 2] * inv, oacc[eb][4 * cg + 3] * inv);
      }
    if (g == 0) p.lse[(int64_t)bh * p.Sq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int E, int NW, int BN>
hipError_t launch_fwd_t(const FwdParams& p, bool causal, bool dropout, hipStream_t stream) {
  constexpr int BM = NW * 32;
  const int n_qtiles = (p.Sq + BM - 1) / BM;
  const dim3 grid((unsigned)n_qtiles * (unsigned)(p.B * p.H));
  const dim3 block(NW * 64);
  if (causal) {
    if (dropout)
      hipLaunchKernelGGL((fwd_kernel<E, NW, BN, true, true>), grid, block, 0, stream, p, n_qtiles);
    else
      hipLaunchKernelGGL((fwd_kernel<E, NW, BN, true, false>), grid, block, 0, stream, p, n_qtiles);
  } else {
    if (dropout)
      hipLaunchKernelGGL((fwd_kernel<E, NW, BN, false, true>), grid, block, 0, stream, p, n_qtiles);
    else
      hipLaunchKernelGGL((fwd_kernel<E, NW, BN, false, false>), grid, block, 0, stream, p, n_qtiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int E, bool causal, bool dropout,
                      const TileChoice& tiles, hipStream_t stream) {
  int nw = tiles.fwd_waves;
  if (nw != 2 && nw != 4) {
    // Fill the chip: prefer 4-wave workgroups unless that leaves fewer than two
    // workgroups per compute unit.
    const long wg4 = (long)((p.Sq + 127) / 128) * p.B * p.H;
    nw = (wg4 >= 512) ? 4 : 2;
  }
  if (E == 64) {
    return nw == 4 ? launch_fwd_t<64, 4, 64>(p, causal, dropout, stream)
                   : launch_fwd_t<64, 2, 64>(p, causal, dropout, stream);
  }
  return nw == 4 ? launch_fwd_t<128, 4, 64>(p, causal, dropout, stream)
                 : launch_fwd_t<128, 2, 64>(p, causal, dropout, stream);
}

}  // namespace sdpa14

// Fused attention backward for gfx950, recomputing the probabilities from the
// stashed log-sum-exp (nvFuser issue 2278: what the forward stashes is chosen
// by what the backward needs; here O and LSE are stashed and P is recomputed).
// The backward statement follows sdpfa_bwd of the nvFuser PR "DID loop split
// for SDPA"; dropout regenerates the forward's mask from (seed, offset) and the
// absolute element index (PyTorch PR "REDO of dropout support for mem eff").
//
// Three kernels, in stream order:
//   1. bwd_pre:  D_i = sum_e dO_ie * O_ie (fp32), and zero the fp32 dQ accumulator.
//                Memory-bound: one read of dO and O, one write of dQ_acc.
//   2. bwd_main: key-block parallel.  A workgroup owns 128 keys (32 per wave),
//                keeps K and V fragments in registers and dK, dV accumulators in
//                registers, and walks the query tiles (64 rows each) that can see
//                its keys.  Per wave and 32-row query block:
//                  S   = Q K_w^T           (A = Q rows from LDS, B = K_w in registers)
//                  dPd = dO V_w^T          (A = dO rows from LDS, B = V_w in registers)
//                  P   = exp2(S*scale*log2e - LSE*log2e); dropout mask M;
//                  dS  = P * (dPd*M - D) * scale
//                  dV^T += dO^T (P*M)       (A = dO read transposed from LDS,
//                  dK^T += Q^T dS            B = P*M / dS straight from registers)
//                dS goes to LDS; then each wave computes one 32x32 block of
//                  dQ = dS K                (A = dS, B = K, both read transposed)
//                and adds it to the fp32 accumulator with global float atomics.
//   3. bwd_dq:   dQ = bf16(dQ_acc) in q's stride order.
#include "device_common.h"
#include "kernels.h"

namespace sdpa14 {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O) and dQ_acc = 0.
template <int E>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = E / 8;        // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;    // rows per workgroup
  const int tid = threadIdx.x;
  const int c = tid % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;  // over B*H*Sq
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  float acc = 0.f;
  if (row < rows) {
    const int bh = (int)(row / p.Sq);
    const int qi = (int)(row - (int64_t)bh * p.Sq);
    const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
    const bf16x8 d = load_bf16x8(p.dout + b * p.sdo.b + h * p.sdo.h + (int64_t)qi * p.sdo.s + c * 8);
    const bf16x8 o = load_bf16x8(p.o + b * p.so.b + h * p.so.h + (int64_t)qi * p.so.s + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)d[i], (float)o[i], acc);
    float4* z = reinterpret_cast<float4*>(p.dq_acc + row * E + c * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. Main pass.
template <int E, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdParams p, int n_kblocks) {
  constexpr int BK = 128;     // keys per workgroup, 32 per wave
  constexpr int BQ = 64;      // query rows per iteration
  constexpr int QP = E + 8;   // Q / dO tile pitch (elements)
  constexpr int KP = E + 8;   // K tile pitch
  constexpr int SP = BQ + 8;  // dS tile pitch, stored [key][query]
  constexpr int CPR = E / 8;  // 16-byte chunks per row
  constexpr int QCH = BQ * CPR;
  constexpr int QPER = (QCH + 255) / 256;
  constexpr int NEB = E / 32;                    // 32-wide column blocks of E
  constexpr int DQ_BLOCKS_PER_WAVE = (2 * NEB) / 4;  // dQ tile: 2 row blocks x NEB col blocks

  __shared__ __attribute__((aligned(16))) uint16_t qs[BQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t dos[BQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t kls[BK * KP];
  __shared__ __attribute__((aligned(16))) uint16_t dsl[BK * SP];
  __shared__ float lse_s[BQ];
  __shared__ float d_s[BQ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh_count = p.B * p.H;
  const int kblk = blockIdx.x / bh_count;  // key block 0 (most work when causal) first
  const int bh = blockIdx.x - kblk * bh_count;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int kb0 = kblk * BK;
  const int kw0 = kb0 + 32 * wave;
  const int key = kw0 + l32;  // key column of this lane in S / dP

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;
  const uint16_t* dop = p.dout + b * p.sdo.b + h * p.sdo.h;
  const float* lsep = p.lse + (int64_t)bh * p.Sq;
  const float* dlp = p.delta + (int64_t)bh * p.Sq;
  float* dqa = p.dq_acc + (int64_t)bh * p.Sq * E;

  // K_w, V_w as B operands of S = Q K^T and dPd = dO V^T: lane = key, e = 16*es + 8*g + 0..7.
  bf16x8 kf[E / 16], vf[E / 16];
#pragma unroll
  for (int es = 0; es < E / 16; ++es) {
    if (key < p.Sk) {
      kf[es] = load_bf16x8(kp + (int64_t)key * p.sk.s + es * 16 + 8 * g);
      vf[es] = load_bf16x8(vp + (int64_t)key * p.sv.s + es * 16 + 8 * g);
    } else {
      kf[es] = zero_bf16x8();
      vf[es] = zero_bf16x8();
    }
  }
  // The whole K block in LDS (row-major) for the dQ product.
  for (int cidx = tid; cidx < BK * CPR; cidx += 256) {
    const int row = cidx / CPR, col = cidx - (cidx / CPR) * CPR;
    const int kr = kb0 + row;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kr < p.Sk) val = *reinterpret_cast<const uint4*>(kp + (int64_t)kr * p.sk.s + col * 8);
    *reinterpret_cast<uint4*>(kls + row * KP + col * 8) = val;
  }

  f32x16 dv_acc[NEB], dk_acc[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    dv_acc[eb] = zero16();
    dk_acc[eb] = zero16();
  }

  const int n_qt = (p.Sq + BQ - 1) / BQ;
  int qt_begin = 0;
  if (CAUSAL) qt_begin = (kb0 < p.Sq) ? kb0 / BQ : n_qt;  // queries below kb0 see none of these keys

  // Transposed-read addressing (device_common.h).  "perm": contraction slot
  // (g, i) <-> row 8*(i/4) + 4*g + i%4, matching the C-register order of S.
  // "nat": slot (g, i) <-> row 8*g + i.
  const int tr_row_perm = 4 * g + ((lane & 15) >> 2);
  const int tr_row_nat = 8 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  const float c = p.scale_log2;
  const int sk4 = (p.Sk + 3) >> 2;

  uint4 qreg[QPER], doreg[QPER];
  float lse_r = 0.f, d_r = 0.f;
  auto load_tile = [&](int q0) {
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int cidx = tid + i * 256;
      const int row = cidx / CPR, col = cidx - (cidx / CPR) * CPR;
      const int qr = q0 + row;
      if (cidx < QCH && qr < p.Sq) {
        qreg[i] = *reinterpret_cast<const uint4*>(qp + (int64_t)qr * p.sq.s + col * 8);
        doreg[i] = *reinterpret_cast<const uint4*>(dop + (int64_t)qr * p.sdo.s + col * 8);
      } else {
        qreg[i] = make_uint4(0, 0, 0, 0);
        doreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BQ) {
      const int qr = q0 + tid;
      lse_r = (qr < p.Sq) ? lsep[qr] * kLog2e : 0.f;
      d_r = (qr < p.Sq) ? dlp[qr] : 0.f;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < QPER; ++i) {
      const int cidx = tid + i * 256;
      if (cidx < QCH) {
        const int row = cidx / CPR, col = cidx - (cidx / CPR) * CPR;
        *reinterpret_cast<uint4*>(qs + row * QP + col * 8) = qreg[i];
        *reinterpret_cast<uint4*>(dos + row * QP + col * 8) = doreg[i];
      }
    }
    if (tid < BQ) {
      lse_s[tid] = lse_r;
      d_s[tid] = d_r;
    }
  };

  if (qt_begin < n_qt) load_tile(qt_begin * BQ);
  for (int qt = qt_begin; qt < n_qt; ++qt) {
    const int q0 = qt * BQ;
    __syncthreads();  // previous iteration is done with qs, dos, dsl
    store_tile();
    __syncthreads();
    if (qt + 1 < n_qt) load_tile(q0 + BQ);

#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int qb = q0 + qh * 32;  // first query row of this 32-row block
      uint16_t* dsw = dsl + (32 * wave + l32) * SP + qh * 32 + 4 * g;
      if (CAUSAL && kw0 > qb + 31) {  // every key of this wave is after every row
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) *reinterpret_cast<uint2*>(dsw + 8 * cg) = make_uint2(0, 0);
        continue;
      }
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int es = 0; es < E / 16; ++es) {
        const bf16x8 aq = lds_bf16x8(qs + (qh * 32 + l32) * QP + es * 16 + 8 * g);
        sacc = mfma32x32x16(aq, kf[es], sacc);
        const bf16x8 ad = lds_bf16x8(dos + (qh * 32 + l32) * QP + es * 16 + 8 * g);
        dpacc = mfma32x32x16(ad, vf[es], dpacc);
      }
      // C layout: lane = key, register r = query row qh*32 + 8*(r/4) + 4*g + r%4.
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qh * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const int qa = q0 + ql;
        const bool ok = (qa < p.Sq) && (key < p.Sk) && (!CAUSAL || key <= qa);
        const float pv = ok ? fast_exp2(fmaf(sacc[r], c, -lse_s[ql])) : 0.f;
        float dp = dpacc[r];
        float pd = pv;
        if (DROPOUT) {
          const uint64_t ctr = philox_row_base(p.drop, bh, p.Sq, qa, sk4) + (uint32_t)(key >> 2);
          const PhiloxOut w = philox4x32_10(ctr, p.drop.seed_lo, p.drop.seed_hi);
          const uint32_t word = w.w[key & 3];
          const bool keep = word >= p.drop.threshold;
          pd = keep ? pv * p.drop.keep_scale : 0.f;
          dp = keep ? dp * p.drop.keep_scale : 0.f;
        }
        const float ds = pv * (dp - d_s[ql]) * p.scale;
        pb[r >> 3][r & 7] = (__bf16)pd;
        dsb[r >> 3][r & 7] = (__bf16)ds;
      }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int rb = qh * 32 + 16 * hf + tr_row_perm;
          const uint16_t* ad = dos + rb * QP + eb * 32 + tr_col;
          dv_acc[eb] = mfma32x32x16(concat(lds_tr4(ad), lds_tr4(ad + 8 * QP)), pb[hf], dv_acc[eb]);
          const uint16_t* aq = qs + rb * QP + eb * 32 + tr_col;
          dk_acc[eb] = mfma32x32x16(concat(lds_tr4(aq), lds_tr4(aq + 8 * QP)), dsb[hf], dk_acc[eb]);
        }
      // dS to LDS as [key][query]: registers 4*cg..4*cg+3 are rows 8*cg + 4*g + 0..3.
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        bf16x4 v4;
#pragma unroll
        for (int t = 0; t < 4; ++t) v4[t] = dsb[(4 * cg + t) >> 3][(4 * cg + t) & 7];
        *reinterpret_cast<uint2*>(dsw + 8 * cg) = __builtin_bit_cast(uint2, v4);
      }
    }
    __syncthreads();  // dS of all four waves is in LDS

    // dQ tile [64 rows x E] = dS [64 x 128] K [128 x E]; block (row half, column block).
#pragma unroll
    for (int bi = 0; bi < DQ_BLOCKS_PER_WAVE; ++bi) {
      const int blk = wave * DQ_BLOCKS_PER_WAVE + bi;
      const int rh = blk / NEB;   // 32-row half of the query tile
      const int eb = blk % NEB;   // 32-wide column block
      const int qmax = q0 + rh * 32 + 31;
      if (CAUSAL && kb0 > qmax) continue;  // all of dS is zero here
      int ks_end = BK / 16;
      if (CAUSAL) ks_end = min(ks_end, (qmax - kb0) / 16 + 1);
      f32x16 acc = zero16();
      for (int ksx = 0; ksx < ks_end; ++ksx) {
        const uint16_t* as = dsl + (ksx * 16 + tr_row_nat) * SP + rh * 32 + tr_col;
        const uint16_t* bs = kls + (ksx * 16 + tr_row_nat) * KP + eb * 32 + tr_col;
        const bf16x8 a = concat(lds_tr4(as), lds_tr4(as + 4 * SP));
        const bf16x8 bb = concat(lds_tr4(bs), lds_tr4(bs + 4 * KP));
        acc = mfma32x32x16(a, bb, acc);
      }
      // C layout: lane = column eb*32 + l32, register r = row rh*32 + 8*(r/4) + 4*g + r%4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qa = q0 + rh * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (qa < p.Sq) unsafeAtomicAdd(dqa + (int64_t)qa * E + eb * 32 + l32, acc[r]);
      }
    }
  }

  // dK^T, dV^T: lane = key, register r = column eb*32 + 8*(r/4) + 4*g + r%4.
  if (key < p.Sk) {
    uint16_t* dkp = p.dk + b * p.sdk.b + h * p.sdk.h + (int64_t)key * p.sdk.s;
    uint16_t* dvp = p.dv + b * p.sdv.b + h * p.sdv.h + (int64_t)key * p.sdv.s;
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const int e = eb * 32 + 8 * cg + 4 * g;
        *reinterpret_cast<uint2*>(dkp + e) =
            pack_bf16x4(dk_acc[eb][4 * cg], dk_acc[eb][4 * cg + 1], dk_acc[eb][4 * cg + 2],
                        dk_acc[eb][4 * cg + 3]);
        *reinterpret_cast<uint2*>(dvp + e) =
            pack_bf16x4(dv_acc[eb][4 * cg], dv_acc[eb][4 * cg + 1], dv_acc[eb][4 * cg + 2],
                        dv_acc[eb][4 * cg + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ = bf16(dQ_acc) in q's layout.
template <int E>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  constexpr int TPR = E / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const int64_t row = t / TPR;
  if (row >= rows) return;
  const int c = (int)(t - row * TPR);
  const int bh = (int)(row / p.Sq);
  const int qi = (int)(row - (int64_t)bh * p.Sq);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const float4* src = reinterpret_cast<const float4*>(p.dq_acc + row * E + c * 8);
  const float4 x = src[0], y = src[1];
  uint2 lo = pack_bf16x4(x.x, x.y, x.z, x.w);
  uint2 hi = pack_bf16x4(y.x, y.y, y.z, y.w);
  *reinterpret_cast<uint4*>(p.dq + b * p.sdq.b + h * p.sdq.h + (int64_t)qi * p.sdq.s + c * 8) =
      make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <int E>
hipError_t launch_main_t(const BwdParams& p, bool causal, bool dropout, hipStream_t stream) {
  const int n_kblocks = (p.Sk + 127) / 128;
  const dim3 grid((unsigned)n_kblocks * (unsigned)(p.B * p.H));
  if (causal) {
    if (dropout)
      hipLaunchKernelGGL((bwd_main_kernel<E, true, true>), grid, dim3(256), 0, stream, p, n_kblocks);
    else
      hipLaunchKernelGGL((bwd_main_kernel<E, true, false>), grid, dim3(256), 0, stream, p, n_kblocks);
  } else {
    if (dropout)
      hipLaunchKernelGGL((bwd_main_kernel<E, false, true>), grid, dim3(256), 0, stream, p, n_kblocks);
    else
      hipLaunchKernelGGL((bwd_main_kernel<E, false, false>), grid, dim3(256), 0, stream, p, n_kblocks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const BwdParams& p, int E, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const int rpb = 256 / (E / 8);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (E == 64)
    hipLaunchKernelGGL(bwd_pre_kernel<64>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<128>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdParams& p, int E, bool causal, bool dropout,
                           hipStream_t stream) {
  return E == 64 ? launch_main_t<64>(p, causal, dropout, stream)
                 : launch_main_t<128>(p, causal, dropout, stream);
}

hipError_t launch_bwd_dq(const BwdParams& p, int E, hipStream_t stream) {
  const int64_t threads = (int64_t)p.B * p.H * p.Sq * (E / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (E == 64)
    hipLaunchKernelGGL(bwd_dq_kernel<64>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<128>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sdpa14

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
// Workgroup: NQ x NS waves.  Each wave owns 32 query rows (a workgroup covers
// BM = 32*NQ rows) and one of NS interleaved shares of the key tiles: at
// iteration `it` the workgroup stages NS key/value tiles of BN rows in LDS and
// wave (qs, ks) consumes tile it*NS + ks for query sub-tile qs.  The NS partial
// softmax states (max, sum, O) of a query sub-tile are merged through LDS at
// the end.  Splitting the keys shortens the longest chain of dependent tiles,
// which is what limits small causal problems.
//
// Per wave and key tile:
//   S^T = K_tile Q^T       v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                          B = Q fragments held in registers for the whole loop.
//                          Result layout: lane = query (l%32), registers run
//                          over keys, four consecutive keys per register group.
//   online softmax         every lane owns one query row; the row max needs one
//                          exchange with lane l^32 (permlane32_swap).  The
//                          reference is lazy: the row maximum is taken only on a
//                          row's first visible tile and when a tile's sum shows
//                          that a probability may pass 2^16 (in the exp2
//                          domain), so most tiles take no maximum and skip the
//                          rescale of the O accumulator; probabilities stay
//                          below 2^16, harmless for fp32 sums and bf16 operands.
//   dropout                the four consecutive keys of a register group are
//                          exactly one Philox call.
//   O^T += V^T P^T         A = V^T read transposed from the row-major V tile
//                          (ds_read_b64_tr_b16), B = P taken straight from the
//                          S^T registers (converted to bf16): no LDS round trip
//                          for P.  The contraction index is permuted
//                          consistently on both operands.
// The O^T accumulator keeps lane = query, so every rescale is a per-lane multiply.
//
// Workgroup order: heaviest causal query tiles first, and the tiles of one head
// on one XCD (workgroups are dealt to the 8 XCDs round-robin), so a head's K/V
// stay in that XCD's L2.  When the whole grid is resident at once, every
// workgroup asks for its Q and first K/V stage at the same moment; a light
// causal tile then waits a little before its first loads (longer the fewer
// steps it has), so that the heaviest tiles, which set the kernel's length,
// are served first.
#include <algorithm>
#include <type_traits>

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

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLazyLimit = 65536.f;  // a lane's tile sum above this re-takes the row maximum

// Maps a workgroup id to (head, rank); rank 0 is the heaviest query tile.
__device__ __forceinline__ void wg_to_tile(int bid, int bh_count, int& bh, int& rank) {
  if ((bh_count & 7) == 0) {
    const int per_xcd = bh_count >> 3;
    const int xcd = bid & 7, slot = bid >> 3;
    rank = slot / per_xcd;
    bh = xcd * per_xcd + (slot - rank * per_xcd);
  } else {
    rank = bid / bh_count;
    bh = bid - rank * bh_count;
  }
}

// Tile geometry and LDS layout of a workgroup of NQ x NS waves with key tiles
// of BN rows per share.
template <int E, int NQ, int NS, int BN, bool BIAS>
struct FwdGeom {
  static_assert(E % 64 == 0 && BN % 32 == 0, "tile shape");
  static constexpr int NW = NQ * NS;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NQ * 32;
  static constexpr int ROWS = NS * BN;       // key rows staged per iteration
  static constexpr int ROW_B = 2 * E;
  static constexpr int KT_B = ROWS * ROW_B;  // bytes of the K (and of the V) rows of a stage
  static constexpr int STAGE = 2 * KT_B;     // [K rows][V rows], swizzled, unpadded
  static constexpr int NSTAGE = (3 * STAGE <= 64 * 1024) ? 3 : 2;  // keep two workgroups per CU
  static_assert(KT_B % (NT * 16) == 0, "whole loads per thread");
  static constexpr int NLD = KT_B / (NT * 16);  // loads per thread per tensor per stage
  // Merge buffer.  Four shares: for each (sending share, receiving share,
  // query sub-tile) the receiver's 8-column groups of the sender's partial O,
  // then each share's m and l.  Two: each ksp > 0 wave's whole partial result.
  static constexpr int MG = E / 8 / NS;  // 8-column groups a share finalizes
  static constexpr int CMB_FLOATS = NS == 4 ? NS * NS * NQ * MG * 4 * 64 + NS * NQ * 2 * 64
                                            : (NS - 1) * NQ * (E / 32 * 16 + 2) * 64;
  // Per-wave bias scratch after the ring: 32 rows x 32 keys, rows padded to
  // 72 bytes (8-byte aligned, at most two lanes of a 32-lane read per bank).
  static constexpr int BS_ROW_B = 72;
  static constexpr int BS_WAVE_B = 32 * BS_ROW_B;
  static constexpr int BS_OFF = NSTAGE * STAGE;
  static constexpr int RING_AND_BIAS = BS_OFF + (BIAS ? NW * BS_WAVE_B : 0);
  static constexpr int LDS_BYTES =
      RING_AND_BIAS > CMB_FLOATS * 4 ? RING_AND_BIAS : CMB_FLOATS * 4;
};

// One workgroup's query tile qt (BM rows) of head bh.  n_it_max: steps of the
// heaviest tile of its kind, for the start-up hold.
// IGLP >= 0 asks LLVM's scheduler for one of its instruction-group strategies
// (__builtin_amdgcn_iglp_opt) over the step's products and exponentials; the
// split launch uses it (strategy 1 measured 1.3% faster there, and slower in
// the other launches).  It changes only the instruction order.
template <int E, int NQ, int NS, int BN, bool CAUSAL, bool DROPOUT, bool BIAS, bool F16,
          int IGLP = -1>
__device__ __forceinline__ void fwd_tile(const FwdParams& p, int bh, int qt, int n_it_max,
                                         int hold, unsigned char* lds, bool split = false) {
  using G = FwdGeom<E, NQ, NS, BN, BIAS>;
  constexpr int NT = G::NT, BM = G::BM;
  constexpr int NES = E / 16;
  constexpr int NEB = E / 32;
  constexpr int ROWS = G::ROWS, ROW_B = G::ROW_B, KT_B = G::KT_B, STAGE = G::STAGE;
  constexpr int NSTAGE = G::NSTAGE, NLD = G::NLD;
  constexpr int NPS = 2 * NLD;  // loads per thread per stage
  constexpr int BS_ROW_B = G::BS_ROW_B, BS_WAVE_B = G::BS_WAVE_B, BS_OFF = G::BS_OFF;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int qs = wave % NQ;   // query sub-tile of this wave
  const int ksp = wave / NQ;  // key share of this wave

  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int q0 = qt * BM + qs * 32;  // first query row of this wave
  const int qrow = q0 + l32;         // query row of this lane

  const uint16_t* qp = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kp = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vp = p.v + b * p.sv.b + h * p.sv.h;

  int kend = p.Sk;
  if (CAUSAL) kend = min(kend, min(p.Sq, (qt + 1) * BM));  // keys <= last row of the tile
  const int n_kt = (kend + BN - 1) / BN;
  const int n_it = (n_kt + NS - 1) / NS;

  // Start-up hold: up to `hold` sleeps of ~640 clocks, one per step this tile
  // has fewer than the heaviest one (the split launch's dispatch table gives
  // the count itself, with n_it_max out of reach).
  if (CAUSAL && hold > 0) {
    const int units = min(n_it_max - n_it, hold);
    for (int i = 0; i < units; ++i) __builtin_amdgcn_s_sleep(10);
  }

  // Q as the B operand of S^T = K Q^T: lane holds its row, e = 16*es + 8*g + 0..7.
  // Rows past Sq read as zeros through the buffer range check.
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(qp, (uint32_t)(((int64_t)(p.Sq - 1) * p.sq.s + p.E) * 2));
  bf16x8 qf[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es)
    qf[es] = __builtin_bit_cast(
        bf16x8, buffer_load16(qr, (uint32_t)(((int64_t)qrow * p.sq.s + es * 16 + 8 * g) * 2) |
                                      (es * 16 + 8 * g < p.E ? 0u : 0x80000000u)));

  // Additive bias.  The wave's 32 rows x BN keys of tile t are fetched one step
  // ahead with row-contiguous loads (lane l: row 16*i + l/4 of the wave's rows,
  // keys 8*(l%4) .. +7 of a 32-key block, 16 bytes), then passed through a
  // per-wave LDS scratch so that each lane reads its own row: register group cg
  // of key block kb holds keys 32*kb + 8*cg + 4*g + 0..3.  Rows past Sq read
  // zeros (never stored); keys past Sk are masked.
  __amdgpu_buffer_rsrc_t br = make_rsrc(p.q, 0u);
  if (BIAS) br = make_rsrc(p.bias + b * p.sbias.b + h * p.sbias.h, bias_bytes(p));
  const int bl_row = lane >> 2, bl_chunk = lane & 3;  // load pattern
  uint4 bias_pf[BN / 32][2];
  auto load_bias = [&](int t) {
    const int64_t k0t = (int64_t)(t * NS + ksp) * BN + 8 * bl_chunk;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        bias_pf[kb][i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       br, (uint32_t)(((int64_t)(q0 + 16 * i + bl_row) * p.sbias.s + k0t + 32 * kb) * 2),
                       0, 0));
  };
  unsigned char* bscr = lds + BS_OFF + wave * BS_WAVE_B;
  if (BIAS && n_it > 0) load_bias(0);

  // K and V rows past kend read as zeros.  Stage it % NSTAGE of the ring holds
  // key rows it*ROWS .. it*ROWS + ROWS-1, loaded straight into LDS.
  const uint32_t kbytes = (uint32_t)(((int64_t)(kend - 1) * p.sk.s + p.E) * 2);
  const uint32_t vbytes = (uint32_t)(((int64_t)(kend - 1) * p.sv.s + p.E) * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp, kend > 0 ? kbytes : 0);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp, kend > 0 ? vbytes : 0);
  const uint32_t kstride = (uint32_t)(p.sk.s * 2), vstride = (uint32_t)(p.sv.s * 2);
  uint32_t ok[NLD], ov[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    ok[k] = dma_src_offset_e<E, NT>(k, tid, p.sk.s, p.E);
    ov[k] = dma_src_offset_e<E, NT>(k, tid, p.sv.s, p.E);
  }
  auto stage = [&](int it) { return lds + ring_offset<STAGE, NSTAGE>(it); };
  auto issue = [&](int it) {
    unsigned char* st = stage(it);
    const uint32_t r0 = (uint32_t)(it * ROWS);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      dma16(kr, st + k * NT * 16 + wave * 1024, r0 * kstride + ok[k]);
      dma16(vr, st + KT_B + k * NT * 16 + wave * 1024, r0 * vstride + ov[k]);
    }
  };

  // Per-lane LDS offsets.  S^T reads key row ksp*BN + 32*kb + l32 (the A
  // operand: lane = key, 8 consecutive e per lane); the transposed reads of V^T
  // map contraction slot (g, i) of 16-key step ksx to key row 16*ksx + 8*(i/4)
  // + 4*g + i%4 of the share, the C-register order of S^T.
  int aoff[NES];
#pragma unroll
  for (int es = 0; es < NES; ++es) aoff[es] = chunk_off<E>(l32, 2 * es + g) + ksp * BN * ROW_B;
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int troff[2][NEB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
      troff[t][eb] = KT_B + ksp * BN * ROW_B + tr_off<E>(8 * t + tr_row, 32 * eb + tr_col);

  f32x16 oacc[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) oacc[eb] = zero16();
  float m_run = -INFINITY;  // reference max of scale*log2(e)*S for this row
  float l_run = 0.f;        // this lane's share of the row sum, relative to m_run
  const float c = p.scale_log2;
  const float inv_scale = kLog2e / c;  // 1 / scale, for the bias
  // Last visible key of this lane's row, for masking (top-left causal; ragged Sk).
  const int key_limit = CAUSAL ? min(qrow, p.Sk - 1) : p.Sk - 1;

  const int sk4 = (p.Sk + 3) >> 2;
  uint64_t drow = 0;
  DropoutParams drop = p.drop;  // the device-resident RNG state, when used, is read into this copy
  if (DROPOUT) {
    load_dropout_state(drop);
    drow = philox_row_base(drop, dropout_head(drop, b, h), p.Sq, qrow, sk4);
  }

  // Stage 0 goes out with Q; with three stages, stage 1 follows once both are
  // in, so the start-up burst of every workgroup carries only what its first
  // step needs.
  if (n_it > 0) issue(0);
#pragma unroll
  for (int es = 0; es < NES; ++es) settle(qf[es]);  // waits for stage 0 too
  ring_barrier<0>();
  if (NSTAGE == 3 && n_it > 1) issue(1);

  for (int it = 0; it < n_it; ++it) {
    const int j = it * NS + ksp;
    const int k0 = j * BN;
    // Skip tiles past the key range and, when causal, above the diagonal.
    const bool active = (j < n_kt) && (!CAUSAL || k0 <= q0 + 31);
    const bool more = it + NSTAGE - 1 < n_it;
    // This step's prefetched bias, before the next tile's loads overwrite it.
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 bias_w[BN / 32][4];
    if (BIAS && active) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          unsigned char* dst = bscr + (16 * i + bl_row) * BS_ROW_B + 16 * bl_chunk;
          *reinterpret_cast<uint2*>(dst) = make_uint2(bias_pf[kb][i].x, bias_pf[kb][i].y);
          *reinterpret_cast<uint2*>(dst + 8) = make_uint2(bias_pf[kb][i].z, bias_pf[kb][i].w);
        }
#pragma unroll
        for (int cg = 0; cg < 4; ++cg)
          bias_w[kb][cg] = lds_at<u32x2>(bscr, l32 * BS_ROW_B + 16 * cg + 8 * g);
      }
    }
    if (BIAS && it + 1 < n_it) load_bias(it + 1);
    // With two stages the next one is free at the top of the step.  From the
    // second step on, the split launch's tiles, one sub-tile with four 64-key
    // shares and four sub-tiles at head dim 128 issue it there; their first
    // step keeps it behind the first products, out of the start-up burst of
    // every workgroup (3-6% faster across the split shapes and 1.2% at b2 h12
    // s1024, 2-2.5% for the other two shapes; from the first step the split
    // launch was 1.1% slower at b2 h12 s1024).  Two by two keeps it behind the
    // first products (1.5-4% slower the other way).  With three stages the
    // stage two ahead is free at the top of the step too; causal grids issue
    // it there from the second step on (b4 h16 s1000 and s2048: 2.6% faster),
    // non-causal ones keep it behind the first products (1.7% slower the
    // other way at b2 h16 s2048).
    const bool early =
        (NSTAGE == 2 ? (split || NQ == 4 || (NQ == 1 && BN == 64)) : CAUSAL) && it > 0;
    if ((early || !active) && more) issue(it + NSTAGE - 1);
    if (active) {
      if constexpr (IGLP >= 0) __builtin_amdgcn_iglp_opt(IGLP);
      const unsigned char* st = stage(it);
      // S^T for BN keys x 32 queries.  A bias enters as the accumulator's
      // starting value bias / scale, so the products leave S + bias / scale and
      // the softmax below scales by scale * log2(e) as without one.
      f32x16 s[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        s[kb] = zero16();
        if (BIAS) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t w = bias_w[kb][r >> 2][(r >> 1) & 1];
            s[kb][r] = from16<F16>((r & 1) ? (w >> 16) : w) * inv_scale;
          }
        }
#pragma unroll
        for (int es = 0; es < NES; ++es)
          s[kb] = mfma16<F16>(lds_at<bf16x8>(st, aoff[es] + kb * 32 * ROW_B), qf[es], s[kb]);
      }
      // The next stage's loads go out behind the first products.
      if (!early && more) issue(it + NSTAGE - 1);

      if (k0 + BN - 1 > (CAUSAL ? min(q0, p.Sk - 1) : p.Sk - 1)) {
        const int lim = key_limit - k0 - 4 * g;  // key offset past which scores are hidden
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
      }

      // Online softmax against a lazy reference: P = exp2(c*S - m) with the
      // row's current reference m.  The row maximum is taken, and m raised to
      // it with the sum and O rescaled, only for a row that has seen no visible
      // key yet or whose tile sum shows that an exponential may pass 2^16 (NaN
      // included); most tiles take no maximum.  Only the rows that ask move
      // their reference, so a row's values never depend on the other rows of
      // the wave.
      // P (bf16) as the B operand: 16-key step ksx takes registers 8*(ksx%2)..+7
      // of block ksx/2, i.e. keys 16*ksx + 8*(i/4) + 4*g + i%4 for element i.  The
      // row sum adds the fp32 probabilities (the log-sum-exp needs them unrounded).
      bf16x8 pb[BN / 16];
      float rs = 0.f;
      auto exps = [&](float m_use) {
        rs = 0.f;
#pragma unroll
        for (int ksx = 0; ksx < BN / 16; ++ksx)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float pv = fast_exp2(fmaf(s[ksx >> 1][8 * (ksx & 1) + i], c, -m_use));
            rs += pv;
            pb[ksx][i] = to16<F16>(pv);
          }
      };
      bool fresh = m_run == -INFINITY;
      if (__builtin_amdgcn_ballot_w64(!fresh)) {
        exps(fresh ? 0.f : m_run);
        fresh = fresh || !(rs <= kLazyLimit);
        fresh = pair_or(fresh ? 1u : 0u) != 0u;  // both lanes of a row agree
      }
      if (__builtin_amdgcn_ballot_w64(fresh)) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
        mx = pair_max(mx) * c;
        const bool grow = fresh && mx > m_run;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? mx : m_run;
          // A row that has seen only hidden keys (-inf bias entries) keeps
          // m_run = -inf while another row of the wave grows: its sum and O are
          // still zero, and -inf - -inf must not turn them into NaN.
          const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[eb][r] *= alpha;
        }
        exps((m_run == -INFINITY) ? 0.f : m_run);  // never -inf - -inf
      }
      l_run += rs;

      if (DROPOUT) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
          uint32_t bits = 0;  // keep bits of this lane's 16 keys of the block, at key % 32
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            // keys k0 + 32*kb + 8*cg + 4*g + 0..3: one Philox group
            const uint32_t grp = (uint32_t)(k0 >> 2) + kb * 8 + cg * 2 + g;
            const PhiloxOut w = philox4x32_10(drow + grp, drop.seed_lo, drop.seed_hi);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const bool keep = w.w[t] >= drop.threshold;
              if (!keep) pb[2 * kb + (cg >> 1)][4 * (cg & 1) + t] = (__bf16)0.f;
              bits |= (keep ? 1u : 0u) << (8 * cg + 4 * g + t);
            }
          }
          // Optionally keep the mask for the backward: the two lanes of a row
          // hold complementary halves of the block's word.
          if (p.keep != nullptr) {
            const uint32_t word = pair_or(bits);
            if (g == 0 && qrow < p.Sq)
              p.keep[((int64_t)bh * p.Sq + qrow) * p.keep_w + ((k0 + 32 * kb) >> 5)] = word;
          }
        }
      }

#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int ksx = 0; ksx < BN / 16; ++ksx) {
          const int o0 = troff[0][eb] + 16 * ksx * ROW_B, o1 = troff[1][eb] + 16 * ksx * ROW_B;
          oacc[eb] = mfma16<F16>(tr_pair(st, o0, o1), pb[ksx], oacc[eb]);
        }
    }
    // The next stage must have landed; this one is free once every wave is past here.
    if (NSTAGE == 3 && it + 2 < n_it)
      ring_barrier<NPS>();
    else
      ring_barrier<0>();
  }

  // Merge of the key shares of each query sub-tile (the loop's last barrier
  // freed the stages).  With four shares it is symmetric: 8-column group c of
  // the tile belongs to share c % 4, every share sends each other share the
  // groups that share owns, then merges and stores its own, so each wave
  // finalizes a quarter of the columns (1-3% faster than one wave finalizing
  // all of them, at b2 h3 / h8 / h12 s1024 causal).  With two shares the
  // ksp = 1 wave hands its whole partial result to the ksp = 0 wave, which
  // merges and stores the row: the symmetric form was 2-4% slower there.
  constexpr bool SYM = NS == 4;
  constexpr int NG = E / 8;  // 8-column groups of a row
  if constexpr (SYM) {
    constexpr int MG = G::MG, PART = MG * 4 * 64;
    float* cmb = reinterpret_cast<float*>(lds);
    float* mls = cmb + NS * NS * NQ * PART;
#pragma unroll
    for (int c = 0; c < NG; ++c) {
      const int owner = c % NS, eb = c >> 2, cg = c & 3;
      if (owner != ksp) {
        f32x4* dst = reinterpret_cast<f32x4*>(cmb + ((ksp * NS + owner) * NQ + qs) * PART);
        f32x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = oacc[eb][4 * cg + t];
        dst[(c / NS) * 64 + lane] = v;
      }
    }
    mls[((ksp * NQ + qs) * 2 + 0) * 64 + lane] = m_run;
    mls[((ksp * NQ + qs) * 2 + 1) * 64 + lane] = l_run;
    __syncthreads();
    float m_sh[NS], l_sh[NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      m_sh[s2] = mls[((s2 * NQ + qs) * 2 + 0) * 64 + lane];
      l_sh[s2] = mls[((s2 * NQ + qs) * 2 + 1) * 64 + lane];
    }
    float m_new = m_sh[0];
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2) m_new = fmaxf(m_new, m_sh[s2]);
    // A share whose keys were all hidden has m = -inf and contributes nothing.
    float a_sh[NS];
    float l_new = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      a_sh[s2] = (m_sh[s2] == -INFINITY) ? 0.f : fast_exp2(m_sh[s2] - m_new);
      l_new += l_sh[s2] * a_sh[s2];
    }
#pragma unroll
    for (int c = 0; c < NG; ++c) {
      const int owner = c % NS, eb = c >> 2, cg = c & 3;
      if (owner == ksp) {
        f32x4 acc;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) {
          f32x4 v;
          if (s2 == ksp) {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = oacc[eb][4 * cg + t];
          } else {
            v = reinterpret_cast<const f32x4*>(cmb + ((s2 * NS + ksp) * NQ + qs) * PART)[(c / NS) * 64 + lane];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t] = fmaf(v[t], a_sh[s2], acc[t]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) oacc[eb][4 * cg + t] = acc[t];
      }
    }
    l_run = l_new;
    m_run = m_new;
  } else if constexpr (NS > 1) {
    // A lane's 16 values of a block go out as four 16-byte writes.
    float* cmb = reinterpret_cast<float*>(lds);
    constexpr int SLOT = (NEB * 16 + 2) * 64;
    if (ksp > 0) {
      float* dst = cmb + ((ksp - 1) * NQ + qs) * SLOT;
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          f32x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = oacc[eb][4 * cg + t];
          reinterpret_cast<f32x4*>(dst)[(eb * 4 + cg) * 64 + lane] = v;
        }
      dst[(NEB * 16) * 64 + lane] = m_run;
      dst[(NEB * 16 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (ksp == 0) {
#pragma unroll
      for (int s2 = 1; s2 < NS; ++s2) {
        const float* src = cmb + ((s2 - 1) * NQ + qs) * SLOT;
        const float m_o = src[(NEB * 16) * 64 + lane];
        const float l_o = src[(NEB * 16 + 1) * 64 + lane];
        const float m_new = fmaxf(m_run, m_o);
        // A share whose keys were all hidden has m = -inf and contributes nothing.
        const float a_s = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        const float a_o = (m_o == -INFINITY) ? 0.f : fast_exp2(m_o - m_new);
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            const f32x4 v = reinterpret_cast<const f32x4*>(src)[(eb * 4 + cg) * 64 + lane];
#pragma unroll
            for (int t = 0; t < 4; ++t)
              oacc[eb][4 * cg + t] = oacc[eb][4 * cg + t] * a_s + v[t] * a_o;
          }
        l_run = l_run * a_s + l_o * a_o;
        m_run = m_new;
      }
    }
    if (ksp != 0) return;
  }

  const float l_tot = pair_sum(l_run);
  const float inv = (DROPOUT ? drop.keep_scale : 1.f) / l_tot;
  if (qrow < p.Sq) {
    uint16_t* op = p.o + b * p.so.b + h * p.so.h + (int64_t)qrow * p.so.s;
#pragma unroll
    for (int c = 0; c < NG; ++c) {
      const int eb = c >> 2, cg = c & 3;
      const int e = eb * 32 + 8 * cg + 4 * g;
      if ((!SYM || c % NS == ksp) && e < p.E)
        *reinterpret_cast<uint2*>(op + e) =
          pack16x4<F16>(oacc[eb][4 * cg + 0] * inv, oacc[eb][4 * cg + 1] * inv,
                      oacc[eb][4 * cg + 2] * inv, oacc[eb][4 * cg + 3] * inv);
    }
    if (ksp == 0 && g == 0 && p.lse != nullptr)
      p.lse[(int64_t)bh * p.Sq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// Steps of the heaviest causal tile of BM rows, key tiles of BN rows dealt to
// NS shares, among query rows below `rows`.
__device__ __forceinline__ int causal_steps_max(const FwdParams& p, int rows, int BN, int NS) {
  const int kend = min(p.Sk, min(p.Sq, rows));
  return ((kend + BN - 1) / BN + NS - 1) / NS;
}

template <int E, int NQ, int NS, int BN, bool CAUSAL, bool DROPOUT, bool BIAS, bool F16>
__global__ __launch_bounds__(NQ* NS * 64) void fwd_kernel(FwdParams p, int n_qtiles, int hold) {
  using G = FwdGeom<E, NQ, NS, BN, BIAS>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS_BYTES];
  warm_kernargs<sizeof(FwdParams) + 2 * sizeof(int)>();
  int bh, rank;
  wg_to_tile(blockIdx.x, p.B * p.H, bh, rank);
  const int qt = CAUSAL ? (n_qtiles - 1 - rank) : rank;
  const int n_it_max = CAUSAL ? causal_steps_max(p, n_qtiles * G::BM, BN, NS) : 0;
  fwd_tile<E, NQ, NS, BN, CAUSAL, DROPOUT, BIAS, F16>(p, bh, qt, n_it_max, hold, lds);
}

// Causal forward with two workgroup kinds in one launch.  The last rows of
// each head, whose tiles see the most keys, go to 32-row workgroups with the
// keys dealt to four waves in 32-key tiles; the rows before them to 64-row
// workgroups of two sub-tiles x two shares of 64-key tiles.  Both kinds use 64
// KB of LDS, so two workgroups share a compute unit whatever their kind, and
// the longest chain of steps of a head is cut where it starts to dominate.
// Without a dispatch table, workgroups 0 .. n_heavy*B*H-1 are the 32-row
// tiles, heaviest first, and the 64-row tiles follow, heaviest first; each
// kind keeps a head on one XCD.
//
// A dispatch table (below) can instead name each workgroup's tile, in one of
// two forms, each its own kernel so that the smaller one keeps the kernel
// arguments short (a longer argument block measured 1-3% slower per launch).
// With B*H a multiple of 8, SplitOrderXcd: every XCD has the same number of
// heads, and one 64-entry table, indexed by the workgroup's slot in its XCD,
// serves them all.
constexpr int kXcdSlots = 64;
struct SplitOrderXcd {
  int n;  // workgroups the table covers; 0 when there is none
  // Tile of workgroup 8*s + x, for XCD x, 16 bits, two to a word (s even in
  // the low half): bit 15 set for the 32-row kind, bits 12..14 its start-up
  // hold in sleep units, bits 6..11 its head among the XCD's B*H/8, bits 0..5
  // its rank in its kind.
  uint32_t slot[kXcdSlots / 2];
};
// Otherwise SplitOrderAll, one entry per workgroup.
constexpr int kSplitSlots = 512;
struct SplitOrderAll {
  int n;
  // Tile of workgroup w: bit 31 set for the 32-row kind, bits 28..30 its
  // start-up hold, bits 12..27 its (batch, head) index b*H + h, bits 0..11 its
  // rank in its kind.
  uint32_t slot[kSplitSlots];
};

template <int E, bool DROPOUT, bool BIAS, bool F16, typename ORD>
__global__ __launch_bounds__(256) void fwd_split_kernel(FwdParams p, int n_heavy, int n_light,
                                                        int hold, ORD ord) {
  using GH = FwdGeom<E, 1, 4, 32, BIAS>;
  using GL = FwdGeom<E, 2, 2, 64, BIAS>;
  constexpr int LDS_B = GH::LDS_BYTES > GL::LDS_BYTES ? GH::LDS_BYTES : GL::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_B];
  constexpr bool ALL = std::is_same<ORD, SplitOrderAll>::value;
  constexpr int ARG_B = (int)(sizeof(FwdParams) + 3 * sizeof(int) + sizeof(ORD));
  // The workgroup's table word is read in the same batch as the warm-up.
  uint32_t word;
  if constexpr (ALL)
    word = ord.slot[min((int)blockIdx.x, kSplitSlots - 1)];
  else
    word = ord.slot[min((int)blockIdx.x >> 4, kXcdSlots / 2 - 1)];
  warm_kernargs<(ARG_B < 8 * 64 ? ARG_B : 8 * 64)>(word);
  const int bh_count = p.B * p.H;
  const int light_rows = n_light * 64;
  const int nh = n_heavy * bh_count;
  int bh, rank;
  bool heavy;
  // With a table the hold comes from it: n_it_max past any tile's steps makes
  // the hold's count the table's.
  int nmax_h = causal_steps_max(p, light_rows + 32 * n_heavy, 32, 4);
  int nmax_l = causal_steps_max(p, light_rows, 64, 2);
  if (ord.n > 0) {
    nmax_h = nmax_l = 1 << 20;
    if constexpr (ALL) {
      heavy = (word >> 31) != 0;
      hold = (int)((word >> 28) & 7);
      bh = (int)((word >> 12) & 0xFFFF);
      rank = (int)(word & 0xFFF);
    } else {
      const uint32_t code = (word >> (16 * ((blockIdx.x >> 3) & 1))) & 0xFFFF;
      heavy = (code >> 15) != 0;
      hold = (int)((code >> 12) & 7);
      bh = (int)(blockIdx.x & 7) * (bh_count >> 3) + (int)((code >> 6) & 63);
      rank = (int)(code & 63);
    }
  } else {
    heavy = (int)blockIdx.x < nh;
    wg_to_tile(heavy ? (int)blockIdx.x : (int)blockIdx.x - nh, bh_count, bh, rank);
  }
  if (heavy) {
    const int qt = light_rows / 32 + (n_heavy - 1 - rank);
    fwd_tile<E, 1, 4, 32, true, DROPOUT, BIAS, F16, 1>(p, bh, qt, nmax_h, hold, lds, true);
  } else {
    const int qt = n_light - 1 - rank;
    fwd_tile<E, 2, 2, 64, true, DROPOUT, BIAS, F16, 1>(p, bh, qt, nmax_l, hold, lds, true);
  }
}

constexpr int kHoldSteps = 4;  // longest start-up hold, in steps of slack

template <int E, int NQ, int NS, int BN>
hipError_t launch_fwd_t(const FwdParams& p, bool causal, bool dropout, bool f16,
                        hipStream_t stream) {
  constexpr int BM = NQ * 32;
  const int n_qtiles = (p.Sq + BM - 1) / BM;
  const dim3 grid((unsigned)n_qtiles * (unsigned)(p.B * p.H));
  const dim3 block(NQ * NS * 64);
  auto go2 = [&](auto c, auto d, auto bias, auto half) {
    constexpr auto kernel = &fwd_kernel<E, NQ, NS, BN, decltype(c)::value, decltype(d)::value,
                                        decltype(bias)::value, decltype(half)::value>;
    // Hold light tiles back only when the whole grid runs in one round.
    const long slots = (long)device_cus() * resident_per_cu<kernel>((int)block.x);
    const int hold = (decltype(c)::value && (long)grid.x <= slots) ? kHoldSteps : 0;
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, p, n_qtiles, hold);
  };
  auto go = [&](auto c, auto d, auto bias) {
    if (f16)
      go2(c, d, bias, Flag<true>{});
    else
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

// Rows of each head that go to the 32-row, four-share kind of the split
// forward: the last quarter (at least 192 rows), shortened 64 rows at a time
// until the whole grid is resident at two workgroups per CU; the rows before
// them go to 64-row tiles.  Measured against a fixed 256: the same at
// Sq = 1024, 4-16% faster from Sq = 1536 to 4096.
struct SplitRows {
  int n_light, n_heavy;
};
inline SplitRows split_rows_tail(int Sq, int tail) {
  const int light_rows = Sq > tail ? (Sq - tail) / 64 * 64 : 0;
  return {light_rows / 64, (Sq - light_rows + 31) / 32};
}
inline SplitRows split_rows(const FwdParams& p) {
  const long slots = 2L * device_cus();
  int tail = std::max(192, (p.Sq / 4 + 32) / 64 * 64);
  SplitRows r = split_rows_tail(p.Sq, tail);
  while (tail > 192 && (long)(r.n_light + r.n_heavy) * p.B * p.H > slots) {
    tail -= 64;
    r = split_rows_tail(p.Sq, tail);
  }
  return r;
}

// Dispatch table that pairs long tiles with short ones on a compute unit when
// the whole grid is resident.  The dispatcher deals workgroups to the XCDs in
// turn (workgroup w to XCD w % 8) and, within an XCD, gives every compute unit
// one workgroup before any gets a second, so the XCD's slots s and s + C
// (workgroups 8s + x and 8(s + C) + x, C compute units per XCD) share a unit.
// Tiles are costed as steps times the cost of a step of their kind.  With B*H
// a multiple of 8 each XCD takes B*H/8 whole heads, so their K and V stay in
// its L2; otherwise the tiles go out longest first to the XCD with the least
// work so far (plus a penalty for a head it does not hold yet) that has room.
// Within an XCD the longest tiles run alone in the slots the second round
// leaves empty, and the rest pair longest with shortest.  Placement only moves
// time around: each tile computes the same values wherever it runs.
struct SplitPlan {
  int n;  // workgroups planned; 0: no table
  struct Tile {
    bool heavy;
    int hold, bh, rank;
  } tile[kSplitSlots];  // by workgroup
};

void plan_split(const FwdParams& p, const SplitRows& r, SplitPlan& plan) {
  plan.n = 0;
  const int bh_count = p.B * p.H, cus = device_cus();
  // Fewer than 8 heads would spread each head over several XCDs: measured
  // slower than the default order there.
  if (cus % 8 != 0 || bh_count < 8) return;
  const int C = cus / 8;
  const long nl = (long)bh_count * (r.n_light + r.n_heavy);
  if (nl > 2L * cus || nl > kSplitSlots) return;
  const int n = (int)nl;
  auto steps = [&](int rows, int bn, int ns) {
    const int kend = std::min(p.Sk, std::min(p.Sq, rows));
    return ((kend + bn - 1) / bn + ns - 1) / ns;
  };
  struct Item {
    int cost, bh, rank;
    bool heavy;
  };
  auto longer = [](const Item& a, const Item& b) { return a.cost > b.cost; };
  // Cost of a step: 32-row 3 and 2x2 5 (the traced 0.87-0.9 and 1.2-1.5 us)
  // when each XCD holds whole heads; 7 and 10 when heads are dealt over the
  // XCDs (measured 3% faster at b1 h12 s2048 there, 0.3% slower at b2 h12
  // s1024 in the per-XCD form).
  const int w32 = bh_count % 8 == 0 ? 3 : 7, w22 = bh_count % 8 == 0 ? 5 : 10;
  static thread_local Item items[kSplitSlots], by_xcd[8][kSplitSlots / 8 + 1];
  int k = 0;
  for (int bh = 0; bh < bh_count; ++bh) {
    for (int rank = 0; rank < r.n_heavy; ++rank) {
      const int qt = r.n_light * 2 + r.n_heavy - 1 - rank;  // in 32-row tiles
      items[k++] = {w32 * steps((qt + 1) * 32, 32, 4), bh, rank, true};
    }
    for (int rank = 0; rank < r.n_light; ++rank) {
      const int qt = r.n_light - 1 - rank;
      items[k++] = {w22 * steps((qt + 1) * 64, 64, 2), bh, rank, false};
    }
  }
  int cnt[8] = {0};
  if (bh_count % 8 == 0) {
    const int per = bh_count / 8;
    for (int i = 0; i < n; ++i) {
      const int x = items[i].bh / per;
      by_xcd[x][cnt[x]++] = items[i];
    }
  } else {
    std::stable_sort(items, items + n, longer);
    long load[8] = {0}, total = 0;
    for (int i = 0; i < n; ++i) total += items[i].cost;
    const long penalty = 2 * total / n;  // two average tiles
    static thread_local unsigned char holds[8][kSplitSlots];  // XCD x has tiles of head bh
    for (int x = 0; x < 8; ++x) std::fill(holds[x], holds[x] + bh_count, 0);
    for (int i = 0; i < n; ++i) {
      const Item& it = items[i];
      int best = -1;
      long best_score = 0;
      for (int x = 0; x < 8; ++x) {
        if (cnt[x] >= (n - x + 7) / 8) continue;  // XCD x runs (n - x + 7) / 8 workgroups
        const long score = load[x] + (holds[x][it.bh] ? 0 : penalty);
        if (best < 0 || score < best_score) best = x, best_score = score;
      }
      by_xcd[best][cnt[best]++] = it;
      load[best] += it.cost;
      holds[best][it.bh] = 1;
    }
  }
  for (int x = 0; x < 8; ++x) {
    Item* v = by_xcd[x];
    const int nx = cnt[x];
    std::stable_sort(v, v + nx, longer);
    const int m = std::max(nx - C, 0);      // compute units that get two tiles
    const int alone = std::min(nx, C) - m;  // compute units that get one
    auto put = [&](int s, const Item& it, int hold) {
      plan.tile[8 * s + x] = {it.heavy, hold, it.bh, it.rank};
    };
    // The shorter tile of a pair holds back one sleep unit (~0.3 us) per
    // 32-row step (w32 cost units) of estimated length it has less than its
    // partner; the longer one and the tiles alone start at once.  Of two
    // equal tiles one holds a unit, so that the two do not run their phases in
    // lockstep (0.4% at b2 h12 s1024, where four such pairs per XCD are forced).
    for (int j = 0; j < m; ++j) {
      const Item& a = v[alone + j];   // longest of the paired ...
      const Item& b = v[nx - 1 - j];  // ... with the shortest
      put(j, a, 0);
      put(C + j, b, a.cost == b.cost ? 1 : std::min(kHoldSteps, (a.cost - b.cost) / w32));
    }
    for (int t = 0; t < alone; ++t) put(m + t, v[t], 0);
  }
  plan.n = n;
}

// The plan and its two encodings for the last shape seen on this thread.
struct SplitTables {
  int key[7];
  SplitPlan plan;
  SplitOrderXcd xcd;
  SplitOrderAll all;
};

const SplitTables& split_tables(const FwdParams& p, const SplitRows& r) {
  static thread_local SplitTables t{{-1, 0, 0, 0, 0, 0, 0}, {}, {}, {}};
  const int key[7] = {p.B, p.H, p.Sq, p.Sk, r.n_light, r.n_heavy, device_cus()};
  if (std::equal(key, key + 7, t.key)) return t;
  std::copy(key, key + 7, t.key);
  plan_split(p, r, t.plan);
  t.xcd = SplitOrderXcd{};
  t.all = SplitOrderAll{};
  const int n = t.plan.n, bh_count = p.B * p.H;
  if (n == 0) return t;
  if (bh_count % 8 == 0 && n / 8 <= kXcdSlots) {
    // Per-XCD form: entries of XCD 0 (the others hold the same pattern).
    const int per = bh_count / 8;
    for (int w = 0; w < n; w += 8) {
      const SplitPlan::Tile& tl = t.plan.tile[w];
      const int s = w / 8;
      const uint32_t code = (tl.heavy ? 0x8000u : 0u) | (uint32_t)tl.hold << 12 |
                            (uint32_t)(tl.bh % per) << 6 | (uint32_t)tl.rank;
      t.xcd.slot[s >> 1] |= code << (16 * (s & 1));
    }
    t.xcd.n = n;
  } else if (bh_count % 8 != 0) {
    for (int w = 0; w < n; ++w) {
      const SplitPlan::Tile& tl = t.plan.tile[w];
      t.all.slot[w] = (tl.heavy ? 1u << 31 : 0u) | (uint32_t)tl.hold << 28 |
                      (uint32_t)tl.bh << 12 | (uint32_t)tl.rank;
    }
    t.all.n = n;
  }
  return t;
}

template <int E>
hipError_t launch_fwd_split(const FwdParams& p, bool dropout, bool f16, bool table,
                            hipStream_t stream) {
  const SplitRows r = split_rows(p);
  const dim3 grid((unsigned)(r.n_light + r.n_heavy) * (unsigned)(p.B * p.H));
  auto go = [&](auto d, auto bias, auto half) {
    constexpr bool D = decltype(d)::value, Bi = decltype(bias)::value, H = decltype(half)::value;
    constexpr auto kernel = &fwd_split_kernel<E, D, Bi, H, SplitOrderXcd>;
    constexpr auto kernel_all = &fwd_split_kernel<E, D, Bi, H, SplitOrderAll>;
    const long slots = (long)device_cus() * resident_per_cu<kernel>(256);
    const bool resident = (long)grid.x <= slots;
    const int hold = resident ? kHoldSteps : 0;
    if (resident && table) {
      const SplitTables& t = split_tables(p, r);
      if (t.all.n > 0) {
        hipLaunchKernelGGL(kernel_all, grid, dim3(256), 0, stream, p, r.n_heavy, r.n_light, hold,
                           t.all);
        return;
      }
      hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, p, r.n_heavy, r.n_light, hold, t.xcd);
      return;
    }
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, p, r.n_heavy, r.n_light, hold,
                       SplitOrderXcd{});
  };
  auto with_half = [&](auto d, auto bias) {
    if (f16)
      go(d, bias, Flag<true>{});
    else
      go(d, bias, Flag<false>{});
  };
  auto with_bias = [&](auto d) {
    if (p.bias != nullptr)
      with_half(d, Flag<true>{});
    else
      with_half(d, Flag<false>{});
  };
  if (dropout)
    with_bias(Flag<true>{});
  else
    with_bias(Flag<false>{});
  return hipGetLastError();
}

// Whole grid of the split forward resident at once (two workgroups per CU).
bool split_fits(const FwdParams& p) {
  const SplitRows r = split_rows(p);
  return (long)(r.n_light + r.n_heavy) * p.B * p.H <= 2L * device_cus();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, bool causal, bool dropout, bool f16,
                      const TileChoice& tiles, hipStream_t stream) {
  const int E = tile_head_dim(p.E);
  // Shape: 4 query sub-tiles sharing each key tile when there are enough
  // 128-row tiles to give every compute unit two workgroups; otherwise two
  // query sub-tiles with the keys split in two, for a shorter critical path.
  // When even 32-row tiles leave a compute unit per workgroup (head dim 64,
  // e.g. a few heads of one GPU's share) and there are keys for four shares,
  // one sub-tile with the keys split in four: its 128 KB of LDS then costs no
  // concurrency.
  // A causal problem that would take two by two, with at least 512 rows and a
  // grid that fits the chip at once, takes the split launch (4): about the
  // last quarter of each head's rows in 32-row, four-share workgroups.
  // At head dim 64, a causal grid of four-by-one workgroups that runs in one
  // round is as long as its last tile's walk over the keys; two by two halves
  // that walk and wins there with dropout or past 1024 rows (8-14%: b4 h16
  // s1000 p=0.1 32.5 vs 35.6 us, b2 h16 s2048 p=0.1 53.7 vs 62.2 us, b2 h16
  // s2048 32.9 vs 36.6 us; b4 h16 s1000 without dropout 22.0 vs 21.2 us).
  // Once four by one needs two rounds or more it stays ahead.
  int shape = tiles.fwd_shape;  // 1: NQ=4,NS=1   2: NQ=2,NS=2   3: NQ=1,NS=4   4: split
  if (shape < 1 || shape > 4) {
    const long wg4 = (long)((p.Sq + 127) / 128) * p.B * p.H;
    const long wg1 = (long)((p.Sq + 31) / 32) * p.B * p.H;
    if (E == 64 && p.Sk >= 4 * 64 && wg1 <= device_cus())
      shape = 3;
    else if (wg4 >= 512)
      shape = (E == 64 && causal && wg4 <= 2L * device_cus() && (dropout || p.Sq > 1024)) ? 2 : 1;
    else if (E == 64 && causal && p.Sq >= 512 && split_fits(p))
      shape = 4;
    else
      shape = 2;
  }
  if (shape == 4 && (E != 64 || !causal)) shape = 2;  // the split launch is causal, head dim 64
  if (shape == 4) return launch_fwd_split<64>(p, dropout, f16, tiles.fwd_order != 1, stream);
  if (E == 64) {
    if (shape == 1) return launch_fwd_t<64, 4, 1, 64>(p, causal, dropout, f16, stream);
    if (shape == 2) return launch_fwd_t<64, 2, 2, 64>(p, causal, dropout, f16, stream);
    return launch_fwd_t<64, 1, 4, 64>(p, causal, dropout, f16, stream);
  }
  // One query sub-tile with four key shares needs more registers than head dim
  // 128 leaves; it falls back to two by two.
  if (shape == 1) return launch_fwd_t<128, 4, 1, 64>(p, causal, dropout, f16, stream);
  return launch_fwd_t<128, 2, 2, 64>(p, causal, dropout, f16, stream);
}

}  // namespace sdpa14

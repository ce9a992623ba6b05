// zl_tile.h -- the per-tile math shared by the decode kernels: one 32-token
// tile already in LDS -> scores (MFMA), online-softmax update, PV (MFMA).
//
// Lane (g, n) = (lane / 16, lane % 16).  The unit's query heads sit on the
// MFMA N dimension (head n), so every per-head quantity lives in the lanes
// with that n.  Token order inside a tile is chosen once, by the QK^T result
// layout, and reused unchanged as the PV contraction order:
//   score register r of 16-token block tb in lane (g, n) = token 16tb + 4g + r
//   PV k-slot 8g + i                                  = token 16(i/4) + 4g + i%4
//
// LDS banks (gfx950, measured with the SQ_LDS_BANK_CONFLICT counter): 64
// banks of 4 bytes, i.e. 16 groups of 16 bytes per 256-byte line.
//  * ds_read_b128 serves a wave in four passes of 16 lanes: the lanes of one
//    half-wave whose lane-index bits 2, 3 and 4 have the same parity.  A pass
//    costs one cycle per lane that shares a 16-byte bank group with another.
//    For the operand reads below (lane (g, n) reads row n, slot 4kb + g) a pass
//    holds g = 2h with 8 rows and g = 2h + 1 with the other 8, so the swizzle
//    must map those 16 (row, slot) pairs to 16 different bank groups.
//  * ds_read_b64_tr_b16 serves all 64 lanes in two cycles and is free of
//    conflicts when no bank is hit more than twice.
#pragma once

#include "zl_device.h"

namespace zl {

// Running softmax state of head n (kept in every lane of that head).
struct SoftmaxState {
  float m;  // running max of scaled scores, log2 units (-inf before any token)
  float l;  // this lane's share of the running sum (summed over g at the end)
};

// S = K Q^T over the tile: A = K rows (16 tokens x 32 dims) from LDS, B = the
// query heads' k-step fragments.  slot(c, t) locates 16-byte chunk c of row t.
template <int DT, int KSTEPS, int ROWB, typename SlotFn>
__device__ __forceinline__ void scores(const ZL_LDS char* kt, const i16x8 (&qop)[KSTEPS], int n, int g,
                                       SlotFn slot, f32x4 (&s)[2]) {
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int t = 16 * tb + n;
#pragma unroll
    for (int kb = 0; kb < KSTEPS; ++kb) {
      const int c = 4 * kb + g;
      u32x4 av = lds_read_b128(kt + t * ROWB + (slot(c, t) << 4));
      acc = mfma16x16x32<DT>(__builtin_bit_cast(i16x8, av), qop[kb], acc);
    }
    s[tb] = acc;
  }
}

// P^T operand of the PV product.  For bf16 (8 significant bits) the
// probabilities are split as P = hi + lo with both halves in bf16, and PV runs
// twice (V hi + V lo): P keeps about 16 significant bits, so the PV result is
// not limited by bf16 rounding of the weights.  fp16 (11 bits) uses hi only.
struct POperand {
  i16x8 hi;
  i16x8 lo;
};

// Largest rise (log2 units) of a head's running max that the update absorbs
// without moving its reference max: the probabilities are then at most
// 2^kLazyMax, well inside the range of both 16-bit formats and of the fp32
// sums, and most tiles skip the rescale of the accumulators (an exact
// identity: out = sum 2^(x - m) v / sum 2^(x - m) for any reference m).
constexpr float kLazyMax = 8.f;

// Online-softmax update with the tile's scores.  Tokens at or past nvalid are
// masked.  Returns the P^T operand (16-bit probabilities in PV k-slot order)
// and the factor alpha by which the accumulators must be rescaled; rescale
// (wave-uniform) is false when alpha is 1 in every lane.
template <int DT>
__device__ __forceinline__ POperand softmax_update(const f32x4 (&s)[2], int g, int nvalid,
                                                   float scale_log2, SoftmaxState& st, float& alpha,
                                                   bool& rescale) {
  float x[8];
  float tmax = -INFINITY;
  if (__builtin_amdgcn_ballot_w64(nvalid < 32) == 0) {
    // Every lane's tile is full: no mask.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[4 * tb + r] = s[tb][r] * scale_log2;
        tmax = fmaxf(tmax, x[4 * tb + r]);
      }
  } else {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * tb + 4 * g + r;
        const float xv = tok < nvalid ? s[tb][r] * scale_log2 : -INFINITY;
        x[4 * tb + r] = xv;
        tmax = fmaxf(tmax, xv);
      }
  }
  tmax = max_over_groups(tmax);
  // The reference max moves only when the tile's max passes it by more than
  // kLazyMax (always for the first finite max: -inf + kLazyMax = -inf).
  const bool grow = tmax > st.m + kLazyMax;
  const float m_new = grow ? tmax : st.m;
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  alpha = grow ? exp2_fast(st.m - m_use) : 1.f;
  rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = exp2_fast(x[i] - m_use);
    psum += x[i];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  POperand p;
  u32x4 pw;
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[i] = pack2<DT>(x[2 * i], x[2 * i + 1]);
  p.hi = __builtin_bit_cast(i16x8, pw);
  if constexpr (DT == kBF16) {
    // lo = x - hi, exact in fp32; hi read back from the packed pairs.
    u32x4 pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float h0 = __builtin_bit_cast(float, pw[i] << 16);
      const float h1 = __builtin_bit_cast(float, pw[i] & 0xffff0000u);
      pl[i] = pack2<DT>(x[2 * i] - h0, x[2 * i + 1] - h1);
    }
    p.lo = __builtin_bit_cast(i16x8, pl);
  } else {
    p.lo = p.hi;  // unused
  }
  return p;
}

// O^T[16 dims x 16 heads] += V^T P^T for NB consecutive 16-dim blocks starting
// at block blk0.  V^T (the A operand) is read transposed: lane m of group g
// points at token 4g + m/4 (and +16), dims 16blk + 4(m%4) .. +3.  Reads go out
// in groups of 4 blocks (8 reads) with one group of lookahead.
template <int DT, int NB, int ROWB, typename SlotFn>
__device__ __forceinline__ void pv_blocks(const ZL_LDS char* vt, const POperand& pop, int n, int g,
                                          int blk0, SlotFn slot, f32x4 (&o)[NB]) {
  static_assert(NB % 4 == 0, "blocks come in groups of 4");
  constexpr int NG = NB / 4;
  const int r0 = 4 * g + (n >> 2);
  const int r1 = r0 + 16;
  const int half = (n & 1) << 3;
  const int csub = (n & 3) >> 1;
  const ZL_LDS char* row0 = vt + r0 * ROWB + half;
  const ZL_LDS char* row1 = vt + r1 * ROWB + half;
  i16x4 lo[2][4], hi[2][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 2 * (blk0 + k) + csub;
    lo[0][k] = lds_read_tr16(row0 + (slot(c, r0) << 4));
    hi[0][k] = lds_read_tr16(row1 + (slot(c, r1) << 4));
  }
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    const int buf = grp & 1;
    if (grp + 1 < NG) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = 2 * (blk0 + 4 * (grp + 1) + k) + csub;
        lo[buf ^ 1][k] = lds_read_tr16(row0 + (slot(c, r0) << 4));
        hi[buf ^ 1][k] = lds_read_tr16(row1 + (slot(c, r1) << 4));
      }
      lds_wait<8>(lo[buf][0], lo[buf][1], lo[buf][2], lo[buf][3], hi[buf][0], hi[buf][1], hi[buf][2],
                  hi[buf][3]);
    } else {
      lds_wait<0>(lo[buf][0], lo[buf][1], lo[buf][2], lo[buf][3], hi[buf][0], hi[buf][1], hi[buf][2],
                  hi[buf][3]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      i16x8 av = __builtin_shufflevector(lo[buf][k], hi[buf][k], 0, 1, 2, 3, 4, 5, 6, 7);
      o[4 * grp + k] = mfma16x16x32<DT>(av, pop.hi, o[4 * grp + k]);
      if constexpr (DT == kBF16) o[4 * grp + k] = mfma16x16x32<DT>(av, pop.lo, o[4 * grp + k]);
    }
  }
}

template <int DT>
__device__ __forceinline__ void store_out4(uint16_t* dst, f32x4 o, float inv) {
  u32x2 w;
  w[0] = pack2<DT>(o[0] * inv, o[1] * inv);
  w[1] = pack2<DT>(o[2] * inv, o[3] * inv);
  *(u32x2*)dst = w;
}

}  // namespace zl

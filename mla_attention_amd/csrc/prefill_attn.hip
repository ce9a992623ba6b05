// prefill_attn.hip -- causal attention of long runs of new tokens (prefill and
// large prefill chunks) for gfx950 (MI355X), grouped-query layout (K, V [T,
// Hkv, D], D = 64 or 128).  The pages list flash-attention prefill and chunked
// prefill among the engine's kernels (first page, sections "技术架构" and
// "功能生态"; second page, section "Dual streams, host all-reduce and the memory
// model").  The operation is the one of zl_attn_varlen_gqa: new token i of the
// nq of sequence b sees its cache rows 0 .. lk - nq + i (causal, aligned to
// the bottom right) or all lk rows.
//
// Unlike decode, every cache row is used by many query rows, so the work is
// matrix-unit bound.  Structure (two workgroups of four wavefronts per CU):
//  * A block is one key/value head and 128 query rows of one sequence -- the
//    pairs (new token i, head hh of the head's group), numbered i*G + hh, so
//    the group's heads share every K/V tile.  Wave w owns rows 32w .. 32w+31
//    as two 16-row MFMA column blocks.  Blocks are ordered longest first
//    (the last blocks of a sequence see the most keys).
//  * The workgroups are persistent (two per CU): each takes one block per
//    round, walking the order forwards and backwards in turn, so that equal
//    prompts give every workgroup the same number of tiles.  A block's start
//    (its query operands, the first tiles' latency) used to cost as much as
//    several tiles when every block was a workgroup of its own.
//  * A workgroup streams the keys each block's last token can see in
//    32-token tiles through a four-stage LDS ring that runs on from one
//    block into the next; each wave DMAs a quarter of every tile
//    (global_load_lds, SADDR form) and one barrier per tile both publishes
//    the tile and frees the stage refilled next.
//  * Per tile and wave: S^T = K Q^T for 2 token blocks x 2 column blocks
//    (each K fragment read from LDS once and used for both), the causal mask
//    and online softmax per column, and O^T += V^T P^T (each transposed V
//    fragment read once, used for both) -- the decode kernels' tile math and
//    layouts (zl_tile.h), widened to 32 query rows per wave.
#include "zl_device.h"
#include "zl_kernels.h"
#include "zl_split.h"
#include "zl_tile.h"

#include <type_traits>

namespace zl {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfCB = 2;                       // 16-row column blocks per wave
constexpr int kPfRowsLog2 = kPrefillRowsLog2;  // 128 query rows per workgroup
constexpr int kPfStages = 4;

template <int D>
struct PfGeo {
  static constexpr int ROWB = D * 2;           // bytes per K or V row in LDS
  static constexpr int CPR = D / 8;            // 16-byte slots per row
  static constexpr int KBYTES = 32 * ROWB;
  static constexpr int STAGE = 2 * KBYTES;     // K tile then V tile
  static constexpr int NI = STAGE / 1024;      // 1 KB DMA instructions per tile
  static constexpr int NIW = NI / kPfWaves;    // per wave
  static constexpr int KSTEPS = D / 32;
  static constexpr int VBLK = D / 16;
  static_assert(NI % kPfWaves == 0, "tile splits evenly over the waves");
  static_assert(kPfWaves * kPfCB * 16 == 1 << kPfRowsLog2, "the waves' columns are the block's rows");
  // The decode kernels' conflict-free swizzles (zl_tile.h bank rules).
  __device__ static int slot(int c, int r) {
    if constexpr (D == 128)
      return c ^ (r & 15);
    else
      return c ^ ((r >> 1) & 7);
  }
};

// This wave's quarter of a tile: instruction k covers 1 KB block i = NIW*w + k
// of [K tile | V tile]; lane l loads row r = lin / CPR, slot slot(lin % CPR, r)
// of that tile, lin = 64*(i mod NI/2) + l.
template <int D>
struct PfMap {
  uint32_t chunk[PfGeo<D>::NIW];  // 16 * source slot
  int row[PfGeo<D>::NIW];
};

template <int D>
__device__ __forceinline__ PfMap<D> pf_map(int wave, int lane) {
  using GE = PfGeo<D>;
  PfMap<D> m;
#pragma unroll
  for (int k = 0; k < GE::NIW; ++k) {
    const int i = GE::NIW * wave + k;
    const int half = GE::NI / 2;
    const int lin = 64 * (i % half) + lane;
    const int r = lin / GE::CPR;
    m.row[k] = r;
    m.chunk[k] = 16u * (uint32_t)GE::slot(lin - r * GE::CPR, r);
  }
  return m;
}

// Rows past nvalid repeat row nvalid - 1 (finite data, masked out).
template <int D>
__device__ __forceinline__ void pf_dma_tile(const char* kbase, const char* vbase, uint32_t row_bytes,
                                            const PfMap<D>& m, int nvalid, ZL_LDS char* stage, int wave) {
  using GE = PfGeo<D>;
#pragma unroll
  for (int k = 0; k < GE::NIW; ++k) {
    const int i = GE::NIW * wave + k;
    const int rr = m.row[k] < nvalid ? m.row[k] : nvalid - 1;
    const char* base = (i >= GE::NI / 2) ? vbase : kbase;  // wave-uniform
    dma16_saddr(base, (uint32_t)rr * row_bytes + m.chunk[k], stage + i * 1024);
  }
}

// Per-lane LDS byte offsets of the fragments a lane reads from a stage (the
// stage's base is OR-ed in once per tile: it lies above every offset bit):
//  K (scores): row n, slot(4kb + g, n), for k-step kb;
//  V (PV): row r0 = 4g + n/4, bytes 8(n & 1) into slot(2m + (n & 3)/2, r0),
//  for group m of 16 output dims.
// Both swizzles map rows r and r + 16 to the same slots, so one offset serves
// both 16-row halves of a tile.  In both, the bits that kb (or m) changes are
// disjoint from the lane's other bits, so every offset is the lane's first
// one XOR 64 kb (or 32 m): one instruction per offset and tile, two registers.
template <int D>
struct PfOffsets {
  uint32_t k0, v0;
};

template <int D>
__device__ __forceinline__ PfOffsets<D> pf_offsets(int n, int g) {
  using GE = PfGeo<D>;
  const int r0 = 4 * g + (n >> 2);
  return PfOffsets<D>{(uint32_t)(n * GE::ROWB + (GE::slot(g, n) << 4)),
                      (uint32_t)(r0 * GE::ROWB + ((n & 1) << 3) + (GE::slot((n & 3) >> 1, r0) << 4))};
}

// S^T for the tile's 2 token blocks and this wave's column blocks: lane (g, n)
// gets tokens 16tb + 4g .. +3 of column 16cb + n.  off.k0 includes the
// stage's base.
template <int DT, int D>
__device__ __forceinline__ void pf_scores(const ZL_LDS char* smem, PfOffsets<D> off,
                                          const i16x8 (&qop)[kPfCB][PfGeo<D>::KSTEPS], f32x4 (&s)[kPfCB][2]) {
  using GE = PfGeo<D>;
  // The base offset passes through an empty asm so that the compiler derives
  // the offsets here (one XOR each, the 16-row step as an immediate) instead
  // of holding an address per block across the loop.
  uint32_t k0 = off.k0;
  asm volatile("" : "+v"(k0));
#pragma unroll
  for (int cb = 0; cb < kPfCB; ++cb) s[cb][0] = s[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < GE::KSTEPS; ++kb) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const i16x8 av = __builtin_bit_cast(i16x8, lds_read_b128(smem + 16 * tb * GE::ROWB + (k0 ^ (64 * kb))));
#pragma unroll
      for (int cb = 0; cb < kPfCB; ++cb) s[cb][tb] = mfma16x16x32<DT>(av, qop[cb][kb], s[cb][tb]);
    }
  }
}

// O^T[cb] += V^T P^T[cb] over all D/16 output blocks; every transposed V
// fragment is read once and used for the column blocks.  Reads go out in
// groups of 4 blocks with one group of lookahead (as pv_blocks).  off.v0
// includes the stage's base; the V tile starts VT bytes after it and its rows
// 16 .. 31 another 16 rows further on (both immediates).
template <int DT, int D, int VT>
__device__ __forceinline__ void pf_pv(const ZL_LDS char* smem, PfOffsets<D> off,
                                      const POperand (&pop)[kPfCB], f32x4 (&o)[kPfCB][PfGeo<D>::VBLK]) {
  using GE = PfGeo<D>;
  constexpr int NG = GE::VBLK / 4;
  constexpr int VT1 = VT + 16 * GE::ROWB;
  static_assert(VT1 <= 65535, "immediate LDS offsets are 16-bit");
  uint32_t v0 = off.v0;  // (as k0 in pf_scores)
  asm volatile("" : "+v"(v0));
  const auto vrow = [&](int m) { return smem + (v0 ^ (32u * m)); };
  i16x4 lo[2][4], hi[2][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    lo[0][k] = lds_read_tr16<VT>(vrow(k));
    hi[0][k] = lds_read_tr16<VT1>(vrow(k));
  }
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    const int buf = grp & 1;
    if (grp + 1 < NG) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo[buf ^ 1][k] = lds_read_tr16<VT>(vrow(4 * (grp + 1) + k));
        hi[buf ^ 1][k] = lds_read_tr16<VT1>(vrow(4 * (grp + 1) + k));
      }
      lds_wait<8>(lo[buf][0], lo[buf][1], lo[buf][2], lo[buf][3], hi[buf][0], hi[buf][1], hi[buf][2],
                  hi[buf][3]);
    } else {
      lds_wait<0>(lo[buf][0], lo[buf][1], lo[buf][2], lo[buf][3], hi[buf][0], hi[buf][1], hi[buf][2],
                  hi[buf][3]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const i16x8 av = __builtin_shufflevector(lo[buf][k], hi[buf][k], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int cb = 0; cb < kPfCB; ++cb) {
        o[cb][4 * grp + k] = mfma16x16x32<DT>(av, pop[cb].hi, o[cb][4 * grp + k]);
        if constexpr (DT == kBF16) o[cb][4 * grp + k] = mfma16x16x32<DT>(av, pop[cb].lo, o[cb][4 * grp + k]);
      }
    }
  }
}

// The group maxima of the wave's column blocks (one overload per count).
[[maybe_unused]] __device__ __forceinline__ void max_over_groups_n(float (&x)[2]) { max_over_groups2(x); }
[[maybe_unused]] __device__ __forceinline__ void max_over_groups_n(float (&x)[4]) { max_over_groups4(x); }

// Online-softmax update of the wave's column blocks at once (as
// softmax_update in zl_tile.h per block).  The blocks are independent, so
// every step is written across them: the reductions and exponentials form
// interleavable chains instead of one long one.  The token mask is compiled
// in only where a tile needs it.
//
// scale_log2 is never negative here (the kernel negates the query operands
// when the softmax scale is), so the scaled maximum is the raw maximum times
// the scale and each probability is 2^fma(s, scale, -m): one instruction
// per score instead of a multiply and a subtract.  Masked scores are zeroed
// after the exponential (a zero scale would turn -inf into NaN).
template <int DT, bool MASK>
__device__ __forceinline__ void pf_softmax4(const f32x4 (&s)[kPfCB][2], int g, const int (&nvalid)[kPfCB],
                                            float scale_log2, SoftmaxState (&st)[kPfCB], bool (&grow)[kPfCB],
                                            float (&dexp)[kPfCB], float (&psum)[kPfCB], POperand (&p)[kPfCB]) {
  static_assert(kPfCB == 2 || kPfCB == 4, "two or four column blocks");
  float x[kPfCB][8];
  float tmax[kPfCB];
#pragma unroll
  for (int cb = 0; cb < kPfCB; ++cb) tmax[cb] = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cb = 0; cb < kPfCB; ++cb) {
        float xv = s[cb][tb][r];
        if constexpr (MASK) xv = 16 * tb + 4 * g + r < nvalid[cb] ? xv : -INFINITY;
        tmax[cb] = fmaxf(tmax[cb], xv);  // (MFMA results: the compiler forms v_max3)
      }
  max_over_groups_n(tmax);
#pragma unroll
  for (int cb = 0; cb < kPfCB; ++cb) tmax[cb] = tmax[cb] == -INFINITY ? -INFINITY : tmax[cb] * scale_log2;
  // Lazy rescale (kLazyMax, zl_tile.h): a column's reference max moves only
  // when the tile's max passes it by more than 2^kLazyMax.
  float m_use[kPfCB];
#pragma unroll
  for (int cb = 0; cb < kPfCB; ++cb) {
    grow[cb] = tmax[cb] > st[cb].m + kLazyMax;
    const float m_new = grow[cb] ? tmax[cb] : st[cb].m;
    m_use[cb] = (m_new == -INFINITY) ? 0.f : m_new;
    dexp[cb] = st[cb].m - m_use[cb];
    st[cb].m = m_new;
    psum[cb] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int cb = 0; cb < kPfCB; ++cb) {
      float xv = exp2_fast(__builtin_fmaf(s[cb][i >> 2][i & 3], scale_log2, -m_use[cb]));
      if constexpr (MASK) xv = 16 * (i >> 2) + 4 * g + (i & 3) < nvalid[cb] ? xv : 0.f;
      x[cb][i] = xv;
      psum[cb] += xv;
    }
#pragma unroll
  for (int cb = 0; cb < kPfCB; ++cb) {
    u32x4 pw;
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = pack2<DT>(x[cb][2 * i], x[cb][2 * i + 1]);
    p[cb].hi = __builtin_bit_cast(i16x8, pw);
    if constexpr (DT == kBF16) {
      // lo = x - hi (exact), hi read back from the packed pairs
      u32x4 pl;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pl[i] = pack2<DT>(x[cb][2 * i] - __builtin_bit_cast(float, pw[i] << 16),
                          x[cb][2 * i + 1] - __builtin_bit_cast(float, pw[i] & 0xffff0000u));
      p[cb].lo = __builtin_bit_cast(i16x8, pl);
    } else {
      p[cb].lo = p[cb].hi;
    }
  }
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __builtin_amdgcn_ds_bpermute((__lane_id() ^ m) << 2, v));
  return v;
}

// One block: 128 query rows of one sequence for one key/value head, and the
// keys its last row sees.
struct PfBlock {
  int kvh;
  VSeqInfo si;
  int kend;    // keys seen by the block's last row
  int ntiles;  // 32-token tiles holding them
};

// Block p of the order: key/value head p mod Hkv, and per head the blocks
// longest first (a sequence's last block first, sequences in reverse batch
// order).
__device__ __forceinline__ PfBlock pf_block(const VirtualSeqs& vs, const DecodeArgs& a, int p) {
  PfBlock bk;
  bk.kvh = p % a.Hkv;
  bk.si = vs.info(vs.V - 1 - p / a.Hkv);
  const int last_row = bk.si.nq * a.G - 1;
  const int blk_last = ((bk.si.hb + 1) << kPfRowsLog2) - 1;
  const int last_tok = (blk_last < last_row ? blk_last : last_row) / a.G;
  const int kend = a.causal ? bk.si.lk - bk.si.nq + last_tok + 1 : bk.si.lk;
  bk.kend = kend < bk.si.lk ? kend : bk.si.lk;
  bk.ntiles = bk.kend > 0 ? (bk.kend + 31) >> 5 : 0;
  return bk;
}

// The position in that order that workgroup w of P takes in round r: rounds
// walk the order P positions at a time, alternately forwards and backwards,
// so over two rounds a workgroup gets one block from each end of a stretch
// of decreasing lengths (equal-length prompts balance exactly).
__device__ __forceinline__ long long pf_position(int r, int w, int P) {
  return (long long)r * P + ((r & 1) ? P - 1 - w : w);
}

// This lane's columns of a block: query rows 128 hb + 16 kPfCB wave + 16 cb + n.
struct PfRows {
  long long orow[kPfCB];  // output row (clamped to the block's last valid one)
  bool valid[kPfCB];
  int lim[kPfCB];         // last visible cache row, counted from the sequence's first
  int lim_min;            // the wave's smallest lim: tiles below it need no mask
};

__device__ __forceinline__ PfRows pf_rows(const PfBlock& bk, const DecodeArgs& a, int wave, int n) {
  PfRows rw;
  const int last_row = bk.si.nq * a.G - 1;
  int lim_lane = 0x7fffffff;
#pragma unroll
  for (int cb = 0; cb < kPfCB; ++cb) {
    const int r = (bk.si.hb << kPfRowsLog2) + 16 * kPfCB * wave + 16 * cb + n;
    const int rr = r < last_row ? r : last_row;
    const int qi = rr / a.G;
    rw.orow[cb] = (long long)(bk.si.q0 + qi) * a.Hq + bk.kvh * a.G + (rr - qi * a.G);
    rw.valid[cb] = r <= last_row;
    rw.lim[cb] = a.causal ? bk.si.lk - bk.si.nq + qi : bk.si.lk - 1;
    lim_lane = min(lim_lane, rw.lim[cb]);
  }
  rw.lim_min = readfirstlane(wave_min(lim_lane));
  return rw;
}

// The stream's next tile to load: tile t of round r's block, and what its
// loads need of that block.
struct PfCursor {
  int r, t;
  int kvh, row0;  // row0: the sequence's first cache row (packed) or its block-table row (paged)
  int kend, ntiles;
  bool live;
};

}  // namespace

// Persistent: a workgroup takes the blocks of its rounds one after another,
// and its tile ring runs on across their boundaries, so the first tiles of
// the next block are in flight while the current one ends.
template <int D, int DT, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kPfWaves, 64 * kPfWaves),
                          amdgpu_waves_per_eu(2, 2))) void
prefill_kernel(DecodeArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ block_table) {
  using GE = PfGeo<D>;
  static_assert((kPfStages & (kPfStages - 1)) == 0, "ring stage of a tile by masking");
  __shared__ __attribute__((aligned(1024))) char smem_raw[kPfStages * GE::STAGE];
  ZL_LDS char* smem = (ZL_LDS char*)smem_raw;
  const int tid = threadIdx.x;
  const int wave = readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int P = (int)gridDim.x;
  const int w = (int)blockIdx.x;

  VirtualSeqs vs;
  vs.init(a.cu_q, cu, a.B, a.G, 0, a.max_len, kPfRowsLog2);
  const int N = a.Hkv * vs.V;  // blocks of the batch (the host bounds this below 2^31)
  if (pf_position(0, w, P) >= N) return;  // workgroup-uniform, before any barrier

  // The softmax takes a non-negative scale: a negative one is moved onto the
  // query operands (sign flip of every 16-bit value, exact).
  const bool flip = a.scale_log2 < 0.f;
  const float scale_log2 = flip ? -a.scale_log2 : a.scale_log2;
  i16x8 qop[kPfCB][GE::KSTEPS];
  auto load_q = [&](const long long (&orow)[kPfCB]) {
#pragma unroll
    for (int cb = 0; cb < kPfCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < GE::KSTEPS; ++kb)
        qop[cb][kb] = *(const i16x8*)(a.q + orow[cb] * D + 32 * kb + 8 * g);
  };
  auto flip_q = [&]() {
    if (flip) {
#pragma unroll
      for (int cb = 0; cb < kPfCB; ++cb)
#pragma unroll
        for (int kb = 0; kb < GE::KSTEPS; ++kb) qop[cb][kb] = qop[cb][kb] ^ (short)0x8000;
    }
  };

  int r = 0;
  PfBlock bk = pf_block(vs, a, (int)pf_position(0, w, P));
  PfRows rw = pf_rows(bk, a, wave, n);
  // The first block's query operands, waited for before any DMA.
  if (bk.ntiles > 0) {
    load_q(rw.orow);
#pragma unroll
    for (int cb = 0; cb < kPfCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < GE::KSTEPS; ++kb) touch(qop[cb][kb]);
  }

  // Tile loads.  Packed caches: the sequence's rows from cache row k0.
  // Paged caches: the pools' rows [page, row in page] through the sequence's
  // block-table row; a tile starts on a multiple of 32 tokens, so its rows
  // 0-15 lie in one page and rows 16-31 in that page or (16-token pages) the
  // next (tile_rows), and each wave's DMA covers rows of one half only:
  // waves 0 and 2 rows 0-15 (of K and of V), waves 1 and 3 rows 16-31.
  const uint32_t row_bytes = (uint32_t)a.Hkv * D * 2;
  const PfMap<D> map = pf_map<D>(wave, lane);
  // The cursor's first block with tiles at or after round r0 (live = false
  // past the last).
  auto seek = [&](int r0) {
    PfCursor c;
    c.live = false;
    c.t = 0;
    for (int rr = r0;; ++rr) {
      const long long p = pf_position(rr, w, P);
      if (p >= N) break;
      const PfBlock bb = pf_block(vs, a, (int)p);
      if (bb.ntiles > 0) {
        c.r = rr;
        c.kvh = bb.kvh;
        c.row0 = PAGED ? bb.si.b : bb.si.k0;
        c.kend = bb.kend;
        c.ntiles = bb.ntiles;
        c.live = true;
        break;
      }
    }
    return c;
  };
  PfCursor cur = seek(0);
  int issued = 0;  // tiles of the stream issued so far
  auto issue = [&]() {
    const int t0 = 32 * cur.t;
    const int nv = cur.kend - t0 < 32 ? cur.kend - t0 : 32;
    const long long seq_row0 = PAGED ? 0 : cur.row0;
    const char* kseq = (const char*)(a.k + (seq_row0 * a.Hkv + cur.kvh) * D);
    const char* vseq = (const char*)(a.v + (seq_row0 * a.Hkv + cur.kvh) * D);
    size_t tile_off;  // bytes from kseq / vseq to this wave's rows of the tile, less 32-row steps
    if constexpr (PAGED) {
      const TileRows tr = tile_rows(block_table + (long long)cur.row0 * a.max_pages, t0, nv, a.page_shift);
      tile_off = (size_t)((wave & 1) ? tr.half1 : tr.half0) * row_bytes;
    } else {
      tile_off = (size_t)t0 * row_bytes;
    }
    pf_dma_tile<D>(kseq + tile_off, vseq + tile_off, row_bytes, map, nv,
                   smem + (issued & (kPfStages - 1)) * GE::STAGE, wave);
    ++issued;
    if (++cur.t == cur.ntiles) cur = seek(cur.r + 1);
  };
  for (int s = 0; s < kPfStages - 1 && cur.live; ++s) issue();

  // Ring: a tile must have landed before its scores; the stage of tile c-1
  // (whose PV every wave has finished at the barrier) takes tile c+3.  The
  // waits count only the ring's loads; query loads and output stores issued
  // in between are older or newer memory operations of the same in-order
  // counter, so a wait may cover some of them too but never too few.
  int waited = 0;  // tiles of the stream known to be in LDS for every wave
  auto wait_tile = [&](int t) {
    const int after = issued - t - 1;  // tiles issued after t may be in flight
    if (after >= 2)
      wait_vmcnt<2 * GE::NIW>();
    else if (after == 1)
      wait_vmcnt<GE::NIW>();
    else
      wait_vmcnt<0>();
    barrier_lds();
    waited = t + 1;
  };
  const PfOffsets<D> off = pf_offsets<D>(n, g);
  // Lane offsets lie within the first 16 rows; stage bases are multiples of
  // a power of two at least that large, so OR-ing them in adds them.
  static_assert((GE::STAGE & (GE::STAGE - 1)) == 0 && GE::STAGE >= 16 * GE::ROWB, "stage bases above offsets");
  auto stage = [](int t) { return (uint32_t)(t & (kPfStages - 1)) * GE::STAGE; };

  f32x4 o[kPfCB][GE::VBLK];
  SoftmaxState sm[kPfCB];
  // Scores of a block's tile i live in sb[i & 1]: the loop body is compiled
  // twice, once per parity, so the buffers are fixed registers and need no
  // copies.
  f32x4 sb[2][kPfCB][2];
  int c0 = 0;  // the block's first tile in the stream
  if (bk.ntiles > 0) {
    wait_tile(0);
    flip_q();
    pf_scores<DT, D>(smem, PfOffsets<D>{off.k0 | stage(0), off.v0}, qop, sb[0]);
  }

  for (;;) {
#pragma unroll
    for (int cb = 0; cb < kPfCB; ++cb) {
      sm[cb] = SoftmaxState{-INFINITY, 0.f};
#pragma unroll
      for (int bb = 0; bb < GE::VBLK; ++bb) o[cb][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const long long pn = pf_position(r + 1, w, P);  // this workgroup's next block
    const bool has_next = pn < N;

    // Software pipeline: the scores of tile i+1 (matrix units) are computed
    // in the same basic block as the softmax of tile i (vector unit), so the
    // two overlap; then tile i's PV.
    int i = 0;
    auto step = [&](auto parity) __attribute__((always_inline)) {
      constexpr int CUR = decltype(parity)::value, NXT = CUR ^ 1;
      const int c = c0 + i;
      if (c + 1 < issued) {
        wait_tile(c + 1);
        if (cur.live) issue();  // into the stage of tile c-1
      }
      const bool more = i + 1 < bk.ntiles;
      const PfOffsets<D> offn{off.k0 | stage(c + 1), off.v0 | stage(c)};
      const int nv = bk.kend - 32 * i < 32 ? bk.kend - 32 * i : 32;
      POperand pop[kPfCB];
      bool grow[kPfCB];
      float dexp[kPfCB], psum[kPfCB];
      int nvc[kPfCB];
#pragma unroll
      for (int cb = 0; cb < kPfCB; ++cb) {
        const int lv = rw.lim[cb] - 32 * i + 1;
        nvc[cb] = nv < lv ? nv : lv;
      }
      const bool full = nv == 32 && 32 * i + 31 <= rw.lim_min;
      // The next scores and this tile's softmax run at raised wave priority:
      // when both waves of a SIMD can issue, the one in this mixed matrix and
      // vector phase goes first, and the other's PV MFMAs fill the matrix
      // unit behind it (measured 1-3% faster than no priority; raising the
      // PV phase instead was slower).
      __builtin_amdgcn_s_setprio(1);
      if (more && full) {
        pf_scores<DT, D>(smem, offn, qop, sb[NXT]);
        pf_softmax4<DT, false>(sb[CUR], g, nvc, scale_log2, sm, grow, dexp, psum, pop);
      } else if (more) {
        pf_scores<DT, D>(smem, offn, qop, sb[NXT]);
        pf_softmax4<DT, true>(sb[CUR], g, nvc, scale_log2, sm, grow, dexp, psum, pop);
      } else {
        pf_softmax4<DT, true>(sb[CUR], g, nvc, scale_log2, sm, grow, dexp, psum, pop);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int cb = 0; cb < kPfCB; ++cb) {
        // Rescale only when some column's running maximum moved.
        if (__ballot(grow[cb])) {
          const float alpha = grow[cb] ? exp2_fast(dexp[cb]) : 1.f;
          sm[cb].l *= alpha;
#pragma unroll
          for (int bb = 0; bb < GE::VBLK; ++bb) o[cb][bb] *= alpha;
        }
        sm[cb].l += psum[cb];
      }
      pf_pv<DT, D, GE::KBYTES>(smem, offn, pop, o);
    };
    while (i < bk.ntiles) {
      step(std::integral_constant<int, 0>{});
      if (++i == bk.ntiles) break;
      step(std::integral_constant<int, 1>{});
      ++i;
    }

    // Epilogue: lane (g, n) holds column 16cb + n, dims 16blk + 4g .. +3.
#pragma unroll
    for (int cb = 0; cb < kPfCB; ++cb) {
      const float l_tot = sum_over_groups(sm[cb].l);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const float lse_v = l_tot > 0.f ? sm[cb].m * kLn2 + __logf(l_tot) : -INFINITY;
      if (rw.valid[cb]) {
        uint16_t* dst = a.out + rw.orow[cb] * D + 4 * g;
#pragma unroll
        for (int bb = 0; bb < GE::VBLK; ++bb) store_out4<DT>(dst + 16 * bb, o[cb][bb], inv);
        if (a.lse && g == 0) a.lse[rw.orow[cb]] = lse_v;
      }
    }
    if (!has_next) break;
    c0 += bk.ntiles;
    ++r;
    bk = pf_block(vs, a, (int)pn);
    rw = pf_rows(bk, a, wave, n);
    if (bk.ntiles > 0) {
      // The query operands are loaded here, at the block's start, and
      // waited for before its first scores, outside the tile loop: loaded
      // inside it (during the previous block's last tile), they made the
      // compiler wait for them before every tile's scores, and with them for
      // every tile load in flight.
      load_q(rw.orow);
      if (waited <= c0) wait_tile(c0);
      flip_q();
      pf_scores<DT, D>(smem, PfOffsets<D>{off.k0 | stage(c0), off.v0}, qop, sb[0]);
    }
  }
}

// Two workgroups per CU (their LDS and registers), persistent over the blocks.
constexpr int kPfResident = 2 * 256;

template <int D, int DT>
static void launch_prefill_t(const DecodeArgs& a, int nblocks, hipStream_t stream) {
  const long long total = (long long)a.Hkv * nblocks;
  const dim3 grid((unsigned)(total < kPfResident ? total : kPfResident)), block(64 * kPfWaves);
  if (a.block_table)
    hipLaunchKernelGGL((prefill_kernel<D, DT, true>), grid, block, 0, stream, a, a.cu, a.block_table);
  else
    hipLaunchKernelGGL((prefill_kernel<D, DT, false>), grid, block, 0, stream, a, a.cu, a.block_table);
}

hipError_t launch_prefill(const DecodeArgs& a, int head_dim, int dtype, int max_blocks, hipStream_t stream) {
  if (max_blocks <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (dtype == kF16)
      launch_prefill_t<128, kF16>(a, max_blocks, stream);
    else
      launch_prefill_t<128, kBF16>(a, max_blocks, stream);
  } else {
    if (dtype == kF16)
      launch_prefill_t<64, kF16>(a, max_blocks, stream);
    else
      launch_prefill_t<64, kBF16>(a, max_blocks, stream);
  }
  return hipGetLastError();
}

}  // namespace zl

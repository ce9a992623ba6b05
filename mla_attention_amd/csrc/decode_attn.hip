// decode_attn.hip -- fused batched decode attention for gfx950 (MI355X),
// grouped-query layout (K, V [T, Hkv, D], D = 64 or 128).  The absorbed-MLA
// variant (576-wide latent, V inside the K row) is decode_mla.hip.
//
// One query token per (sequence, query head) attends over a packed ragged
// cache: the decode-stage fused batch attention that the ZhiLight pages put on
// the matrix units (first page, section 4 "Tensor Core 上的 Flash Attention").
//
// Kernel structure (one wavefront per workgroup, one worker per wavefront):
//  * Work split: every worker streams the same number of (unit, token) rows,
//    whatever the mix of sequence lengths; see zl_split.h.  Sequences cut
//    between workers are merged by split_merge.hip, launched right after.
//  * Data path: 32-token tiles go HBM -> LDS with 16-byte global_load_lds
//    (no VGPR round trip), each 16-lane group reading contiguous bytes of one
//    row.  The worker's run is one stream of items through a STAGES-deep LDS
//    ring (for each segment its query rows, then its tiles), STAGES-1 items
//    in flight while the oldest is consumed, across segment boundaries.  16-byte slots are XOR-swizzled per row so that both
//    the MFMA operand reads and the transposing V reads are free of bank
//    conflicts (the LDS bank rules are in zl_tile.h).
//  * QK^T: v_mfma_f32_16x16x32 with the K tile as A (16 tokens x 32 dims) and
//    the unit's query heads as B (32 dims x 16 heads, zero-padded when fewer).
//    Result lane (g, n) = 16g + n: head n, tokens 4g..4g+3 (and +16).
//  * Online softmax in fp32 per head; max and sum over the four lane groups by
//    lane exchange; exp2 with log2(e) folded into the scale.
//  * PV: O^T = V^T P^T.  V^T is the A operand, read from LDS with
//    ds_read_b64_tr_b16; P^T is the B operand straight from the score
//    registers (the tr read's token order equals the score layout, so no lane
//    exchange is needed).  O^T keeps head n in lane n, so the per-head rescale
//    is lane-local.
#include "zl_device.h"
#include "zl_kernels.h"
#include "zl_split.h"
#include "zl_tile.h"

namespace zl {

// Tile geometry per cache layout.
template <int L>
struct Geo;

template <>
struct Geo<kGqaD64> {
  static constexpr int DK = 64, DV = 64;
  static constexpr bool SHARED_KV = false;
  static constexpr int STAGES = 3;
  static constexpr int WAVES_PER_CU = 6;
  static constexpr int MAX_WAVES_PER_SIMD = 2;
  // 128-byte rows: two rows per 256-byte bank line, so row parity already
  // separates the two halves of the bank line; XOR the 8 slots with r / 2.
  __device__ static int slot(int c, int r) { return c ^ ((r >> 1) & 7); }
};

template <>
struct Geo<kGqaD128> {
  static constexpr int DK = 128, DV = 128;
  static constexpr bool SHARED_KV = false;
  static constexpr int STAGES = 3;
  static constexpr int WAVES_PER_CU = 3;
  static constexpr int MAX_WAVES_PER_SIMD = 1;
  // 256-byte rows, one bank line each: XOR the 16 slots with the row.
  __device__ static int slot(int c, int r) { return c ^ (r & 15); }
};

template <int L>
struct Tile {
  using G = Geo<L>;
  static constexpr int DK = G::DK, DV = G::DV;
  static constexpr int KROWB = DK * 2;                 // bytes per K row in LDS
  static constexpr int VROWB = G::SHARED_KV ? KROWB : DV * 2;
  static constexpr int KCPR = DK / 8;                  // 16-byte chunks per K row
  static constexpr int VCPR = DV / 8;
  static constexpr int KBYTES = 32 * KROWB;            // one tile of K
  static constexpr int VBYTES = G::SHARED_KV ? 0 : 32 * VROWB;
  static constexpr int STAGE_BYTES = KBYTES + VBYTES;
  static constexpr int NI_K = KBYTES / 1024;           // 1 KB DMA instructions per tile
  static constexpr int NI_V = VBYTES / 1024;
  static constexpr int PER_TILE = NI_K + NI_V;
  static constexpr int KSTEPS = DK / 32;
  static constexpr int VBLK = DV / 16;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tile must be whole DMA blocks");
};

// DMA one tensor's 32-row tile: 1 KB instruction i covers the tile's 16-byte
// slots 64i .. 64i+63 in row-major order, lane l loading row r = lin / CPR and
// the global chunk that the swizzle stores in slot lin % CPR (the slot
// permutation is an involution).  These per-lane byte offsets do not change
// from tile to tile, so they are computed once: a tile then costs a scalar
// base (its first row) and one 32-bit offset per instruction.  Rows past
// nvalid (a segment's last tile) are clamped to row nvalid - 1: finite data,
// masked out of the softmax.
template <int L, int NI>
struct TileMap {
  uint32_t off[NI];  // r * row_bytes + 16 * chunk
  int row[NI];       // r
  uint32_t chunk[NI];
};

template <int L, int CPR, int NI>
__device__ __forceinline__ TileMap<L, NI> tile_map(uint32_t row_bytes, int lane) {
  TileMap<L, NI> m;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int lin = 64 * i + lane;
    const int r = lin / CPR;
    m.row[i] = r;
    m.chunk[i] = 16u * (uint32_t)Geo<L>::slot(lin - r * CPR, r);
    m.off[i] = (uint32_t)r * row_bytes + m.chunk[i];
  }
  return m;
}

template <int L, int NI>
__device__ __forceinline__ void dma_tile(const char* rows, uint32_t row_bytes, const TileMap<L, NI>& m, int nvalid,
                                         ZL_LDS char* dst) {
  if (nvalid >= 32) {
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_saddr(rows, m.off[i], dst + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = m.row[i] < nvalid ? m.row[i] : nvalid - 1;
      dma16_saddr(rows, (uint32_t)rr * row_bytes + m.chunk[i], dst + i * 1024);
    }
  }
}

// The same tile from a paged cache: tile rows 0-15 and 16-31 are runs of
// rows from two scalar bases (one per half of the DMA instructions; the same
// base unless pages hold 16 tokens).  Rows past nvalid are clamped to row
// nvalid - 1, which lies in the half whose base the instruction uses.
template <int L, int NI>
__device__ __forceinline__ void dma_tile_paged(const char* pool, uint32_t row_bytes, const TileMap<L, NI>& m,
                                               const TileRows& tr, int nvalid, ZL_LDS char* dst) {
  static_assert(NI % 2 == 0 && 32 % NI == 0, "each instruction covers 32 / NI whole rows of one 16-row half");
  const char* b0 = (const char*)((uintptr_t)pool + (uintptr_t)(tr.half0 * row_bytes));
  const char* b1 = (const char*)((uintptr_t)pool + (uintptr_t)(tr.half1 * row_bytes));
  if (nvalid >= 32) {
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_saddr(i < NI / 2 ? b0 : b1, m.off[i], dst + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = m.row[i] < nvalid ? m.row[i] : nvalid - 1;
      dma16_saddr(i < NI / 2 ? b0 : b1, (uint32_t)rr * row_bytes + m.chunk[i], dst + i * 1024);
    }
  }
}

// The query item of a segment: rows h0 .. h0+15 (padding rows repeat h0; their
// results are never stored) in the K-row slot layout, repeated to fill the
// item's PER_TILE instructions so that every ring item costs the same.
template <int L>
__device__ __forceinline__ void dma_query_item(const uint16_t* qb, int nh, ZL_LDS char* dst, int lane) {
  using TL = Tile<L>;
  constexpr int QI = kHeadsPerUnit * TL::DK * 2 / 1024;  // 1 KB blocks of query rows
  static_assert(TL::PER_TILE % QI == 0, "query copies fill the item");
#pragma unroll
  for (int i = 0; i < TL::PER_TILE; ++i) {
    const int lin = 64 * (i % QI) + lane;
    const int r = lin / TL::KCPR;
    const int c = Geo<L>::slot(lin - r * TL::KCPR, r);
    dma16(qb + (long long)(r < nh ? r : 0) * TL::DK + c * 8, dst + i * 1024);
  }
}

// The query item of a virtual sequence (several new tokens per sequence): row
// r of the block is query row 16 hb + r of the sequence (new token (16 hb +
// r) / G, head kvh*G + (16 hb + r) % G); rows past the sequence's last repeat
// it.
template <int L>
__device__ __forceinline__ void dma_query_item_mq(const uint16_t* q, const VSeqInfo& si, int kvh, int G, int Hq,
                                                  ZL_LDS char* dst, int lane) {
  using TL = Tile<L>;
  constexpr int QI = kHeadsPerUnit * TL::DK * 2 / 1024;
  static_assert(TL::PER_TILE % QI == 0, "query copies fill the item");
  const uint16_t* src[QI];
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int lin = 64 * i + lane;
    const int r = lin / TL::KCPR;
    const int c = Geo<L>::slot(lin - r * TL::KCPR, r);
    src[i] = q + mq_column(si, r, kvh, G, Hq, false).row * TL::DK + c * 8;
  }
#pragma unroll
  for (int i = 0; i < TL::PER_TILE; ++i) dma16(src[i % QI], dst + i * 1024);
}

template <int L, int DT, bool PAGED, bool MQ>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64),
                          amdgpu_waves_per_eu(1, Geo<L>::MAX_WAVES_PER_SIMD))) void
decode_kernel(DecodeArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ block_table) {
  using TL = Tile<L>;
  using GE = Geo<L>;
  constexpr int STAGES = GE::STAGES;
  constexpr int DK = TL::DK, DV = TL::DV;
  // One LDS object: the ring.  (With a second __shared__ variable the
  // compiler tracks DMA per object and makes every LDS read wait for all
  // in-flight DMA.)
  __shared__ __attribute__((aligned(1024))) char smem_raw[STAGES * TL::STAGE_BYTES];
  ZL_LDS char* smem = (ZL_LDS char*)smem_raw;

  const int lane = __lane_id();
  const int n = lane & 15;
  const int g = lane >> 4;
  const int w = worker_id(blockIdx.x, a.P);
  const int B = a.B;
  const int U = a.Hkv * a.HB;
  const uint32_t k_row_bytes = (uint32_t)a.Hkv * DK * 2;  // one token's K row (all kv heads)
  const uint32_t v_row_bytes = (uint32_t)a.Hkv * DV * 2;
  const auto slot = [](int c, int r) { return GE::slot(c, r); };
  const TileMap<L, TL::NI_K> kmap = tile_map<L, TL::KCPR, TL::NI_K>(k_row_bytes, lane);
  const TileMap<L, TL::NI_V> vmap = tile_map<L, TL::VCPR, TL::NI_V>(v_row_bytes, lane);

  // (Empty sequences are written by the merge launch: no run covers them.)
  // The batch: decode sequences, or with several new tokens per sequence the
  // virtual sequences of 16 query rows.  Sequence boundaries for the lookups
  // are loaded here, before any tile load, and waited for, so that no later
  // lookup has to drain the tile loads in flight (B <= 64).
  int window = 0;
  VirtualSeqs vs;
  int NB;  // sequences on the work line
  int T;
  if constexpr (MQ) {
    vs.init(a.cu_q, cu, B, a.G, a.seg_cost, kMqRowsLog2);
    asm volatile("" : "+v"(vs.first.q0), "+v"(vs.first.nq), "+v"(vs.first.k0), "+v"(vs.first.lk));
    NB = vs.V;
    T = vs.T;
  } else {
    T = cu[B];
    window = bounds_window(cu, B, a.seg_cost);
    asm volatile("" : "+v"(window));
    NB = B;
  }
  const Line line = make_line(T, NB, a.seg_cost);
  const long long N = (long long)U * line.Tp;
  const long long per = positions_per_worker(N, a.P);
  const long long p_begin = (long long)w * per;
  const long long p_end = N < p_begin + per ? N : p_begin + per;
  const auto next_segment = [&](long long p) {
    if constexpr (MQ)
      return segment_at(p, p_end, line, vs);
    else
      return segment_at(p, p_end, line, cu, window);
  };
  Segment ds = next_segment(p_begin);
  if (lane == 0) a.first_key[w] = ds.len > 0 ? seq_key(ds.u, ds.b, NB) : -1;
  if (ds.len == 0) return;
  VSeqInfo dsi{}, sgi{};  // several new tokens: the virtual sequences of ds, sg
  if constexpr (MQ) dsi = vs.info(ds.b);

  // The run is one stream of ring items: for every segment (the part of one
  // sequence of one work unit in the run) its query rows, then its 32-token
  // K/V tiles.  Loads run STAGES-1 items ahead of the math, across segment
  // boundaries, so a new segment does not drain the pipeline.
  int dj = 0;  // next item of segment ds: 0 = query rows, 1 + k = tile k
  bool dmore = true;
  int issued = 0;
  // Paged caches: the page ids of the next tile to issue, read one item ahead
  // so that the scalar loads' latency passes under a tile of math.
  TileRows pf{0, 0};
  auto prefetch_pages = [&]() {
    if constexpr (PAGED) {
      if (dmore && dj >= 1) {
        const int k = dj - 1;
        // (Several new tokens: the pages of the virtual sequence's sequence;
        // its virtual tokens are that sequence's rows from 0.)
        const int seq = MQ ? dsi.b : ds.b;
        pf = tile_rows(block_table + (long long)seq * a.max_pages, ds.t0 + 32 * k - ds.cs,
                       min(32, ds.len - 32 * k), a.page_shift);
      }
    }
  };
  auto issue = [&]() {
    ZL_LDS char* st = smem + (issued % STAGES) * TL::STAGE_BYTES;
    const int ntl = (ds.len + 31) >> 5;
    const int kvh = ds.u / a.HB, hb = ds.u - (ds.u / a.HB) * a.HB;
    if (dj == 0) {
      if constexpr (MQ) {
        dma_query_item_mq<L>(a.q, dsi, kvh, a.G, a.Hq, st, lane);
      } else {
        const int h0 = kvh * a.G + hb * kHeadsPerUnit;
        const int nh = min(kHeadsPerUnit, a.G - hb * kHeadsPerUnit);
        dma_query_item<L>(a.q + ((long long)ds.b * a.Hq + h0) * DK, nh, st, lane);
      }
    } else {
      const int k = dj - 1;
      // Cache row of the tile's first token (virtual tokens map onto the
      // sequence's rows).
      const int tok = MQ ? dsi.k0 + (ds.t0 - ds.cs) + 32 * k : ds.t0 + 32 * k;
      const int nv = min(32, ds.len - 32 * k);
      if constexpr (PAGED) {
        dma_tile_paged<L, TL::NI_K>((const char*)(a.k + (long long)kvh * DK), k_row_bytes, kmap, pf, nv, st);
        dma_tile_paged<L, TL::NI_V>((const char*)(a.v + (long long)kvh * DV), v_row_bytes, vmap, pf, nv,
                                    st + TL::KBYTES);
      } else {
        dma_tile<L, TL::NI_K>((const char*)(a.k + (long long)kvh * DK) + (size_t)tok * k_row_bytes, k_row_bytes,
                              kmap, nv, st);
        dma_tile<L, TL::NI_V>((const char*)(a.v + (long long)kvh * DV) + (size_t)tok * v_row_bytes, v_row_bytes,
                              vmap, nv, st + TL::KBYTES);
      }
    }
    ++issued;
    if (++dj > ntl) {
      ds = next_segment(ds.p + ds.len);
      dj = 0;
      dmore = ds.len > 0;
      if constexpr (MQ)
        if (dmore) dsi = vs.info(ds.b);
    }
    prefetch_pages();
  };
  Segment sg = ds;  // the segment being computed
  int cj = 0;       // its current item
  bool first_seg = true;
  MqColumn col{};   // several new tokens: this lane's column of sg's row block
  if constexpr (MQ) {
    sgi = dsi;
    col = mq_column(sgi, n, sg.u, a.G, a.Hq, a.causal != 0);
  }
  for (int s = 0; s < STAGES - 1 && dmore; ++s) issue();

  f32x4 o[TL::VBLK];
  SoftmaxState sm{-INFINITY, 0.f};
  i16x8 qop[TL::KSTEPS];

  for (int i = 0;; ++i) {
    // Refill the stage of item i-1 (consumed), then wait for item i: at most
    // the items issued after it may still be in flight.
    if (dmore) issue();
    const int after = issued - i - 1;
    if (after >= 2)
      wait_vmcnt<2 * TL::PER_TILE>();
    else if (after == 1)
      wait_vmcnt<TL::PER_TILE>();
    else
      wait_vmcnt<0>();
    const ZL_LDS char* st = smem + (i % STAGES) * TL::STAGE_BYTES;
    const int ntl = (sg.len + 31) >> 5;
    if (cj == 0) {
      // Query item.  B operand: lane (g, n) = head n, dims 32kb + 8g .. +7.
#pragma unroll
      for (int kb = 0; kb < TL::KSTEPS; ++kb)
        qop[kb] = __builtin_bit_cast(i16x8, lds_read_b128(st + n * TL::KROWB + (slot(4 * kb + g, n) << 4)));
#pragma unroll
      for (int bb = 0; bb < TL::VBLK; ++bb) o[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
      sm = SoftmaxState{-INFINITY, 0.f};
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage free for refill
    } else {
      const int j = cj - 1;
      const ZL_LDS char* vt = GE::SHARED_KV ? st : st + TL::KBYTES;
      f32x4 s[2];
      scores<DT, TL::KSTEPS, TL::KROWB>(st, qop, n, g, slot, s);
      float alpha;
      int nvalid = min(32, sg.len - 32 * j);
      if constexpr (MQ) {
        // Causal limit of this lane's query row: cache rows up to col.lim.
        const int j0 = sg.t0 - sg.cs + 32 * j;
        nvalid = min(nvalid, col.lim - j0 + 1);
      }
      bool rescale;
      const POperand pop = softmax_update<DT>(s, g, nvalid, a.scale_log2, sm, alpha, rescale);
      if (rescale) {
#pragma unroll
        for (int bb = 0; bb < TL::VBLK; ++bb) o[bb] *= alpha;
      }
      pv_blocks<DT, TL::VBLK, TL::VROWB>(vt, pop, n, g, 0, slot, o);

      if (j == ntl - 1) {
        // ---- segment epilogue: lane (g, n) holds head n, dims 16blk + 4g .. +3.
        // Stores only; the next items are already in flight.  A split
        // sequence leaves its partial for the merge launch.
        const SeqWorkers sw = seq_workers(line, sg.u, sg.b, sg.cs, sg.ce, per);
        const int kvh = sg.u / a.HB, hb = sg.u - (sg.u / a.HB) * a.HB;
        const int h0 = kvh * a.G + hb * kHeadsPerUnit;
        const int nh = min(kHeadsPerUnit, a.G - hb * kHeadsPerUnit);
        const float l_tot = sum_over_groups(sm.l);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float lse_v = l_tot > 0.f ? sm.m * kLn2 + __logf(l_tot) : -INFINITY;
        const bool has_row = MQ ? col.valid : n < nh;
        const long long row = MQ ? col.row : (long long)sg.b * a.Hq + h0 + n;
        if (has_row) {
          if (sw.first == sw.last) {
            uint16_t* orow = a.out + row * DV + 4 * g;
#pragma unroll
            for (int blk = 0; blk < TL::VBLK; ++blk) store_out4<DT>(orow + 16 * blk, o[blk], inv);
            if (a.lse && g == 0) a.lse[row] = lse_v;
          } else {
            const int sl = 2 * w + (first_seg ? 0 : 1);
            float* po = a.part_o + ((long long)sl * kHeadsPerUnit + n) * DV + 4 * g;
#pragma unroll
            for (int blk = 0; blk < TL::VBLK; ++blk) *(f32x4*)(po + 16 * blk) = o[blk] * inv;
            if (g == 0) a.part_lse[sl * kLseSlot + n] = lse_v;
          }
        }
      }
    }
    if (++cj > ntl) {
      sg = next_segment(sg.p + sg.len);
      if (sg.len == 0) break;
      cj = 0;
      first_seg = false;
      if constexpr (MQ) {
        sgi = vs.info(sg.b);
        col = mq_column(sgi, n, sg.u, a.G, a.Hq, a.causal != 0);
      }
    }
  }
}

int default_workers(Layout layout) {
  switch (layout) {
    case kGqaD64: return 256 * Geo<kGqaD64>::WAVES_PER_CU;
    case kGqaD128: return 256 * Geo<kGqaD128>::WAVES_PER_CU;
    default: return mla_default_workers();
  }
}

template <int L, int DT>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.cu_q && a.block_table)
    hipLaunchKernelGGL((decode_kernel<L, DT, true, true>), dim3(a.P), dim3(64), 0, stream, a, a.cu,
                       a.block_table);
  else if (a.cu_q)
    hipLaunchKernelGGL((decode_kernel<L, DT, false, true>), dim3(a.P), dim3(64), 0, stream, a, a.cu,
                       a.block_table);
  else if (a.block_table)
    hipLaunchKernelGGL((decode_kernel<L, DT, true, false>), dim3(a.P), dim3(64), 0, stream, a, a.cu,
                       a.block_table);
  else
    hipLaunchKernelGGL((decode_kernel<L, DT, false, false>), dim3(a.P), dim3(64), 0, stream, a, a.cu,
                       a.block_table);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, Layout layout, int dtype, hipStream_t stream) {
  switch (layout) {
    case kGqaD64:
      return dtype == kF16 ? launch_t<kGqaD64, kF16>(a, stream) : launch_t<kGqaD64, kBF16>(a, stream);
    case kGqaD128:
      return dtype == kF16 ? launch_t<kGqaD128, kF16>(a, stream) : launch_t<kGqaD128, kBF16>(a, stream);
    default:
      return launch_mla(a, dtype, stream);
  }
}

}  // namespace zl

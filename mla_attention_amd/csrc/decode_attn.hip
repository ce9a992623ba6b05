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
//  * Data path: a worker's run is one stream of items -- for each segment its
//    query rows, then its 32-token K/V tiles.  Each item is read with
//    coalesced 16-byte loads (lane l of load i reads 16-byte chunk 64i + l of
//    the tile in row-major order, so a load covers whole 128- or 256-byte
//    rows) into one of two register buffers, two items ahead of the math.
//    When an item's turn comes its registers are written to LDS in the
//    swizzled layout the MFMA operand reads need, and the buffer is refilled
//    with the item two ahead.  (Loads into registers sustain more HBM
//    bandwidth on gfx950 than the global_load_lds path, which a plain read
//    of the same bytes and launch shape measures at 71-78% of peak against
//    78-87% for register loads.)  16-byte slots are XOR-swizzled per row so
//    that both the operand reads and the transposing V reads are free of bank
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
  static constexpr int NI_K = KBYTES / 1024;           // 16-byte loads per lane for a tile of K
  static constexpr int NI_V = VBYTES / 1024;
  static constexpr int NI = NI_K + NI_V;
  static constexpr int QI = kHeadsPerUnit * KROWB / 1024;  // ... for the 16 query rows
  static constexpr int KSTEPS = DK / 32;
  static constexpr int VBLK = DV / 16;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tile must be whole 1 KB loads");
  static_assert(QI <= NI_K, "query rows are rows 0-15 of a K tile");
};

// Load i of a 32-row tile, lane l: 16-byte chunk lin = 64i + l of the tile in
// row-major order, i.e. row r = i * RPL + l / CPR (RPL = 64 / CPR rows per
// load), chunk c = l % CPR, which lands in LDS at row r, slot slot(c, r).
// The per-lane part is computed once: the global offset grows by RPL rows per
// load (a wave-uniform step), and the LDS offset is i KB plus one of PERIOD
// per-lane values (the swizzle depends on r only through bits that repeat
// every PERIOD loads).  Rows past nvalid (a segment's last tile) are clamped
// to row nvalid - 1: finite data, masked out of the softmax.
template <int L, int CPR>
struct RowLane {
  static constexpr int RPL = 64 / CPR;
  // slot(c, r) reads r through bits 0-3 (D = 128: r & 15) or bits 1-3
  // (D = 64: (r >> 1) & 7); RPL * PERIOD = 16 rows covers both.
  static constexpr int PERIOD = 16 / RPL;
  int row0;                // l / CPR
  uint32_t chunk;          // 16 c
  uint32_t lpat[PERIOD];   // LDS offset of load k < PERIOD, less k KB
  __device__ __forceinline__ RowLane(int lane) {
    row0 = lane / CPR;
    const int c = lane - row0 * CPR;
    chunk = 16u * (uint32_t)c;
#pragma unroll
    for (int k = 0; k < PERIOD; ++k) {
      const int r = k * RPL + row0;
      lpat[k] = (uint32_t)(row0 * CPR + Geo<L>::slot(c, r)) * 16u;
    }
  }
  __device__ __forceinline__ int row(int i) const { return i * RPL + row0; }
  __device__ __forceinline__ uint32_t loff(int i) const { return (uint32_t)i * 1024u + lpat[i % PERIOD]; }
};

// N loads' registers into LDS (a whole tensor's tile, or the 16 query rows).
template <int N, class RL>
__device__ __forceinline__ void store_rows(ZL_LDS char* st, const RL& m, const u32x4* src) {
#pragma unroll
  for (int i = 0; i < N; ++i) lds_write_b128(st + m.loff(i), src[i]);
}

template <int L, int DT, bool PAGED, bool MQ>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64),
                          amdgpu_waves_per_eu(1, Geo<L>::MAX_WAVES_PER_SIMD))) void
decode_kernel(DecodeArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ block_table) {
  using TL = Tile<L>;
  using GE = Geo<L>;
  constexpr int DK = TL::DK, DV = TL::DV;
  constexpr int NI = TL::NI, NIK = TL::NI_K, QI = TL::QI;
  // One LDS object: two stages, the item being computed and the next one.
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * TL::STAGE_BYTES];
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
  static_assert(TL::KCPR == TL::VCPR, "K and V rows share the per-lane load map");
  const RowLane<L, TL::KCPR> rmap(lane);

  // (Empty sequences are written by the merge launch: no run covers them.)
  // The batch: decode sequences, or with several new tokens per sequence the
  // virtual sequences of 16 query rows.  Sequence boundaries for the lookups
  // are loaded here, once, for batches of up to 64 sequences.
  VirtualSeqs vs;
  PlainSeqs ps;
  int NB;  // sequences on the work line
  int T;
  if constexpr (MQ) {
    vs.init(a.cu_q, cu, B, a.G, a.seg_cost, a.max_len, kMqRowsLog2);
    NB = vs.V;
    T = vs.T;
  } else {
    const BatchBounds bb = batch_bounds(cu, B, a.max_len);
    ps = PlainSeqs{cu, B, a.seg_cost, a.max_len, bb.first};
    NB = B;
    T = bb.T;
  }
  const Line line = make_line(T, NB, a.seg_cost);
  const long long N = (long long)U * line.Tp;
  const long long per = positions_per_worker(N, a.P);
  const long long p_begin = (long long)w * per;
  const long long p_end = N < p_begin + per ? N : p_begin + per;
  const auto next_segment = [&](long long p) __attribute__((always_inline)) {
    if constexpr (MQ)
      return segment_at(p, p_end, line, vs);
    else
      return segment_at(p, p_end, line, ps);
  };
  Segment ds = next_segment(p_begin);
  if (ds.len == 0) return;
  VSeqInfo dsi{}, sgi{};  // several new tokens: the virtual sequences of ds, sg
  if constexpr (MQ) dsi = vs.info(ds.b);

  // The run is one stream of items: for every segment (the part of one
  // sequence of one work unit in the run) its query rows, then its 32-token
  // K/V tiles.  Items go to registers two ahead of the math, across segment
  // boundaries, so a new segment does not drain the pipeline.
  int dj = 0;  // next item of segment ds: 0 = query rows, 1 + k = tile k
  bool dmore = true;
  // Paged caches: the page ids of the next tile to load, read one item ahead
  // so that the scalar loads' latency passes under a tile of math.
  TileRows pf{0, 0};
  auto prefetch_pages = [&]() __attribute__((always_inline)) {
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
  // Load the next item into r (returns whether it is a tile).
  auto issue = [&](u32x4 (&r)[NI]) __attribute__((always_inline)) -> bool {
    if (!dmore) {
      // The run has no further item: the same number of loads from the
      // first query row (always present; the data is never used), so that
      // every step of the loop below issues NI loads.
#pragma unroll
      for (int i = 0; i < NI; ++i) r[i] = load16_stream((const char*)a.q + rmap.chunk);
      return false;
    }
    const int ntl = (ds.len + 31) >> 5;
    const int kvh = ds.u / a.HB, hb = ds.u - (ds.u / a.HB) * a.HB;
    const bool tile = dj > 0;
    // Tile k = dj - 1 (meaningless for the query item, whose addresses are
    // the ones used then): its first token's cache row (virtual tokens map
    // onto the sequence's rows) and its valid rows.
    const int k = dj - 1;
    const int last = min(32, ds.len - 32 * k) - 1;
    const char* kbase = (const char*)(a.k + (long long)kvh * DK);
    const char* vbase = (const char*)(a.v + (long long)kvh * DV);
    if constexpr (!PAGED) {
      const int tok = (MQ ? dsi.k0 : ds.row0) + (ds.t0 - ds.cs) + 32 * k;
      kbase += (long long)tok * k_row_bytes;
      vbase += (long long)tok * v_row_bytes;
    }
    // Address of row-load i of a tile of one tensor.
    const auto tile_addr = [&](const char* base, uint32_t row_bytes, int i) __attribute__((always_inline)) {
      const int rr = min(rmap.row(i), last);
      if constexpr (PAGED) {
        // Tile row r < 16 is pool row half0 + r, r >= 16 is half1 + r
        // (zl_split.h, TileRows); a clamped row takes the half it is in.
        const long long prow = (rr < 16 ? pf.half0 : pf.half1) + rr;
        return base + (size_t)prow * row_bytes + rmap.chunk;
      } else {
        return base + ((uint32_t)rr * row_bytes + rmap.chunk);
      }
    };
    // Query item: the 16 query rows (DK values each, in the layout of K-tile
    // rows 0-15; rows past the unit's heads repeat its first and are never
    // stored), loaded NI / QI times over so that every item is NI loads (the
    // repeats hit the caches) and the compiler's count of loads in flight is
    // exact.
    const char* qaddr[QI];
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int rr = rmap.row(i);
      long long qrow;
      if constexpr (MQ) {
        qrow = mq_column(dsi, rr, kvh, a.G, a.Hq, false).row;
      } else {
        const int h0 = kvh * a.G + hb * kHeadsPerUnit;
        const int nh = min(kHeadsPerUnit, a.G - hb * kHeadsPerUnit);
        qrow = (long long)ds.b * a.Hq + h0 + (rr < nh ? rr : 0);
      }
      qaddr[i] = (const char*)(a.q + qrow * DK) + rmap.chunk;
    }
#pragma unroll
    for (int i = 0; i < NIK; ++i) r[i] = load16_stream(tile ? tile_addr(kbase, k_row_bytes, i) : qaddr[i % QI]);
#pragma unroll
    for (int i = 0; i < TL::NI_V; ++i)
      r[NIK + i] = load16_stream(tile ? tile_addr(vbase, v_row_bytes, i) : qaddr[i % QI]);
    if (++dj > ntl) {
      ds = next_segment(ds.p + ds.len);
      dj = 0;
      dmore = ds.len > 0;
      if constexpr (MQ)
        if (dmore) dsi = vs.info(ds.b);
    }
    prefetch_pages();
    return tile;
  };

  Segment sg = ds;  // the segment being computed
  int cj = 0;       // its current item
  MqColumn col{};   // several new tokens: this lane's column of sg's row block
  if constexpr (MQ) {
    sgi = dsi;
    col = mq_column(sgi, n, sg.u, a.G, a.Hq, a.causal != 0);
  }

  f32x4 o[TL::VBLK];
  SoftmaxState sm{-INFINITY, 0.f};
  i16x8 qop[TL::KSTEPS];

  // Compute item cj of segment sg from LDS stage st; returns true when the
  // run is done.
  auto compute = [&](const ZL_LDS char* st) __attribute__((always_inline)) -> bool {
    const int ntl = (sg.len + 31) >> 5;
    if (cj == 0) {
      // Query item.  B operand: lane (g, n) = head n, dims 32kb + 8g .. +7.
#pragma unroll
      for (int kb = 0; kb < TL::KSTEPS; ++kb)
        qop[kb] = __builtin_bit_cast(i16x8, lds_read_b128(st + n * TL::KROWB + (slot(4 * kb + g, n) << 4)));
#pragma unroll
      for (int bb = 0; bb < TL::VBLK; ++bb) o[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
      sm = SoftmaxState{-INFINITY, 0.f};
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
            const int sl = own_slot(w, sg.t0, sg.cs);
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
      if (sg.len == 0) return true;
      cj = 0;
      if constexpr (MQ) {
        sgi = vs.info(sg.b);
        col = mq_column(sgi, n, sg.u, a.G, a.Hq, a.causal != 0);
      }
    }
    return false;
  };

  // Items alternate between two register buffers and two LDS stages: the
  // item in buffer X is written to stage X, X is refilled with the item two
  // ahead, and the item is computed from stage X.
  u32x4 ra[NI], rb[NI];
  bool ta = issue(ra);
  bool tb = issue(rb);
  auto step = [&](u32x4 (&r)[NI], bool& is_tile, ZL_LDS char* st) __attribute__((always_inline)) -> bool {
    if (is_tile) {
      store_rows<NIK>(st, rmap, r);
      store_rows<TL::NI_V>(st + TL::KBYTES, rmap, r + NIK);
    } else {
      store_rows<QI>(st, rmap, r);
    }
    is_tile = issue(r);
    return compute(st);
  };
  for (;;) {
    if (step(ra, ta, smem)) break;
    if (step(rb, tb, smem + TL::STAGE_BYTES)) break;
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

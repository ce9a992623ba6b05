// decode_mla.hip -- absorbed multi-head latent attention (DeepSeek-V2 MLA)
// decode for gfx950 (MI355X).
//
// MLA is listed as natively supported on the ZhiLight pages (first page,
// sections "技术架构" (flash_mla) and "功能生态"; second page, section "Dual
// streams, host all-reduce and the memory model").  In the absorbed form every
// query head attends over one latent row per token: 512 latent values then 64
// rotary values (1152 bytes).  K is the whole row, V its first 512 columns, so
// each row crosses HBM exactly once and both products read it from LDS.
//
// Kernel structure (one workgroup of four wavefronts per CU, one worker per
// workgroup):
//  * Work split: every worker streams the same number of (head block, token)
//    rows; see zl_split.h.  Fewer, larger workers than the GQA kernel keep the
//    number of 32 KB fp32 partials (one per split point) small; the split
//    sequences are merged by split_merge.hip.
//  * A worker's run is one stream of items through a four-stage LDS ring: for
//    each segment (the part of one sequence in the run) its query rows, then
//    its 32-token tiles.  A tile is 36 KB of contiguous HBM; the four waves
//    DMA a quarter each (9 x 1 KB global_load_lds) and the query item is
//    loaded twice to cost the same.  Three items are in flight while one is
//    used, across segment boundaries, so a new sequence does not drain the
//    pipeline.  Slots are XOR-swizzled within groups of 8 (rows are 72 slots
//    long).
//  * QK^T is split over the waves: wave w computes the 16 x 16 score block of
//    tokens 16(w % 2) .. +15 over k-steps 9(w / 2) .. +8 (half of the 576
//    dims), leaves it in a 4 KB exchange area of LDS, and after a barrier every
//    wave adds the two halves of both token blocks.  Each wave thus does a
//    quarter of the QK^T work and reads a quarter of the tile for it; the
//    softmax is computed identically in all waves.
//  * PV: wave w accumulates output dims [128w, 128w + 128) as O^T = V^T P^T with
//    V^T read transposed from the tile (ds_read_b64_tr_b16).
//  * Several new tokens per sequence: a segment's query item holds 32 query
//    rows (two blocks of 16 MFMA columns), which fill the stage, and the
//    workgroup has two groups of four waves, one per column block, each
//    doing the work above for its block on the same tiles (waves 0-3 issue
//    the loads).  16 heads of two draft tokens thus cost one pass over the
//    latent rows, and the two waves on each SIMD hide each other's MFMA and
//    LDS latency: one wave holding both blocks left the tile math exposed.
//  * Barriers: one per item when it has landed (every wave is then also done
//    with the previous item, whose stage is refilled right after), and one per
//    tile when the score halves are in LDS.
#include "zl_device.h"
#include "zl_kernels.h"
#include "zl_split.h"
#include "zl_tile.h"

namespace zl {

namespace {

constexpr int kDK = 576;                         // latent 512 + rotary 64
constexpr int kDV = 512;                         // value = latent columns [0, 512)
constexpr int kRowB = kDK * 2;                   // 1152 bytes per row
constexpr int kCPR = kDK / 8;                    // 72 16-byte slots per row
constexpr int kTileB = 32 * kRowB;               // 36 KB per 32-token tile
constexpr int kQB = kHeadsPerUnit * kRowB;       // 18 KB of query rows
constexpr int kWaves = 4;
constexpr int kNI = kTileB / 1024;               // 36 DMA instructions per tile
constexpr int kNIw = kNI / kWaves;               // 9 per wave
constexpr int kNIq = kQB / 1024;                 // 18 for the query rows
static_assert(2 * kNIq == kNI, "a query item is two copies of the rows");
constexpr int kStages = 4;
constexpr int kKSteps = kDK / 32;                // 18
constexpr int kKHalf = kKSteps / 2;              // 9 k-steps per wave
constexpr int kBlkPerWave = kDV / 16 / kWaves;   // 8 output blocks of 16 dims
constexpr int kWorkgroupsPerCU = 1;
// Blocks of 16 query columns per tile, one group of kWaves waves each: 16
// heads of one token, or with several new tokens per sequence 32 query rows
// (kMlaMqRowsLog2), so that a tile read from HBM serves e.g. 16 heads of two
// draft tokens at once.
template <bool MQ>
constexpr int column_blocks() { return MQ ? 2 : 1; }
// Score exchange: one f32x4 per lane and wave.
template <int NCB>
constexpr int lds_bytes() { return kStages * kTileB + NCB * kWaves * 1024; }  // 148 or 152 KB of 160
static_assert(kQB <= kTileB, "query rows fit one ring stage");
static_assert(2 * kQB == kTileB && (16 << (kMlaMqRowsLog2 - 4)) == 32,
              "32 query rows are exactly one ring stage");

// A 1152-byte row starts half a bank line (8 slots) after the previous one, so
// row parity separates bank-line halves; XOR inside each group of 8 slots with
// r / 2 makes the operand and transposing reads conflict-free (zl_tile.h).
__device__ __forceinline__ int slot(int c, int r) { return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)); }

// This wave's quarter of a tile: 1 KB instruction k of wave w covers slots
// 64(9w + k) .. +63 of the row-major tile, lane l loading row r = lin / 72
// and chunk slot(lin % 72, r).  These per-lane byte offsets are the same for
// every tile, so they are computed once; a tile then costs one scalar base
// (its first token's row) plus one 32-bit offset per instruction.
struct QuarterMap {
  uint32_t off[kNIw];  // r * 1152 + 16 * chunk
  int row[kNIw];       // r
};

__device__ __forceinline__ QuarterMap quarter_map(int wave, int lane) {
  QuarterMap m;
#pragma unroll
  for (int k = 0; k < kNIw; ++k) {
    const int lin = 64 * (wave * kNIw + k) + lane;
    const int r = lin / kCPR;
    m.row[k] = r;
    m.off[k] = (uint32_t)(r * kRowB + 16 * slot(lin - r * kCPR, r));
  }
  return m;
}

// Rows past nvalid (< 32 only for a segment's last tile or a short run) are
// clamped to row nvalid - 1: finite data, masked out of the softmax.  (The
// nine loads go out back to back: issued one per k-step of the score product
// instead, each still holds its wave as long -- the CU's load path, not the
// issue order, sets that cost.)
__device__ __forceinline__ void dma_quarter(const uint16_t* rows, int tok0, int nvalid, const QuarterMap& m,
                                            ZL_LDS char* dst, int wave) {
  const char* base = (const char*)rows + (size_t)tok0 * kRowB;
  if (nvalid >= 32) {
#pragma unroll
    for (int k = 0; k < kNIw; ++k) dma16_saddr(base, m.off[k], dst + (wave * kNIw + k) * 1024);
  } else {
#pragma unroll
    for (int k = 0; k < kNIw; ++k) {
      const int over = m.row[k] - (nvalid - 1);
      const uint32_t off = m.off[k] - (over > 0 ? (uint32_t)(over * kRowB) : 0u);
      dma16_saddr(base, off, dst + (wave * kNIw + k) * 1024);
    }
  }
}

// The same quarter from a paged pool.  Tile rows 0-15 (18 KB: the quarters of
// waves 0 and 1) and rows 16-31 (waves 2 and 3) are runs of rows from one
// scalar base each (the same base unless pages hold 16 tokens); rows past
// nvalid are clamped to row nvalid - 1, which lies in the wave's own half.
__device__ __forceinline__ void dma_quarter_paged(const uint16_t* pool, const TileRows& tr, int nvalid,
                                                  const QuarterMap& m, ZL_LDS char* dst, int wave) {
  static_assert(16 * kRowB == 2 * kNIw * 1024, "16 rows are the quarters of two waves");
  const long long half = wave < 2 ? tr.half0 : tr.half1;
  dma_quarter((const uint16_t*)((uintptr_t)pool + (uintptr_t)(half * kRowB)), 0, nvalid, m, dst, wave);
}

// The query item of a segment: rows h0 .. h0+15 (rows past nh repeat h0) in
// the tile's slot layout, 18 KB, loaded twice so that it costs the same nine
// instructions per wave as a tile (the second copy is never read).
__device__ __forceinline__ void dma_query_item(const uint16_t* qb, int nh, ZL_LDS char* dst, int wave,
                                               int lane) {
#pragma unroll
  for (int k = 0; k < kNIw; ++k) {
    const int i = wave * kNIw + k;
    const int lin = 64 * (i % kNIq) + lane;
    const int r = lin / kCPR;
    const int s = lin - r * kCPR;
    dma16(qb + (long long)(r < nh ? r : 0) * kDK + slot(s, r) * 8, dst + i * 1024);
  }
}

// The query item of a virtual sequence (several new tokens per sequence): row
// r (0 .. 31) is query row 32 hb + r of the sequence (new token (32 hb + r) /
// H, head (32 hb + r) % H); rows past the sequence's last repeat it.  32 rows
// fill the stage, so every instruction loads distinct data.
__device__ __forceinline__ void dma_query_item_mq(const uint16_t* q, const VSeqInfo& si, int H, ZL_LDS char* dst,
                                                  int wave, int lane) {
#pragma unroll
  for (int k = 0; k < kNIw; ++k) {
    const int i = wave * kNIw + k;
    const int lin = 64 * i + lane;
    const int r = lin / kCPR;
    const int s = lin - r * kCPR;
    dma16(q + mq_column(si, r, 0, H, H, false, kMlaMqRowsLog2).row * kDK + slot(s, r) * 8, dst + i * 1024);
  }
}

}  // namespace

// Partial scores of one 16-token block over half of the k-steps:
// lane (g, n) gets tokens 16tb + 4g .. +3 of column n, summed over dims
// [288kh, 288kh + 288).  Two accumulators halve the MFMA dependency chain.
template <int DT>
__device__ __forceinline__ f32x4 half_scores(const ZL_LDS char* kt, const i16x8 (&qop)[kKHalf], int tb,
                                             int kh, int n, int g) {
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int t = 16 * tb + n;
#pragma unroll
  for (int kb = 0; kb < kKHalf; ++kb) {
    const int c = 4 * (kKHalf * kh + kb) + g;
    const u32x4 av = lds_read_b128(kt + t * kRowB + (slot(c, t) << 4));
    if (kb & 1)
      acc1 = mfma16x16x32<DT>(__builtin_bit_cast(i16x8, av), qop[kb], acc1);
    else
      acc0 = mfma16x16x32<DT>(__builtin_bit_cast(i16x8, av), qop[kb], acc0);
  }
  return acc0 + acc1;
}

template <int DT, bool PAGED, bool MQ>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves * column_blocks<MQ>(),
                                                      64 * kWaves * column_blocks<MQ>()),
                          amdgpu_waves_per_eu(column_blocks<MQ>(), column_blocks<MQ>()))) void
mla_decode_kernel(DecodeArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ block_table) {
  constexpr int NCB = column_blocks<MQ>();
  // One LDS object only (see decode_attn.hip): [4 ring stages][score exchange].
  __shared__ __attribute__((aligned(1024))) char smem_raw[lds_bytes<NCB>()];
  ZL_LDS char* smem = (ZL_LDS char*)smem_raw;
  ZL_LDS char* xchg = smem + kStages * kTileB;
  static_assert(16 * NCB <= kMlaSlotCols, "a partial slot holds the item's columns");

  const int tid = threadIdx.x;
  const int wave = readfirstlane((tid >> 6) & (kWaves - 1));  // quarter of the tile (scalar)
  const int cb = readfirstlane(tid >> 8);                     // column block of the wave group
  const bool loader = cb == 0;                                // waves that issue the loads
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int tb_own = wave & 1;   // token block of this wave's score half
  const int kh_own = wave >> 1;  // k-step half of this wave's score half
  const int w = worker_id(blockIdx.x, a.P);
  const int B = a.B;
  const int U = a.HB;
  const int dim0 = wave * (kDV / kWaves) + 4 * g;
  const auto slot_fn = [](int c, int r) { return slot(c, r); };
  const QuarterMap qmap = quarter_map(wave, lane);

  // (Empty sequences are written by the merge launch: no run covers them.)
  // The batch: decode sequences, or with several new tokens per sequence the
  // virtual sequences of 32 query rows.  Sequence boundaries for the lookups
  // are loaded here, before any tile load, and waited for, so that no later
  // lookup has to drain the tile loads in flight (B <= 64).
  int window = 0;
  VirtualSeqs vs;
  int NB;  // sequences on the work line
  int T;
  if constexpr (MQ) {
    vs.init(a.cu_q, cu, B, a.G, a.seg_cost, kMlaMqRowsLog2);
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
  if (tid == 0) a.first_key[w] = ds.len > 0 ? seq_key(ds.u, ds.b, NB) : -1;
  if (ds.len == 0) return;  // the whole workgroup: w is per workgroup
  VSeqInfo dsi{}, sgi{};  // several new tokens: the virtual sequences of ds, sg
  if constexpr (MQ) dsi = vs.info(ds.b);

  // The run is one stream of ring items: for every segment its query item,
  // then its 32-token tiles.  The issuing side runs up to three items ahead
  // of the computing side, across segment boundaries, so a new segment does
  // not drain the pipeline.  Every item is nine DMA instructions per wave.
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
    ZL_LDS char* dst = smem + (issued % kStages) * kTileB;
    const int ntl = (ds.len + 31) >> 5;
    if (!loader) {
    } else if (dj == 0) {
      if constexpr (MQ) {
        dma_query_item_mq(a.q, dsi, a.G, dst, wave, lane);
      } else {
        const int h0 = ds.u * kHeadsPerUnit;
        dma_query_item(a.q + ((long long)ds.b * a.Hq + h0) * kDK, min(kHeadsPerUnit, a.G - h0), dst, wave,
                       lane);
      }
    } else {
      const int k = dj - 1;
      const int nv = min(32, ds.len - 32 * k);
      if constexpr (PAGED) {
        dma_quarter_paged(a.k, pf, nv, qmap, dst, wave);
      } else if constexpr (MQ) {
        // Cache row of the tile's first token (virtual tokens map onto the
        // sequence's rows).
        dma_quarter(a.k, dsi.k0 + (ds.t0 - ds.cs) + 32 * k, nv, qmap, dst, wave);
      } else {
        dma_quarter(a.k, ds.t0 + 32 * k, nv, qmap, dst, wave);
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
  // Several new tokens: this lane's column 16 cb + n of sg's row block.
  MqColumn col{};
  if constexpr (MQ) {
    sgi = dsi;
    col = mq_column(sgi, 16 * cb + n, 0, a.G, a.Hq, a.causal != 0, kMlaMqRowsLog2);
  }
  for (int s = 0; s < kStages - 1 && dmore; ++s) issue();

  f32x4 o[kBlkPerWave];
  SoftmaxState sm{-INFINITY, 0.f};
  i16x8 qop[kKHalf];

  for (int i = 0;; ++i) {
    // Item i has landed once at most the items issued after it are in flight.
    const int after = issued - i - 1;
    if (after >= 2)
      wait_vmcnt<2 * kNIw>();
    else if (after == 1)
      wait_vmcnt<kNIw>();
    else
      wait_vmcnt<0>();
    barrier_lds();  // item i complete in LDS, and every wave is past item i-1
    if (dmore) issue();  // into the stage of item i-1
    const ZL_LDS char* it = smem + (i % kStages) * kTileB;
    const int ntl = (sg.len + 31) >> 5;
    if (cj == 0) {
      // Query item: this wave's half of the k-steps of its column block, B
      // operand layout (column n is query row 16 cb + n of the item).
      const int r = 16 * cb + n;
#pragma unroll
      for (int kb = 0; kb < kKHalf; ++kb) {
        const int c = 4 * (kKHalf * kh_own + kb) + g;
        qop[kb] = __builtin_bit_cast(i16x8, lds_read_b128(it + r * kRowB + (slot(c, r) << 4)));
      }
#pragma unroll
      for (int bb = 0; bb < kBlkPerWave; ++bb) o[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
      sm = SoftmaxState{-INFINITY, 0.f};
    } else {
      const int j = cj - 1;
      ZL_LDS char* xc = xchg + cb * (kWaves * 1024) + lane * 16;  // this group's exchange area
      *(ZL_LDS f32x4*)(xc + wave * 1024) = half_scores<DT>(it, qop, tb_own, kh_own, n, g);
      barrier_lds();  // all score halves in LDS
      // Waves 0 and 2 of the group hold the halves of token block 0, waves 1
      // and 3 those of block 1.
      f32x4 s[2];
      s[0] = *(const ZL_LDS f32x4*)(xc + 0 * 1024) + *(const ZL_LDS f32x4*)(xc + 2 * 1024);
      s[1] = *(const ZL_LDS f32x4*)(xc + 1 * 1024) + *(const ZL_LDS f32x4*)(xc + 3 * 1024);
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
        for (int bb = 0; bb < kBlkPerWave; ++bb) o[bb] *= alpha;
      }
      pv_blocks<DT, kBlkPerWave, kRowB>(it, pop, n, g, wave * kBlkPerWave, slot_fn, o);

      if (j == ntl - 1) {
        // ---- segment epilogue: lane (g, n) of wave w in group cb holds
        // column 16 cb + n, dims 128w + 16bb + 4g .. +3.  Stores only; the
        // next items are in flight.  A partial slot holds 16 NCB columns.
        const SeqWorkers sw = seq_workers(line, sg.u, sg.b, sg.cs, sg.ce, per);
        const int h0 = sg.u * kHeadsPerUnit;
        const int nh = min(kHeadsPerUnit, a.G - h0);
        const float l_tot = sum_over_groups(sm.l);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float lse_v = l_tot > 0.f ? sm.m * kLn2 + __logf(l_tot) : -INFINITY;
        const bool has_row = MQ ? col.valid : n < nh;
        const long long row = MQ ? col.row : (long long)sg.b * a.Hq + h0 + n;
        if (has_row) {
          if (sw.first == sw.last) {
            uint16_t* orow = a.out + row * kDV + dim0;
#pragma unroll
            for (int bb = 0; bb < kBlkPerWave; ++bb) store_out4<DT>(orow + 16 * bb, o[bb], inv);
            if (a.lse && wave == 0 && g == 0) a.lse[row] = lse_v;
          } else {
            const int sl = 2 * w + (first_seg ? 0 : 1);
            const int c = 16 * cb + n;
            float* po = a.part_o + ((long long)sl * (16 * NCB) + c) * kDV + dim0;
#pragma unroll
            for (int bb = 0; bb < kBlkPerWave; ++bb) *(f32x4*)(po + 16 * bb) = o[bb] * inv;
            if (wave == 0 && g == 0) a.part_lse[sl * kLseSlot + c] = lse_v;
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
        col = mq_column(sgi, 16 * cb + n, 0, a.G, a.Hq, a.causal != 0, kMlaMqRowsLog2);
      }
    }
  }
}

int mla_default_workers() { return 256 * kWorkgroupsPerCU; }

template <int DT>
static void launch_mla_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.P), block(64 * kWaves);
  if (a.cu_q && a.block_table)
    hipLaunchKernelGGL((mla_decode_kernel<DT, true, true>), grid, dim3(64 * kWaves * column_blocks<true>()), 0,
                       stream, a, a.cu, a.block_table);
  else if (a.cu_q)
    hipLaunchKernelGGL((mla_decode_kernel<DT, false, true>), grid, dim3(64 * kWaves * column_blocks<true>()), 0,
                       stream, a, a.cu, a.block_table);
  else if (a.block_table)
    hipLaunchKernelGGL((mla_decode_kernel<DT, true, false>), grid, block, 0, stream, a, a.cu, a.block_table);
  else
    hipLaunchKernelGGL((mla_decode_kernel<DT, false, false>), grid, block, 0, stream, a, a.cu, a.block_table);
}

hipError_t launch_mla(const DecodeArgs& a, int dtype, hipStream_t stream) {
  if (dtype == kF16)
    launch_mla_t<kF16>(a, stream);
  else
    launch_mla_t<kBF16>(a, stream);
  return hipGetLastError();
}

}  // namespace zl

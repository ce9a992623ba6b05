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
//  * A worker's run is one stream of items: for each segment (the part of one
//    sequence in the run) its query rows, then its 32-token tiles.  A tile is
//    36 KB of contiguous HBM; each wave reads a quarter (9 x 1 KB).  One new
//    token per sequence (mla_decode_rs_kernel): the quarters go to registers
//    with coalesced 16-byte loads two items ahead of the math and are written
//    to LDS when their turn comes (two LDS stages).  Several new tokens per
//    sequence (mla_mq_kernel): global_load_lds DMA into a four-stage LDS
//    ring, three items in flight.  Either way items flow across segment
//    boundaries, so a new sequence does not drain the pipeline.  Slots are
//    XOR-swizzled within groups of 8 (rows are 72 slots long).
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
//  * Barriers: one per item once it is whole in LDS (every wave is then also
//    done with the previous item), and one per tile when the score halves are
//    in LDS.
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
constexpr int kMqColumnBlocks = 2;
// The several-new-tokens kernel's LDS: the ring, then a score exchange area
// of one f32x4 per lane and wave: 152 KB of 160.
constexpr int kMqLdsBytes = kStages * kTileB + kMqColumnBlocks * kWaves * 1024;
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

// Several new tokens per sequence (virtual sequences of 32 query rows): two
// groups of four waves, one per 16-column block, on the same tiles.
template <int DT, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves * kMqColumnBlocks, 64 * kWaves * kMqColumnBlocks),
                          amdgpu_waves_per_eu(kMqColumnBlocks, kMqColumnBlocks))) void
mla_mq_kernel(DecodeArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ block_table) {
  constexpr int NCB = kMqColumnBlocks;
  // One LDS object only (see decode_attn.hip): [4 ring stages][score exchange].
  __shared__ __attribute__((aligned(1024))) char smem_raw[kMqLdsBytes];
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
  // The batch: the virtual sequences of 32 query rows.  Sequence boundaries
  // for the lookups are loaded here, before any tile load, and waited for, so
  // that no later lookup has to drain the tile loads in flight (B <= 64).
  VirtualSeqs vs;
  vs.init(a.cu_q, cu, B, a.G, a.seg_cost, a.max_len, kMlaMqRowsLog2);
  asm volatile("" : "+v"(vs.first.q0), "+v"(vs.first.nq), "+v"(vs.first.k0), "+v"(vs.first.lk));
  const int NB = vs.V;  // sequences on the work line
  const int T = vs.T;
  const Line line = make_line(T, NB, a.seg_cost);
  const long long N = (long long)U * line.Tp;
  const long long per = positions_per_worker(N, a.P);
  const long long p_begin = (long long)w * per;
  const long long p_end = N < p_begin + per ? N : p_begin + per;
  const auto next_segment = [&](long long p) { return segment_at(p, p_end, line, vs); };
  Segment ds = next_segment(p_begin);
  if (ds.len == 0) return;  // the whole workgroup: w is per workgroup
  VSeqInfo dsi = vs.info(ds.b), sgi{};  // the virtual sequences of ds, sg

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
        // The pages of the virtual sequence's sequence; its virtual tokens
        // are that sequence's rows from 0.
        pf = tile_rows(block_table + (long long)dsi.b * a.max_pages, ds.t0 + 32 * k - ds.cs,
                       min(32, ds.len - 32 * k), a.page_shift);
      }
    }
  };
  auto issue = [&]() {
    ZL_LDS char* dst = smem + (issued % kStages) * kTileB;
    const int ntl = (ds.len + 31) >> 5;
    if (!loader) {
    } else if (dj == 0) {
      dma_query_item_mq(a.q, dsi, a.G, dst, wave, lane);
    } else {
      const int k = dj - 1;
      const int nv = min(32, ds.len - 32 * k);
      if constexpr (PAGED) {
        dma_quarter_paged(a.k, pf, nv, qmap, dst, wave);
      } else {
        // Cache row of the tile's first token (virtual tokens map onto the
        // sequence's rows).
        dma_quarter(a.k, dsi.k0 + (ds.t0 - ds.cs) + 32 * k, nv, qmap, dst, wave);
      }
    }
    ++issued;
    if (++dj > ntl) {
      ds = next_segment(ds.p + ds.len);
      dj = 0;
      dmore = ds.len > 0;
      if (dmore) dsi = vs.info(ds.b);
    }
    prefetch_pages();
  };
  Segment sg = ds;  // the segment being computed
  int cj = 0;       // its current item
  // This lane's column 16 cb + n of sg's row block.
  sgi = dsi;
  MqColumn col = mq_column(sgi, 16 * cb + n, 0, a.G, a.Hq, a.causal != 0, kMlaMqRowsLog2);
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
      {
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
        const float l_tot = sum_over_groups(sm.l);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float lse_v = l_tot > 0.f ? sm.m * kLn2 + __logf(l_tot) : -INFINITY;
        const bool has_row = col.valid;
        const long long row = col.row;
        if (has_row) {
          if (sw.first == sw.last) {
            uint16_t* orow = a.out + row * kDV + dim0;
#pragma unroll
            for (int bb = 0; bb < kBlkPerWave; ++bb) store_out4<DT>(orow + 16 * bb, o[bb], inv);
            if (a.lse && wave == 0 && g == 0) a.lse[row] = lse_v;
          } else {
            const int sl = own_slot(w, sg.t0, sg.cs);
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
      sgi = vs.info(sg.b);
      col = mq_column(sgi, 16 * cb + n, 0, a.G, a.Hq, a.causal != 0, kMlaMqRowsLog2);
    }
  }
}

// One new token per sequence: the same tile math, with each wave's quarter
// of every item read by coalesced 16-byte loads into one of two register
// buffers (two items ahead of the math) and written to LDS when its turn
// comes.  Register loads sustain more HBM bandwidth on gfx950 than the
// global_load_lds path that the several-new-tokens kernel above keeps (its
// two wave groups share each SIMD and have no registers to spare for the
// buffers).  Two LDS stages suffice: a wave writes item i into the stage of
// item i - 2 only after passing the barrier that closes the writes of item
// i - 1, which every wave reaches only after it has finished computing item
// i - 2.  The same barrier orders the score exchange area between items.
namespace {

// This wave's quarter of an item: load k, lane l covers the 16-byte chunk
// lin = 64 (9 w + k) + l of the tile in row-major order (row r = lin / 72,
// chunk c = lin % 72).  The global offset from the tile's first row is
// 16 lin (rows are contiguous), and the chunk lands in LDS at row r, slot
// slot(c, r) = 16 lin XOR 16 ((r >> 1) & 7) (the swizzle only permutes
// chunks inside aligned groups of 8, and a row starts on a 128-byte line).
// Both offsets are kept per load, so a full tile's loads and LDS writes take
// no address arithmetic.  Wave w's rows are 8w .. 8w + 7, all in one half of
// the tile.
struct QuarterLane {
  uint32_t goff[kNIw];  // 16 lin of load k
  uint32_t loff[kNIw];  // its LDS offset in a stage
  int row[kNIw];        // r of load k
  __device__ __forceinline__ QuarterLane(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < kNIw; ++k) {
      const int lin = 64 * (wave * kNIw + k) + lane;
      const int r = lin / kCPR;
      row[k] = r;
      goff[k] = 16u * (uint32_t)lin;
      loff[k] = goff[k] ^ (16u * (uint32_t)((r >> 1) & 7));
    }
  }
  // Offset of row rr (in place of this load's row) at this load's chunk.
  __device__ __forceinline__ uint32_t moved(int k, int rr) const {
    return goff[k] + (uint32_t)(rr - row[k]) * (uint32_t)kRowB;
  }
};

}  // namespace

template <int DT, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(1, 1))) void
mla_decode_rs_kernel(DecodeArgs a, const int32_t* __restrict__ cu, const int32_t* __restrict__ block_table) {
  constexpr int kRsStages = 2;
  // One LDS object only (see decode_attn.hip): [2 stages][score exchange].
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRsStages * kTileB + kWaves * 1024];
  ZL_LDS char* smem = (ZL_LDS char*)smem_raw;
  ZL_LDS char* xchg = smem + kRsStages * kTileB;

  const int tid = threadIdx.x;
  const int wave = readfirstlane(tid >> 6);  // quarter of the tile (scalar)
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
  const QuarterLane ql(wave, lane);

  // (Empty sequences are written by the merge launch: no run covers them.)
  const BatchBounds bb = batch_bounds(cu, B, a.max_len);
  const PlainSeqs ps{cu, B, a.seg_cost, a.max_len, bb.first};
  const Line line = make_line(bb.T, B, a.seg_cost);
  const long long N = (long long)U * line.Tp;
  const long long per = positions_per_worker(N, a.P);
  const long long p_begin = (long long)w * per;
  const long long p_end = N < p_begin + per ? N : p_begin + per;
  const auto next_segment = [&](long long p) __attribute__((always_inline)) {
    return segment_at(p, p_end, line, ps);
  };
  Segment ds = next_segment(p_begin);
  if (ds.len == 0) return;  // the whole workgroup: w is per workgroup

  // The run is one stream of items: for every segment its query rows, then
  // its 32-token tiles.  Every item is kNIw loads per wave (the 18 KB of
  // query rows are loaded twice over), so the compiler's count of loads in
  // flight is exact.
  int dj = 0;  // next item of segment ds: 0 = query rows, 1 + k = tile k
  bool dmore = true;
  TileRows pf{0, 0};  // paged: the page ids of the next tile, one item ahead
  auto prefetch_pages = [&]() __attribute__((always_inline)) {
    if constexpr (PAGED) {
      if (dmore && dj >= 1) {
        const int k = dj - 1;
        pf = tile_rows(block_table + (long long)ds.b * a.max_pages, ds.t0 + 32 * k - ds.cs, min(32, ds.len - 32 * k),
                       a.page_shift);
      }
    }
  };
  auto issue = [&](u32x4 (&r)[kNIw]) __attribute__((always_inline)) {
    // A wave-uniform base and one 32-bit offset per load: a full tile uses
    // the precomputed offsets; a short tile clamps rows past the last to it
    // (finite data, masked out of the softmax); the query item reads query
    // rows 0-15 (rows past the unit's heads repeat its first; tile rows
    // 16-31 fetch rows 0-15 again, never read); with no further item the
    // loads re-read the first 1 KB of the queries (never used), so that
    // every item is kNIw loads and the compiler's count of loads in flight
    // is exact.
    const char* base;
    uint32_t off[kNIw];
    const int t = dj - 1;  // tile index
    if (!dmore) {
      base = (const char*)a.q;
#pragma unroll
      for (int k = 0; k < kNIw; ++k) off[k] = ql.goff[k] & 1023u;
    } else if (dj == 0) {
      const int h0 = ds.u * kHeadsPerUnit;
      const int nh = min(kHeadsPerUnit, a.G - h0);
      base = (const char*)(a.q + ((long long)ds.b * a.Hq + h0) * kDK);
#pragma unroll
      for (int k = 0; k < kNIw; ++k) {
        const int qr = ql.row[k] & 15;
        off[k] = ql.moved(k, qr < nh ? qr : 0);
      }
    } else {
      const int last = min(32, ds.len - 32 * t) - 1;
      if constexpr (PAGED)
        base = (const char*)a.k + (size_t)(wave < 2 ? pf.half0 : pf.half1) * kRowB;
      else
        base = (const char*)a.k + (size_t)(ds.row0 + (ds.t0 - ds.cs) + 32 * t) * kRowB;
      if (last == 31) {
#pragma unroll
        for (int k = 0; k < kNIw; ++k) off[k] = ql.goff[k];
      } else {
#pragma unroll
        for (int k = 0; k < kNIw; ++k) off[k] = ql.moved(k, min(ql.row[k], last));
      }
    }
#pragma unroll
    for (int k = 0; k < kNIw; ++k) r[k] = load16_stream(base + off[k]);
    if (dmore) {
      const int ntl = (ds.len + 31) >> 5;
      if (++dj > ntl) {
        ds = next_segment(ds.p + ds.len);
        dj = 0;
        dmore = ds.len > 0;
      }
      prefetch_pages();
    }
  };

  Segment sg = ds;  // the segment being computed
  int cj = 0;       // its current item
  f32x4 o[kBlkPerWave];
  SoftmaxState sm{-INFINITY, 0.f};
  i16x8 qop[kKHalf];

  // Compute item cj of segment sg from stage `it`; true when the run is done.
  auto compute = [&](const ZL_LDS char* it) __attribute__((always_inline)) -> bool {
    const int ntl = (sg.len + 31) >> 5;
    if (cj == 0) {
      // Query item: this wave's half of the k-steps, B operand layout.
#pragma unroll
      for (int kb = 0; kb < kKHalf; ++kb) {
        const int c = 4 * (kKHalf * kh_own + kb) + g;
        qop[kb] = __builtin_bit_cast(i16x8, lds_read_b128(it + n * kRowB + (slot(c, n) << 4)));
      }
#pragma unroll
      for (int bb = 0; bb < kBlkPerWave; ++bb) o[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
      sm = SoftmaxState{-INFINITY, 0.f};
    } else {
      const int j = cj - 1;
      ZL_LDS char* xc = xchg + lane * 16;
      *(ZL_LDS f32x4*)(xc + wave * 1024) = half_scores<DT>(it, qop, tb_own, kh_own, n, g);
      barrier_lds();  // all score halves in LDS
      f32x4 s[2];
      s[0] = *(const ZL_LDS f32x4*)(xc + 0 * 1024) + *(const ZL_LDS f32x4*)(xc + 2 * 1024);
      s[1] = *(const ZL_LDS f32x4*)(xc + 1 * 1024) + *(const ZL_LDS f32x4*)(xc + 3 * 1024);
      float alpha;
      bool rescale;
      const POperand pop = softmax_update<DT>(s, g, min(32, sg.len - 32 * j), a.scale_log2, sm, alpha, rescale);
      if (rescale) {
#pragma unroll
        for (int bb = 0; bb < kBlkPerWave; ++bb) o[bb] *= alpha;
      }
      pv_blocks<DT, kBlkPerWave, kRowB>(it, pop, n, g, wave * kBlkPerWave, slot_fn, o);

      if (j == ntl - 1) {
        // ---- segment epilogue: lane (g, n) of wave w holds head n, dims
        // 128w + 16bb + 4g .. +3.  Stores only.
        const SeqWorkers sw = seq_workers(line, sg.u, sg.b, sg.cs, sg.ce, per);
        const int h0 = sg.u * kHeadsPerUnit;
        const int nh = min(kHeadsPerUnit, a.G - h0);
        const float l_tot = sum_over_groups(sm.l);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float lse_v = l_tot > 0.f ? sm.m * kLn2 + __logf(l_tot) : -INFINITY;
        const long long row = (long long)sg.b * a.Hq + h0 + n;
        if (n < nh) {
          if (sw.first == sw.last) {
            uint16_t* orow = a.out + row * kDV + dim0;
#pragma unroll
            for (int bb = 0; bb < kBlkPerWave; ++bb) store_out4<DT>(orow + 16 * bb, o[bb], inv);
            if (a.lse && wave == 0 && g == 0) a.lse[row] = lse_v;
          } else {
            const int sl = own_slot(w, sg.t0, sg.cs);
            float* po = a.part_o + ((long long)sl * kHeadsPerUnit + n) * kDV + dim0;  // 16-column slots
#pragma unroll
            for (int bb = 0; bb < kBlkPerWave; ++bb) *(f32x4*)(po + 16 * bb) = o[bb] * inv;
            if (wave == 0 && g == 0) a.part_lse[sl * kLseSlot + n] = lse_v;
          }
        }
      }
    }
    if (++cj > ntl) {
      sg = next_segment(sg.p + sg.len);
      if (sg.len == 0) return true;
      cj = 0;
    }
    return false;
  };

  // Items alternate between two register buffers and two LDS stages.
  u32x4 ra[kNIw], rb[kNIw];
  issue(ra);
  issue(rb);
  auto step = [&](u32x4 (&r)[kNIw], ZL_LDS char* st) __attribute__((always_inline)) -> bool {
#pragma unroll
    for (int k = 0; k < kNIw; ++k) lds_write_b128(st + ql.loff[k], r[k]);
    issue(r);
    barrier_lds();  // the item is whole in LDS
    return compute(st);
  };
  for (;;) {
    if (step(ra, smem)) break;
    if (step(rb, smem + kTileB)) break;
  }
}

int mla_default_workers() { return 256 * kWorkgroupsPerCU; }

template <int DT>
static void launch_mla_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.P), block(64 * kWaves), mq_block(64 * kWaves * kMqColumnBlocks);
  if (a.cu_q && a.block_table)
    hipLaunchKernelGGL((mla_mq_kernel<DT, true>), grid, mq_block, 0, stream, a, a.cu, a.block_table);
  else if (a.cu_q)
    hipLaunchKernelGGL((mla_mq_kernel<DT, false>), grid, mq_block, 0, stream, a, a.cu, a.block_table);
  else if (a.block_table)
    hipLaunchKernelGGL((mla_decode_rs_kernel<DT, true>), grid, block, 0, stream, a, a.cu, a.block_table);
  else
    hipLaunchKernelGGL((mla_decode_rs_kernel<DT, false>), grid, block, 0, stream, a, a.cu, a.block_table);
}

hipError_t launch_mla(const DecodeArgs& a, int dtype, hipStream_t stream) {
  if (dtype == kF16)
    launch_mla_t<kF16>(a, stream);
  else
    launch_mla_t<kBF16>(a, stream);
  return hipGetLastError();
}

}  // namespace zl

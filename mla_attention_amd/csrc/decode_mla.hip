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
//  * A 32-token tile is 36 KB of contiguous HBM.  The four waves DMA a quarter
//    each (9 x 1 KB global_load_lds); a three-stage LDS ring keeps two tiles in
//    flight while one is used, with a single barrier per tile.  The unit's 16
//    query rows (18 KB) arrive by DMA with the first tiles of each segment.
//    Slots are XOR-swizzled within groups of 8 (rows are 72 slots long).
//  * QK^T: every wave computes the full 32 x 16 score tile (18 MFMA k-steps per
//    16 tokens).  The duplicate work is cheap next to the memory time and keeps
//    the waves free of score exchanges; the softmax is identical in all waves.
//  * PV: wave w accumulates output dims [128w, 128w + 128) as O^T = V^T P^T with
//    V^T read transposed from the tile (ds_read_b64_tr_b16).
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
constexpr int kStages = 3;
constexpr int kKSteps = kDK / 32;                // 18
constexpr int kBlkPerWave = kDV / 16 / kWaves;   // 8 output blocks of 16 dims
constexpr int kWorkgroupsPerCU = 1;              // 3 x 36 KB + 18 KB of LDS
constexpr int kLdsBytes = kStages * kTileB + kQB;

// XOR inside each group of 8 slots; for 64 banks this keeps the 16 rows of an
// operand read and the 4 rows of a transposing read in distinct banks.
__device__ __forceinline__ int slot(int c, int r) {
  return (c & ~7) | ((c & 7) ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1)));
}

// This wave's quarter of a tile: 1 KB instruction i covers slots 64i .. 64i+63
// of the row-major tile; rows past the segment are clamped to its last row.
__device__ __forceinline__ void dma_quarter(const uint16_t* c, int tok0, int nvalid, ZL_LDS char* dst,
                                            int wave, int lane) {
#pragma unroll
  for (int k = 0; k < kNIw; ++k) {
    const int i = wave * kNIw + k;
    const int lin = 64 * i + lane;
    const int r = lin / kCPR;
    const int s = lin - r * kCPR;
    const int rr = r < nvalid ? r : nvalid - 1;
    dma16(c + (long long)(tok0 + rr) * kDK + slot(s, r) * 8, dst + i * 1024);
  }
}

// Query rows h0 .. h0+15 (rows past nh repeat h0), same slot layout as a tile;
// instruction i goes to wave i % 4.
__device__ __forceinline__ void dma_query(const uint16_t* qb, int nh, ZL_LDS char* dst, int wave,
                                          int lane) {
#pragma unroll
  for (int k = 0; k < (kNIq + kWaves - 1) / kWaves; ++k) {
    const int i = k * kWaves + wave;
    if (i < kNIq) {
      const int lin = 64 * i + lane;
      const int r = lin / kCPR;
      const int s = lin - r * kCPR;
      dma16(qb + (long long)(r < nh ? r : 0) * kDK + slot(s, r) * 8, dst + i * 1024);
    }
  }
}

}  // namespace

template <int DT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves),
                          amdgpu_waves_per_eu(1, 1))) void
mla_decode_kernel(DecodeArgs a, const int32_t* __restrict__ cu) {
  // One LDS object only (see decode_attn.hip): [3 tiles][query rows].
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
  ZL_LDS char* smem = (ZL_LDS char*)smem_raw;
  ZL_LDS char* qlds = smem + kStages * kTileB;

  const int tid = threadIdx.x;
  const int wave = readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int w = worker_id(blockIdx.x, a.P);
  const int B = a.B;
  const int U = a.HB;
  const int dim0 = wave * (kDV / kWaves) + 4 * g;
  const auto slot_fn = [](int c, int r) { return slot(c, r); };

  // Empty sequences: out = 0, lse = -inf (no worker run covers them).
  for (int idx = w; idx < B * U; idx += a.P) {
    const int b = idx / U, hb = idx - (idx / U) * U;
    if (cu[b + 1] - cu[b] != 0) continue;
    const int h0 = hb * kHeadsPerUnit;
    const int nh = min(kHeadsPerUnit, a.G - h0);
    for (int e = tid; e < nh * kDV; e += 64 * kWaves) a.out[((long long)b * a.Hq + h0) * kDV + e] = 0;
    if (a.lse && tid < nh) a.lse[(long long)b * a.Hq + h0 + tid] = -INFINITY;
  }

  const int T = cu[B];
  const long long N = (long long)U * T;
  const long long per = positions_per_worker(N, a.P);
  long long p = (long long)w * per;
  const long long p_end = N < p + per ? N : p + per;


  while (p < p_end) {
    const int u = (int)(p / T);
    const int t0 = (int)(p - (long long)u * T);
    const int b = seq_of_token(cu, B, t0);
    const int cs = cu[b], ce = cu[b + 1];
    const long long rem = p_end - p;
    const int t1 = (long long)(ce - t0) < rem ? ce : (int)(t0 + rem);
    const int len = t1 - t0;
    const long long seq_p0 = (long long)u * T + cs;
    const long long seq_p1 = (long long)u * T + ce;
    const int w_first = (int)(seq_p0 / per);
    const int w_last = (int)((seq_p1 - 1) / per);
    const int h0 = u * kHeadsPerUnit;
    const int nh = min(kHeadsPerUnit, a.G - h0);
    const int ntiles = (len + 31) >> 5;

    barrier_lds();  // every wave is done with the LDS of the previous segment
    dma_query(a.q + ((long long)b * a.Hq + h0) * kDK, nh, qlds, wave, lane);
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      const bool real = s < ntiles;
      dma_quarter(a.k, real ? t0 + 32 * s : t0, real ? min(32, len - 32 * s) : min(32, len),
                  smem + s * kTileB, wave, lane);
    }

    f32x4 o[kBlkPerWave];
#pragma unroll
    for (int i = 0; i < kBlkPerWave; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState sm{-INFINITY, 0.f};
    i16x8 qop[kKSteps];

    for (int j = 0; j < ntiles; ++j) {
      // This wave's share of tile j; tile j+1 (issued before) may still fly.
      if (j + 1 < ntiles)
        wait_vmcnt<kNIw>();
      else
        wait_vmcnt<0>();
      barrier_lds();  // tile j complete in LDS, and every wave is past tile j-1
      if (j + kStages - 1 < ntiles) {
        const int jn = j + kStages - 1;
        dma_quarter(a.k, t0 + 32 * jn, min(32, len - 32 * jn), smem + (jn % kStages) * kTileB, wave,
                    lane);
      }
      if (j == 0) {
#pragma unroll
        for (int kb = 0; kb < kKSteps; ++kb)
          qop[kb] = __builtin_bit_cast(i16x8, lds_read_b128(qlds + n * kRowB + (slot(4 * kb + g, n) << 4)));
      }
      const ZL_LDS char* kt = smem + (j % kStages) * kTileB;
      f32x4 s[2];
      scores<DT, kKSteps, kRowB>(kt, qop, n, g, slot_fn, s);
      float alpha;
      const POperand pop = softmax_update<DT>(s, g, min(32, len - 32 * j), a.scale_log2, sm, alpha);
#pragma unroll
      for (int i = 0; i < kBlkPerWave; ++i) o[i] *= alpha;
      pv_blocks<DT, kBlkPerWave, kRowB>(kt, pop, n, g, wave * kBlkPerWave, slot_fn, o);
    }

    // ---- epilogue: lane (g, n) of wave w holds head n, dims 128w + 16bb + 4g .. +3
    const float l_tot = sum_over_groups(sm.l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? sm.m * kLn2 + __logf(l_tot) : -INFINITY;
    if (n < nh) {
      if (w_first == w_last) {
        uint16_t* orow = a.out + ((long long)b * a.Hq + h0 + n) * kDV + dim0;
#pragma unroll
        for (int bb = 0; bb < kBlkPerWave; ++bb) store_out4<DT>(orow + 16 * bb, o[bb], inv);
        if (a.lse && wave == 0 && g == 0) a.lse[(long long)b * a.Hq + h0 + n] = lse_v;
      } else {
        const int sl = partial_slot(w, per, seq_p0);
        float* po = a.part_o + ((long long)sl * kHeadsPerUnit + n) * kDV + dim0;
#pragma unroll
        for (int bb = 0; bb < kBlkPerWave; ++bb) *(f32x4*)(po + 16 * bb) = o[bb] * inv;
        if (wave == 0 && g == 0) a.part_lse[sl * kLseSlot + n] = lse_v;
      }
    }
    p += len;
  }
}

int mla_default_workers() { return 256 * kWorkgroupsPerCU; }

hipError_t launch_mla(const DecodeArgs& a, int dtype, hipStream_t stream) {
  if (dtype == kF16)
    hipLaunchKernelGGL(mla_decode_kernel<kF16>, dim3(a.P), dim3(64 * kWaves), 0, stream, a, a.cu);
  else
    hipLaunchKernelGGL(mla_decode_kernel<kBF16>, dim3(a.P), dim3(64 * kWaves), 0, stream, a, a.cu);
  return hipGetLastError();
}

}  // namespace zl

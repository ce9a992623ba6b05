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
// Kernel structure (two wavefronts per workgroup, one worker per workgroup):
//  * Work split: as for the GQA kernel, every worker streams the same number
//    of (head block, token) rows; see zl_split.h.
//  * A 32-token tile is 36 KB of contiguous HBM.  The two waves DMA half of it
//    each (18 x 1 KB global_load_lds), wait for their own loads, then meet at a
//    barrier; two LDS stages let tile j+1 stream in while tile j is used.
//    Slots are XOR-swizzled within groups of 8 (rows are 72 slots long).
//  * QK^T: both waves compute the full 32 x 16 score tile (18 MFMA k-steps per
//    16 tokens; the duplicate work is cheap next to the memory time and keeps
//    the waves independent).  The softmax is identical in both waves.
//  * PV: wave w accumulates output dims [256w, 256w + 256) as O^T = V^T P^T with
//    V^T read transposed from the tile (ds_read_b64_tr_b16).  Splitting the
//    output keeps each wave's accumulators at 64 registers.
#include "zl_device.h"
#include "zl_kernels.h"
#include "zl_split.h"
#include "zl_tile.h"

namespace zl {

namespace {

constexpr int kDK = 576;               // latent 512 + rotary 64
constexpr int kDV = 512;               // value = latent columns [0, 512)
constexpr int kRowB = kDK * 2;         // 1152 bytes per row
constexpr int kCPR = kDK / 8;          // 72 16-byte slots per row
constexpr int kTileB = 32 * kRowB;     // 36 KB per 32-token tile
constexpr int kWaves = 2;
constexpr int kNIw = kTileB / 1024 / kWaves;  // 18 DMA instructions per wave per tile
constexpr int kStages = 2;
constexpr int kKSteps = kDK / 32;      // 18
constexpr int kBlkPerWave = kDV / 16 / kWaves;  // 16 output blocks of 16 dims
constexpr int kWorkgroupsPerCU = 2;    // 2 x 72 KB of LDS

// XOR inside each group of 8 slots; for 64 banks this keeps the 16 rows of an
// operand read and the 4 rows of a transposing read in distinct banks.
__device__ __forceinline__ int slot(int c, int r) {
  return (c & ~7) | ((c & 7) ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1)));
}

// This wave's half of a tile: 1 KB instruction i covers slots 64i .. 64i+63 of
// the row-major tile; rows past the segment are clamped to its last row.
__device__ __forceinline__ void dma_half(const uint16_t* c, int tok0, int nvalid, ZL_LDS char* dst,
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

}  // namespace

template <int DT>
__global__ __attribute__((amdgpu_flat_work_group_size(128, 128), amdgpu_waves_per_eu(1, 1))) void
mla_decode_kernel(DecodeArgs a, const int32_t* __restrict__ cu) {
  // One LDS object only: with a second __shared__ variable the compiler starts
  // tracking global->LDS DMA per object and makes every LDS read wait for all
  // in-flight DMA (vmcnt(0)), which would serialise the tile pipeline.
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStages * kTileB + 16];
  ZL_LDS char* smem = (ZL_LDS char*)smem_raw;
  ZL_LDS uint32_t& sh_old = *(ZL_LDS uint32_t*)(smem + kStages * kTileB);

  const int tid = threadIdx.x;
  const int wave = readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int w = worker_id(blockIdx.x, a.P);
  const int B = a.B;
  const int U = a.HB;

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
  long long per = (N + a.P - 1) / a.P;
  if (per < kMinPerWorker) per = kMinPerWorker;
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

    barrier_lds();  // both waves are done with the LDS of the previous segment
    wait_vmcnt<0>();

    i16x8 qop[kKSteps];
    {
      const uint16_t* qrow = a.q + ((long long)b * a.Hq + h0 + n) * kDK + 8 * g;
#pragma unroll
      for (int kb = 0; kb < kKSteps; ++kb) {
        u32x4 v4 = {0u, 0u, 0u, 0u};
        if (n < nh) v4 = *(const u32x4*)(qrow + 32 * kb);
        qop[kb] = __builtin_bit_cast(i16x8, v4);
      }
    }

    const int ntiles = (len + 31) >> 5;
    dma_half(a.k, t0, min(32, len), smem, wave, lane);
    // The query loads were issued before the tile DMA: waiting for them here
    // leaves the tile in flight.
#pragma unroll
    for (int kb = 0; kb < kKSteps; ++kb) touch(qop[kb]);

    f32x4 o[kBlkPerWave];
#pragma unroll
    for (int i = 0; i < kBlkPerWave; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState sm{-INFINITY, 0.f};
    const auto slot_fn = [](int c, int r) { return slot(c, r); };

    for (int j = 0; j < ntiles; ++j) {
      barrier_lds();  // stage (j+1)%2 held tile j-1: both waves finished it
      if (j + 1 < ntiles) {
        dma_half(a.k, t0 + 32 * (j + 1), min(32, len - 32 * (j + 1)),
                 smem + ((j + 1) % kStages) * kTileB, wave, lane);
        wait_vmcnt<kNIw>();
      } else {
        wait_vmcnt<0>();
      }
      barrier_lds();  // tile j complete in LDS (both halves)

      const ZL_LDS char* kt = smem + (j % kStages) * kTileB;
      f32x4 s[2];
      scores<DT, kKSteps, kRowB>(kt, qop, n, g, slot_fn, s);
      float alpha;
      const POperand pop = softmax_update<DT>(s, g, min(32, len - 32 * j), a.scale_log2, sm, alpha);
#pragma unroll
      for (int i = 0; i < kBlkPerWave; ++i) o[i] *= alpha;
      pv_blocks<DT, kBlkPerWave, kRowB>(kt, pop, n, g, wave * kBlkPerWave, slot_fn, o);
    }

    // ---- epilogue: lane (g, n) of wave w holds head n, dims 256w + 16bb + 4g .. +3
    const float l_tot = sum_over_groups(sm.l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? sm.m * kLn2 + __logf(l_tot) : -INFINITY;
    const int dim0 = wave * (kDV / kWaves) + 4 * g;
    if (w_first == w_last) {
      if (n < nh) {
        uint16_t* orow = a.out + ((long long)b * a.Hq + h0 + n) * kDV + dim0;
#pragma unroll
        for (int bb = 0; bb < kBlkPerWave; ++bb) store_out4<DT>(orow + 16 * bb, o[bb], inv);
        if (a.lse && wave == 0 && g == 0) a.lse[(long long)b * a.Hq + h0 + n] = lse_v;
      }
    } else {
      const int sl_own = partial_slot(w, per, seq_p0);
      float* po = a.part_o + ((long long)sl_own * kHeadsPerUnit + n) * kDV + dim0;
#pragma unroll
      for (int bb = 0; bb < kBlkPerWave; ++bb) store_coherent(po + 16 * bb, o[bb] * inv);
      if (wave == 0 && g == 0) store_coherent(a.part_lse + sl_own * kHeadsPerUnit + n, lse_v);
      stores_done();  // this wave's half of the partial is in memory
      __syncthreads();
      uint32_t* ctr = a.counters + (long long)u * B + b;
      if (tid == 0) sh_old = counter_add(ctr);
      __syncthreads();
      const uint32_t old = sh_old;
      const uint32_t nparts = (uint32_t)(w_last - w_first + 1);
      if (old == nparts - 1) {
        float M = -INFINITY;
        for (int wi = w_first; wi <= w_last; ++wi)
          M = fmaxf(M, load_coherent(a.part_lse + partial_slot(wi, per, seq_p0) * kHeadsPerUnit + n));
        f32x4 acc[kBlkPerWave];
#pragma unroll
        for (int i = 0; i < kBlkPerWave; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        float wsum = 0.f;
        for (int wi = w_first; wi <= w_last; ++wi) {
          const int sl = partial_slot(wi, per, seq_p0);
          const float ls = load_coherent(a.part_lse + sl * kHeadsPerUnit + n);
          const float wt = (ls == -INFINITY) ? 0.f : exp2_fast((ls - M) * kLog2e);
          wsum += wt;
          const float* pi = a.part_o + ((long long)sl * kHeadsPerUnit + n) * kDV + dim0;
#pragma unroll
          for (int bb = 0; bb < kBlkPerWave; ++bb) acc[bb] += wt * load_coherent4(pi + 16 * bb);
        }
        if (n < nh) {
          const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
          uint16_t* orow = a.out + ((long long)b * a.Hq + h0 + n) * kDV + dim0;
#pragma unroll
          for (int bb = 0; bb < kBlkPerWave; ++bb) store_out4<DT>(orow + 16 * bb, acc[bb], winv);
          if (a.lse && wave == 0 && g == 0)
            a.lse[(long long)b * a.Hq + h0 + n] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
        }
        if (tid == 0) counter_reset(ctr);  // leave the counter at zero for the next call
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

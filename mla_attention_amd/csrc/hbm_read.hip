// hbm_read.hip -- a plain streaming read of one contiguous buffer, HBM -> LDS,
// at the launch shape of a decode kernel and with its load instruction
// (16-byte global_load_lds per lane, 1 KB per wave instruction, a ring of
// STAGES items of which STAGES - 1 stay in flight), but with no arithmetic.
//
// It measures what reads of a given size and launch shape reach on this GPU:
// the ceiling against which the decode kernels' bandwidth is judged.  The
// ZhiLight pages single out HBM traffic as the cost their fused kernels cut
// (first page, section 3 "自研 Fusion Kernel"); decode attention is bound by
// it, so a read of the same bytes with nothing else to do is the honest upper
// bound for a kernel of that shape.
#include "zl_device.h"
#include "zl_kernels.h"
#include "zl_split.h"

namespace zl {

namespace {

// Workgroup w reads 1 KB blocks [w * per, min(blocks, (w + 1) * per)) of src,
// ITEM = WAVES * NI blocks per ring item, wave v taking blocks v*NI .. +NI-1 of
// each item.  Blocks past the workgroup's range re-read its last block, so
// every access stays inside the buffer.  One word of the ring goes to sink[w]
// at the end, so the reads have an observable result.
template <int WAVES, int NI, int STAGES>
__global__ __launch_bounds__(64 * WAVES) void hbm_read_kernel(const char* __restrict__ src, long long blocks,
                                                             long long per, uint32_t* __restrict__ sink) {
  static_assert((STAGES - 1) * NI < 64, "vmcnt range");
  constexpr int ITEM = WAVES * NI;
  __shared__ __attribute__((aligned(1024))) char ring_raw[STAGES * ITEM * 1024];
  ZL_LDS char* ring = (ZL_LDS char*)ring_raw;
  const int wave = readfirstlane((int)threadIdx.x >> 6);
  const int lane = (int)threadIdx.x & 63;
  const int w = worker_id((int)blockIdx.x, (int)gridDim.x);
  const long long b0 = (long long)w * per;
  const long long b1 = blocks < b0 + per ? blocks : b0 + per;
  const long long nitems = b1 > b0 ? (b1 - b0 + ITEM - 1) / ITEM : 0;
  for (long long it = 0; it < nitems; ++it) {
    ZL_LDS char* st = ring + (int)(it % STAGES) * (ITEM * 1024) + wave * (NI * 1024);
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      long long blk = b0 + it * ITEM + wave * NI + k;
      blk = blk < b1 ? blk : b1 - 1;
      dma16(src + blk * 1024 + lane * 16, st + k * 1024);
    }
    wait_vmcnt<(STAGES - 1) * NI>();
  }
  wait_vmcnt<0>();
  if (threadIdx.x == 0) sink[w] = *(const ZL_LDS uint32_t*)ring;
}

}  // namespace

int read_probe_default_workgroups(int head_dim_k) {
  return head_dim_k == 576 ? mla_default_workers() : default_workers(head_dim_k == 64 ? kGqaD64 : kGqaD128);
}

hipError_t launch_read_probe(const void* src, long long bytes, int head_dim_k, int workgroups, uint32_t* sink,
                             hipStream_t stream) {
  const long long blocks = bytes / 1024;
  if (blocks == 0) return hipSuccess;
  const long long per = (blocks + workgroups - 1) / workgroups;
  const char* s = static_cast<const char*>(src);
  // The decode kernels' shapes: GQA D = 64 and 128 (one wave, 8 KB and 16 KB
  // K+V tiles, three stages), MLA (four waves, 36 KB tiles, four stages).
  if (head_dim_k == 64)
    hipLaunchKernelGGL((hbm_read_kernel<1, 8, 3>), dim3(workgroups), dim3(64), 0, stream, s, blocks, per, sink);
  else if (head_dim_k == 128)
    hipLaunchKernelGGL((hbm_read_kernel<1, 16, 3>), dim3(workgroups), dim3(64), 0, stream, s, blocks, per, sink);
  else
    hipLaunchKernelGGL((hbm_read_kernel<4, 9, 4>), dim3(workgroups), dim3(256), 0, stream, s, blocks, per, sink);
  return hipGetLastError();
}

}  // namespace zl

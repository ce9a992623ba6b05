// hbm_read.hip -- a plain streaming read of one contiguous buffer at the
// launch shape of a decode kernel (workgroups, waves per workgroup, bytes per
// item) and with its load path -- coalesced 16-byte loads into registers, two
// items in flight per wave -- but with no arithmetic and nothing written to
// LDS.
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
// ITEM = WAVES * NI blocks per item, wave v taking blocks v*NI .. +NI-1 of
// each item into one of two register buffers (the next item's loads are in
// flight while the previous one is folded into a checksum).  Blocks past the
// workgroup's range re-read its last block, so every access stays inside the
// buffer.  The checksum goes to sink[w] only if it equals `key` (a value the
// host picks and the compiler cannot see), so the loads have a use and, in
// practice, nothing is written.
template <int WAVES, int NI>
__global__ __launch_bounds__(64 * WAVES) void hbm_read_kernel(const char* __restrict__ src, long long blocks,
                                                             long long per, uint32_t* __restrict__ sink,
                                                             uint32_t key) {
  constexpr int ITEM = WAVES * NI;
  const int wave = readfirstlane((int)threadIdx.x >> 6);
  const int lane = (int)threadIdx.x & 63;
  const int w = worker_id((int)blockIdx.x, (int)gridDim.x);
  const long long b0 = (long long)w * per;
  const long long b1 = blocks < b0 + per ? blocks : b0 + per;
  const long long nitems = b1 > b0 ? (b1 - b0 + ITEM - 1) / ITEM : 0;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 ra[NI], rb[NI];
  const auto load = [&](u32x4 (&r)[NI], long long it) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      long long blk = b0 + it * ITEM + wave * NI + k;
      blk = blk < b1 ? blk : b1 - 1;
      r[k] = load16_stream(src + blk * 1024 + lane * 16);
    }
  };
  if (nitems > 0) load(ra, 0);
  for (long long it = 0; it < nitems; it += 2) {
    if (it + 1 < nitems) load(rb, it + 1);
#pragma unroll
    for (int k = 0; k < NI; ++k) acc ^= ra[k];
    if (it + 2 < nitems) load(ra, it + 2);
    if (it + 1 < nitems) {
#pragma unroll
      for (int k = 0; k < NI; ++k) acc ^= rb[k];
    }
  }
  const uint32_t h = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (h == key) sink[w] = h;
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
  const uint32_t key = 0x9e3779b9u;
  // The decode kernels' shapes: GQA D = 64 and 128 (one wave, 8 KB and 16 KB
  // K+V tiles), MLA (four waves, 36 KB tiles, 9 KB per wave).
  if (head_dim_k == 64)
    hipLaunchKernelGGL((hbm_read_kernel<1, 8>), dim3(workgroups), dim3(64), 0, stream, s, blocks, per, sink, key);
  else if (head_dim_k == 128)
    hipLaunchKernelGGL((hbm_read_kernel<1, 16>), dim3(workgroups), dim3(64), 0, stream, s, blocks, per, sink, key);
  else
    hipLaunchKernelGGL((hbm_read_kernel<4, 9>), dim3(workgroups), dim3(256), 0, stream, s, blocks, per, sink, key);
  return hipGetLastError();
}

}  // namespace zl

// attn_combine.hip -- log-sum-exp combine of split partial attention results.
//
// Split-KV ("flash decoding", named among the engine's third-party kernels on
// the first ZhiLight page, section "技术架构") computes attention over
// disjoint token subsets and merges them exactly: with M = max_s lse_s and
// w_s = exp(lse_s - M), out = sum_s w_s O_s / sum_s w_s and
// lse = M + ln(sum_s w_s).  One wavefront per output row; HBM-bound
// (reads S * (Dv + 1) floats, writes Dv 16-bit values per row).
#include "zl_device.h"
#include "zl_kernels.h"

namespace zl {

template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // whole wavefront leaves together
  const long long rows = a.rows;

  float M = -INFINITY;
  for (int s = lane; s < a.S; s += 64) M = fmaxf(M, a.part_lse[s * rows + row]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, shfl_xor(M, off));

  uint16_t* orow = (uint16_t*)a.out + (long long)row * a.Dv;
  if (M == -INFINITY) {
    for (int e = lane; e < a.Dv; e += 64) orow[e] = 0;
    if (a.lse && lane == 0) a.lse[row] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int s = lane; s < a.S; s += 64) {
    const float ls = a.part_lse[s * rows + row];
    wsum += ls == -INFINITY ? 0.f : exp2_fast((ls - M) * kLog2e);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) wsum += shfl_xor(wsum, off);
  const float winv = 1.f / wsum;

  // Partials are loaded kBatch at a time (past the last split the loads
  // repeat it and carry no weight) and added in split order.
  constexpr int kBatch = 8;
  for (int c4 = lane; c4 * 4 < a.Dv; c4 += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.S; s0 += kBatch) {
      float ls[kBatch];
      f32x4 v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int s = min(s0 + j, a.S - 1);
        ls[j] = s0 + j < a.S ? a.part_lse[s * rows + row] : -INFINITY;
        v[j] = *(const f32x4*)(a.part_o + ((long long)s * rows + row) * a.Dv + 4 * c4);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (ls[j] == -INFINITY) continue;  // an empty split carries no weight
        acc += exp2_fast((ls[j] - M) * kLog2e) * v[j];
      }
    }
    u32x2 w;
    w[0] = pack2<DT>(acc[0] * winv, acc[1] * winv);
    w[1] = pack2<DT>(acc[2] * winv, acc[3] * winv);
    *(u32x2*)(orow + 4 * c4) = w;
  }
  if (a.lse && lane == 0) a.lse[row] = M + __logf(wsum);
}

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream) {
  const dim3 grid((a.rows + 3) / 4);
  if (dtype == kF16)
    hipLaunchKernelGGL(combine_kernel<kF16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<kBF16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace zl

// split_merge.hip -- the log-sum-exp merge of split sequences, as a second
// launch after the decode kernel.
//
// The decode kernels cut the ragged batch into equal runs of (unit, token)
// positions, so a sequence may be shared by several workers; each of them
// leaves an fp32 partial (O / l and lse per head) in the workspace.  This
// kernel merges them exactly (split-KV "flash decoding"; the first ZhiLight
// page names flash_decoding among the engine's kernels, section "技术架构"):
//   M = max_s lse_s,  w_s = exp(lse_s - M),
//   out = sum_s w_s O_s / sum_s w_s,  lse = M + ln(sum_s w_s).
// One workgroup per (unit, sequence) -- several for wide rows -- so that the
// sequence's bounds and its range of workers are worked out once, in scalar
// registers; one thread per (head, 4-float column) then loads up to 16
// partials at once, so a merge costs about one memory round trip after the
// bounds.  Sequences that one worker covered alone were already written by
// the decode kernel; their workgroups return at once.  Empty sequences, which
// no worker covers, get out = 0 and lse = -inf here.  The partials are
// visible here because kernels on one stream are ordered and caches are
// written back / invalidated between launches.
#include "zl_device.h"
#include "zl_kernels.h"
#include "zl_split.h"
#include "zl_tile.h"

namespace zl {

// Several new query tokens per sequence (MQ): one workgroup per (key/value
// head, virtual sequence of 2^rows_log2 query rows), for an upper bound on
// the number of virtual sequences; the workgroups past the batch's count
// return at once.  A partial slot holds a.slot_cols columns.
template <int DT, int DV, bool MQ>
__global__ __launch_bounds__(256) void split_merge_kernel(DecodeArgs a, const int32_t* __restrict__ cu,
                                                          int heads_per_unit, int wg_per_seq, int seqs) {
  constexpr int C4 = DV / 4;  // float4 columns per output row
  // Workgroup -> (unit u, sequence b, part); all wave-uniform.
  const int part = (int)blockIdx.x % wg_per_seq;
  const int ub = (int)blockIdx.x / wg_per_seq;
  const int b = ub % seqs;
  const int u = ub / seqs;
  const int kvh = u / a.HB, hb = u - (u / a.HB) * a.HB;
  const int nh = MQ ? (1 << a.rows_log2) : min(kHeadsPerUnit, a.G - hb * kHeadsPerUnit);
  const long long sc = a.slot_cols;
  const int h0 = kvh * a.G + hb * kHeadsPerUnit;
  const int item = part * 256 + (int)threadIdx.x;
  const int h = item / C4;
  const int c4 = item - h * C4;
  // The sequence's bounds come from wave-wide steps (ballots, lane reads and
  // a prefix sum over the lanes; zl_split.h) that need every lane of the
  // wave: they run before any thread leaves.  Everything below them is
  // per-thread.
  int NB, T, cs, ce;
  VirtualSeqs vs;
  VSeqInfo si{};
  if constexpr (MQ) {
    vs.init(a.cu_q, cu, a.B, a.G, a.seg_cost, a.max_len, a.rows_log2);
    if (b >= vs.V) return;  // workgroup-uniform
    si = vs.info(b);
    NB = vs.V;
    T = vs.T;
    cs = si.cs;
    ce = si.ce;
  } else {
    // Clamped lengths (zl_split.h): sequence b is tokens [ccu[b], ccu[b+1])
    // of the work line; T = ccu[B].
    const BatchBounds bb = batch_bounds(cu, a.B, a.max_len);
    const SeqSpan sb = seq_bounds(cu, a.B, a.max_len, b, bb.first);
    NB = a.B;
    T = bb.T;
    cs = sb.cs;
    ce = sb.ce;
  }
  if (h >= nh || h >= heads_per_unit) return;
  long long row;  // output row of this thread's column
  if constexpr (MQ) {
    const MqColumn col = mq_column(si, h, kvh, a.G, a.Hq, false, a.rows_log2);
    if (!col.valid) return;
    row = col.row;
  } else {
    row = (long long)b * a.Hq + h0 + h;
  }
  if (ce == cs) {
    // An empty sequence (no worker run covers it): out = 0, lse = -inf.
    *(u32x2*)(a.out + row * DV + 4 * c4) = u32x2{0u, 0u};
    if (a.lse && c4 == 0) a.lse[row] = -INFINITY;
    return;
  }
  const int U = a.Hkv * a.HB;
  const Line line = make_line(T, NB, a.seg_cost);
  const long long per = positions_per_worker((long long)U * line.Tp, a.P);
  const SeqWorkers sw = seq_workers(line, u, b, cs, ce, per);
  const int w_first = sw.first, w_last = sw.last;
  if (w_first == w_last) return;
  const int nparts = w_last - w_first + 1;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, wsum = 0.f;
  constexpr int BATCH = 16;  // partials whose loads are in flight together
  for (int i0 = 0; i0 < nparts; i0 += BATCH) {
    float ls[BATCH];
    f32x4 v[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = min(i0 + j, nparts - 1);  // tail of the batch re-reads the last one
      const long long sl = part_slot(w_first, i);
      ls[j] = i0 + j < nparts ? a.part_lse[sl * kLseSlot + h] : -INFINITY;
      v[j] = *(const f32x4*)(a.part_o + (sl * sc + h) * DV + 4 * c4);
    }
    float bm = ls[0];
#pragma unroll
    for (int j = 1; j < BATCH; ++j) bm = fmaxf(bm, ls[j]);
    const float m_new = fmaxf(M, bm);
    if (m_new == -INFINITY) continue;
    const float rs = exp2_fast((M - m_new) * kLog2e);  // 0 while M is -inf
    wsum *= rs;
    acc *= rs;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const float wt = exp2_fast((ls[j] - m_new) * kLog2e);  // 0 for -inf
      wsum += wt;
      acc += wt * v[j];
    }
    M = m_new;
  }
  const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
  store_out4<DT>(a.out + row * DV + 4 * c4, acc, winv);
  if (a.lse && c4 == 0) a.lse[row] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

template <int DT, int DV>
static hipError_t launch_merge_t(const DecodeArgs& a, int max_vseqs, hipStream_t stream) {
  const bool mq = a.cu_q != nullptr;
  const int hpu = mq ? (1 << a.rows_log2) : (a.G < kHeadsPerUnit ? a.G : kHeadsPerUnit);
  const int wg_per_seq = (hpu * (DV / 4) + 255) / 256;
  const int seqs = mq ? max_vseqs : a.B;
  const long long blocks = (long long)a.Hkv * a.HB * seqs * wg_per_seq;
  if (blocks == 0) return hipSuccess;
  if (mq)
    hipLaunchKernelGGL((split_merge_kernel<DT, DV, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a, a.cu,
                       hpu, wg_per_seq, seqs);
  else
    hipLaunchKernelGGL((split_merge_kernel<DT, DV, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a,
                       a.cu, hpu, wg_per_seq, seqs);
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, int dv, int dtype, int max_vseqs, hipStream_t stream) {
  if (dv == 64)
    return dtype == kF16 ? launch_merge_t<kF16, 64>(a, max_vseqs, stream)
                         : launch_merge_t<kBF16, 64>(a, max_vseqs, stream);
  if (dv == 128)
    return dtype == kF16 ? launch_merge_t<kF16, 128>(a, max_vseqs, stream)
                         : launch_merge_t<kBF16, 128>(a, max_vseqs, stream);
  return dtype == kF16 ? launch_merge_t<kF16, 512>(a, max_vseqs, stream)
                       : launch_merge_t<kBF16, 512>(a, max_vseqs, stream);
}

}  // namespace zl

// zl_split.h -- token-balanced work split shared by the decode kernels.
//
// The ragged batch is viewed as one line of "positions": position
// p = u * T + t for work unit u (a key/value head, or a block of up to 16 query
// heads of it) and packed token t (T = total tokens).  Each of the P workers
// (one wavefront each) owns an equal run of `per` positions, so every worker
// streams the same number of K/V bytes whatever the mix of sequence lengths.
// A run that covers a whole sequence writes that sequence's output directly;
// a sequence cut between workers gets one fp32 partial (O / l, lse) per worker,
// merged by the split-merge kernel (split_merge.hip) launched right after.
//
// Partial slots: worker w owns slots 2w (the sequence its run starts in) and
// 2w+1 (the sequence its run ends in, when that is another one).
#pragma once

#include <stdint.h>

namespace zl {

// Positions per worker for N positions over P workers (at least 64, so that a
// tiny batch is not scattered over many workers).  The decode and the merge
// kernels must agree on it exactly.
__device__ __forceinline__ long long positions_per_worker(long long N, int P) {
  const long long per = (N + P - 1) / P;
  return per < 64 ? 64 : per;
}

// Largest b in [0, B) with cu[b] <= t; for 0 <= t < cu[B] this is the
// sequence that owns token t (empty sequences are stepped over).
__device__ __forceinline__ int seq_of_token(const int32_t* cu, int B, int t) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Slot of worker w's partial for the sequence occupying positions
// [seq_p0, seq_p1), when that sequence is split between workers.
__device__ __forceinline__ int partial_slot(int w, long long per, long long seq_p0) {
  long long w_first = seq_p0 / per;
  bool run_started_before = (w == w_first) && (seq_p0 > (long long)w * per);
  return 2 * w + (run_started_before ? 1 : 0);
}

// Worker id from the block id: consecutive worker ids are placed on the same
// XCD (blocks are dealt round-robin over the 8 XCDs), so the workers that
// share a split sequence mostly share one L2.
__device__ __forceinline__ int worker_id(int block, int P) {
  int per_xcd = P >> 3;
  return (block & 7) * per_xcd + (block >> 3);
}

}  // namespace zl

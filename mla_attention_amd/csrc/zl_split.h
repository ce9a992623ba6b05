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
// sequence that owns token t (empty sequences are stepped over).  Because cu
// is non-decreasing with cu[0] = 0, it equals the number of b in [1, B) with
// cu[b] <= t.  The lanes of the wave load cu 64 entries at a time and count
// with a ballot, so a batch of up to 64 sequences costs one memory round trip
// instead of the log2(B) dependent loads of a bisection.  Call from
// wave-uniform control flow with all 64 lanes active.
__device__ __forceinline__ int seq_of_token(const int32_t* cu, int B, int t) {
  const int lane = __lane_id();
  int count = 0;
  for (int i0 = 1; i0 < B; i0 += 64) {
    const int i = i0 + lane;
    const bool le = i < B && cu[i] <= t;
    count += __popcll(__ballot(le));
  }
  return __builtin_amdgcn_readfirstlane(count);
}

// Lane l holds cu[1 + l] (INT_MAX past cu[B]): the boundaries of a batch of
// up to 64 sequences in one vector load.  Issue it before a segment's
// prologue DMA: its use then waits only for itself, not for the tiles.
__device__ __forceinline__ int bounds_window(const int32_t* cu, int B) {
  const int i = 1 + __lane_id();
  const int v = cu[i < B ? i : B];  // unpredicated load (a branch here would
                                    // make the compiler's wait drain the DMA)
  return i <= B ? v : 0x7fffffff;
}

struct SeqSpan {
  int b;       // sequence owning the token
  int cs, ce;  // cu[b], cu[b + 1]
};

// The sequence owning token t (0 <= t < cu[B]) and its bounds: from the
// window when B <= 64 (a ballot and two lane reads), else by the search above.
__device__ __forceinline__ SeqSpan find_seq(const int32_t* cu, int B, int t, int window) {
  SeqSpan r;
  if (B <= 64) {
    r.b = __popcll(__ballot(window <= t));
    r.ce = __builtin_amdgcn_readlane(window, r.b);
    r.cs = r.b == 0 ? 0 : __builtin_amdgcn_readlane(window, r.b - 1);
  } else {
    r.b = seq_of_token(cu, B, t);
    r.cs = cu[r.b];
    r.ce = cu[r.b + 1];
  }
  return r;
}

// One segment of a worker's run: tokens [t0, t0 + len) of sequence b (whose
// tokens are [cs, ce)) in work unit u, starting at position p.
struct Segment {
  long long p;
  int u, t0, len, b, cs, ce;
};

// Position p -> (unit, token); 32-bit division when the position line fits.
__device__ __forceinline__ void split_position(long long p, int T, int& u, int& t) {
  if (p < 0x7fffffffLL) {
    u = (int)p / T;
    t = (int)p - u * T;
  } else {
    u = (int)(p / T);
    t = (int)(p - (long long)u * T);
  }
}

// The segment that starts at position p of a run ending at p_end (p < p_end).
__device__ __forceinline__ Segment segment_at(long long p, long long p_end, int T, const int32_t* cu, int B,
                                              int window) {
  Segment s;
  s.p = p;
  split_position(p, T, s.u, s.t0);
  const SeqSpan q = find_seq(cu, B, s.t0, window);
  s.b = q.b;
  s.cs = q.cs;
  s.ce = q.ce;
  const long long rem = p_end - p;
  s.len = (long long)(q.ce - s.t0) < rem ? q.ce - s.t0 : (int)rem;
  return s;
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

// zl_split.h -- the work split shared by the decode kernels and the merge.
//
// The ragged batch is viewed as one line of "positions".  Work unit u (a
// key/value head, or a block of up to 16 query heads of it) owns positions
// [u*Tp, (u+1)*Tp) with Tp = T + B*C (T = total tokens, B = batch, C = the
// segment cost below).  Inside a unit, sequence b owns [cpos(b), cpos(b+1))
// with cpos(b) = ccu[b] + b*C (ccu: the prefix sums of the clamped sequence
// lengths, below): first C "phantom" positions that carry no token, then one
// position per token.  Each of the P workers owns an equal run of `per`
// positions.
//
// The phantom positions stand for the fixed cost of starting a sequence in a
// run (its query rows, a partly filled last tile, the epilogue stores): a run
// that starts k sequences carries about k*C fewer tokens, so runs that cross
// sequence boundaries do not finish last.  A run starting inside a phantom
// stretch begins at the sequence's first token.
//
// Cuts between runs are aligned to a grid of kTokenGrid tokens counted from
// each sequence's first token: the cut for a run boundary at position B is
// the first grid token at or after the first token at a position >= B.  So
// every tile of a run starts on the grid (only a sequence's last tile is
// partial), and with a paged cache a tile never straddles a page boundary
// when pages hold at least kTokenGrid tokens.  Token t is then held by the
// run that holds position token_position(cs + floor_grid(t - cs)), and every
// run between a sequence's first and last holds at least kTokenGrid of its
// tokens (runs are at least 64 positions long).
//
// A run that covers a whole sequence writes that sequence's output directly;
// a sequence cut between runs gets one fp32 partial (O / l, lse) per run,
// merged by the split-merge kernel (split_merge.hip) launched right after.
// Partial slots: run w writes slot 2w for a segment cut at its start (the
// sequence began in an earlier run) and slot 2w + 1 for a segment cut only at
// its end (it began in this run).  A run holds at most one of each: only its
// first segment can be cut at its start, only its last at its end, and a
// segment cut at both ends is the run's only one.  So part k of a sequence
// whose first run is wf is in slot 2wf + 1 for k = 0 and 2(wf + k) for k >= 1
// (part_slot), which the merge computes with no lookup.
#pragma once

#include <stdint.h>

namespace zl {

constexpr int kTokenGrid = 32;  // the tile height of both decode kernels

// Positions per worker for N positions over P workers (at least 64, so that a
// tiny batch is not scattered over many workers).  The decode and the merge
// kernels must agree on it exactly.
__device__ __forceinline__ long long positions_per_worker(long long N, int P) {
  const long long per = (N + P - 1) / P;
  return per < 64 ? 64 : per;
}

// Sequence lengths are clamped: sequence b has L_b = clamp(cu[b+1] - cu[b],
// 0, M) tokens (M = max_seqlen_k), its rows start at cache row cu[b], and the
// work line numbers the batch's tokens by the prefix sums ccu of the clamped
// lengths (ccu[0] = 0, ccu[b+1] = ccu[b] + L_b).  A sequence longer than M
// thus attends over its first M rows, and a length below 0 (cu decreasing)
// counts as 0; with a valid cu (non-decreasing, lengths at most M) ccu = cu.
//
// Sequences c0 .. c0+63, one per lane (lanes past the batch hold an empty
// sequence): the clamped length, the prefix sums ccu around the lane's
// sequence, and its first cache row.  carry = ccu[c0].  Call from
// wave-uniform control flow with all 64 lanes active.
struct SeqChunk {
  int len;   // L_b
  int excl;  // ccu[b]
  int incl;  // ccu[b + 1]
  int row0;  // cu[b]
};

__device__ __forceinline__ SeqChunk seq_chunk(const int32_t* cu, int B, int M, int c0, int carry) {
  const int b = c0 + __lane_id();
  // Unpredicated loads at clamped indices (a branch here would make the
  // compiler's wait drain the tile loads in flight).
  const int s = cu[b < B ? b : B];
  const int e = cu[b < B ? b + 1 : B];
  const long long raw = (long long)e - (long long)s;
  SeqChunk c;
  c.len = b < B ? (int)(raw < 0 ? 0 : (raw > M ? M : raw)) : 0;
  c.incl = carry + wave_inclusive_sum(c.len);
  c.excl = c.incl - c.len;
  c.row0 = s;
  return c;
}

// The first chunk (sequences 0 .. 63), and T = ccu[B] for the whole batch.
struct BatchBounds {
  SeqChunk first;
  int T;
};

__device__ __forceinline__ BatchBounds batch_bounds(const int32_t* cu, int B, int M) {
  BatchBounds bb;
  bb.first = seq_chunk(cu, B, M, 0, 0);
  int T = __builtin_amdgcn_readlane(bb.first.incl, 63);
  for (int c0 = 64; c0 < B; c0 += 64) T = __builtin_amdgcn_readlane(seq_chunk(cu, B, M, c0, T).incl, 63);
  bb.T = T;
  return bb;
}

struct SeqSpan {
  int b;       // sequence whose stretch holds the position
  int cs, ce;  // ccu[b], ccu[b + 1]: its tokens on the work line
  int row0;    // cu[b]: the cache row of its first token
};

// The sequence whose stretch holds in-unit position r (0 <= r < Tp; an empty
// sequence owns only its phantom stretch): the largest b with cpos(b) =
// ccu[b] + b*C <= r, i.e. the number of boundaries i in [1, B) with
// cpos(i) <= r (cpos increases with i).  A chunk answers with a ballot and
// lane reads; the first chunk is the one held in registers, later chunks
// (batches over 64 sequences) are loaded as the search reaches them.
__device__ __forceinline__ SeqSpan find_seq(const int32_t* cu, int B, int M, int C, int r, const SeqChunk& first) {
  SeqChunk ch = first;
  int c0 = 0;
  for (;;) {
    // Lane l holds boundary i = c0 + l + 1: cpos(i) = ch.incl + i*C.
    const int i = c0 + __lane_id() + 1;
    const unsigned long long m = __ballot(i < B && ch.incl + i * C <= r);
    if (m != ~0ull || c0 + 64 >= B) {
      const int l = __popcll(m);  // sequence c0 + l
      SeqSpan s;
      s.b = c0 + l;
      s.cs = __builtin_amdgcn_readlane(ch.excl, l);
      s.ce = __builtin_amdgcn_readlane(ch.incl, l);
      s.row0 = __builtin_amdgcn_readlane(ch.row0, l);
      return s;
    }
    const int carry = __builtin_amdgcn_readlane(ch.incl, 63);
    c0 += 64;
    ch = seq_chunk(cu, B, M, c0, carry);
  }
}

// Sequence b's bounds (for the merge, which knows b): ccu[b], ccu[b + 1].
__device__ __forceinline__ SeqSpan seq_bounds(const int32_t* cu, int B, int M, int b, const SeqChunk& first) {
  SeqChunk ch = first;
  int c0 = 0;
  while (b >= c0 + 64) {
    const int carry = __builtin_amdgcn_readlane(ch.incl, 63);
    c0 += 64;
    ch = seq_chunk(cu, B, M, c0, carry);
  }
  SeqSpan s;
  s.b = b;
  s.cs = __builtin_amdgcn_readlane(ch.excl, b - c0);
  s.ce = __builtin_amdgcn_readlane(ch.incl, b - c0);
  s.row0 = __builtin_amdgcn_readlane(ch.row0, b - c0);
  return s;
}

// The position line of one call.
struct Line {
  int T;         // total tokens
  int B;         // batch
  int C;         // phantom positions per sequence
  long long Tp;  // positions per unit
};

__device__ __forceinline__ Line make_line(int T, int B, int C) {
  return Line{T, B, C, (long long)T + (long long)B * C};
}

// Position of token t of sequence b in unit u.
__device__ __forceinline__ long long token_position(const Line& L, int u, int b, int t) {
  return (long long)u * L.Tp + t + (long long)(b + 1) * L.C;
}

// One segment of a worker's run: tokens [t0, t0 + len) of sequence b (whose
// tokens are [cs, ce)) in work unit u; p is the position of token t0.
// len == 0 means that the run holds no further token.
struct Segment {
  long long p;
  int u, t0, len, b, cs, ce;
  int row0;  // cache row of the sequence's first token (plain batches)
};

// Position -> (unit, in-unit position); 32-bit division when it fits.
__device__ __forceinline__ void split_position(long long p, long long Tp, int& u, int& r) {
  if (p < 0x7fffffffLL && Tp < 0x7fffffffLL) {
    u = (int)p / (int)Tp;
    r = (int)p - u * (int)Tp;
  } else {
    u = (int)(p / Tp);
    r = (int)(p - (long long)u * Tp);
  }
}

// The cut in sequence [cs, ce) for a run boundary whose token index is x (the
// boundary lies at the position of token x, which may be outside [cs, ce)):
// the first grid token at or after clamp(x, cs, ce), at most ce.
__device__ __forceinline__ int grid_cut(long long x, int cs, int ce) {
  const int raw = x <= cs ? cs : (x >= ce ? ce : (int)x);
  const int up = cs + ((raw - cs + kTokenGrid - 1) & ~(kTokenGrid - 1));
  return up < ce ? up : ce;
}

// The first segment of the run [p, p_end): tokens [grid_cut(p), grid_cut(p_end))
// of the first sequence, at a position >= p, where that range is not empty
// (phantom stretches, empty sequences and sequences whose share of the run
// rounds away are stepped over).
template <class Seqs>
__device__ __forceinline__ Segment segment_at(long long p, long long p_end, const Line& L, const Seqs& seqs) {
  Segment s;
  s.p = p;
  s.u = 0;
  s.t0 = 0;
  s.len = 0;
  s.b = 0;
  s.cs = 0;
  s.ce = 0;
  s.row0 = 0;
  while (p < p_end) {
    int u, r;
    split_position(p, L.Tp, u, r);
    const SeqSpan q = seqs.span(r);
    // Position of token t of this sequence: base + t.
    const long long base = (long long)u * L.Tp + (long long)(q.b + 1) * L.C;
    const int t0 = grid_cut(p - base, q.cs, q.ce);
    const int t1 = grid_cut(p_end - base, q.cs, q.ce);
    if (t1 > t0) {
      s.p = base + t0;
      s.u = u;
      s.t0 = t0;
      s.len = t1 - t0;
      s.b = q.b;
      s.cs = q.cs;
      s.ce = q.ce;
      s.row0 = q.row0;
      return s;
    }
    if (p_end - base < q.ce) return s;  // the run ends inside this sequence
    // Nothing of this sequence in the run: go on at the start of the next one.
    p = base + q.ce;
  }
  return s;
}

// The sequences of a decode batch (one query token each): sequence b is
// tokens [ccu[b], ccu[b+1]) of the work line, rows cu[b] .. of the cache.
struct PlainSeqs {
  const int32_t* cu;
  int B, C, M;
  SeqChunk first;  // sequences 0 .. 63 (batch_bounds)
  __device__ __forceinline__ SeqSpan span(int r) const { return find_seq(cu, B, M, C, r, first); }
};

// Several new query tokens per sequence.  Sequence b has nq = cu_q[b+1] -
// cu_q[b] new tokens and lk = cu_k[b+1] - cu_k[b] cached key/value rows.  For
// one key/value head, its query rows (new token i, head hh of the head's
// group of G) are numbered r = i*G + hh and cut into nblk = ceil(nq*G / 16)
// blocks of 16 -- one MFMA N dimension each (the prefill kernel uses blocks
// of 256 rows: rows_log2 = 8).  Virtual sequence (b, hb) pairs
// row block hb with all lk rows of b.  The virtual sequences of all b, in
// order, are the ragged batch that the work split cuts: virtual sequence v =
// VB(b) + hb owns virtual tokens [KB(b) + hb*lk, + lk), where VB and KB count
// the virtual sequences and virtual tokens of the sequences before b.  With
// one new token per sequence and G <= 16 this is the decode batch itself.
struct VSeqInfo {
  int v;       // virtual sequence
  int cs, ce;  // its virtual tokens
  int b, hb;   // sequence and row block
  int q0, nq;  // cu_q[b] and the sequence's new tokens
  int k0, lk;  // cu_k[b] (the key row of virtual token cs) and the cached rows
};

// Lane l describes sequence c0 + l (an empty one past the batch) given the
// virtual sequences (vcarry) and tokens (kcarry) of the sequences before c0.
struct VChunk {
  int q0, nq, k0, lk, nblk;
  int vb, vbi;     // virtual sequences before / up to and including this one
  int kb;          // virtual tokens before this one
  int start, end;  // in-unit positions of its virtual sequences: [start, end)
};

// The cache length lk is clamped to [0, M] and nq to at least 0, as for
// decode batches (lengths clamped in the kernels; see the top of the file).
__device__ __forceinline__ VChunk vchunk(const int32_t* cu_q, const int32_t* cu_k, int B, int G, int C, int M,
                                         int c0, int vcarry, int kcarry, int shift) {
  const int b = c0 + __lane_id();
  const int i0 = b < B ? b : B, i1 = b < B ? b + 1 : B;
  // Unpredicated loads (clamped indices): a branch here would make the
  // compiler's wait drain the tile loads in flight.
  const int q0 = cu_q[i0], q1 = cu_q[i1], k0 = cu_k[i0], k1 = cu_k[i1];
  const long long rawq = (long long)q1 - q0, rawk = (long long)k1 - k0;
  VChunk c;
  c.q0 = q0;
  c.nq = rawq < 0 ? 0 : (int)rawq;
  c.k0 = k0;
  c.lk = rawk < 0 ? 0 : (rawk > M ? M : (int)rawk);
  c.nblk = (c.nq * G + (1 << shift) - 1) >> shift;
  const int tok = c.nblk * c.lk;
  c.vbi = vcarry + wave_inclusive_sum(c.nblk);
  c.vb = c.vbi - c.nblk;
  c.kb = kcarry + wave_inclusive_sum(tok) - tok;
  c.start = c.kb + c.vb * C;
  c.end = c.kb + tok + c.vbi * C;
  return c;
}

struct VirtualSeqs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, G, C;
  int M;         // max_seqlen_k: cache lengths are clamped to [0, M]
  int shift;     // rows per block: 2^shift
  VChunk first;  // sequences 0 .. 63 (the whole batch when B <= 64)
  int V, T;      // virtual sequences and tokens of the batch

  __device__ __forceinline__ void init(const int32_t* cq, const int32_t* ck, int b, int g, int c, int m,
                                       int rows_log2) {
    cu_q = cq;
    cu_k = ck;
    B = b;
    G = g;
    C = c;
    M = m;
    shift = rows_log2;
    first = vchunk(cu_q, cu_k, B, G, C, M, 0, 0, 0, shift);
    V = __builtin_amdgcn_readlane(first.vbi, 63);
    T = __builtin_amdgcn_readlane(first.kb + first.nblk * first.lk, 63);
    for (int c0 = 64; c0 < B; c0 += 64) {
      const VChunk ch = vchunk(cu_q, cu_k, B, G, C, M, c0, V, T, shift);
      V = __builtin_amdgcn_readlane(ch.vbi, 63);
      T = __builtin_amdgcn_readlane(ch.kb + ch.nblk * ch.lk, 63);
    }
  }

  // The chunk holding the sequence that `pred` selects: pred(chunk) is the
  // ballot of lanes lying wholly before the target; the target is in the
  // first chunk where not every lane does.
  template <class Before>
  __device__ __forceinline__ VSeqInfo locate(Before before, int v_or_r, bool by_position) const {
    VChunk ch = first;
    int c0 = 0;
    unsigned long long m = __ballot(before(ch));
    while (m == ~0ull && c0 + 64 < B) {
      c0 += 64;
      ch = vchunk(cu_q, cu_k, B, G, C, M, c0, __builtin_amdgcn_readlane(ch.vbi, 63),
                  __builtin_amdgcn_readlane(ch.kb + ch.nblk * ch.lk, 63), shift);
      m = __ballot(before(ch));
    }
    const int l = __popcll(m);
    VSeqInfo s;
    s.b = c0 + l;
    s.q0 = __builtin_amdgcn_readlane(ch.q0, l);
    s.nq = __builtin_amdgcn_readlane(ch.nq, l);
    s.k0 = __builtin_amdgcn_readlane(ch.k0, l);
    s.lk = __builtin_amdgcn_readlane(ch.lk, l);
    const int vb = __builtin_amdgcn_readlane(ch.vb, l);
    const int kb = __builtin_amdgcn_readlane(ch.kb, l);
    if (by_position) {
      const int o = v_or_r - __builtin_amdgcn_readlane(ch.start, l);
      s.hb = o / (s.lk + C);
    } else {
      s.hb = v_or_r - vb;
    }
    s.v = vb + s.hb;
    s.cs = kb + s.hb * s.lk;
    s.ce = s.cs + s.lk;
    return s;
  }

  // The virtual sequence whose stretch holds in-unit position r (0 <= r < Tp).
  __device__ __forceinline__ VSeqInfo at_position(int r) const {
    return locate([r](const VChunk& c) { return c.end <= r; }, r, true);
  }

  // Virtual sequence v (0 <= v < V).
  __device__ __forceinline__ VSeqInfo info(int v) const {
    return locate([v](const VChunk& c) { return c.vbi <= v; }, v, false);
  }

  __device__ __forceinline__ SeqSpan span(int r) const {
    const VSeqInfo s = at_position(r);
    return SeqSpan{s.v, s.cs, s.ce, s.k0};
  }
};

// Column n of a virtual sequence's row block, for key/value head kvh: the
// query row it holds (row index into [tokens, Hq] arrays), whether that row
// exists, and the last cache row (counted from the sequence's first) it sees.
struct MqColumn {
  long long row;
  bool valid;
  int lim;
};

// (Column n counts from the block's first row; blocks hold 2^rows_log2 rows.)
__device__ __forceinline__ MqColumn mq_column(const VSeqInfo& s, int n, int kvh, int G, int Hq, bool causal,
                                              int rows_log2 = 4) {
  const int last = s.nq * G - 1;  // the sequence's last query row
  const int r = (s.hb << rows_log2) + n;
  const int rr = r < last ? r : last;
  const int qi = rr / G;
  MqColumn c;
  c.row = (long long)(s.q0 + qi) * Hq + kvh * G + (rr - qi * G);
  c.valid = r <= last;
  c.lim = causal ? s.lk - s.nq + qi : s.lk - 1;
  return c;
}

// The runs (workers) holding tokens of sequence [cs, ce) of unit u, for a
// non-empty sequence: first .. last.
struct SeqWorkers {
  int first, last;
};

__device__ __forceinline__ SeqWorkers seq_workers(const Line& L, int u, int b, int cs, int ce, long long per) {
  const int t_last = cs + ((ce - 1 - cs) & ~(kTokenGrid - 1));
  return SeqWorkers{(int)(token_position(L, u, b, cs) / per), (int)(token_position(L, u, b, t_last) / per)};
}

// The rows of one tile of a paged cache (token i of a sequence is row
// i & (2^shift - 1) of page table_row[i >> shift]).  Tiles start on the token
// grid of their sequence and pages hold 2^shift >= 16 tokens, so tile rows
// 0-15 lie in one page and rows 16-31 in the same page or, with 16-token
// pages, in the next page of the sequence.  Tile row r < 16 is pool row
// half0 + r; tile row r >= 16 is pool row half1 + r, and so is the clamped row
// nvalid - 1 of a short tile.  The page ids are read with scalar loads (the
// table row is wave-uniform).
struct TileRows {
  long long half0, half1;
};

__device__ __forceinline__ TileRows tile_rows(const int32_t* table_row, int l0, int nvalid, int shift) {
  const int pi = l0 >> shift;
  const bool two = shift == 4 && nvalid > 16;
  const long long p0 = table_row[pi];
  const long long p1 = table_row[two ? pi + 1 : pi];
  TileRows t;
  t.half0 = (p0 << shift) + (l0 & ((1 << shift) - 1));
  t.half1 = two ? (p1 << 4) - 16 : t.half0;
  return t;
}

// Slot of part k of a sequence whose first run is wf (see the top of the file).
__device__ __forceinline__ int part_slot(int wf, int k) { return k == 0 ? 2 * wf + 1 : 2 * (wf + k); }

// Slot that run w writes for its cut segment starting at token t0 of a
// sequence whose first token is cs.
__device__ __forceinline__ int own_slot(int w, int t0, int cs) { return t0 > cs ? 2 * w : 2 * w + 1; }

// Worker id from the block id: consecutive worker ids are placed on the same
// XCD (blocks are dealt round-robin over the 8 XCDs).
__device__ __forceinline__ int worker_id(int block, int P) {
  int per_xcd = P >> 3;
  return (block & 7) * per_xcd + (block >> 3);
}

}  // namespace zl

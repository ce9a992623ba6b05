"""A CPU model of the decode kernels' work split (the contract stated at the
top of mla_attention_amd/csrc/zl_split.h), run on clamped lengths.

The model follows the stated rules, not the lane mechanics of the device
code: sequence b has L_b = clamp(cu[b+1] - cu[b], 0, max_seqlen_k) tokens
from cache row cu[b]; the work line numbers them by the prefix sums of the
L_b, with C phantom positions before each sequence; worker w owns positions
[w * per, (w + 1) * per); cuts sit on a 32-token grid from each sequence's
first token.  For every case it checks that

  * every token of every (unit, sequence) is computed by exactly one run;
  * every tile starts on the grid and holds at most 32 tokens;
  * every row read lies in [cu[b], cu[b] + L_b) of a packed cache, and every
    block-table entry read (token index // page_size) is below
    ceil(max_seqlen_k / page_size) <= max_pages_per_seq -- whatever cu holds
    (lengths above the clamp, cu decreasing, cu[0] above 0);
  * a run holds at most two cut sequences, its first and its last (the
    partial slots 2w and 2w+1), and the merge's worker range of a sequence
    (from the positions of its first and last tiles) is exactly the set of
    runs that hold its tokens.

Several new tokens per sequence: each sequence's query rows are cut into
blocks of 2^rows_log2 rows, and each block is a "virtual sequence" of all of
its (clamped) cache rows, in sequence order.
"""
import numpy as np
import pytest

GRID = 32


def clamped(cu, M):
    cu = np.asarray(cu, dtype=np.int64)
    return np.clip(np.diff(cu), 0, M)


def line_seqs_decode(cu, M):
    """(tokens, cache row of token 0, sequence) per line sequence."""
    L = clamped(cu, M)
    return [(int(L[b]), int(cu[b]), b) for b in range(len(L))]


def line_seqs_varlen(cu_q, cu_k, M, G, rows_log2):
    Lk = clamped(cu_k, M)
    nq = np.maximum(np.diff(np.asarray(cu_q, dtype=np.int64)), 0)
    out = []
    for b in range(len(Lk)):
        nblk = -(-int(nq[b]) * G // (1 << rows_log2))
        out += [(int(Lk[b]), int(cu_k[b]), b)] * nblk
    return out


def grid_cut(x, cs, ce):
    raw = min(max(x, cs), ce)
    up = cs + -(-(raw - cs) // GRID) * GRID
    return min(up, ce)


def split(seqs, C, units, P):
    """Runs of the P workers: lists of (unit, line sequence, t0, t1) in line
    order, tokens numbered on the work line."""
    lens = [s[0] for s in seqs]
    ccu = np.concatenate([[0], np.cumsum(lens, dtype=np.int64)]).astype(np.int64)
    V = len(seqs)
    T = int(ccu[-1])
    Tp = T + V * C
    N = units * Tp
    per = max(64, -(-N // P))
    cpos = [int(ccu[v]) + v * C for v in range(V)]

    def segment_at(p, p_end):
        while p < p_end:
            u, r = divmod(p, Tp)
            v = max(i for i in range(V) if cpos[i] <= r)
            cs, ce = int(ccu[v]), int(ccu[v + 1])
            base = u * Tp + (v + 1) * C
            t0 = grid_cut(p - base, cs, ce)
            t1 = grid_cut(p_end - base, cs, ce)
            if t1 > t0:
                return (base + t0, u, v, t0, t1)
            if p_end - base < ce:
                return None
            p = base + ce
        return None

    runs = []
    for w in range(P):
        p0 = w * per
        p1 = min(N, p0 + per)
        segs = []
        s = segment_at(p0, p1) if p0 < p1 else None
        while s is not None:
            segs.append(s[1:])
            s = segment_at(s[0] + (s[4] - s[3]), p1)
        runs.append(segs)
    return runs, ccu, Tp, per


def check_split(seqs, C, units, P, M, page_size=16):
    runs, ccu, Tp, per = split(seqs, C, units, P)
    V = len(seqs)
    held = {}
    max_pages = -(-M // page_size) if M > 0 else 1
    for w, segs in enumerate(runs):
        for i, (u, v, t0, t1) in enumerate(segs):
            L, row0, _ = seqs[v]
            cs, ce = int(ccu[v]), int(ccu[v + 1])
            assert cs <= t0 < t1 <= ce
            whole = t0 == cs and t1 == ce
            assert whole or i == 0 or i == len(segs) - 1, "a cut sequence inside a run"
            for k0 in range(t0, t1, GRID):
                assert (k0 - cs) % GRID == 0
                n = min(GRID, t1 - k0)
                for t in (k0, k0 + n - 1):
                    idx = t - cs                 # token index in its sequence
                    assert 0 <= idx < L <= M
                    assert cu_row_ok(row0, idx, L)
                    assert (idx // page_size) < max_pages
            for t in range(t0, t1):
                key = (u, v, t)
                assert key not in held, f"token {key} in two runs"
                held[key] = w
    for u in range(units):
        for v in range(V):
            cs, ce = int(ccu[v]), int(ccu[v + 1])
            ws = {held.get((u, v, t)) for t in range(cs, ce)}
            assert None not in ws, f"unit {u} sequence {v}: a token no run holds"
            if ce > cs:
                # the merge's worker range: positions of the first and last tiles
                first = (u * Tp + cs + (v + 1) * C) // per
                t_last = cs + ((ce - 1 - cs) // GRID) * GRID
                last = (u * Tp + t_last + (v + 1) * C) // per
                assert ws == set(range(first, last + 1)), (u, v, ws, first, last)


def cu_row_ok(row0, idx, L):
    return 0 <= row0 + idx < row0 + L


def walk(start, steps):
    cu = [start]
    for d in steps:
        cu.append(max(0, cu[-1] + d))
    return cu


DECODE = [
    # (cu, max_seqlen_k, units) -- units: key/value heads x head blocks
    ([5, 705, 745, 300, 1200, 1200, 1233], 600, 2),
    (walk(100, [((i * 97) % 420) - 60 for i in range(80)]), 256, 4),
    ([0, 300, 310, 200, 700], 128, 2),
    ([7, 7, 3, 2000], 1000, 1),
    ([3, 900, 950, 400, 1500, 1530], 700, 1),
    (walk(50, [((i * 131) % 300) - 40 for i in range(70)]), 200, 1),
    ([0, 0, 0], 10, 3),
    ([0, 5000], 4097, 8),
]


@pytest.mark.parametrize("cu,M,units", DECODE)
@pytest.mark.parametrize("P", [1, 7, 64, 512, 1024])
@pytest.mark.parametrize("C", [32, 64])
def test_decode_split_model(cu, M, units, P, C):
    check_split(line_seqs_decode(cu, M), C, units, P, M, page_size=16)
    check_split(line_seqs_decode(cu, M), C, units, P, M, page_size=256)


VARLEN = [
    # (cu_q, cu_k, max_seqlen_k, group, rows_log2)
    ([0, 3, 4, 4, 9, 9, 11], [5, 705, 745, 300, 1200, 1200, 1233], 600, 4, 4),
    ([0, 2, 9, 9, 10], [0, 300, 310, 200, 700], 128, 32, 4),
    ([0, 2, 3, 3, 7, 10], [3, 900, 950, 400, 1500, 1530], 700, 16, 5),
    ([0, 600, 640, 640, 940, 940, 973], [5, 705, 745, 300, 1200, 1200, 1233], 600, 4, 8),
    ([0, 5, 3, 8], [0, 100, 50, 400], 64, 2, 4),   # cu_q decreasing too
]


@pytest.mark.parametrize("cu_q,cu_k,M,G,rows_log2", VARLEN)
@pytest.mark.parametrize("P", [1, 13, 256, 1024])
def test_varlen_split_model(cu_q, cu_k, M, G, rows_log2, P):
    check_split(line_seqs_varlen(cu_q, cu_k, M, G, rows_log2), 32, 2, P, M, page_size=16)


def test_random_batches_split_model():
    rng = np.random.default_rng(11)
    for _ in range(40):
        B = int(rng.integers(1, 150))
        M = int(rng.integers(1, 3000))
        steps = rng.integers(-200, 2 * M, size=B)
        cu = walk(int(rng.integers(0, 100)), [int(s) for s in steps])
        P = int(rng.choice([1, 3, 64, 256, 1024, 2048]))
        check_split(line_seqs_decode(cu, M), int(rng.choice([32, 64])), int(rng.integers(1, 9)), P, M,
                    page_size=int(rng.choice([16, 32, 64, 256])))


def test_model_catches_an_unclamped_length():
    """The checks are live: without the clamp the page reads leave the
    table row."""
    cu, M = [0, 700], 600
    seqs = [(700, 0, 0)]  # the raw length
    with pytest.raises(AssertionError):
        check_split(seqs, 32, 1, 4, M, page_size=16)


# ---------------------------------------------------------------------------
# The chunked lookups of zl_split.h (seq_chunk, batch_bounds, find_seq,
# seq_bounds, vchunk) as 64-lane vector code: lane values are numpy arrays,
# a ballot is a boolean array, a lane read indexes one.  Checked against the
# plain prefix sums of the clamped lengths for batches above 64 sequences.
LANES = np.arange(64)


def lane_seq_chunk(cu, B, M, c0, carry):
    b = c0 + LANES
    s = cu[np.where(b < B, b, B)]
    e = cu[np.where(b < B, b + 1, B)]
    raw = e.astype(np.int64) - s
    ln = np.where(b < B, np.clip(raw, 0, M), 0)
    incl = carry + np.cumsum(ln)
    return {"len": ln, "excl": incl - ln, "incl": incl, "row0": s}


def lane_batch_bounds(cu, B, M):
    first = lane_seq_chunk(cu, B, M, 0, 0)
    T = int(first["incl"][63])
    for c0 in range(64, B, 64):
        T = int(lane_seq_chunk(cu, B, M, c0, T)["incl"][63])
    return first, T


def lane_find_seq(cu, B, M, C, r, first):
    ch, c0 = first, 0
    while True:
        i = c0 + LANES + 1
        m = (i < B) & (ch["incl"] + i * C <= r)
        if not m.all() or c0 + 64 >= B:
            ln = int(m.sum())
            assert np.all(m[:ln]) and not np.any(m[ln:]), "ballot is not a prefix"
            return c0 + ln, int(ch["excl"][ln]), int(ch["incl"][ln]), int(ch["row0"][ln])
        carry = int(ch["incl"][63])
        c0 += 64
        ch = lane_seq_chunk(cu, B, M, c0, carry)


def lane_seq_bounds(cu, B, M, b, first):
    ch, c0 = first, 0
    while b >= c0 + 64:
        carry = int(ch["incl"][63])
        c0 += 64
        ch = lane_seq_chunk(cu, B, M, c0, carry)
    return int(ch["excl"][b - c0]), int(ch["incl"][b - c0]), int(ch["row0"][b - c0])


@pytest.mark.parametrize("seed", range(12))
def test_lane_lookups_match_the_prefix_sums(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([1, 63, 64, 65, 80, 128, 129, 200]))
    M = int(rng.integers(1, 500))
    cu = np.asarray(walk(int(rng.integers(0, 50)), [int(s) for s in rng.integers(-100, 2 * M, size=B)]),
                    dtype=np.int64)
    C = int(rng.choice([32, 64]))
    L = clamped(cu, M)
    ccu = np.concatenate([[0], np.cumsum(L)])
    first, T = lane_batch_bounds(cu, B, M)
    assert T == ccu[-1]
    for b in range(B):
        assert lane_seq_bounds(cu, B, M, b, first) == (ccu[b], ccu[b + 1], cu[b])
    Tp = int(ccu[-1]) + B * C
    for r in sorted(set(rng.integers(0, Tp, size=300).tolist()) | {0, Tp - 1}):
        want = max(v for v in range(B) if ccu[v] + v * C <= r)
        assert lane_find_seq(cu, B, M, C, r, first) == (want, ccu[want], ccu[want + 1], cu[want])

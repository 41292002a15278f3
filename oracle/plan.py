"""Split plan: a plain reference of the cut rule, and its invariants.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FlashMLA backend page (``init_forward_metadata``, ``get_mla_metadata``
call) only fixes the shapes of the plan: a tile-scheduler table of
``[num_sm_parts, 8]`` int32 with num_sm_parts at most the multiprocessor
count (the assert in ``_apply_decode_target_verify_metadata``) and a
``num_splits`` vector of length bs+1.  The planning rule itself is not on the
pages, and several plans are correct.  What every correct plan satisfies is
checked by :func:`check_plan`; :func:`plan_reference` writes out the one rule
this library documents, so that the device planner can also be compared
exactly.

The rule.  Costs are in quarter pages.  Request b has N_b = ceil(L_b / 64)
pages and costs 4 N_b + c, c = plan_overhead(rows) (0 when N_b = 0); C is
the total cost and T = ceil(C / parts).  A position x inside request b
(cum_b <= x < cum_b + cost_b) maps to the flattened page index
pagecum_b + clamp(floor((x - cum_b - c + 2) / 4), 0, N_b): the first c units
of a request are its fixed overhead, and a position inside a page goes to
the nearer of its two boundaries.  With x_p = floor(p*C / parts), part p owns
flattened pages [G(x_p), G(x_{p+1})), so every part spans at most T cost
units, give or take half a page at each end.

Table row (8 int32): begin_req, begin_page, end_req (inclusive),
end_page (exclusive, inside end_req), piece index of the first piece inside
begin_req, number of pages, 0, 0.  An empty part has 0 pages and zeros
elsewhere.  split_indptr[b] counts the pieces before request b; a request's
pieces are the parts that touch it, in part order.
"""

from __future__ import annotations

import numpy as np

PAGE_SIZE = 64


def plan_overhead(rows_per_req: int) -> int:
    """Fixed per-piece cost in quarter pages: loading q and writing the
    result of ``rows_per_req`` rows (and the waits these cause), plus one
    page.  (A measured choice of this library: a 128-row piece costs about
    3 pages of work.)"""
    return 4 + (8 * rows_per_req + 127) // 128


def _locate(g: int, pagecum: np.ndarray, npages: np.ndarray):
    """Flattened page index g -> (request, page) for a page that exists."""
    b = int(np.searchsorted(pagecum, g, side="right") - 1)
    while npages[b] == 0 or g >= pagecum[b] + npages[b]:
        b += 1
    return b, g - int(pagecum[b])


def plan_reference(seq_lens, num_parts: int, rows_per_req: int):
    L = np.asarray(seq_lens, dtype=np.int64)
    bs = len(L)
    c = plan_overhead(rows_per_req)
    npages = -(-L // PAGE_SIZE)
    cost = np.where(npages > 0, 4 * npages + c, 0)
    cum = np.concatenate([[0], np.cumsum(cost)])
    pagecum = np.concatenate([[0], np.cumsum(npages)])
    C = int(cum[-1])
    T = max(1, -(-C // num_parts))

    def G(x: int) -> int:
        if x >= C:
            return int(pagecum[-1])
        b = int(np.searchsorted(cum, x, side="right") - 1)
        o = x - int(cum[b])
        return int(pagecum[b]) + int(min(max(o - c + 2, 0) // 4, npages[b]))

    cuts = [G(p * C // num_parts) for p in range(num_parts + 1)]
    cuts[num_parts] = int(pagecum[-1])

    # interior cut positions, distinct, per request
    interior = set()
    for g in cuts[1:num_parts]:
        if 0 < g < pagecum[-1]:
            b, pg = _locate(g, pagecum, npages)
            if pg > 0:
                interior.add(g)
    pieces = np.zeros(bs, dtype=np.int64)
    for b in range(bs):
        if npages[b] == 0:
            continue
        lo, hi = int(pagecum[b]), int(pagecum[b] + npages[b])
        pieces[b] = 1 + sum(1 for g in interior if lo < g < hi)
    indptr = np.concatenate([[0], np.cumsum(pieces)]).astype(np.int32)

    table = np.zeros((num_parts, 8), dtype=np.int32)
    for p in range(num_parts):
        g0, g1 = cuts[p], cuts[p + 1]
        if g1 <= g0:
            continue
        b0, pg0 = _locate(g0, pagecum, npages)
        b1, pg1 = _locate(g1 - 1, pagecum, npages)
        first_idx = sum(1 for g in interior if pagecum[b0] < g <= g0)
        table[p] = [b0, pg0, b1, pg1 + 1, first_idx, g1 - g0, 0, 0]
    return table, indptr


def check_plan(table, indptr, seq_lens, num_parts: int, rows_per_req: int) -> None:
    """Raise AssertionError unless (table, indptr) is a correct plan:

    * shapes [num_parts, 8] and [bs+1]; indptr[0] = 0, non-decreasing,
      indptr[bs] <= bs + num_parts;
    * every page of every request lies in exactly one part, parts are
      page-aligned ranges of the (request, page) sequence in order;
    * request b has indptr[b+1]-indptr[b] pieces, one per part touching it,
      numbered 0.. in part order (the first one given by field 4);
    * each part costs (4 per page plus c per piece, in quarter pages) at most
      ceil(total cost / num_parts) + c + 4.
    """
    table = np.asarray(table)
    indptr = np.asarray(indptr, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    bs = len(L)
    c = plan_overhead(rows_per_req)
    assert table.shape == (num_parts, 8), table.shape
    assert indptr.shape == (bs + 1,), indptr.shape
    assert indptr[0] == 0
    assert np.all(np.diff(indptr) >= 0)
    assert indptr[-1] <= bs + num_parts
    npages = -(-L // PAGE_SIZE)
    C = int(np.where(npages > 0, 4 * npages + c, 0).sum())
    T = max(1, -(-C // num_parts))

    seen = [np.zeros(int(n), dtype=np.int64) for n in npages]
    pieces_seen = [[] for _ in range(bs)]
    last = (0, 0)  # next (request, page) expected, in order
    for p in range(num_parts):
        b0, pg0, b1, pg1, first_idx, npg, r0, r1 = [int(v) for v in table[p]]
        assert r0 == 0 and r1 == 0
        if npg == 0:
            assert (b0, pg0, b1, pg1, first_idx) == (0, 0, 0, 0, 0), table[p]
            continue
        assert 0 <= b0 <= b1 < bs, table[p]
        assert (b0, pg0) >= last, f"part {p} out of order"
        count = 0
        cost = 0
        for b in range(b0, b1 + 1):
            lo = pg0 if b == b0 else 0
            hi = pg1 if b == b1 else int(npages[b])
            assert 0 <= lo <= hi <= npages[b], table[p]
            if hi == lo:
                continue
            seen[b][lo:hi] += 1
            idx = first_idx if b == b0 else 0
            pieces_seen[b].append((p, idx, lo, hi))
            count += hi - lo
            cost += 4 * (hi - lo) + c
        assert count == npg, table[p]
        assert cost <= T + c + 4, f"part {p} cost {cost} > {T} + {c} + 4"
        last = (b1, pg1)
    for b in range(bs):
        assert np.all(seen[b] == 1), f"request {b} pages not covered exactly once"
        k = int(indptr[b + 1] - indptr[b])
        assert k == len(pieces_seen[b]), f"request {b}: {k} pieces declared, {len(pieces_seen[b])} found"
        for j, (_, idx, _, _) in enumerate(pieces_seen[b]):
            assert idx == j, f"request {b}: piece numbering"


# ------------------------------------------------------------ fixed-size tiles

def plan_fixed(seq_lens, tile_pages: int, max_parts: int):
    """Deterministic plan with fixed-size tiles (the FlashInfer backend page's
    deterministic mode: with enable_deterministic the decode KV is split into
    tiles of decode_split_tile_size = 2048 tokens, and graph-mode KV splitting
    is switched off).  Every request is cut at the multiples of ``tile_pages``
    pages of its own sequence, so where it is cut does not depend on the rest
    of the batch.

    Request b has N_b = ceil(L_b / 64) pages and n_b = ceil(N_b / tile_pages)
    pieces; split_indptr is the running sum of n_b.  Piece k of request b is
    part split_indptr[b] + k, row (b, k*T, b, min((k+1)*T, N_b), k, pages, 0, 0),
    T = tile_pages.  Rows from split_indptr[bs] to max_parts - 1 are zeros.
    If the pieces do not fit in max_parts, nothing is planned: every row and
    every split_indptr entry is 0 (so each request then has no piece).
    """
    L = np.asarray(seq_lens, dtype=np.int64)
    bs = len(L)
    T = int(tile_pages)
    npages = -(-L // PAGE_SIZE)
    pieces = -(-npages // T)
    indptr = np.zeros(bs + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(pieces)
    table = np.zeros((max_parts, 8), dtype=np.int32)
    if indptr[-1] > max_parts:
        return table, np.zeros(bs + 1, dtype=np.int32)
    for b in range(bs):
        for k in range(int(pieces[b])):
            pg0, pg1 = k * T, min((k + 1) * T, int(npages[b]))
            table[indptr[b] + k] = (b, pg0, b, pg1, k, pg1 - pg0, 0, 0)
    return table, indptr.astype(np.int32)


def check_fixed_plan(table, indptr, seq_lens, tile_pages: int) -> None:
    """Raise AssertionError unless (table, indptr) covers every page of every
    request exactly once, in order, by pieces that each lie inside one request,
    start at a multiple of ``tile_pages`` pages and hold at most that many."""
    table = np.asarray(table)
    indptr = np.asarray(indptr, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    npages = -(-L // PAGE_SIZE)
    assert indptr[0] == 0 and np.all(np.diff(indptr) >= 0)
    for b in range(len(L)):
        covered = 0
        for k in range(int(indptr[b]), int(indptr[b + 1])):
            b0, pg0, b1, pg1, idx, npg, r0, r1 = [int(v) for v in table[k]]
            assert b0 == b1 == b and idx == k - indptr[b] and r0 == r1 == 0
            assert pg0 == covered and pg0 % tile_pages == 0
            assert 0 < npg == pg1 - pg0 <= tile_pages
            covered = pg1
        assert covered == npages[b]
    assert not np.any(table[int(indptr[-1]):])


# ------------------------------------------------------------ packed fixed-size tiles

def plan_fixed_packed(seq_lens, tile_pages: int, num_parts: int, rows_per_req: int):
    """The fixed-size tiles of :func:`plan_fixed` (the same pieces, the same
    split_indptr), packed into ``num_parts`` contiguous parts of about equal
    cost, so that a batch whose tiles outnumber or undercut the CUs keeps
    every CU busy.  A tile stays a piece of its own wherever it lands, so a
    request still decodes bit for bit the same in any batch.

    The rule, in quarter pages: tile t (in request order, then tile order)
    costs 4 n_t + c, n_t its pages, c = plan_overhead(rows_per_req); Q_t is
    the cost of the tiles before t (Q_0 = 0, Q_NT = C).  With
    x_p = floor(p C / num_parts), cut p is the tile boundary t whose Q_t is
    nearest x_p (the lower one on a tie); part p holds tiles [cut_p, cut_p+1).

    Table row: (first request, its first page, last request, end page in the
    last request, piece index of the first tile in its request, pages,
    tile_pages, 0); an empty part is all zeros.  Field 6 tells the decode to
    end a piece at every multiple of tile_pages pages of a request.
    """
    L = np.asarray(seq_lens, dtype=np.int64)
    bs = len(L)
    T = int(tile_pages)
    c = plan_overhead(rows_per_req)
    npages = -(-L // PAGE_SIZE)
    tiles = []  # (request, tile index, first page, end page)
    for b in range(bs):
        n = int(npages[b])
        for k in range(-(-n // T)):
            tiles.append((b, k, k * T, min((k + 1) * T, n)))
    pieces = np.array([-(-int(n) // T) for n in npages], dtype=np.int64)
    indptr = np.concatenate([[0], np.cumsum(pieces)]).astype(np.int32)
    Q = [0]
    for (_, _, pg0, pg1) in tiles:
        Q.append(Q[-1] + 4 * (pg1 - pg0) + c)
    C = Q[-1]
    NT = len(tiles)

    def nearest(x: int) -> int:
        best = 0
        for t in range(NT + 1):
            if abs(Q[t] - x) < abs(Q[best] - x):
                best = t
        return best

    cuts = [nearest(p * C // num_parts) for p in range(num_parts)] + [NT]
    cuts[0] = 0
    table = np.zeros((num_parts, 8), dtype=np.int32)
    for p in range(num_parts):
        t0, t1 = cuts[p], cuts[p + 1]
        if t1 <= t0:
            continue
        b0, k0, pg0, _ = tiles[t0]
        b1, _, _, pg1 = tiles[t1 - 1]
        pages = sum(e - s for (_, _, s, e) in tiles[t0:t1])
        table[p] = (b0, pg0, b1, pg1, k0, pages, T, 0)
    return table, indptr


def check_fixed_packed_plan(table, indptr, seq_lens, tile_pages: int, num_parts: int,
                            rows_per_req: int) -> None:
    """Raise AssertionError unless (table, indptr) is a packed fixed-tile plan:
    split_indptr is that of :func:`plan_fixed` (one piece per tile); the parts
    cover the (request, page) sequence in order, each page exactly once, and
    start and end on tile boundaries; field 4 is the first tile's index in
    its request, field 6 the tile size; and every part costs at most
    ceil(C / num_parts) plus one tile's cost (4 tile_pages + c)."""
    table = np.asarray(table)
    indptr = np.asarray(indptr, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    T = int(tile_pages)
    c = plan_overhead(rows_per_req)
    npages = -(-L // PAGE_SIZE)
    _, ref_indptr = plan_fixed(L, T, 1 << 30)
    assert np.array_equal(indptr, ref_indptr)
    assert table.shape == (num_parts, 8)
    C = int(sum(4 * int(n) + c * (-(-int(n) // T)) for n in npages))
    bound = -(-C // num_parts) + 4 * T + c
    seen = [np.zeros(int(n), dtype=np.int64) for n in npages]
    last = (0, 0)
    for p in range(num_parts):
        b0, pg0, b1, pg1, k0, npg, tc, r1 = [int(v) for v in table[p]]
        if npg == 0:
            assert not np.any(table[p]), table[p]
            continue
        assert tc == T and r1 == 0 and 0 <= b0 <= b1 < len(L), table[p]
        assert (b0, pg0) >= last, f"part {p} out of order"
        assert pg0 % T == 0 and k0 == pg0 // T, table[p]
        assert pg1 == npages[b1] or pg1 % T == 0, table[p]
        count = cost = 0
        for b in range(b0, b1 + 1):
            lo = pg0 if b == b0 else 0
            hi = pg1 if b == b1 else int(npages[b])
            assert 0 <= lo <= hi <= npages[b], table[p]
            seen[b][lo:hi] += 1
            count += hi - lo
            cost += 4 * (hi - lo) + c * len(range(lo // T, -(-hi // T))) if hi > lo else 0
        assert count == npg, table[p]
        assert cost <= bound, f"part {p} cost {cost} > {bound}"
        last = (b1, pg1)
    for b in range(len(L)):
        assert np.all(seen[b] == 1), f"request {b} pages not covered exactly once"

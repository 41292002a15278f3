"""The plan reference satisfies the plan invariants, and the invariant
checker catches broken plans (CPU only)."""

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, workload_seq_lens


@pytest.mark.parametrize("name", sorted(CONFIGS))
@pytest.mark.parametrize("parts", [1, 7, 64, 256])
def test_reference_plan_is_valid_on_named_workloads(name, parts):
    lens = workload_seq_lens(name)
    rows = CONFIGS[name]["heads"] * CONFIGS[name]["q_len"]
    t, ip = oracle.plan_reference(lens, parts, rows)
    oracle.check_plan(t, ip, lens, parts, rows)


@pytest.mark.parametrize("lens,parts", [
    ([1], 1), ([1], 256), ([64] * 300, 256), ([65, 1, 64, 2000], 3),
    ([0, 5, 0, 700], 4), ([0, 0], 8), ([8192], 256), ([129, 129, 129], 1000),
])
@pytest.mark.parametrize("rows", [16, 128, 512])
def test_reference_plan_edge_shapes(lens, parts, rows):
    t, ip = oracle.plan_reference(lens, parts, rows)
    oracle.check_plan(t, ip, lens, parts, rows)
    assert ip[-1] <= len(lens) + parts


def test_plan_splits_long_requests_across_parts():
    lens = workload_seq_lens("long")
    t, ip = oracle.plan_reference(lens, 256, 128)
    pieces = np.diff(ip)
    assert pieces.min() >= 20           # ~32 pieces each at 256 parts
    assert (t[:, 5] > 0).sum() == 256   # every part has work


def _broken(t, ip, what):
    t = t.copy()
    ip = ip.copy()
    if what == "drop_page":
        p = int(np.nonzero(t[:, 5] > 1)[0][0])
        t[p, 3] -= 1
        t[p, 5] -= 1
    elif what == "overlap":
        p = int(np.nonzero(t[:, 5] > 0)[0][1])
        t[p, 1] -= 1
        t[p, 5] += 1
    elif what == "pieces":
        ip[1:] += 1
    elif what == "numbering":
        p = int(np.nonzero(t[:, 4] > 0)[0][0])
        t[p, 4] += 1
    elif what == "imbalance":
        # move every page of part 1 into part 0
        t[0, 2], t[0, 3] = t[1, 2], t[1, 3]
        t[0, 5] += t[1, 5]
        t[1] = 0
    return t, ip


@pytest.mark.parametrize("what", ["drop_page", "overlap", "pieces", "numbering", "imbalance"])
def test_check_plan_rejects_broken_plans(what):
    lens = workload_seq_lens("dsv3")
    t, ip = oracle.plan_reference(lens, 256, 128)
    oracle.check_plan(t, ip, lens, 256, 128)
    bt, bip = _broken(t, ip, what)
    with pytest.raises(AssertionError):
        oracle.check_plan(bt, bip, lens, 256, 128)


# ------------------------------------------------------------ fixed-size tiles

def _pieces_by_page(lens, T):
    """Brute force: page p of request b belongs to piece p // T of b."""
    out = []
    for b, L in enumerate(lens):
        n = -(-int(L) // 64)
        pieces = {}
        for p in range(n):
            pieces.setdefault(p // T, []).append(p)
        out.append([(b, pg[0], pg[-1] + 1) for _, pg in sorted(pieces.items())])
    return out


@pytest.mark.parametrize("lens", [[1], [0], [64 * 32], [64 * 32 + 1], [37, 130], [0, 5, 0, 700],
                                  [2048, 2049, 4095, 4096, 4097, 1]])
@pytest.mark.parametrize("T", [1, 4, 32])
def test_fixed_plan_matches_page_enumeration(lens, T):
    bf = _pieces_by_page(lens, T)
    need = sum(len(x) for x in bf)
    t, ip = oracle.plan_fixed(lens, T, max(need, 1) + 3)
    oracle.check_fixed_plan(t, ip, lens, T)
    got = [[(int(r[0]), int(r[1]), int(r[3])) for r in t[ip[b]:ip[b + 1]]] for b in range(len(lens))]
    assert got == bf


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_fixed_plan_on_named_workloads_and_batch_invariance(name):
    lens = workload_seq_lens(name)
    T = 32                                  # 2048 tokens, the page's default tile
    need = int(sum(-(-(-(-int(L) // 64)) // T) for L in lens))
    t, ip = oracle.plan_fixed(lens, T, need)
    oracle.check_fixed_plan(t, ip, lens, T)
    # A request's pieces do not depend on the rest of the batch: plan request 1
    # alone, and inside a reversed batch, and compare its rows (request field aside).
    b = min(1, len(lens) - 1)
    cols = [1, 3, 4, 5, 6, 7]                # every field but the request index
    mine = t[ip[b]:ip[b + 1]][:, cols]
    t1, ip1 = oracle.plan_fixed(lens[b:b + 1], T, need)
    assert np.array_equal(mine, t1[ip1[0]:ip1[1]][:, cols])
    rb = len(lens) - 1 - b
    t2, ip2 = oracle.plan_fixed(lens[::-1], T, need)
    assert np.array_equal(mine, t2[ip2[rb]:ip2[rb + 1]][:, cols])


def test_fixed_plan_overflow_plans_nothing_and_checker_catches_mutations():
    lens = [4096, 100, 70000]
    t, ip = oracle.plan_fixed(lens, 4, 5)           # needs 16 + 1 + 274 pieces
    assert not t.any() and not ip.any()
    t, ip = oracle.plan_fixed(lens, 4, 400)
    oracle.check_fixed_plan(t, ip, lens, 4)
    for mutate in (lambda a: a.__setitem__((0, 3), a[0, 3] + 1),     # overlaps piece 1
                   lambda a: a.__setitem__((1, 1), a[1, 1] + 1),     # gap, off the grid
                   lambda a: a.__setitem__((0, 4), 3),               # wrong piece index
                   lambda a: a.__setitem__((300, 5), 1)):            # junk past the end
        bad = t.copy()
        mutate(bad)
        with pytest.raises(AssertionError):
            oracle.check_fixed_plan(bad, ip, lens, 4)


# ------------------------------------------------------------ packed fixed tiles

def test_fixed_packed_plan_worked_example():
    """Hand-worked case.  L = [130, 64, 300, 4000], T = 8, 128 rows (c = 12
    quarter pages), 5 parts.  Pages 3, 1, 5, 63; tiles: one each for the first
    three requests (costs 24, 16, 32), eight for the last (seven of 8 pages,
    cost 44 each, and one of 7, cost 40).  Boundaries Q = 0, 24, 40, 72, 116,
    160, 204, 248, 292, 336, 380, 420 (C = 420); positions x_p = 0, 84, 168,
    252, 336 pick boundaries 72 (t = 3), 160 (t = 5), 248 (t = 7), 336 (t = 9)."""
    t, ip = oracle.plan_fixed_packed([130, 64, 300, 4000], 8, 5, 128)
    assert ip.tolist() == [0, 1, 2, 3, 11]
    assert t.tolist() == [[0, 0, 2, 5, 0, 9, 8, 0],
                          [3, 0, 3, 16, 0, 16, 8, 0],
                          [3, 16, 3, 32, 2, 16, 8, 0],
                          [3, 32, 3, 48, 4, 16, 8, 0],
                          [3, 48, 3, 63, 6, 15, 8, 0]]


def test_fixed_packed_plan_tie_goes_to_the_lower_boundary():
    """Two requests of one 1-page tile each, 32 rows (c = 6 quarter pages):
    each tile costs 10, Q = 0, 10, 20, C = 20.  With 4 parts the positions
    5 and 15 sit exactly between two boundaries and take the lower one (0 and
    10), so parts 0 and 2 stay empty."""
    assert oracle.plan_overhead(32) == 6
    t, ip = oracle.plan_fixed_packed([10, 20], 4, 4, 32)
    assert ip.tolist() == [0, 1, 2]
    assert t.tolist() == [[0] * 8, [0, 0, 0, 1, 0, 1, 4, 0], [0] * 8, [1, 0, 1, 1, 0, 1, 4, 0]]


@pytest.mark.parametrize("seed", range(6))
def test_fixed_packed_plan_random_batches_are_valid(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        bs = int(rng.integers(1, 60))
        L = rng.integers(0, 9000, size=bs)
        L[rng.random(bs) < 0.2] = 0
        T = int(rng.integers(1, 48))
        P = int(rng.integers(1, 300))
        R = int(rng.choice([1, 16, 64, 128, 512]))
        t, ip = oracle.plan_fixed_packed(L, T, P, R)
        oracle.check_fixed_packed_plan(t, ip, L, T, P, R)


def test_fixed_packed_plan_keeps_the_fixed_plan_pieces():
    """Packing changes which part holds a tile, never the tiles: with one
    part per tile and equal tile costs every part holds one tile, in the
    fixed plan's order, and the tiles of a request do not depend on the rest
    of the batch."""
    L = np.full(10, 64 * 8, dtype=np.int64)          # every request: two 4-page tiles
    t, ip = oracle.plan_fixed_packed(L, 4, 20, 128)
    tf, ipf = oracle.plan_fixed(L, 4, 20)
    assert np.array_equal(ip, ipf)
    assert np.array_equal(t[:, :6], tf[:, :6]) and np.all(t[:, 6] == 4)
    for name in ("dsv3", "verify"):
        lens = workload_seq_lens(name)
        t, ip = oracle.plan_fixed_packed(lens, 16, 256, CONFIGS[name]["heads"] * CONFIGS[name]["q_len"])
        sub = lens[5:9]
        t2, ip2 = oracle.plan_fixed_packed(sub, 16, 3, 128)
        assert np.array_equal(np.diff(ip)[5:9], np.diff(ip2))


@pytest.mark.parametrize("what", ["drop", "overlap", "tile", "field6", "order", "cost"])
def test_check_fixed_packed_plan_rejects_broken_plans(what):
    L = [130, 64, 300, 4000]
    t, ip = oracle.plan_fixed_packed(L, 8, 5, 128)
    t = t.copy()
    if what == "drop":
        t[4, 3] = 60; t[4, 5] = 12          # lose the last 3 pages
    elif what == "overlap":
        t[2, 1] = 8; t[2, 4] = 1; t[2, 5] = 24
    elif what == "tile":
        t[2, 4] = 1                          # wrong tile index for page 16
    elif what == "field6":
        t[1, 6] = 4
    elif what == "order":
        t[[1, 2]] = t[[2, 1]]
    elif what == "cost":
        # part 0 takes everything up to page 40 of the last request (292 > 128)
        t[0] = [0, 0, 3, 40, 0, 49, 8, 0]; t[1] = 0; t[2] = 0; t[3] = [3, 40, 3, 48, 5, 8, 8, 0]
    with pytest.raises(AssertionError):
        oracle.check_fixed_packed_plan(t, ip, L, 8, 5, 128)

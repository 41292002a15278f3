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

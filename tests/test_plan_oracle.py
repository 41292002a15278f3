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

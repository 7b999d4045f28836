"""Hand-worked pins of the oracle's window-search decision rule (Compact
Attention page, Fig. 3 caption: windows shrunk step by step under a recall
constraint tau and a cost constraint lambda; Fig. 4 caption: starting from
full coverage in every temporal-distance group).

tests/golden/search_cases.json holds small cases (at most 2 x 2 x 2 tiles)
whose expected windows, recall and cost were derived by hand, step by step,
from the rule as read (least lost weight per saved cost; ties to the larger
saving, then the lower group, then the lower move; admissible when recall
stays >= tau and lost recall <= lambda x saved cost fraction).  The second
half plants plausible mistakes in the oracle (a flipped ratio comparison,
the wrong tie-breaks, a reversed lambda inequality) and checks that each one
fails at least one hand-worked case."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import search

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "search_cases.json")) as f:
    CASES = json.load(f)["cases"]


def _mass(case):
    """A[i, j] = n[|dt|][|dy|][|dx|] / den over the case's tile grid."""
    a, b, e, _ = search._tile_coords(case["grid"], case["tile"])
    n = np.asarray(case["n"], dtype=np.float64)
    da = np.abs(a[:, None] - a[None, :])
    dy = np.abs(b[:, None] - b[None, :])
    dx = np.abs(e[:, None] - e[None, :])
    return (n[da, dy, dx] / case["den"])[None]


def _run(case):
    lam = math.inf if case["lam"] == "inf" else float(case["lam"])
    counts = oracle.tile_counts(case["grid"], case["tile"])
    groups = [[tuple(g) for g in case["groups"]]]
    return search.search(case["grid"], case["tile"], counts, _mass(case), groups, case["tau"], lam)


def _matches(case):
    rows, _, rec, cost = _run(case)
    return (rows.tolist() == case["expected_rows"] and rec[0] == case["expected_recall"]
            and cost[0] == case["expected_cost"])


def test_cases_have_full_tiles_and_unit_mass_rows():
    for case in CASES:
        assert np.all(oracle.tile_counts(case["grid"], case["tile"]) == 16)
        assert np.allclose(_mass(case)[0].sum(axis=1), 1.0)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_worked_case(case):
    rows, gph, rec, cost = _run(case)
    assert rows.tolist() == case["expected_rows"]
    assert gph.tolist() == [len(case["groups"])]
    assert rec[0] == case["expected_recall"]
    assert cost[0] == case["expected_cost"]


# ---- planted mistakes: each must fail at least one hand-worked case ----

def _flipped_ratio(c1, c2):
    w1, k1, g1, m1 = c1
    w2, k2, g2, m2 = c2
    if k1 and k2 and w1 * k2 != w2 * k1:
        return w1 * k2 > w2 * k1
    if k1 != k2:
        return k1 > k2
    return (g1, m1) < (g2, m2)


def _least_weight(c1, c2):
    w1, k1, g1, m1 = c1
    w2, k2, g2, m2 = c2
    return (w1, g1, m1) < (w2, g2, m2)


def _smaller_saving(c1, c2):
    w1, k1, g1, m1 = c1
    w2, k2, g2, m2 = c2
    if k1 and k2 and w1 * k2 != w2 * k1:
        return w1 * k2 < w2 * k1
    if k1 != k2:
        return k1 < k2
    return (g1, m1) < (g2, m2)


def _higher_group(c1, c2):
    w1, k1, g1, m1 = c1
    w2, k2, g2, m2 = c2
    if k1 and k2 and w1 * k2 != w2 * k1:
        return w1 * k2 < w2 * k1
    if k1 != k2:
        return k1 > k2
    return (-g1, m1) < (-g2, m2)


def _higher_move(c1, c2):
    w1, k1, g1, m1 = c1
    w2, k2, g2, m2 = c2
    if k1 and k2 and w1 * k2 != w2 * k1:
        return w1 * k2 < w2 * k1
    if k1 != k2:
        return k1 > k2
    return (g1, -m1) < (g2, -m2)


def _reversed_lambda(dw, dc, w_total, c_total, lam):
    if math.isinf(lam):
        return True
    return float(dw) * float(c_total) >= lam * float(dc) * float(w_total)


@pytest.mark.parametrize("name,attr,fn", [
    ("flipped ratio comparison", "_ranks_before", _flipped_ratio),
    ("least lost weight instead of least ratio", "_ranks_before", _least_weight),
    ("smaller saving wins a ratio tie", "_ranks_before", _smaller_saving),
    ("higher group wins a tie", "_ranks_before", _higher_group),
    ("higher move wins a tie", "_ranks_before", _higher_move),
    ("reversed lambda inequality", "_within_cost_bound", _reversed_lambda),
])
def test_planted_mistake_fails_a_case(monkeypatch, name, attr, fn):
    monkeypatch.setattr(search, attr, fn)
    failing = [c["name"] for c in CASES if not _matches(c)]
    assert failing, f"planted mistake '{name}' passes every hand-worked case"

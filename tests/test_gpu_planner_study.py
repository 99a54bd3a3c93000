"""The planner study (No balance / Zigzag / LPT on §5.5's workloads) on the GPU:
its imbalance figures equal the oracle's on the same seeded draws, and the
study runs end to end."""
import numpy as np
import pytest

import oracle
from block_sparse_cross_amd import inputs as I
from block_sparse_cross_amd import planner_study as ps

pytestmark = pytest.mark.gpu


def oracle_imbalances(L, P, J, seed):
    w = ps.workload(L, P, J)
    s, a = I.workload_anchors(w, seed)
    prof = oracle.anchor_profile(s, a, w.B, w.S)
    st, ln = I.sample_bounds(w)
    out = {}
    for k, strategy in (("no_balance", 0), ("zigzag", 1)):
        _, load = oracle.baseline_plan(strategy, st, ln, prof, P)
        out[k] = 100.0 * (oracle.imbalance(load, w.N, w.B) - 1.0)
    _, _, bundles, load = oracle.plan(s, a, w.B, w.S, w.m, P, J)
    out["lpt"] = 100.0 * (oracle.imbalance(load, w.N, w.B) - 1.0)
    _, _, _, moved = oracle.locality_match(bundles, w.m)
    out["moved_matched"] = 100.0 * moved / w.S
    return out


@pytest.mark.parametrize("L,P,J", [(16384, 8, 8), (262144, 64, 8), (262144, 8, 1)])
def test_case_matches_oracle(L, P, J):
    got = ps.run_case(L, P, J, seed=1, reps=2)
    want = oracle_imbalances(L, P, J, seed=1)
    for k in ("no_balance", "zigzag", "lpt"):
        assert got[k] == pytest.approx(want[k], rel=1e-12, abs=1e-12), k
        assert got[k + "_us"] > 0
    assert got["moved_matched"] == pytest.approx(want["moved_matched"], rel=1e-12, abs=1e-12)
    assert got["moved_matched"] <= got["moved_plan_order"] and got["match_us"] > 0


def test_study_runs_and_orders_the_rules():
    res = ps.study(seeds=1, reps=1)
    s = res["summary"]
    for group in ("context", "cp"):
        assert s[group + "_lpt"][0] < s[group + "_zigzag"][0] < s[group + "_no_balance"][0]
    md = ps.to_markdown(res)
    assert md.count("\n| j_sweep |") == 2 * 2 * len(ps.J_SWEEP)   # imbalance and all-to-all tables

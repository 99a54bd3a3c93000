"""Pins for the oracle's planner half (load profile, chunk costs, LPT, Zigzag).

Each check ties the oracle to something other than itself: values printed in
the paper's Figures 3 and 5 (tests/golden/figures.json), closed forms (Eq. 1),
conservation of work, brute force over positions, and an independent
literal-rescan greedy written here.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from block_sparse_cross_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "figures.json")))


def fig5_anchors():
    f = GOLD["fig5"]
    s, a = [], []
    for smp in f["samples"]:
        for x in smp["anchors_local"]:
            s.append(smp["start"])
            a.append(smp["start"] + x)
    return np.array(s), np.array(a)


# ----------------------------------------------------------- worked examples
def test_fig3_profile():
    f = GOLD["fig3"]
    prof = oracle.anchor_profile(np.zeros(4, np.int64), f["anchors"], f["B"], f["L"])
    assert prof.tolist() == f["profile"]


def test_fig3_causal_profile_eq1_and_mirror():
    # Eq. 1: causal self-attention is the special case B=1 with one block per
    # position x whose window is [0, x+1): c_self(x) = L - x.
    L = GOLD["fig3"]["L"]
    prof = oracle.anchor_profile(np.zeros(L, np.int64), np.arange(1, L + 1), 1, L)
    assert prof.tolist() == [L - x for x in range(L)]
    mirror = prof + prof[::-1]
    assert (mirror == GOLD["fig3"]["causal_mirror_sum"]).all()


def test_fig5_profiles():
    f = GOLD["fig5"]
    s, a = fig5_anchors()
    prof = oracle.anchor_profile(s, a, f["B"], 24)
    assert prof[:16].tolist() == f["profile_sample0"]
    assert prof[16:].tolist() == f["profile_sample1"]


def test_fig5_chunk_costs_both_forms():
    f = GOLD["fig5"]
    s, a = fig5_anchors()
    for form in ("direct", "prefix"):
        c = oracle.chunk_costs(s, a, f["B"], 12, f["m"], form=form)
        assert c.tolist() == f["lpt_chunk_costs"], form


def test_fig5_lpt_loads_and_rho():
    f = GOLD["fig5"]
    s, a = fig5_anchors()
    cost, owner, bundles, load = oracle.plan(s, a, f["B"], 24, f["m"], f["P"], f["J"])
    assert load.tolist() == f["lpt_loads"]
    assert (load + f["D"]).tolist() == f["lpt_W"]
    assert round(oracle.imbalance(load, len(s), f["B"]), 3) == f["lpt_rho"]
    assert sorted(bundles.reshape(-1).tolist()) == list(range(12))
    for p in range(f["P"]):
        assert list(bundles[p]) == sorted(bundles[p])
        assert all(owner[j] == p for j in bundles[p])


def test_fig5_zigzag():
    f = GOLD["fig5"]
    s, a = fig5_anchors()
    prof = oracle.anchor_profile(s, a, f["B"], 24)
    # per-sample Zigzag chunk costs as printed in Figure 5(b)
    z0 = [int(prof[2 * t:2 * t + 2].sum()) for t in range(8)]
    z1 = [int(prof[16 + t]) for t in range(8)]
    assert z0 == f["zigzag_chunk_costs_sample0"]
    assert z1 == f["zigzag_chunk_costs_sample1"]
    load = oracle.zigzag_loads([0, 16], [16, 8], prof, f["P"])
    assert load.tolist() == f["zigzag_loads"]
    assert (load + f["D"]).tolist() == f["zigzag_W"]
    assert round(oracle.imbalance(load, len(s), f["B"]), 3) == f["zigzag_rho"]


# ------------------------------------------------------------- invariants
def _random_case(seed):
    g = np.random.default_rng(seed)
    n_samples = int(g.integers(1, 4))
    P = int(g.integers(1, 9))
    J = int(g.integers(1, 5))
    m = int(g.integers(1, 7))
    S = P * J * m
    # samples partition [0, S) (last sample takes the rest)
    cuts = sorted(set(g.integers(1, S, size=n_samples - 1).tolist())) if S > 1 else []
    bounds = [0] + cuts + [S]
    s, a = [], []
    B = int(g.integers(1, 17))
    for u in range(len(bounds) - 1):
        st, en = bounds[u], bounds[u + 1]
        n_anchor = int(g.integers(0, min(6, en - st) + 1))
        if n_anchor:
            pos = np.sort(g.choice(en - st, size=n_anchor, replace=False)) + st
            for x in pos:
                s.append(st)
                a.append(int(x))
    return np.array(s, np.int64), np.array(a, np.int64), B, S, m, P, J


@pytest.mark.parametrize("seed", range(200))
def test_costs_conservation_and_bruteforce(seed):
    s, a, B, S, m, P, J = _random_case(seed)
    c = oracle.chunk_costs(s, a, B, S // m, m)
    c2 = oracle.chunk_costs(s, a, B, S // m, m, form="prefix")
    assert (c == c2).all()
    assert c.sum() == B * int((a - s).sum())           # sum_j c_j = B sum_i (a_i - s_i)
    prof = oracle.anchor_profile(s, a, B, S)
    # brute force: cost of a chunk is the profile summed over its positions
    brute = np.array([sum(B for i in range(len(s)) for x in range(j * m, (j + 1) * m)
                          if s[i] <= x < a[i]) for j in range(S // m)], dtype=np.int64)
    assert (c == brute).all()
    assert (c == prof.reshape(-1, m).sum(axis=1)).all()


def _greedy_literal(cost, P, J):
    """Literal reading of the LPT rule, written independently of the oracle:
    rescan everything at every step."""
    remaining = list(range(len(cost)))
    load = [0] * P
    held = [[] for _ in range(P)]
    owner = [-1] * len(cost)
    while remaining:
        best_c = max(cost[j] for j in remaining)
        j = min(x for x in remaining if cost[x] == best_c)
        remaining.remove(j)
        open_ranks = [p for p in range(P) if len(held[p]) < J]
        low = min(load[p] for p in open_ranks)
        p = min(q for q in open_ranks if load[q] == low)
        held[p].append(j)
        load[p] += cost[j]
        owner[j] = p
    return owner, [sorted(h) for h in held], load


@pytest.mark.parametrize("seed", range(1000))
def test_lpt_matches_literal_greedy(seed):
    g = np.random.default_rng(10_000 + seed)
    P = int(g.integers(1, 9))
    J = int(g.integers(1, 5))
    # few distinct values so that ties are frequent
    cost = g.integers(0, 6, size=P * J).astype(np.int64) * int(g.integers(1, 100))
    owner, bundles, load = oracle.lpt(cost, P, J)
    o2, b2, l2 = _greedy_literal(cost.tolist(), P, J)
    assert owner.tolist() == o2
    assert bundles.tolist() == b2
    assert load.tolist() == l2
    assert load.sum() == cost.sum()
    assert all(len(b) == J for b in bundles.tolist())


def test_lpt_single_chunk_per_rank_is_cost_order():
    # J = 1: the k-th costliest chunk goes to rank k (every rank starts empty).
    cost = np.array([5, 9, 9, 1, 7, 3], dtype=np.int64)
    owner, bundles, load = oracle.lpt(cost, 6, 1)
    order = sorted(range(6), key=lambda j: (-cost[j], j))
    assert [owner[j] for j in order] == list(range(6))
    assert load.tolist() == [cost[j] for j in order]


def test_lpt_rejects_wrong_chunk_count():
    with pytest.raises(ValueError):
        oracle.lpt(np.ones(7, np.int64), 2, 3)


@pytest.mark.parametrize("seed", range(20))
def test_lpt_gap_to_exhaustive_optimum_reported(seed):
    # Information only: LPT is a heuristic; it must never beat the optimum and
    # must place every chunk.
    g = np.random.default_rng(20_000 + seed)
    P, J = 2, 3
    cost = g.integers(0, 20, size=P * J).astype(np.int64)
    _, _, load = oracle.lpt(cost, P, J)
    best = min(max(cost[list(c)].sum(), cost.sum() - cost[list(c)].sum())
               for c in itertools.combinations(range(P * J), J))
    assert load.max() >= best


# ------------------------------------------- LPT vs Zigzag on the workloads
def _rho_pair(w, seed=0):
    s, a = inputs.workload_anchors(w, seed)
    cost, owner, bundles, load = oracle.plan(s, a, w.B, w.S, w.m, w.P, w.J)
    prof = oracle.anchor_profile(s, a, w.B, w.S)
    st, ln = inputs.sample_bounds(w)
    zz = oracle.zigzag_loads(st, ln, prof, w.P)
    assert zz.sum() == load.sum() == cost.sum()
    return oracle.imbalance(load, w.N, w.B), oracle.imbalance(zz, w.N, w.B)


@pytest.mark.parametrize("name", ["tiny", "weak8", "strong8", "weak64", "qs8", "qs16"])
def test_lpt_not_worse_than_zigzag_on_workloads(name):
    r_lpt, r_zz = _rho_pair(inputs.WORKLOADS[name])
    assert r_lpt <= r_zz + 1e-12, (r_lpt, r_zz)


def test_lpt_vs_zigzag_coarse_chunks_reported_only():
    # With J=2 chunks per rank (Q:S 1:4 point) LPT's chunks are coarser than
    # Zigzag's, so the inequality is not guaranteed; report only.
    r_lpt, r_zz = _rho_pair(inputs.WORKLOADS["qs4"])
    assert r_lpt >= 1.0 and r_zz >= 1.0


def test_rho_counterexample_is_possible():
    # rho_LPT <= rho_Zigzag is not a theorem: two 8-token samples, B=1,
    # P=2, J=2, m=4.
    s = np.array([0, 0, 8, 8])
    a = np.array([6, 7, 11, 12])
    cost, owner, bundles, load = oracle.plan(s, a, 1, 16, 4, 2, 2)
    prof = oracle.anchor_profile(s, a, 1, 16)
    zz = oracle.zigzag_loads([0, 8], [8, 8], prof, 2)
    assert cost.tolist() == [4 + 4, 2 + 3, 3 + 4, 0]
    assert oracle.imbalance(load, 4, 1) > oracle.imbalance(zz, 4, 1)


def test_contiguous_loads_sum_profile():
    w = inputs.WORKLOADS["tiny"]
    s, a = inputs.workload_anchors(w, 0)
    prof = oracle.anchor_profile(s, a, w.B, w.S)
    cl = oracle.contiguous_loads(prof, 4)
    assert cl.tolist() == [int(prof[i * 256:(i + 1) * 256].sum()) for i in range(4)]

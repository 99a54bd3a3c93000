"""Pins of oracle.locality_match: the LPT bundles placed on physical ranks so
that the step's all-to-all moves the fewest context rows (§4.2: a final
matching maps bundles to physical ranks without changing their loads).
Reading: physical rank r first holds chunks r*J .. r*J + J - 1."""
import itertools

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment

import oracle
from block_sparse_cross_amd import inputs


def keep_matrix(b, m):
    P, J = b.shape
    keep = np.zeros((P, P), np.int64)
    for i in range(P):
        for j in b[i]:
            if 0 <= j < P * J:
                keep[i, j // J] += m
    return keep


def check_invariants(b, m, perm, send, kept, moved):
    P, J = b.shape
    assert sorted(perm.tolist()) == list(range(P))
    keep = keep_matrix(b, m)
    assert kept == int(keep[np.arange(P), perm].sum())
    assert kept + moved == P * J * m
    assert (np.diag(send) == 0).all() and (send >= 0).all()
    assert int(send.sum()) == moved
    # rank dst receives every row of its bundle it does not already hold
    inv = np.argsort(perm)
    for dst in range(P):
        assert send[:, dst].sum() == J * m - keep[inv[dst], dst]
    # rank src gives away every row of its home range the bundle placed on it does not keep
    for src in range(P):
        assert send[src, :].sum() == J * m - keep[inv[src], src]


@pytest.mark.parametrize("P,J", [(1, 1), (2, 2), (3, 2), (4, 3), (5, 2), (6, 2)])
def test_optimal_by_brute_force(P, J):
    g = np.random.default_rng(P * 10 + J)
    for _ in range(30):
        b = g.permutation(P * J).reshape(P, J)
        perm, send, kept, moved = oracle.locality_match(b, 3)
        keep = keep_matrix(b, 3)
        best = max(sum(keep[i, p[i]] for i in range(P)) for p in itertools.permutations(range(P)))
        assert kept == best
        check_invariants(b, 3, perm, send, kept, moved)


@pytest.mark.parametrize("P,J", [(16, 4), (64, 8), (200, 2)])
def test_optimal_against_library_assignment(P, J):
    g = np.random.default_rng(P + J)
    for _ in range(5):
        b = g.permutation(P * J).reshape(P, J)
        perm, send, kept, moved = oracle.locality_match(b, 4096)
        keep = keep_matrix(b, 4096)
        r, c = linear_sum_assignment(keep, maximize=True)
        assert kept == int(keep[r, c].sum())
        check_invariants(b, 4096, perm, send, kept, moved)


def test_home_layouts_move_nothing():
    P, J = 6, 3
    home = np.arange(P * J).reshape(P, J)
    perm, send, kept, moved = oracle.locality_match(home, 10)
    assert perm.tolist() == list(range(P)) and moved == 0 and not send.any()
    sigma = np.array([3, 0, 5, 1, 4, 2])
    perm, send, kept, moved = oracle.locality_match(home[sigma], 10)
    assert perm.tolist() == sigma.tolist() and moved == 0


@pytest.mark.parametrize("name", ["tiny", "weak8", "strong8", "qs8", "weak64"])
def test_never_worse_than_keeping_plan_order(name):
    w = inputs.WORKLOADS[name]
    s, a = inputs.workload_anchors(w, 0)
    _, _, bundles, _ = oracle.plan(s, a, w.B, w.S, w.m, w.P, w.J)
    perm, send, kept, moved = oracle.locality_match(bundles, w.m)
    keep = keep_matrix(np.asarray(bundles), w.m)
    assert kept >= int(np.trace(keep))       # bundle b on rank b
    check_invariants(np.asarray(bundles), w.m, perm, send, kept, moved)

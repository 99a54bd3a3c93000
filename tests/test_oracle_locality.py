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


def rows_by_position(b, perm, m):
    """The all-to-all of a placement counted one context position at a time:
    position x sits in chunk x // m, which starts on rank x // (J m) and must
    end on the rank its bundle is placed on."""
    P, J = b.shape
    owner = np.full(P * J, -1)
    for i in range(P):
        for j in b[i]:
            if 0 <= j < P * J:
                owner[j] = i
    send = np.zeros((P, P), np.int64)
    kept = 0
    for x in range(P * J * m):
        j = x // m
        if owner[j] < 0:
            continue
        src, dst = x // (J * m), perm[owner[j]]
        if src == dst:
            kept += 1
        else:
            send[src, dst] += 1
    return send, kept


@pytest.mark.parametrize("P,J,m", [(1, 1, 3), (2, 3, 2), (4, 2, 5), (5, 3, 1), (7, 2, 3)])
def test_placement_rows_by_position(P, J, m):
    g = np.random.default_rng(P * 7 + J)
    for trial in range(10):
        b = g.permutation(P * J).reshape(P, J)
        if trial == 0:
            b[0, 0] = -1          # ids outside the plan are neither kept nor sent
        perm = g.permutation(P)
        send, kept, moved = oracle.placement_rows(b, perm, m)
        s_ref, k_ref = rows_by_position(b, perm, m)
        np.testing.assert_array_equal(send, s_ref)
        assert kept == k_ref and moved == P * J * m - kept


def test_placement_rows_of_the_matching_and_of_home():
    g = np.random.default_rng(5)
    b = g.permutation(40).reshape(8, 5)
    perm, send, kept, moved = oracle.locality_match(b, 16)
    s2, k2, m2 = oracle.placement_rows(b, perm, 16)
    np.testing.assert_array_equal(send, s2)
    assert (kept, moved) == (k2, m2)
    home = np.arange(40).reshape(8, 5)
    s3, k3, m3 = oracle.placement_rows(home, np.arange(8), 16)
    assert not s3.any() and k3 == 8 * 5 * 16 and m3 == 0
    # every bundle placed one rank further: all rows move
    s4, k4, m4 = oracle.placement_rows(home, (np.arange(8) + 1) % 8, 16)
    assert k4 == 0 and m4 == 640 and s4[np.arange(8), (np.arange(8) + 1) % 8].tolist() == [80] * 8


def test_placement_rows_rejects_non_permutations():
    b = np.arange(6).reshape(3, 2)
    for bad in ([0, 0, 1], [0, 1, 3], [-1, 0, 1]):
        with pytest.raises(ValueError):
            oracle.placement_rows(b, np.array(bad), 4)

"""Pins of oracle.validate_anchors (the device-side anchor check's oracle):
block i is valid when its window [s_i, a_i) lies inside the packed context
[0, S) (§3.1 and Figure 1 of the Split-KV paper; empty windows allowed)."""
import numpy as np
import pytest

import oracle
from block_sparse_cross_amd import inputs


def test_hand_cases():
    S = 100
    assert oracle.validate_anchors([], [], S) == (0, -1)
    # valid: ordinary, empty at 0, empty at S, the whole context
    assert oracle.validate_anchors([0, 0, 100, 0, 30], [10, 0, 100, 100, 70], S) == (0, -1)
    # one violation of each kind, at known places
    assert oracle.validate_anchors([0, -1, 5], [10, 4, 6], S) == (1, 1)       # s < 0
    assert oracle.validate_anchors([0, 0, 50], [10, 101, 40], S) == (2, 1)    # a > S, s > a
    assert oracle.validate_anchors([7, 0], [6, 10], S) == (1, 0)              # s > a first
    assert oracle.validate_anchors([0], [0], 0) == (0, -1)                    # S = 0, empty


def test_against_position_count():
    """Counted with the Eq. 2 profile instead of comparisons: a non-empty window
    is inside [0, S) exactly when the profile of that block alone, summed over
    [0, S), counts all a - s of its positions; an empty window [s, s) is valid
    when s = S or the one-position window [s, s + 1) is counted once."""
    g = np.random.default_rng(5)
    S = 64
    for _ in range(200):
        n = int(g.integers(1, 8))
        s = g.integers(-10, S + 10, n)
        a = s + g.integers(-5, 40, n)
        bad = []
        for i in range(n):
            if a[i] > s[i]:
                ok = int(oracle.anchor_profile([s[i]], [a[i]], 1, S).sum()) == a[i] - s[i]
            elif a[i] == s[i]:
                ok = s[i] == S or int(oracle.anchor_profile([s[i]], [s[i] + 1], 1, S).sum()) == 1
            else:
                ok = False
            if not ok:
                bad.append(i)
        assert oracle.validate_anchors(s, a, S) == (len(bad), bad[0] if bad else -1)


@pytest.mark.parametrize("name", ["tiny", "weak8", "strong8", "qs4"])
def test_generated_workloads_are_valid(name):
    w = inputs.WORKLOADS[name]
    s, a = inputs.workload_anchors(w, 0)
    assert oracle.validate_anchors(s, a, w.S) == (0, -1)

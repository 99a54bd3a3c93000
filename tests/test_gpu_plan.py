"""GPU planner (Eq. 6 costs + cost-aware LPT) against the oracle: bit-exact."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "figures.json")))


def gpu_plan(s, a, B, S, m, P, J):
    out = binding.splitkv_plan(to_dev(np.asarray(s, np.int64)), to_dev(np.asarray(a, np.int64)),
                               B, S, m, P, J)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check_plan(s, a, B, S, m, P, J):
    cost, owner, bundles, load = gpu_plan(s, a, B, S, m, P, J)
    c_o, ow_o, b_o, l_o = oracle.plan(s, a, B, S, m, P, J)
    np.testing.assert_array_equal(cost, c_o)
    np.testing.assert_array_equal(owner, ow_o)
    np.testing.assert_array_equal(bundles, b_o)
    np.testing.assert_array_equal(load, l_o)
    return cost, owner, bundles, load


def test_fig5_plan():
    f = GOLD["fig5"]
    s, a = [], []
    for smp in f["samples"]:
        for x in smp["anchors_local"]:
            s.append(smp["start"])
            a.append(smp["start"] + x)
    cost, owner, bundles, load = check_plan(s, a, f["B"], 24, f["m"], f["P"], f["J"])
    assert cost.tolist() == f["lpt_chunk_costs"]
    assert load.tolist() == f["lpt_loads"]


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_plans(name):
    w = inputs.WORKLOADS[name]
    s, a = inputs.workload_anchors(w, 0)
    check_plan(s, a, w.B, w.S, w.m, w.P, w.J)


def test_plan_many_random_tiny_cases():
    g = np.random.default_rng(7)
    for case in range(1000):
        P = int(g.integers(1, 9))
        J = int(g.integers(1, 5))
        m = int(g.integers(1, 9))
        S = P * J * m
        B = int(g.integers(1, 17))
        n_s = min(int(g.integers(1, 4)), S)
        L = max(1, S // n_s)
        s, a = [], []
        for u in range(n_s):
            st = u * L
            en = S if u == n_s - 1 else st + L
            k = int(g.integers(0, min(5, en - st) + 1))
            for x in np.sort(g.choice(en - st, size=k, replace=False)) + st:
                s.append(st)
                a.append(int(x))
        if not s:
            s, a = [0], [0]
        check_plan(s, a, B, S, m, P, J)


def test_plan_edge_sizes():
    # many ranks (multi-wave greedy), the chunk limit, a single chunk, no anchors
    g = np.random.default_rng(3)
    s, a = inputs.random_tiny_anchors(g, 4, 4096, 50, 1024)
    check_plan(s, a, 16, 4 * 4096, 4, 1024, 4)      # P=1024, 4096 chunks
    check_plan(s, a, 16, 4 * 4096, 4096, 1, 4)      # P=1, J=4
    check_plan(s, a, 16, 4 * 4096, 4 * 4096, 1, 1)  # one chunk
    check_plan(s, a, 16, 4 * 4096, 16, 128, 8)      # P=128 (2 waves)
    check_plan(np.zeros(0, np.int64), np.zeros(0, np.int64), 16, 64, 8, 4, 2)


def test_plan_rejects_bad_arguments():
    s = to_dev(np.array([0], np.int64))
    a = to_dev(np.array([5], np.int64))
    with pytest.raises(binding.SplitKVError) as e:
        binding.splitkv_plan(s, a, 16, 100, 8, 4, 3)  # P*J*m != S
    assert e.value.status == binding.SPLITKV_ERR_INVALID_ARG
    with pytest.raises(binding.SplitKVError) as e:
        binding.splitkv_plan(s, a, 16, 2048 * 4, 1, 2048, 4)  # over the rank limit
    assert e.value.status == binding.SPLITKV_ERR_UNSUPPORTED

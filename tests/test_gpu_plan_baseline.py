"""GPU position-based assignments (No balance, Zigzag) against the oracle: bit-exact.

Zigzag follows §3.3 / Figure 5(b) of the Split-KV paper; No balance is the
contiguous split of §5.5. The GPU prices the ranges with Eq. 6 overlaps, the
oracle sums the Eq. 2 profile over them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding
from block_sparse_cross_amd import inputs as I
from tests.helpers import to_dev
from tests.test_oracle_baseline import _random_case, fig5_anchors, fig9_workload

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "figures.json")))


def gpu_baseline(strategy, s, a, B, st, ln, P):
    out = binding.splitkv_plan_baseline(strategy, to_dev(np.asarray(s, np.int64)),
                                        to_dev(np.asarray(a, np.int64)), B, list(st), list(ln), P)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check(strategy, s, a, B, st, ln, P):
    cost, load = gpu_baseline(strategy, s, a, B, st, ln, P)
    prof = oracle.anchor_profile(s, a, B, int(np.sum(ln)))
    c_o, l_o = oracle.baseline_plan(strategy, st, ln, prof, P)
    np.testing.assert_array_equal(cost, c_o)
    np.testing.assert_array_equal(load, l_o)
    return cost, load


def test_fig5_zigzag():
    f = GOLD["fig5"]
    s, a = fig5_anchors()
    cost, load = check(binding.SPLITKV_BASELINE_ZIGZAG, s, a, f["B"], [0, 16], [16, 8], f["P"])
    assert cost.tolist() == f["zigzag_chunk_costs_sample0"] + f["zigzag_chunk_costs_sample1"]
    assert load.tolist() == f["zigzag_loads"]


@pytest.mark.parametrize("strategy", [0, 1])
def test_random_tiny_cases(strategy):
    for seed in range(200):
        P = int(np.random.default_rng(seed).integers(1, 9))
        st, ln, s, a, B = _random_case(seed, P)
        check(strategy, s, a, B, st, ln, P)


@pytest.mark.parametrize("strategy", [0, 1])
def test_no_anchors_gives_zero_loads(strategy):
    e = np.zeros(0, dtype=np.int64)
    cost, load = gpu_baseline(strategy, e, e, 16, [0, 64], [64, 128], 4)
    assert not cost.any() and not load.any()
    assert len(cost) == binding.baseline_range_count(strategy, 2, 4)


@pytest.mark.parametrize("L,P", [(16384, 8), (65536, 8), (262144, 8), (262144, 16),
                                 (262144, 32), (262144, 64)])
def test_fig9_workloads(L, P):
    w = fig9_workload(L, P, 8)
    s, a = I.workload_anchors(w, 0)
    st, ln = I.sample_bounds(w)
    for strategy in (0, 1):
        check(strategy, s, a, w.B, st, ln, P)


def test_many_samples_and_ranks():
    # 128 samples (the sample-table limit) and P = 1024 ranks (the rank limit)
    P = 1024
    ln = [2 * P] * 128
    st = np.concatenate([[0], np.cumsum(ln)[:-1]])
    g = np.random.default_rng(3)
    s, a = [], []
    for u in range(128):
        for x in np.sort(g.choice(np.arange(1, 2 * P + 1), size=8, replace=False)):
            s.append(st[u])
            a.append(st[u] + x)
    for strategy in (0, 1):
        check(strategy, s, a, 16, st, ln, P)


def test_invalid_arguments_enqueue_nothing():
    dev = torch.device("cuda")
    s = torch.zeros(2, dtype=torch.int64, device=dev)
    a = torch.full((2,), 8, dtype=torch.int64, device=dev)
    cost = torch.full((64,), -7, dtype=torch.int64, device=dev)
    load = torch.full((8,), -7, dtype=torch.int64, device=dev)
    bad = [
        (1, [0, 16], [16, 8], 3),    # 8 % (2*3) != 0
        (0, [0], [24], 5),           # 24 % 5 != 0
        (1, [0, 20], [16, 8], 2),    # not packed
        (1, [8], [16], 2),           # does not start at 0
        (2, [0], [16], 2),           # unknown strategy
        (1, [0], [0], 2),            # empty sample
        (1, [0], [16], 0),           # P < 1
    ]
    for strategy, st, ln, P in bad:
        with pytest.raises(binding.SplitKVError) as e:
            binding.splitkv_plan_baseline(strategy, s, a, 16, st, ln, P, out=(cost, load))
        assert e.value.status == binding.SPLITKV_ERR_INVALID_ARG
    with pytest.raises(binding.SplitKVError) as e:
        binding.splitkv_plan_baseline(1, s, a, 16, list(range(0, 129 * 4, 4)), [4] * 129, 2,
                                      out=(cost, load))
    assert e.value.status == binding.SPLITKV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (cost == -7).all() and (load == -7).all()

"""splitkv_validate_anchors (device-side anchor check) against the oracle:
count of blocks whose window [s_i, a_i) is not inside [0, S) and the first
such index, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def gpu_check(s, a, S):
    out = binding.splitkv_validate_anchors(to_dev(np.asarray(s, np.int64)),
                                           to_dev(np.asarray(a, np.int64)), 16, S)
    torch.cuda.synchronize()
    r = out.cpu().numpy()
    return int(r[0]), int(r[1])


def test_workload_anchors_are_valid():
    for name in ("weak8", "strong8", "weak64"):
        w = inputs.WORKLOADS[name]
        s, a = inputs.workload_anchors(w, 0)
        assert gpu_check(s, a, w.S) == (0, -1) == oracle.validate_anchors(s, a, w.S)


@pytest.mark.parametrize("seed", range(6))
def test_random_corruptions(seed):
    g = np.random.default_rng(seed)
    S = int(g.integers(1, 1 << 20))
    n = int(g.integers(1, 5000))
    s = g.integers(0, S, n)
    a = s + g.integers(0, S, n) % np.maximum(S - s + 1, 1)
    k = int(g.integers(0, 12))
    idx = g.choice(n, size=min(k, n), replace=False)
    for j, i in enumerate(idx):
        kind = j % 3
        if kind == 0:
            s[i] = -int(g.integers(1, 100))
        elif kind == 1:
            a[i] = S + int(g.integers(1, 100))
        else:
            s[i], a[i] = a[i] + 1, a[i]
    assert gpu_check(s, a, S) == oracle.validate_anchors(s, a, S)


def test_large_and_edges():
    n = 300_000
    S = 1 << 30
    s = np.arange(n, dtype=np.int64) * 16
    a = s + 8
    assert gpu_check(s, a, S) == (0, -1)
    a[n - 3] = S + 1                           # a late violation only
    assert gpu_check(s, a, S) == oracle.validate_anchors(s, a, S) == (1, n - 3)
    s[5] = -1                                  # and an early one
    assert gpu_check(s, a, S) == oracle.validate_anchors(s, a, S) == (2, 5)
    assert gpu_check([0, 0], [0, 0], 0) == (0, -1)            # S = 0, empty windows
    e = torch.zeros(0, dtype=torch.int64, device="cuda")
    out = binding.splitkv_validate_anchors(e, e, 16, 10)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [0, -1]                        # no blocks


def test_invalid_arguments():
    s = to_dev(np.zeros(4, np.int64))
    with pytest.raises(binding.SplitKVError):
        binding.splitkv_validate_anchors(s, s, 16, -1)          # S < 0
    with pytest.raises(binding.SplitKVError):
        binding.splitkv_validate_anchors(s, s, 0, 10)           # B < 1

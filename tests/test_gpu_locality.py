"""splitkv_locality_match (placement of the LPT bundles on physical ranks,
§4.2) against the definition: many placements keep the same number of rows in
place, so the GPU's placement is not compared with the oracle's. It must be a
permutation, keep as many rows as the optimum (the oracle's kept count, pinned
by brute force and a library assignment solver), and its send-row matrix and
kept/moved counts must be those that its own placement implies."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_amd import binding, inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def gpu_match(bundles, m):
    perm, send, km = binding.splitkv_locality_match(to_dev(np.asarray(bundles, np.int32)), m)
    torch.cuda.synchronize()
    return perm.cpu().numpy(), send.cpu().numpy(), km.cpu().numpy()


def assert_optimal_placement(bundles, m):
    perm, send, km = gpu_match(bundles, m)
    P = np.asarray(bundles).shape[0]
    assert sorted(perm.tolist()) == list(range(P)), "placement is not a permutation"
    _, _, best_kept, _ = oracle.locality_match(bundles, m)
    s_ref, kept, moved = oracle.placement_rows(bundles, perm, m)
    assert kept == best_kept, "placement keeps %d rows, the optimum keeps %d" % (kept, best_kept)
    np.testing.assert_array_equal(send, s_ref)
    assert km.tolist() == [kept, moved]


@pytest.mark.parametrize("P,J", [(1, 1), (2, 2), (3, 5), (8, 4), (16, 8), (64, 8), (65, 3),
                                 (100, 6), (128, 8), (129, 2), (256, 16)])
def test_random_bundles(P, J):
    g = np.random.default_rng(P * 100 + J)
    for trial in range(3):
        b = g.permutation(P * J).reshape(P, J)
        if trial == 1:
            b = np.arange(P * J).reshape(P, J)[g.permutation(P)]  # a permuted home layout
        assert_optimal_placement(b, 4096)


def test_permuted_home_layout_moves_nothing():
    P, J = 12, 3
    sigma = np.random.default_rng(3).permutation(P)
    b = np.arange(P * J).reshape(P, J)[sigma]
    perm, send, km = gpu_match(b, 64)
    assert perm.tolist() == sigma.tolist()    # the only placement that keeps everything
    assert not send.any() and km.tolist() == [P * J * 64, 0]


def test_ids_outside_the_plan_are_ignored():
    b = np.arange(24).reshape(6, 4)
    b[1, 2], b[4, 0] = -1, 10_000
    assert_optimal_placement(b, 7)


@pytest.mark.parametrize("name,P,J", [("weak8", 8, 4), ("cp64", 64, 8), ("cp16", 16, 8)])
def test_lpt_plans(name, P, J):
    if name == "weak8":
        w = inputs.WORKLOADS["weak8"]
    else:   # the CP-size study workloads of §5.5: 4 samples x 256k
        w = inputs.Workload(name, b=4, L=262144, A=512, B=16, hq=32, hkv=8, d=128,
                            dtype="bf16", scale=1.0, P=P, m=(4 * 262144) // (P * J))
    s, a = inputs.workload_anchors(w, 0)
    _, _, bundles, _ = binding.splitkv_plan(to_dev(s), to_dev(a), w.B, w.S, w.m, P, J)
    torch.cuda.synchronize()
    assert_optimal_placement(bundles.cpu().numpy(), w.m)


def test_invalid_arguments():
    with pytest.raises(binding.SplitKVError):
        binding.splitkv_locality_match(torch.zeros((257, 1), dtype=torch.int32, device="cuda"), 8)
    with pytest.raises(binding.SplitKVError):
        binding.splitkv_locality_match(torch.zeros((4, 2), dtype=torch.int32, device="cuda"), 0)
    with pytest.raises(ValueError):
        binding.splitkv_locality_match(torch.zeros((4, 2), dtype=torch.int64, device="cuda"), 8)

"""Pins for Eq. 4 in its two per-rank halves (the form Algorithm 1's MERGE takes
when the partials sit on different devices): an LSE reduction, then each rank
rescales its own partial by exp(lse_p - lse); and the backward's Delta summed
over ranks from the rescaled partials.

Pinned against: the unsplit attention (the Eq. 3 oracle over all keys, itself
pinned to torch SDPA) for a disjoint split of the keys; numpy's logaddexp
reduction; closed forms of the rescale; the weights summing to one.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_attn import _rand, _split_case


@pytest.mark.parametrize("seed", range(5))
def test_split_form_equals_unsplit_attention(seed):
    g, s, a, B, S, m, q, k, v, do = _split_case(seed)
    Q, hq, d = q.shape
    rows = np.arange(Q)
    o_full, l_full = oracle.partial_attn(rows, B, s, a, q, np.arange(S), k, v, 0.35)
    perm = g.permutation(S // m)
    groups = [sorted(perm[0:3]), sorted(perm[3:4]), sorted(perm[4:])]
    parts = []
    for ch in groups:
        pos = oracle.local_key_positions(ch, m)
        o_p, l_p = oracle.partial_attn(rows, B, s, a, q, pos, k[pos], v[pos], 0.35)
        parts.append((o_p.reshape(-1, d), l_p.reshape(-1)))
    lse = oracle.lse_reduce(np.stack([l for _, l in parts]))
    bars = [oracle.lse_rescale(o_p, l_p, lse) for o_p, l_p in parts]
    live = np.isfinite(l_full.reshape(-1))
    np.testing.assert_allclose(sum(bars), o_full.reshape(-1, d), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[live], l_full.reshape(-1)[live], rtol=0, atol=1e-12)
    assert np.isneginf(lse[~live]).all()
    # Delta summed over ranks from the rescaled partials = Delta of the unsplit output
    dsum = sum(oracle.delta(b.reshape(Q, hq, d), do) for b in bars)
    np.testing.assert_allclose(dsum, oracle.delta(o_full, do), rtol=0, atol=1e-12)


def test_lse_reduce_is_logaddexp():
    g = np.random.default_rng(11)
    P, R = 6, 50
    lp = _rand(g, P, R) * 20
    lp[:, 3] = -np.inf
    lp[1:, 8] = -np.inf
    got = oracle.lse_reduce(lp)
    with np.errstate(divide="ignore"):
        want = np.logaddexp.reduce(lp, axis=0)
    fin = np.isfinite(want)
    np.testing.assert_allclose(got[fin], want[fin], rtol=0, atol=1e-12)
    assert np.isneginf(got[3]) and got[8] == lp[0, 8]
    # one partial: the identity
    np.testing.assert_array_equal(oracle.lse_reduce(lp[:1]), lp[0])


def test_rescale_closed_forms_and_weights():
    g = np.random.default_rng(12)
    R, d = 40, 16
    o = _rand(g, R, d)
    lp = _rand(g, R) * 5
    # lse_p = lse: unchanged; lse_p = lse + log(1/4): a quarter; lse_p = -inf: zero
    np.testing.assert_array_equal(oracle.lse_rescale(o, lp, lp), o)
    q4 = oracle.lse_rescale(o, lp + np.log(0.25), lp)
    np.testing.assert_allclose(q4, 0.25 * o, rtol=1e-14, atol=0)
    z = oracle.lse_rescale(o, np.full(R, -np.inf), lp)
    assert (z == 0).all()
    # the weights exp(lse_p - lse) over the partials of a row sum to one
    P = 5
    lps = _rand(g, P, R) * 4
    lps[2, :7] = -np.inf
    lse = oracle.lse_reduce(lps)
    ones = sum(oracle.lse_rescale(np.ones((R, 1)), lps[p], lse) for p in range(P))
    np.testing.assert_allclose(ones[:, 0], 1.0, rtol=0, atol=1e-14)

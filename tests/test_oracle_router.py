"""Pins for the router oracle (CPU only): softmax over all experts, top-k with
ties to the lower id ("Running 125B MoE on Two 32 GB Cards", section 4.2), and
the gathered (not renormalised) gate weights the library takes as input."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import router


def test_softmax_matches_torch_and_sums_to_one():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((7, 8)) * 5
    p = router.softmax(z)
    ref = torch.softmax(torch.from_numpy(z), dim=-1).numpy()
    np.testing.assert_allclose(p, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # shift invariance: adding a constant to every logit changes nothing
    np.testing.assert_allclose(router.softmax(z + 123.0), p, rtol=1e-12, atol=1e-15)


def test_closed_form_two_experts():
    """E = 2: p0 = 1 / (1 + exp(z1 - z0))."""
    for z0, z1 in [(0.0, 0.0), (1.0, -2.0), (-3.5, 4.25)]:
        p = router.softmax(np.array([[z0, z1]]))[0]
        assert math.isclose(p[0], 1.0 / (1.0 + math.exp(z1 - z0)), rel_tol=1e-14)


def _brute_topk(p, k):
    """Enumerate every k-subset in every order; keep the one whose sequence of
    (-p, id) is lexicographically smallest: largest p first, lower id on ties."""
    E = len(p)
    best = None
    for perm in itertools.permutations(range(E), k):
        key = [(-p[e], e) for e in perm]
        if best is None or key < best[0]:
            best = (key, perm)
    return list(best[1])


def test_topk_by_enumeration_at_tiny_shape():
    """8 experts, top-2 (the fp32 single-layer workload's router), random logits
    and logits with many exact ties."""
    rng = np.random.default_rng(2)
    cases = [rng.standard_normal(8) for _ in range(50)]
    cases += [rng.integers(0, 3, 8).astype(np.float64) for _ in range(50)]    # ties galore
    for z in cases:
        p = router.softmax(z[None, :])[0]
        for k in (1, 2, 3):
            assert router.top_k(p[None, :], k)[0].tolist() == _brute_topk(p, k)


def test_hand_made_tie_goes_to_lower_id():
    p = np.array([[0.1, 0.3, 0.3, 0.05, 0.25]])
    assert router.top_k(p, 1).tolist() == [[1]]
    assert router.top_k(p, 2).tolist() == [[1, 2]]
    assert router.top_k(p, 3).tolist() == [[1, 2, 4]]
    # all equal: ids ascending
    assert router.top_k(np.full((1, 6), 1 / 6), 4).tolist() == [[0, 1, 2, 3]]


def test_route_gathers_without_renormalising():
    rng = np.random.default_rng(3)
    E, H, T, K = 8, 64, 5, 2
    Wg = rng.standard_normal((E, H)) * 0.02
    x = rng.standard_normal((T, H))
    ids, w = router.route(Wg, x, K)
    p = torch.softmax(torch.from_numpy(x) @ torch.from_numpy(Wg).T, dim=-1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-12)
    assert (w.sum(axis=1) < 1.0).all()          # top-2 of 8: not renormalised
    assert (w[:, 0] >= w[:, 1]).all()
    np.testing.assert_allclose(router.gate_weights(Wg, x, ids), w, rtol=0, atol=0)


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        router.top_k(np.ones((1, 4)) / 4, 5)

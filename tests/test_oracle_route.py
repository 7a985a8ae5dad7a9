"""Pins for the oracle's router producer (oracle.route) and expert histogram.

The definition (softmax over all experts, top-k by descending probability with ties to the
lower id, optional renormalisation) is checked against closed forms written here with
math.exp, against brute force over every expert subset, against scipy's softmax, and
against invariants (shift of all logits, renormalised sums, histogram = bincount).
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def test_worked_example_ties_no_renorm():
    # logits 1, 3, 2, 3: experts 1 and 3 tie for the top; the lower id comes first.
    ids, w = oracle.route(np.array([[1.0, 3.0, 2.0, 3.0]]), 2, False)
    assert ids.tolist() == [[1, 3]]
    den = math.exp(1) + 2 * math.exp(3) + math.exp(2)
    assert np.allclose(w, [[math.exp(3) / den, math.exp(3) / den]], rtol=1e-14, atol=0)


def test_worked_example_renormalised_subset():
    ids, w = oracle.route(np.array([[1.0, 3.0, 2.0, 3.0]]), 3, True)
    assert ids.tolist() == [[1, 3, 2]]
    den = 2 * math.exp(3) + math.exp(2)
    assert np.allclose(w, [[math.exp(3) / den, math.exp(3) / den, math.exp(2) / den]],
                       rtol=1e-14, atol=0)


def test_renormalised_pair_is_a_logistic():
    # two chosen experts with logits a > b: weights 1/(1+e^{b-a}) and 1/(1+e^{a-b})
    a, b = 0.7, -1.3
    ids, w = oracle.route(np.array([[b, -5.0, a, -9.0]]), 2, True)
    assert ids.tolist() == [[2, 0]]
    assert np.allclose(w, [[1 / (1 + math.exp(b - a)), 1 / (1 + math.exp(a - b))]], rtol=1e-14)


@pytest.mark.parametrize("renorm", [False, True])
def test_all_equal_logits(renorm):
    E, k = 7, 3
    ids, w = oracle.route(np.full((2, E), 0.25), k, renorm)
    assert ids.tolist() == [[0, 1, 2]] * 2
    assert np.allclose(w, 1 / k if renorm else 1 / E, rtol=1e-14)


def test_k_equals_E_is_the_sorted_softmax():
    lg = np.array([[0.5, -1.0, 2.0, 0.5, 3.0]])
    ids, w = oracle.route(lg, 5, False)
    assert ids.tolist() == [[4, 2, 0, 3, 1]]
    assert np.allclose(w[0], softmax(lg[0])[ids[0]], rtol=1e-13)
    _, wr = oracle.route(lg, 5, True)
    assert np.allclose(wr, w, rtol=1e-13)


def _brute_force_choice(row, k):
    """The k-subset with the largest logits, order by (logit desc, id asc); among subsets with
    the same multiset of logits the one with the smallest ids -- enumerated, not sorted."""
    E = len(row)
    best = None
    for sub in itertools.combinations(range(E), k):
        key = (sorted((-row[e] for e in sub)), sorted(sub))
        if best is None or key < best[0]:
            best = (key, sub)
    sub = best[1]
    return sorted(sub, key=lambda e: (-row[e], e))


def test_selection_matches_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(300):
        E = int(rng.integers(1, 8))
        k = int(rng.integers(1, E + 1))
        # few distinct values so that ties are common
        row = rng.integers(-2, 3, E).astype(np.float64) * 0.5
        ids, _ = oracle.route(row[None, :], k, False)
        assert ids[0].tolist() == _brute_force_choice(row, k), (row, k)


def test_weights_are_the_softmax_probabilities():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 16)) * 3
    ids, w = oracle.route(lg, 4, False)
    p = softmax(lg, axis=1)
    assert np.allclose(w, np.take_along_axis(p, ids.astype(np.int64), axis=1), rtol=1e-12)
    # non-increasing along j
    assert (np.diff(w, axis=1) <= 1e-15).all()
    _, wr = oracle.route(lg, 4, True)
    assert np.allclose(wr.sum(axis=1), 1.0, rtol=1e-14)
    assert np.allclose(wr, w / w.sum(axis=1, keepdims=True), rtol=1e-14)


def test_shift_invariance():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((20, 9))
    ids_a, w_a = oracle.route(lg, 3, False)
    ids_b, w_b = oracle.route(lg + 100.0, 3, False)
    assert np.array_equal(ids_a, ids_b)
    assert np.allclose(w_a, w_b, rtol=1e-12)


def test_histogram_is_bincount():
    rng = np.random.default_rng(8)
    ids = rng.integers(-1, 12, (40, 3))
    h = oracle.expert_histogram(ids, 10)
    ref = np.bincount(ids[(ids >= 0) & (ids < 10)], minlength=10)
    assert h.tolist() == ref.tolist()


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((1, 3)), 4, False)


@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_prefill_bf16", "dsv3_decode_bf16",
                                  "skewed_prefill_bf16", "dsv3_fp8_e4m3"])
def test_agrees_with_the_input_generator(name):
    """The workloads' routing inputs are made by a separate implementation (probabilities,
    stable argsort); on the same logits the two must pick the same experts."""
    from moe_inputs import CONFIGS, make_logits, make_routing
    cfg = CONFIGS[name]
    ids_gen, w_gen, _ = make_routing(cfg, 0)
    ids, w = oracle.route(make_logits(cfg, 0), cfg.top_k, cfg.renormalize)
    assert np.array_equal(ids, ids_gen)
    assert np.allclose(w, w_gen, rtol=1e-6, atol=0)


def test_agrees_with_the_input_generator_on_the_shard_workload():
    """Production-like logits over 128 experts (the expert-parallel shard's router)."""
    from moe_inputs import get_config, make_logits, make_routing
    cfg = get_config("gptoss_shard_bf16", T=512)
    ids_gen, w_gen, _ = make_routing(cfg, 0)
    lg = make_logits(cfg, 0)
    assert lg.shape == (512, 128)
    ids, w = oracle.route(lg, cfg.top_k, cfg.renormalize)
    assert np.array_equal(ids, ids_gen)
    assert np.allclose(w, w_gen, rtol=1e-6, atol=0)

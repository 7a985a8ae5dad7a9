"""Pins for the oracle's alignment (expert sort, padding, tile table).

The oracle is a stable counting sort; here it is checked against a hand-worked
fixture, against a comparison sort (a different algorithm), and against the
invariants that define the layout.
"""
import json
import os

import numpy as np
import pytest

import oracle
from moe_inputs import CONFIGS, make_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "align_worked_examples.json")


def brute_force_layout(ids, E, BM):
    """Comparison sort by (expert, slot); then cut into padded segments."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    N = len(flat)
    valid = [s for s in range(N) if 0 <= flat[s] < E]
    order = sorted(valid, key=lambda s: (flat[s], s))
    rows = []
    tiles = []
    for e in range(E):
        seg = [s for s in order if flat[s] == e]
        if not seg:
            continue
        pad = (-len(seg)) % BM
        first = len(rows)
        rows += seg + [N] * pad
        tiles += [(e, first + b * BM) for b in range((len(seg) + pad) // BM)]
    return rows, tiles


def check_invariants(a: oracle.Alignment, ids, E, BM):
    flat = np.asarray(ids).reshape(-1)
    N = flat.size
    valid = (flat >= 0) & (flat < E)
    assert a.counts.sum() == valid.sum()
    assert a.n_invalid == N - valid.sum()
    assert a.offsets[0] == 0
    assert np.all(np.diff(a.offsets) >= 0)
    assert np.all(a.offsets % BM == 0)
    assert np.all(np.diff(a.offsets) == -(-a.counts // BM) * BM)
    assert a.sorted_slots.size == oracle.max_padded_slots(N, E, BM)
    assert a.offsets[-1] <= a.sorted_slots.size
    # every valid slot appears once, at slot_row, inside its expert's segment, ascending
    real = a.sorted_slots[a.sorted_slots != N]
    assert sorted(real.tolist()) == np.nonzero(valid)[0].tolist()
    for s in range(N):
        if valid[s]:
            r = a.slot_row[s]
            assert a.sorted_slots[r] == s
            e = flat[s]
            assert a.offsets[e] <= r < a.offsets[e] + a.counts[e]
        else:
            assert a.slot_row[s] == -1
    for e in range(E):
        seg = a.sorted_slots[a.offsets[e]:a.offsets[e] + a.counts[e]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)
        assert np.all(a.sorted_slots[a.offsets[e] + a.counts[e]:a.offsets[e + 1]] == N)
    assert np.all(a.sorted_slots[a.offsets[-1]:] == N)
    assert a.num_tiles == int((-(-a.counts // BM)).sum())
    assert a.tiles.shape == (oracle.max_tiles(N, E, BM), 2)
    assert np.all(a.tiles[a.num_tiles:] == -1)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_align_worked_examples(case):
    a = oracle.align(np.array(case["topk_ids"], np.int32), case["num_experts"], case["block_m"])
    assert a.counts.tolist() == case["counts"]
    assert a.offsets.tolist() == case["offsets"]
    assert a.sorted_slots.tolist() == case["sorted_slots"]
    assert a.slot_row.tolist() == case["slot_row"]
    assert a.tiles.tolist() == case["tiles"]
    assert a.num_tiles == case["num_tiles"]
    assert a.n_invalid == case["n_invalid"]
    check_invariants(a, np.array(case["topk_ids"]), case["num_experts"], case["block_m"])


def adversarial_routings():
    rng = np.random.default_rng(7)
    yield "all_on_one_expert", np.full((37, 3), 5, np.int32), 8, 16
    yield "one_expert_nonempty_E256", np.full((4, 2), 200, np.int32), 256, 16
    yield "E256_fewer_slots_than_experts", rng.integers(0, 256, (5, 8)).astype(np.int32), 256, 16
    yield "duplicate_ids_within_token", rng.integers(0, 3, (50, 4)).astype(np.int32), 3, 4
    yield "single_slot", np.array([[2]], np.int32), 4, 16
    yield "invalid_ids_mixed", np.array([[0, -1], [4, 1], [1, 1]], np.int32), 4, 2
    yield "block_m_1", rng.integers(0, 6, (20, 2)).astype(np.int32), 6, 1
    yield "exact_multiples", np.repeat(np.arange(4, dtype=np.int32), 32).reshape(64, 2), 4, 32


@pytest.mark.parametrize("name,ids,E,BM", list(adversarial_routings()), ids=lambda v: v if isinstance(v, str) else "")
def test_align_matches_brute_force(name, ids, E, BM):
    a = oracle.align(ids, E, BM)
    rows, tiles = brute_force_layout(ids, E, BM)
    assert a.sorted_slots[:len(rows)].tolist() == rows
    assert a.offsets[-1] == len(rows)
    assert [tuple(t) for t in a.tiles[:a.num_tiles].tolist()] == tiles
    check_invariants(a, ids, E, BM)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_align_workload_routings(name):
    cfg = CONFIGS[name]
    ids, w, _ = make_routing(cfg, seed=0)
    for BM in (16, 64, 128):
        a = oracle.align(ids, cfg.E, BM)
        check_invariants(a, ids, cfg.E, BM)
        counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
        assert a.counts.tolist() == counts.tolist()

"""Pins for the routing oracle: hand-derived examples and brute force through
numpy's stable argsort, plus the structural invariants."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("case", range(3))
def test_route_handworked(case):
    c = json.load(open(os.path.join(GOLDEN, "route_handworked.json")))["cases"][case]
    r = oracle.route(np.array(c["ids"], np.int32), c["E"], c["M"])
    for key in ("counts", "offsets", "sorted", "slot_of", "tile_expert"):
        np.testing.assert_array_equal(r[key], np.array(c[key], np.int32), err_msg=key)
    assert r["num_tiles"] == c["num_tiles"]


def _brute(ids, E, M):
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")  # groups by expert, keeps f order inside
    counts = np.bincount(flat, minlength=E)
    padded = -(-counts // M) * M
    offsets = np.concatenate([[0], np.cumsum(padded)])
    sorted_ = -np.ones(offsets[-1], np.int64)
    pos = 0
    for e in range(E):
        members = order[pos:pos + counts[e]]
        sorted_[offsets[e]:offsets[e] + counts[e]] = members
        pos += counts[e]
    slot_of = np.empty(flat.size, np.int64)
    slot_of[sorted_[sorted_ >= 0]] = np.nonzero(sorted_ >= 0)[0]
    tile_expert = np.repeat(np.arange(E), padded // M)
    return counts, offsets, sorted_, slot_of, tile_expert


@pytest.mark.parametrize("T,K,E,M,pattern", [
    (64, 2, 8, 32, "random"), (1, 8, 128, 64, "random"), (300, 8, 128, 64, "random"),
    (1000, 2, 8, 128, "random"), (257, 4, 16, 16, "one"), (100, 3, 32, 64, "skewed"),
    (5, 1, 1, 8, "random"), (33, 7, 7, 4, "random"),
])
def test_route_vs_stable_argsort(T, K, E, M, pattern):
    rng = np.random.default_rng(T * 31 + E)
    if pattern == "random":
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    elif pattern == "one":  # expert 3 takes every token's first choice
        ids = np.stack([np.concatenate([[3], rng.permutation([e for e in range(E) if e != 3])[:K - 1]])
                        for _ in range(T)])
    else:  # most experts empty
        ids = np.stack([rng.permutation(4)[:K] * 3 for _ in range(T)])
    ids = ids.astype(np.int32)
    r = oracle.route(ids, E, M)
    counts, offsets, sorted_, slot_of, tile_expert = _brute(ids, E, M)
    np.testing.assert_array_equal(r["counts"], counts)
    np.testing.assert_array_equal(r["offsets"], offsets)
    np.testing.assert_array_equal(r["sorted"], sorted_)
    np.testing.assert_array_equal(r["slot_of"], slot_of)
    np.testing.assert_array_equal(r["tile_expert"], tile_expert)
    # invariants
    assert r["counts"].sum() == T * K
    assert np.all(r["offsets"] % M == 0)
    assert r["num_tiles"] * M == r["offsets"][-1]
    real = r["sorted"][r["sorted"] >= 0]
    assert np.array_equal(np.sort(real), np.arange(T * K))
    assert np.all(r["sorted"][r["slot_of"]] == np.arange(T * K))
    for e in range(E):
        seg = r["sorted"][r["offsets"][e]:r["offsets"][e + 1]]
        live = seg[seg >= 0]
        assert np.all(ids.ravel()[live] == e)
        assert np.all(np.diff(live) > 0)  # stable: ascending slot index
        assert np.all(seg[len(live):] == -1)  # pads trail the live rows


def test_route_drops_out_of_range_ids():
    ids = np.array([[0, 5], [-1, 1], [2, 1]], np.int32)
    r = oracle.route(ids, 3, 2)
    np.testing.assert_array_equal(r["counts"], [1, 2, 1])
    assert r["slot_of"][1] == -1 and r["slot_of"][2] == -1
    assert sorted(r["sorted"][r["sorted"] >= 0].tolist()) == [0, 3, 4, 5]


def test_route_empty():
    r = oracle.route(np.zeros((0, 2), np.int32), 4, 16)
    assert r["num_tiles"] == 0 and r["offsets"].tolist() == [0] * 5

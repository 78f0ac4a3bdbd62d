"""Pins of the oracle's cross-scan / cross-merge (exact permutations).

Checked against a hand-derived fixture, against numpy transposes/flips (a second,
independent way to write the routes), and against the algebra the merge must obey
(merge o scan = 4*identity, merge = scan^T).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cross_scan_2x3.txt")
SHAPES = [(1, 1), (1, 7), (7, 1), (2, 3), (8, 8), (5, 9), (14, 14), (3, 56)]


def _load_golden():
    routes = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, vals = line.split(":")
                routes[int(k[1:])] = [int(v) for v in vals.split()]
    return np.array([routes[k] for k in range(4)])


def test_golden_2x3():
    assert (oracle.perm_indices(2, 3) == _load_golden()).all()
    x = np.arange(6, dtype=float).reshape(1, 1, 2, 3)
    xs = oracle.cross_scan(x)
    assert (xs[0, :, 0, :] == _load_golden()).all()


@pytest.mark.parametrize("H,W", SHAPES)
def test_routes_are_bijections(H, W):
    idx = oracle.perm_indices(H, W)
    for k in range(4):
        assert sorted(idx[k].tolist()) == list(range(H * W))


@pytest.mark.parametrize("H,W", SHAPES)
def test_routes_vs_transpose_and_flip(H, W):
    rng = np.random.default_rng(H * 100 + W)
    x = rng.standard_normal((2, 3, H, W))
    xs = oracle.cross_scan(x)
    row = x.reshape(2, 3, H * W)
    col = np.transpose(x, (0, 1, 3, 2)).reshape(2, 3, H * W)
    assert (xs[:, 0] == row).all()
    assert (xs[:, 1] == col).all()
    assert (xs[:, 2] == np.flip(row, -1)).all()
    assert (xs[:, 3] == np.flip(col, -1)).all()


@pytest.mark.parametrize("H,W", SHAPES)
def test_merge_of_scan_is_four_times_identity(H, W):
    assert (oracle.cross_merge(oracle.cross_scan(np.ones((1, 2, H, W))), H, W) == 4.0).all()
    rng = np.random.default_rng(7)
    x = rng.integers(-1000, 1000, size=(2, 3, H, W)).astype(float)
    assert (oracle.cross_merge(oracle.cross_scan(x), H, W) == 4 * x).all()


@pytest.mark.parametrize("H,W", SHAPES)
def test_merge_is_adjoint_of_scan(H, W):
    rng = np.random.default_rng(11)
    x = rng.integers(-50, 50, size=(2, 3, H, W)).astype(float)
    y = rng.integers(-50, 50, size=(2, 4, 3, H * W)).astype(float)
    lhs = float((oracle.cross_scan(x) * y).sum())
    rhs = float((x * oracle.cross_merge(y, H, W)).sum())
    assert lhs == rhs  # integers: exact


def test_merge_single_route_is_inverse_permutation():
    H, W = 5, 9
    rng = np.random.default_rng(3)
    ys = np.zeros((1, 4, 2, H * W))
    x = rng.standard_normal((1, 2, H, W))
    xs = oracle.cross_scan(x)
    for k in range(4):
        only = ys.copy()
        only[:, k] = xs[:, k]
        assert (oracle.cross_merge(only, H, W) == x).all()

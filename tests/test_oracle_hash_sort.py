"""Pins of the oracle's ANN hash and bucket grouping (CPU only).

The hash is pinned by a hand-worked basis-plane fixture (bit order, sign of
zero, tie flag), by scale and negation identities, and by the SimHash
collision law: for random Gaussian hyperplanes two vectors at angle theta get
the same bit with probability 1 - theta/pi.  The grouping is pinned against
NumPy's stable argsort and bincount.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import ann_hash, bucket_sort
from tests.conftest import GOLDEN


def test_hash_basis_planes_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "hash_basis.json")))
    planes = np.array(fx["planes"], np.float32)
    X = np.array([c["x"] for c in fx["cases"]], np.float32)
    ids, tie = ann_hash(X, planes)
    assert ids.tolist() == [c["id"] for c in fx["cases"]]
    assert tie.tolist() == [c["tie_bits"] for c in fx["cases"]]


def test_hash_no_planes_is_one_bucket():
    X = np.random.default_rng(1).standard_normal((50, 16))
    ids, tie = ann_hash(X, np.zeros((0, 16)))
    assert (ids == 0).all() and (tie == 0).all()


def test_hash_scale_and_negation():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((400, 32))
    R = rng.standard_normal((7, 32))
    ids, tie = ann_hash(X, R)
    for a in (0.5, 3.7, 1e3):
        ids_a, _ = ann_hash(a * X, R)
        assert (ids_a == ids).all()
    ids_n, _ = ann_hash(-X, R)
    ok = tie == 0
    assert ok.sum() > 390
    assert (ids_n[ok] == (~ids[ok].astype(np.int64)) & 0x7F).all()


def test_hash_simhash_collision_law():
    """Pr[bit agrees] = 1 - theta/pi for Gaussian hyperplanes (Charikar)."""
    rng = np.random.default_rng(3)
    d = 8
    for theta in (math.pi / 6, math.pi / 3, math.pi / 2, 2 * math.pi / 3):
        x = np.zeros(d); x[0] = 1
        y = np.zeros(d); y[0] = math.cos(theta); y[1] = math.sin(theta)
        agree = 0
        total = 0
        for _ in range(256):
            R = rng.standard_normal((16, d))
            ids, _ = ann_hash(np.stack([x, y]), R)
            diff = int(ids[0]) ^ int(ids[1])
            agree += 16 - bin(diff).count("1")
            total += 16
        frac = agree / total
        assert abs(frac - (1 - theta / math.pi)) < 0.03, (theta, frac)


def test_hash_orthogonal_plane_flags_tie():
    R = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]])
    X = np.array([[0.0, 2.0, 1.0], [1e-7, -2.0, 1.0], [3.0, -1.0, 0.0]])
    ids, tie = ann_hash(X, R)
    assert tie.tolist() == [1, 1, 0]
    assert ids.tolist() == [3, 1, 1]


@pytest.mark.parametrize("N,P", [(0, 3), (1, 0), (1000, 5), (4096, 7), (333, 10)])
def test_bucket_sort_matches_stable_argsort(N, P):
    rng = np.random.default_rng(N + P)
    ids = rng.integers(0, 1 << P, size=N).astype(np.uint16)
    off, perm = bucket_sort(ids, P)
    assert off.shape == ((1 << P) + 1,)
    assert (perm == np.argsort(ids, kind="stable")).all()
    counts = np.bincount(ids.astype(np.int64), minlength=1 << P)
    assert (off == np.concatenate([[0], np.cumsum(counts)])).all()


def test_bucket_sort_single_bucket_is_identity():
    ids = np.full(77, 5, np.uint16)
    off, perm = bucket_sort(ids, 3)
    assert (perm == np.arange(77)).all()
    assert off.tolist() == [0, 0, 0, 0, 0, 0, 77, 77, 77]

"""Pins of the oracle's AnnSA and AnnCA (CPU only).

AnnSA with a single bucket must be textbook softmax attention, and in general
it must equal dense attention under the mask [id(q_i) == id(k_j)]; both are
checked against torch's scaled_dot_product_attention in fp64 (a library
routine), lse against torch.logsumexp.  AnnCA with every prompt token kept is
full cross-attention; with pruning it is cross-attention masked to the kept
tokens, and the keep mask is checked by brute force over (query, token) pairs.
Hand-worked fixtures pin the numbers and the bucket restriction.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ann_hash, annca, annsa
from tests.conftest import GOLDEN


def sdpa(q, k, v, mask, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(q, np.float64))[None],
        torch.from_numpy(np.asarray(k, np.float64))[None],
        torch.from_numpy(np.asarray(v, np.float64))[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None], scale=scale)
    return out[0].numpy()


def masked_lse(q, k, mask, scale):
    S = torch.from_numpy(np.asarray(q, np.float64) @ np.asarray(k, np.float64).T * scale)
    S = S.masked_fill(~torch.from_numpy(mask), -math.inf)
    return torch.logsumexp(S, dim=1).numpy()


def test_annsa_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "annsa_hand.json")))
    O, lse = annsa(fx["q"], fx["q_ids"], fx["k"], fx["v"], fx["k_ids"], fx["scale"])
    np.testing.assert_allclose(O, fx["expected_o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, fx["expected_lse"], rtol=0, atol=1e-12)


def test_annsa_one_bucket_is_dense_attention():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((n, 64)) for n in (50, 300, 300))
    scale = 1 / 8
    O, lse = annsa(q, np.zeros(50), k, v, np.zeros(300), scale)
    np.testing.assert_allclose(O, sdpa(q, k, v, None, scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, masked_lse(q, k, np.ones((50, 300), bool), scale), atol=1e-12)


@pytest.mark.parametrize("P", [2, 4, 6])
def test_annsa_equals_bucket_masked_dense_attention(P):
    rng = np.random.default_rng(P)
    d = 32
    q, k, v = (rng.standard_normal((n, d)) for n in (120, 500, 500))
    R = rng.standard_normal((P, d))
    qi, _ = ann_hash(q, R)
    ki, _ = ann_hash(k, R)
    scale = 1 / math.sqrt(d)
    O, lse = annsa(q, qi, k, v, ki, scale)
    mask = qi[:, None] == ki[None, :]
    has = mask.any(1)
    assert has.sum() >= 100
    np.testing.assert_allclose(O[has], sdpa(q[has], k, v, mask[has], scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[has], masked_lse(q[has], k, mask[has], scale), atol=1e-12)
    assert (O[~has] == 0).all() and np.isneginf(lse[~has]).all()


def test_annsa_key_order_does_not_matter():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((n, 16)) for n in (40, 200, 200))
    qi = rng.integers(0, 8, 40)
    ki = rng.integers(0, 8, 200)
    O, lse = annsa(q, qi, k, v, ki, 0.25)
    p = rng.permutation(200)
    O2, lse2 = annsa(q, qi, k[p], v[p], ki[p], 0.25)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


def test_annsa_empty_bucket():
    O, lse = annsa(np.ones((2, 4)), [1, 3], np.ones((3, 4)), np.ones((3, 4)), [1, 1, 2], 1.0)
    assert (O[1] == 0).all() and np.isneginf(lse[1])
    np.testing.assert_allclose(O[0], 1.0)


def test_annca_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "annca_hand.json")))
    O, keep = annca(fx["q"], fx["q_ids"], fx["frame_len"], fx["kp"], fx["vp"], fx["kp_ids"],
                    fx["scale"])
    assert keep.tolist() == fx["expected_keep"]
    np.testing.assert_allclose(O, fx["expected_o"], rtol=0, atol=1e-12)


def test_annca_all_kept_is_full_cross_attention():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((90, 32))
    kp, vp = rng.standard_normal((64, 32)), rng.standard_normal((64, 32))
    O, keep = annca(q, np.zeros(90), 30, kp, vp, np.zeros(64), 0.2)
    assert keep.all()
    np.testing.assert_allclose(O, sdpa(q, kp, vp, None, 0.2), rtol=0, atol=1e-12)


def test_annca_pruned_equals_masked_cross_attention_and_bruteforce_keep():
    rng = np.random.default_rng(8)
    d, P, fl, F = 16, 5, 20, 3
    R = rng.standard_normal((P, d))
    q = rng.standard_normal((fl * F, d)) * 0.3 + rng.standard_normal(d)  # few buckets
    kp, vp = rng.standard_normal((48, d)), rng.standard_normal((48, d))
    qi, _ = ann_hash(q, R)
    pi, _ = ann_hash(kp, R)
    O, keep = annca(q, qi, fl, kp, vp, pi, 0.3)
    for f in range(F):
        for t in range(48):
            brute = any(int(qi[i]) == int(pi[t]) for i in range(f * fl, (f + 1) * fl))
            assert keep[f, t] == brute
        rows = slice(f * fl, (f + 1) * fl)
        if keep[f].any():
            mask = np.broadcast_to(keep[f], (fl, 48)).copy()
            np.testing.assert_allclose(O[rows], sdpa(q[rows], kp, vp, mask, 0.3), atol=1e-12)
        else:
            assert (O[rows] == 0).all()
    assert 0 < keep.sum() < keep.size


def test_annca_nothing_kept_gives_zero():
    O, keep = annca(np.ones((4, 3)), [1, 1, 2, 2], 2, np.ones((5, 3)), np.ones((5, 3)),
                    [0, 0, 3, 3, 3], 1.0)
    assert not keep.any() and (O == 0).all()


def test_annca_rejects_ragged_frames():
    with pytest.raises(ValueError):
        annca(np.ones((5, 3)), [0] * 5, 2, np.ones((2, 3)), np.ones((2, 3)), [0, 0], 1.0)

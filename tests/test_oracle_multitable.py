"""Pins of the oracle's multi-table AnnSA and union search (CPU only).

* brute force: for tiny inputs, explicit per-pair set membership ("some table
  shares the bucket") and a per-query softmax written with math.exp;
* one table reduces to the single-table ``annsa`` (a different formulation:
  per-bucket loops instead of a union mask);
* two identical tables give the same attention as one (the union counts a
  key once, not once per table);
* a table whose planes are all zero puts every token in one bucket, so the
  union is every key: dense softmax attention (scipy's softmax);
* the union search equals a brute-force argmax of the cosine over the union,
  and with one table it equals the single-table search;
* the id fields are those of one hash over the T*P planes of all tables.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import ann_hash, annsa, annsa_multi, bucket_fields, tempcache_top1


def _draw(seed, nq, nk, d):
    rng = np.random.default_rng(seed)
    return (rng, rng.standard_normal((nq, d)), rng.standard_normal((nk, d)),
            rng.standard_normal((nk, d)))


def test_brute_force_tiny():
    rng, q, k, v = _draw(0, 12, 20, 6)
    P, T = 2, 3
    planes = rng.standard_normal((T * P, 6))
    qi, ki = ann_hash(q, planes)[0], ann_hash(k, planes)[0]
    counts = rng.integers(1, 4, 20)
    O, lse = annsa_multi(q, qi, k, v, ki, 0.4, P, T, counts)
    for i in range(12):
        members = [j for j in range(20)
                   if any(((int(qi[i]) >> (t * P)) & 3) == ((int(ki[j]) >> (t * P)) & 3)
                          for t in range(T))]
        if not members:
            assert np.isneginf(lse[i]) and not O[i].any()
            continue
        logits = [0.4 * float(np.dot(q[i], k[j])) + math.log(counts[j]) for j in members]
        top = max(logits)
        w = [math.exp(x - top) for x in logits]
        tot = sum(w)
        ref = sum(wj * v[j] for wj, j in zip(w, members)) / tot
        np.testing.assert_allclose(O[i], ref, rtol=0, atol=1e-12)
        assert abs(lse[i] - (top + math.log(tot))) < 1e-12


def test_one_table_is_single_table_annsa():
    rng, q, k, v = _draw(1, 80, 300, 16)
    planes = rng.standard_normal((4, 16))
    qi, ki = ann_hash(q, planes)[0], ann_hash(k, planes)[0]
    O1, L1 = annsa_multi(q, qi, k, v, ki, 0.25, 4, 1, block=32)
    O0, L0 = annsa(q, qi, k, v, ki, 0.25)
    np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(L1), np.isfinite(L0))
    np.testing.assert_allclose(L1[np.isfinite(L1)], L0[np.isfinite(L0)], rtol=0, atol=1e-12)


def test_duplicate_tables_count_each_key_once():
    rng, q, k, v = _draw(2, 60, 200, 8)
    pl = rng.standard_normal((3, 8))
    planes = np.concatenate([pl, pl])                  # table 1 = table 0
    qi, ki = ann_hash(q, planes)[0], ann_hash(k, planes)[0]
    O2, L2 = annsa_multi(q, qi, k, v, ki, 0.3, 3, 2)
    O1, L1 = annsa(q, qi & 7, k, v, ki & 7, 0.3)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    fin = np.isfinite(L1)
    np.testing.assert_allclose(L2[fin], L1[fin], rtol=0, atol=1e-12)


def test_all_matching_table_is_dense_attention():
    rng, q, k, v = _draw(3, 40, 90, 8)
    planes = np.concatenate([rng.standard_normal((3, 8)), np.zeros((3, 8))])
    qi, ki = ann_hash(q, planes)[0], ann_hash(k, planes)[0]
    assert ((qi >> 3) == 7).all() and ((ki >> 3) == 7).all()   # <x, 0> = 0 -> bit 1
    O, L = annsa_multi(q, qi, k, v, ki, 0.5, 3, 2)
    S = 0.5 * q @ k.T
    np.testing.assert_allclose(O, softmax(S, axis=1) @ v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.log(np.exp(S).sum(axis=1)), rtol=0, atol=1e-12)


def test_union_search_brute_force_and_one_table():
    rng, q, k, _ = _draw(4, 30, 70, 6)
    P, T = 2, 2
    planes = rng.standard_normal((T * P, 6))
    qi, ki = ann_hash(q, planes)[0], ann_hash(k, planes)[0]
    n = 55
    best, cos, tie, near = tempcache_top1(q, qi, k, ki, n, P, T)
    fq, fk = bucket_fields(qi, P, T), bucket_fields(ki, P, T)
    for i in range(30):
        cands = [j for j in range(n) if (fq[i] == fk[j]).any()]
        if not cands:
            assert best[i] == -1 and np.isneginf(cos[i])
            continue
        cs = [float(q[i] @ k[j]) / (np.linalg.norm(q[i]) * np.linalg.norm(k[j])) for j in cands]
        a = int(np.argmax(cs))
        assert best[i] == cands[a] and abs(cos[i] - cs[a]) < 1e-12
    b1 = tempcache_top1(q, qi & 3, k, ki & 3, n)
    b2 = tempcache_top1(q, qi & 3, k, ki & 3, n, P, 1)
    np.testing.assert_array_equal(b1[0], b2[0])


@pytest.mark.parametrize("P,T", [(3, 2), (4, 4), (7, 2)])
def test_fields_are_per_table_hashes(P, T):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 16))
    planes = rng.standard_normal((T * P, 16))
    f = bucket_fields(ann_hash(x, planes)[0], P, T)
    for t in range(T):
        np.testing.assert_array_equal(f[:, t], ann_hash(x, planes[t * P:(t + 1) * P])[0])

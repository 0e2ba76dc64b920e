"""Pins of the oracle's mean-merge variant (CPU only).

The summary's Lemma 5.1 (Core Components A) states when merging keys is
exact: identical keys, values averaged, logits shifted by the group size.
That statement is itself the strongest pin, so most tests build histories in
which keys repeat exactly and compare the merged cache against the
uncompressed history attended directly:

* Lemma 5.1 closed form: attention over a history whose keys repeat equals
  attention over one slot per distinct key with the mean value and the
  ln(group size) logit shift (with one bucket and with several);
* the commit keeps that identity: chunks whose keys copy cached keys (some
  slots claimed by several tokens, over two consecutive commits) leave a
  cache whose attention equals attention over every token seen so far;
* a hand-worked commit (group mean, group size, the representative's key,
  an append);
* the variant changes only values and group sizes: slots, keys, ids,
  timestamps, dest, evicted and counts equal the replacement rule's, and the
  group sizes account for every token (sum of sizes = old sum + chunk size -
  sizes of the evicted groups);
* without claims (threshold above 1) the variant is the replacement rule
  with group sizes of one for the written slots.
"""
import numpy as np
import pytest

from oracle import ann_hash, annsa, key_counts, key_context, tempcache_commit, tempcache_update
from workloads import commit_case


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


@pytest.mark.parametrize("P", [0, 3])
def test_lemma_identical_keys_closed_form(P):
    rng = np.random.default_rng(7)
    d, G, Nq = 16, 12, 40
    keys = rng.standard_normal((G, d))
    mult = rng.integers(1, 6, G)                        # group sizes 1..5
    hist_k = np.repeat(keys, mult, axis=0)
    hist_v = rng.standard_normal((hist_k.shape[0], d))
    planes = rng.standard_normal((P, d))
    q = rng.standard_normal((Nq, d))
    qi = ann_hash(q, planes)[0]
    hk_ids = ann_hash(hist_k, planes)[0]
    o_full, lse_full = annsa(q, qi, hist_k, hist_v, hk_ids, 0.3)
    # one slot per distinct key: mean value, group size as the count
    ends = np.cumsum(mult)
    means = np.stack([hist_v[e - m:e].mean(axis=0) for e, m in zip(ends, mult)])
    o_m, lse_m = annsa(q, qi, keys, means, ann_hash(keys, planes)[0], 0.3, mult)
    np.testing.assert_allclose(o_m, o_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_m, lse_full, rtol=0, atol=1e-12)
    # without the shift the identity fails (the shift is load-bearing)
    o_nb, _ = annsa(q, qi, keys, means, ann_hash(keys, planes)[0], 0.3)
    assert np.abs(o_nb - o_full).max() > 1e-3


def _merge_cache(k, v, ids, ts, count):
    return {"k": np.asarray(k, np.float64), "v": np.asarray(v, np.float64),
            "ids": np.asarray(ids), "ts": np.asarray(ts, np.int64),
            "count": np.asarray(count, np.int64)}


@pytest.mark.parametrize("P", [0, 2])
def test_commit_preserves_uncompressed_attention(P):
    """Two consecutive commits of chunks that copy cached keys: after each,
    attention over [merged cache ; nothing] equals attention over the whole
    uncompressed token history."""
    rng = np.random.default_rng(11 + P)
    d, cap, n0, N = 8, 64, 20, 16
    planes = rng.standard_normal((P, d))
    K = np.zeros((cap, d)); V = np.zeros((cap, d))
    K[:n0] = _unit(rng, n0, d) * rng.uniform(0.5, 2.0, (n0, 1))
    V[:n0] = rng.standard_normal((n0, d))
    ids = np.zeros(cap, np.int64)
    ids[:n0] = ann_hash(K[:n0], planes)[0]
    cache = _merge_cache(K, V, ids, np.zeros(cap), np.ones(cap))
    hist_k, hist_v = [K[i] for i in range(n0)], [V[i] for i in range(n0)]
    n = n0
    probe = rng.standard_normal((30, d))
    for step in (1, 2):
        # half the chunk copies cached keys (slot 3 three times), half is new
        src = np.concatenate([[3, 3, 3], rng.integers(0, n, N // 2 - 3)])
        kc = np.concatenate([cache["k"][src], _unit(rng, N - src.size, d)])
        vc = rng.standard_normal((N, d))
        kci = ann_hash(kc, planes)[0]
        out = tempcache_update(cache, n, kc, kci, kc, vc, kci, tau=0.999, step=step, merge=True)
        assert out["matched"][:src.size].all() and not out["matched"][src.size:].any()
        assert out["counts"][4] == 0                     # room left: nothing evicted
        cache, n = out["cache"], out["n"]
        hist_k += list(kc); hist_v += list(vc)
        Hk, Hv = np.array(hist_k), np.array(hist_v)
        pi = ann_hash(probe, planes)[0]
        o_full, lse_full = annsa(probe, pi, Hk, Hv, ann_hash(Hk, planes)[0], 0.5)
        o_m, lse_m = annsa(probe, pi, cache["k"][:n], cache["v"][:n], cache["ids"][:n], 0.5,
                           cache["count"][:n])
        np.testing.assert_allclose(o_m, o_full, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse_m, lse_full, rtol=0, atol=1e-12)
        assert cache["count"][:n].sum() == len(hist_k)


def test_hand_worked_commit():
    # slot 0: key (1,0), value (2,4), group of 3; slot 1: key (0,1), value (0,0)
    cache = _merge_cache([[1, 0], [0, 1], [0, 0], [0, 0]], [[2, 4], [0, 0], [0, 0], [0, 0]],
                         [0, 0, 0, 0], [5, 5, 0, 0], [3, 1, 0, 0])
    k_cur = np.array([[1.0, 0.0], [2.0, 0.0], [-1.0, 0.0]])
    v_cur = np.array([[8.0, 0.0], [0.0, 8.0], [1.0, 1.0]])
    # tokens 0 and 1 pick slot 0 with cosine 1; token 2 has cosine -1 to it
    out = tempcache_commit(cache, 2, k_cur, v_cur, [0, 0, 0], [0, 0, 0], [1.0, 1.0, -1.0],
                           tau=0.9, step=9, merge=True)
    new = out["cache"]
    # (3 * (2,4) + (8,0) + (0,8)) / 5 = (14/5, 20/5)
    assert new["v"][0].tolist() == [14 / 5, 4.0]
    assert new["count"].tolist() == [5, 1, 1, 0]
    assert new["k"][0].tolist() == [2.0, 0.0]           # the most recent claimant
    assert new["v"][2].tolist() == [1.0, 1.0] and new["k"][2].tolist() == [-1.0, 0.0]
    assert new["ts"].tolist() == [9, 5, 9, 0]
    assert out["dest"].tolist() == [-1, 0, 2]
    assert out["counts"].tolist() == [2, 1, 1, 1, 0]
    assert out["n"] == 3


@pytest.mark.parametrize("seed", [0, 1])
def test_variant_differs_only_in_values_and_sizes(seed):
    rng = np.random.default_rng(100 + seed)
    H, N, cap, d = 1, 96, 128, 16
    c = commit_case(seed, H, N, cap, d, n_valid=[cap - 10], P=2, match_frac=0.6, pool=24, ts_span=6)
    count = rng.integers(1, 9, cap)
    cache = {"k": c["cache_k"][0], "v": c["cache_v"][0], "ids": c["cache_ids"][0],
             "ts": c["cache_ts"][0], "count": count}
    n = int(c["n_valid"][0])
    args = (cache, n, c["k_cur"][0], c["v_cur"][0], c["kcur_ids"][0], c["best"][0], c["cos"][0],
            0.95, 6)
    rep = tempcache_commit(*args)
    mer = tempcache_commit(*args, merge=True)
    assert rep["counts"][1] > 0 and rep["counts"][2] > 0 and rep["counts"][4] > 0
    for key in ("dest", "evicted", "counts", "matched"):
        np.testing.assert_array_equal(rep[key], mer[key])
    assert rep["n"] == mer["n"]
    for key in ("k", "ids", "ts"):
        np.testing.assert_array_equal(rep["cache"][key], mer["cache"][key])
    n_new = mer["n"]
    ev = mer["evicted"][mer["evicted"] >= 0]
    assert mer["cache"]["count"][:n_new].sum() == count[:n].sum() - count[ev].sum() + N
    # written slots of unmatched tokens hold exactly their token's value
    for i, j in enumerate(mer["dest"]):
        if j >= 0 and not mer["matched"][i]:
            assert mer["cache"]["count"][j] == 1
            np.testing.assert_array_equal(mer["cache"]["v"][j], c["v_cur"][0][i])
    # untouched slots keep value and size
    touched = set(int(j) for j in mer["dest"] if j >= 0)
    for j in range(n):
        if j not in touched:
            np.testing.assert_array_equal(mer["cache"]["v"][j], c["cache_v"][0][j])
            assert mer["cache"]["count"][j] == count[j]


def test_no_claims_is_replacement_with_unit_groups():
    rng = np.random.default_rng(5)
    cap, n, N, d = 40, 30, 20, 4
    K = rng.standard_normal((cap, d)); V = rng.standard_normal((cap, d))
    ids = np.zeros(cap, np.int64); ts = rng.integers(0, 4, cap)
    count = rng.integers(1, 5, cap)
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    q = rng.standard_normal((N, d))
    cache = {"k": K, "v": V, "ids": ids, "ts": ts, "count": count}
    rep = tempcache_update(cache, n, q, np.zeros(N, int), kc, vc, np.zeros(N, int), tau=1.5, step=7)
    mer = tempcache_update(cache, n, q, np.zeros(N, int), kc, vc, np.zeros(N, int), tau=1.5, step=7,
                           merge=True)
    np.testing.assert_array_equal(rep["cache"]["v"], mer["cache"]["v"])
    written = rep["dest"]
    assert (mer["cache"]["count"][written] == 1).all()
    keep = np.setdiff1d(np.arange(cap), written)
    np.testing.assert_array_equal(mer["cache"]["count"][keep], count[keep])


def test_key_counts_layout():
    assert key_counts(np.array([4, 2, 7, 9]), 3, 2).tolist() == [4, 2, 7, 1, 1]
    K, V, kid = key_context(np.ones((4, 2)), np.ones((4, 2)), np.arange(4), 3, np.zeros((2, 2)),
                            np.zeros((2, 2)), [5, 6])
    assert K.shape[0] == key_counts(np.ones(4), 3, 2).size

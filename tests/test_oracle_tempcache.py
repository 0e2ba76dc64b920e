"""Pins of the oracle's TempCache (CPU only).

* hand-worked fixture: top-1, claims, drops, appends and timestamp eviction;
* threshold above 1 with room: the update is plain concatenation;
* threshold above 1 on a full frame-major cache: a FIFO rolling window;
* threshold -2 with one bucket: the top-1 is the global cosine argmax
  (scipy's cdist, a library routine);
* queries that are positive multiples of distinct cached keys: best = that
  slot, cosine = 1 (closed form);
* invariants on the tiny workload: the cache never exceeds its cap, dest is
  injective, refreshed slots are never evicted, evicted slots are the oldest,
  written rows are the current tokens and nothing else changed;
* eviction candidates: a hand-worked fixture, numpy's lexsort (a library
  routine) on tied timestamps, and the evicted slots of random updates always
  among them -- including the tight case where refreshed slots are the oldest
  and the last evicted slot is the N-th in (timestamp, slot) order.
"""
import json
import os

import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import ann_hash, eviction_candidates, tempcache_commit, tempcache_top1, tempcache_update
from tests.conftest import GOLDEN
from workloads import CONFIGS, make_step


def _cache(k, v, ids, ts):
    return {"k": np.asarray(k, np.float64), "v": np.asarray(v, np.float64),
            "ids": np.asarray(ids), "ts": np.asarray(ts, np.int64)}


def test_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "tempcache_hand.json")))
    K = np.array(fx["cache_k"])
    q = np.array(fx["q"])
    best, cos, tie, _ = tempcache_top1(q, np.zeros(4, int), K, np.zeros(4, int), 3)
    assert best.tolist() == fx["top1"]["best"]
    np.testing.assert_allclose(cos, fx["top1"]["cos"], rtol=0, atol=1e-15)
    assert tie.tolist() == fx["top1"]["argmax_tie"]
    kc, vc = np.array(fx["k_cur"]), np.array(fx["v_cur"])
    for case in fx["cases"]:
        cap = case["cap"]
        toks = case.get("tokens", list(range(4)))
        cache = _cache(K[:cap], np.zeros((cap, 2)), np.zeros(cap, int), case["ts"])
        out = tempcache_update(cache, case["n"], q[toks], np.zeros(len(toks), int), kc[toks],
                               vc[toks], np.zeros(len(toks), int), case["tau"], fx["step"])
        assert out["dest"].tolist() == case["dest"], case["name"]
        assert out["evicted"].tolist() == case["evicted"][:len(toks)], case["name"]
        assert out["counts"].tolist() == case["counts"], case["name"]
        assert out["n"] == case["n_new"], case["name"]
        assert out["cache"]["ts"].tolist() == case["new_ts"], case["name"]
        for i, j in zip(toks, out["dest"]):
            if j >= 0:
                assert out["cache"]["k"][j].tolist() == kc[i].tolist()
                assert out["cache"]["v"][j].tolist() == vc[i].tolist()


def test_no_match_with_room_is_concatenation():
    rng = np.random.default_rng(0)
    cap, n, N, d = 100, 37, 50, 8
    K = rng.standard_normal((cap, d)); V = rng.standard_normal((cap, d))
    ids = rng.integers(0, 4, cap); ts = rng.integers(0, 5, cap)
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    kci = rng.integers(0, 4, N)
    out = tempcache_update(_cache(K, V, ids, ts), n, rng.standard_normal((N, d)),
                           rng.integers(0, 4, N), kc, vc, kci, tau=1.5, step=9)
    assert out["n"] == n + N
    assert out["dest"].tolist() == list(range(n, n + N))
    assert out["counts"].tolist() == [0, 0, 0, N, 0]
    new = out["cache"]
    np.testing.assert_array_equal(new["k"][:n + N], np.concatenate([K[:n], kc]))
    np.testing.assert_array_equal(new["v"][:n + N], np.concatenate([V[:n], vc]))
    np.testing.assert_array_equal(new["ids"][:n + N], np.concatenate([ids[:n], kci]))
    np.testing.assert_array_equal(new["ts"][:n + N], np.concatenate([ts[:n], np.full(N, 9)]))


def test_no_match_full_cache_is_rolling_window():
    rng = np.random.default_rng(1)
    fl, frames, d = 16, 5, 4
    cap = fl * frames
    K = rng.standard_normal((cap, d)); V = rng.standard_normal((cap, d))
    ts = np.repeat(np.arange(frames), fl)
    cache = _cache(K, V, np.zeros(cap, int), ts)
    n = cap
    for step in range(frames, frames + 7):
        kc, vc = rng.standard_normal((fl, d)), rng.standard_normal((fl, d))
        out = tempcache_update(cache, n, kc, np.zeros(fl, int), kc, vc, np.zeros(fl, int),
                               tau=2.0, step=step)
        oldest = step - frames
        slots = np.nonzero(cache["ts"] == oldest)[0]
        assert out["evicted"].tolist() == slots.tolist()
        assert out["dest"].tolist() == slots.tolist()
        cache, n = out["cache"], out["n"]
        assert n == cap
        assert sorted(set(cache["ts"].tolist())) == list(range(step - frames + 1, step + 1))


def test_global_argmax_with_one_bucket():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((300, 12))
    q = rng.standard_normal((60, 12))
    best, cos, _, _ = tempcache_top1(q, np.zeros(60, int), K, np.zeros(300, int), 250)
    sim = 1 - cdist(q, K[:250], metric="cosine")
    assert (best == sim.argmax(1)).all()
    np.testing.assert_allclose(cos, sim.max(1), atol=1e-12)
    out = tempcache_commit(_cache(K, K, np.zeros(300, int), np.zeros(300, int)), 250, q, q,
                           np.zeros(60, int), best, cos, tau=-2.0, step=1)
    assert out["matched"].all()


def test_copies_of_cached_keys_match_exactly():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((64, 16))
    ids, _ = ann_hash(K, rng.standard_normal((3, 16)))
    pick = rng.choice(64, 20, replace=False)
    q = K[pick] * rng.uniform(0.5, 4.0, (20, 1))
    best, cos, _, _ = tempcache_top1(q, ids[pick], K, ids, 64)
    assert (best == pick).all()
    np.testing.assert_allclose(cos, 1.0, atol=1e-14)


def test_no_candidates_and_out_of_range_best():
    K = np.eye(4)
    best, cos, _, _ = tempcache_top1(np.ones((2, 4)), [1, 2], K, [0, 0, 0, 0], 4)
    assert best.tolist() == [-1, -1] and np.isneginf(cos).all()
    cache = _cache(K, K, np.zeros(4, int), np.zeros(4, int))
    out = tempcache_commit(cache, 2, np.ones((2, 4)), np.ones((2, 4)), [0, 0],
                           np.array([3, -1]), np.array([1.0, 1.0]), 0.5, 1)
    assert out["counts"].tolist() == [0, 0, 0, 2, 0]          # slot 3 is not valid (n=2)
    with pytest.raises(ValueError):
        tempcache_commit(cache, 2, np.ones((5, 4)), np.ones((5, 4)), [0] * 5,
                         np.full(5, -1), np.zeros(5), 0.5, 1)


def _check_invariants(cache, n, out, kc, vc, kci, step):
    cap = cache["k"].shape[0]
    new = out["cache"]
    dest = out["dest"]
    assert out["n"] <= cap
    written = dest[dest >= 0]
    assert len(set(written.tolist())) == written.size
    ev = out["evicted"][out["evicted"] >= 0]
    refreshed = set(dest[(dest >= 0) & (dest < n) & out["matched"]].tolist())
    assert not (set(ev.tolist()) & refreshed)
    survivors = [j for j in range(n) if j not in refreshed and j not in set(ev.tolist())]
    for e in ev:
        for j in survivors:
            assert (cache["ts"][e], e) < (cache["ts"][j], j)
    for i, j in enumerate(dest):
        if j >= 0:
            assert (new["k"][j] == kc[i]).all() and (new["v"][j] == vc[i]).all()
            assert new["ids"][j] == kci[i] and new["ts"][j] == step
    untouched = np.setdiff1d(np.arange(cap), written)
    assert (new["k"][untouched] == cache["k"][untouched]).all()
    assert (new["ts"][untouched] == cache["ts"][untouched]).all()
    c = out["counts"]
    assert c[0] == out["matched"].sum() and c[1] + c[2] == c[0]
    assert c[3] + c[4] == (~out["matched"]).sum()
    assert (dest == -1).sum() == c[2]


@pytest.mark.parametrize("tau,cap_extra", [(0.9, 0), (0.95, 0), (0.8, 300), (0.99, 100)])
def test_invariants_on_tiny_workload(tau, cap_extra):
    cfg = CONFIGS["tiny_f32"]
    st = make_step(cfg, seed=0)
    cap = cfg.cap + cap_extra
    K = np.zeros((cap, cfg.d)); V = np.zeros((cap, cfg.d)); ts = np.zeros(cap, np.int64)
    K[:cfg.cap] = st.cache_k[0]; V[:cfg.cap] = st.cache_v[0]; ts[:cfg.cap] = st.cache_ts[0]
    ids = np.zeros(cap, np.int64)
    ids[:cfg.cap], _ = ann_hash(st.cache_k[0], st.planes[0])
    qi, _ = ann_hash(st.q[0], st.planes[0])
    ki, _ = ann_hash(st.k_cur[0], st.planes[0])
    cache = _cache(K, V, ids, ts)
    n = int(st.n_valid[0])
    out = tempcache_update(cache, n, st.q[0], qi, st.k_cur[0], st.v_cur[0], ki, tau, st.step)
    _check_invariants(cache, n, out, st.k_cur[0], st.v_cur[0], ki, st.step)
    assert 0 < out["counts"][0] < cfg.Nq


def test_eviction_candidates_hand_fixture():
    ts = [5, 3, 3, 9, 1, 3]
    # (ts, slot) order: 4, 1, 2, 5, 0, 3
    assert eviction_candidates(ts, 6, 3).tolist() == [1, 2, 4]
    assert eviction_candidates(ts, 4, 3).tolist() == [0, 1, 2]          # slots 4, 5 not valid
    assert eviction_candidates(ts, 6, 8).tolist() == [0, 1, 2, 3, 4, 5, -1, -1]
    assert eviction_candidates(ts, 0, 2).tolist() == [-1, -1]
    assert eviction_candidates(ts, 6, 0).tolist() == []


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_eviction_candidates_by_lexsort(seed):
    rng = np.random.default_rng(seed)
    cap = 500
    ts = rng.integers(0, 20, cap)                     # many equal timestamps
    for n, N in ((cap, 37), (cap, cap), (300, 120), (300, 400)):
        order = np.lexsort((np.arange(n), ts[:n]))    # by ts, then slot
        m = min(n, N)
        got = eviction_candidates(ts, n, N)
        assert got[:m].tolist() == sorted(order[:m].tolist())
        assert (got[m:] == -1).all()


def _random_commit(rng, cap, n, N, match_frac):
    d = 4
    cache = _cache(rng.standard_normal((cap, d)), rng.standard_normal((cap, d)),
                   rng.integers(0, 4, cap), rng.integers(0, 6, cap))
    best = rng.integers(0, max(n, 1), N)
    cos = np.where(rng.random(N) < match_frac, 1.0, 0.0)
    kc, vc = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    out = tempcache_commit(cache, n, kc, vc, rng.integers(0, 4, N), best, cos, 0.5, 99)
    return cache, out


@pytest.mark.parametrize("seed", range(6))
def test_evictions_lie_in_candidates(seed):
    rng = np.random.default_rng(seed)
    cap = 60
    for n, N, frac in ((60, 20, 0.3), (60, 60, 0.5), (55, 12, 0.0), (50, 30, 0.9), (60, 1, 0.0)):
        cache, out = _random_commit(rng, cap, n, N, frac)
        cand = set(eviction_candidates(cache["ts"], n, N).tolist()) - {-1}
        ev = out["evicted"][out["evicted"] >= 0]
        assert set(ev.tolist()) <= cand


def test_eviction_candidates_bound_is_tight():
    # the 3 oldest slots are refreshed and 5 tokens are unmatched: the evicted
    # slots are the 4th..8th oldest, the last of them the N-th (N = 8)
    cap, N = 20, 8
    ts = np.arange(cap)[::-1].copy()                  # slot 19 oldest, then 18, ...
    cache = _cache(np.eye(cap, 4), np.zeros((cap, 4)), np.zeros(cap), ts)
    best = np.array([19, 18, 17, 0, 0, 0, 0, 0])
    cos = np.array([1.0, 1.0, 1.0, 0, 0, 0, 0, 0])
    out = tempcache_commit(cache, cap, np.ones((N, 4)), np.ones((N, 4)), np.zeros(N), best, cos, 0.5, 50)
    assert out["counts"][1] == 3 and out["counts"][4] == 5
    assert out["evicted"][:5].tolist() == [12, 13, 14, 15, 16]
    cand = eviction_candidates(ts, cap, N)
    assert cand.tolist() == list(range(12, 20))
    assert 12 in cand and 12 not in eviction_candidates(ts, cap, N - 1)

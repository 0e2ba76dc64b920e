"""Pins of the oracle's whole step, ``attention_step`` (CPU only).

``attention_step`` wires the stages together per head: hash Q, the current
keys and the prompt keys with the head's planes; AnnSA over [valid cache
slots ; current chunk]; AnnCA per frame; TempCache top-1 + commit (with the
group sizes when the cache is mean-merged).  The stages are pinned on their
own elsewhere; these tests pin the wiring, where a wrong ``n``, a swapped id
set, a wrong ``frame_len`` or a wrong group-size vector would go unnoticed:

* brute force: every output recomputed from the definitions with plain
  Python loops over (query, key) pairs -- a sign loop per plane for the ids,
  an explicit key-context list, a softmax per query, a membership loop for
  AnnCA's keep mask, a slot loop for the top-1 -- on two heads, one with a
  partly filled cache (n < cap) and one full, three frames per chunk, with
  and without group sizes;
* the textbook special case (blog, "3. AnnSA" and "1. TempCache"): with no
  planes (one bucket) and a threshold above 1, AnnSA is dense softmax
  attention over [cache ; chunk] (torch's scaled_dot_product_attention in
  fp64), AnnCA is full cross-attention, and the commit is a plain append;
* Lemma 5.1 (summary, Core Components A): for a mean-merged cache of
  identical keys, the step's AnnSA output equals attention over the expanded
  history in which every slot is repeated as many times as its group size;
* the ``heads`` selection returns exactly the selected heads' results.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_step

H, D, P, FRAME, F, CAP, L = 2, 8, 3, 8, 3, 40, 10
N = FRAME * F
N_VALID = (CAP, 27)                 # one full head, one partly filled head
TAU, STEP = 0.5, 7


def _case(seed: int, merge: bool):
    """Two heads: cached keys near a few centroids, current keys copying some
    cached keys with a little noise (so the threshold splits matched from
    unmatched tokens), queries near the current keys."""
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((H, 5, D))
    cache_k = np.stack([mu[h][rng.integers(0, 5, CAP)] + 0.6 * rng.standard_normal((CAP, D))
                        for h in range(H)])
    cache_v = rng.standard_normal((H, CAP, D))
    src = rng.integers(0, 27, (H, N))               # copy among the slots both heads hold
    k_cur = np.stack([cache_k[h][src[h]] + 0.5 * rng.standard_normal((N, D)) for h in range(H)])
    v_cur = rng.standard_normal((H, N, D))
    q = k_cur + 0.3 * rng.standard_normal((H, N, D))
    planes = rng.standard_normal((H, P, D))
    kp = np.stack([mu[h][rng.integers(0, 5, L)] + rng.standard_normal((L, D)) for h in range(H)])
    vp = rng.standard_normal((H, L, D))
    cache_ts = rng.integers(0, 5, (H, CAP)).astype(np.int64)
    cache_ids = np.stack([[_bucket(cache_k[h][j], planes[h]) for j in range(CAP)] for h in range(H)])
    count = rng.integers(1, 5, (H, CAP)) if merge else None
    return dict(q=q, k_cur=k_cur, v_cur=v_cur, cache_k=cache_k, cache_v=cache_v,
                cache_ids=cache_ids.astype(np.uint16), cache_ts=cache_ts,
                n_valid=np.array(N_VALID), planes=planes, kp=kp, vp=vp, count=count)


def _dot(a, b) -> float:
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def _bucket(x, planes) -> int:
    return sum(1 << p for p in range(len(planes)) if _dot(x, planes[p]) >= 0.0)


def _softmax_attend(qv, keys, scale):
    """keys: list of (k, v, log group size); returns (O, lse)."""
    if not keys:
        return np.zeros(D), -math.inf
    logits = [scale * _dot(qv, k) + b for k, _, b in keys]
    m = max(logits)
    w = [math.exp(l - m) for l in logits]
    s = math.fsum(w)
    O = np.array([math.fsum(wj * float(v[c]) for wj, (_, v, _) in zip(w, keys)) for c in range(D)]) / s
    return O, m + math.log(s)


def _run(c, **kw):
    return attention_step(c["q"], c["k_cur"], c["v_cur"], c["cache_k"], c["cache_v"], c["cache_ids"],
                          c["cache_ts"], c["n_valid"], c["planes"], c["kp"], c["vp"], FRAME, TAU, STEP,
                          cache_count=c["count"], **kw)


@pytest.mark.parametrize("merge", [False, True])
def test_step_matches_brute_force(merge):
    c = _case(3, merge)
    r = _run(c)
    scale = 1.0 / math.sqrt(D)
    assert r["H"] == H
    for h in range(H):
        n = int(c["n_valid"][h])
        pl = c["planes"][h]
        qid = [_bucket(x, pl) for x in c["q"][h]]
        kid = [_bucket(x, pl) for x in c["k_cur"][h]]
        pid = [_bucket(x, pl) for x in c["kp"][h]]
        assert r["q_ids"][h].tolist() == qid
        assert r["kcur_ids"][h].tolist() == kid
        assert r["kp_ids"][h].tolist() == pid
        # AnnSA: the valid slots (with their group-size shift), then the chunk
        ctx = [(c["cache_k"][h][j], c["cache_v"][h][j], int(c["cache_ids"][h][j]),
                math.log(c["count"][h][j]) if merge else 0.0) for j in range(n)]
        ctx += [(c["k_cur"][h][t], c["v_cur"][h][t], kid[t], 0.0) for t in range(N)]
        for i in range(N):
            O, lse = _softmax_attend(c["q"][h][i], [(k, v, b) for k, v, id_, b in ctx if id_ == qid[i]],
                                     scale)
            np.testing.assert_allclose(r["o_sa"][h][i], O, rtol=0, atol=1e-12)
            assert (math.isinf(lse) and math.isinf(r["lse"][h][i])) or abs(r["lse"][h][i] - lse) < 1e-12
        # AnnCA: per frame, the prompt tokens whose bucket a query of the frame holds
        for f in range(F):
            present = set(qid[f * FRAME:(f + 1) * FRAME])
            kept = [t for t in range(L) if pid[t] in present]
            assert r["keep"][h][f].tolist() == [t in kept for t in range(L)]
            for i in range(f * FRAME, (f + 1) * FRAME):
                O, _ = _softmax_attend(c["q"][h][i], [(c["kp"][h][t], c["vp"][h][t], 0.0) for t in kept],
                                       scale)
                np.testing.assert_allclose(r["o_ca"][h][i], O, rtol=0, atol=1e-12)
        # TempCache: top-1 over the valid slots of the query's bucket, then the commit
        tc = r["tc"][h]
        for i in range(N):
            best, bc = -1, -math.inf
            for j in range(n):
                if int(c["cache_ids"][h][j]) != qid[i]:
                    continue
                k = c["cache_k"][h][j]
                cs = _dot(c["q"][h][i], k) / math.sqrt(_dot(c["q"][h][i], c["q"][h][i]) * _dot(k, k))
                if cs > bc:
                    best, bc = j, cs
            assert tc["best"][i] == best
            if best >= 0:
                assert abs(tc["cos"][i] - bc) < 1e-12
            assert tc["matched"][i] == (best >= 0 and bc >= TAU)
        _check_commit(c, h, n, kid, tc, merge)


def _check_commit(c, h, n, kid, tc, merge):
    matched = tc["matched"]
    best = tc["best"]
    winners = {}
    for i in range(N):
        if matched[i]:
            winners[int(best[i])] = max(winners.get(int(best[i]), -1), i)
    unmatched = [i for i in range(N) if not matched[i]]
    e = max(0, n + len(unmatched) - CAP)
    ts = c["cache_ts"][h]
    pool = sorted((int(ts[j]), j) for j in range(n) if j not in winners)
    evicted = sorted(j for _, j in pool[:e])
    free = list(range(n, min(CAP, n + len(unmatched)))) + evicted
    dest = [-1] * N
    for j, i in winners.items():
        dest[i] = j
    for slot, i in zip(free, unmatched):
        dest[i] = slot
    assert tc["dest"].tolist() == dest
    assert tc["n"] == min(CAP, n + len(unmatched)) <= CAP
    assert tc["evicted"][:e].tolist() == evicted and (tc["evicted"][e:] == -1).all()
    assert tc["counts"].tolist() == [int(matched.sum()), len(winners), int(matched.sum()) - len(winners),
                                     tc["n"] - n, e]
    new = tc["cache"]
    for i in range(N):
        if dest[i] >= 0:
            assert np.array_equal(new["k"][dest[i]], c["k_cur"][h][i])
            assert new["ids"][dest[i]] == kid[i] and new["ts"][dest[i]] == STEP
    untouched = [j for j in range(CAP) if j not in set(dest)]
    assert np.array_equal(new["k"][untouched], c["cache_k"][h][untouched])
    assert np.array_equal(new["ts"][untouched], c["cache_ts"][h][untouched])
    for i in range(N):
        j = dest[i]
        if j < 0:
            continue
        if not merge or not matched[i]:
            np.testing.assert_allclose(new["v"][j], c["v_cur"][h][i], rtol=0, atol=0)
            if merge:
                assert new["count"][j] == 1
        else:
            members = [t for t in range(N) if matched[t] and int(best[t]) == j]
            m = int(c["count"][h][j])
            mean = (m * c["cache_v"][h][j] + sum(c["v_cur"][h][t] for t in members)) / (m + len(members))
            np.testing.assert_allclose(new["v"][j], mean, rtol=0, atol=1e-12)
            assert new["count"][j] == m + len(members)
    # the brute-force case really exercises every branch
    assert len(winners) > 0 and len(unmatched) > 0
    assert int(matched.sum()) > len(winners)          # some claimants dropped or merged


def test_step_branches_covered():
    """The brute-force case has an eviction on the full head and an append on
    the partial one (so both sides of the capacity rule run)."""
    r = _run(_case(3, False))
    assert r["tc"][0]["counts"][4] > 0 and r["tc"][0]["n"] == CAP
    assert r["tc"][1]["counts"][3] > 0 and r["tc"][1]["n"] > N_VALID[1]


def _sdpa(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))[None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)[0].numpy()


def test_step_one_bucket_and_no_match_is_dense_attention_and_append():
    c = _case(5, False)
    c["planes"] = np.zeros((H, 0, D))
    c["cache_ids"] = np.zeros((H, CAP), np.uint16)
    cap_big = 2 * CAP                                  # room to append the whole chunk
    pad = lambda a: np.concatenate([a, np.zeros((H, CAP) + a.shape[2:], a.dtype)], axis=1)
    for key in ("cache_k", "cache_v", "cache_ids", "cache_ts"):
        c[key] = pad(c[key])
    r = attention_step(c["q"], c["k_cur"], c["v_cur"], c["cache_k"], c["cache_v"], c["cache_ids"],
                       c["cache_ts"], c["n_valid"], c["planes"], c["kp"], c["vp"], FRAME, 1.5, STEP)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        n = int(c["n_valid"][h])
        K = np.concatenate([c["cache_k"][h][:n], c["k_cur"][h]])
        V = np.concatenate([c["cache_v"][h][:n], c["v_cur"][h]])
        np.testing.assert_allclose(r["o_sa"][h], _sdpa(c["q"][h], K, V, scale), rtol=0, atol=1e-12)
        lse = torch.logsumexp(torch.from_numpy(c["q"][h] @ K.T * scale), dim=1).numpy()
        np.testing.assert_allclose(r["lse"][h], lse, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["o_ca"][h], _sdpa(c["q"][h], c["kp"][h], c["vp"][h], scale),
                                   rtol=0, atol=1e-12)
        assert r["keep"][h].all()
        tc = r["tc"][h]
        assert tc["n"] == n + N and tc["dest"].tolist() == list(range(n, n + N))
        assert tc["counts"].tolist() == [0, 0, 0, N, 0]
        assert np.array_equal(tc["cache"]["k"][:n + N], np.concatenate([c["cache_k"][h][:n], c["k_cur"][h]]))
        assert np.array_equal(tc["cache"]["v"][:n + N], np.concatenate([c["cache_v"][h][:n], c["v_cur"][h]]))
        assert (tc["cache"]["ts"][n:n + N] == STEP).all()


def test_step_mean_merged_cache_equals_expanded_history():
    """Lemma 5.1: a slot of group size m with the group's mean value attends
    like m copies of its key carrying the group's individual values."""
    c = _case(9, True)
    rng = np.random.default_rng(11)
    r = _run(c)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        n = int(c["n_valid"][h])
        qid, kid = r["q_ids"][h], r["kcur_ids"][h]
        # expanded history: slot j -> m_j copies of k_j whose values average to v_j
        ks, vs, ids = [], [], []
        for j in range(n):
            m = int(c["count"][h][j])
            dev = rng.standard_normal((m, D))
            dev -= dev.mean(axis=0)
            ks.append(np.repeat(c["cache_k"][h][j][None], m, 0))
            vs.append(c["cache_v"][h][j][None] + dev)
            ids += [int(c["cache_ids"][h][j])] * m
        K = np.concatenate(ks + [c["k_cur"][h]])
        V = np.concatenate(vs + [c["v_cur"][h]])
        kids = np.array(ids + kid.tolist())
        for b in np.unique(qid):
            qi = np.nonzero(qid == b)[0]
            kj = np.nonzero(kids == b)[0]
            if kj.size == 0:
                assert (r["o_sa"][h][qi] == 0).all()
                continue
            np.testing.assert_allclose(r["o_sa"][h][qi], _sdpa(c["q"][h][qi], K[kj], V[kj], scale),
                                       rtol=0, atol=1e-12)


def test_step_head_selection():
    c = _case(3, False)
    full = _run(c)
    one = _run(c, heads=[1])
    assert one["H"] == 1
    np.testing.assert_array_equal(one["o_sa"][0], full["o_sa"][1])
    np.testing.assert_array_equal(one["tc"][0]["dest"], full["tc"][1]["dest"])

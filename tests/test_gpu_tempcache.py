"""GPU parity of fastar_tempcache_update against the oracle.

* top-1 search: best slot exact except where the oracle flags an argmax
  near-tie (then the GPU's slot must be one of the near-maximal ones), cosine
  within tolerance, match decisions exact except near the threshold;
* commit: with the oracle's (best, cos) passed in as best_in/cos_in (cos
  rounded to fp32 on both sides, so the threshold test is taken in the same
  precision), dest, evicted, counts, n_valid and every cache array must be
  bit-exact -- full cache, partial cache, nothing matched (FIFO), everything
  matched, and scattered timestamps (multi-pass radix select);
* the same commits with the eviction candidates listed beforehand
  (fastar_tempcache_order, checked against the oracle's
  ``eviction_candidates``) and passed as order_in: the same bit-exact results;
* the full GPU path's commit must satisfy the cache invariants;
* a multi-chunk rollout stays bit-identical to the oracle's.
"""
import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import eviction_candidates, tempcache_commit, tempcache_top1
from tests.gpu_util import COS_ABS, dev, dev_ids, device_cache, host_ids, prepared, require_gpu
from workloads import rollout_chunks

pytestmark = pytest.mark.gpu


def oracle_top1(prep, n):
    st, cfg = prep["step"], prep["cfg"]
    res = [tempcache_top1(st.q[h], prep["q_ids"][h], st.cache_k[h], prep["cache_ids"][h], n)
           for h in range(cfg.H)]
    return res


def call(prep, cache, tau, best_in=None, cos_in=None, step=None, order_in=None):
    st, cfg = prep["step"], prep["cfg"]
    return fa.tempcache_update(cache, dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]),
                               dev(st.k_cur, cfg.dtype), dev(st.v_cur, cfg.dtype),
                               dev_ids(prep["k_cur_ids"]), cfg.P, tau,
                               st.step if step is None else step,
                               best_in=best_in, cos_in=cos_in, order_in=order_in)


def checked_order(cache, N, ts, n_valid):
    """fastar_tempcache_order on ``cache``, compared with the oracle."""
    order = fa.tempcache_order(cache, N)
    got = order.cpu().numpy()
    for h in range(got.shape[0]):
        assert np.array_equal(got[h], eviction_candidates(ts[h], int(n_valid[h]), N)), f"order head {h}"
    return order


def cache_host(cache, dtype):
    f = (lambda t: t.float().cpu().numpy()) if dtype == "bf16" else (lambda t: t.cpu().numpy())
    return {"k": f(cache.k), "v": f(cache.v), "ids": host_ids(cache.ids),
            "ts": cache.ts.cpu().numpy(), "n": cache.n_valid.cpu().numpy()}


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_top1_matches_oracle(name):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    res = call(prep, device_cache(prep), cfg.tau)
    best = res["best"].cpu().numpy()
    cos = res["cos"].cpu().numpy().astype(np.float64)
    ties = 0
    for h, (ob, oc, tie, near) in enumerate(oracle_top1(prep, cfg.n0)):
        ok = ~tie
        assert np.array_equal(best[h][ok], ob[ok]), f"head {h}"
        for i in np.nonzero(tie)[0]:
            assert best[h][i] in near[i]
        ties += int(tie.sum())
        fin = np.isfinite(oc)
        assert np.array_equal(np.isfinite(cos[h]), fin)
        assert np.abs(cos[h][fin] - oc[fin]).max() <= COS_ABS
        thr = np.abs(oc - cfg.tau) < 1e-5
        m_gpu = (best[h] >= 0) & (cos[h] >= np.float32(cfg.tau))
        m_ref = (ob >= 0) & (oc >= cfg.tau)
        assert np.array_equal(m_gpu[~thr], m_ref[~thr])
    print(f"top1 {name}: {ties} argmax near-ties (validated)")


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_fused_search_in_annsa_matches_oracle(name):
    """annsa_forward's search output (TempCache's top-1 from the attention pass)
    against the oracle's top-1; the attention output is unchanged by it."""
    require_gpu()
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    cache = device_cache(prep)
    args = (dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
            dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]), cfg.P)
    out, lse, best_t, cos_t = fa.annsa_forward(*args, cache=cache, search=True)
    out0, lse0 = fa.annsa_forward(*args, cache=cache)
    assert torch.equal(out, out0) and torch.equal(lse, lse0)
    best = best_t.cpu().numpy()
    cos = cos_t.cpu().numpy().astype(np.float64)
    for h, (ob, oc, tie, near) in enumerate(oracle_top1(prep, cfg.n0)):
        ok = ~tie
        assert np.array_equal(best[h][ok], ob[ok]), f"head {h}"
        for i in np.nonzero(tie)[0]:
            assert best[h][i] in near[i]
        fin = np.isfinite(oc)
        assert np.array_equal(np.isfinite(cos[h]), fin)
        assert np.abs(cos[h][fin] - oc[fin]).max() <= COS_ABS


def test_commit_keeps_key_norms():
    """After a commit every valid slot's knorm is the norm of the key it holds."""
    require_gpu()
    prep = prepared("single_bf16")
    cfg = prep["cfg"]
    cache = device_cache(prep)
    call(prep, cache, cfg.tau)
    k = cache.k.float().cpu().numpy().astype(np.float64)
    n = int(cache.n_valid[0])
    np.testing.assert_allclose(cache.knorm.cpu().numpy()[0, :n], np.linalg.norm(k[0, :n], axis=1),
                               rtol=2e-6, atol=0)


def _commit_case(prep, cache_dev, n, tau, ts=None, step=None, ordered=False):
    st, cfg = prep["step"], prep["cfg"]
    step = st.step if step is None else step
    tops = oracle_top1(prep, n)
    best = np.stack([t[0] for t in tops]).astype(np.int32)
    cos32 = np.stack([t[1] for t in tops]).astype(np.float32)
    ts0 = st.cache_ts if ts is None else ts
    order = checked_order(cache_dev, cfg.Nq, ts0, [n] * cfg.H) if ordered else None
    res = call(prep, cache_dev, tau, best_in=torch.from_numpy(best).cuda(),
               cos_in=torch.from_numpy(cos32).cuda(), step=step, order_in=order)
    got = cache_host(cache_dev, cfg.dtype)
    tau32 = float(np.float32(tau))
    for h in range(cfg.H):
        ref = tempcache_commit({"k": st.cache_k[h], "v": st.cache_v[h], "ids": prep["cache_ids"][h],
                                "ts": ts0[h]}, n, st.k_cur[h], st.v_cur[h], prep["k_cur_ids"][h],
                               best[h], cos32[h].astype(np.float64), tau32, step)
        assert np.array_equal(res["dest"][h].cpu().numpy(), ref["dest"]), f"dest head {h}"
        assert np.array_equal(res["evicted"][h].cpu().numpy(), ref["evicted"]), f"evicted head {h}"
        assert np.array_equal(res["counts"][h].cpu().numpy(), ref["counts"]), f"counts head {h}"
        assert got["n"][h] == ref["n"]
        assert np.array_equal(got["k"][h], ref["cache"]["k"].astype(np.float32)), f"k head {h}"
        assert np.array_equal(got["v"][h], ref["cache"]["v"].astype(np.float32)), f"v head {h}"
        assert np.array_equal(got["ids"][h], ref["cache"]["ids"]), f"ids head {h}"
        assert np.array_equal(got["ts"][h], ref["cache"]["ts"]), f"ts head {h}"
    return res


@pytest.mark.parametrize("ordered", [False, True])
@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_commit_bit_exact_full_cache(name, ordered):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    res = _commit_case(prep, device_cache(prep), cfg.n0, cfg.tau, ordered=ordered)
    assert (res["counts"][:, 4] > 0).all()          # the full cache evicted


@pytest.mark.parametrize("ordered", [False, True])
@pytest.mark.parametrize("tau", [2.0, -2.0, 0.97])
def test_commit_bit_exact_partial_cache(tau, ordered):
    require_gpu()
    prep = prepared("single_bf16")
    n = prep["cfg"].cap - 1000
    _commit_case(prep, device_cache(prep, n=n), n, tau, ordered=ordered)


@pytest.mark.parametrize("ordered", [False, True])
def test_commit_scattered_timestamps(ordered):
    require_gpu()
    prep = prepared("single_bf16")
    cfg = prep["cfg"]
    rng = np.random.default_rng(3)
    ts = rng.integers(-70000, 70000, size=prep["step"].cache_ts.shape).astype(np.int32)
    ts[:, ::7] = ts[:, 5:6]                      # many equal timestamps
    cache = device_cache(prep)
    cache.ts.copy_(torch.from_numpy(ts).cuda())
    _commit_case(prep, cache, cfg.n0, 2.0, ts=ts, step=100000, ordered=ordered)


def test_order_of_small_caches():
    """n below N (every valid slot listed, then -1) and an empty cache."""
    require_gpu()
    prep = prepared("tiny_f32")
    cfg = prep["cfg"]
    for n in (0, 5, cfg.Nq - 1, cfg.Nq):
        if n > cfg.cap:
            continue
        cache = device_cache(prep, n=n)
        checked_order(cache, cfg.Nq, prep["step"].cache_ts, [n] * cfg.H)


def _check_invariants(old, new, res, N, cap):
    dest = res["dest"].cpu().numpy()
    ev = res["evicted"].cpu().numpy()
    counts = res["counts"].cpu().numpy()
    for h in range(dest.shape[0]):
        d = dest[h]
        n0 = old["n"][h]
        assert new["n"][h] <= cap
        assert new["n"][h] == n0 + counts[h][3]
        w = d[d >= 0]
        assert len(np.unique(w)) == w.size
        e = ev[h][ev[h] >= 0]
        assert e.size == counts[h][4] and np.all(np.diff(e) > 0)
        refreshed = set(d[(d >= 0) & (d < n0)].tolist()) - set(e.tolist())
        survivors = np.setdiff1d(np.arange(n0), np.concatenate([e, np.array(sorted(refreshed), int)]))
        if e.size and survivors.size:
            key = lambda j: (int(old["ts"][h][j]), int(j))
            assert max(key(j) for j in e) < min(key(j) for j in survivors)
        untouched = np.setdiff1d(np.arange(cap), w)
        assert np.array_equal(new["k"][h][untouched], old["k"][h][untouched])
        assert np.array_equal(new["ts"][h][untouched], old["ts"][h][untouched])
        assert counts[h][0] == counts[h][1] + counts[h][2]
        assert counts[h][3] + counts[h][4] == N - counts[h][0]


@pytest.mark.parametrize("name", ["single_bf16", "wan13_bf16"])
def test_full_gpu_update_invariants_and_determinism(name):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    c1 = device_cache(prep)
    old = cache_host(c1, cfg.dtype)
    r1 = call(prep, c1, cfg.tau)
    new = cache_host(c1, cfg.dtype)
    _check_invariants(old, new, r1, cfg.Nq, cfg.cap)
    c2 = device_cache(prep)
    r2 = call(prep, c2, cfg.tau)
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k
    for a, b in ((c1.k, c2.k), (c1.v, c2.v), (c1.ids, c2.ids), (c1.ts, c2.ts), (c1.n_valid, c2.n_valid)):
        assert torch.equal(a, b)


def test_rollout_stays_bit_identical():
    require_gpu()
    from oracle import ann_hash
    prep = prepared("tiny_f32")
    st, cfg = prep["step"], prep["cfg"]
    cache = device_cache(prep)
    state = {"k": st.cache_k[0].copy(), "v": st.cache_v[0].copy(),
             "ids": prep["cache_ids"][0].copy(), "ts": st.cache_ts[0].copy()}
    n = cfg.n0
    planes = st.planes[0]
    for c, ch in enumerate(rollout_chunks(cfg, 6, seed=0)):
        qi, _ = ann_hash(ch["q"][0], planes)
        ki, _ = ann_hash(ch["k_cur"][0], planes)
        b, cs, _, _ = tempcache_top1(ch["q"][0], qi, state["k"], state["ids"], n)
        cs32 = cs.astype(np.float32)
        res = fa.tempcache_update(cache, dev(ch["q"], "f32"), dev_ids(qi[None]),
                                  dev(ch["k_cur"], "f32"), dev(ch["v_cur"], "f32"),
                                  dev_ids(ki[None]), cfg.P, cfg.tau, ch["step"],
                                  best_in=torch.from_numpy(b[None].astype(np.int32)).cuda(),
                                  cos_in=torch.from_numpy(cs32[None]).cuda())
        ref = tempcache_commit(state, n, ch["k_cur"][0], ch["v_cur"][0], ki, b,
                               cs32.astype(np.float64), float(np.float32(cfg.tau)), ch["step"])
        state, n = ref["cache"], ref["n"]
        got = cache_host(cache, "f32")
        assert got["n"][0] == n <= cfg.cap
        assert np.array_equal(res["dest"][0].cpu().numpy(), ref["dest"]), f"chunk {c}"
        assert np.array_equal(got["k"][0], state["k"].astype(np.float32)), f"chunk {c}"
        assert np.array_equal(got["ts"][0], state["ts"]), f"chunk {c}"
        assert np.array_equal(got["ids"][0], state["ids"]), f"chunk {c}"


@pytest.mark.parametrize("ordered", [False, True])
@pytest.mark.parametrize("pool", [0, 50])
def test_commit_bit_exact_multi_chunk(pool, ordered):
    """N above one block pass of tokens (8192) and a cache above one pass of
    slots (32768), full and partial heads; with ``pool`` = 50 thousands of
    tokens claim the same few slots."""
    require_gpu()
    from workloads import commit_case
    H, N, cap, d, P, tau, step = 2, 9000, 40000, 64, 5, 0.95, 1000
    n_valid = np.array([cap, cap - 3000], np.int32)
    c = commit_case(11 + pool, H, N, cap, d, n_valid, P, pool=pool)
    cache = fa.KVCache(k=torch.from_numpy(c["cache_k"]).cuda(), v=torch.from_numpy(c["cache_v"]).cuda(),
                       ids=dev_ids(c["cache_ids"]), ts=torch.from_numpy(c["cache_ts"]).cuda(),
                       n_valid=torch.from_numpy(n_valid).cuda(),
                       knorm=torch.zeros(H, cap, dtype=torch.float32, device="cuda"))
    kc = torch.from_numpy(c["k_cur"]).cuda()
    order = checked_order(cache, N, c["cache_ts"], n_valid) if ordered else None
    res = fa.tempcache_update(cache, kc, dev_ids(c["kcur_ids"]), kc,
                              torch.from_numpy(c["v_cur"]).cuda(), dev_ids(c["kcur_ids"]), P, tau,
                              step, best_in=torch.from_numpy(c["best"]).cuda(),
                              cos_in=torch.from_numpy(c["cos"]).cuda(), order_in=order)
    got = cache_host(cache, "f32")
    for h in range(H):
        ref = tempcache_commit({"k": c["cache_k"][h], "v": c["cache_v"][h], "ids": c["cache_ids"][h],
                                "ts": c["cache_ts"][h]}, int(n_valid[h]), c["k_cur"][h],
                               c["v_cur"][h], c["kcur_ids"][h], c["best"][h],
                               c["cos"][h].astype(np.float64), float(np.float32(tau)), step)
        assert ref["counts"][4] > 0 and ref["counts"][1] > 0
        assert np.array_equal(res["dest"][h].cpu().numpy(), ref["dest"]), f"dest head {h}"
        assert np.array_equal(res["evicted"][h].cpu().numpy(), ref["evicted"]), f"evicted head {h}"
        assert np.array_equal(res["counts"][h].cpu().numpy(), ref["counts"]), f"counts head {h}"
        assert got["n"][h] == ref["n"]
        assert np.array_equal(got["k"][h], ref["cache"]["k"]), f"k head {h}"
        assert np.array_equal(got["v"][h], ref["cache"]["v"]), f"v head {h}"
        assert np.array_equal(got["ids"][h], ref["cache"]["ids"]), f"ids head {h}"
        assert np.array_equal(got["ts"][h], ref["cache"]["ts"]), f"ts head {h}"

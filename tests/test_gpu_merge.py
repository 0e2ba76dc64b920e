"""GPU parity of the mean-merged cache (Lemma 5.1, FAST-AR summary, Core
Components A) against the oracle.

* AnnSA over a merged cache (logits of slot j shifted by ln m_j), with and
  without the fused search: attention within the attention tolerances; the
  search result is the same as without group sizes (cosines ignore them);
* the merged commit with the oracle's (best, cos) as inputs: dest, evicted,
  counts, n_valid, keys, ids, timestamps and group sizes bit-exact; merged
  values within the bound of their fp32 arithmetic (below) -- full cache,
  partial cache, and a multi-chunk case whose groups exceed one wave (the
  members are then ordered by the large-group path);
* a merged rollout: integer state exact over six chunks, values within the
  bound per chunk (the oracle takes the device's values after each chunk, so
  the bound applies to one chunk's arithmetic);
* determinism: two eager merged steps and three graph replays are bit-identical.

Merged value bound.  The kernel forms acc = m*v_old + v_1 + ... + v_c in fp32
(members in ascending token order), divides by m + c and rounds once to the
cache type.  With S = m|v_old| + sum |v_i| each of the c + 2 roundings before
the last is at most 2**-24 * S, so |v_gpu - v_ref| <= (c + 2) 2**-24 S/(m + c)
plus the final rounding: half a bf16 ulp (2**-8 |v_ref|, a full ulp allowed for
values next to a rounding boundary) for bf16 caches, 2**-24 |v_ref| for fp32.
"""
import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import annsa as o_annsa, key_context, key_counts, tempcache_commit, tempcache_top1
from sparse_attention_autoregressive_amd.step import AttentionStep
from tests.gpu_util import (LSE_ABS, assert_attention_close, dev, dev_ids, device_cache,
                            host_ids, prepared, require_gpu)
from workloads import commit_case, group_sizes, rollout_chunks

pytestmark = pytest.mark.gpu


def merged_cache(prep, n=None, max_m=32, seed=0):
    cfg = prep["cfg"]
    c = device_cache(prep, n)
    m = group_sizes(seed, cfg.H, cfg.cap, max_m)
    c.count = torch.from_numpy(m).cuda()
    return c, m


def oracle_annsa_merged(prep, n, m):
    st, cfg = prep["step"], prep["cfg"]
    Os, Ls = [], []
    for h in range(cfg.H):
        K, V, kid = key_context(st.cache_k[h], st.cache_v[h], prep["cache_ids"][h], n,
                                st.k_cur[h], st.v_cur[h], prep["k_cur_ids"][h])
        O, L = o_annsa(st.q[h], prep["q_ids"][h], K, V, kid, st.scale,
                       key_counts(m[h], n, st.k_cur.shape[1]))
        Os.append(O)
        Ls.append(L)
    return np.stack(Os), np.stack(Ls)


def _args(prep):
    st, cfg = prep["step"], prep["cfg"]
    return (dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
            dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]), cfg.P)


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
@pytest.mark.parametrize("search", [False, True])
def test_annsa_merged_matches_oracle(name, search):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    cache, m = merged_cache(prep)
    res = fa.annsa_forward(*_args(prep), cache=cache, search=search)
    O, L = oracle_annsa_merged(prep, cfg.n0, m)
    err = assert_attention_close(res[0], O, cfg.dtype, f"merged annsa {name}")
    g = res[1].cpu().numpy().astype(np.float64)
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.abs(g[fin] - L[fin]).max() <= LSE_ABS
    if search:
        plain = fa.annsa_forward(*_args(prep), cache=device_cache(prep), search=True)
        assert torch.equal(res[2], plain[2]) and torch.equal(res[3], plain[3])
    print(f"merged annsa {name} search={search}: max err {err:.3e}")


def check_merged_commit(res, cache, ref, old_v, old_m, v_cur, best, cos, tau, n, bf16, h, what):
    """Integers exact, merged values within the bound (copied rows exact)."""
    got_v = cache.v[h].float().cpu().numpy().astype(np.float64)
    assert np.array_equal(res["dest"][h].cpu().numpy(), ref["dest"]), f"{what}: dest"
    assert np.array_equal(res["evicted"][h].cpu().numpy(), ref["evicted"]), f"{what}: evicted"
    assert np.array_equal(res["counts"][h].cpu().numpy(), ref["counts"]), f"{what}: counts"
    assert int(cache.n_valid[h]) == ref["n"], f"{what}: n"
    nn = ref["n"]
    assert np.array_equal(cache.count[h].cpu().numpy()[:nn], ref["cache"]["count"][:nn]), f"{what}: sizes"
    assert np.array_equal(cache.k[h].float().cpu().numpy(), np.asarray(ref["cache"]["k"], np.float32))
    assert np.array_equal(host_ids(cache.ids)[h], ref["cache"]["ids"]), f"{what}: ids"
    assert np.array_equal(cache.ts[h].cpu().numpy(), ref["cache"]["ts"]), f"{what}: ts"
    cap = got_v.shape[0]
    members = np.nonzero(ref["matched"])[0]
    c = np.bincount(best[members], minlength=cap)[:cap].astype(np.float64)
    S = np.zeros_like(got_v)
    np.add.at(S, best[members], np.abs(v_cur[members]))
    m = np.maximum(np.asarray(old_m, np.float64), 1.0)[:, None]
    S += m * np.abs(old_v)
    r = np.asarray(ref["cache"]["v"], np.float64)
    tol = (c[:, None] + 2) * 2.0 ** -24 * S / (m + c[:, None])
    tol += (2.0 ** -8 if bf16 else 2.0 ** -24) * np.abs(r) + 1e-30
    tol[c == 0] = 0.0                                      # copied or untouched rows are exact
    err = np.abs(got_v - r)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.any(axis=1).sum())} slots off, max err {err.max():.3e}"
    return int((c > 0).sum())


def _merged_commit_case(prep, n, tau, max_m=32):
    st, cfg = prep["step"], prep["cfg"]
    cache, m = merged_cache(prep, n=n, max_m=max_m)
    tops = [tempcache_top1(st.q[h], prep["q_ids"][h], st.cache_k[h], prep["cache_ids"][h], n)
            for h in range(cfg.H)]
    best = np.stack([t[0] for t in tops]).astype(np.int32)
    cos32 = np.stack([t[1] for t in tops]).astype(np.float32)
    res = fa.tempcache_update(cache, dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]),
                              dev(st.k_cur, cfg.dtype), dev(st.v_cur, cfg.dtype),
                              dev_ids(prep["k_cur_ids"]), cfg.P, tau, st.step,
                              best_in=torch.from_numpy(best).cuda(),
                              cos_in=torch.from_numpy(cos32).cuda())
    tau32 = float(np.float32(tau))
    merged = 0
    for h in range(cfg.H):
        ch = {"k": st.cache_k[h], "v": st.cache_v[h], "ids": prep["cache_ids"][h],
              "ts": st.cache_ts[h], "count": m[h]}
        ref = tempcache_commit(ch, n, st.k_cur[h], st.v_cur[h], prep["k_cur_ids"][h], best[h],
                               cos32[h].astype(np.float64), tau32, st.step, merge=True)
        merged += check_merged_commit(res, cache, ref, st.cache_v[h].astype(np.float64), m[h],
                                      st.v_cur[h].astype(np.float64), best[h], cos32[h], tau32, n,
                                      cfg.dtype == "bf16", h, f"head {h}")
    return res, merged


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_merged_commit_full_cache(name):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    res, merged = _merged_commit_case(prep, cfg.n0, cfg.tau)
    assert merged > 0 and (res["counts"][:, 4] > 0).all()
    if name == "wan13_bf16":
        assert (res["counts"][:, 2] > 0).all()              # groups of several tokens


def test_merged_commit_partial_cache():
    require_gpu()
    prep = prepared("single_bf16")
    n = prep["cfg"].cap - 1000
    _merged_commit_case(prep, n, 0.97)


@pytest.mark.parametrize("N,cap", [(9000, 40000), (8000, 32000), (45000, 50000)])
def test_merged_commit_large_groups(N, cap):
    """Most tokens claim 50 slots: groups of a hundred members and more take
    the large-group ordering path.  The shapes cover every placement of the
    select's tables: claims in the workspace and groups in LDS (40000 slots),
    claims in LDS and groups in the workspace (32000 slots, 8000 tokens), both
    in the workspace (50000 slots, 45000 tokens, several token passes)."""
    require_gpu()
    H, d, P, tau, step = 2, 64, 5, 0.95, 1000
    n_valid = np.array([cap, cap - 3000], np.int32)
    c = commit_case(61, H, N, cap, d, n_valid, P, match_frac=0.7, pool=50)
    m = group_sizes(3, H, cap, 200)
    cache = fa.KVCache(k=torch.from_numpy(c["cache_k"]).cuda(), v=torch.from_numpy(c["cache_v"]).cuda(),
                       ids=dev_ids(c["cache_ids"]), ts=torch.from_numpy(c["cache_ts"]).cuda(),
                       n_valid=torch.from_numpy(n_valid).cuda(),
                       knorm=torch.zeros(H, cap, dtype=torch.float32, device="cuda"),
                       count=torch.from_numpy(m).cuda())
    kc = torch.from_numpy(c["k_cur"]).cuda()
    res = fa.tempcache_update(cache, kc, dev_ids(c["kcur_ids"]), kc,
                              torch.from_numpy(c["v_cur"]).cuda(), dev_ids(c["kcur_ids"]), P, tau,
                              step, best_in=torch.from_numpy(c["best"]).cuda(),
                              cos_in=torch.from_numpy(c["cos"]).cuda())
    for h in range(H):
        ch = {"k": c["cache_k"][h], "v": c["cache_v"][h], "ids": c["cache_ids"][h],
              "ts": c["cache_ts"][h], "count": m[h]}
        ref = tempcache_commit(ch, int(n_valid[h]), c["k_cur"][h], c["v_cur"][h], c["kcur_ids"][h],
                               c["best"][h], c["cos"][h].astype(np.float64), float(np.float32(tau)),
                               step, merge=True)
        sizes = np.bincount(c["best"][h][ref["matched"]], minlength=cap)
        assert sizes.max() > 64
        check_merged_commit(res, cache, ref, c["cache_v"][h].astype(np.float64), m[h],
                            c["v_cur"][h].astype(np.float64), c["best"][h], c["cos"][h],
                            tau, int(n_valid[h]), False, h, f"head {h}")


def test_merged_rollout():
    require_gpu()
    from oracle import ann_hash
    prep = prepared("tiny_f32")
    st, cfg = prep["step"], prep["cfg"]
    cache, m = merged_cache(prep, max_m=8)
    state = {"k": st.cache_k[0].astype(np.float64), "v": st.cache_v[0].astype(np.float64),
             "ids": prep["cache_ids"][0].copy(), "ts": st.cache_ts[0].copy(), "count": m[0].copy()}
    n = cfg.n0
    planes = st.planes[0]
    total = int(m[0][:n].sum())
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
                               cs32.astype(np.float64), float(np.float32(cfg.tau)), ch["step"],
                               merge=True)
        check_merged_commit(res, cache, ref, state["v"], state["count"],
                            ch["v_cur"][0].astype(np.float64), b, cs32, cfg.tau, n, False, 0,
                            f"chunk {c}")
        ev = ref["evicted"][ref["evicted"] >= 0]
        total += ch["k_cur"].shape[1] - int(state["count"][ev].sum())
        state, n = ref["cache"], ref["n"]
        assert int(state["count"][:n].sum()) == total
        # the next chunk starts from the device's values
        state["v"] = cache.v[0].cpu().numpy().astype(np.float64)


def _inputs(cfg, seed):
    from workloads import make_step
    st = make_step(cfg, seed)
    planes = torch.from_numpy(st.planes).cuda()
    t = dict(q=dev(st.q, cfg.dtype), k_cur=dev(st.k_cur, cfg.dtype), v_cur=dev(st.v_cur, cfg.dtype),
             kp=dev(st.kp, cfg.dtype), vp=dev(st.vp, cfg.dtype), planes=planes)
    base = fa.KVCache.from_keys(dev(st.cache_k, cfg.dtype), dev(st.cache_v, cfg.dtype),
                                torch.from_numpy(st.cache_ts).cuda(),
                                torch.from_numpy(st.n_valid).cuda(), planes,
                                count=torch.from_numpy(group_sizes(seed, cfg.H, cfg.cap)).cuda())
    return st, t, base


@pytest.mark.parametrize("name", ["single_bf16", "wan13_bf16"])
def test_merged_step_deterministic_and_graph(name):
    require_gpu()
    from workloads import CONFIGS
    cfg = CONFIGS[name]
    st, t, base = _inputs(cfg, 0)
    s = AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau)
    args = (t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], t["planes"], st.step)

    def snap(cache):
        torch.cuda.synchronize()
        out = {k: getattr(s, k).clone() for k in ("o_sa", "lse", "o_ca", "best", "best_cos")}
        for k in ("k", "v", "ids", "ts", "n_valid", "knorm", "count"):
            out["cache_" + k] = getattr(cache, k).clone()
        return out

    c1 = base.clone()
    s(c1, *args)
    ref = snap(c1)
    assert not torch.equal(ref["cache_count"], base.count)      # groups grew
    c2 = base.clone()
    s(c2, *args)
    for k, v in snap(c2).items():
        assert torch.equal(v, ref[k]), f"eager rerun: {k}"
    cg = base.clone()
    g = s.graph(cg, *args)
    for r in range(3):
        for k in ("k", "v", "ids", "ts", "n_valid", "knorm", "count"):
            getattr(cg, k).copy_(getattr(base, k))
        for buf in (s.o_sa, s.lse, s.o_ca, s.best_cos):
            buf.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        for k, v in snap(cg).items():
            assert torch.equal(v, ref[k]), f"replay {r}: {k}"

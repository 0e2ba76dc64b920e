"""The step exactly as bench.py times it -- the two-stream ``AttentionStep`` on
the Wan-1.3B-like chunk (12 heads, 4680 queries, full 32760-slot cache, 128
buckets, 512 prompt tokens) and on the Wan-14B-like layer (40 heads, 256
buckets, 128 centroids per head) -- against the oracle on every head.

Tie protocol (the oracle's flags):
* bucket ids must agree outside flagged hash bits; the oracle's later stages
  then run on the GPU's ids;
* the TempCache slot must agree outside flagged argmax near-ties (there the
  GPU's slot must be one of the near-maximal ones), the cosine within the
  flag width, and the match decision outside flagged threshold ties;
* the oracle's commit then runs on the ORACLE's own (slot, cosine), with the
  GPU's decision injected only for flagged tokens, and the cache (keys,
  values, ids, timestamps, valid count) must agree bit for bit.
Attention outputs within the attention tolerances.
"""
import math

import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import ann_hash, annca, annsa, key_context, tempcache_commit, tempcache_top1
from sparse_attention_autoregressive_amd.step import AttentionStep
from tests.gpu_util import (LSE_ABS, TIE_EPS, assert_attention_close, assert_ids_match,
                            assert_top1_matches, dev, host_ids, require_gpu)
from workloads import CONFIGS, make_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["wan13_bf16", "wan14_bf16"])
def test_bench_step_matches_oracle_on_every_head(name):
    require_gpu()
    cfg = CONFIGS[name]
    st = make_step(cfg, 0)
    planes = torch.from_numpy(st.planes).cuda()
    t = {k: dev(getattr(st, k), cfg.dtype) for k in ("q", "k_cur", "v_cur", "kp", "vp")}
    cache = fa.KVCache.from_keys(dev(st.cache_k, cfg.dtype), dev(st.cache_v, cfg.dtype),
                                 torch.from_numpy(st.cache_ts).cuda(), torch.from_numpy(st.n_valid).cuda(),
                                 planes)
    cache_ids = host_ids(cache.ids)                       # before the commit rewrites them
    s = AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau, overlap=True)
    s(cache, t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], planes, st.step)
    torch.cuda.synchronize()
    ids = {k: host_ids(v) for k, v in s.ids.items()}
    best, bcos = s.best.cpu().numpy(), s.best_cos.cpu().numpy()
    lse = s.lse.cpu().numpy()
    o_sa, o_ca, keep = s.o_sa.cpu(), s.o_ca.cpu(), s.keep.cpu().numpy().astype(bool)
    ck, cv = cache.k.float().cpu().numpy(), cache.v.float().cpu().numpy()
    cids, cts, cn = host_ids(cache.ids), cache.ts.cpu().numpy(), cache.n_valid.cpu().numpy()
    scale = 1.0 / math.sqrt(cfg.d)
    tau32 = float(np.float32(cfg.tau))
    flags = {"argmax": 0, "threshold": 0, "evicted": 0}
    for h in range(cfg.H):
        for key, arr, g in (("q", st.q, ids["q"]), ("k", st.k_cur, ids["k"]), ("p", st.kp, ids["p"]),
                            ("c", st.cache_k, cache_ids)):
            ref, tie = ann_hash(arr[h], st.planes[h])
            assert_ids_match(g[h], ref, tie, f"{key} ids head {h}")
        qi, ki, pi, ci = ids["q"][h], ids["k"][h], ids["p"][h], cache_ids[h]
        n = int(st.n_valid[h])
        K, V, kid = key_context(st.cache_k[h], st.cache_v[h], ci, n, st.k_cur[h], st.v_cur[h], ki)
        O, L = annsa(st.q[h], qi, K, V, kid, scale)
        assert_attention_close(o_sa[h], O, cfg.dtype, f"annsa head {h}")
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(lse[h]), fin)
        assert np.abs(lse[h][fin] - L[fin]).max() <= LSE_ABS
        Oc, kp_keep = annca(st.q[h], qi, cfg.frame_len, st.kp[h], st.vp[h], pi, scale)
        assert np.array_equal(keep[h], kp_keep), f"keep head {h}"
        assert_attention_close(o_ca[h], Oc, cfg.dtype, f"annca head {h}")
        # top-1 and match decisions under the tie protocol
        _, n_tie, n_thr = assert_top1_matches(best[h], bcos[h], st.q[h], qi, st.cache_k[h], ci, n, cfg.tau,
                                              f"top1 head {h}")
        flags["argmax"] += n_tie
        flags["threshold"] += n_thr
        # the commit on the oracle's own top-1, the GPU's decision injected
        # only where the oracle flags a tie
        ob, oc, tie, _ = tempcache_top1(st.q[h], qi, st.cache_k[h], ci, n)
        flagged = tie | (np.isfinite(oc) & (np.abs(oc - cfg.tau) < TIE_EPS))
        b_in, c_in = ob.copy(), oc.copy()
        b_in[flagged] = best[h][flagged]
        c_in[flagged] = bcos[h][flagged].astype(np.float64)
        ref = tempcache_commit({"k": st.cache_k[h], "v": st.cache_v[h], "ids": ci, "ts": st.cache_ts[h]}, n,
                               st.k_cur[h], st.v_cur[h], ki, b_in, c_in, tau32, st.step)
        assert int(cn[h]) == ref["n"]
        assert np.array_equal(ck[h], ref["cache"]["k"].astype(np.float32)), f"cache k head {h}"
        assert np.array_equal(cv[h], ref["cache"]["v"].astype(np.float32)), f"cache v head {h}"
        assert np.array_equal(cids[h], ref["cache"]["ids"]), f"cache ids head {h}"
        assert np.array_equal(cts[h], ref["cache"]["ts"]), f"cache ts head {h}"
        # the step's commit reports no counts; the cache equality above covers dest and evicted
        assert ref["counts"][4] > 0 and ref["counts"][2] > 0
        flags["evicted"] += int(ref["counts"][4])
    print(f"bench step {name}: {cfg.H} heads, flags {flags}")

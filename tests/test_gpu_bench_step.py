"""The step exactly as bench.py times it -- the two-stream ``AttentionStep`` on
the Wan-1.3B-like chunk (12 heads, 4680 queries, full 32760-slot cache, 128
buckets, 512 prompt tokens) -- against the oracle on sampled heads; the same
for the Wan-14B-like layer (40 heads, 256 buckets, 128 centroids per head).

Tie protocol (the oracle's flags): bucket ids must agree outside flagged hash
bits, and the oracle's later stages then run on the GPU's ids; the TempCache
slot must agree outside flagged argmax near-ties (there the GPU's slot must be
one of the near-maximal ones); the oracle's commit then runs on the GPU's
(slot, cosine) decisions, and the cache, dest, evicted and counts must agree
bit for bit.  Attention outputs within the attention tolerances.
"""
import math

import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import ann_hash, annca, annsa, key_context, tempcache_commit, tempcache_top1
from sparse_attention_autoregressive_amd.step import AttentionStep
from tests.gpu_util import (COS_ABS, LSE_ABS, assert_attention_close, assert_ids_match, dev, host_ids,
                            require_gpu)
from workloads import CONFIGS, make_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,heads", [("wan13_bf16", (0, 6, 11)), ("wan14_bf16", (0, 19, 39))])
def test_bench_step_matches_oracle_on_sampled_heads(name, heads):
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
    scale = 1.0 / math.sqrt(cfg.d)
    for h in heads:
        for key, arr, g in (("q", st.q, ids["q"]), ("k", st.k_cur, ids["k"]), ("p", st.kp, ids["p"]),
                            ("c", st.cache_k, cache_ids)):
            ref, tie = ann_hash(arr[h], st.planes[h])
            assert_ids_match(g[h], ref, tie, f"{key} ids head {h}")
        qi, ki, pi, ci = ids["q"][h], ids["k"][h], ids["p"][h], cache_ids[h]
        n = int(st.n_valid[h])
        K, V, kid = key_context(st.cache_k[h], st.cache_v[h], ci, n, st.k_cur[h], st.v_cur[h], ki)
        O, L = annsa(st.q[h], qi, K, V, kid, scale)
        assert_attention_close(s.o_sa[h], O, cfg.dtype, f"annsa head {h}")
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(lse[h]), fin)
        assert np.abs(lse[h][fin] - L[fin]).max() <= LSE_ABS
        Oc, keep = annca(st.q[h], qi, cfg.frame_len, st.kp[h], st.vp[h], pi, scale)
        assert np.array_equal(s.keep[h].cpu().numpy().astype(bool), keep)
        assert_attention_close(s.o_ca[h], Oc, cfg.dtype, f"annca head {h}")
        b, c, tie, near = tempcache_top1(st.q[h], qi, st.cache_k[h], ci, n)
        ok = ~tie
        assert np.array_equal(best[h][ok], b[ok]), f"best head {h}"
        for i in np.nonzero(tie)[0]:
            assert best[h][i] in near[i]
        f = np.isfinite(c)
        assert np.array_equal(np.isfinite(bcos[h]), f)
        assert np.abs(bcos[h][f].astype(np.float64) - c[f]).max() <= COS_ABS
        # the commit on the GPU's decisions
        ref = tempcache_commit({"k": st.cache_k[h], "v": st.cache_v[h], "ids": ci, "ts": st.cache_ts[h]}, n,
                               st.k_cur[h], st.v_cur[h], ki, best[h], bcos[h].astype(np.float64),
                               float(np.float32(cfg.tau)), st.step)
        assert int(cache.n_valid[h]) == ref["n"]
        assert np.array_equal(cache.k[h].float().cpu().numpy(), ref["cache"]["k"].astype(np.float32))
        assert np.array_equal(cache.v[h].float().cpu().numpy(), ref["cache"]["v"].astype(np.float32))
        assert np.array_equal(host_ids(cache.ids)[h], ref["cache"]["ids"])
        assert np.array_equal(cache.ts[h].cpu().numpy(), ref["cache"]["ts"])
        # the step's commit reports no counts; the cache equality above covers dest and evicted
        assert ref["counts"][4] > 0 and ref["counts"][2] > 0

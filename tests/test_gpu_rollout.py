"""Consecutive chunks of the step exactly as the bench runs it (the two-stream
``AttentionStep``, all heads on the GPU) at the Wan-1.3B-like shape, against
the oracle on sampled heads -- the long-rollout setting (summary, "Key
Results": a bounded cache keeps memory and per-chunk cost flat) taken over
several commits, so each chunk attends to and commits into a cache the
previous commits wrote.

Per chunk and sampled head, under the tie protocol: bucket ids agree outside
flagged hash bits (the oracle then uses the GPU's ids); AnnSA and AnnCA outputs
within the attention tolerances; the top-1 slot, cosine and match decision
under the argmax / threshold flags; the oracle commits on its own top-1 with
the GPU's decision injected only for flagged tokens, and the GPU cache (keys,
values, ids, timestamps, valid count) must then equal the oracle's bit for
bit -- after every chunk, so the states never drift apart.
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
from workloads import CONFIGS, make_step, rollout_chunks

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,heads,chunks", [("wan13_bf16", (0, 7, 11), 5)])
def test_rollout_of_the_bench_step_matches_oracle(name, heads, chunks):
    require_gpu()
    cfg = CONFIGS[name]
    st = make_step(cfg, 0)
    planes = torch.from_numpy(st.planes).cuda()
    kp, vp = dev(st.kp, cfg.dtype), dev(st.vp, cfg.dtype)
    cache = fa.KVCache.from_keys(dev(st.cache_k, cfg.dtype), dev(st.cache_v, cfg.dtype),
                                 torch.from_numpy(st.cache_ts).cuda(), torch.from_numpy(st.n_valid).cuda(),
                                 planes)
    gpu_cache_ids = host_ids(cache.ids)
    state = {}
    for h in heads:
        ref, tie = ann_hash(st.cache_k[h], st.planes[h])
        assert_ids_match(gpu_cache_ids[h], ref, tie, f"cache ids head {h}")
        state[h] = {"k": st.cache_k[h].copy(), "v": st.cache_v[h].copy(), "ids": gpu_cache_ids[h].copy(),
                    "ts": st.cache_ts[h].copy(), "n": int(st.n_valid[h])}
    s = AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau, overlap=True)
    scale = 1.0 / math.sqrt(cfg.d)
    tau32 = float(np.float32(cfg.tau))
    for c, ch in enumerate(rollout_chunks(cfg, chunks, seed=0)):
        print(f"rollout {name}: chunk {c} step {ch['step']}", flush=True)
        q, kc, vc = (dev(ch[k], cfg.dtype) for k in ("q", "k_cur", "v_cur"))
        s(cache, q, kc, vc, kp, vp, planes, ch["step"])
        torch.cuda.synchronize()
        ids = {k: host_ids(v) for k, v in s.ids.items()}
        best, bcos, lse = s.best.cpu().numpy(), s.best_cos.cpu().numpy(), s.lse.cpu().numpy()
        keep = s.keep.cpu().numpy().astype(bool)
        n_gpu = cache.n_valid.cpu().numpy()
        for h in heads:
            o = state[h]
            for key, arr, g in (("q", ch["q"], ids["q"]), ("k", ch["k_cur"], ids["k"]), ("p", st.kp, ids["p"])):
                ref, tie = ann_hash(arr[h], st.planes[h])
                assert_ids_match(g[h], ref, tie, f"chunk {c} {key} ids head {h}")
            qi, ki, pi = ids["q"][h], ids["k"][h], ids["p"][h]
            n = o["n"]
            K, V, kid = key_context(o["k"], o["v"], o["ids"], n, ch["k_cur"][h], ch["v_cur"][h], ki)
            O, L = annsa(ch["q"][h], qi, K, V, kid, scale)
            assert_attention_close(s.o_sa[h], O, cfg.dtype, f"chunk {c} annsa head {h}")
            fin = np.isfinite(L)
            assert np.array_equal(np.isfinite(lse[h]), fin)
            assert np.abs(lse[h][fin] - L[fin]).max() <= LSE_ABS
            Oc, kk = annca(ch["q"][h], qi, cfg.frame_len, st.kp[h], st.vp[h], pi, scale)
            assert np.array_equal(keep[h], kk), f"chunk {c} keep head {h}"
            assert_attention_close(s.o_ca[h], Oc, cfg.dtype, f"chunk {c} annca head {h}")
            assert_top1_matches(best[h], bcos[h], ch["q"][h], qi, o["k"], o["ids"], n, cfg.tau,
                                f"chunk {c} top1 head {h}")
            ob, oc, tie, _ = tempcache_top1(ch["q"][h], qi, o["k"], o["ids"], n)
            flagged = tie | (np.isfinite(oc) & (np.abs(oc - cfg.tau) < TIE_EPS))
            b_in, c_in = ob.copy(), oc.copy()
            b_in[flagged] = best[h][flagged]
            c_in[flagged] = bcos[h][flagged].astype(np.float64)
            ref = tempcache_commit({k: o[k] for k in ("k", "v", "ids", "ts")}, n, ch["k_cur"][h],
                                   ch["v_cur"][h], ki, b_in, c_in, tau32, ch["step"])
            o.update(ref["cache"])
            o["n"] = ref["n"]
            assert int(n_gpu[h]) == o["n"] <= cfg.cap
            assert np.array_equal(cache.k[h].float().cpu().numpy(), o["k"].astype(np.float32)), f"chunk {c} k {h}"
            assert np.array_equal(cache.v[h].float().cpu().numpy(), o["v"].astype(np.float32)), f"chunk {c} v {h}"
            assert np.array_equal(host_ids(cache.ids)[h], o["ids"]), f"chunk {c} ids head {h}"
            assert np.array_equal(cache.ts[h].cpu().numpy(), o["ts"]), f"chunk {c} ts head {h}"
            if c > 0:
                assert ref["counts"][4] > 0        # a full cache keeps evicting

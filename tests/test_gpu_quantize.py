"""GPU parity of fastar_ann_quantize (nearest-codeword buckets) against the
oracle's ``ann_quantize``, and of a whole step whose buckets come from it.

* ids bit-exact except where the oracle flags a near-tie (then the GPU's
  codeword must score within the flag margin of the best), norms within fp32
  rounding: queries, current keys and cached keys of the tiny fp32,
  single-head bf16 and Wan-1.3B-like workloads, codebooks drawn from the
  cached keys (plus noise) and pure Gaussian ones;
* edge shapes: one codeword, a codebook that is not a multiple of the
  64-codeword LDS chunk, sixteen chunks, token counts that leave a partial
  block;
* a two-stream step with quantized buckets (``AttentionStep(ann="quantize")``)
  against the oracle's stages: ids equal outside flagged near-ties, then the
  oracle's AnnSA, AnnCA and TempCache run on the GPU's ids.
"""
import math

import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import TIE_EPS, ann_quantize, annca, annsa, key_context, tempcache_update
from sparse_attention_autoregressive_amd.step import AttentionStep
from tests.gpu_util import (LSE_ABS, assert_attention_close, dev, host_ids, require_gpu)
from workloads import CONFIGS, codebook_from_keys, make_step

pytestmark = pytest.mark.gpu


def _check_ids(gpu_ids, x, C, what):
    ref, tie = ann_quantize(x, C)
    g = gpu_ids.astype(np.int64)
    ok = ~tie
    assert np.array_equal(g[ok], ref[ok].astype(np.int64)), \
        f"{what}: {int((g[ok] != ref[ok]).sum())} ids differ outside flagged ties"
    if tie.any():
        X, Cd = x.astype(np.float64), C.astype(np.float64)
        sc = X[tie] @ Cd.T - 0.5 * (Cd * Cd).sum(1)[None, :]
        cn = np.linalg.norm(Cd, axis=1)
        margin = TIE_EPS * (np.linalg.norm(X[tie], axis=1) * cn.max() + (cn ** 2).max())
        got = sc[np.arange(sc.shape[0]), g[tie]]
        assert (got >= sc.max(axis=1) - margin).all(), f"{what}: a flagged id is not near-best"
    return int(tie.sum())


@pytest.mark.parametrize("name,B,src", [("tiny_f32", 16, "keys"), ("tiny_f32", 100, "gauss"),
                                        ("single_bf16", 64, "keys"), ("wan13_bf16", 128, "keys"),
                                        ("wan13_bf16", 128, "gauss")])
def test_quantize_matches_oracle(name, B, src):
    require_gpu()
    cfg = CONFIGS[name]
    st = make_step(cfg, 0)
    if src == "keys":
        C = codebook_from_keys(st.cache_k, st.n_valid, B, 0)
    else:
        C = np.random.default_rng(5).standard_normal((cfg.H, B, cfg.d)).astype(np.float32)
    Cd = torch.from_numpy(C).cuda()
    ties = 0
    for key, arr in (("q", st.q), ("k_cur", st.k_cur), ("cache", st.cache_k)):
        x = dev(arr, cfg.dtype)
        norms = torch.empty(cfg.H, arr.shape[1], dtype=torch.float32, device="cuda")
        ids = host_ids(fa.ann_quantize(x, Cd, norms=norms))
        for h in range(cfg.H):
            ties += _check_ids(ids[h], arr[h], C[h], f"{name} {key} head {h}")
        np.testing.assert_allclose(norms.cpu().numpy(), np.linalg.norm(arr.astype(np.float64), axis=2),
                                   rtol=2e-6, atol=0)
    print(f"quantize {name} B={B} {src}: {ties} flagged near-ties")


@pytest.mark.parametrize("N,B", [(100, 1), (100, 65), (257, 1000), (64, 64), (513, 129)])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_quantize_edge_shapes(N, B, dtype, d):
    require_gpu()
    rng = np.random.default_rng(N + B)
    H = 2
    x = rng.standard_normal((H, N, d)).astype(np.float32)
    if dtype == "bf16":
        from workloads import bf16_round
        x = bf16_round(x)
    C = rng.standard_normal((H, B, d)).astype(np.float32) * rng.uniform(0.5, 2, (H, B, 1)).astype(np.float32)
    ids = host_ids(fa.ann_quantize(dev(x, dtype), torch.from_numpy(C).cuda()))
    for h in range(H):
        _check_ids(ids[h], x[h], C[h], f"N={N} B={B} head {h}")


@pytest.mark.parametrize("name", ["tiny_f32", "wan13_bf16"])
def test_quantized_step_matches_oracle(name):
    require_gpu()
    cfg = CONFIGS[name]
    st = make_step(cfg, 0)
    B = 1 << cfg.P
    C = codebook_from_keys(st.cache_k, st.n_valid, B, 1)
    Cd = torch.from_numpy(C).cuda()
    t = {k: dev(getattr(st, k), cfg.dtype) for k in ("q", "k_cur", "v_cur", "kp", "vp")}
    k = dev(st.cache_k, cfg.dtype)
    knorm = torch.empty(cfg.H, cfg.cap, dtype=torch.float32, device="cuda")
    cids = fa.ann_quantize(k, Cd, norms=knorm)
    g_cache_ids = host_ids(cids)                 # before the commit rewrites them
    cache = fa.KVCache(k=k, v=dev(st.cache_v, cfg.dtype), ids=cids,
                       ts=torch.from_numpy(st.cache_ts).cuda(),
                       n_valid=torch.from_numpy(st.n_valid).cuda(), knorm=knorm)
    s = AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau,
                      ann="quantize")
    s(cache, t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], Cd, st.step)
    torch.cuda.synchronize()
    heads = range(cfg.H) if cfg.H == 1 else [0, 7]
    lse = s.lse.cpu().numpy()
    g_ids = {k: host_ids(v) for k, v in s.ids.items()}
    for h in heads:
        # tie protocol: ids must agree outside flagged near-ties; downstream
        # stages then run in the oracle on the GPU's ids
        got = {}
        for key, arr, gid in (("q", st.q, g_ids["q"]), ("k", st.k_cur, g_ids["k"]),
                              ("p", st.kp, g_ids["p"]), ("c", st.cache_k, g_cache_ids)):
            ref, tie = ann_quantize(arr[h], C[h])
            assert np.array_equal(gid[h][~tie], ref[~tie]), f"{key} ids head {h}"
            got[key] = gid[h]
        qi, ki, pi, ci = got["q"], got["k"], got["p"], got["c"]
        n = int(st.n_valid[h])
        K, V, kid = key_context(st.cache_k[h], st.cache_v[h], ci, n, st.k_cur[h], st.v_cur[h], ki)
        O, L = annsa(st.q[h], qi, K, V, kid, 1.0 / math.sqrt(cfg.d))
        assert_attention_close(s.o_sa[h], O, cfg.dtype, f"annsa head {h}")
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(lse[h]), fin)
        assert np.abs(lse[h][fin] - L[fin]).max() <= LSE_ABS
        Oc, keep = annca(st.q[h], qi, cfg.frame_len, st.kp[h], st.vp[h], pi, 1.0 / math.sqrt(cfg.d))
        assert np.array_equal(s.keep[h].cpu().numpy().astype(bool), keep)
        assert_attention_close(s.o_ca[h], Oc, cfg.dtype, f"annca head {h}")
        tcres = tempcache_update({"k": st.cache_k[h], "v": st.cache_v[h], "ids": ci,
                                  "ts": st.cache_ts[h]}, n, st.q[h], qi, st.k_cur[h], st.v_cur[h],
                                 ki, cfg.tau, st.step)
        ok = ~(tcres["argmax_tie"] | tcres["thr_tie"])
        assert np.array_equal(s.best[h].cpu().numpy()[ok], tcres["best"][ok])
        if ok.all():
            assert int(cache.n_valid[h]) == tcres["n"]
            assert np.array_equal(host_ids(cache.ids)[h], tcres["cache"]["ids"])
            assert np.array_equal(cache.ts[h].cpu().numpy(), tcres["cache"]["ts"])


@pytest.mark.parametrize("name,B", [("tiny_f32", 16), ("wan13_bf16", 128)])
def test_quantize_batch_equals_separate_calls(name, B):
    """fastar_ann_quantize_batch (queries, current keys and prompt keys in one
    launch, sets of different sizes) gives exactly the ids and norms of one
    fastar_ann_quantize per set."""
    require_gpu()
    cfg = CONFIGS[name]
    st = make_step(cfg, 0)
    C = torch.from_numpy(codebook_from_keys(st.cache_k, st.n_valid, B, 0)).cuda()
    xs = [dev(a, cfg.dtype) for a in (st.q, st.k_cur, st.kp)]
    norms = [torch.empty(cfg.H, x.shape[1], dtype=torch.float32, device="cuda") for x in xs]
    got = fa.ann_quantize_batch(xs, C, norms=norms)
    for x, g, nb in zip(xs, got, norms):
        n1 = torch.empty_like(nb)
        one = fa.ann_quantize(x, C, norms=n1)
        assert torch.equal(g, one) and torch.equal(nb, n1)

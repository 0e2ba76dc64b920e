"""End-to-end step on the GPU (hash -> AnnSA -> AnnCA -> TempCache commit, every
stage on the device, nothing fed from the oracle) against the oracle's own
end-to-end step.  The tiny workload's seeds 0, 2 and 4 have no hash, argmax or
threshold near-tie anywhere, so every integer must agree exactly and every
float within tolerance."""
import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import ann_hash, attention_step
from tests.gpu_util import (LSE_ABS, assert_attention_close, dev, dev_ids, host_ids, require_gpu)
from workloads import CONFIGS, make_step

pytestmark = pytest.mark.gpu


def gpu_step(st, cfg, fused):
    planes = torch.from_numpy(st.planes).cuda()
    q, kc, vc = dev(st.q, cfg.dtype), dev(st.k_cur, cfg.dtype), dev(st.v_cur, cfg.dtype)
    cache = fa.KVCache.from_keys(dev(st.cache_k, cfg.dtype), dev(st.cache_v, cfg.dtype),
                                 torch.from_numpy(st.cache_ts).cuda(),
                                 torch.from_numpy(st.n_valid).cuda(), planes)
    q_ids = fa.ann_hash(q, planes)
    k_ids = fa.ann_hash(kc, planes)
    kp = dev(st.kp, cfg.dtype)
    p_ids = fa.ann_hash(kp, planes)
    if fused:       # the attention pass also returns TempCache's top-1
        o_sa, lse, best, cos = fa.annsa_forward(q, q_ids, kc, vc, k_ids, cfg.P, cache=cache, search=True)
    else:
        o_sa, lse = fa.annsa_forward(q, q_ids, kc, vc, k_ids, cfg.P, cache=cache)
        best = cos = None
    o_ca, keep, cnt = fa.annca_forward(q, q_ids, cfg.frame_len, kp, dev(st.vp, cfg.dtype), p_ids, cfg.P)
    tc = fa.tempcache_update(cache, q, q_ids, kc, vc, k_ids, cfg.P, cfg.tau, st.step,
                             best_in=best, cos_in=cos)
    torch.cuda.synchronize()
    return dict(q_ids=host_ids(q_ids), k_ids=host_ids(k_ids), p_ids=host_ids(p_ids), o_sa=o_sa,
                lse=lse, o_ca=o_ca, keep=keep, tc=tc, cache=cache)


@pytest.mark.parametrize("seed,fused", [(0, False), (2, False), (4, False), (0, True), (2, True)])
def test_end_to_end_tiny_exact(seed, fused):
    require_gpu()
    cfg = CONFIGS["tiny_f32"]
    st = make_step(cfg, seed)
    g = gpu_step(st, cfg, fused)
    cache_ids = np.stack([ann_hash(st.cache_k[h], st.planes[h])[0] for h in range(cfg.H)])
    r = attention_step(st.q, st.k_cur, st.v_cur, st.cache_k, st.cache_v, cache_ids, st.cache_ts,
                       st.n_valid, st.planes, st.kp, st.vp, cfg.frame_len, cfg.tau, st.step)
    assert np.array_equal(g["q_ids"][0], r["q_ids"][0])
    assert np.array_equal(g["k_ids"][0], r["kcur_ids"][0])
    assert np.array_equal(g["p_ids"][0], r["kp_ids"][0])
    assert_attention_close(g["o_sa"], np.stack(r["o_sa"]), cfg.dtype, "annsa")
    lse = g["lse"].cpu().numpy()
    assert np.abs(lse - np.stack(r["lse"])).max() <= LSE_ABS
    assert np.array_equal(g["keep"].cpu().numpy().astype(bool), np.stack(r["keep"]))
    assert_attention_close(g["o_ca"], np.stack(r["o_ca"]), cfg.dtype, "annca")
    tc = r["tc"][0]
    assert not tc["argmax_tie"].any() and not tc["thr_tie"].any()
    assert np.array_equal(g["tc"]["best"][0].cpu().numpy(), tc["best"])
    assert np.array_equal(g["tc"]["dest"][0].cpu().numpy(), tc["dest"])
    assert np.array_equal(g["tc"]["evicted"][0].cpu().numpy(), tc["evicted"])
    assert np.array_equal(g["tc"]["counts"][0].cpu().numpy(), tc["counts"])
    assert int(g["cache"].n_valid[0]) == tc["n"]
    assert np.array_equal(g["cache"].k[0].cpu().numpy(), tc["cache"]["k"].astype(np.float32))
    assert np.array_equal(g["cache"].v[0].cpu().numpy(), tc["cache"]["v"].astype(np.float32))
    assert np.array_equal(host_ids(g["cache"].ids)[0], tc["cache"]["ids"])
    assert np.array_equal(g["cache"].ts[0].cpu().numpy(), tc["cache"]["ts"])

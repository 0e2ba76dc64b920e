"""The step orchestrator (two streams, HIP graph capture) on the GPU.

* the two-stream step on the tiny workload agrees with the oracle's end-to-end
  step exactly as the one-stream calls do (integers exact, floats within the
  attention tolerances);
* one-stream and two-stream eager steps give bit-identical results, with and
  without the eviction candidates listed on the side stream;
* a captured step, replayed several times with eager work (cache restore,
  output poisoning) and synchronisation between the replays, reproduces the
  eager step bit for bit on every replay;
* several steps captured into one graph (one per cache copy, or chained on
  one cache) reproduce the eager steps bit for bit.
"""
import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import ann_hash, attention_step
from sparse_attention_autoregressive_amd.step import AttentionStep
from tests.gpu_util import LSE_ABS, assert_attention_close, dev, host_ids, require_gpu
from workloads import CONFIGS, make_step

pytestmark = pytest.mark.gpu


def _inputs(cfg, seed):
    st = make_step(cfg, seed)
    planes = torch.from_numpy(st.planes).cuda()
    t = dict(q=dev(st.q, cfg.dtype), k_cur=dev(st.k_cur, cfg.dtype), v_cur=dev(st.v_cur, cfg.dtype),
             kp=dev(st.kp, cfg.dtype), vp=dev(st.vp, cfg.dtype), planes=planes)
    base = fa.KVCache.from_keys(dev(st.cache_k, cfg.dtype), dev(st.cache_v, cfg.dtype),
                                torch.from_numpy(st.cache_ts).cuda(),
                                torch.from_numpy(st.n_valid).cuda(), planes)
    return st, t, base


def _stepper(cfg, overlap, order_list=None):
    return AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau,
                         overlap=overlap, order_list=order_list)


def _run(stepper, cache, t, step):
    stepper(cache, t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], t["planes"], step)


def _snapshot(s, cache):
    torch.cuda.synchronize()
    out = {k: v.clone() for k, v in (("o_sa", s.o_sa), ("lse", s.lse), ("o_ca", s.o_ca),
                                      ("best", s.best), ("best_cos", s.best_cos), ("keep", s.keep),
                                      ("keep_count", s.keep_count))}
    for k, v in s.ids.items():
        out["ids_" + k] = v.clone()
    for k in ("k", "v", "ids", "ts", "n_valid", "knorm"):
        out["cache_" + k] = getattr(cache, k).clone()
    return out


def _assert_same(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs"


@pytest.mark.parametrize("seed", [0, 2])
def test_two_stream_step_matches_oracle(seed):
    require_gpu()
    cfg = CONFIGS["tiny_f32"]
    st, t, base = _inputs(cfg, seed)
    s = _stepper(cfg, overlap=True)
    cache = base.clone()
    _run(s, cache, t, st.step)
    torch.cuda.synchronize()
    cache_ids = np.stack([ann_hash(st.cache_k[h], st.planes[h])[0] for h in range(cfg.H)])
    r = attention_step(st.q, st.k_cur, st.v_cur, st.cache_k, st.cache_v, cache_ids, st.cache_ts,
                       st.n_valid, st.planes, st.kp, st.vp, cfg.frame_len, cfg.tau, st.step)
    assert np.array_equal(host_ids(s.ids["q"])[0], r["q_ids"][0])
    assert np.array_equal(host_ids(s.ids["k"])[0], r["kcur_ids"][0])
    assert np.array_equal(host_ids(s.ids["p"])[0], r["kp_ids"][0])
    assert_attention_close(s.o_sa, np.stack(r["o_sa"]), cfg.dtype, "annsa")
    assert np.abs(s.lse.cpu().numpy() - np.stack(r["lse"])).max() <= LSE_ABS
    assert np.array_equal(s.keep.cpu().numpy().astype(bool), np.stack(r["keep"]))
    assert_attention_close(s.o_ca, np.stack(r["o_ca"]), cfg.dtype, "annca")
    tc = r["tc"][0]
    assert not tc["argmax_tie"].any() and not tc["thr_tie"].any()
    assert np.array_equal(s.best[0].cpu().numpy(), tc["best"])
    assert int(cache.n_valid[0]) == tc["n"]
    assert np.array_equal(cache.k[0].cpu().numpy(), tc["cache"]["k"].astype(np.float32))
    assert np.array_equal(host_ids(cache.ids)[0], tc["cache"]["ids"])
    assert np.array_equal(cache.ts[0].cpu().numpy(), tc["cache"]["ts"])


@pytest.mark.parametrize("name", ["single_bf16", "wan13_bf16"])
def test_graph_replays_match_eager(name):
    require_gpu()
    cfg = CONFIGS[name]
    st, t, base = _inputs(cfg, 0)

    one = _stepper(cfg, overlap=False)
    c1 = base.clone()
    _run(one, c1, t, st.step)
    ref = _snapshot(one, c1)

    listed = _stepper(cfg, overlap=True, order_list=True)
    c3 = base.clone()
    _run(listed, c3, t, st.step)
    _assert_same(ref, _snapshot(listed, c3), "two streams with the order list vs one")
    del c3

    two = _stepper(cfg, overlap=True)
    c2 = base.clone()
    _run(two, c2, t, st.step)
    _assert_same(ref, _snapshot(two, c2), "two streams vs one")

    cg = base.clone()
    g = two.graph(cg, t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], t["planes"], st.step)
    for r in range(3):
        # eager work between replays: restore the cache, poison every output
        for k in ("k", "v", "ids", "ts", "n_valid", "knorm"):
            getattr(cg, k).copy_(getattr(base, k))
        for buf in (two.o_sa, two.lse, two.o_ca, two.best_cos):
            buf.fill_(float("nan"))
        for buf in (two.best, two.keep, two.keep_count, *two.ids.values()):
            buf.fill_(-1 if buf.dtype != torch.uint8 else 255)
        torch.cuda.synchronize()
        g.replay()
        _assert_same(ref, _snapshot(two, cg), f"replay {r}")


def _restore_and_poison(s, caches, bases):
    for c, b in zip(caches, bases):
        for k in ("k", "v", "ids", "ts", "n_valid", "knorm"):
            getattr(c, k).copy_(getattr(b, k))
    for buf in (s.o_sa, s.lse, s.o_ca, s.best_cos):
        buf.fill_(float("nan"))
    for buf in (s.best, s.keep, s.keep_count, *s.ids.values()):
        buf.fill_(-1 if buf.dtype != torch.uint8 else 255)
    torch.cuda.synchronize()


def _cache_state(cache):
    torch.cuda.synchronize()
    return {k: getattr(cache, k).clone() for k in ("k", "v", "ids", "ts", "n_valid", "knorm")}


@pytest.mark.parametrize("name", ["single_bf16", "wan13_bf16"])
def test_steps_in_one_graph_match_eager(name):
    """Several steps captured into one graph, as the bench times them and as
    a model's layers would be captured: (a) one step per cache copy, (b) three
    chained steps on one cache, each seeing the commit of the one before.
    Every replay (eager restores and poisoned outputs between them)
    reproduces the eager steps bit for bit: every cache, and the outputs of
    the last step."""
    require_gpu()
    cfg = CONFIGS[name]
    st, t, base = _inputs(cfg, 0)
    s = _stepper(cfg, overlap=True)
    steps = [st.step, st.step + 1, st.step + 2]

    # (a) one step on each of three cache copies
    eager = [base.clone() for _ in steps]
    for c in eager:
        _run(s, c, t, st.step)
    ref_out = _snapshot(s, eager[-1])
    ref_caches = [_cache_state(c) for c in eager]
    del eager
    copies = [base.clone() for _ in steps]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in copies:
            _run(s, c, t, st.step)
    for r in range(2):
        _restore_and_poison(s, copies, [base] * len(copies))
        g.replay()
        _assert_same(ref_out, _snapshot(s, copies[-1]), f"copies, replay {r}")
        for i, c in enumerate(copies):
            _assert_same(ref_caches[i], _cache_state(c), f"copies, replay {r}, cache {i}")
    del g, copies

    # (b) three chained steps on one cache
    ce = base.clone()
    states = []
    for sn in steps:
        _run(s, ce, t, sn)
        states.append(_cache_state(ce))
    ref_out = _snapshot(s, ce)
    assert not torch.equal(states[0]["ts"], states[-1]["ts"]), "the chained steps must change the cache"
    del ce
    cg = base.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for sn in steps:
            _run(s, cg, t, sn)
    for r in range(2):
        _restore_and_poison(s, [cg], [base])
        g.replay()
        _assert_same(ref_out, _snapshot(s, cg), f"chained, replay {r}")
        _assert_same(states[-1], _cache_state(cg), f"chained, replay {r}, cache")

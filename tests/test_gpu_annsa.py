"""GPU parity of fastar_annsa_forward against the oracle (same inputs, the
oracle's bucket ids), at the tiny fp32, single-head bf16 and full Wan-1.3B-like
shapes, plus one bucket (dense attention), a partly filled cache, no cache,
empty buckets, bf16 outputs and run-to-run determinism.  Few buckets (at least
256 queries per bucket on average) take the wide kernel's 256-query items:
checked at 2, 4 and 8 buckets, with a partly filled cache and with buckets
that hold queries but no keys.  Calls that ask for the fused TempCache search
also have its (slot, cosine) checked against the oracle's top-1 under the
tie protocol (``assert_top1_matches``).  Head counts of 3 and 5 give grids
where only part of the blocks take the XCD-run order."""

import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import annsa as o_annsa, key_context
from tests.gpu_util import (LSE_ABS, assert_attention_close, assert_top1_matches, dev, dev_ids,
                            device_cache, prepared, require_gpu)

pytestmark = pytest.mark.gpu


def check_search(prep, best, bcos, n, P=None, what=""):
    """The fused search's result on every head against the oracle's top-1."""
    st, cfg = prep["step"], prep["cfg"]
    b, c = best.cpu().numpy(), bcos.cpu().numpy()
    mask = (1 << (cfg.P if P is None else P)) - 1
    worst, ties = 0.0, 0
    for h in range(cfg.H):
        err, t, _ = assert_top1_matches(b[h], c[h], st.q[h], prep["q_ids"][h] & mask, st.cache_k[h],
                                        prep["cache_ids"][h] & mask, n, cfg.tau, f"{what} head {h}")
        worst, ties = max(worst, err), ties + t
    print(f"search {what}: max cos err {worst:.2e}, {ties} argmax near-ties")


def oracle_annsa(prep, n, q_ids=None, kcur_ids=None, cache_ids=None, heads=None, use_cache=True):
    st, cfg = prep["step"], prep["cfg"]
    q_ids = prep["q_ids"] if q_ids is None else q_ids
    kcur_ids = prep["k_cur_ids"] if kcur_ids is None else kcur_ids
    cache_ids = prep["cache_ids"] if cache_ids is None else cache_ids
    Os, Ls = [], []
    for h in (range(cfg.H) if heads is None else heads):
        nn = n if use_cache else 0
        K, V, kid = key_context(st.cache_k[h], st.cache_v[h], cache_ids[h], nn, st.k_cur[h],
                                st.v_cur[h], kcur_ids[h])
        O, L = o_annsa(st.q[h], q_ids[h], K, V, kid, st.scale)
        Os.append(O)
        Ls.append(L)
    return np.stack(Os), np.stack(Ls)


def check_lse(lse_gpu, lse_ref):
    g = lse_gpu.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(g), fin)
    assert (np.isneginf(g) == np.isneginf(lse_ref)).all()
    if fin.any():
        assert np.abs(g[fin] - lse_ref[fin]).max() <= LSE_ABS


def run(prep, cache=None, q_ids=None, kcur_ids=None, P=None, out_dtype=torch.float32):
    st, cfg = prep["step"], prep["cfg"]
    q_ids = prep["q_ids"] if q_ids is None else q_ids
    kcur_ids = prep["k_cur_ids"] if kcur_ids is None else kcur_ids
    return fa.annsa_forward(dev(st.q, cfg.dtype), dev_ids(q_ids), dev(st.k_cur, cfg.dtype),
                            dev(st.v_cur, cfg.dtype), dev_ids(kcur_ids), cfg.P if P is None else P,
                            cache=cache, out_dtype=out_dtype)


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_annsa_matches_oracle(name):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    out, lse = run(prep, cache=device_cache(prep))
    O, L = oracle_annsa(prep, cfg.n0)
    err = assert_attention_close(out, O, cfg.dtype, f"annsa {name}")
    check_lse(lse, L)
    print(f"annsa {name}: max err {err:.3e}")


@pytest.mark.parametrize("H", [3, 5])
def test_annsa_head_counts_off_the_block_rounds(H):
    """Head counts whose (heads x work-list entries) grid is not a whole number
    of rounds of eight four-item runs (3 x 24 and 5 x 24 entries at the tiny
    shape): part of the grid takes the XCD-run block order and the rest the
    plain order.  Every item must still run exactly once: outputs, lse and
    the fused search on every head against the oracle."""
    require_gpu()
    prep = prepared("tiny_f32", H=H)
    st, cfg = prep["step"], prep["cfg"]
    out, lse, best, bcos = fa.annsa_forward(dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
                                            dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]), cfg.P,
                                            cache=device_cache(prep), search=True)
    O, L = oracle_annsa(prep, cfg.n0)
    assert_attention_close(out, O, cfg.dtype, f"annsa H={H}")
    check_lse(lse, L)
    check_search(prep, best, bcos, cfg.n0, what=f"H={H}")


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16"])
def test_annsa_one_bucket_is_dense(name):
    require_gpu()
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    z = lambda a: np.zeros_like(a)
    cache = device_cache(prep)
    cache.ids.zero_()
    out, lse = run(prep, cache=cache, q_ids=z(prep["q_ids"]), kcur_ids=z(prep["k_cur_ids"]), P=0)
    O, L = oracle_annsa(prep, cfg.n0, q_ids=z(prep["q_ids"]), kcur_ids=z(prep["k_cur_ids"]),
                        cache_ids=z(prep["cache_ids"]))
    assert_attention_close(out, O, cfg.dtype, f"dense {name}")
    check_lse(lse, L)


def test_annsa_partial_cache_and_no_cache():
    require_gpu()
    prep = prepared("single_bf16")
    cfg = prep["cfg"]
    n = cfg.cap // 2 + 37
    out, lse = run(prep, cache=device_cache(prep, n=n))
    O, L = oracle_annsa(prep, n)
    assert_attention_close(out, O, cfg.dtype, "partial cache")
    check_lse(lse, L)
    out, lse = run(prep, cache=None)
    O, L = oracle_annsa(prep, 0, use_cache=False)
    assert_attention_close(out, O, cfg.dtype, "no cache")
    check_lse(lse, L)


def test_annsa_empty_buckets():
    require_gpu()
    prep = prepared("tiny_f32")
    st, cfg = prep["step"], prep["cfg"]
    rng = np.random.default_rng(0)
    q_ids = rng.integers(0, 16, size=prep["q_ids"].shape).astype(np.uint16)
    k_ids = rng.integers(0, 8, size=prep["k_cur_ids"].shape).astype(np.uint16)
    c_ids = rng.integers(0, 8, size=prep["cache_ids"].shape).astype(np.uint16)
    cache = device_cache(prep)
    cache.ids.copy_(dev_ids(c_ids))
    out, lse = run(prep, cache=cache, q_ids=q_ids, kcur_ids=k_ids)
    O, L = oracle_annsa(prep, cfg.n0, q_ids=q_ids, kcur_ids=k_ids, cache_ids=c_ids)
    assert np.isneginf(L).sum() > 50
    assert_attention_close(out, O, cfg.dtype, "empty buckets")
    check_lse(lse, L)


def test_annsa_bf16_output_and_determinism():
    require_gpu()
    prep = prepared("wan13_bf16")
    cfg = prep["cfg"]
    cache = device_cache(prep)
    out_b, _ = run(prep, cache=cache, out_dtype=torch.bfloat16)
    heads = [0, 5, 11]
    O, _ = oracle_annsa(prep, cfg.n0, heads=heads)
    assert_attention_close(out_b[heads], O, cfg.dtype, "bf16 out")
    a, la = run(prep, cache=cache)
    b, lb = run(prep, cache=cache)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("name,P,heads", [("single_bf16", 1, None), ("single_bf16", 2, None),
                                          ("tiny_f32", 0, None), ("wan13_bf16", 3, (0, 7))])
@pytest.mark.parametrize("partial", [False, True])
def test_annsa_wide_items(name, P, heads, partial):
    """Buckets from the low P bits of the step's ids (a P-plane hash): every
    bucket averages >= 256 queries, so the call runs 256-query items."""
    require_gpu()
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    assert (256 << P) <= cfg.Nq
    m = (1 << P) - 1
    q_ids, k_ids, c_ids = (prep[k] & m for k in ("q_ids", "k_cur_ids", "cache_ids"))
    n = cfg.cap // 2 + 37 if partial else cfg.n0
    cache = device_cache(prep, n=n)
    cache.ids.copy_(dev_ids(c_ids))
    out, lse = run(prep, cache=cache, q_ids=q_ids, kcur_ids=k_ids, P=P)
    hs = list(range(cfg.H)) if heads is None else list(heads)
    O, L = oracle_annsa(prep, n, q_ids=q_ids, kcur_ids=k_ids, cache_ids=c_ids, heads=hs)
    assert_attention_close(out[hs], O, cfg.dtype, f"wide {name} P={P}")
    check_lse(lse[hs], L)


def test_annsa_wide_items_empty_bucket():
    """Wide items for a bucket whose queries have no keys: O = 0, lse = -inf."""
    require_gpu()
    prep = prepared("single_bf16")
    st, cfg = prep["step"], prep["cfg"]
    P = 2
    q_ids = prep["q_ids"] & 3
    k_ids = np.minimum(prep["k_cur_ids"] & 3, 2).astype(np.uint16)
    c_ids = np.minimum(prep["cache_ids"] & 3, 2).astype(np.uint16)
    cache = device_cache(prep)
    cache.ids.copy_(dev_ids(c_ids))
    out, lse = run(prep, cache=cache, q_ids=q_ids, kcur_ids=k_ids, P=P)
    O, L = oracle_annsa(prep, cfg.n0, q_ids=q_ids, kcur_ids=k_ids, cache_ids=c_ids)
    assert np.isneginf(L).sum() == int((q_ids == 3).sum()) > 0
    assert_attention_close(out, O, cfg.dtype, "wide, empty bucket")
    check_lse(lse, L)


@pytest.mark.parametrize("search", [False, True])
def test_annsa_f32_d128(search):
    """fp32 inputs at d = 128 (the register-heavy kernel form) against the oracle."""
    require_gpu()
    prep = prepared("tiny_f32", d=128)
    st, cfg = prep["step"], prep["cfg"]
    cache = device_cache(prep)
    res = fa.annsa_forward(dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
                           dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]), cfg.P, cache=cache,
                           search=search)
    O, L = oracle_annsa(prep, cfg.n0)
    assert_attention_close(res[0], O, cfg.dtype, f"f32 d=128 search={search}")
    check_lse(res[1], L)
    if search:
        check_search(prep, res[2], res[3], cfg.n0, what="f32 d=128")


@pytest.mark.parametrize("Fc,cap", [(300, 80000), (550, 150000)])
def test_annsa_long_key_set(Fc, cap):
    """Caches of 76 800 and 140 800 keys (75 and 138 sort tiles per head with
    the chunk: the second takes the sort's scan-launch form) with the fused
    search, against the oracle."""
    require_gpu()
    prep = prepared("tiny_f32", Fc=Fc, cap=cap)
    st, cfg = prep["step"], prep["cfg"]
    assert cfg.n0 == Fc * 256
    cache = device_cache(prep)
    out, lse, best, bcos = fa.annsa_forward(dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
                                            dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]), cfg.P,
                                            cache=cache, search=True)
    O, L = oracle_annsa(prep, cfg.n0)
    assert_attention_close(out, O, cfg.dtype, "long key set")
    check_lse(lse, L)
    check_search(prep, best, bcos, cfg.n0, what=f"cache {cfg.n0}")


@pytest.mark.parametrize("P", [9, 10])
def test_annsa_many_buckets(P):
    """512 and 1024 buckets (the most the bucketed calls take): the sort's
    several-buckets-per-thread paths, with the fused search, against the oracle."""
    require_gpu()
    prep = prepared("single_bf16", P=P)
    st, cfg = prep["step"], prep["cfg"]
    cache = device_cache(prep)
    out, lse, best, bcos = fa.annsa_forward(dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
                                            dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]), P, cache=cache,
                                            search=True)
    O, L = oracle_annsa(prep, cfg.n0)
    assert_attention_close(out, O, cfg.dtype, f"P={P}")
    check_lse(lse, L)
    check_search(prep, best, bcos, cfg.n0, P=P, what=f"P={P}")

"""GPU parity of fastar_ann_hash and fastar_bucket_sort against the oracle."""
import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import ann_hash as o_hash, bucket_sort as o_sort
from tests.gpu_util import (assert_ids_match, dev, dev_ids, host_ids, prepared, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_hash_matches_oracle_on_workloads(name):
    require_gpu()
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    planes = torch.from_numpy(st.planes).cuda()
    flagged = 0
    for key, arr in (("q", st.q), ("k_cur", st.k_cur), ("cache", st.cache_k), ("kp", st.kp)):
        ids = host_ids(fa.ann_hash(dev(arr, cfg.dtype), planes))
        flagged += assert_ids_match(ids, prep[key + "_ids"], prep[key + "_tie"], f"{name}/{key}")
    torch.cuda.synchronize()
    print(f"{name}: {flagged} flagged ids differ (allowed)")


@pytest.mark.parametrize("dtype,d,P,N", [("f32", 64, 0, 100), ("f32", 128, 16, 333),
                                         ("bf16", 64, 9, 1025), ("bf16", 128, 16, 4097),
                                         ("bf16", 128, 1, 1)])
def test_hash_random_shapes(dtype, d, P, N):
    require_gpu()
    rng = np.random.default_rng(N + P)
    H = 3
    x = rng.standard_normal((H, N, d)).astype(np.float32)
    if dtype == "bf16":
        from workloads import bf16_round
        x = bf16_round(x)
    planes = rng.standard_normal((H, P, d)).astype(np.float32)
    ids = host_ids(fa.ann_hash(dev(x, dtype), torch.from_numpy(planes).cuda()))
    for h in range(H):
        ref, tie = o_hash(x[h], planes[h])
        assert_ids_match(ids[h], ref, tie, f"head {h}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_hash_norms(dtype, d):
    """The optional norm output equals |x| (fp32 sum of squares of the stored values)."""
    require_gpu()
    rng = np.random.default_rng(d)
    x = rng.standard_normal((2, 777, d)).astype(np.float32) * 3
    if dtype == "bf16":
        from workloads import bf16_round
        x = bf16_round(x)
    x[0, 5] = 0.0
    norms = torch.empty(2, 777, dtype=torch.float32, device="cuda")
    fa.ann_hash(dev(x, dtype), torch.from_numpy(rng.standard_normal((2, 3, d)).astype(np.float32)).cuda(),
                norms=norms)
    ref = np.linalg.norm(x.astype(np.float64), axis=2)
    np.testing.assert_allclose(norms.cpu().numpy(), ref, rtol=2e-6, atol=0)
    assert norms[0, 5].item() == 0.0


@pytest.mark.parametrize("P,N", [(0, 17), (3, 0), (5, 1), (7, 1023), (7, 1025), (7, 37440),
                                 (10, 5000), (8, 4096),
                                 # past 128 tiles per head the sort adds a scan launch
                                 (7, 65537), (10, 100000), (0, 140000), (9, 299520), (7, 131073)])
def test_bucket_sort_bit_exact(P, N):
    require_gpu()
    rng = np.random.default_rng(10 * P + N)
    H = 4
    # skewed bucket sizes, like the workloads' clusters
    w = rng.dirichlet(np.full(1 << P, 0.3))
    ids = rng.choice(1 << P, size=(H, N), p=w).astype(np.uint16)
    off, perm = fa.bucket_sort(dev_ids(ids), P)
    off2, perm2 = fa.bucket_sort(dev_ids(ids), P)
    off, perm = off.cpu().numpy(), perm.cpu().numpy()
    for h in range(H):
        ro, rp = o_sort(ids[h], P)
        assert np.array_equal(off[h], ro)
        assert np.array_equal(perm[h], rp)
    assert torch.equal(off2.cpu(), torch.from_numpy(off)) and torch.equal(perm2.cpu(), torch.from_numpy(perm))


def test_bucket_sort_ignores_high_bits():
    require_gpu()
    ids = np.array([[5, 5 + 8, 2, 2 + 64, 7]], np.uint16)
    off, perm = fa.bucket_sort(dev_ids(ids), 3)
    ro, rp = o_sort(ids[0] & 7, 3)
    assert np.array_equal(off.cpu().numpy()[0], ro) and np.array_equal(perm.cpu().numpy()[0], rp)


@pytest.mark.parametrize("name", ["tiny_f32", "wan13_bf16"])
def test_hash_batch_equals_single_calls(name):
    """One launch over the step's queries, current keys and prompt keys (three
    sizes) gives the ids and norms of three separate calls, bit for bit."""
    require_gpu()
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    planes = torch.from_numpy(st.planes).cuda()
    xs = [dev(a, cfg.dtype) for a in (st.q, st.k_cur, st.kp)]
    norms = [torch.empty(cfg.H, x.shape[1], dtype=torch.float32, device="cuda") for x in xs]
    got = fa.ann_hash_batch(xs, planes, norms=norms)
    for x, g, nb in zip(xs, got, norms):
        n1 = torch.empty_like(nb)
        one = fa.ann_hash(x, planes, norms=n1)
        assert torch.equal(one, g) and torch.equal(n1, nb)

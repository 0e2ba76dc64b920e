"""The no-allocation AnnSA entry point, fastar_annsa_forward_static, called
through the C ABI against fastar_annsa_forward on the same inputs: two calls
in a row on the library's static scratch array, the first at the
Wan-1.3B-like layer (2.2 MiB of scratch) and the second at the smaller
single-head shape, both with the fused TempCache search.  The two entry
points run the same kernels on the same inputs, so every output must agree
bit for bit (stricter than the oracle tolerances), and the first call's
leftovers in the array must not change the second call's results."""
import ctypes

import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from sparse_attention_autoregressive_amd import _lib
from tests.gpu_util import dev, dev_ids, device_cache, prepared, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(name):
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    return cfg, device_cache(prep), (dev(st.q, cfg.dtype), dev_ids(prep["q_ids"]), dev(st.k_cur, cfg.dtype),
                                     dev(st.v_cur, cfg.dtype), dev_ids(prep["k_cur_ids"]))


def _static_call(cfg, cache, q, qi, kc, vc, ki):
    """fastar_annsa_forward_static through ctypes, outputs allocated here."""
    H, Nq, d = q.shape
    out = torch.full((H, Nq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    best = torch.full((H, Nq), -7, dtype=torch.int32, device="cuda")
    bcos = torch.full((H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    cs = cache.struct()
    st = _lib.load().fastar_annsa_forward_static(
        q.data_ptr(), qi.data_ptr(), H, Nq, d, 1 if cfg.dtype == "bf16" else 0, ctypes.byref(cs),
        kc.data_ptr(), vc.data_ptr(), ki.data_ptr(), kc.shape[1], cfg.P, 1.0 / d ** 0.5, out.data_ptr(), 0,
        lse.data_ptr(), best.data_ptr(), bcos.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == _lib.FASTAR_OK, _lib.load().fastar_status_string(st)
    return out, lse, best, bcos


def test_static_scratch_matches_workspace_entry_two_calls():
    require_gpu()
    for name in ("wan13_bf16", "single_bf16"):           # the second call is smaller
        cfg, cache, (q, qi, kc, vc, ki) = _inputs(name)
        print(f"no-alloc AnnSA: {name}", flush=True)
        got = _static_call(cfg, cache, q, qi, kc, vc, ki)
        ref = fa.annsa_forward(q, qi, kc, vc, ki, cfg.P, cache=cache, search=True)
        torch.cuda.synchronize()
        for what, a, b in zip(("out", "lse", "best", "best_cos"), got, ref):
            assert torch.equal(a, b), f"{name}: {what} differs from fastar_annsa_forward"
        assert (got[2] >= -1).all()


def test_static_scratch_binding_and_oversize_rejection():
    require_gpu()
    cfg, cache, (q, qi, kc, vc, ki) = _inputs("tiny_f32")
    o, l, b, c = fa.annsa_forward_static(q, qi, kc, vc, ki, cfg.P, cache=cache, search=True)
    o2, l2, b2, c2 = fa.annsa_forward(q, qi, kc, vc, ki, cfg.P, cache=cache, search=True)
    assert torch.equal(o, o2) and torch.equal(l, l2) and torch.equal(b, b2) and torch.equal(c, c2)
    # a call whose workspace exceeds the array is refused before anything runs
    big = fa.KVCache.empty(8, 600_000, 128, dtype=torch.bfloat16)
    assert _lib.load().fastar_annsa_workspace(8, 4680, 600_000, 4680, 10) > _lib.FASTAR_STATIC_SCRATCH_BYTES
    qb = torch.zeros(8, 4680, 128, dtype=torch.bfloat16, device="cuda")
    ib = torch.zeros(8, 4680, dtype=torch.int16, device="cuda")
    with pytest.raises(fa.FastarError, match="FASTAR_ESCRATCH"):
        fa.annsa_forward_static(qb, ib, qb, qb, ib, 10, cache=big)

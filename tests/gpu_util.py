"""Shared helpers of the GPU parity tests: moving seeded inputs to the device
and the comparison rules.

Tolerances
----------
* attention outputs (fp32 output buffers): max|err| <= 1e-2 * RMS(oracle) for
  bf16 inputs, <= 1e-4 absolute for fp32 inputs;
* bf16 output buffers add the output's own rounding: one bf16 ulp of the
  oracle value, 2**-8 * |O| (half an ulp is the rounding bound; a full ulp
  also covers values that sit next to a rounding boundary);
* log-sum-exp: 1e-3 absolute.  A logit is an fp32 sum of d exact bf16 (or
  fp32) products of magnitude up to |q||k|*scale (about 25 here); its error is
  below d * 2**-24 * 25 < 2e-4, and the lse inherits at most that;
* cosines of the TempCache search: 1e-5 absolute, the width of the oracle's
  threshold-tie flag.  A cosine is an fp32 sum of d products whose
  magnitudes add up to at most |q||k|: bf16 products are exact and fp32
  products carry one rounding each (at most 2**-24 |q||k| in all), and the
  sum's error is below (d - 1) * 2**-24 |q||k|, so the dot product is within
  d * 2**-24 ~ 7.6e-6 of |q||k| at d = 128; 1/|q| and 1/|k| add a few fp32
  ulps.  Match decisions (cos >= tau, taken in fp32 on the GPU) must agree
  with the oracle's for every token outside the flag;
* integers (bucket ids, permutations, keep masks, slots, counts): bit-exact,
  except tokens the oracle flags as within 1e-5 of a hash or argmax tie.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from workloads import f32_to_bf16_bits

ATTN_REL_RMS_BF16 = 1e-2
ATTN_ABS_F32 = 1e-4
LSE_ABS = 1e-3
COS_ABS = 1e-5
TIE_EPS = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 values (already representable in ``dtype``) -> device tensor."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(np.ascontiguousarray(a, np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_ids(ids: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(ids, np.uint16).view(np.int16)).cuda()


def host_ids(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_attention_close(gpu: torch.Tensor, ref: np.ndarray, in_dtype: str, what: str,
                           rows=None):
    g = to_f64(gpu)
    r = np.asarray(ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    err = np.abs(g - r)
    if in_dtype == "bf16":
        rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
        tol = ATTN_REL_RMS_BF16 * rms
        if gpu.dtype == torch.bfloat16:
            tol = tol + 2.0 ** -8 * np.abs(r)
        bad = err > tol
    else:
        tol = ATTN_ABS_F32
        if gpu.dtype == torch.bfloat16:
            tol = tol + 2.0 ** -8 * np.abs(r)
        bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3e}, rms(ref) {np.sqrt(np.mean(r ** 2)):.3e}")
    return float(err.max()) if err.size else 0.0


def assert_ids_match(gpu_ids: np.ndarray, ref_ids: np.ndarray, tie_bits: np.ndarray, what: str):
    g = gpu_ids.astype(np.int64)
    r = ref_ids.astype(np.int64)
    t = tie_bits.astype(np.int64)
    diff = g ^ r
    assert not (diff & ~t).any(), f"{what}: {int(((diff & ~t) != 0).sum())} ids differ outside flagged bits"
    return int((diff != 0).sum())


# ---------------------------------------------------------------- workloads
import functools  # noqa: E402

from oracle import ann_hash  # noqa: E402
from workloads import CONFIGS, make_step  # noqa: E402


@functools.lru_cache(maxsize=4)
def prepared(name: str, seed: int = 0, **overrides):
    """A seeded step plus the oracle's bucket ids of every token set.

    The oracle's ids are the inputs of the bucketed GPU calls in the stage
    tests, so each stage is compared on identical inputs."""
    cfg = CONFIGS[name].replace(**overrides) if overrides else CONFIGS[name]
    st = make_step(cfg, seed)
    out = {"step": st, "cfg": cfg}
    for key, arr in (("q", st.q), ("k_cur", st.k_cur), ("cache", st.cache_k), ("kp", st.kp)):
        ids, ties = zip(*(ann_hash(arr[h], st.planes[h]) for h in range(cfg.H)))
        out[key + "_ids"] = np.stack(ids)
        out[key + "_tie"] = np.stack(ties)
    return out


def device_cache(prep, n=None):
    """KVCache on the device holding the step's initial cache: bucket ids from the
    oracle (the same inputs both sides get), key norms from the library's hash."""
    import sparse_attention_autoregressive_amd as fa
    st, cfg = prep["step"], prep["cfg"]
    n_valid = st.n_valid if n is None else np.full(cfg.H, n, np.int32)
    k = dev(st.cache_k, cfg.dtype)
    knorm = torch.empty(cfg.H, cfg.cap, dtype=torch.float32, device="cuda")
    fa.ann_hash(k, torch.from_numpy(st.planes).cuda(), norms=knorm)
    return fa.KVCache(k=k, v=dev(st.cache_v, cfg.dtype), ids=dev_ids(prep["cache_ids"]),
                      ts=torch.from_numpy(st.cache_ts).cuda(),
                      n_valid=torch.from_numpy(np.ascontiguousarray(n_valid, np.int32)).cuda(),
                      knorm=knorm)


def assert_top1_matches(best_gpu, cos_gpu, q, q_ids, cache_k, cache_ids, n, tau, what):
    """TempCache top-1 of one head against the oracle, under the tie protocol:
    the slot must be the oracle's except where it flags an argmax near-tie
    (then one of the near-maximal slots), the cosine within COS_ABS, and the
    match decision (cos >= tau) the oracle's except where |cos - tau| is
    within the flag.  Returns (max cosine error, argmax flags, threshold flags)."""
    from oracle import tempcache_top1
    best_gpu = np.asarray(best_gpu)
    cos_gpu = np.asarray(cos_gpu).astype(np.float64)
    ob, oc, tie, near = tempcache_top1(q, q_ids, cache_k, cache_ids, n)
    ok = ~tie
    bad = np.nonzero(best_gpu[ok] != ob[ok])[0]
    assert bad.size == 0, f"{what}: {bad.size} slots differ outside argmax ties"
    for i in np.nonzero(tie)[0]:
        assert best_gpu[i] in near[i], f"{what}: token {i} slot {best_gpu[i]} not near-maximal"
    fin = np.isfinite(oc)
    assert np.array_equal(np.isfinite(cos_gpu), fin), f"{what}: no-candidate tokens differ"
    err = float(np.abs(cos_gpu[fin] - oc[fin]).max()) if fin.any() else 0.0
    assert err <= COS_ABS, f"{what}: cosine error {err:.3e}"
    thr = fin & (np.abs(oc - tau) < TIE_EPS)
    m_gpu = (best_gpu >= 0) & (cos_gpu.astype(np.float32) >= np.float32(tau))
    m_ref = (ob >= 0) & (oc >= tau)
    assert np.array_equal(m_gpu[~thr], m_ref[~thr]), f"{what}: match decisions differ outside ties"
    return err, int(tie.sum()), int(thr.sum())

"""GPU parity of fastar_annca_forward against the oracle: keep masks and counts
bit-exact, outputs within tolerance; workloads as generated (nearly every
prompt token kept), constructed ids that prune most of the prompt, frames with
nothing kept, an empty prompt, fp32 / bf16 at d = 64 and 128 with frames
that end in a partial block, prompts on either side of the longest one
whose selection the attention blocks do themselves, and logits that grow or
shrink by hundreds of powers of two along the kept list (the softmax's
reference then moves, or stays, across many tiles)."""
import numpy as np
import pytest
import torch

import sparse_attention_autoregressive_amd as fa
from oracle import annca as o_annca
from workloads.gen import bf16_round
from tests.gpu_util import assert_attention_close, dev, dev_ids, prepared, require_gpu

pytestmark = pytest.mark.gpu


def run_and_check(prep, q_ids, kp_ids, P, what, out_dtype=torch.float32, kp=None, vp=None):
    st, cfg = prep["step"], prep["cfg"]
    kp = st.kp if kp is None else kp
    vp = st.vp if vp is None else vp
    out, keep, cnt = fa.annca_forward(dev(st.q, cfg.dtype), dev_ids(q_ids), cfg.frame_len,
                                      dev(kp, cfg.dtype), dev(vp, cfg.dtype), dev_ids(kp_ids), P,
                                      out_dtype=out_dtype)
    Os, Ks = [], []
    for h in range(cfg.H):
        O, keep_ref = o_annca(st.q[h], q_ids[h], cfg.frame_len, kp[h], vp[h], kp_ids[h], st.scale)
        Os.append(O)
        Ks.append(keep_ref)
    keep_ref = np.stack(Ks)
    assert np.array_equal(keep.cpu().numpy().astype(bool), keep_ref), what
    assert np.array_equal(cnt.cpu().numpy(), keep_ref.sum(-1)), what
    assert_attention_close(out, np.stack(Os), cfg.dtype, what)
    return keep_ref


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "wan13_bf16"])
def test_annca_matches_oracle(name):
    require_gpu()
    prep = prepared(name)
    keep = run_and_check(prep, prep["q_ids"], prep["kp_ids"], prep["cfg"].P, f"annca {name}")
    print(f"annca {name}: kept {keep.mean():.3f}")


@pytest.mark.parametrize("name", ["tiny_f32", "wan13_bf16"])
def test_annca_pruned(name):
    require_gpu()
    prep = prepared(name)
    cfg = prep["cfg"]
    rng = np.random.default_rng(1)
    B = 1 << cfg.P
    F = cfg.Nq // cfg.frame_len
    q_ids = np.empty_like(prep["q_ids"])
    for f in range(F):   # each frame occupies its own small set of buckets
        lo = (f * 5) % max(1, B - 8)
        q_ids[:, f * cfg.frame_len:(f + 1) * cfg.frame_len] = rng.integers(lo, lo + 6, size=(cfg.H, cfg.frame_len))
    kp_ids = rng.integers(0, B, size=prep["kp_ids"].shape).astype(np.uint16)
    keep = run_and_check(prep, q_ids.astype(np.uint16), kp_ids, cfg.P, f"pruned {name}")
    assert 0 < keep.mean() < 0.5
    keep = run_and_check(prep, q_ids.astype(np.uint16), kp_ids, cfg.P, f"pruned bf16 out {name}",
                         out_dtype=torch.bfloat16)


def test_annca_nothing_kept_and_empty_prompt():
    require_gpu()
    prep = prepared("single_bf16")
    cfg = prep["cfg"]
    q_ids = np.zeros_like(prep["q_ids"])
    kp_ids = np.ones_like(prep["kp_ids"])
    keep = run_and_check(prep, q_ids, kp_ids, cfg.P, "nothing kept")
    assert not keep.any()
    st = prep["step"]
    empty = np.zeros((cfg.H, 0, cfg.d), np.float32)
    run_and_check(prep, prep["q_ids"], np.zeros((cfg.H, 0), np.uint16), cfg.P, "empty prompt",
                  kp=empty, vp=empty)


@pytest.mark.parametrize("name,d", [("tiny_f32", 128), ("tiny_f32", 64), ("single_bf16", 64),
                                    ("single_bf16", 128)])
def test_annca_dtypes_widths_ragged_frames(name, d):
    """Three frames of 200 queries (fp32 d = 128 blocks take 64 queries, the
    others 128: every frame ends in a partial block), P = 2 so some prompt
    tokens are pruned per frame."""
    require_gpu()
    prep = prepared(name, d=d, frame_len=200, Fq=3, Fc=2)
    cfg = prep["cfg"]
    assert cfg.Nq == 600
    P = 2
    rng = np.random.default_rng(d)
    q_ids = np.empty_like(prep["q_ids"])
    for f in range(3):      # frame f occupies buckets {f, f + 1} only
        q_ids[:, f * 200:(f + 1) * 200] = rng.integers(f, f + 2, size=(cfg.H, 200))
    kp_ids = (prep["kp_ids"] & 3).astype(np.uint16)
    keep = run_and_check(prep, q_ids.astype(np.uint16), kp_ids, P, f"ragged {name} d={d}")
    assert 0 < keep.mean() < 1


@pytest.mark.parametrize("P", [9, 10])
def test_annca_many_buckets(P):
    """512 and 1024 buckets: the selection's bucket bitmap at its largest."""
    require_gpu()
    prep = prepared("single_bf16", P=P)
    keep = run_and_check(prep, prep["q_ids"], prep["kp_ids"], P, f"annca P={P}")
    assert 0 < keep.mean() < 1


@pytest.mark.parametrize("L", [1000, 1024, 1025, 2100])
def test_annca_prompt_lengths_around_the_fused_selection(L):
    """Up to 1024 prompt tokens every attention block selects its frame's
    prompt tokens in LDS (no workspace); a longer prompt takes the separate
    selection launch and its index list, which the blocks then stage in
    chunks of 1024 (2100 kept tokens: three chunks, the last one ragged).
    Two frames of 600 queries; as generated (nearly everything kept) and with
    each frame confined to six buckets (most of the prompt pruned)."""
    require_gpu()
    prep = prepared("single_bf16", L=L, frame_len=600, Fq=2, Fc=2)
    cfg = prep["cfg"]
    assert prep["kp_ids"].shape == (1, L)
    need = fa.load().fastar_annca_workspace(cfg.H, cfg.Nq, cfg.frame_len, L, cfg.P)
    assert (need == 0) == (L <= 1024)
    keep = run_and_check(prep, prep["q_ids"], prep["kp_ids"], cfg.P, f"annca L={L}")
    assert keep.mean() > 0.9
    rng = np.random.default_rng(L)
    q_ids = np.empty_like(prep["q_ids"])
    for f in range(2):
        q_ids[:, f * 600:(f + 1) * 600] = rng.integers(10 * f, 10 * f + 6, size=(cfg.H, 600))
    kp_ids = rng.integers(0, cfg.B, size=(cfg.H, L)).astype(np.uint16)
    keep = run_and_check(prep, q_ids.astype(np.uint16), kp_ids, cfg.P, f"annca pruned L={L}",
                         out_dtype=torch.bfloat16)
    assert 0 < keep.mean() < 0.3


@pytest.mark.parametrize("frame_len,Fq", [(201, 3), (7, 5), (1, 4)])
def test_annca_unaligned_frames(frame_len, Fq):
    """Frames whose query ids start at any offset: the selection inside the
    attention blocks reads them in 16-byte loads with a scalar run before and
    after the aligned part (201 ids: both; 7 and 1: the whole frame scalar),
    and every frame confines its queries to a few buckets so the keep masks
    differ from frame to frame."""
    require_gpu()
    prep = prepared("single_bf16", frame_len=frame_len, Fq=Fq, Fc=2, P=5)
    cfg = prep["cfg"]
    assert cfg.Nq == frame_len * Fq
    rng = np.random.default_rng(frame_len)
    q_ids = np.empty_like(prep["q_ids"])
    for f in range(Fq):
        q_ids[:, f * frame_len:(f + 1) * frame_len] = rng.integers(3 * f, 3 * f + 4, size=(cfg.H, frame_len))
    kp_ids = rng.integers(0, cfg.B, size=prep["kp_ids"].shape).astype(np.uint16)
    keep = run_and_check(prep, q_ids.astype(np.uint16), kp_ids, cfg.P, f"unaligned frames {frame_len}x{Fq}")
    assert 0 < keep.mean() < 0.5


@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16"])
@pytest.mark.parametrize("ramp", [1.0, -1.0])
def test_annca_logits_spanning_many_tiles(name, ramp):
    """Every prompt token kept (P = 0), scale 1, and prompt keys that move
    along the queries' mean direction with the token index: the logits of a
    query grow (ramp 1, for most queries) or shrink (ramp -1) by about 300 in
    natural units over the kept list, so the softmax's reference has to move
    many times, or never after the first tile, while the outputs stay within
    tolerance of the oracle."""
    require_gpu()
    prep = prepared(name)
    st, cfg = prep["step"], prep["cfg"]
    rng = np.random.default_rng(7)
    L = st.kp.shape[1]
    kp = np.empty_like(st.kp)
    for h in range(cfg.H):
        u = st.q[h].mean(0)
        u = u / np.linalg.norm(u)
        proj = st.q[h] @ u
        c = ramp * 300.0 / max(float(np.abs(proj).mean()), 1e-3) * (np.arange(L) / L - 0.5)
        kp[h] = c[:, None] * u[None, :] + 0.05 * rng.standard_normal((L, cfg.d))
    if cfg.dtype == "bf16":
        kp = bf16_round(kp.astype(np.float32))
    kp = kp.astype(np.float32)
    zq = np.zeros_like(prep["q_ids"])
    zk = np.zeros((cfg.H, L), np.uint16)
    out, keep, _ = fa.annca_forward(dev(st.q, cfg.dtype), dev_ids(zq), cfg.frame_len, dev(kp, cfg.dtype),
                                    dev(st.vp, cfg.dtype), dev_ids(zk), 0, scale=1.0)
    assert keep.cpu().numpy().all()
    Os = [o_annca(st.q[h], zq[h], cfg.frame_len, kp[h], st.vp[h], zk[h], 1.0)[0] for h in range(cfg.H)]
    assert_attention_close(out, np.stack(Os), cfg.dtype, f"annca ramp {ramp} {name}")

"""The seeded generator: determinism, per-head independence, bf16 rounding."""
import numpy as np
import torch

from workloads import CONFIGS, bf16_round, f32_to_bf16_bits, make_step, rollout_chunks


def test_deterministic_and_head_subsets_match():
    cfg = CONFIGS["tiny_f32"].replace(H=3)
    a = make_step(cfg, seed=0)
    b = make_step(cfg, seed=0)
    c = make_step(cfg, seed=0, heads=range(1, 3))
    for name in ("q", "k_cur", "v_cur", "cache_k", "cache_v", "planes", "kp", "vp"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
        assert np.array_equal(getattr(a, name)[1:], getattr(c, name))
    assert not np.array_equal(make_step(cfg, seed=1).q, a.q)


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    assert np.array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_shapes_and_structure():
    cfg = CONFIGS["single_bf16"]
    st = make_step(cfg, seed=0)
    assert st.q.shape == (1, 1560, 128) and st.cache_k.shape == (1, 9360, 128)
    assert st.kp.shape == (1, 512, 128) and st.planes.shape == (1, 6, 128)
    assert st.cache_ts[0, 0] == 0 and st.cache_ts[0, -1] == 5 and st.step == 6
    assert np.array_equal(bf16_round(st.q), st.q)            # stored values are bf16
    # drift: the current frame is close to the last cached frame, position by position
    diff = st.k_cur[0] - st.cache_k[0, -1560:]
    assert 0.03 < diff.std() < 0.08


def test_rollout_first_chunk_is_the_step_chunk():
    cfg = CONFIGS["tiny_f32"].replace(H=2)
    st = make_step(cfg, seed=0)
    it = rollout_chunks(cfg, 3, seed=0)
    c0 = next(it)
    assert np.array_equal(c0["q"], st.q) and np.array_equal(c0["v_cur"], st.v_cur)
    c1 = next(it)
    assert c1["step"] == cfg.Fc + cfg.Fq
    moved = np.abs(c1["k_cur"] - c0["k_cur"]).max(axis=2) > 1.0
    assert 0 < moved.mean() < 0.2          # ~5% of positions re-drawn


def test_commit_case_is_seeded_and_in_range():
    from workloads import commit_case
    a = commit_case(3, 2, 100, 300, 64, [300, 200], 5, pool=10)
    b = commit_case(3, 2, 100, 300, 64, [300, 200], 5, pool=10)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["cache_ids"].max() < 32 and a["kcur_ids"].max() < 32
    assert (a["best"][1] < 10).all() and (a["best"] >= -1).all()
    assert a["cos"].dtype == np.float32 and a["cache_k"].shape == (2, 300, 64)

"""Seeded generator of synthetic FAST-AR attention-step inputs.

The workloads stand in for the video-diffusion rollouts the FAST-AR pages
measure on (Rolling-Forcing / LongVie2 on LongVBench and LongVGenBench, page
"Fast Autoregressive Video Diffusion ... " on gist.science, section "Key
Results"): no dataset or trained weight is used. Their structure follows the
redundancy the pages describe (page 2, "Motivation: Sources of Redundancy"):
keys cluster around semantic centroids, persist from frame to frame with a
small drift, and queries sit near their own token's key.

Recipe, per head h (its own ``PCG64(SeedSequence([seed, h]))`` stream, draws
in exactly this order, all ``float32``):

1. ``mu``      [C, d]   centroids ~ N(0, 1)
2. ``assign``  [frame_len] centroid of each grid position, uniform on 0..C-1
3. frame 0:    k = mu[assign] + N(0, 1); v = N(0, 1)         ([frame_len, d] each)
4. frames 1 .. Fc+Fq-1: k += drift * N(0, 1); v += drift * N(0, 1)
5. queries of the Fq current frames: q = k + qnoise * N(0, 1)
6. ``planes``  [P, d]   ~ N(0, 1) (random hyperplanes, kept fp32)
7. prompt: ``n_near = round(near_frac * L)`` tokens at ``mu[U{C}] + N(0, 1)``,
   then ``C`` prompt-only centroids ``nu ~ N(0, 1)`` and ``L - n_near`` tokens
   at ``nu[U{C}] + N(0, 1)``; prompt values ~ N(0, 1).

The first Fc frames fill the cache frame-major (slot = frame * frame_len + pos,
timestamp = frame index); the next Fq frames are the current chunk, whose
tokens get timestamp ``step = Fc``. bf16 workloads round every stored tensor
to bfloat16 (round to nearest even) after drawing; the fp32 process itself is
never rounded, so drift accumulates exactly as drawn.

Nothing here hashes, attends or edits a cache.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterator, Optional

import numpy as np


# --------------------------------------------------------------------------
# bfloat16 storage helpers (input preparation, not method arithmetic)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly the bf16-rounded values of x."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    dtype: str          # "f32" or "bf16": storage and compute input type
    H: int              # heads
    d: int              # head dim
    frame_len: int      # tokens per latent frame
    Fq: int             # frames in the current chunk
    Fc: int             # frames held in the initial cache
    C: int              # centroids per head
    drift: float        # per-frame drift sigma
    qnoise: float       # query = key + qnoise * N(0, 1)
    P: int              # hyperplanes per head (2**P buckets)
    L: int              # prompt tokens
    near_frac: float    # fraction of prompt tokens drawn from the query centroids
    tau: float          # TempCache cosine threshold
    cap: int            # TempCache capacity (slots per head)
    redraw_frac: float = 0.05   # rollout only: positions re-drawn per chunk

    @property
    def Nq(self) -> int:
        return self.Fq * self.frame_len

    @property
    def n0(self) -> int:
        """Valid slots of the initial cache."""
        return min(self.cap, self.Fc * self.frame_len)

    @property
    def B(self) -> int:
        return 1 << self.P

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, WorkloadConfig] = {
    # 1 head, d=64, fp32; 256-token frame; 4 cached frames; 16 centroids, drift 0.1.
    "tiny_f32": WorkloadConfig("tiny_f32", "f32", H=1, d=64, frame_len=256, Fq=1, Fc=4,
                               C=16, drift=0.1, qnoise=0.2, P=4, L=64, near_frac=1.0,
                               tau=0.9, cap=1024),
    # 1 head, d=128, bf16; 30x52 latent frame; 6 cached frames; 32 centroids.
    "single_bf16": WorkloadConfig("single_bf16", "bf16", H=1, d=128, frame_len=1560, Fq=1,
                                  Fc=6, C=32, drift=0.05, qnoise=0.2, P=6, L=512,
                                  near_frac=0.1, tau=0.95, cap=9360),
    # Wan-1.3B-like layer: 12 heads, 3-frame chunk, 21-frame cache.
    "wan13_bf16": WorkloadConfig("wan13_bf16", "bf16", H=12, d=128, frame_len=1560, Fq=3,
                                 Fc=21, C=64, drift=0.05, qnoise=0.2, P=7, L=512,
                                 near_frac=0.1, tau=0.95, cap=32760),
    # Wan-14B-like layer: 40 heads, otherwise the same chunk and cache.
    "wan14_bf16": WorkloadConfig("wan14_bf16", "bf16", H=40, d=128, frame_len=1560, Fq=3,
                                 Fc=21, C=128, drift=0.05, qnoise=0.2, P=8, L=512,
                                 near_frac=0.1, tau=0.95, cap=32760),
}


# --------------------------------------------------------------------------
# one step
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Step:
    """All inputs of one attention step, values as float32 (exactly representable
    in ``cfg.dtype``).  Shapes: q/k_cur/v_cur [H, Nq, d]; cache_k/cache_v
    [H, cap, d]; cache_ts [H, cap] int32; n_valid [H] int32; planes [H, P, d]
    float32; kp/vp [H, L, d]."""
    cfg: WorkloadConfig
    q: np.ndarray
    k_cur: np.ndarray
    v_cur: np.ndarray
    cache_k: np.ndarray
    cache_v: np.ndarray
    cache_ts: np.ndarray
    n_valid: np.ndarray
    planes: np.ndarray
    kp: np.ndarray
    vp: np.ndarray
    step: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.cfg.d)

    def storage(self, name: str) -> np.ndarray:
        """The tensor as it sits in device memory: uint16 bf16 bits or float32."""
        a = getattr(self, name)
        if self.cfg.dtype == "bf16" and name not in ("planes", "cache_ts", "n_valid"):
            return f32_to_bf16_bits(a)
        return a


class _HeadStream:
    """Per-head generator state (positions persist across chunks)."""

    def __init__(self, cfg: WorkloadConfig, seed: int, h: int):
        self.cfg = cfg
        self.rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, h])))
        r = self.rng
        fl, d = cfg.frame_len, cfg.d
        self.mu = r.standard_normal((cfg.C, d), dtype=np.float32)
        self.assign = r.integers(0, cfg.C, size=fl)
        self.k = self.mu[self.assign] + r.standard_normal((fl, d), dtype=np.float32)
        self.v = r.standard_normal((fl, d), dtype=np.float32)

    def next_frame(self):
        r, cfg = self.rng, self.cfg
        fl, d = cfg.frame_len, cfg.d
        self.k = self.k + np.float32(cfg.drift) * r.standard_normal((fl, d), dtype=np.float32)
        self.v = self.v + np.float32(cfg.drift) * r.standard_normal((fl, d), dtype=np.float32)

    def redraw(self):
        """Rollout: re-draw ``redraw_frac`` of the positions from fresh centroids."""
        r, cfg = self.rng, self.cfg
        fl, d = cfg.frame_len, cfg.d
        n_re = int(round(cfg.redraw_frac * fl))
        n_new = max(1, math.ceil(cfg.redraw_frac * cfg.C))
        pos = r.choice(fl, size=n_re, replace=False)
        fresh = r.standard_normal((n_new, d), dtype=np.float32)
        which = r.integers(0, n_new, size=n_re)
        self.k = self.k.copy()
        self.v = self.v.copy()
        self.k[pos] = fresh[which] + r.standard_normal((n_re, d), dtype=np.float32)
        self.v[pos] = r.standard_normal((n_re, d), dtype=np.float32)

    def chunk(self):
        """Fq frames of keys/values (each one drift step after the previous
        frame) and the chunk's queries."""
        cfg, r = self.cfg, self.rng
        ks, vs = [], []
        for _ in range(cfg.Fq):
            self.next_frame()
            ks.append(self.k)
            vs.append(self.v)
        k = np.concatenate(ks, 0)
        v = np.concatenate(vs, 0)
        q = k + np.float32(cfg.qnoise) * r.standard_normal(k.shape, dtype=np.float32)
        return q, k, v

    def planes_and_prompt(self):
        cfg, r = self.cfg, self.rng
        d = cfg.d
        planes = r.standard_normal((cfg.P, d), dtype=np.float32)
        n_near = int(round(cfg.near_frac * cfg.L))
        near = self.mu[r.integers(0, cfg.C, size=n_near)] + \
            r.standard_normal((n_near, d), dtype=np.float32)
        nu = r.standard_normal((cfg.C, d), dtype=np.float32)
        n_far = cfg.L - n_near
        far = nu[r.integers(0, cfg.C, size=n_far)] + r.standard_normal((n_far, d), dtype=np.float32)
        kp = np.concatenate([near, far], 0)
        vp = r.standard_normal((cfg.L, d), dtype=np.float32)
        return planes, kp, vp


def _round(cfg: WorkloadConfig, a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return bf16_round(a) if cfg.dtype == "bf16" else a


def make_step(cfg: WorkloadConfig, seed: int = 0, heads: Optional[range] = None) -> Step:
    """The single-step workload: a full cache of Fc frames plus an Fq-frame chunk.

    ``heads`` selects a subset of heads (each head's stream is independent, so a
    subset is bit-identical to the same heads of the full draw)."""
    heads = range(cfg.H) if heads is None else heads
    Hs = len(heads)
    fl, d, cap = cfg.frame_len, cfg.d, cfg.cap
    n0 = cfg.n0
    cache_k = np.zeros((Hs, cap, d), np.float32)
    cache_v = np.zeros((Hs, cap, d), np.float32)
    cache_ts = np.zeros((Hs, cap), np.int32)
    q = np.empty((Hs, cfg.Nq, d), np.float32)
    k_cur = np.empty_like(q)
    v_cur = np.empty_like(q)
    planes = np.empty((Hs, cfg.P, d), np.float32)
    kp = np.empty((Hs, cfg.L, d), np.float32)
    vp = np.empty_like(kp)
    for hi, h in enumerate(heads):
        s = _HeadStream(cfg, seed, h)
        for f in range(cfg.Fc):
            if f > 0:
                s.next_frame()
            lo = f * fl
            if lo < cap:
                hi_ = min(cap, lo + fl)
                cache_k[hi, lo:hi_] = s.k[: hi_ - lo]
                cache_v[hi, lo:hi_] = s.v[: hi_ - lo]
                cache_ts[hi, lo:hi_] = f
        q[hi], k_cur[hi], v_cur[hi] = s.chunk()
        planes[hi], kp[hi], vp[hi] = s.planes_and_prompt()
    n_valid = np.full((Hs,), n0, np.int32)
    return Step(cfg=cfg, q=_round(cfg, q), k_cur=_round(cfg, k_cur), v_cur=_round(cfg, v_cur),
                cache_k=_round(cfg, cache_k), cache_v=_round(cfg, cache_v),
                cache_ts=cache_ts, n_valid=n_valid, planes=planes,
                kp=_round(cfg, kp), vp=_round(cfg, vp), step=cfg.Fc)


def rollout_chunks(cfg: WorkloadConfig, n_chunks: int, seed: int = 0,
                   heads: Optional[range] = None) -> Iterator[dict]:
    """Long-rollout stream: chunk 0 is ``make_step``'s current chunk; every later
    chunk first re-draws ``redraw_frac`` of the positions from fresh centroids,
    then advances Fq frames with drift.  Yields dicts with q, k_cur, v_cur
    ([H, Nq, d] float32 values in cfg.dtype) and the chunk's ``step``.
    The initial cache, planes and prompt are those of ``make_step``."""
    heads = range(cfg.H) if heads is None else heads
    streams = []
    for h in heads:
        s = _HeadStream(cfg, seed, h)
        for f in range(1, cfg.Fc):
            s.next_frame()
        streams.append(s)
    for c in range(n_chunks):
        qs, ks, vs = [], [], []
        for s in streams:
            if c > 0:
                s.redraw()
            q, k, v = s.chunk()
            qs.append(q)
            ks.append(k)
            vs.append(v)
            if c == 0:
                s.planes_and_prompt()   # keep the stream aligned with make_step
        yield dict(q=_round(cfg, np.stack(qs)), k_cur=_round(cfg, np.stack(ks)),
                   v_cur=_round(cfg, np.stack(vs)), step=cfg.Fc + c * cfg.Fq)


def commit_case(seed: int, H: int, N: int, cap: int, d: int, n_valid, P: int,
                match_frac: float = 0.5, pool: int = 0, ts_span: int = 64) -> dict:
    """Random inputs for a cache commit taken on its own: a cache of ``cap``
    slots per head (``n_valid[h]`` of them valid, timestamps drawn from
    ``ts_span`` values so many are equal), a chunk of N tokens with bucket ids,
    and per-token (best slot, cosine) pairs standing in for a search result.
    About ``match_frac`` of the cosines lie in [0.95, 1], the rest in [-1, 0.9].
    With ``pool`` > 0 the best slots are drawn from the first ``pool`` valid
    slots so that many tokens name the same slot; some tokens get no slot (-1).
    All float arrays are float32; ids are uint16 values below 2**P."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7919])))
    n_valid = np.broadcast_to(np.asarray(n_valid, np.int32), (H,)).copy()
    f = np.float32
    out = dict(
        cache_k=rng.standard_normal((H, cap, d)).astype(f),
        cache_v=rng.standard_normal((H, cap, d)).astype(f),
        cache_ids=rng.integers(0, 1 << P, (H, cap)).astype(np.uint16),
        cache_ts=rng.integers(0, ts_span, (H, cap)).astype(np.int32),
        k_cur=rng.standard_normal((H, N, d)).astype(f),
        v_cur=rng.standard_normal((H, N, d)).astype(f),
        kcur_ids=rng.integers(0, 1 << P, (H, N)).astype(np.uint16),
        n_valid=n_valid)
    best = np.empty((H, N), np.int32)
    cos = np.empty((H, N), f)
    for h in range(H):
        n = int(n_valid[h])
        hi = max(1, min(pool, n) if pool > 0 else n)
        best[h] = rng.integers(0, hi, N) if n > 0 else -1
        best[h][rng.random(N) < 0.02] = -1
        m = rng.random(N) < match_frac
        cos[h] = np.where(m, rng.uniform(0.95, 1.0, N), rng.uniform(-1.0, 0.9, N)).astype(f)
    out["best"], out["cos"] = best, cos
    return out


def group_sizes(seed: int, H: int, cap: int, max_m: int = 32) -> np.ndarray:
    """Group sizes of a mean-merged cache standing in for one that has been
    merged for a while: ``[H, cap]`` int32 drawn uniformly from 1..max_m
    (``PCG64(SeedSequence([seed, 104729]))``).  Slot 0 of every head is
    given ``max_m`` so the largest size always occurs."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 104729])))
    m = rng.integers(1, max_m + 1, (H, cap)).astype(np.int32)
    if cap:
        m[:, 0] = max_m
    return m


def table_planes(seed: int, H: int, tables: int, P: int, d: int) -> np.ndarray:
    """Hyperplanes of ``tables`` independent hash tables: ``[H, tables*P, d]``
    float32 ~ N(0, 1), table t in rows t*P .. t*P+P-1
    (``PCG64(SeedSequence([seed, 130363]))``)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 130363])))
    return rng.standard_normal((H, tables * P, d)).astype(np.float32)


def codebook_from_keys(cache_k: np.ndarray, n_valid, B: int, seed: int, noise: float = 0.1) -> np.ndarray:
    """A codebook per head standing in for one fitted to the keys: ``B``
    distinct valid cached keys (``PCG64(SeedSequence([seed, 155921]))``
    chooses them) plus ``noise`` * N(0, 1); ``[H, B, d]`` float32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 155921])))
    H, _, d = cache_k.shape
    out = np.empty((H, B, d), np.float32)
    for h in range(H):
        n = int(np.asarray(n_valid).reshape(-1)[h if np.size(n_valid) > 1 else 0])
        pick = rng.choice(n, size=B, replace=False)
        out[h] = cache_k[h][pick] + noise * rng.standard_normal((B, d))
    return out

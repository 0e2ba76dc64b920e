"""One FAST-AR attention step for one layer: the four library calls issued over
two HIP streams, eagerly or as a captured HIP graph.

The step (FAST-AR summary, "2. Core Components"; blog, sections 1-3):

    ids of Q, K_cur and the prompt keys      (ann_hash, or ann_quantize)
    AnnSA over [cache ; chunk] + TempCache top-1 in the same pass
    AnnCA over each frame's kept prompt tokens
    TempCache commit of the chunk into the cache

Stream layout (both at the default priority).  The caller's stream carries
the critical path: hash(Q, K_cur) in one launch -> AnnSA (bucket sort +
attention) -> commit.  A side stream hashes the prompt keys, then runs AnnCA
once AnnSA is done: AnnCA needs only Q, the prompt and the ids, so it
overlaps the commit, whose select kernel occupies one CU per head.  The step
ends by joining the side stream into the caller's stream, so consecutive steps
never overlap (they share the id buffers, workspaces and outputs).

Optionally the side stream also lists the commit's eviction candidates (the N
oldest slots; they depend only on the cache as it was before the step) while
AnnSA runs, so the commit's select searches N slots instead of the whole
cache.  That costs the caller's stream one more cross-stream wait: inside a
captured graph the wait is a plain dependency and the step is shorter with
the list; issued eagerly the wait costs about what the list saves.  By
default the list is used only while a graph is being captured.

``graph()`` captures the same step into a HIP graph bound to one cache and one
set of input tensors (their addresses are baked in): replaying it removes the
host's per-launch cost, which otherwise exceeds the GPU time of the small
kernels.  The library clears nothing with memset, so a captured step holds
kernel and event nodes only.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import (KVCache, ann_hash, ann_hash_batch, ann_quantize, ann_quantize_batch, annca_forward,
               annsa_forward, load, tempcache_order, tempcache_update)


class AttentionStep:
    """Buffers and streams for repeated steps of one layer shape.

    Outputs of the latest step: ``o_sa`` [H, Nq, d] and ``lse`` [H, Nq] (AnnSA),
    ``o_ca`` [H, Nq, d] (AnnCA), ``best`` / ``best_cos`` [H, Nq] (TempCache
    top-1), ``keep`` [H, F, L] / ``keep_count`` [H, F] (AnnCA's kept prompt
    tokens), ``ids`` (bucket ids of Q, K_cur and the prompt keys)."""

    def __init__(self, H: int, Nq: int, d: int, cap: int, P: int, frame_len: int, L: int,
                 tau: float, out_dtype=torch.float32, device="cuda", overlap: bool = True,
                 scale: Optional[float] = None, ann: str = "lsh", order_list: Optional[bool] = None):
        """``ann``: "lsh" (the step's ``planes`` are [H, P, d] hyperplanes) or
        "quantize" (they are an [H, B, d] codebook, B <= 2^P: nearest-codeword
        buckets).  ``order_list``: list the eviction candidates on the side
        stream (True), never (False), or only under graph capture (None)."""
        if frame_len <= 0 or Nq % frame_len:
            raise ValueError("frame_len must divide Nq")
        if ann not in ("lsh", "quantize"):
            raise ValueError("ann must be 'lsh' or 'quantize'")
        self.ann = ann
        dev = torch.device(device)
        lib = load()
        self.H, self.Nq, self.d, self.cap, self.P = H, Nq, d, cap, P
        self.frame_len, self.L, self.tau = frame_len, L, tau
        self.scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.overlap = overlap
        self.order_list = order_list
        F = Nq // frame_len
        u8 = torch.uint8
        self.ws_sa = torch.empty(lib.fastar_annsa_workspace(H, Nq, cap, Nq, P), dtype=u8, device=dev)
        self.ws_ca = torch.empty(lib.fastar_annca_workspace(H, Nq, frame_len, L, P), dtype=u8, device=dev)
        self.ws_tc = torch.empty(lib.fastar_tempcache_workspace(H, Nq, cap, P), dtype=u8, device=dev)
        i16 = torch.int16
        self.ids = {"q": torch.empty(H, Nq, dtype=i16, device=dev),
                    "k": torch.empty(H, Nq, dtype=i16, device=dev),
                    "p": torch.empty(H, L, dtype=i16, device=dev)}
        self.o_sa = torch.empty(H, Nq, d, dtype=out_dtype, device=dev)
        self.lse = torch.empty(H, Nq, dtype=torch.float32, device=dev)
        self.o_ca = torch.empty(H, Nq, d, dtype=out_dtype, device=dev)
        self.best = torch.empty(H, Nq, dtype=torch.int32, device=dev)
        self.best_cos = torch.empty(H, Nq, dtype=torch.float32, device=dev)
        self.keep = torch.empty(H, F, L, dtype=u8, device=dev)
        self.keep_count = torch.empty(H, F, dtype=torch.int32, device=dev)
        self.order = torch.empty(H, Nq, dtype=torch.int32, device=dev)
        self.side = torch.cuda.Stream(dev)
        self._ev_sa, self._ev_side, self._ev_order = (torch.cuda.Event() for _ in range(3))

    # ------------------------------------------------------------------ pieces
    def _ids(self, x, planes, out):
        if self.ann == "lsh":
            ann_hash(x, planes, ids=out)
        else:
            ann_quantize(x, planes, ids=out)

    def _annsa(self, cache, q, k_cur, v_cur):
        annsa_forward(q, self.ids["q"], k_cur, v_cur, self.ids["k"], self.P, cache=cache,
                      scale=self.scale, out=self.o_sa, lse=self.lse, ws=self.ws_sa, search=True,
                      best=self.best, best_cos=self.best_cos)

    def _annca(self, q, kp, vp):
        annca_forward(q, self.ids["q"], self.frame_len, kp, vp, self.ids["p"], self.P,
                      scale=self.scale, out=self.o_ca, ws=self.ws_ca, keep=self.keep,
                      keep_count=self.keep_count)

    def _commit(self, cache, q, k_cur, v_cur, step, order=None):
        tempcache_update(cache, q, self.ids["q"], k_cur, v_cur, self.ids["k"], self.P, self.tau,
                         step, best_in=self.best, cos_in=self.best_cos, outputs=False,
                         ws=self.ws_tc, order_in=order)

    # ------------------------------------------------------------------ step
    def __call__(self, cache: KVCache, q, k_cur, v_cur, kp, vp, planes, step: int) -> None:
        """Enqueues one step on the current stream (and the side stream)."""
        main = torch.cuda.current_stream(q.device)
        if not self.overlap:
            batch = ann_hash_batch if self.ann == "lsh" else ann_quantize_batch
            batch([q, k_cur, kp], planes, ids=[self.ids["q"], self.ids["k"], self.ids["p"]])
            self._annsa(cache, q, k_cur, v_cur)
            self._annca(q, kp, vp)
            self._commit(cache, q, k_cur, v_cur, step)
            return
        use_order = (torch.cuda.is_current_stream_capturing() if self.order_list is None
                     else self.order_list)
        side = self.side
        side.wait_stream(main)
        if not use_order:
            with torch.cuda.stream(side):
                self._ids(kp, planes, self.ids["p"])
        batch = ann_hash_batch if self.ann == "lsh" else ann_quantize_batch
        batch([q, k_cur], planes, ids=[self.ids["q"], self.ids["k"]])
        self._annsa(cache, q, k_cur, v_cur)
        self._ev_sa.record(main)
        if use_order:
            # enqueued after AnnSA so the critical path starts first
            with torch.cuda.stream(side):
                tempcache_order(cache, self.Nq, out=self.order)
                self._ev_order.record(side)
        side.wait_event(self._ev_sa)
        with torch.cuda.stream(side):
            if use_order:
                # The prompt hash waits for AnnSA too, so the commit's select
                # (one block per head, each holding most of a CU's LDS) is
                # dispatched before AnnCA's blocks spread over every CU.
                self._ids(kp, planes, self.ids["p"])
            self._annca(q, kp, vp)
            self._ev_side.record(side)
        if use_order:
            main.wait_event(self._ev_order)
        self._commit(cache, q, k_cur, v_cur, step, self.order if use_order else None)
        main.wait_event(self._ev_side)

    def graph(self, cache: KVCache, q, k_cur, v_cur, kp, vp, planes, step: int) -> "StepGraph":
        """The step captured into a graph; ``replay()`` runs it on the current
        stream against exactly these tensors (contents may change, addresses
        may not).  The returned object keeps the tensors alive.

        Scalars are fixed at capture too: every replay stamps the slots it
        writes with this ``step`` (the TempCache timestamp that orders
        eviction).  A graph is therefore one step's work; a rollout replays a
        graph captured for each chunk's step (or steps eagerly)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self(cache, q, k_cur, v_cur, kp, vp, planes, step)
        return StepGraph(g, (self, cache, q, k_cur, v_cur, kp, vp, planes))


class StepGraph:
    """A captured step and every tensor its kernels address: the cache, the
    inputs and the step's own buffers stay allocated as long as the graph
    does, so a replay never writes into memory that was freed and handed to
    another tensor.  The step's scalars (the timestamp ``step``, tau, scale)
    are the ones given at capture: every replay writes the same timestamp."""

    def __init__(self, graph: torch.cuda.CUDAGraph, bound):
        self.graph = graph
        self._bound = bound

    def replay(self) -> None:
        self.graph.replay()

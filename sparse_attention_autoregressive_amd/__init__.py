"""FAST-AR attention step on AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of ``libfastar.so`` (include/fastar.h): each
function checks tensor shapes and dtypes, passes raw device pointers and the
current HIP stream, and returns the output tensors.  Every step of the
computation runs in the library's HIP kernels; PyTorch only provides device
memory and the stream.  Names follow the C ABI without its ``fastar_`` prefix.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import torch

from . import _lib
from ._lib import FASTAR_BF16, FASTAR_F32, FastarError, check, load

__all__ = ["ann_hash", "ann_hash_batch", "ann_quantize", "ann_quantize_batch", "bucket_sort", "annsa_forward",
           "annsa_forward_static", "annca_forward", "tempcache_update",
           "tempcache_order",
           "KVCache", "kernel_timer", "load", "FastarError"]

_DT = {torch.float32: FASTAR_F32, torch.bfloat16: FASTAR_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Tuple[Optional[int], int]:
    if nbytes == 0:
        return None, 0
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws.data_ptr(), ws.numel()


@dataclass
class KVCache:
    """Device tensors of one layer's bounded cache (all heads).

    With ``count`` the cache is mean-merged (Lemma 5.1 of the FAST-AR summary,
    Core Components A): slot j stands for count[h, j] tokens sharing one key
    and holds their mean value; AnnSA shifts its logits by ln(count) and the
    commit folds matched tokens into their slot's group.  Without it a
    matched slot is replaced by the newest token."""
    k: torch.Tensor          # [H, cap, d]
    v: torch.Tensor          # [H, cap, d]
    ids: torch.Tensor        # [H, cap] int16 (uint16 bit pattern)
    ts: torch.Tensor         # [H, cap] int32
    n_valid: torch.Tensor    # [H] int32
    knorm: torch.Tensor      # [H, cap] float32, |k| of each slot's key
    count: Optional[torch.Tensor] = None   # [H, cap] int32 group sizes (mean merge)

    @classmethod
    def empty(cls, H: int, cap: int, d: int, dtype=torch.bfloat16, device="cuda",
              merge: bool = False) -> "KVCache":
        return cls(k=torch.zeros(H, cap, d, dtype=dtype, device=device),
                   v=torch.zeros(H, cap, d, dtype=dtype, device=device),
                   ids=torch.zeros(H, cap, dtype=torch.int16, device=device),
                   ts=torch.zeros(H, cap, dtype=torch.int32, device=device),
                   n_valid=torch.zeros(H, dtype=torch.int32, device=device),
                   knorm=torch.zeros(H, cap, dtype=torch.float32, device=device),
                   count=torch.ones(H, cap, dtype=torch.int32, device=device) if merge else None)

    @classmethod
    def from_keys(cls, k: torch.Tensor, v: torch.Tensor, ts: torch.Tensor, n_valid: torch.Tensor,
                  planes: torch.Tensor, count: Optional[torch.Tensor] = None) -> "KVCache":
        """A cache holding ``k``/``v`` with bucket ids and norms computed by
        ann_hash (``count``: group sizes of a mean-merged cache)."""
        H, cap, _ = k.shape
        c = cls(k=k, v=v, ids=torch.empty(H, cap, dtype=torch.int16, device=k.device), ts=ts,
                n_valid=n_valid, knorm=torch.empty(H, cap, dtype=torch.float32, device=k.device),
                count=count)
        ann_hash(k, planes, ids=c.ids, norms=c.knorm)
        return c

    def clone(self) -> "KVCache":
        return KVCache(k=self.k.clone(), v=self.v.clone(), ids=self.ids.clone(),
                       ts=self.ts.clone(), n_valid=self.n_valid.clone(), knorm=self.knorm.clone(),
                       count=None if self.count is None else self.count.clone())

    @property
    def merge(self) -> bool:
        return self.count is not None

    @property
    def H(self) -> int:
        return self.k.shape[0]

    @property
    def cap(self) -> int:
        return self.k.shape[1]

    @property
    def d(self) -> int:
        return self.k.shape[2]

    def struct(self) -> _lib.FastarCache:
        for t in (self.k, self.v, self.ids, self.ts, self.n_valid, self.knorm):
            if not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous")
        if self.ids.dtype != torch.int16 or self.ts.dtype != torch.int32 \
                or self.n_valid.dtype != torch.int32 or self.knorm.dtype != torch.float32:
            raise TypeError("cache ids must be int16, ts and n_valid int32, knorm float32")
        if self.count is not None and (self.count.dtype != torch.int32
                                       or tuple(self.count.shape) != (self.H, self.cap)):
            raise TypeError("cache count must be int32 [H, cap]")
        return _lib.FastarCache(self.H, self.cap, self.d, _dtype_code(self.k), _ptr(self.k),
                                _ptr(self.v), _ptr(self.ids), _ptr(self.ts), _ptr(self.n_valid),
                                _ptr(self.knorm), _ptr(self.count))


def _ids_check(ids: torch.Tensor, shape) -> None:
    if ids.dtype != torch.int16 or tuple(ids.shape) != tuple(shape):
        raise ValueError(f"ids must be int16 of shape {tuple(shape)}, got {ids.dtype} {tuple(ids.shape)}")


def _int32_check(t: torch.Tensor, shape, what: str) -> None:
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be int32 of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def ann_hash(x: torch.Tensor, planes: torch.Tensor, ids: Optional[torch.Tensor] = None,
             norms: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Bucket ids [H, N] (int16 holding uint16 bits) of x [H, N, d] under planes [H, P, d]
    fp32; with ``norms`` ([H, N] float32) also writes |x|."""
    H, N, d = x.shape
    P = planes.shape[1]
    if planes.dtype != torch.float32 or tuple(planes.shape) != (H, P, d):
        raise ValueError("planes must be float32 [H, P, d]")
    if ids is None:
        ids = torch.empty(H, N, dtype=torch.int16, device=x.device)
    _ids_check(ids, (H, N))
    if norms is not None and (norms.dtype != torch.float32 or tuple(norms.shape) != (H, N)):
        raise ValueError("norms must be float32 [H, N]")
    check("fastar_ann_hash", load().fastar_ann_hash(_ptr(x), _dtype_code(x), H, N, d, _ptr(planes),
                                                    P, _ptr(ids), _ptr(norms), _stream(x.device)))
    return ids


def _batch_call(fn: str, xs, table: torch.Tensor, what: str, ids, norms):
    """Shared marshalling of the batched id calls (hash planes or codebook)."""
    xs = list(xs)
    count = len(xs)
    if not 1 <= count <= _lib.FASTAR_HASH_BATCH:
        raise ValueError(f"between 1 and {_lib.FASTAR_HASH_BATCH} tensors")
    H, _, d = xs[0].shape
    P = table.shape[1]
    if table.dtype != torch.float32 or tuple(table.shape) != (H, P, d):
        raise ValueError(f"{what} must be float32 [H, {'P' if what == 'planes' else 'B'}, d]")
    dt = _dtype_code(xs[0])
    ids = list(ids) if ids is not None else [None] * count
    norms = list(norms) if norms is not None else [None] * count
    for i, x in enumerate(xs):
        if x.shape[0] != H or x.shape[2] != d or _dtype_code(x) != dt:
            raise ValueError("all tensors must share H, d and dtype")
        if ids[i] is None:
            ids[i] = torch.empty(H, x.shape[1], dtype=torch.int16, device=x.device)
        _ids_check(ids[i], (H, x.shape[1]))
        if norms[i] is not None and (norms[i].dtype != torch.float32
                                     or tuple(norms[i].shape) != (H, x.shape[1])):
            raise ValueError("norms must be float32 [H, N]")
    arr = lambda vals: (ctypes.c_void_p * count)(*vals)
    check(fn, getattr(load(), fn)(
        count, arr([_ptr(x) for x in xs]), (ctypes.c_int32 * count)(*[x.shape[1] for x in xs]),
        arr([_ptr(t) for t in ids]), arr([_ptr(t) for t in norms]), dt, H, d, _ptr(table), P,
        _stream(xs[0].device)))
    return ids


def ann_hash_batch(xs, planes: torch.Tensor, ids=None, norms=None):
    """Bucket ids of several [H, N_i, d] tensors under the same planes in one
    launch (at most ``FASTAR_HASH_BATCH`` tensors); returns the list of id
    tensors.  ``ids`` / ``norms``: optional lists of outputs (entries may be
    None)."""
    return _batch_call("fastar_ann_hash_batch", xs, planes, "planes", ids, norms)


def ann_quantize_batch(xs, codebook: torch.Tensor, ids=None, norms=None):
    """Nearest-codeword ids of several [H, N_i, d] tensors under the same
    codebook [H, B, d] in one launch (at most ``FASTAR_HASH_BATCH`` tensors);
    returns the list of id tensors, as ``ann_hash_batch``."""
    return _batch_call("fastar_ann_quantize_batch", xs, codebook, "codebook", ids, norms)


def ann_quantize(x: torch.Tensor, codebook: torch.Tensor, ids: Optional[torch.Tensor] = None,
                 norms: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Nearest-codeword bucket ids [H, N] (int16 holding uint16 bits) of x
    [H, N, d] under codebook [H, B, d] float32; with ``norms`` ([H, N]
    float32) also writes |x|.  Bucketed calls take P = ceil(log2 B)."""
    H, N, d = x.shape
    B = codebook.shape[1]
    if codebook.dtype != torch.float32 or tuple(codebook.shape) != (H, B, d):
        raise ValueError("codebook must be float32 [H, B, d]")
    if ids is None:
        ids = torch.empty(H, N, dtype=torch.int16, device=x.device)
    _ids_check(ids, (H, N))
    if norms is not None and (norms.dtype != torch.float32 or tuple(norms.shape) != (H, N)):
        raise ValueError("norms must be float32 [H, N]")
    check("fastar_ann_quantize", load().fastar_ann_quantize(
        _ptr(x), _dtype_code(x), H, N, d, _ptr(codebook), B, _ptr(ids), _ptr(norms),
        _stream(x.device)))
    return ids


def bucket_sort(ids: torch.Tensor, P: int, ws: Optional[torch.Tensor] = None):
    """Stable grouping by bucket: (off [H, 2^P + 1], perm [H, N]) int32."""
    H, N = ids.shape
    _ids_check(ids, (H, N))
    lib = load()
    off = torch.empty(H, (1 << P) + 1, dtype=torch.int32, device=ids.device)
    perm = torch.empty(H, N, dtype=torch.int32, device=ids.device)
    wsp, wsn = _workspace(lib.fastar_bucket_sort_workspace(H, N, P), ids.device, ws)
    check("fastar_bucket_sort", lib.fastar_bucket_sort(_ptr(ids), H, N, P, _ptr(off), _ptr(perm),
                                                       wsp, wsn, _stream(ids.device)))
    return off, perm


def annsa_forward(q: torch.Tensor, q_ids: torch.Tensor, k_cur: torch.Tensor, v_cur: torch.Tensor,
                  kcur_ids: torch.Tensor, P: int, cache: Optional[KVCache] = None,
                  scale: Optional[float] = None, out_dtype=torch.float32,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  want_lse: bool = True, ws: Optional[torch.Tensor] = None,
                  search: bool = False, best: Optional[torch.Tensor] = None,
                  best_cos: Optional[torch.Tensor] = None, tables: int = 1):
    """Bucket-restricted self-attention over [cache ; current chunk]: (out, lse), or
    (out, lse, best, best_cos) with ``search`` (TempCache's top-1 from the same pass).

    With ``tables`` > 1 the ids hold one ``P``-bit field per table (hash with
    planes [H, tables*P, d]) and each query attends to the union of its
    buckets' keys, each key once."""
    H, Nq, d = q.shape
    Ncur = k_cur.shape[1]
    _ids_check(q_ids, (H, Nq))
    _ids_check(kcur_ids, (H, Ncur))
    if k_cur.shape != (H, Ncur, d) or v_cur.shape != (H, Ncur, d):
        raise ValueError("k_cur / v_cur must be [H, Ncur, d]")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    lib = load()
    if out is None:
        out = torch.empty(H, Nq, d, dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(H, Nq, dtype=torch.float32, device=q.device)
    if search:
        if best is None:
            best = torch.empty(H, Nq, dtype=torch.int32, device=q.device)
        if best_cos is None:
            best_cos = torch.empty(H, Nq, dtype=torch.float32, device=q.device)
    cs = cache.struct() if cache is not None else None
    cap = cache.cap if cache is not None else 0
    if tables == 1:
        wsp, wsn = _workspace(lib.fastar_annsa_workspace(H, Nq, cap, Ncur, P), q.device, ws)
        check("fastar_annsa_forward", lib.fastar_annsa_forward(
            _ptr(q), _ptr(q_ids), H, Nq, d, _dtype_code(q), ctypes.byref(cs) if cs else None,
            _ptr(k_cur), _ptr(v_cur), _ptr(kcur_ids), Ncur, P, scale, _ptr(out), _dtype_code(out),
            _ptr(lse), _ptr(best) if search else None, _ptr(best_cos) if search else None,
            wsp, wsn, _stream(q.device)))
    else:
        wsp, wsn = _workspace(lib.fastar_annsa_multi_workspace(H, Nq, cap, Ncur, d, P, tables),
                              q.device, ws)
        check("fastar_annsa_multi_forward", lib.fastar_annsa_multi_forward(
            _ptr(q), _ptr(q_ids), H, Nq, d, _dtype_code(q), ctypes.byref(cs) if cs else None,
            _ptr(k_cur), _ptr(v_cur), _ptr(kcur_ids), Ncur, P, tables, scale, _ptr(out),
            _dtype_code(out), _ptr(lse), _ptr(best) if search else None,
            _ptr(best_cos) if search else None, wsp, wsn, _stream(q.device)))
    return (out, lse, best, best_cos) if search else (out, lse)


def annsa_forward_static(q: torch.Tensor, q_ids: torch.Tensor, k_cur: torch.Tensor,
                         v_cur: torch.Tensor, kcur_ids: torch.Tensor, P: int,
                         cache: Optional[KVCache] = None, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         best: Optional[torch.Tensor] = None, best_cos: Optional[torch.Tensor] = None,
                         search: bool = False, out_dtype=torch.float32):
    """``annsa_forward`` through fastar_annsa_forward_static: the library's
    static per-device scratch array is the workspace, so the call itself
    allocates nothing (pass ``out``, ``lse`` and, with ``search``, ``best`` /
    ``best_cos`` to allocate nothing here either).  Overlapping calls on one
    device race on that array."""
    H, Nq, d = q.shape
    Ncur = k_cur.shape[1]
    _ids_check(q_ids, (H, Nq))
    _ids_check(kcur_ids, (H, Ncur))
    if k_cur.shape != (H, Ncur, d) or v_cur.shape != (H, Ncur, d):
        raise ValueError("k_cur / v_cur must be [H, Ncur, d]")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty(H, Nq, d, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(H, Nq, dtype=torch.float32, device=q.device)
    if search:
        if best is None:
            best = torch.empty(H, Nq, dtype=torch.int32, device=q.device)
        if best_cos is None:
            best_cos = torch.empty(H, Nq, dtype=torch.float32, device=q.device)
    cs = cache.struct() if cache is not None else None
    check("fastar_annsa_forward_static", load().fastar_annsa_forward_static(
        _ptr(q), _ptr(q_ids), H, Nq, d, _dtype_code(q), ctypes.byref(cs) if cs else None,
        _ptr(k_cur), _ptr(v_cur), _ptr(kcur_ids), Ncur, P, scale, _ptr(out), _dtype_code(out),
        _ptr(lse), _ptr(best) if search else None, _ptr(best_cos) if search else None,
        _stream(q.device)))
    return (out, lse, best, best_cos) if search else (out, lse)


def annca_forward(q: torch.Tensor, q_ids: torch.Tensor, frame_len: int, kp: torch.Tensor,
                  vp: torch.Tensor, kp_ids: torch.Tensor, P: int, scale: Optional[float] = None,
                  out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                  want_keep: bool = True, ws: Optional[torch.Tensor] = None,
                  keep: Optional[torch.Tensor] = None, keep_count: Optional[torch.Tensor] = None):
    """Frame-pruned cross-attention: (out, keep [H, F, L] uint8, keep_count [H, F])."""
    H, Nq, d = q.shape
    L = kp.shape[1]
    _ids_check(q_ids, (H, Nq))
    _ids_check(kp_ids, (H, L))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    F = Nq // frame_len if frame_len > 0 else 0
    lib = load()
    if out is None:
        out = torch.empty(H, Nq, d, dtype=out_dtype, device=q.device)
    if keep is None and want_keep:
        keep = torch.empty(H, F, L, dtype=torch.uint8, device=q.device)
    cnt = keep_count
    if cnt is None and want_keep:
        cnt = torch.empty(H, F, dtype=torch.int32, device=q.device)
    if keep is not None and (keep.dtype != torch.uint8 or tuple(keep.shape) != (H, F, L)):
        raise ValueError("keep must be uint8 [H, F, L]")
    if cnt is not None and (cnt.dtype != torch.int32 or tuple(cnt.shape) != (H, F)):
        raise ValueError("keep_count must be int32 [H, F]")
    wsp, wsn = _workspace(lib.fastar_annca_workspace(H, Nq, frame_len, L, P), q.device, ws)
    check("fastar_annca_forward", lib.fastar_annca_forward(
        _ptr(q), _ptr(q_ids), H, Nq, frame_len, d, _dtype_code(q), _ptr(kp), _ptr(vp),
        _ptr(kp_ids), L, P, scale, _ptr(out), _dtype_code(out), _ptr(keep), _ptr(cnt), wsp, wsn,
        _stream(q.device)))
    return out, keep, cnt


def tempcache_update(cache: KVCache, q: torch.Tensor, q_ids: torch.Tensor, k_cur: torch.Tensor,
                     v_cur: torch.Tensor, kcur_ids: torch.Tensor, P: int, tau: float, step: int,
                     best_in: Optional[torch.Tensor] = None, cos_in: Optional[torch.Tensor] = None,
                     outputs: bool = True, ws: Optional[torch.Tensor] = None,
                     order_in: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Commits one chunk to ``cache`` in place; returns best, cos, dest, evicted, counts.
    ``order_in``: ``tempcache_order(cache, N)`` made since the cache last changed."""
    H, N, d = q.shape
    _ids_check(q_ids, (H, N))
    _ids_check(kcur_ids, (H, N))
    lib = load()
    dev = q.device
    res: Dict[str, torch.Tensor] = {}
    if outputs:
        res = {"best": torch.empty(H, N, dtype=torch.int32, device=dev),
               "cos": torch.empty(H, N, dtype=torch.float32, device=dev),
               "dest": torch.empty(H, N, dtype=torch.int32, device=dev),
               "evicted": torch.empty(H, N, dtype=torch.int32, device=dev),
               "counts": torch.empty(H, 5, dtype=torch.int32, device=dev)}
    cs = cache.struct()
    if order_in is not None:
        _int32_check(order_in, (H, N), "order_in")
    wsp, wsn = _workspace(lib.fastar_tempcache_workspace(H, N, cache.cap, P), dev, ws)
    check("fastar_tempcache_update", lib.fastar_tempcache_update(
        ctypes.byref(cs), _ptr(q), _ptr(q_ids), _ptr(k_cur), _ptr(v_cur), _ptr(kcur_ids), N, P,
        tau, step, _ptr(best_in), _ptr(cos_in), _ptr(order_in), _ptr(res.get("best")), _ptr(res.get("cos")),
        _ptr(res.get("dest")), _ptr(res.get("evicted")), _ptr(res.get("counts")), wsp, wsn,
        _stream(dev)))
    return res


def tempcache_order(cache: KVCache, N: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The eviction candidates of a commit of ``N`` tokens: per head the
    min(n_valid, N) slots of smallest (ts, slot), ascending, -1 padded ([H, N]
    int32); pass it to ``tempcache_update(order_in=...)`` before the cache
    changes."""
    H = cache.k.shape[0]
    if out is None:
        out = torch.empty(H, N, dtype=torch.int32, device=cache.k.device)
    else:
        _int32_check(out, (H, N), "out")
    cs = cache.struct()
    check("fastar_tempcache_order", load().fastar_tempcache_order(ctypes.byref(cs), N, _ptr(out),
                                                                   _stream(cache.k.device)))
    return out


class kernel_timer:
    """Context manager around fastar_timer_start/stop: ``.times`` maps each kernel
    name to (launches, total_ms) measured with HIP events on the launch stream."""

    def __enter__(self):
        check("fastar_timer_start", load().fastar_timer_start())
        self.times: Dict[str, Tuple[int, float]] = {}
        return self

    def __exit__(self, *exc):
        buf = (_lib.FastarKernelTime * 64)()
        n = load().fastar_timer_stop(buf, 64)
        for i in range(min(n, 64)):
            self.times[buf[i].name.decode()] = (buf[i].launches, buf[i].total_ms)
        return False

"""FAST-AR attention step: plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the cpu_baseline leg of
``bench.py`` may import this module.  It never runs on the product path.

Sources (the FAST-AR pages; cited below by page and section):

* "FAST-AR: NVIDIA Cracks the Video Diffusion Bottleneck" (deltav-cc blog),
  sections "1. TempCache", "2. AnnCA", "3. AnnSA"  -- cited as *blog, <section>*.
* "Fast Autoregressive Video Diffusion and World Models with Temporal Cache
  Compression and Sparse Attention" (gist.science technical summary),
  "2. Core Components", parts A (TempCache), B (AnnCA), C (AnnSA)
  -- cited as *summary, Core Components <part>*.
* the arXiv abstract of the same paper (mlsanity.com index page)
  -- cited as *abstract*.

Every function works on one attention head; heads are independent (the pages
never couple them).  Floating point is fp64 throughout; inputs that are stored
as bf16 or fp32 enter as their exact values.

Readings of points the pages leave open (each repeated where it is used):

R1  ANN = random-hyperplane (sign) LSH: bit p of a token's bucket id is
    [<x, r_p> >= 0]; plane p is bit p.  Queries, cached keys, current keys
    and prompt keys are hashed with the same planes of their head (the
    summary, Core Components B, puts queries and prompt keys in one space).
R2  One hash table, one bucket per token (blog, "3. AnnSA", allows one or
    several buckets per token; one is the plainest case).
R3  AnnSA key context = [valid cache slots 0..n-1 ; current chunk in token
    order]; a query attends to every key of its bucket, no causal mask; an
    empty bucket gives O = 0 and lse = -inf; softmax scale is a parameter
    (1/sqrt(d) by default).
R4  AnnCA keeps, per frame, the prompt tokens whose bucket holds at least one
    query of that frame, and attends densely over the kept tokens in
    ascending order; no kept token gives O = 0.
R5  TempCache top-1: cosine between the current query and each cached key of
    the query's own bucket (ANN instead of a full attention map, summary,
    Core Components A); candidates are previous-frame keys only (the valid
    cache slots).  Ties go to the lowest slot.  A zero norm gives cosine 0.
R6  Merge: matched = has a candidate and cosine >= tau (inclusive).  The
    current token replaces the matched slot (blog, "1. TempCache": a group of
    corresponding keys keeps just its newest member).  When several current
    tokens match one slot, the largest token index (the most recent) wins
    and the others are dropped.
R7  Unmatched tokens are appended in token order; once the cache is full they
    replace the slots with the oldest timestamps (ties: lower slot first),
    never a slot refreshed in this update.  The replaced slots are filled in
    ascending slot order.
R8  Inserted and refreshed slots get timestamp ``step``.
R9  A ``best`` value outside [0, n) counts as "no candidate".

Mean-merge variant (summary, Core Components A, Lemma 5.1: identical keys
merge without error when the values are averaged and the logits shifted by
the group size).  A cache in this mode carries a group size m_j >= 1 per
slot:

R10 Slot j stands for m_j tokens with one key; its value is their mean.  The
    shift is + ln m_j on the logit, which makes it exact: for a group G of
    identical keys, sum_{t in G} exp(l) v_t = exp(l + ln m) * mean_G(v), and
    likewise for the softmax denominator.  Current-chunk keys have m = 1.
R11 Every matched token joins the group of its top-1 slot (none is dropped):
    with C_j the slot's claimants, v_j <- (m_j v_j + sum_{i in C_j} v_i) /
    (m_j + |C_j|) and m_j <- m_j + |C_j|.  The key, id and timestamp become
    those of the most recent claimant, as in R6 (for identical keys the
    choice is immaterial).
R12 Appended and replacing tokens start groups of size 1; an evicted slot's
    group leaves the cache with it.  Selection of the evicted slots is R7's.

Multi-table variant (blog, "3. AnnSA": a token may fall in several buckets;
summary, Core Components C):

R16 T hash tables, each with its own P planes; a token's id holds T fields of
    P bits, table t in bits t*P .. t*P+P-1 (so one hash over the T*P planes of
    all tables gives every field at once; T*P <= 16).
R17 A query attends to the union over tables of the keys that share its
    bucket in that table; a key matching in several tables is counted once
    (a set union, not a sum of per-table attentions).
R18 The TempCache top-1 searches the same union of buckets.

Quantization variant (summary, Core Components A and B name quantization as
the alternative ANN):

R19 A head's codebook holds B codewords; a token's bucket is its nearest
    codeword in Euclidean distance, argmin_c |x - c|^2, i.e. argmax_c
    <x, c> - |c|^2 / 2; ties go to the lowest index.  The codebook is an
    input (how it is learned is not described).  Its tie flag: the runner-up
    score within 1e-5 * (|x| max_c |c| + max_c |c|^2) of the best.

Tie flags (the decision is numerically fragile; a parallel fp32 result may
legitimately differ there): a hash bit whose |<x, r>| / (|x| |r|) < 1e-5; an
argmax whose runner-up cosine is within 1e-5; a threshold test with
|cos - tau| < 1e-5.

Parity pins (tests/test_oracle_*.py): every function is pinned by closed forms,
library routines or hand-worked fixtures; see the tests' docstrings.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np

TIE_EPS = 1e-5


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# ANN hash  (summary, Core Components A and B: an LSH or a quantizer; R1, R2)
# ---------------------------------------------------------------------------

def ann_hash(x, planes) -> Tuple[np.ndarray, np.ndarray]:
    """Bucket id of every row of ``x`` [N, d] under the hyperplanes ``planes``
    [P, d]:  id = sum_p [<x, r_p> >= 0] * 2**p.

    Returns ``(ids, tie_bits)``, both uint16 [N]; ``tie_bits`` marks the planes
    whose normalised projection is within 1e-5 of zero."""
    X = _f64(x)
    R = _f64(planes).reshape(-1, X.shape[1]) if np.size(planes) else np.zeros((0, X.shape[1]))
    N, P = X.shape[0], R.shape[0]
    ids = np.zeros(N, np.int64)
    tie = np.zeros(N, np.int64)
    if P == 0:
        return ids.astype(np.uint16), tie.astype(np.uint16)
    proj = X @ R.T
    denom = np.linalg.norm(X, axis=1)[:, None] * np.linalg.norm(R, axis=1)[None, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(denom > 0, np.abs(proj) / np.where(denom > 0, denom, 1.0), 0.0)
    for p in range(P):
        ids |= (proj[:, p] >= 0).astype(np.int64) << p
        tie |= (rel[:, p] < TIE_EPS).astype(np.int64) << p
    return ids.astype(np.uint16), tie.astype(np.uint16)


def ann_quantize(x, codebook) -> Tuple[np.ndarray, np.ndarray]:
    """Bucket id of every row of ``x`` [N, d]: the index of its nearest
    codeword in ``codebook`` [B, d] (R19), as argmax_c <x, c> - |c|^2 / 2
    (lowest index on ties).

    Returns ``(ids uint16 [N], tie bool [N])``: ``tie`` marks rows whose
    runner-up is within the R19 margin."""
    X = _f64(x)
    C = _f64(codebook).reshape(-1, X.shape[1])
    N, B = X.shape[0], C.shape[0]
    if B == 1:
        return np.zeros(N, np.uint16), np.zeros(N, bool)
    score = X @ C.T - 0.5 * np.sum(C * C, axis=1)[None, :]
    ids = np.argmax(score, axis=1)
    top = score[np.arange(N), ids]
    masked = score.copy()
    masked[np.arange(N), ids] = -np.inf
    second = masked.max(axis=1)
    cn = np.linalg.norm(C, axis=1)
    margin = TIE_EPS * (np.linalg.norm(X, axis=1) * cn.max() + (cn ** 2).max())
    return ids.astype(np.uint16), (top - second) < margin


# ---------------------------------------------------------------------------
# Bucket grouping  (summary, Core Components C: block-sparse attention needs
# the tokens of each bucket gathered together)
# ---------------------------------------------------------------------------

def bucket_sort(ids, P: int) -> Tuple[np.ndarray, np.ndarray]:
    """Stable grouping of token indices by bucket.

    ``off[b]`` = number of tokens whose id is below b (``off[B]`` = N);
    ``perm[off[b]:off[b+1]]`` = the indices with id b, ascending."""
    ids = np.asarray(ids).astype(np.int64)
    B = 1 << P
    off = np.zeros(B + 1, np.int64)
    parts: List[np.ndarray] = []
    for b in range(B):
        members = np.nonzero(ids == b)[0]
        parts.append(members)
        off[b + 1] = off[b] + members.size
    perm = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return off.astype(np.int32), perm.astype(np.int32)


def key_context(cache_k, cache_v, cache_ids, n: int, k_cur, v_cur, kcur_ids):
    """AnnSA's key context (R3): valid cache slots 0..n-1, then the current chunk."""
    return (np.concatenate([_f64(cache_k[:n]), _f64(k_cur)], 0),
            np.concatenate([_f64(cache_v[:n]), _f64(v_cur)], 0),
            np.concatenate([np.asarray(cache_ids[:n]), np.asarray(kcur_ids)]).astype(np.int64))


def key_counts(cache_count, n: int, n_cur: int) -> np.ndarray:
    """Group sizes of AnnSA's key context in merge mode (R10): the valid
    slots' counts, then 1 for every current-chunk key."""
    return np.concatenate([np.asarray(cache_count[:n], np.int64), np.ones(n_cur, np.int64)])


# ---------------------------------------------------------------------------
# AnnSA  (blog, "3. AnnSA"; summary, Core Components C; R2, R3)
# ---------------------------------------------------------------------------

def annsa(q, q_ids, k, v, k_ids, scale: float, k_counts=None) -> Tuple[np.ndarray, np.ndarray]:
    """Each query attends only to the keys of its own bucket:
    O_i = sum_{j: idk_j = idq_i} softmax_j(l_ij) v_j,  l_ij = scale * <q_i, k_j>,
    lse_i = log sum_{j in bucket} exp(l_ij).
    Queries whose bucket holds no key get O = 0, lse = -inf.

    With ``k_counts`` (group sizes m_j >= 1 of a mean-merged cache, R10) the
    logit of key j is scale * <q_i, k_j> + ln m_j."""
    Q, K, V = _f64(q), _f64(k), _f64(v)
    qid = np.asarray(q_ids).astype(np.int64)
    kid = np.asarray(k_ids).astype(np.int64)
    bias = np.zeros(K.shape[0]) if k_counts is None else np.log(_f64(k_counts))
    O = np.zeros((Q.shape[0], V.shape[1]))
    lse = np.full(Q.shape[0], -np.inf)
    for b in np.unique(qid):
        qi = np.nonzero(qid == b)[0]
        kj = np.nonzero(kid == b)[0]
        if kj.size == 0:
            continue
        S = (Q[qi] @ K[kj].T) * scale + bias[kj][None, :]
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        O[qi] = (E @ V[kj]) / l
        lse[qi] = m[:, 0] + np.log(l[:, 0])
    return O, lse


def bucket_fields(ids, P: int, T: int) -> np.ndarray:
    """The T per-table bucket ids held in each id (R16): [N, T] int64,
    column t = bits t*P .. t*P+P-1."""
    ids = np.asarray(ids).astype(np.int64)
    return np.stack([(ids >> (t * P)) & ((1 << P) - 1) for t in range(T)], axis=1)


def annsa_multi(q, q_ids, k, v, k_ids, scale: float, P: int, T: int, k_counts=None,
                block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Multi-table AnnSA (R16, R17): query i attends to every key that shares
    its bucket in at least one of the T tables, each such key once:
    O_i = sum_{j in U_i} softmax_j(l_ij) v_j with U_i = {j : some t has
    field_t(q_i) = field_t(k_j)} and l_ij as in ``annsa`` (group-size shift
    included).  Empty U_i gives O = 0, lse = -inf.  Written as a masked dense
    attention over ``block`` queries at a time."""
    Q, K, V = _f64(q), _f64(k), _f64(v)
    fq, fk = bucket_fields(q_ids, P, T), bucket_fields(k_ids, P, T)
    bias = np.zeros(K.shape[0]) if k_counts is None else np.log(_f64(k_counts))
    O = np.zeros((Q.shape[0], V.shape[1]))
    lse = np.full(Q.shape[0], -np.inf)
    for s0 in range(0, Q.shape[0], block):
        rows = slice(s0, min(Q.shape[0], s0 + block))
        member = np.zeros((fq[rows].shape[0], K.shape[0]), bool)
        for t in range(T):
            member |= fq[rows, t][:, None] == fk[None, :, t]
        S = np.where(member, (Q[rows] @ K.T) * scale + bias[None, :], -np.inf)
        has = member.any(axis=1)
        if not has.any():
            continue
        m = np.where(has, S.max(axis=1), 0.0)
        E = np.where(member, np.exp(S - m[:, None]), 0.0)
        l = E.sum(axis=1)
        idx = np.arange(rows.start, rows.stop)[has]
        O[idx] = (E[has] @ V) / l[has][:, None]
        lse[idx] = m[has] + np.log(l[has])
    return O, lse


# ---------------------------------------------------------------------------
# AnnCA  (blog, "2. AnnCA"; summary, Core Components B; R4)
# ---------------------------------------------------------------------------

def annca(q, q_ids, frame_len: int, kp, vp, kp_ids, scale: float):
    """Per frame f (queries f*frame_len .. (f+1)*frame_len-1): keep the prompt
    tokens whose bucket holds at least one query of the frame, then dense
    softmax cross-attention over the kept tokens.

    Returns ``(O [Nq, d], keep [F, L] bool)``."""
    Q, Kp, Vp = _f64(q), _f64(kp), _f64(vp)
    Nq, L = Q.shape[0], Kp.shape[0]
    if frame_len <= 0 or Nq % frame_len:
        raise ValueError("frame_len must divide the number of queries")
    F = Nq // frame_len
    qid = np.asarray(q_ids).astype(np.int64)
    pid = np.asarray(kp_ids).astype(np.int64)
    keep = np.zeros((F, L), bool)
    O = np.zeros((Nq, Vp.shape[1]))
    for f in range(F):
        rows = slice(f * frame_len, (f + 1) * frame_len)
        present = set(int(i) for i in qid[rows])
        keep[f] = [int(t) in present for t in pid]
        idx = np.nonzero(keep[f])[0]
        if idx.size == 0:
            continue
        S = (Q[rows] @ Kp[idx].T) * scale
        E = np.exp(S - S.max(axis=1, keepdims=True))
        O[rows] = (E @ Vp[idx]) / E.sum(axis=1, keepdims=True)
    return O, keep


# ---------------------------------------------------------------------------
# TempCache  (blog, "1. TempCache"; summary, Core Components A; R5-R9)
# ---------------------------------------------------------------------------

def tempcache_top1(q, q_ids, cache_k, cache_ids, n: int, P: Optional[int] = None, T: int = 1):
    """For each current query, its most similar previous-frame key within the
    query's bucket (R5); with ``T`` > 1 tables of ``P`` bits, within the union
    of its buckets (R16-R18).

    Returns ``(best [N] int64 (-1: no candidate), cos [N] (-inf: none),
    argmax_tie [N] bool, near: list of the candidate slots whose cosine is
    within 1e-5 of the maximum)``."""
    if T > 1:
        return _top1_union(q, q_ids, cache_k, cache_ids, n, P, T)
    Q = _f64(q)
    K = _f64(cache_k[:n])
    kid = np.asarray(cache_ids[:n]).astype(np.int64)
    qid = np.asarray(q_ids).astype(np.int64)
    N = Q.shape[0]
    best = np.full(N, -1, np.int64)
    cos = np.full(N, -np.inf)
    tie = np.zeros(N, bool)
    near: List[np.ndarray] = [np.zeros(0, np.int64) for _ in range(N)]
    qn = np.linalg.norm(Q, axis=1)
    kn = np.linalg.norm(K, axis=1)
    for b in np.unique(qid):
        qi = np.nonzero(qid == b)[0]
        kj = np.nonzero(kid == b)[0]
        if kj.size == 0:
            continue
        den = qn[qi][:, None] * kn[kj][None, :]
        dots = Q[qi] @ K[kj].T
        c = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        a = np.argmax(c, axis=1)            # first maximum = lowest slot
        s = c[np.arange(qi.size), a]
        best[qi] = kj[a]
        cos[qi] = s
        for r, i in enumerate(qi):
            close = kj[c[r] >= s[r] - TIE_EPS]
            near[i] = close
            tie[i] = close.size > 1
    return best, cos, tie, near


def _top1_union(q, q_ids, cache_k, cache_ids, n: int, P: int, T: int):
    """tempcache_top1 over the union of a query's T buckets (R18): the same
    cosine, ties and flags, candidates from any table."""
    Q = _f64(q)
    K = _f64(cache_k[:n])
    fq, fk = bucket_fields(q_ids, P, T), bucket_fields(np.asarray(cache_ids)[:n], P, T)
    N = Q.shape[0]
    best = np.full(N, -1, np.int64)
    cos = np.full(N, -np.inf)
    tie = np.zeros(N, bool)
    near: List[np.ndarray] = [np.zeros(0, np.int64) for _ in range(N)]
    qn = np.linalg.norm(Q, axis=1)
    kn = np.linalg.norm(K, axis=1)
    for i in range(N):
        kj = np.nonzero((fk == fq[i][None, :]).any(axis=1))[0]
        if kj.size == 0:
            continue
        den = qn[i] * kn[kj]
        dots = K[kj] @ Q[i]
        c = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        a = int(np.argmax(c))
        best[i], cos[i] = kj[a], c[a]
        near[i] = kj[c >= c[a] - TIE_EPS]
        tie[i] = near[i].size > 1
    return best, cos, tie, near


def tempcache_commit(cache: Dict[str, np.ndarray], n: int, k_cur, v_cur, kcur_ids,
                     best, cos, tau: float, step: int, merge: bool = False):
    """Apply one chunk's merge/append/evict to one head's cache (R6-R9).

    ``cache`` holds ``k``, ``v`` [cap, d], ``ids`` [cap], ``ts`` [cap]; it is
    not modified.  Returns a dict with the new ``cache``, ``n`` (valid slots
    after the update), ``dest`` [N] (slot each token was written to, -1 if it
    was merged away), ``evicted`` [N] (-1 padded, ascending slots),
    ``counts`` = (matched, refreshed, dropped, appended, evicted),
    ``matched`` [N] and ``thr_tie`` [N] (|cos - tau| < 1e-5).

    ``merge`` selects the mean-merge variant (R10-R12): ``cache`` then also
    holds ``count`` [cap] (group sizes), the new cache's ``v`` is float64 and
    its ``count`` is updated; slot choice, keys, ids, timestamps, dest,
    evicted and counts are those of the replacement rule."""
    K, V = cache["k"], cache["v"]
    ids, ts = np.asarray(cache["ids"]), np.asarray(cache["ts"])
    cap = K.shape[0]
    best = np.asarray(best).astype(np.int64)
    cos = _f64(cos)
    N = best.size
    if N > cap:
        raise ValueError("a chunk larger than the cache capacity cannot be committed")
    if not 0 <= n <= cap:
        raise ValueError("n must lie in [0, cap]")
    has_cand = (best >= 0) & (best < n)                      # R9
    matched = has_cand & (cos >= tau)                          # R6, inclusive
    claim = np.full(cap, -1, np.int64)
    for i in range(N):
        if matched[i]:
            claim[best[i]] = max(claim[best[i]], i)            # most recent wins
    refreshed = claim >= 0
    dest = np.full(N, -1, np.int64)
    for j in np.nonzero(refreshed)[0]:
        dest[claim[j]] = j
    unmatched = [i for i in range(N) if not matched[i]]
    u = len(unmatched)
    e = max(0, n + u - cap)
    candidates = [j for j in range(n) if not refreshed[j]]
    oldest = sorted(candidates, key=lambda j: (int(ts[j]), j))[:e]    # R7
    evicted_slots = sorted(oldest)
    n_new = min(cap, n + u)
    free = list(range(n, n_new)) + evicted_slots
    for slot, i in zip(free, unmatched):
        dest[i] = slot
    new = {"k": np.array(K, copy=True), "v": np.array(V, copy=True),
           "ids": np.array(ids, copy=True), "ts": np.array(ts, copy=True)}
    kcur_ids = np.asarray(kcur_ids)
    if merge:
        if "count" not in cache:
            raise ValueError("the mean-merge variant needs the cache's group sizes")
        m_old = np.asarray(cache["count"], np.int64)
        new["v"] = _f64(V).copy()
        new["count"] = m_old.copy()
        # R11: every claimant joins its slot's group; the group's value is the
        # mean over old members and claimants, its size grows by the claimants
        for j in np.nonzero(refreshed)[0]:
            members = [i for i in range(N) if matched[i] and best[i] == j]
            total = m_old[j] * _f64(V[j]) + sum(_f64(v_cur[i]) for i in members)
            new["count"][j] = m_old[j] + len(members)
            new["v"][j] = total / new["count"][j]
    for i in range(N):
        j = dest[i]
        if j >= 0:
            new["k"][j] = k_cur[i]
            new["ids"][j] = kcur_ids[i]
            new["ts"][j] = step                                # R8
            if not merge:
                new["v"][j] = v_cur[i]
            elif not matched[i]:                               # R12: a new group of one
                new["v"][j] = v_cur[i]
                new["count"][j] = 1
    evicted = np.full(N, -1, np.int64)
    evicted[:e] = evicted_slots
    n_matched = int(matched.sum())
    n_ref = int(refreshed.sum())
    counts = np.array([n_matched, n_ref, n_matched - n_ref, n_new - n, e], np.int64)
    thr_tie = has_cand & (np.abs(cos - tau) < TIE_EPS)
    return {"cache": new, "n": n_new, "dest": dest, "evicted": evicted, "counts": counts,
            "matched": matched, "thr_tie": thr_tie}


def eviction_candidates(ts, n: int, N: int) -> np.ndarray:
    """The slots an update of N tokens may evict (R7): the min(n, N) valid
    slots that come first in (timestamp, slot) order, listed by slot,
    padded with -1 to length N.  R7 evicts the e oldest non-refreshed slots;
    with r refreshed slots and u unmatched tokens, e <= u and r + u <= N, so
    each evicted slot has at most e - 1 + r <= N - 1 slots before it in that
    order and always lies in this list."""
    ts = np.asarray(ts)
    if not 0 <= n <= ts.shape[0] or N < 0:
        raise ValueError("need 0 <= n <= cap and N >= 0")
    m = min(n, N)
    first = sorted(range(n), key=lambda j: (int(ts[j]), j))[:m]
    out = np.full(N, -1, np.int64)
    out[:m] = sorted(first)
    return out


def tempcache_update(cache: Dict[str, np.ndarray], n: int, q, q_ids, k_cur, v_cur, kcur_ids,
                     tau: float, step: int, merge: bool = False):
    """Top-1 search, then commit (blog, "1. TempCache"; ``merge``: R10-R12)."""
    best, cos, tie, near = tempcache_top1(q, q_ids, cache["k"], cache["ids"], n)
    out = tempcache_commit(cache, n, k_cur, v_cur, kcur_ids, best, cos, tau, step, merge)
    out.update(best=best, cos=cos, argmax_tie=tie, near=near)
    return out


# ---------------------------------------------------------------------------
# One attention step, all heads: hash -> AnnSA -> AnnCA -> TempCache commit
# (attend to [old cache ; current chunk], then commit the chunk)
# ---------------------------------------------------------------------------

def attention_step(q, k_cur, v_cur, cache_k, cache_v, cache_ids, cache_ts, n_valid,
                   planes, kp, vp, frame_len: int, tau: float, step: int,
                   scale: Optional[float] = None, heads=None,
                   cache_count=None) -> Dict[str, object]:
    """Runs the whole step head by head; arrays carry a leading head axis.
    ``cache_count`` [H, cap] selects the mean-merge variant (R10-R12)."""
    H = q.shape[0] if heads is None else len(heads)
    heads = range(q.shape[0]) if heads is None else heads
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    res: Dict[str, list] = {k: [] for k in ("q_ids", "kcur_ids", "kp_ids", "hash_tie",
                                            "o_sa", "lse", "o_ca", "keep", "tc")}
    for h in heads:
        qi, tq = ann_hash(q[h], planes[h])
        ki, tk = ann_hash(k_cur[h], planes[h])
        pi, tp = ann_hash(kp[h], planes[h])
        n = int(n_valid[h])
        K, V, kid = key_context(cache_k[h], cache_v[h], cache_ids[h], n, k_cur[h], v_cur[h], ki)
        merge = cache_count is not None
        cnt = key_counts(cache_count[h], n, k_cur.shape[1]) if merge else None
        o_sa, lse = annsa(q[h], qi, K, V, kid, scale, cnt)
        o_ca, keep = annca(q[h], qi, frame_len, kp[h], vp[h], pi, scale)
        ch = {"k": cache_k[h], "v": cache_v[h], "ids": cache_ids[h], "ts": cache_ts[h]}
        if merge:
            ch["count"] = cache_count[h]
        tc = tempcache_update(ch, n, q[h], qi, k_cur[h], v_cur[h], ki, tau, step, merge)
        for key, val in (("q_ids", qi), ("kcur_ids", ki), ("kp_ids", pi),
                         ("hash_tie", (tq, tk, tp)), ("o_sa", o_sa), ("lse", lse),
                         ("o_ca", o_ca), ("keep", keep), ("tc", tc)):
            res[key].append(val)
    res["H"] = H
    return res

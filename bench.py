"""Benchmark of one FAST-AR attention step on one MI355X.

A step is the whole hot path over one chunk of the Wan-1.3B-like layer
(12 heads x d=128, bf16; a 3-frame chunk of 4680 tokens; a full 32760-slot
cache; 7 hyperplanes = 128 buckets; 512 prompt tokens):

    ann_hash(q), ann_hash(k_cur), ann_hash(prompt k)
    annsa_forward   (bucket sort + gathered MFMA attention over [cache ; chunk];
                     the same pass returns TempCache's top-1 for every query)
    annca_forward   (prompt selection + cross-attention over the kept tokens)
    tempcache_update(claims from that top-1 + select + row scatter)

The step runs on two streams: AnnCA (independent of the cache) overlaps the
TempCache commit, whose select phase keeps only one CU per head busy, and
the side stream lists the commit's eviction candidates while AnnSA runs.  The
headline (``ms_per_step`` = ``ms_per_step_graph``) replays the K timed steps
captured as one HIP graph, each step on its own cache copy -- the way a
model's forward pass captures its layers, so each step is one layer's
attention and no step waits on the host's per-launch cost or on a graph
launch of its own; ``ms_per_step_graph_one_per_step`` captures one graph per
step and replays the K graphs back to back (each replay's start-up then falls
inside every step); ``ms_per_step_eager_two_stream`` issues the same calls one
by one and ``ms_per_step_eager_one_stream`` issues them on one stream.
``mean_merge`` times the same step on a mean-merged cache (Lemma 5.1 of the
FAST-AR summary: slots carry group sizes, AnnSA adds ln m to their logits and
the commit folds matched tokens into their slot's group).  ``multi_table``
times AnnSA (with the search) over two hash tables of P planes each -- the
union of a query's two buckets -- against one table on the same chunk.
``quantize`` times the step with nearest-codeword buckets (a 2^P-codeword
codebook per head) in place of the hyperplanes.

Inputs are seeded synthetic tensors, resident in HBM before the timed region.
Every timed step starts from its own pristine copy of the cache (the commit
mutates it), so each step sees exactly the same workload.

Output: one JSON line.  ``value`` is the achieved bf16 TFLOP/s on kept pairs,
4*d*(AnnSA kept pairs + AnnCA kept pairs) / step time; ``ms_per_step`` is the
step latency.  ``roofline`` describes the dominant kernel (AnnSA's bucket
attention, HBM-bound): algorithmic bytes per launch / its mean duration from
HIP events on its launch stream, taken in a one-stream pass where every
kernel runs alone.  ``cpu_baseline`` times the CPU oracle on a
bounded sample of heads of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
HBM_TARGET_FRAC = 0.60         # targets: hash / sort / compaction at 60% of HBM peak,
MFMA_TARGET_FRAC = 0.40        # bucket attention at 40% of the bf16 MFMA peak

# HBM bytes per launch of the AnnSA attention kernel, from rocprofv3's
# FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) scaled by what the same
# counters read for a device copy of known size.  ``--ingest-counters`` writes
# them to TRAFFIC_FILE together with the SHA-256 of the kernel's sources; the
# bench line reports them only while those sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "annsa_traffic_wan13.json")
KERNEL_SOURCES = ["sparse_attention_autoregressive_amd/csrc/attn.hip",
                  "sparse_attention_autoregressive_amd/csrc/common.hpp",
                  "sparse_attention_autoregressive_amd/csrc/launch.hpp",
                  "sparse_attention_autoregressive_amd/build.py"]
ANNSA_KERNEL = "attn_kv_kernel<unsigned short, 128, 0, true, float, 4, false, false>"


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(config: str, out_dtype: str):
    """(bytes per launch, note) for the AnnSA kernel built from the current
    sources (their SHA-256 must match the record's), or (None, why not)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("config") != config or rec.get("out_dtype") != out_dtype:
        return None, f"counters taken on {rec.get('config')} / {rec.get('out_dtype')}"
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    return rec["traffic_bytes"], f"{os.path.relpath(TRAFFIC_FILE, ROOT)} (sources sha256 {rec['sources_sha256'][:12]})"


def ingest_counters(paths):
    """Writes TRAFFIC_FILE from four rocprofv3 counter CSVs: FETCH_SIZE and
    WRITE_SIZE of a bench run, then of ``--copy-calibration`` (a device copy of
    known size, whose counters give the scale factors)."""
    import csv
    fetch, write, cfetch, cwrite = paths

    def per_kernel(path):
        acc = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                v = acc.setdefault(row["Kernel_Name"], [0, 0.0])
                v[0] += 1
                v[1] += float(row["Counter_Value"])
        return {k: (n, tot / n) for k, (n, tot) in acc.items()}

    def copy_kib(path):
        rows = [v for k, v in per_kernel(path).items() if "copyBuffer" in k]
        if not rows:
            raise SystemExit(f"{path}: no device-copy dispatch")
        return max(r[1] for r in rows)

    def annsa(path):
        rows = [v for k, v in per_kernel(path).items() if ANNSA_KERNEL in k]
        if len(rows) != 1:
            raise SystemExit(f"{path}: expected one {ANNSA_KERNEL} kernel, found {len(rows)}")
        return rows[0]

    copy_bytes = 512 * (1 << 20)
    f_scale = copy_bytes / 1024 / copy_kib(cfetch)
    w_scale = copy_bytes / 1024 / copy_kib(cwrite)
    nf, fk = annsa(fetch)
    nw, wk = annsa(write)
    rec = {"kernel": ANNSA_KERNEL, "config": "wan13_bf16", "out_dtype": "f32",
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk, "dispatches": [nf, nw],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "traffic_bytes": (f_scale * fk + w_scale * wk) * 1024,
           "sources": KERNEL_SOURCES, "sources_sha256": kernel_sources_sha256(),
           "commands": [
               "cd /tmp && export TMPDIR=/tmp",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/FETCH_SIZE -o FETCH_SIZE "
               "-- python3 <repo>/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-merge --no-multi --no-quantize",
               "rocprofv3 --pmc WRITE_SIZE (the same bench command)",
               "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE -- python3 <repo>/bench.py --copy-calibration 512",
               "python3 bench.py --ingest-counters <the four counter_collection.csv files>"],
           "counter_files": [os.path.relpath(p, ROOT) for p in paths]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec), flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="wan13_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU-oracle sample budget (heads are added until it is spent)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge", action="store_true",
                    help="skip the mean-merged-cache variant of the step")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the two-table AnnSA measurement")
    ap.add_argument("--no-quantize", action="store_true",
                    help="skip the quantization-bucket step")
    ap.add_argument("--mfma-sweep", action="store_true",
                    help="only time the bucket-attention kernel at P = 0, 1, 2, 3 and the "
                         "config's P (one JSON line: TFLOP/s on kept pairs vs the bf16 MFMA peak)")
    ap.add_argument("--size-sweep", action="store_true",
                    help="only run hash, bucket sort and AnnCA selection at batched sizes "
                         "(the step's heads x 1..64) and report their GB/s")
    ap.add_argument("--rollout", type=int, default=0, metavar="CHUNKS",
                    help="only run a rollout of CHUNKS chunks: per-chunk step latency and cache "
                         "size, next to a dense uncapped-cache baseline (one JSON line)")
    ap.add_argument("--cpu-baseline-calls", action="store_true",
                    help="only time the oracle per ABI call and per step (tiny and single-head "
                         "configs) and per step over every head (Wan-1.3B and Wan-14B shapes), next "
                         "to the library on the same inputs (one JSON line)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only write the AnnSA traffic record from rocprofv3 counter CSVs "
                         "(FETCH_SIZE and WRITE_SIZE of a bench run, then of --copy-calibration 512)")
    ap.add_argument("--graph-only", action="store_true",
                    help="only replay the K timed steps captured in one graph (after a W-step "
                         "warm-up graph): the headline timing alone, for kernel traces (one JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (the plain copy whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the traffic figures), then exit")
    return ap.parse_args()


def copy_calibration(mib):
    """Five device-to-device copies of ``mib`` MiB: a kernel whose HBM traffic
    is known exactly (reads = writes = mib MiB per copy)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda").mul_(1.0001)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 5}), flush=True)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.mfma_sweep:
        mfma_sweep(args)
        return
    if args.rollout > 0:
        rollout(args)
        return
    if args.size_sweep:
        size_sweep(args)
        return
    if args.cpu_baseline_calls:
        cpu_baseline_calls(args)
        return
    if args.graph_only:
        graph_only(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(every head is independent, so several GPUs would each take a share of the heads "
              "with no exchange inside the step)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_autoregressive_amd as fa
    from workloads import CONFIGS, f32_to_bf16_bits, make_step

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = make_step(cfg, args.seed)

    def to_dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    H, Nq, d, cap, P = cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P
    q, kc, vc = to_dev(st.q), to_dev(st.k_cur), to_dev(st.v_cur)
    kp, vp = to_dev(st.kp), to_dev(st.vp)
    planes = torch.from_numpy(st.planes).to(dev)
    # cached keys carry their bucket ids and norms
    base = fa.KVCache.from_keys(to_dev(st.cache_k), to_dev(st.cache_v),
                                torch.from_numpy(st.cache_ts).to(dev),
                                torch.from_numpy(st.n_valid).to(dev), planes)
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    from sparse_attention_autoregressive_amd.step import AttentionStep
    mk = lambda overlap: AttentionStep(H, Nq, d, cap, P, cfg.frame_len, cfg.L, cfg.tau,
                                       out_dtype=out_dt, device=dev, overlap=overlap)
    two, one = mk(True), mk(False)
    ids = two.ids
    # every step commits into its own pristine copy of the cache
    n_copies = 4 * args.warmup + 8 * args.steps
    caches = [base.clone() for _ in range(n_copies)]
    it = iter(caches)
    run = lambda s, c: s(c, q, kc, vc, kp, vp, planes, st.step)

    for _ in range(args.warmup):
        run(two, next(it))
        run(one, next(it))
    torch.cuda.synchronize()
    # one captured graph per cache copy (addresses are baked into a graph)
    graphs = [two.graph(next(it), q, kc, vc, kp, vp, planes, st.step)
              for _ in range(args.warmup + args.steps)]
    for g in graphs[:args.warmup]:
        g.replay()

    # the K timed steps captured into one graph, each on its own cache copy
    # (as a model's layers); a graph of W steps warms the same path first
    def steps_graph(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                run(two, next(it))
        return g

    g_warm, g_steps = steps_graph(args.warmup), steps_graph(args.steps)
    if args.warmup > 0:
        g_warm.replay()
    torch.cuda.synchronize()

    def timed(fn):
        main = torch.cuda.current_stream(dev)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(main)
        for i in range(args.steps):
            fn(i)
        t1.record(main)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    # ---- timed regions: the step as K graph replays (the headline); K
    # two-stream steps issued call by call, and K issued on one stream
    main_s = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(main_s)
    g_steps.replay()
    e1.record(main_s)
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / args.steps
    ms_graph_each = timed(lambda i: graphs[args.warmup + i].replay())
    ms_eager_two = timed(lambda i: run(two, next(it)))
    ms_one_stream = timed(lambda i: run(one, next(it)))
    cnt = two.keep_count

    # ---- latency distribution: K two-stream steps, each between its own
    # events; warm (back to back) and cold (a 512 MiB write before each step
    # evicts the 256 MB last-level cache; the write is outside the events)
    def per_step(cold):
        main = torch.cuda.current_stream(dev)
        flush = torch.empty(512 << 18, dtype=torch.float32, device=dev) if cold else None
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            if cold:
                flush.fill_(1.0)
            a.record(main)
            run(two, next(it))
            b.record(main)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        pick = lambda f: ts[min(len(ts) - 1, int(f * len(ts)))]
        return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9)}
    latency = {"warm": per_step(False), "cold": per_step(True)}

    # ---- K eager one-stream steps again with per-kernel HIP events: every
    # kernel runs alone, so its mean duration is its own
    with fa.kernel_timer() as kt:
        for _ in range(args.steps):
            run(one, next(it))
    torch.cuda.synchronize()
    kernel_ms = {k: v[1] / max(1, v[0]) for k, v in kt.times.items()}
    kernel_launches = {k: v[0] // args.steps for k, v in kt.times.items()}

    # ---- the commit's select with the eviction candidates listed on the side
    # stream beforehand (what a captured step does): K eager two-stream steps
    # with the list, per-kernel HIP events on each kernel's own stream (the
    # list overlaps AnnSA, so its duration includes that sharing)
    listed = AttentionStep(H, Nq, d, cap, P, cfg.frame_len, cfg.L, cfg.tau, out_dtype=out_dt,
                           device=dev, overlap=True, order_list=True)
    run(listed, next(it))
    torch.cuda.synchronize()
    with fa.kernel_timer() as kt_l:
        for _ in range(args.steps - 1):
            run(listed, next(it))
    torch.cuda.synchronize()
    kl = {k: v[1] / max(1, v[0]) for k, v in kt_l.times.items()}
    eviction_list = {"tempcache_order_ms": kl.get("tempcache_order"),
                     "tempcache_select_ms_listed": kl.get("tempcache_select"),
                     "tempcache_select_ms_full_scan": kernel_ms.get("tempcache_select")}

    # ---- work accounting (not timed): kept pairs and algorithmic bytes
    B = 1 << P
    qi = ids["q"].long() & 0xFFFF
    ki = torch.cat([base.ids.long() & 0xFFFF, ids["k"].long() & 0xFFFF], dim=1)
    nqb = torch.stack([torch.bincount(qi[h], minlength=B) for h in range(H)]).double()
    nkb = torch.stack([torch.bincount(ki[h], minlength=B) for h in range(H)]).double()
    sa_pairs = float((nqb * nkb).sum())
    ca_pairs = float(cnt.double().sum() * cfg.frame_len)
    flops = 4.0 * d * (sa_pairs + ca_pairs)
    ms_per_step = ms_graph
    value_tflops = flops / (ms_per_step * 1e-3) / 1e12

    esz = 2 if cfg.dtype == "bf16" else 4
    osz = 4 if out_dt == torch.float32 else 2
    keys_read = float((nkb * (nqb > 0)).sum())                 # each kept key row once
    ci = base.ids.long() & 0xFFFF
    nkc = torch.stack([torch.bincount(ci[h], minlength=B) for h in range(H)]).double()
    cached_read = float((nkc * (nqb > 0)).sum())                # their norms, for the search
    # Q in; K and V of every kept key; O, lse, best slot and cosine out; key norms
    sa_bytes = (Nq * H * d * esz + keys_read * 2 * d * esz + Nq * H * (d * osz + 4 + 8)
                + cached_read * 4)
    attn_ms = kernel_ms.get("annsa_attn")
    achieved = sa_bytes / (attn_ms * 1e-3) / 1e9 if attn_ms else None
    traffic, traffic_note = measured_traffic(args.config, args.out_dtype)
    roofline = {"kernel": "annsa_attn", "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                "traffic": traffic, "traffic_source": traffic_note,
                "algorithmic_bytes": sa_bytes,
                "mean_ms": attn_ms}

    # algorithmic bytes of the other kernels, per step (all launches of the kernel)
    F = Nq // cfg.frame_len
    probe = base.clone()                      # one more commit, for the written-token count
    res = fa.tempcache_update(probe, q, ids["q"], kc, vc, ids["k"], P, cfg.tau, st.step,
                              best_in=two.best, cos_in=two.best_cos)
    written = float((res["dest"] >= 0).sum())
    ca_keys = float(cnt.double().sum())
    # AnnCA's prompt selection: ids read, keep mask and counts written (and the
    # kept index lists when a long prompt takes the separate launch); up to
    # 1024 prompt tokens the attention launch does it
    sel_bytes = H * (Nq + F * cfg.L) * 2.0 + H * F * (cfg.L + 4.0)
    sel_fused = "annca_select" not in kernel_ms
    step_bytes = {
        "ann_hash": (2 * Nq + cfg.L) * H * (d * esz + 2),
        "sort": 6.0 * H * (2 * Nq + cap),                       # id read, perm written
        "annca_select": sel_bytes + H * F * cfg.L * 4.0,
        "annca_attn": Nq * H * (d * esz + d * osz) + ca_keys * 2 * d * esz + (sel_bytes if sel_fused else 0),
        "tempcache_select": H * Nq * 12.0 + H * cap * 4.0,      # best, cos in, dest out; ts
        "tempcache_scatter": written * (4 * d * esz + 10) + H * Nq * 4.0,
        "annsa_attn": sa_bytes,
    }
    step_ms = {
        "ann_hash": kernel_ms.get("ann_hash", 0) * kernel_launches.get("ann_hash", 0),
        "sort": sum(kernel_ms.get(k, 0) for k in ("sort_hist", "sort_scan", "sort_scatter")),
        "annca_select": kernel_ms.get("annca_select"), "annca_attn": kernel_ms.get("annca_attn"),
        "tempcache_select": kernel_ms.get("tempcache_select"),
        "tempcache_scatter": kernel_ms.get("tempcache_scatter"), "annsa_attn": attn_ms,
    }
    kernel_gbs = {k: {"bytes": step_bytes[k], "GB/s": step_bytes[k] / (step_ms[k] * 1e-3) / 1e9,
                      "frac_hbm_peak": step_bytes[k] / (step_ms[k] * 1e-3) / 1e9 / HBM_PEAK_GBS}
                  for k in step_bytes if step_ms.get(k)}
    # the HBM target for hash, sort and compaction (60% of peak), stated
    # beside each such kernel's fraction
    for k in ("ann_hash", "sort", "annca_select"):
        if k in kernel_gbs:
            kernel_gbs[k]["target_frac_hbm_peak"] = HBM_TARGET_FRAC
            kernel_gbs[k]["target_met"] = kernel_gbs[k]["frac_hbm_peak"] >= HBM_TARGET_FRAC
    # bucket attention against the bf16 MFMA peak (kept-pair products,
    # 4 d flops per pair), with its 40% target
    kernel_mfma = {}
    for k, pairs in (("annsa_attn", sa_pairs), ("annca_attn", ca_pairs)):
        if step_ms.get(k):
            tf = 4.0 * d * pairs / (step_ms[k] * 1e-3) / 1e12
            kernel_mfma[k] = {"kept_pair_TFLOP/s": tf, "frac_bf16_mfma_peak": tf / BF16_PEAK_TFLOPS,
                              "target_frac": MFMA_TARGET_FRAC, "target_met": tf / BF16_PEAK_TFLOPS >= MFMA_TARGET_FRAC}

    # ---- the same step on a mean-merged cache (Lemma 5.1 of the FAST-AR
    # summary): slots carry group sizes (uniform 1..32), AnnSA shifts their
    # logits by ln m and the commit folds every matched token into its slot
    merge = None
    if not args.no_merge:
        from workloads import group_sizes
        mbase = base.clone()
        mbase.count = torch.from_numpy(group_sizes(args.seed, H, cap)).to(dev)
        mit = iter([mbase.clone() for _ in range(args.warmup + 2 * args.steps)])
        for _ in range(args.warmup):
            run(two, next(mit))
        ms_merge = timed(lambda i: run(two, next(mit)))
        with fa.kernel_timer() as kt2:
            for _ in range(args.steps):
                run(one, next(mit))
        torch.cuda.synchronize()
        mk_ms = {k: v[1] / max(1, v[0]) for k, v in kt2.times.items()}
        mprobe = mbase.clone()
        mres = fa.tempcache_update(mprobe, q, ids["q"], kc, vc, ids["k"], P, cfg.tau, st.step,
                                   best_in=two.best, cos_in=two.best_cos)
        mcounts = mres["counts"].double().sum(0)
        matched, groups = float(mcounts[0]), float(mcounts[1])
        mwritten = float((mres["dest"] >= 0).sum())
        # K row copied, norm/id/ts per written token; a group reads its old value,
        # its members' values and its size, writes value and size; the other
        # written tokens copy their value; dest and group size/offset per token
        mbytes = (mwritten * (2 * d * esz + 10) + groups * (2 * d * esz + 8)
                  + matched * (d * esz + 4) + (mwritten - groups) * (2 * d * esz + 4)
                  + H * Nq * 12.0)
        ms_ms = mk_ms.get("tempcache_merge_scatter")
        merge = {"ms_per_step": ms_merge, "launch": "eager, two streams",
                 "ms_per_step_replacement_same_launch": ms_eager_two,
                 "value_tflops": flops / (ms_merge * 1e-3) / 1e12,
                 "group_sizes": "uniform 1..32 per slot",
                 "kernel_ms": mk_ms,
                 "merge_scatter": {"bytes": mbytes,
                                   "GB/s": mbytes / (ms_ms * 1e-3) / 1e9 if ms_ms else None,
                                   "groups": groups, "matched": matched},
                 "annsa_attn_GB/s": sa_bytes / (mk_ms["annsa_attn"] * 1e-3) / 1e9
                 if mk_ms.get("annsa_attn") else None}

    # ---- multi-table AnnSA (blog, "3. AnnSA": several buckets per token): the
    # same chunk and cache hashed into two tables of P planes each; AnnSA with
    # the fused search over the union of buckets, timed alone (the cache is
    # only read), against the one-table call on the same ids' first field
    multi = None
    if not args.no_multi:
        from workloads import table_planes
        T = 2
        mpl = torch.from_numpy(table_planes(args.seed, H, T, P, d)).to(dev)
        mq, mk = fa.ann_hash(q, mpl), fa.ann_hash(kc, mpl)
        mc = base.clone()
        fa.ann_hash(mc.k, mpl, ids=mc.ids, norms=mc.knorm)
        lib = fa.load()
        mws = torch.empty(lib.fastar_annsa_multi_workspace(H, Nq, cap, Nq, d, P, T), dtype=torch.uint8,
                          device=dev)
        mo = torch.empty(H, Nq, d, dtype=out_dt, device=dev)
        ml = torch.empty(H, Nq, dtype=torch.float32, device=dev)
        mb = torch.empty(H, Nq, dtype=torch.int32, device=dev)
        mcos = torch.empty(H, Nq, dtype=torch.float32, device=dev)
        one_mask = (1 << P) - 1
        mq1, mk1 = (mq.int() & one_mask).short(), (mk.int() & one_mask).short()
        mc1 = mc.clone()
        mc1.ids.copy_((mc.ids.int() & one_mask).short())
        call = lambda tb, qq, kk, cc: fa.annsa_forward(q, qq, kc, vc, kk, P, cache=cc, out=mo, lse=ml,
                                                       ws=mws, search=True, best=mb, best_cos=mcos,
                                                       tables=tb)
        for _ in range(args.warmup):
            call(T, mq, mk, mc)
            call(1, mq1, mk1, mc1)
        ms_multi = timed(lambda i: call(T, mq, mk, mc))
        ms_single = timed(lambda i: call(1, mq1, mk1, mc1))
        with fa.kernel_timer() as kt3:
            for _ in range(args.steps):
                call(T, mq, mk, mc)
        torch.cuda.synchronize()
        k3 = {k: (v[0] // args.steps, v[1] / args.steps) for k, v in kt3.times.items()}
        # kept pairs: the union over tables by inclusion-exclusion over table subsets
        qid = mq.long() & 0xFFFF
        kid = torch.cat([mc.ids.long() & 0xFFFF, mk.long() & 0xFFFF], dim=1)
        union = 0.0
        per_table_keys = 0.0
        for sub in range(1, 1 << T):
            fmask = sum(one_mask << (t * P) for t in range(T) if (sub >> t) & 1)
            sgn = 1.0 if bin(sub).count("1") % 2 else -1.0
            for h in range(H):
                nq = torch.bincount(qid[h] & fmask, minlength=1 << 16).double()
                nk = torch.bincount(kid[h] & fmask, minlength=1 << 16).double()
                union += sgn * float((nq * nk).sum())
                if bin(sub).count("1") == 1:
                    per_table_keys += float((nk * (nq > 0)).sum())
        attn_ms_total = k3.get("annsa_attn", (0, 0.0))[1]
        # per table: Q, each kept key row (K, V, id, norm); state out/in between
        # tables; the last table writes O, lse, best and cosine
        mbytes = (T * H * Nq * (2 * d + 2) + per_table_keys * (4 * d + 6)
                  + (T - 1) * 2 * H * Nq * (4 * d + 16) + H * Nq * (d * osz + 12))
        multi = {"tables": T, "planes_per_table": P, "ms_annsa": ms_multi,
                 "ms_annsa_one_table": ms_single,
                 "kept_pairs_union": union, "kept_pairs_one_table_equiv": sa_pairs,
                 "tflops_union_pairs": 4.0 * d * union / (ms_multi * 1e-3) / 1e12,
                 "kernel_ms_per_call": {k: v[1] for k, v in k3.items()},
                 "launches_per_call": {k: v[0] for k, v in k3.items()},
                 "attn": {"bytes": mbytes, "ms": attn_ms_total,
                          "GB/s": mbytes / (attn_ms_total * 1e-3) / 1e9 if attn_ms_total else None}}

    # ---- quantization buckets (summary, Core Components A/B): the same step
    # with nearest-codeword ids from a 2^P-codeword codebook per head (drawn from
    # the cached keys) instead of the hyperplanes
    quant = None
    if not args.no_quantize:
        from workloads import codebook_from_keys
        Bq = 1 << P
        cbk = torch.from_numpy(codebook_from_keys(st.cache_k, st.n_valid, Bq, args.seed)).to(dev)
        qbase = base.clone()
        fa.ann_quantize(qbase.k, cbk, ids=qbase.ids, norms=qbase.knorm)
        qs = AttentionStep(H, Nq, d, cap, P, cfg.frame_len, cfg.L, cfg.tau, out_dtype=out_dt,
                           device=dev, overlap=True, ann="quantize")
        qs1 = AttentionStep(H, Nq, d, cap, P, cfg.frame_len, cfg.L, cfg.tau, out_dtype=out_dt,
                            device=dev, overlap=False, ann="quantize")
        qit = iter([qbase.clone() for _ in range(args.warmup + 2 * args.steps)])
        qrun = lambda s_, c_: s_(c_, q, kc, vc, kp, vp, cbk, st.step)
        for _ in range(args.warmup):
            qrun(qs, next(qit))
        ms_quant = timed(lambda i: qrun(qs, next(qit)))
        with fa.kernel_timer() as kt4:
            for _ in range(args.steps):
                qrun(qs1, next(qit))
        torch.cuda.synchronize()
        q_ms = {k: v[1] / max(1, v[0]) for k, v in kt4.times.items()}
        q_launch = {k: v[0] // args.steps for k, v in kt4.times.items()}
        # the quantize launches of a one-stream step (one launch for Q, K_cur and
        # the prompt): 2 N B d flops per vector set (N = Nq, Nq, L per head)
        qz_launches = max(1, q_launch.get("ann_quantize", 1))
        qz_flops = 2.0 * H * (2 * Nq + cfg.L) * Bq * d / qz_launches
        qz_bytes = H * (2 * Nq + cfg.L) * (d * esz + 2) / qz_launches
        qz_ms = q_ms.get("ann_quantize")
        quant = {"codewords": Bq, "ms_per_step": ms_quant, "launch": "eager, two streams",
                 "ms_per_step_hyperplanes_same_launch": ms_eager_two, "kernel_ms": q_ms,
                 "kernel_launches_per_step": q_launch,
                 "ann_quantize": {"flops_per_launch": qz_flops, "bytes_per_launch": qz_bytes,
                                  "TFLOP/s": qz_flops / (qz_ms * 1e-3) / 1e12 if qz_ms else None,
                                  "GB/s": qz_bytes / (qz_ms * 1e-3) / 1e9 if qz_ms else None,
                                  "fp32_mfma_peak_TFLOP/s": 157.3}}

    line = {
        "metric": "attention step latency (ms) + achieved bf16 TFLOP/s on kept pairs, Wan-1.3B chunk",
        "value": value_tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "ms_per_step_graph": ms_graph,
        "ms_per_step_graph_one_per_step": ms_graph_each,
        "ms_per_step_eager_two_stream": ms_eager_two, "ms_per_step_eager_one_stream": ms_one_stream,
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {H} heads x d={d}, chunk {cfg.Fq} frames x "
                               f"{cfg.frame_len} = {Nq} tokens, cache {cap} slots (full), "
                               f"P={P} ({B} buckets), prompt {cfg.L}, tau={cfg.tau}",
                   "out_dtype": args.out_dtype, "seed": args.seed, "streams": 2,
                   "launch": "hip graph: the timed steps captured in one graph, one cache copy each "
                             "(as a model's layers), replayed once"},
        "roofline": roofline,
        "latency_ms": latency,
        "kernel_ms": kernel_ms, "kernel_launches_per_step": kernel_launches,
        "kernel_gbs": kernel_gbs, "kernel_mfma": kernel_mfma, "eviction_list": eviction_list,
        "kept_pairs": {"annsa": sa_pairs, "annca": ca_pairs,
                       "annsa_frac_of_dense": sa_pairs / (H * Nq * (cap + Nq))},
        "mean_merge": merge,
        "multi_table": multi,
        "quantize": quant,
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.seed, args.cpu_seconds, line)
    print(json.dumps(line), flush=True)


def graph_only(args):
    """The headline timing alone: W warm-up steps and then the K timed steps,
    each captured into one graph (one pristine cache copy per step), the
    timed graph replayed once."""
    import torch

    import sparse_attention_autoregressive_amd as fa
    from sparse_attention_autoregressive_amd.step import AttentionStep
    from workloads import CONFIGS, make_step

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = make_step(cfg, args.seed)
    to_dev = _device(cfg, dev)
    t = {k: to_dev(getattr(st, k)) for k in ("q", "k_cur", "v_cur", "kp", "vp")}
    t["planes"] = torch.from_numpy(st.planes).to(dev)
    base = fa.KVCache.from_keys(to_dev(st.cache_k), to_dev(st.cache_v), torch.from_numpy(st.cache_ts).to(dev),
                                torch.from_numpy(st.n_valid).to(dev), t["planes"])
    out_dt = torch.float32 if args.out_dtype == "f32" else torch.bfloat16
    s = AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau, out_dtype=out_dt,
                      device=dev)

    def steps_graph(caches):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in caches:
                s(c, t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], t["planes"], st.step)
        return g

    warm = [base.clone() for _ in range(max(1, args.warmup))]
    timed = [base.clone() for _ in range(args.steps)]
    g_warm, g_steps = steps_graph(warm), steps_graph(timed)
    g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_steps.replay()
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"graph_only": True, "config": cfg.name, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step_graph": e0.elapsed_time(e1) / args.steps}), flush=True)


def _device(cfg, dev):
    import numpy as np
    import torch
    from workloads import f32_to_bf16_bits

    def to_dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    return to_dev


def _pairs(qi, ki, B):
    import torch
    H = qi.shape[0]
    nqb = torch.stack([torch.bincount(qi[h].long() & 0xFFFF, minlength=B) for h in range(H)]).double()
    nkb = torch.stack([torch.bincount(ki[h].long() & 0xFFFF, minlength=B) for h in range(H)]).double()
    return float((nqb * nkb).sum())


def mfma_sweep(args):
    """Bucket attention (AnnSA without the search) at fewer buckets: P = 0 is
    dense attention over [cache ; chunk], where the kernel's arithmetic
    intensity is far above the ridge, so its TFLOP/s on kept pairs against the
    dense bf16 MFMA peak measures the matrix-core side of the kernel."""
    import torch
    import sparse_attention_autoregressive_amd as fa
    from workloads import CONFIGS, make_step
    cfg0 = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    lib = fa.load()
    rows = []
    for P in sorted({0, 1, 2, 3, cfg0.P}):
        cfg = cfg0.replace(P=P)
        st = make_step(cfg, args.seed)
        to_dev = _device(cfg, dev)
        H, Nq, d, cap = cfg.H, cfg.Nq, cfg.d, cfg.cap
        q, kc, vc = to_dev(st.q), to_dev(st.k_cur), to_dev(st.v_cur)
        planes = torch.from_numpy(st.planes).to(dev)
        cache = fa.KVCache.from_keys(to_dev(st.cache_k), to_dev(st.cache_v),
                                     torch.from_numpy(st.cache_ts).to(dev),
                                     torch.from_numpy(st.n_valid).to(dev), planes)
        qi, ki = fa.ann_hash(q, planes), fa.ann_hash(kc, planes)
        ws = torch.empty(lib.fastar_annsa_workspace(H, Nq, cap, Nq, P), dtype=torch.uint8, device=dev)
        out = torch.empty(H, Nq, d, dtype=torch.float32, device=dev)
        lse = torch.empty(H, Nq, dtype=torch.float32, device=dev)
        call = lambda: fa.annsa_forward(q, qi, kc, vc, ki, P, cache=cache, out=out, lse=lse, ws=ws)
        call()
        torch.cuda.synchronize()
        reps = 3 if P == 0 else 10
        with fa.kernel_timer() as kt:
            for _ in range(reps):
                call()
        torch.cuda.synchronize()
        launches, total = kt.times["annsa_attn"]
        ms = total / launches
        pairs = _pairs(qi, torch.cat([cache.ids, ki], dim=1), 1 << P)
        tflops = 4.0 * d * pairs / (ms * 1e-3) / 1e12
        rows.append({"P": P, "buckets": 1 << P, "kept_pairs": pairs, "ms": ms, "TFLOP/s": tflops,
                     "frac_mfma_peak": tflops / BF16_PEAK_TFLOPS,
                     "arith_intensity": 4.0 * d * pairs / (
                         Nq * H * (d * 2 + d * 4 + 4) + float(H * (cap + Nq)) * 4 * d)})
        print(json.dumps({"progress": "mfma_sweep", "P": P, "ms": ms}), file=sys.stderr, flush=True)
        del cache, ws, q, kc, vc
        torch.cuda.empty_cache()
    print(json.dumps({"mfma_sweep": rows, "kernel": "annsa_attn (no search)", "peak_tflops": BF16_PEAK_TFLOPS,
                      "config": cfg0.name, "dtype": cfg0.dtype, "out_dtype": "f32"}), flush=True)


def size_sweep(args):
    """The step's small kernels at batched sizes: the hash over H x (k x Nq)
    bf16 vectors, the bucket sort over as many ids, and AnnCA's prompt
    selection over k x H heads (k chunks' worth of heads, the real 4680
    queries each and a 2048-token prompt: the separate selection launch
    serves prompts longer than 1024 tokens, shorter ones are selected inside
    the attention launch).  At the step's own size these
    kernels move a few MB and are bound by launch latency; the sweep shows
    the bandwidth each reaches once the work is large enough.  Algorithmic
    bytes: hash 2d + 2 per vector (row in, id out); sort 2 + 4 per id (id in,
    perm out); selection 2 per query id and per prompt id read, 1 + 4 per
    (frame, prompt token) written (keep byte, index) plus the frame's count."""
    import numpy as np
    import torch
    import sparse_attention_autoregressive_amd as fa
    from workloads import CONFIGS
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, Nq, d, P, L, fl = cfg.H, cfg.Nq, cfg.d, cfg.P, cfg.L, cfg.frame_len
    B = 1 << P
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    esz = 2 if cfg.dtype == "bf16" else 4
    planes = torch.randn(H, P, d, generator=gen, device=dev)
    reps = 10
    rows = []

    def kernel_ms(call, names):
        call()
        torch.cuda.synchronize()
        with fa.kernel_timer() as kt:
            for _ in range(reps):
                call()
        torch.cuda.synchronize()
        return sum(kt.times[n][1] for n in names if n in kt.times) / reps

    for k in (1, 4, 16, 64):
        N = k * Nq
        x = torch.randn(H, N, d, generator=gen, device=dev).to(dt)
        ids = torch.empty(H, N, dtype=torch.int16, device=dev)
        ms = kernel_ms(lambda: fa.ann_hash(x, planes, ids=ids), ["ann_hash"])
        nbytes = H * N * (d * esz + 2.0)
        rows.append({"kernel": "ann_hash", "vectors": H * N, "bytes": nbytes, "ms": ms,
                     "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del x
        sid = torch.randint(0, B, (H, N), generator=gen, device=dev, dtype=torch.int32).to(torch.int16)
        ws = torch.empty(fa.load().fastar_bucket_sort_workspace(H, N, P), dtype=torch.uint8, device=dev)
        ms = kernel_ms(lambda: fa.bucket_sort(sid, P, ws=ws), ["sort_hist", "sort_scan", "sort_scatter"])
        nbytes = H * N * 6.0
        rows.append({"kernel": "bucket_sort", "ids": H * N, "bytes": nbytes, "ms": ms,
                     "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del sid, ws
        print(json.dumps({"progress": "size_sweep", "k": k}), file=sys.stderr, flush=True)
    # the separate selection launch serves prompts longer than 1024 tokens
    # (shorter ones are selected inside the attention launch): 2048 here
    F, L = Nq // fl, 2048
    for k in (1, 16, 64):
        Hk = k * H
        qi = torch.randint(0, B, (Hk, Nq), generator=gen, device=dev, dtype=torch.int32).to(torch.int16)
        pi = torch.randint(0, B, (Hk, L), generator=gen, device=dev, dtype=torch.int32).to(torch.int16)
        q = torch.randn(Hk, Nq, d, generator=gen, device=dev).to(dt)
        kp = torch.randn(Hk, L, d, generator=gen, device=dev).to(dt)
        vp = torch.randn(Hk, L, d, generator=gen, device=dev).to(dt)
        out = torch.empty(Hk, Nq, d, dtype=torch.float32, device=dev)
        keep = torch.empty(Hk, F, L, dtype=torch.uint8, device=dev)
        ws = torch.empty(fa.load().fastar_annca_workspace(Hk, Nq, fl, L, P), dtype=torch.uint8, device=dev)
        ms = kernel_ms(lambda: fa.annca_forward(q, qi, fl, kp, vp, pi, P, out=out, keep=keep, ws=ws),
                       ["annca_select"])
        nbytes = Hk * (Nq + F * L) * 2.0 + Hk * F * (L * 5.0 + 4.0)
        rows.append({"kernel": "annca_select", "heads": Hk, "prompt": L, "bytes": nbytes, "ms": ms,
                     "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
        del q, kp, vp, out, ws
        print(json.dumps({"progress": "size_sweep annca", "k": k}), file=sys.stderr, flush=True)
    print(json.dumps({"size_sweep": rows, "config": cfg.name, "dtype": cfg.dtype, "P": P,
                      "peak_GB/s": HBM_PEAK_GBS, "inputs": "uniform random ids, N(0,1) vectors"}),
          flush=True)


def rollout(args):
    """A long rollout on the same layer: every chunk runs the full step on a
    bounded cache (two streams), each between its own events; beside it a
    dense baseline (one bucket, no merging, the cache grows by a chunk per
    step: the same kernels at P = 0) is timed every 10th chunk, and so is the
    CPU oracle (after the GPU loop, on one head per sampled chunk, from a copy
    of the cache state the GPU step started that chunk from)."""
    import torch
    import sparse_attention_autoregressive_amd as fa
    from sparse_attention_autoregressive_amd.step import AttentionStep
    from workloads import CONFIGS, make_step, rollout_chunks
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    lib = fa.load()
    to_dev = _device(cfg, dev)
    H, Nq, d, cap, P = cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P
    n_chunks = args.rollout
    st = make_step(cfg, args.seed)
    planes = torch.from_numpy(st.planes).to(dev)
    kp, vp = to_dev(st.kp), to_dev(st.vp)
    cache = fa.KVCache.from_keys(to_dev(st.cache_k), to_dev(st.cache_v),
                                 torch.from_numpy(st.cache_ts).to(dev),
                                 torch.from_numpy(st.n_valid).to(dev), planes)
    stepper = AttentionStep(H, Nq, d, cap, P, cfg.frame_len, cfg.L, cfg.tau, device=dev)
    # dense baseline: uncapped cache, all ids 0
    n0 = int(st.n_valid[0])
    cap_d = n0 + n_chunks * Nq
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dk = torch.zeros(H, cap_d, d, dtype=dt, device=dev)
    dv = torch.zeros(H, cap_d, d, dtype=dt, device=dev)
    dk[:, :n0] = cache.k[:, :n0]
    dv[:, :n0] = cache.v[:, :n0]
    dense = fa.KVCache(k=dk, v=dv, ids=torch.zeros(H, cap_d, dtype=torch.int16, device=dev),
                       ts=torch.zeros(H, cap_d, dtype=torch.int32, device=dev),
                       n_valid=torch.full((H,), n0, dtype=torch.int32, device=dev),
                       knorm=torch.zeros(H, cap_d, dtype=torch.float32, device=dev))
    zq = torch.zeros(H, Nq, dtype=torch.int16, device=dev)
    zp = torch.zeros(H, cfg.L, dtype=torch.int16, device=dev)
    ws_sa = torch.empty(lib.fastar_annsa_workspace(H, Nq, cap_d, Nq, 0), dtype=torch.uint8, device=dev)
    ws_ca = torch.empty(lib.fastar_annca_workspace(H, Nq, cfg.frame_len, cfg.L, 0), dtype=torch.uint8,
                        device=dev)
    o_sa = torch.empty(H, Nq, d, dtype=torch.float32, device=dev)
    o_ca = torch.empty_like(o_sa)
    main = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # every chunk is generated and moved to the device first, so the timed
    # loop never waits on the host (an idle GPU drops its clocks)
    chunks = []
    for c, ch in enumerate(rollout_chunks(cfg, n_chunks, args.seed)):
        chunks.append((to_dev(ch["q"]), to_dev(ch["k_cur"]), to_dev(ch["v_cur"]), ch["step"]))
        if c % 20 == 0:
            print(json.dumps({"progress": "rollout inputs", "chunk": c}), file=sys.stderr, flush=True)
    slots_dev = torch.zeros(n_chunks, H, dtype=torch.int32, device=dev)
    fast_ev, dense_ev, dense_slots = [], {}, {}
    snaps = {}                 # every 10th chunk: one head's cache as the step found it (device copies)
    n_dense = n0
    torch.cuda.synchronize()
    for c, (q, kc, vc, step) in enumerate(chunks):
        if c % 10 == 0 and not args.no_cpu_baseline:
            hs = (c // 10) % H
            snaps[c] = (hs, cache.k[hs].clone(), cache.v[hs].clone(), cache.ids[hs].clone(),
                        cache.ts[hs].clone(), cache.n_valid[hs:hs + 1].clone())
        a, b = ev(), ev()
        a.record(main)
        stepper(cache, q, kc, vc, kp, vp, planes, step)
        b.record(main)
        fast_ev.append((a, b))
        slots_dev[c].copy_(cache.n_valid)
        if c % 10 == 0 or c == n_chunks - 1:
            a, b = ev(), ev()
            a.record(main)
            fa.annsa_forward(q, zq, kc, vc, zq, 0, cache=dense, out=o_sa, ws=ws_sa)
            fa.annca_forward(q, zq, cfg.frame_len, kp, vp, zp, 0, out=o_ca, ws=ws_ca)
            b.record(main)
            dense_ev[c] = (a, b)
            dense_slots[c] = n_dense
        dk[:, n_dense:n_dense + Nq] = kc                # the dense cache appends the chunk
        dv[:, n_dense:n_dense + Nq] = vc
        n_dense += Nq
        dense.n_valid.fill_(n_dense)
    torch.cuda.synchronize()
    slots = slots_dev.max(dim=1).values.tolist()
    fast_ms = [a.elapsed_time(b) for a, b in fast_ev]
    dense_ms = {c: a.elapsed_time(b) for c, (a, b) in dense_ev.items()}
    row_bytes = d * (2 if cfg.dtype == "bf16" else 4) * 2 * H
    # the oracle on every 10th chunk, one head each (cycling), from the cache
    # state the GPU step started that chunk from
    oracle = None
    if snaps:
        import numpy as np
        from oracle import attention_step
        host = lambda t: t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
        per_chunk = {}
        for c, (hs, k_, v_, ids_, ts_, n_) in snaps.items():
            q, kc, vc, step = chunks[c]
            sl = slice(hs, hs + 1)
            t0 = time.perf_counter()
            attention_step(host(q[sl]), host(kc[sl]), host(vc[sl]), host(k_)[None], host(v_)[None],
                           ids_.cpu().numpy().view(np.uint16)[None], ts_.cpu().numpy()[None], n_.cpu().numpy(),
                           st.planes[sl], host(kp[sl]), host(vp[sl]), cfg.frame_len, cfg.tau, step)
            per_chunk[c] = (time.perf_counter() - t0) * 1e3
        oracle = {"ms_per_head": per_chunk, "ms_per_step_equiv_median": float(np.median(list(per_chunk.values()))) * H,
                  "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                  "sample": f"one head per sampled chunk (heads cycled), every 10th chunk, "
                            f"started from the GPU's cache state of that chunk; step = {H} heads"}
    print(json.dumps({"rollout": {
        "config": cfg.name, "chunks": n_chunks, "fastar_step_ms": fast_ms,
        "fastar_cache_slots": slots, "fastar_cache_kv_bytes": cap * row_bytes,
        "dense_attention_ms": dense_ms, "dense_cache_slots": dense_slots,
        "dense_cache_kv_bytes_final": n_dense * row_bytes, "cpu_oracle": oracle,
        "note": "FAST-AR: the whole step (hash, AnnSA + search, AnnCA, commit) on a cache capped at "
                f"{cap} slots; dense: AnnSA + AnnCA at one bucket over the uncapped cache "
                "(attention only), timed every 10th chunk"}}), flush=True)


def cpu_baseline(cfg, seed, budget_s, line):
    """The oracle (unchanged) on whole heads of the same workload until the
    budget is spent; scaled to TFLOP/s on kept pairs."""
    import numpy as np
    from oracle import ann_hash, attention_step
    from workloads import make_step
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:                                        # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    t_total, pairs, heads = 0.0, 0.0, 0
    h = 0
    while t_total < budget_s and heads < 16 * cfg.H:
        st = make_step(cfg, seed, heads=range(h, h + 1))
        cid = np.stack([ann_hash(st.cache_k[0], st.planes[0])[0]])
        t0 = time.perf_counter()
        r = attention_step(st.q, st.k_cur, st.v_cur, st.cache_k, st.cache_v, cid, st.cache_ts,
                           st.n_valid, st.planes, st.kp, st.vp, cfg.frame_len, cfg.tau, st.step)
        t_total += time.perf_counter() - t0
        qi = r["q_ids"][0].astype(np.int64)
        ki = np.concatenate([cid[0], r["kcur_ids"][0]]).astype(np.int64)
        B = 1 << cfg.P
        pairs += float((np.bincount(qi, minlength=B) * np.bincount(ki, minlength=B)).sum())
        pairs += float(r["keep"][0].sum() * cfg.frame_len)
        heads += 1
        h = (h + 1) % cfg.H
    value = 4.0 * cfg.d * pairs / t_total / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": min(cores, threads) if threads else cores,
            "kind": "oracle",
            "sample": f"{heads} head-passes (heads cycled, {cfg.H} per step) of the same step "
                      f"(hash + AnnSA + AnnCA + TempCache), "
                      f"{t_total:.1f} s on the host; BLAS threads {threads}, affinity cores {cores}",
            "ms_per_step_equiv": t_total / heads * cfg.H * 1e3}


def cpu_baseline_calls(args):
    """The cpu_baseline leg per call: the oracle (unchanged) timed per ABI call
    and per step on the tiny and single-head configs, and per step over every
    head on the Wan-1.3B and Wan-14B shapes, each next to the library's time
    for the same work on the same inputs.  Library calls are eager (host
    launch cost included; H = 1 calls are launch-bound), each averaged over
    20 calls between two events; every commit and every step gets a cache
    copy made before timing starts.  The library's step is the two-stream
    ``AttentionStep`` (eagerly at the small configs, as a graph replay at the
    Wan shapes, as the main bench line times it).  One JSON line."""
    import math
    import numpy as np
    import torch
    import sparse_attention_autoregressive_amd as fa
    from oracle import (ann_hash as o_hash, annca as o_annca, annsa as o_annsa, attention_step,
                        bucket_sort as o_sort, key_context, tempcache_commit, tempcache_top1)
    from sparse_attention_autoregressive_amd.step import AttentionStep
    from workloads import CONFIGS, f32_to_bf16_bits, make_step
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:                                        # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    reps = 20

    def cpu_ms(fn, n=3):
        fn()                                                 # untimed: first-call costs
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        return (time.perf_counter() - t0) / n * 1e3

    def gpu_ms(fns):
        """``fns``: one callable per timed call (a list, so each may use its own copy)."""
        fns[0]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for fn in fns[1:]:
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (len(fns) - 1)

    def inputs(cfg, st):
        def to_dev(a):
            if cfg.dtype == "bf16":
                return torch.from_numpy(f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        t = {k: to_dev(getattr(st, k)) for k in ("q", "k_cur", "v_cur", "kp", "vp")}
        t["planes"] = torch.from_numpy(st.planes).to(dev)
        t["cache"] = fa.KVCache.from_keys(to_dev(st.cache_k), to_dev(st.cache_v),
                                          torch.from_numpy(st.cache_ts).to(dev),
                                          torch.from_numpy(st.n_valid).to(dev), t["planes"])
        return t

    out = {"calls": [], "steps": []}
    for name in ("tiny_f32", "single_bf16"):
        cfg = CONFIGS[name]
        st = make_step(cfg, args.seed)
        P, fl, d = cfg.P, cfg.frame_len, cfg.d
        scale = 1.0 / math.sqrt(d)
        n = int(st.n_valid[0])
        q, kc, vc, kp, vp, pl = st.q[0], st.k_cur[0], st.v_cur[0], st.kp[0], st.vp[0], st.planes[0]
        cid = o_hash(st.cache_k[0], pl)[0]
        qi, ki, pi = (o_hash(x, pl)[0] for x in (q, kc, kp))
        K, V, kid = key_context(st.cache_k[0], st.cache_v[0], cid, n, kc, vc, ki)
        best, bcos = tempcache_top1(q, qi, st.cache_k[0], cid, n)[:2]
        cache0 = {"k": st.cache_k[0], "v": st.cache_v[0], "ids": cid, "ts": st.cache_ts[0]}
        tau32 = float(np.float32(cfg.tau))
        oracle = {
            "ann_hash (Q, K_cur, prompt keys)": lambda: [o_hash(x, pl) for x in (q, kc, kp)],
            "bucket sort (query ids, key ids)": lambda: (o_sort(qi, P), o_sort(kid, P)),
            "annsa_forward (attention)": lambda: o_annsa(q, qi, K, V, kid, scale),
            "TempCache top-1 (fused into annsa_forward on the GPU)":
                lambda: tempcache_top1(q, qi, st.cache_k[0], cid, n),
            "annca_forward": lambda: o_annca(q, qi, fl, kp, vp, pi, scale),
            "tempcache_update (commit on the given top-1)":
                lambda: tempcache_commit({k: v.copy() for k, v in cache0.items()}, n, kc, vc, ki,
                                         best, bcos, tau32, st.step),
        }
        t = inputs(cfg, st)
        ids = {k: torch.empty(1, x.shape[1], dtype=torch.int16, device=dev)
               for k, x in (("q", t["q"]), ("k", t["k_cur"]), ("p", t["kp"]))}
        fa.ann_hash_batch([t["q"], t["k_cur"], t["kp"]], t["planes"], ids=[ids["q"], ids["k"], ids["p"]])
        keyset = torch.cat([t["cache"].ids[:, :n], ids["k"]], dim=1).contiguous()
        sa = lambda: fa.annsa_forward(t["q"], ids["q"], t["k_cur"], t["v_cur"], ids["k"], P, cache=t["cache"],
                                      search=True)
        _, _, gbest, gcos = sa()
        copies = [t["cache"].clone() for _ in range(reps + 1)]
        gpu = {
            "ann_hash (Q, K_cur, prompt keys)": [lambda: fa.ann_hash_batch(
                [t["q"], t["k_cur"], t["kp"]], t["planes"], ids=[ids["q"], ids["k"], ids["p"]])] * (reps + 1),
            "bucket sort (query ids, key ids)": [lambda: (fa.bucket_sort(ids["q"], P),
                                                          fa.bucket_sort(keyset, P))] * (reps + 1),
            "annsa_forward (attention)": [sa] * (reps + 1),
            "annca_forward": [lambda: fa.annca_forward(t["q"], ids["q"], fl, t["kp"], t["vp"], ids["p"], P)]
                             * (reps + 1),
            "tempcache_update (commit on the given top-1)": [
                (lambda c=c: fa.tempcache_update(c, t["q"], ids["q"], t["k_cur"], t["v_cur"], ids["k"], P,
                                                 cfg.tau, st.step, best_in=gbest, cos_in=gcos))
                for c in copies],
        }
        for call, fn in oracle.items():
            row = {"config": name, "call": call, "oracle_ms": cpu_ms(fn)}
            if call in gpu:
                row["gpu_ms"] = gpu_ms(gpu[call])
                row["ratio"] = row["oracle_ms"] / row["gpu_ms"]
            out["calls"].append(row)
            print(json.dumps({"progress": row}), file=sys.stderr, flush=True)
        cpu_step = cpu_ms(lambda: attention_step(st.q, st.k_cur, st.v_cur, st.cache_k, st.cache_v, cid[None],
                                                 st.cache_ts, st.n_valid, st.planes, st.kp, st.vp, fl, cfg.tau,
                                                 st.step))
        s = AttentionStep(cfg.H, cfg.Nq, d, cfg.cap, P, fl, cfg.L, cfg.tau, device=dev)
        scopies = [t["cache"].clone() for _ in range(reps + 1)]
        g = gpu_ms([(lambda c=c: s(c, t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], t["planes"], st.step))
                    for c in scopies])
        out["steps"].append({"config": name, "heads": cfg.H, "oracle_ms": cpu_step, "gpu_ms": g,
                             "gpu_form": "eager, two streams", "ratio": cpu_step / g})
        print(json.dumps({"progress": out["steps"][-1]}), file=sys.stderr, flush=True)
        del t, copies, scopies
    for name in ("wan13_bf16", "wan14_bf16"):
        cfg = CONFIGS[name]
        t_cpu = 0.0
        for h in range(cfg.H):                   # one head at a time: the oracle's memory stays small
            st = make_step(cfg, args.seed, heads=range(h, h + 1))
            cid = o_hash(st.cache_k[0], st.planes[0])[0]
            t0 = time.perf_counter()
            attention_step(st.q, st.k_cur, st.v_cur, st.cache_k, st.cache_v, cid[None], st.cache_ts,
                           st.n_valid, st.planes, st.kp, st.vp, cfg.frame_len, cfg.tau, st.step)
            t_cpu += time.perf_counter() - t0
        st = make_step(cfg, args.seed)
        t = inputs(cfg, st)
        s = AttentionStep(cfg.H, cfg.Nq, cfg.d, cfg.cap, cfg.P, cfg.frame_len, cfg.L, cfg.tau, device=dev)
        graphs = [s.graph(t["cache"].clone(), t["q"], t["k_cur"], t["v_cur"], t["kp"], t["vp"], t["planes"],
                          st.step) for _ in range(reps + 1)]
        g = gpu_ms([gr.replay for gr in graphs])
        out["steps"].append({"config": name, "heads": cfg.H, "oracle_ms": t_cpu * 1e3, "gpu_ms": g,
                             "gpu_form": "graph replay, two streams", "ratio": t_cpu * 1e3 / g})
        print(json.dumps({"progress": out["steps"][-1]}), file=sys.stderr, flush=True)
        del t, graphs
    out.update({"kind": "oracle", "cores": min(cores, threads) if threads else cores,
                "blas_threads": threads, "affinity_cores": cores, "seed": args.seed,
                "oracle_reps": "3 calls averaged after one untimed call (small configs); one pass over every head (Wan shapes)"})
    print(json.dumps({"cpu_baseline_calls": out}), flush=True)


if __name__ == "__main__":
    main()

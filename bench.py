"""Throughput of the two-tier sparse-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: compressor for the group each
query completes, indexer scores, candidate-block + top-512 selection, gather attention.
Default workload: decode, 128 sequences at 131072 raw tokens (65536 compressed latents
at ratio 2), fp8-e4m3 index keys. Inputs are synthetic (seeded) and resident in HBM
before timing starts.

Prints one JSON line with queries/s, the indexer kernel's HBM roofline fraction (HIP
events on the launch stream), the step's fraction of HBM, a prefill chunk's fraction of
bf16 MFMA peak, and the fp64 CPU oracle timed on a bounded sample.

A second object times a layer that only indexes: it re-scores the 2048 candidate blocks
the two-stage pass kept (candidate-bounded indexer, selection inside them, attention).
A third times a multi-token decode step: 128 sequences x 6 queries (a verified token and
5 drafted ones) whose indexer streams each sequence's keys once per group. A fourth times
the headline decode batch with MXFP4 index keys (the 4-bit indexer cache), and a fifth its
indexer, selection and attention on paged stores (64-row pages, block tables). A sixth
times a ragged serving batch (prefill chunks, drafted decode steps and single decode queries
in one call), a seventh the headline batch with e4m3 latent and window rows, and an eighth
with MXFP4 latent rows and e4m3 window rows. The other layer configurations get one object
each: the 4-query batch at 2K context (latency), the 64-query batch at 32K context (warm, and
cold: two copies of its stores used in turn, 2 x 319 MB against the 256 MiB last-level cache),
the 8-query batch at 1M context, and a 1-to-1 layer at 1M context (2 queries, 2^20 positions
each). The compressor alone runs over the raw context of the 64-query batch (64 x 32768 raw
latents into 64 x 16384 compressed ones).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-prefill] [--no-rescore] [--no-multiquery] [--no-mxfp4] [--no-paged]
                       [--no-ragged] [--no-fp8kv] [--no-configs] [--no-compress]
                       [--only LEG[,LEG...]] [--no-cpu-baseline] [--profile]
Legs for --only: paged, rescore, multiquery, mxfp4, fp8kv, ragged, prefill, c1, c2, c5, r1m,
compress, cpu (the headline decode batch always runs: it is the reported value).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # flop/s, MI355X dense bf16 MFMA
IDX_BYTES_PER_QUERY_FIXED = 16 * 128 * 2 + 16 * 4        # index query + head weights
LATENT_ROW = 512 * 2


INDEXER_SOURCES = ("sparse_attention_score_amd/csrc/indexer.hip", "sparse_attention_score_amd/csrc/sa_device.h",
                   "sparse_attention_score_amd/csrc/sa_launch.h", "sparse_attention_score_amd/csrc/sa_compress.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_decode-b128-ctx128k-fp8_traffic.json")
RESCORE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_cand_decode-b128-ctx128k-fp8_traffic.json")
GROUP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_group_decode-mq6-b128-ctx128k-fp8_traffic.json")
MX_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_mx_decode-b128-ctx128k-mxfp4_traffic.json")
CONFIG_TRAFFIC_FILES = {"decode-b64-ctx32k": os.path.join(ROOT, "profiles", "indexer_decode-b64-ctx32k_traffic.json"),
                        "decode-b8-ctx1m-fp8": os.path.join(ROOT, "profiles", "indexer_decode-b8-ctx1m-fp8_traffic.json")}
COMPRESS_SOURCES = ("sparse_attention_score_amd/csrc/compress.hip", "sparse_attention_score_amd/csrc/sa_compress.h",
                    "sparse_attention_score_amd/csrc/sa_device.h", "sparse_attention_score_amd/csrc/sa_launch.h")
COMPRESS_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "compress_raw-64x32768_traffic.json")
COPY_BYTES = 1 << 30


def indexer_source_hash(sources=INDEXER_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload: str, path: str = TRAFFIC_FILE, sources=INDEXER_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if there is
    none for this workload or the kernel's sources changed since it was taken."""
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("workload") != workload or d.get("source_sha256") != indexer_source_hash(sources):
        return None
    return d.get("traffic_bytes_per_launch")


def copy_bandwidth(torch):
    """A plain 1 GiB device-to-device copy: measured ceiling, and the calibration kernel for
    the FETCH_SIZE / WRITE_SIZE counters."""
    n = COPY_BYTES // 4
    x = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del x, y
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (ms * 1e-3)


def key_row_bytes(key_dtype: str) -> int:
    """Bytes of one index key row with its scales: e4m3 + fp32 scale, MXFP4 + 4 E8M0, bf16."""
    return {"fp8": 128 + 4, "mxfp4": 64 + 4}.get(key_dtype, 256)


def indexer_bytes(wl) -> float:
    """Algorithmic bytes of one indexer launch: every visible index key (and its fp8 row
    scale) of every query, plus the index queries and weights."""
    n = wl.visible().astype(np.float64)
    return float((n * key_row_bytes(wl.key_dtype)).sum() + wl.T * IDX_BYTES_PER_QUERY_FIXED)


def step_bytes(wl) -> float:
    """Algorithmic bytes of one whole step: index keys, selected latents, window rows,
    q, output, index query/weights, selected ids (materialised scores excluded)."""
    n = wl.visible().astype(np.float64)
    k = np.minimum(512, n)
    win = np.minimum(128, wl.pos.astype(np.float64) + 1)
    per_q = (n * key_row_bytes(wl.key_dtype) + k * LATENT_ROW + win * LATENT_ROW
             + 64 * 512 * 2 * 2 + IDX_BYTES_PER_QUERY_FIXED + 512 * 4)
    groups = len(wl.compress_groups())
    return float(per_q.sum() + groups * (2 * 2 * 512 * 2 + 512 * 2) + 2 * 512 * 4)


def group_indexer_bytes(wl) -> float:
    """Algorithmic bytes of one grouped indexer launch: each sequence's visible index keys
    (and fp8 row scales) once, up to the largest n of its queries, plus every query's index
    query and weights."""
    nseq = np.zeros(wl.B, dtype=np.float64)
    np.maximum.at(nseq, wl.seq.astype(np.int64), wl.visible().astype(np.float64))
    return float((nseq * key_row_bytes(wl.key_dtype)).sum() + wl.T * IDX_BYTES_PER_QUERY_FIXED)


def rescore_bytes(wl, carried: np.ndarray) -> float:
    """Algorithmic bytes of one candidate-bounded indexer launch: the index keys (and fp8
    row scales) of the visible positions inside every query's carried blocks, the carried
    block ids, and the index queries and weights."""
    n = wl.visible().astype(np.int64)[:, None]
    ids = carried.astype(np.int64)
    valid = (ids >= 0) & (ids < (n + 7) // 8)
    rows = np.where(valid, np.minimum(8, n - 8 * ids), 0).sum()
    return float(rows * key_row_bytes(wl.key_dtype) + wl.T * (IDX_BYTES_PER_QUERY_FIXED + 2048 * 4))


def step_flops(wl) -> tuple:
    n = wl.visible().astype(np.float64)
    k = np.minimum(512, n)
    win = np.minimum(128, wl.pos.astype(np.float64) + 1)
    idx = float((n * 16 * 128 * 2).sum())
    attn = float((64 * (k + win) * 512 * 4).sum())
    return idx, attn


class Timer:
    """HIP events recorded on the launch stream around each stage of every timed step."""

    def __init__(self, torch, names):
        self.torch = torch
        self.names = names
        self.ev = []

    def step(self, fns):
        t = self.torch
        evs = [t.cuda.Event(enable_timing=True)]
        evs[0].record()
        for f in fns:
            f()
            e = t.cuda.Event(enable_timing=True)
            e.record()
            evs.append(e)
        self.ev.append(evs)

    def mean_ms(self):
        out = {n: 0.0 for n in self.names}
        for evs in self.ev:
            for i, n in enumerate(self.names):
                out[n] += evs[i].elapsed_time(evs[i + 1])
        return {n: v / max(1, len(self.ev)) for n, v in out.items()}


def warm_up(torch, fns, warmup, min_seconds):
    """W untimed steps, then more until `min_seconds` of GPU work have run, so the clocks
    have left their idle state before anything is timed."""
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < min_seconds:
        for f in fns:
            f()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def run_batch(torch, d, steps, warmup, min_warm_s=0.5):
    """Eager steps with HIP events on the launch stream around every stage.
    Returns (seconds per step, mean stage milliseconds)."""
    stages = ["compress", "indexer", "select", "attention"]
    fns = [d.compress, d.index, d.select, d.attend]
    warm_up(torch, fns, warmup, min_warm_s)
    timer = Timer(torch, stages)
    t0 = time.perf_counter()
    for _ in range(steps):
        timer.step(fns)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps, timer.mean_ms()


def run_plain(torch, d, steps):
    """`steps` eager steps launched back to back on one stream (no events between stages),
    bracketed by device synchronisation; the compressor rides in the indexer's launch."""
    fns = d.step_fns()
    for _ in range(3):
        for f in fns:
            f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def run_graph(torch, d, steps):
    """The same step captured once in a HIP graph and replayed `steps` times: the timed
    region holds exactly those replays, bracketed by device synchronisation."""
    g = d.capture()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del g
    return (t1 - t0) / steps, e0.elapsed_time(e1) * 1e-3 / steps


def best_step(torch, d, steps):
    """Seconds per step of the faster of HIP graph replays and plain back-to-back launches
    (each timed over `steps` steps bracketed by device synchronisation), and which it was."""
    graph_s, _ = run_graph(torch, d, steps)
    plain_s = run_plain(torch, d, steps)
    return min((plain_s, "eager launches back to back"), (graph_s, "HIP graph replays of the whole step"))


def capture(torch, fns):
    """The launches of `fns` captured once in a HIP graph (first run outside capture)."""
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def run_rescore(torch, d, steps, warmup, profile=False):
    """A layer that only indexes: it re-scores the candidate blocks an earlier layer's
    candidate stage kept (here the batch's own two-stage pass), selects the top-512 inside
    them and attends. Eager steps with HIP events on the launch stream around each stage,
    then the same three launches as graph replays.
    Returns (carried block ids [T][2048], eager s/layer, graph s/layer or None, stage ms)."""
    import sparse_attention_score_amd as S
    d.index()
    d.select()
    torch.cuda.synchronize()
    carried = d.cand.clone()
    T = d.T
    sc = torch.empty((T, 2048 * 8), dtype=torch.float32, device="cuda")
    bm = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
    tk = torch.empty((T, 512), dtype=torch.int32, device="cuda")
    fns = [lambda: S.indexer_score_cand(d.plan, d.queries, d.cache, d.qI, d.w, carried, sc, bm),
           lambda: S.select_topk_cand(d.plan, d.queries, carried, sc, bm, tk),
           lambda: d.attend(topk=tk)]
    warm_up(torch, fns, warmup, 0.0 if profile else 0.5)
    timer = Timer(torch, ["indexer", "select", "attention"])
    t0 = time.perf_counter()
    for _ in range(steps):
        timer.step(fns)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / steps
    graph = None
    if not profile:
        g = capture(torch, fns)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph = (time.perf_counter() - t0) / steps
        del g
    return carried.cpu().numpy(), eager, graph, timer.mean_ms()


def paged_copy(torch, d, P, seed=0):
    """The batch's latents, index keys and e4m3 scales as pools of P-row pages in a shuffled
    order, with the block table that addresses them."""
    import sparse_attention_score_amd as S
    B, cap = d.C.shape[0], d.C.shape[1]
    assert cap % P == 0
    per = cap // P
    ids = torch.from_numpy(np.random.default_rng(seed).permutation(B * per).astype(np.int64)).cuda()

    def pool_of(x):
        pages = x.reshape((B * per, P) + tuple(x.shape[2:]))
        pool = torch.empty_like(pages)
        pool[ids] = pages
        return pool.reshape((B * per * P,) + tuple(x.shape[2:]))

    table = ids.to(torch.int32).reshape(B, per).contiguous()
    return S.Cache(latents=pool_of(d.C), window=d.R, idx_keys=pool_of(d.KI),
                   idx_scales=pool_of(d.KS) if d.KS is not None else None, num_seqs=B,
                   compressed_cap=cap, block_table=table, page_size=P)


def run_paged(torch, d, steps, warmup, P=64, profile=False):
    """Indexer, selection and attention of the batch on paged stores (eager, HIP events),
    then the same three launches as graph replays."""
    import sparse_attention_score_amd as S
    cache = paged_copy(torch, d, P)
    torch.cuda.synchronize()
    fns = [lambda: S.indexer_score(d.plan, d.queries, cache, d.qI, d.w, d.scores, d.block_max),
           d.select,
           lambda: S.sparse_attn_fwd(d.plan, d.queries, cache, d.q, d.topk, d.out, d.lse,
                                     workspace=d.workspace)]
    warm_up(torch, fns, warmup, 0.0 if profile else 0.5)
    timer = Timer(torch, ["indexer", "select", "attention"])
    for _ in range(steps):
        timer.step(fns)
    torch.cuda.synchronize()
    graph = None
    if not profile:
        g = capture(torch, fns)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph = (time.perf_counter() - t0) / steps
        del g
    ms = timer.mean_ms()
    del cache
    torch.cuda.empty_cache()
    return graph, ms


def cpu_baseline(wl, budget_s=20.0, max_queries=None):
    """The fp64 oracle, as it stands, over the first queries of the batch until the time
    budget is spent (at least one query). Returns queries/s and the sample description."""
    from oracle import oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = 1
    t0 = time.perf_counter()
    C_new = O.step_compress(wl)
    done = 0
    keys = {}
    limit = wl.T if max_queries is None else min(wl.T, max_queries)
    for t in range(limit):
        b = int(wl.seq[t])
        if b not in keys:
            nn = int(wl.visible()[wl.seq == b].max())
            keys = {b: O.index_keys_f64(wl.KI[b, :nn], None if wl.KS is None else wl.KS[b, :nn])}
        O.run_query(wl, t, keys[b], C_new)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return done / dt, done, dt, cores


def run_alternating(torch, ds, steps):
    """Plain launches back to back, each step on the next of `ds` (copies of one batch in
    separate memory) in turn, so no step finds the previous step's stores in cache.
    Returns seconds per step."""
    fns = [d.step_fns() for d in ds]
    for i in range(3 * len(ds)):
        for f in fns[i % len(ds)]:
            f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for f in fns[i % len(ds)]:
            f()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def config_leg(torch, name, steps, warmup, profile, cold=False, log=None):
    """One layer configuration: eager steps with stage events, then the faster of graph
    replays and plain back-to-back launches; with `cold`, a second copy of the batch's stores
    and plain launches alternating between the two copies."""
    import workloads as W
    from sparse_attention_score_amd.step import DeviceBatch
    t0 = time.perf_counter()
    wl = W.make(name)
    d = DeviceBatch(wl)
    torch.cuda.synchronize()
    if log:
        log(f"{name} inputs ready in {time.perf_counter() - t0:.1f}s")
    eager_s, ms = run_batch(torch, d, steps, warmup, 0.0 if profile else 0.5)
    best_s, timing = (eager_s, "eager launches with events around every stage") if profile else \
        best_step(torch, d, steps)
    ib, sb = indexer_bytes(wl), step_bytes(wl)
    out = {"workload": name, "queries": int(wl.T), "ms_per_step": best_s * 1e3,
           "queries_per_s": wl.T / best_s, "tokens_per_s": wl.T / best_s, "timing": timing,
           "eager_ms_per_step": eager_s * 1e3, "stage_ms": ms,
           "algorithmic_bytes_per_step": sb, "hbm_frac": sb / best_s / HBM_PEAK,
           "indexer": {"bound": "hbm", "achieved": ib / (ms["indexer"] * 1e-3) / 1e9,
                       "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                       "frac": ib / (ms["indexer"] * 1e-3) / HBM_PEAK,
                       "algorithmic_bytes_per_launch": ib, "avg_launch_ms": ms["indexer"],
                       "traffic": stored_traffic(name, CONFIG_TRAFFIC_FILES[name]) if name in CONFIG_TRAFFIC_FILES
                       else None}}
    if cold and not profile:
        d2 = DeviceBatch(wl)
        torch.cuda.synchronize()
        cold_s = run_alternating(torch, [d, d2], steps)
        out["cold"] = {"ms_per_step": cold_s * 1e3, "queries_per_s": wl.T / cold_s,
                       "hbm_frac": sb / cold_s / HBM_PEAK,
                       "timing": "plain launches back to back, alternating between two copies of the stores"}
        out["warm"] = {"ms_per_step": best_s * 1e3, "queries_per_s": wl.T / best_s,
                       "hbm_frac": sb / best_s / HBM_PEAK, "timing": timing}
        del d2
    del d, wl
    torch.cuda.empty_cache()
    return out


def compress_leg(torch, steps, profile, B=64, n_raw=32768):
    """The compressor alone (sparse_attn_compress, ratio 2) over B x n_raw raw latents and
    gate logits into B x n_raw/2 compressed rows, one launch over all groups; HIP events on
    the launch stream. Algorithmic bytes per group: two raw rows and two gate rows in,
    one row out (bf16)."""
    import sparse_attention_score_amd as S
    import workloads as W
    from sparse_attention_score_amd.step import to_device_bf16
    X, Z, beta = W.make_compress_input(B, n_raw)
    Xd, Zd = to_device_bf16(X), to_device_bf16(Z)
    del X, Z
    bd = torch.from_numpy(beta).cuda()
    G = B * (n_raw // 2)
    out = torch.empty((G, 512), dtype=torch.bfloat16, device="cuda")
    plan = S.Plan(ratio=2, key_dtype="bf16", max_queries=1, max_compressed=n_raw // 2)
    fn = lambda: S.sparse_attn_compress(plan, Xd, 1024, Zd, 1024, bd, out, 512, G)  # noqa: E731
    warm_up(torch, [fn], 3, 0.0 if profile else 0.3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = float(G * (2 * 2 * 512 * 2 + 512 * 2))
    del Xd, Zd, out
    torch.cuda.empty_cache()
    return {"what": f"sparse_attn_compress over {B} x {n_raw} raw latents ({G} groups, one launch)",
            "groups": G, "ms_per_launch": ms, "bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
            "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / HBM_PEAK,
            "algorithmic_bytes_per_launch": nbytes,
            "traffic": stored_traffic(f"compress raw {B} x {n_raw}", COMPRESS_TRAFFIC_FILE, COMPRESS_SOURCES)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode-b128-ctx128k-fp8")
    ap.add_argument("--prefill-workload", default="prefill-4096-at-61440")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-rescore", action="store_true")
    ap.add_argument("--mq-workload", default="decode-mq6-b128-ctx128k-fp8")
    ap.add_argument("--mq-mxfp4-workload", default="decode-mq6-b128-ctx128k-mxfp4")
    ap.add_argument("--no-multiquery", action="store_true")
    ap.add_argument("--mxfp4-workload", default="decode-b128-ctx128k-mxfp4")
    ap.add_argument("--no-mxfp4", action="store_true")
    ap.add_argument("--no-paged", action="store_true")
    ap.add_argument("--fp8kv-workload", default="decode-b128-ctx128k-fp8kv")
    ap.add_argument("--fp4kv-workload", default="decode-b128-ctx128k-fp4kv")
    ap.add_argument("--no-fp8kv", action="store_true", help="skip the e4m3 and MXFP4 latent-row batches")
    ap.add_argument("--ragged-workload", default="ragged-2x1024+64+16x6-ctx128k-fp8")
    ap.add_argument("--no-ragged", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other layer configurations")
    ap.add_argument("--no-compress", action="store_true")
    ap.add_argument("--only", default=None, help="comma-separated legs to run besides the headline batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--profile", action="store_true", help="timed steps only (for rocprofv3)")
    args = ap.parse_args()
    LEGS = ("paged", "rescore", "multiquery", "mxfp4", "fp8kv", "ragged", "prefill", "c1", "c2", "c5", "r1m",
            "compress", "cpu")
    if args.only is not None:
        keep = set(x for x in args.only.split(",") if x)
        unknown = keep - set(LEGS)
        if unknown:
            ap.error(f"unknown legs {sorted(unknown)}; known: {', '.join(LEGS)}")
        for leg in LEGS:
            if leg not in keep:
                setattr(args, {"multiquery": "no_multiquery", "cpu": "no_cpu_baseline", "c1": "skip_c1",
                               "c2": "skip_c2", "c5": "skip_c5", "r1m": "skip_r1m"}.get(leg, f"no_{leg}"), True)
    for leg in ("c1", "c2", "c5", "r1m"):
        if args.no_configs:
            setattr(args, f"skip_{leg}", True)
        elif not hasattr(args, f"skip_{leg}"):
            setattr(args, f"skip_{leg}", False)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(batch- or context-sharding is a design note only). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from sparse_attention_score_amd.step import DeviceBatch

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    t0 = time.perf_counter()
    wl = W.make(args.workload)
    log(f"generated {args.workload} in {time.perf_counter() - t0:.1f}s")
    d = DeviceBatch(wl)
    torch.cuda.synchronize()
    log("uploaded")
    eager_s, stage_ms = run_batch(torch, d, args.steps, args.warmup, 0.0 if args.profile else 0.5)
    log(f"decode eager: {eager_s * 1e3:.3f} ms/step, stages {stage_ms}")
    plain_s = graph_s = None
    if args.profile:
        sec_per_step, timing = eager_s, "eager launches with events around every stage"
    else:
        # the step as a serving loop would run it: plain launches back to back, or one HIP
        # graph replay per step; both are timed and the faster is the step time
        graph_s, graph_gpu_s = run_graph(torch, d, args.steps)
        log(f"decode graph replay: {graph_s * 1e3:.3f} ms/step (events {graph_gpu_s * 1e3:.3f})")
        plain_s = run_plain(torch, d, args.steps)
        log(f"decode eager, back to back: {plain_s * 1e3:.3f} ms/step")
        sec_per_step, timing = min((plain_s, "eager launches back to back"),
                                   (graph_s, "HIP graph replays of the whole step"))

    idx_bytes = indexer_bytes(wl)
    idx_s = stage_ms["indexer"] * 1e-3
    sbytes = step_bytes(wl)
    copy_bw = copy_bandwidth(torch)
    result = {
        "metric": "sparse-attn decode queries/s at 128K ctx",
        "value": wl.T / sec_per_step,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": int(wl.B), "queries": int(wl.T),
                   "raw_context": int(wl.pos.max()) + 1, "compressed": int(wl.visible().max()),
                   "ratio": int(wl.ratio), "index_keys": "fp8-e4m3" if wl.key_dtype == "fp8" else "bf16",
                   "heads": 64, "latent": 512, "window": 128, "topk": 512, "cand_blocks": 2048,
                   "block": 8, "index_heads": 16, "index_dim": 128},
        "roofline": {"kernel": "indexer_score (S1)", "bound": "hbm",
                     "achieved": idx_bytes / idx_s / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": idx_bytes / idx_s / HBM_PEAK, "traffic": stored_traffic(args.workload),
                     "algorithmic_bytes_per_launch": idx_bytes, "avg_launch_ms": stage_ms["indexer"],
                     "measured_copy_GBps": copy_bw / 1e9},
        "step": {"stage_ms": stage_ms, "eager_ms_per_step": eager_s * 1e3,
                 "plain_eager_ms_per_step": plain_s * 1e3 if plain_s else None,
                 "graph_ms_per_step": graph_s * 1e3 if graph_s else None,
                 "timing": timing,
                 "algorithmic_bytes": sbytes,
                 "hbm_frac": sbytes / sec_per_step / HBM_PEAK,
                 "tokens_per_s": wl.T / sec_per_step},
    }
    if not args.no_paged:
        p_graph, pms = run_paged(torch, d, args.steps, args.warmup, 64, args.profile)
        result["paged"] = {
            "what": "indexer, selection and attention of the same batch on 64-row pages in shuffled "
                    "order (block tables)",
            "ms_per_step": p_graph * 1e3 if p_graph else None, "stage_ms": pms,
            "indexer_frac": idx_bytes / (pms["indexer"] * 1e-3) / HBM_PEAK,
            "contiguous_stage_ms": {k: stage_ms[k] for k in ("indexer", "select", "attention")},
        }
        log(f"paged: {p_graph * 1e3 if p_graph else float('nan'):.3f} ms (no compressor), stages {pms}")
    if not args.no_rescore:
        carried, r_eager, r_graph, rms = run_rescore(torch, d, args.steps, args.warmup, args.profile)
        rb = rescore_bytes(wl, carried)
        r_s = r_graph or r_eager
        result["rescore"] = {
            "what": "layer that re-scores the 2048 candidate blocks carried from the two-stage "
                    "pass (indexer_score_cand, select_topk_cand, attention)",
            "ms_per_layer": r_s * 1e3, "queries_per_s": wl.T / r_s,
            "eager_ms_per_layer": r_eager * 1e3,
            "timing": "HIP graph replays" if r_graph else "eager launches",
            "stage_ms": rms,
            "indexer": {"bound": "hbm", "achieved": rb / (rms["indexer"] * 1e-3) / 1e9,
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": rb / (rms["indexer"] * 1e-3) / HBM_PEAK,
                        "algorithmic_bytes_per_launch": rb, "avg_launch_ms": rms["indexer"],
                        "traffic": stored_traffic(args.workload, RESCORE_TRAFFIC_FILE),
                        "key_bytes_per_query": rb / wl.T,
                        "full_scan_key_bytes_per_query": idx_bytes / wl.T},
        }
        log(f"rescore layer: {r_s * 1e3:.3f} ms, stages {rms}")
    del d
    torch.cuda.empty_cache()

    mq_legs = [] if args.no_multiquery else [("multi_query", args.mq_workload, GROUP_TRAFFIC_FILE),
                                              ("multi_query_mxfp4", args.mq_mxfp4_workload, None)]
    for mq_key, mq_name, mq_traffic in mq_legs:
        t0 = time.perf_counter()
        wm = W.make(mq_name)
        dm = DeviceBatch(wm)
        torch.cuda.synchronize()
        log(f"multi-token decode inputs ready in {time.perf_counter() - t0:.1f}s")
        m_eager, mms = run_batch(torch, dm, args.steps, args.warmup, 0.0 if args.profile else 0.5)
        m_s, m_timing = (m_eager, "eager launches") if args.profile else best_step(torch, dm, args.steps)
        gb = group_indexer_bytes(wm)
        fi, fa = step_flops(wm)
        mi_s = mms["indexer"] * 1e-3
        result[mq_key] = {
            "workload": mq_name, "queries": int(wm.T), "group": int(wm.group),
            "ms_per_step": m_s * 1e3, "queries_per_s": wm.T / m_s,
            "eager_ms_per_step": m_eager * 1e3,
            "timing": m_timing,
            "stage_ms": mms,
            "indexer": {"bound": "hbm", "achieved": gb / mi_s / 1e9, "peak": HBM_PEAK / 1e9,
                        "unit": "GB/s", "frac": gb / mi_s / HBM_PEAK,
                        "traffic": stored_traffic(mq_name, mq_traffic) if mq_traffic else None,
                        "algorithmic_bytes_per_launch": gb, "avg_launch_ms": mms["indexer"],
                        "key_bytes_per_query": gb / wm.T,
                        "mfma_tflop": fi / 1e12, "mfma_frac": fi / mi_s / BF16_PEAK},
        }
        log(f"{mq_key}: {m_s * 1e3:.3f} ms/step, stages {mms}")
        del dm, wm
        torch.cuda.empty_cache()

    if not args.no_mxfp4:
        t0 = time.perf_counter()
        wx = W.make(args.mxfp4_workload)
        dx = DeviceBatch(wx)
        torch.cuda.synchronize()
        log(f"MXFP4-key decode inputs ready in {time.perf_counter() - t0:.1f}s")
        x_eager, xms = run_batch(torch, dx, args.steps, args.warmup, 0.0 if args.profile else 0.5)
        x_s, x_timing = (x_eager, "eager launches") if args.profile else best_step(torch, dx, args.steps)
        xb = indexer_bytes(wx)
        xi_s = xms["indexer"] * 1e-3
        result["mxfp4_keys"] = {
            "workload": args.mxfp4_workload, "queries": int(wx.T),
            "ms_per_step": x_s * 1e3, "queries_per_s": wx.T / x_s,
            "eager_ms_per_step": x_eager * 1e3,
            "timing": x_timing,
            "stage_ms": xms,
            "indexer": {"bound": "hbm", "achieved": xb / xi_s / 1e9, "peak": HBM_PEAK / 1e9,
                        "unit": "GB/s", "frac": xb / xi_s / HBM_PEAK,
                        "traffic": stored_traffic(args.mxfp4_workload, MX_TRAFFIC_FILE),
                        "algorithmic_bytes_per_launch": xb, "avg_launch_ms": xms["indexer"]},
        }
        log(f"MXFP4-key decode: {x_s * 1e3:.3f} ms/step, stages {xms}")
        del dx, wx
        torch.cuda.empty_cache()

    kv_cases = [("fp8_kv", args.fp8kv_workload, "e4m3 latent and window rows"),
                ("mxfp4_kv", args.fp4kv_workload, "MXFP4 latent rows and e4m3 window rows")]
    for key, name, rows in kv_cases if not args.no_fp8kv and not args.profile else []:
        t0 = time.perf_counter()
        wk = W.make(name)
        dk = DeviceBatch(wk)
        torch.cuda.synchronize()
        log(f"{key} decode inputs ready in {time.perf_counter() - t0:.1f}s")
        k_eager, kms = run_batch(torch, dk, args.steps, args.warmup)
        k_s, k_timing = best_step(torch, dk, args.steps)
        result[key] = {
            "workload": name, "queries": int(wk.T),
            "what": f"the headline batch with {rows}; the compressor writes each new latent as codes and scales",
            "ms_per_step": k_s * 1e3, "queries_per_s": wk.T / k_s, "eager_ms_per_step": k_eager * 1e3,
            "timing": k_timing,
            "stage_ms": kms,
        }
        log(f"{key} decode: {k_s * 1e3:.3f} ms/step, stages {kms}")
        del dk, wk
        torch.cuda.empty_cache()

    if not args.no_ragged and not args.profile:
        import sparse_attention_score_amd as S
        t0 = time.perf_counter()
        wr = W.make(args.ragged_workload)
        dr = DeviceBatch(wr)
        torch.cuda.synchronize()
        log(f"ragged inputs ready in {time.perf_counter() - t0:.1f}s")
        r_eager, rms2 = run_batch(torch, dr, max(3, args.steps // 2), args.warmup)
        r_s, r_timing = best_step(torch, dr, max(3, args.steps // 2))
        flat = S.Queries(dr.seq, dr.pos, dr.max_visible)   # the same batch as independent queries
        flat_idx = lambda: S.indexer_score(dr.plan, flat, dr.cache, dr.qI, dr.w, dr.scores, dr.block_max)
        warm_up(torch, [flat_idx], 2, 0.2)
        ft = Timer(torch, ["indexer"])
        for _ in range(max(3, args.steps // 4)):
            ft.step([flat_idx])
        torch.cuda.synchronize()
        result["ragged"] = {
            "workload": args.ragged_workload, "queries": int(wr.T), "runs": len(wr.runs),
            "ms_per_step": r_s * 1e3, "queries_per_s": wr.T / r_s, "eager_ms_per_step": r_eager * 1e3,
            "timing": r_timing,
            "stage_ms": rms2,
            "indexer_ms_as_independent_queries": ft.mean_ms()["indexer"],
        }
        log(f"ragged: {r_s * 1e3:.3f} ms/step, stages {rms2}, indexer without runs {ft.mean_ms()['indexer']:.3f} ms")
        del dr, wr
        torch.cuda.empty_cache()

    if not args.no_prefill:
        t0 = time.perf_counter()
        wp = W.make(args.prefill_workload)
        dp = DeviceBatch(wp)
        torch.cuda.synchronize()
        log(f"prefill inputs ready in {time.perf_counter() - t0:.1f}s")
        sp_eager, sms = run_batch(torch, dp, max(3, args.steps // 2), args.warmup, 0.0 if args.profile else 0.5)
        sp, p_timing = (sp_eager, "eager launches with events around every stage") if args.profile else \
            best_step(torch, dp, max(3, args.steps // 2))
        fi, fa = step_flops(wp)
        result["prefill"] = {
            "workload": args.prefill_workload, "ms_per_chunk": sp * 1e3, "tokens_per_s": wp.T / sp,
            "eager_ms_per_chunk": sp_eager * 1e3, "timing": p_timing,
            "stage_ms": sms, "algorithmic_tflop": (fi + fa) / 1e12,
            "mfma_frac": (fi + fa) / sp / BF16_PEAK,
            "indexer_mfma_frac": fi / (sms["indexer"] * 1e-3) / BF16_PEAK,
            "attention_mfma_frac": fa / (sms["attention"] * 1e-3) / BF16_PEAK,
        }
        log(f"prefill: {sp * 1e3:.3f} ms/chunk, stages {sms}")
        del dp, wp
        torch.cuda.empty_cache()

    for key, name, cold, skip in (("c1_latency", "decode-b4-ctx2k", False, args.skip_c1),
                                  ("c2", "decode-b64-ctx32k", True, args.skip_c2),
                                  ("c5", "decode-b8-ctx1m-fp8", False, args.skip_c5),
                                  ("long_r1", "decode-b2-ctx1m-r1-fp8", False, args.skip_r1m)):
        if skip:
            continue
        result[key] = config_leg(torch, name, args.steps, args.warmup, args.profile, cold=cold, log=log)
        log(f"{key}: {result[key]['ms_per_step']:.4f} ms/step, stages {result[key]['stage_ms']}"
            + (f", cold {result[key]['cold']['ms_per_step']:.4f} ms" if "cold" in result[key] else ""))

    if not args.no_compress:
        result["compress"] = compress_leg(torch, args.steps, args.profile)
        log(f"compress: {result['compress']['ms_per_launch']:.4f} ms/launch, "
            f"{result['compress']['achieved']:.0f} GB/s")

    if not args.no_cpu_baseline and not args.profile:
        qps, done, dt, cores = cpu_baseline(wl, args.cpu_budget)
        result["cpu_baseline"] = {
            "value": qps, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"first {done} of the {wl.T} queries of {args.workload}, whole path "
                      f"(compressor, indexer, selection, attention) in fp64, {dt:.1f}s"}
        log(f"cpu oracle: {done} queries in {dt:.1f}s on {cores} BLAS threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Decode-step benchmark of the paged-KV library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

One step is the whole hot path over one batch: the scatter of the step's new
tokens (one per sequence, at position L - 1) into their slots, then paged
decode attention of every sequence over its paged K/V.  The headline runs the
step as one launch (pa_decode_step); the same step as two calls
(pa_reshape_and_cache, then pa_paged_attention) is timed beside it.  The default workload is the Llama-3-8B-shaped
decode batch: 64 sequences, 32 query heads / 8 KV heads, head size 128,
block size 16, context lengths uniform in [128, 2048], bfloat16.

Inputs are resident in HBM before timing starts; the pools are written by the
library's own reshape_and_cache.  To keep the 256 MB Infinity Cache from
serving repeated steps, the step rotates over ``--replicas`` copies of the
K/V pools (cold headline); ``--warm`` adds a run over one copy.

Prints ONE JSON line with the step throughput (KV bytes read per second), the
step launch's roofline (HIP events around the timed steps on the stream the
launches go to), and the CPU oracle's throughput on a bounded sample of the same workload
(reported baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV GB/s (% of HBM peak) + µs/step, Llama-3-8B shape, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_425_amd", "csrc", "paged_attention.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--op", default="step",
                    choices=["step", "copy_blocks", "prefill", "fp8", "swap", "ceiling",
                             "math", "balance", "coexec", "writes", "suffixes"],
                    help="step: the decode step (default); copy_blocks: the copy-on-write "
                         "copies of the parallel-sampling workload; prefill: paged prefill; "
                         "fp8: the decode step over FP8 (E4M3) K/V pools; swap: swapping a "
                         "quarter of the sequences' blocks out to pinned host memory and back; "
                         "ceiling: the read-bandwidth probe over the workload's KV bytes, "
                         "streaming and as a gather of scattered 4 KB tiles, every launch "
                         "shape of the sweep; math: the fused step of the Llama-3-8B "
                         "batch with its two products on the matrix cores and on the vector "
                         "ALU, at group sizes 1, 2 and 4 over the same KV; balance: the "
                         "fused step of the Llama-3-8B batch against batches of the same "
                         "bytes whose pairs are exactly balanced or whose lengths are equal; "
                         "coexec: the MFMA / VALU co-execution probe; writes: the decode of "
                         "the continuous-batching mix after a scatter of N of its new tokens, "
                         "against the two apart (what dirty cache lines cost the reads); "
                         "suffixes: the prefix-sharing step against the fused step of its "
                         "private suffixes alone (a floor for any way of adding the prefix)")
    ap.add_argument("--prefill-case", default="prefix-cache-prefill",
                    choices=["prefix-cache-prefill", "chunked-prefill-llama3-8b"])
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--block-size", type=int, default=None, help="block size of config 2")
    ap.add_argument("--variant", default=None, help="config 3: prefix | parallel-sampling")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None,
                    help="tokens per partition (0 = library default)")
    ap.add_argument("--replicas", type=int, default=4,
                    help="copies of the K/V pools the steps rotate over")
    ap.add_argument("--order", choices=["host", "device"], default="host",
                    help="order of the sequences for the paired decode: sorted on the host "
                         "from a host copy of the lengths (host_context_lens), or ranked "
                         "inside every workgroup; the other order is timed beside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--plain-step", action="store_true",
                    help="with a shared prefix: time only pa_decode_step (the headline is "
                         "otherwise pa_decode_step_shared_prefix)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the read-probe sweep beside the step (e.g. under a profiler)")
    ap.add_argument("--warm", action="store_true",
                    help="also time K steps over one pool copy (Infinity Cache warm)")
    ap.add_argument("--math", choices=["both", "mfma", "valu"], default="both",
                    help="--op math: the forms to time (one form alone under a profiler)")
    ap.add_argument("--groups", default="1,2,4",
                    help="--op math: query heads per kv head to time")
    ap.add_argument("--rounds", type=int, default=3,
                    help="--op math: alternating rounds of the forms")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work in the CPU baseline")
    return ap.parse_args()


# ---------------------------------------------------------------------------
def algorithmic_bytes(w) -> dict:
    """Bytes one decode step must move at the least.

    kv: every context position's K and V row of its KV head, read once;
    other: the query (read), the output (written), the block-table entries of
    the blocks in use and the context lengths.
    """
    elt = 2 if w.dtype == "bf16" else 4
    lens = w.context_lens.astype(np.int64)
    kv = int(lens.sum()) * 2 * w.num_kv_heads * w.head_dim * elt
    q = w.num_seqs * w.num_heads * w.head_dim * elt
    table = int((-(-lens // w.block_size)).sum()) * 4
    return {"kv": kv, "other": 2 * q + table + 4 * w.num_seqs, "total": kv + 2 * q + table + 4 * w.num_seqs}


def unique_kv_bytes(w) -> int:
    """K+V bytes of the distinct slots the step reads: shared blocks (a common prefix, parallel
    samples) count once, as HBM must deliver them at least once."""
    elt = 2 if w.dtype == "bf16" else 4
    slots = set()
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        nb = -(-L // w.block_size)
        blocks = w.block_table[s, :nb].astype(np.int64)
        pos = np.arange(L)
        slots.update((blocks[pos // w.block_size] * w.block_size + pos % w.block_size).tolist())
    return len(slots) * 2 * w.num_kv_heads * w.head_dim * elt


# ---------------------------------------------------------------------------
# the read ceiling: pa_read_probe over the same number of bytes as the step's KV
# ---------------------------------------------------------------------------
CEILING_SHAPES = [(wg, u) for wg in (256, 512, 1024, 2048) for u in (4, 8, 16)]


def measure_ceiling(kv_bytes: int, steps: int, warmup: int, replicas: int = 4,
                    piece_bytes: int = 4096, shapes=CEILING_SHAPES, seed: int = 0) -> dict:
    """Best rate of the read probe over kv_bytes (rounded down to whole pieces), rotating
    over `replicas` windows of a buffer so that the Infinity Cache cannot serve repeats,
    as a streaming read (pieces in order) and as a gather of randomly placed pieces (the
    paged pattern), for every launch shape in `shapes`.  Rates in GB/s from HIP events."""
    import torch

    import paged_kv_cache_425_amd as pk
    dev = torch.device("cuda:0")
    n = max(1, kv_bytes // piece_bytes)
    window = n * piece_bytes
    buf = torch.empty(replicas * window, dtype=torch.uint8, device=dev)
    buf.random_(0, 256)
    rng = np.random.default_rng(seed)
    offs = {"stream": [], "gather": []}
    for r in range(replicas):
        base = r * window
        offs["stream"].append(torch.from_numpy(base + np.arange(n, dtype=np.int64) * piece_bytes)
                              .to(dev))
        offs["gather"].append(torch.from_numpy(base + rng.permutation(n).astype(np.int64) *
                                               piece_bytes).to(dev))
    for lst in offs.values():                        # every piece inside the buffer
        assert all(int(o.max()) + piece_bytes <= buf.numel() for o in lst)
    sink = torch.empty(max(wg for wg, _ in shapes) * 256, dtype=torch.int32, device=dev)
    table = []
    best = {}              # per pattern, over both load policies
    best_default = {}      # per pattern, default-policy loads only
    for pattern in ("stream", "gather"):
        for nt in (False, True):
            for wg, u in shapes:
                def run(k):
                    for i in range(k):
                        pk.read_probe(buf, offs[pattern][i % replicas], piece_bytes, wg, u, sink,
                                      nontemporal=nt)
                run(warmup)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                run(steps)
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / steps
                gbs = window / (us * 1e-6) / 1e9
                row = {"pattern": pattern, "loads": "nt" if nt else "default", "workgroups": wg,
                       "in_flight": u, "us": round(us, 2), "GB/s": round(gbs, 1)}
                table.append(row)
                if gbs > best.get(pattern, {}).get("GB/s", 0):
                    best[pattern] = {k: row[k] for k in ("GB/s", "us", "workgroups", "in_flight",
                                                         "loads")}
                if not nt and gbs > best_default.get(pattern, {}).get("GB/s", 0):
                    best_default[pattern] = {k: row[k] for k in ("GB/s", "us", "workgroups",
                                                                 "in_flight")}
    del buf
    return {"bytes": window, "piece_bytes": piece_bytes, "replicas": replicas,
            "stream": best["stream"], "gather": best["gather"], "default_loads": best_default,
            "sweep": table}


def bench_ceiling(args) -> int:
    """The read probe's sweep over the workload's KV bytes (one JSON line)."""
    from workloads import make_config
    w = make_config(args.config, seed=args.seed, block_size=args.block_size, variant=args.variant)
    kv = algorithmic_bytes(w)["kv"]
    log(f"read ceiling over {kv / 1e6:.1f} MB ({w.name})")
    c = measure_ceiling(kv, args.steps, args.warmup, replicas=max(1, args.replicas))
    line = {"metric": "read-probe GB/s over the decode step's KV bytes", "value": c["gather"]["GB/s"],
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": "u8", "data": "synthetic (random bytes)",
            "config": {"workload": w.name, "bytes_per_launch": c["bytes"],
                       "piece_bytes": c["piece_bytes"], "replicas": c["replicas"]},
            "stream": c["stream"], "gather": c["gather"], "default_loads": c["default_loads"],
            "hbm_frac_stream": round(c["stream"]["GB/s"] / HBM_PEAK_GBS, 4),
            "hbm_frac_gather": round(c["gather"]["GB/s"] / HBM_PEAK_GBS, 4),
            "sweep": c["sweep"]}
    print(json.dumps(line), flush=True)
    return 0


def pool_utilisation(w) -> dict:
    """Share of the KV memory holding live tokens: paged (the blocks the batch holds; only
    the tail of each sequence's last block is empty) and, for contrast, one contiguous
    region per sequence sized for the batch's longest context."""
    lens = w.context_lens.astype(np.int64)
    used = set()
    for s in range(w.num_seqs):
        used.update(w.block_table[s, :-(-int(lens[s]) // w.block_size)].tolist())
    stored = unique_kv_bytes(w) // (2 * w.num_kv_heads * w.head_dim *
                                    (2 if w.dtype == "bf16" else 4))
    return {"paged": round(stored / (len(used) * w.block_size), 4),
            "contiguous_at_max_len": round(int(lens.sum()) / (w.num_seqs * int(lens.max())), 4),
            "blocks_held": len(used), "tokens_stored": int(stored),
            "pages_claim": ("20-30% before paging, above 95% with it, on A100 ('architecture & "
                            "core features' section 3.1; 'core inference engine' section 2.2)")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def source_digest() -> str:
    from paged_kv_cache_425_amd.rocprof_summary import kernel_source_digest
    return kernel_source_digest(KERNEL_SOURCE)


def load_traffic(workload: str):
    """Measured HBM bytes per decode launch (profiles/traffic_<workload>.json, from the
    calibrated FETCH_SIZE / WRITE_SIZE counters), if they were taken on the current kernel."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
def blas_thread_count() -> int:
    """Threads of the BLAS pool the oracle's matmuls run on."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, budget_s: float) -> dict:
    """The CPU oracle on a bounded sample of the same step (reported baseline)."""
    import oracle
    blas_threads = blas_thread_count()
    hist, new = w.history_records, w.new_records
    kc, vc = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
    oracle.reshape_and_cache(w.rec_key[hist], w.rec_value[hist], w.rec_slot[hist], kc, vc,
                             inplace=True)
    elt = 2 if w.dtype == "bf16" else 4
    per_token = 2 * w.num_kv_heads * w.head_dim * elt
    steps, done, kv = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        # one whole step: the scatter of the new tokens, then every sequence's decode
        oracle.reshape_and_cache(w.rec_key[new], w.rec_value[new], w.rec_slot[new], kc, vc,
                                 inplace=True)
        for s in range(w.num_seqs):
            oracle.paged_attention(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                   w.dtype, seqs=[s])
            done += 1
            kv += int(w.context_lens[s]) * per_token
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            steps += 1
            if time.perf_counter() - t0 < budget_s:
                continue
        break
    dt = time.perf_counter() - t0
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle, same workload: {steps} whole steps (scatter of "
                       f"{len(new)} new tokens + decode of all {w.num_seqs} sequences) plus "
                       f"{done - steps * w.num_seqs} sequences of a partial step, "
                       f"{kv / 1e6:.1f} MB of KV in {dt:.1f} s; {cpu_model()}, "
                       f"{len(os.sched_getaffinity(0))} of {os.cpu_count()} cores visible, "
                       f"BLAS pool {blas_threads} threads")}


# ---------------------------------------------------------------------------
def bench_copy_blocks(args) -> int:
    """Copy-on-write block copies of the parallel-sampling layout (32 prompts x 4 samples)."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config

    dev = torch.device("cuda:0")
    w = make_config(3, seed=args.seed, variant="parallel-sampling")
    tdt = torch.bfloat16
    pairs = w.cow_pairs
    log(f"workload {w.name}: {len(pairs)} block copies, NB={w.num_blocks}")
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)  # noqa: E731
    keep = np.setdiff1d(np.setdiff1d(np.arange(len(w.rec_slot)), w.new_records), w.cow_records)
    kshape = pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    vshape = pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    kc0 = torch.full(kshape, float("nan"), dtype=tdt, device=dev)
    vc0 = torch.full(vshape, float("nan"), dtype=tdt, device=dev)
    pk.reshape_and_cache(up(w.rec_key[keep]), up(w.rec_value[keep]),
                         torch.from_numpy(w.rec_slot[keep]).to(dev), kc0, vc0)
    # enough pool copies that a rotation spans well past the 256 MB Infinity Cache
    pool_bytes = 2 * kc0.numel() * kc0.element_size()
    R = max(args.replicas, int(np.ceil(1.2e9 / pool_bytes)))
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
    pt = torch.from_numpy(pairs).to(dev)
    calls = [pk.prepare_copy_blocks(kc, vc, pt) for kc, vc in pools]
    elt = 2
    moved = 2 * len(pairs) * 2 * w.num_kv_heads * w.head_dim * w.block_size * elt  # read + write
    K, W = args.steps, args.warmup
    for i in range(W):
        calls[i % R]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        calls[i % R]()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = e0.elapsed_time(e1) * 1e-3
    value = moved / (wall / K) / 1e9
    achieved = moved / (ev / K) / 1e9
    log(f"copy_blocks: {wall / K * 1e6:.2f} us/call wall, {ev / K * 1e6:.2f} us/call events")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        kh = kc0.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vc0.view(torch.int16).cpu().numpy().view(np.uint16)
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_budget, 5.0):
            oracle.copy_blocks(kh, vh, pairs, inplace=True)
            n += 1
        dt = time.perf_counter() - t1
        cpu = {"value": round(n * moved / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"NumPy oracle copy_blocks of the same {len(pairs)} pairs, {n} calls "
                         f"in {dt:.1f} s (one thread)"}
    print(json.dumps({
        "metric": "copy-on-write copy_blocks GB/s moved (read + write), 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "pairs": int(len(pairs)), "bytes_moved_per_call": moved,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "pool_replicas": R},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": moved},
        "cpu_baseline": cpu}), flush=True)
    return 0


def bench_prefill(args) -> int:
    """Paged prefill of a named batch (default: prefix-cache prefill of the prefix-sharing
    batch's private suffixes over the cached 1024-token prefix)."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_prefill_config

    dev = torch.device("cuda:0")
    w, pb = make_prefill_config(args.prefill_case, seed=args.seed)
    tdt = torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)  # noqa: E731
    kshape = pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    vshape = pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    kc = torch.full(kshape, float("nan"), dtype=tdt, device=dev)
    vc = torch.full(vshape, float("nan"), dtype=tdt, device=dev)
    pk.reshape_and_cache(up(w.rec_key), up(w.rec_value), torch.from_numpy(w.rec_slot).to(dev),
                         kc, vc)
    query = up(pb.query)
    qsl = torch.from_numpy(pb.query_start_loc).to(dev)
    table = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    out = torch.empty_like(query)
    torch.cuda.synchronize()
    n = np.diff(pb.query_start_loc).astype(np.int64)
    L = w.context_lens.astype(np.int64)
    keys = int(sum(int(((L[s] - n[s] + 1) + L[s]) * n[s] // 2) for s in range(w.num_seqs)))
    flops = 4 * w.num_heads * w.head_dim * keys              # Q.K^T and P.V, 2 flops per MAC
    bytes_q = 2 * query.numel() * 2                          # query read, output written
    log(f"prefill {args.prefill_case}: S={w.num_seqs} T={query.shape[0]} "
        f"attention pairs={keys * w.num_heads / 1e6:.0f} M, {flops / 1e12:.3f} TFLOP")

    def call():
        pk.paged_prefill(query, qsl, table, lens, kc, vc, w.scale,
                         max_query_len=pb.max_query_len, out=out)

    K, W = max(1, args.steps // 10), max(1, args.warmup // 10)
    for _ in range(W):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        call()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = e0.elapsed_time(e1) * 1e-3
    tflops = flops / (ev / K) / 1e12
    log(f"prefill: {wall / K * 1e6:.1f} us/call wall, {ev / K * 1e6:.1f} us/call events, "
        f"{tflops:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        kh = kc.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vc.view(torch.int16).cpu().numpy().view(np.uint16)
        done, kdone, t1 = 0, 0, time.perf_counter()
        for s in range(w.num_seqs):
            oracle.paged_prefill(pb.query, pb.query_start_loc, w.block_table, w.context_lens,
                                 kh, vh, w.scale, w.dtype, seqs=[s])
            done += 1
            kdone += int(((L[s] - n[s] + 1) + L[s]) * n[s] // 2)
            if time.perf_counter() - t1 >= args.cpu_budget:
                break
        dt = time.perf_counter() - t1
        cpu = {"value": round(4 * w.num_heads * w.head_dim * kdone / dt / 1e12, 6),
               "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
               "sample": f"float64 NumPy oracle prefill of the first {done} of {w.num_seqs} "
                         f"sequences in {dt:.1f} s"}
    print(json.dumps({
        "metric": "paged prefill TFLOP/s (causal, bf16), 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.prefill_case, "num_seqs": w.num_seqs,
                   "query_tokens": int(query.shape[0]), "max_chunk": pb.max_query_len,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "attention_pairs": keys * w.num_heads},
        "roofline": {"kernel": "paged_prefill_kernel", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops,
                     "query_and_output_bytes": bytes_q},
        "cpu_baseline": cpu}), flush=True)
    return 0


FP8_K_SCALE = 0.0135           # about 6 / 448 for N(0, 1) records
FP8_V_SCALE = 0.0121


def cpu_baseline_fp8(w, budget_s: float, n_seqs: int = 8) -> dict:
    """The oracle's FP8 step on the first n_seqs sequences (their history quantised first,
    outside the timed budget): scatter of their new tokens, then their decode."""
    import oracle
    seqs = list(range(min(n_seqs, w.num_seqs)))
    new = np.array([w.seq_records[s][-1] for s in seqs], dtype=np.int64)
    hist = np.concatenate([w.seq_records[s][:-1] for s in seqs])
    kc, vc = oracle.empty_fp8_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)
    oracle.reshape_and_cache_fp8(w.rec_key[hist], w.rec_value[hist], w.rec_slot[hist], kc, vc,
                                 w.dtype, FP8_K_SCALE, FP8_V_SCALE, inplace=True)
    per_token = 2 * w.num_kv_heads * w.head_dim
    rounds, kv = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.reshape_and_cache_fp8(w.rec_key[new], w.rec_value[new], w.rec_slot[new], kc, vc,
                                     w.dtype, FP8_K_SCALE, FP8_V_SCALE, inplace=True)
        oracle.paged_attention_fp8(w.query, w.block_table, w.context_lens, kc, vc, w.scale,
                                   FP8_K_SCALE, FP8_V_SCALE, w.dtype, seqs=seqs)
        kv += int(w.context_lens[seqs].astype(np.int64).sum()) * per_token
        rounds += 1
    dt = time.perf_counter() - t0
    threads = blas_thread_count()
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"float64 NumPy oracle, FP8 step of the first {len(seqs)} sequences "
                       f"(quantised scatter of their new tokens + their decode) repeated "
                       f"{rounds} times, {kv / 1e6:.1f} MB of FP8 KV in {dt:.1f} s; "
                       f"{len(os.sched_getaffinity(0))} cores visible, BLAS pool {threads} "
                       "threads")}


def bench_fp8(args) -> int:
    """The decode step over FP8 pools on the Llama-3-8B-shaped batch: pa_decode_step_fp8
    (one launch) as the headline, and the same step as pa_reshape_and_cache_fp8 followed by
    pa_paged_attention_fp8 beside it."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config
    dev = torch.device("cuda:0")
    w = make_config(args.config, seed=args.seed, block_size=args.block_size, variant=args.variant)
    if w.dtype != "bf16":
        print("the FP8 step needs a bf16 workload", file=sys.stderr)
        return 2
    log(f"workload {w.name} (FP8 K/V): S={w.num_seqs} Hq={w.num_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} BS={w.block_size} NB={w.num_blocks} max_len={w.max_context_len}")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    hist = np.setdiff1d(np.arange(len(w.rec_slot)), new)
    kshape = pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size)
    vshape = pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, torch.uint8)
    kc0 = torch.full(kshape, 0x7F, dtype=torch.uint8, device=dev)     # NaN codes
    vc0 = torch.full(vshape, 0x7F, dtype=torch.uint8, device=dev)
    pk.reshape_and_cache_fp8(up(w.rec_key[hist]), up(w.rec_value[hist]),
                             torch.from_numpy(w.rec_slot[hist]).to(dev), kc0, vc0,
                             FP8_K_SCALE, FP8_V_SCALE)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(max(1, args.replicas) - 1)]
    key_new, val_new = up(w.rec_key[new]), up(w.rec_value[new])
    slot_new = torch.from_numpy(w.rec_slot[new]).to(dev)
    query = up(w.query)
    table = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    out = torch.empty_like(query)
    part = args.partition_size if args.partition_size is not None else (w.partition_size or 0)
    need = pk.workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                             w.max_context_len, part, torch.bfloat16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    host_lens = w.context_lens.copy()

    def prep_fused(order):
        hl = host_lens if order == "host" else None
        return [pk.prepare_decode_step_fp8(query, key_new, val_new, slot_new, table, lens, kc,
                                           vc, w.scale, FP8_K_SCALE, FP8_V_SCALE,
                                           max_context_len=w.max_context_len, out=out,
                                           partition_size=part, workspace=ws,
                                           host_context_lens=hl) for kc, vc in pools]
    other_order = "device" if args.order == "host" else "host"
    fused, fused_other = prep_fused(args.order), prep_fused(other_order)
    writes = [pk.prepare_reshape_and_cache_fp8(key_new, val_new, slot_new, kc, vc, FP8_K_SCALE,
                                               FP8_V_SCALE) for kc, vc in pools]
    decodes = [pk.prepare_paged_attention_fp8(query, table, lens, kc, vc, w.scale, FP8_K_SCALE,
                                              FP8_V_SCALE, max_context_len=w.max_context_len,
                                              out=out, partition_size=part, workspace=ws,
                                              host_context_lens=host_lens
                                              if args.order == "host" else None)
               for kc, vc in pools]
    R, K, W = len(pools), args.steps, args.warmup

    def run_fused(steps: int, calls=None) -> None:
        calls = fused if calls is None else calls
        for i in range(steps):
            calls[i % R]()

    def run_two_calls(steps: int) -> None:
        for i in range(steps):
            writes[i % R]()
            decodes[i % R]()

    def timed(fn, steps, *a):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        fn(steps, *a)
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3

    run_fused(W)
    wall, ev = timed(run_fused, K)
    log(f"FP8 fused step: {wall / K * 1e6:.1f} us/step wall, {ev / K * 1e6:.1f} us/launch "
        "(events)")
    run_two_calls(W)
    wall2, ev2 = timed(run_two_calls, K)
    log(f"FP8 two-call step: {wall2 / K * 1e6:.1f} us/step wall")
    run_fused(W, fused_other)
    wall3, ev3 = timed(run_fused, K, fused_other)
    log(f"FP8 fused step, {other_order} order: {wall3 / K * 1e6:.1f} us/step wall")

    lens64 = w.context_lens.astype(np.int64)
    kv = int(lens64.sum()) * 2 * w.num_kv_heads * w.head_dim            # 1 byte per element
    q = w.num_seqs * w.num_heads * w.head_dim * 2
    table_b = int((-(-lens64 // w.block_size)).sum()) * 4
    new_in = w.num_seqs * 2 * w.num_kv_heads * w.head_dim * 2            # bf16 new K and V
    new_out = w.num_seqs * 2 * w.num_kv_heads * w.head_dim               # their codes
    fused_bytes = kv + 2 * q + table_b + 4 * w.num_seqs + new_in + new_out + 8 * w.num_seqs
    ms_step = wall / K * 1e3
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = fused_bytes / (ev / K) / 1e9
    part_used = part or pk.default_partition_size(w.num_seqs, w.num_kv_heads, w.max_context_len,
                                                  torch.bfloat16)
    line = {
        "metric": "paged-attn decode over FP8 (E4M3) K/V: KV GB/s + µs/step, "
                  "Llama-3-8B shape, 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 K/V, bf16 query/out, f32 accumulation",
        "data": "synthetic (seeded N(0,1) q/K/V, random block tables)",
        "config": {"workload": w.name + "-fp8", "num_seqs": w.num_seqs,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "max_context_len": w.max_context_len, "partition_size": part_used,
                   "k_scale": FP8_K_SCALE, "v_scale": FP8_V_SCALE, "kv_bytes_per_step": kv,
                   "step": "pa_decode_step_fp8: quantised scatter of the new tokens + paged "
                           "decode, one launch",
                   "order": args.order,
                   "pool_bytes_each": int(kc0.numel()), "pool_replicas": R,
                   "parallelism": "none (1 GPU)"},
        "launch_us_events": round(ev / K * 1e6, 2),
        "two_call_step": {"us_per_step": round(wall2 / K * 1e6, 2),
                          "us_per_step_events": round(ev2 / K * 1e6, 2),
                          "value": round(kv / (wall2 / K) / 1e9, 2)},
        f"{other_order}_order_step": {"us_per_step": round(wall3 / K * 1e6, 2),
                                      "launch_us_events": round(ev3 / K * 1e6, 2),
                                      "value": round(kv / (wall3 / K) / 1e9, 2)},
        "roofline": {"kernel": "pa_decode_step_fp8: paged_decode_kernel<bf16, e4m3>",
                     "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(w.name + "-fp8"),
                     "algorithmic_bytes_per_launch": fused_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, FP8) ...")
        line["cpu_baseline"] = cpu_baseline_fp8(w, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


PCIE_PEAK_GBS = 64.0           # PCIe 5.0 x16 per direction, the MI355X host link


def bench_swap(args) -> int:
    """Swap-out of a quarter of the Llama-3-8B-shaped batch's sequences (all their blocks,
    K and V) from the HBM pools to pinned host pools, and swap-in back into HBM, each one
    pa_swap_blocks launch; a plain contiguous device-to-host / host-to-device copy of the
    same bytes (copy engine) is timed beside it as the practical ceiling of the link."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config
    dev = torch.device("cuda:0")
    w = make_config(args.config, seed=args.seed, block_size=args.block_size, variant=args.variant)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kshape = pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    vshape = pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    kd = torch.randn(kshape, dtype=torch.float32, device=dev).to(tdt)
    vd = torch.randn(vshape, dtype=torch.float32, device=dev).to(tdt)
    rng = np.random.default_rng(7)
    victims = np.sort(rng.choice(w.num_seqs, max(1, w.num_seqs // 4), replace=False))
    blocks = np.concatenate([w.block_table[s, :-(-int(w.context_lens[s]) // w.block_size)]
                             for s in victims]).astype(np.int64)
    nh = len(blocks)
    out_map = torch.from_numpy(np.stack([blocks, np.arange(nh)], axis=1)).to(dev)
    in_map = torch.from_numpy(np.stack([np.arange(nh), blocks], axis=1)).to(dev)
    hk = torch.empty((nh,) + tuple(kshape[1:]), dtype=tdt, pin_memory=True)
    hv = torch.empty((nh,) + tuple(vshape[1:]), dtype=tdt, pin_memory=True)
    elt = 2 if w.dtype == "bf16" else 4
    moved = 2 * nh * w.num_kv_heads * w.head_dim * w.block_size * elt      # K and V
    log(f"swap: {len(victims)} of {w.num_seqs} sequences, {nh} blocks, {moved / 1e6:.1f} MB "
        "each way")
    swap_out = pk.prepare_swap_blocks(kd, vd, hk, hv, out_map)
    swap_in = pk.prepare_swap_blocks(hk, hv, kd, vd, in_map)
    torch.cuda.synchronize()
    # the same bytes as one contiguous copy each way (the copy engine's ceiling)
    flat_d = torch.empty(moved // 2, dtype=torch.int16, device=dev)
    flat_h = torch.empty(moved // 2, dtype=torch.int16, pin_memory=True)
    K, W = max(1, args.steps // 10), max(1, args.warmup // 10)

    def timed(fn):
        for _ in range(W):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K, e0.elapsed_time(e1) * 1e-3 / K

    out_wall, out_ev = timed(swap_out)
    in_wall, in_ev = timed(swap_in)
    d2h_wall, d2h_ev = timed(lambda: flat_h.copy_(flat_d, non_blocking=True))
    h2d_wall, h2d_ev = timed(lambda: flat_d.copy_(flat_h, non_blocking=True))
    gbs = lambda t: moved / t / 1e9
    log(f"swap-out {out_ev * 1e6:.0f} us = {gbs(out_ev):.1f} GB/s; swap-in {in_ev * 1e6:.0f} us "
        f"= {gbs(in_ev):.1f} GB/s; contiguous copies {gbs(d2h_ev):.1f} / {gbs(h2d_ev):.1f} GB/s")
    # one pass of the path: the blocks out and back in
    step_s = out_ev + in_ev
    line = {
        "metric": "swap_blocks HBM <-> pinned host, GB/s per direction (PCIe), "
                  "Llama-3-8B shape, 1 GPU",
        "value": round(2 * moved / step_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (random pools; the block lists of a seeded quarter of the batch)",
        "config": {"workload": w.name + "-swap", "sequences_swapped": int(len(victims)),
                   "blocks": int(nh), "bytes_each_way": int(moved),
                   "step": "pa_swap_blocks out (HBM -> pinned host) + pa_swap_blocks in",
                   "parallelism": "none (1 GPU)"},
        "swap_out": {"us": round(out_ev * 1e6, 1), "GB/s": round(gbs(out_ev), 2),
                     "us_wall": round(out_wall * 1e6, 1)},
        "swap_in": {"us": round(in_ev * 1e6, 1), "GB/s": round(gbs(in_ev), 2),
                    "us_wall": round(in_wall * 1e6, 1)},
        "contiguous_copy_engine": {"d2h_GB/s": round(gbs(d2h_ev), 2),
                                   "h2d_GB/s": round(gbs(h2d_ev), 2)},
        "roofline": {"kernel": "swap_blocks_kernel (swap-out)", "bound": "pcie",
                     "achieved": round(gbs(out_ev), 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs(out_ev) / PCIE_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": int(moved)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline_swap(w, blocks, min(args.cpu_budget, 5.0))
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_swap(w, blocks: np.ndarray, budget_s: float) -> dict:
    """The oracle's whole-block copies of the same blocks between two host pools (out and
    back in), repeated for about budget_s (reported baseline)."""
    import oracle
    kc, vc = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype,
                                fill="zero")
    nh = len(blocks)
    hk, hv = oracle.empty_pools(nh, w.num_kv_heads, w.head_dim, w.block_size, w.dtype,
                                fill="zero")
    out_map = np.stack([blocks, np.arange(nh)], axis=1)
    in_map = np.stack([np.arange(nh), blocks], axis=1)
    elt = 2 if w.dtype == "bf16" else 4
    moved = 2 * nh * w.num_kv_heads * w.head_dim * w.block_size * elt
    rounds = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.swap_blocks(kc, vc, hk, hv, out_map, inplace=True)
        oracle.swap_blocks(hk, hv, kc, vc, in_map, inplace=True)
        rounds += 1
    dt = time.perf_counter() - t0
    return {"value": round(2 * rounds * moved / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"NumPy oracle, the same {nh} blocks out and back in between host "
                       f"arrays, {rounds} rounds, {2 * rounds * moved / 1e6:.0f} MB in "
                       f"{dt:.1f} s (one thread: NumPy copies)")}


def bench_math(args) -> int:
    """The fused decode step of the Llama-3-8B batch (64 sequences, lengths 128-2048, 8 kv
    heads, D 128, BS 16, bf16) with its products on the matrix cores and on the vector ALU
    (pa_set_decode_math), at 8 g query heads for each g of --groups: the K/V bytes are the
    same at every g, only the query rows differ.  The forms alternate over --rounds
    rounds on the same pools; each round times K steps after W of warm-up, and the
    median round is reported."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config, make_workload
    dev = torch.device("cuda:0")
    base = make_config(1, seed=args.seed)
    forms = ["mfma", "valu"] if args.math == "both" else [args.math]
    K, W = args.steps, args.warmup
    rows = []
    for g in [int(x) for x in args.groups.split(",")]:
        w = base if g == 4 else make_workload(
            name=f"{base.name}-g{g}", context_lens=base.context_lens, num_heads=8 * g,
            num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16", seed=base.info["seed"],
            max_blocks_per_seq=base.block_table.shape[1])
        new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
        hist = np.setdiff1d(np.arange(len(w.rec_slot)), new)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        kshape = pk.k_cache_shape(w.num_blocks, 8, 128, 16, torch.bfloat16)
        vshape = pk.v_cache_shape(w.num_blocks, 8, 128, 16, torch.bfloat16)
        kc0 = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
        vc0 = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
        pk.reshape_and_cache(up(w.rec_key[hist]), up(w.rec_value[hist]),
                             torch.from_numpy(w.rec_slot[hist]).to(dev), kc0, vc0)
        pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone())
                                for _ in range(max(1, args.replicas) - 1)]
        query, table = up(w.query), torch.from_numpy(w.block_table).to(dev)
        lens = torch.from_numpy(w.context_lens).to(dev)
        key, val = up(w.rec_key[new]), up(w.rec_value[new])
        slot = torch.from_numpy(w.rec_slot[new]).to(dev)
        out = torch.empty_like(query)
        ws = torch.empty(1, dtype=torch.uint8, device=dev)
        calls = [pk.prepare_decode_step(query, key, val, slot, table, lens, kc, vc, w.scale,
                                        max_context_len=w.max_context_len, out=out,
                                        workspace=ws, host_context_lens=w.context_lens)
                 for kc, vc in pools]
        kv = unique_kv_bytes(w)
        times = {f: [] for f in forms}
        for _ in range(max(1, args.rounds)):
            for f in forms:
                pk.set_decode_math(f)
                for i in range(W):
                    calls[i % len(calls)]()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for i in range(K):
                    calls[i % len(calls)]()
                e1.record()
                torch.cuda.synchronize()
                times[f].append(e0.elapsed_time(e1) * 1e3 / K)
        pk.set_decode_math("mfma")
        row = {"g": g, "workload": w.name, "num_heads": w.num_heads, "kv_bytes": kv}
        for f in forms:
            us = float(np.median(times[f]))
            row[f] = {"us_per_launch": round(us, 2), "rounds_us": [round(t, 2) for t in times[f]],
                      "GB/s": round(kv / (us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if len(forms) == 2:
            row["valu_over_mfma"] = round(row["valu"]["us_per_launch"] /
                                          row["mfma"]["us_per_launch"], 4)
        log(f"g={g}: " + ", ".join(f"{f} {row[f]['us_per_launch']} us" for f in forms))
        rows.append(row)
        del pools, kc0, vc0
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "fused decode step, matrix cores vs vector ALU", "unit": "us",
                      "steps": K, "warmup": W, "rounds": args.rounds, "dtype": "bf16",
                      "higher_is_better": False, "data": "synthetic",
                      "config": {"workload": f"{base.name} at g = {args.groups}",
                                 "pool_replicas": max(1, args.replicas)},
                      "rows": rows}), flush=True)
    return 0


def balanced_pair_lengths(lens: np.ndarray) -> np.ndarray:
    """The same lengths spread, rearranged so that the paired mode's pairs (r-th longest with
    r-th shortest) all hold the same tokens: the r-th shortest becomes 2 * mean - r-th
    longest (at least 1)."""
    s = np.sort(lens)[::-1].astype(np.int64)
    n = len(s)
    total = 2 * int(round(float(lens.mean())))
    out = s.copy()
    for r in range(n // 2):
        out[n - 1 - r] = max(1, total - int(s[r]))
    return out


def bench_balance(args) -> int:
    """The fused step of the Llama-3-8B batch and of two batches with (about) the same KV
    bytes: one whose pairs (longest with shortest) hold exactly the mean tokens, one with
    every length equal to the mean.  If the pairs' imbalance set the step's time, the
    balanced batches would run faster by the imbalance."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config, make_workload

    dev = torch.device("cuda:0")
    base = make_config(1, seed=args.seed)
    L = base.context_lens
    variants = [("llama3-8b-decode-bf16", base),
                ("balanced-pairs", make_workload(
                    name="balanced-pairs", context_lens=balanced_pair_lengths(L),
                    num_heads=base.num_heads, num_kv_heads=base.num_kv_heads,
                    head_dim=base.head_dim, block_size=base.block_size, dtype="bf16", seed=1)),
                ("equal-lengths", make_workload(
                    name="equal-lengths", context_lens=np.full(len(L), int(round(float(L.mean())))),
                    num_heads=base.num_heads, num_kv_heads=base.num_kv_heads,
                    head_dim=base.head_dim, block_size=base.block_size, dtype="bf16", seed=1))]
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    K, W, R = args.steps, args.warmup, max(4, args.replicas)
    rows = {}
    for name, w in variants:
        tdt = torch.bfloat16
        new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
        hist = np.setdiff1d(np.arange(len(w.rec_slot)), new)
        kc0 = torch.full(pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                          tdt), float("nan"), dtype=tdt, device=dev)
        vc0 = torch.full(pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                          tdt), float("nan"), dtype=tdt, device=dev)
        pk.reshape_and_cache(up(w.rec_key[hist]), up(w.rec_value[hist]),
                             torch.from_numpy(w.rec_slot[hist]).to(dev), kc0, vc0)
        pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
        q, kn, vn = up(w.query), up(w.rec_key[new]), up(w.rec_value[new])
        sl = torch.from_numpy(w.rec_slot[new]).to(dev)
        tb = torch.from_numpy(w.block_table).to(dev)
        ln = torch.from_numpy(w.context_lens).to(dev)
        out = torch.empty_like(q)
        calls = [pk.prepare_decode_step(q, kn, vn, sl, tb, ln, kc, vc, w.scale,
                                        max_context_len=w.max_context_len, out=out,
                                        host_context_lens=w.context_lens.copy())
                 for kc, vc in pools]
        for i in range(W):
            calls[i % R]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            calls[i % R]()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        s = np.sort(w.context_lens)[::-1].astype(np.int64)
        pairs = [int(s[r] + (s[len(s) - 1 - r] if len(s) - 1 - r != r else 0))
                 for r in range((len(s) + 1) // 2)]
        kv = int(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim * 2
        rows[name] = {"launch_us_events": round(us, 2), "kv_bytes": kv,
                      "pair_tokens_max": max(pairs), "pair_tokens_mean": round(float(np.mean(pairs)), 1),
                      "tokens": int(w.context_lens.sum())}
        log(f"{name}: {us:.2f} us/launch, pair tokens max {max(pairs)} mean {np.mean(pairs):.1f}")
        del pools, calls
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "fused decode step us/launch, Llama-3-8B batch vs balanced batches",
                      "unit": "us", "n_gpus": 1, "steps": K, "warmup": W, "pool_replicas": R,
                      "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "llama3-8b-decode-bf16 and two length variants"},
                      "rows": rows}), flush=True)
    return 0


def bench_suffixes(args) -> int:
    """The prefix-sharing batch (128 sequences over one shared 1024-token prefix) against
    the same sequences' private suffixes alone: pa_decode_step_shared_prefix on the batch,
    pa_decode_step on a batch of the suffix lengths (the same heads, block size and new
    tokens' shape).  The suffixes' step is a floor for any way of adding the prefix."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config, make_workload

    dev = torch.device("cuda:0")
    base = make_config(3, seed=args.seed)
    pfx_len = int(base.info["shared_prefix_len"])
    suffix = make_workload(name="prefix-sharing-suffixes", context_lens=base.context_lens - pfx_len,
                           num_heads=base.num_heads, num_kv_heads=base.num_kv_heads,
                           head_dim=base.head_dim, block_size=base.block_size, dtype="bf16",
                           seed=base.info["seed"])
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    K, W, R = args.steps, args.warmup, max(4, args.replicas)
    rows = {}
    for name, w, shared in (("prefix-sharing-bf16-prefix", base, True),
                            ("suffixes-alone", suffix, False)):
        tdt = torch.bfloat16
        new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
        hist = np.setdiff1d(np.arange(len(w.rec_slot)), new)
        kc0 = torch.full(pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                          tdt), float("nan"), dtype=tdt, device=dev)
        vc0 = torch.full(pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                          tdt), float("nan"), dtype=tdt, device=dev)
        pk.reshape_and_cache(up(w.rec_key[hist]), up(w.rec_value[hist]),
                             torch.from_numpy(w.rec_slot[hist]).to(dev), kc0, vc0)
        pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
        q, kn, vn = up(w.query), up(w.rec_key[new]), up(w.rec_value[new])
        sl = torch.from_numpy(w.rec_slot[new]).to(dev)
        tb = torch.from_numpy(w.block_table).to(dev)
        ln = torch.from_numpy(w.context_lens).to(dev)
        out = torch.empty_like(q)
        if shared:
            calls = [pk.prepare_decode_step_shared_prefix(
                q, kn, vn, sl, tb, ln, kc, vc, w.scale, prefix_blocks=pfx_len // w.block_size,
                max_context_len=w.max_context_len, out=out, host_context_lens=w.context_lens.copy())
                for kc, vc in pools]
        else:
            calls = [pk.prepare_decode_step(q, kn, vn, sl, tb, ln, kc, vc, w.scale,
                                            max_context_len=w.max_context_len, out=out,
                                            host_context_lens=w.context_lens.copy())
                     for kc, vc in pools]
        for i in range(W):
            calls[i % R]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            calls[i % R]()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        # unique KV bytes: the shared prefix counted once
        tokens = int(w.context_lens.sum()) - (pfx_len * (w.num_seqs - 1) if shared else 0)
        kv = tokens * 2 * w.num_kv_heads * w.head_dim * 2
        rows[name] = {"launch_us_events": round(us, 2), "kv_unique_bytes": kv,
                      "tokens_unique": tokens}
        log(f"{name}: {us:.2f} us/launch, {kv / 1e6:.1f} MB of unique KV")
        del pools, calls
        torch.cuda.empty_cache()
    whole = rows["prefix-sharing-bf16-prefix"]
    floor_us = rows["suffixes-alone"]["launch_us_events"]
    rows["floor"] = {"roofline_frac_at_floor": round(whole["kv_unique_bytes"] / (floor_us * 1e-6) / 8e12, 3),
                     "roofline_frac": round(whole["kv_unique_bytes"] / (whole["launch_us_events"] * 1e-6) / 8e12, 3)}
    print(json.dumps({"metric": "prefix-sharing step vs its private suffixes alone, us/launch",
                      "unit": "us", "n_gpus": 1, "steps": K, "warmup": W, "pool_replicas": R,
                      "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "prefix-sharing-bf16-prefix and its suffixes alone",
                                 "shared_prefix_len": pfx_len},
                      "rows": rows}), flush=True)
    return 0


def bench_coexec(args) -> int:
    """The co-execution probe (pa_coexec_probe): MFMA work only, VALU work only, both
    interleaved in every wave, and split between the two waves of each SIMD, at one to four
    waves per SIMD (4- or 8-wave workgroups, one to three of them per compute unit, all
    launched together); best of 5 launches each.  `ms_per_unit` divides a row's time by the
    units of work each SIMD does (one unit: one wave's iterations of its kind of work; M + V
    for the interleaved and split rows)."""
    import torch

    import paged_kv_cache_425_amd as pk
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4096
    # (mode, waves per workgroup, workgroups per compute unit)
    cases = [("mfma", 4, 1), ("valu", 4, 1), ("interleaved", 4, 1), ("mfma", 8, 1),
             ("valu", 8, 1), ("split", 8, 1), ("interleaved", 8, 1),
             ("mfma", 4, 3), ("valu", 4, 3), ("interleaved", 4, 3),
             ("mfma", 8, 2), ("valu", 8, 2), ("split", 8, 2), ("interleaved", 8, 2)]
    out = torch.empty(3 * cus * 8 * 64, dtype=torch.float32, device=dev)
    # where the waves run: the split rows need waves w and w + 4 of a workgroup on one SIMD
    pk.coexec_probe("placement", cus, 8, 1, out)
    torch.cuda.synchronize()
    simd = out[:cus * 8 * 64].view(cus, 8, 64)[:, :, 0].cpu()
    paired = bool((simd[:, :4] == simd[:, 4:]).all())
    log(f"placement: waves w and w + 4 share a SIMD in every workgroup: {paired}")
    rows = []
    for mode, waves, per_cu in cases:
        wgs = cus * per_cu
        per_simd = waves // 4 * per_cu
        units = per_simd // 2 if mode == "split" else per_simd
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pk.coexec_probe(mode, wgs, waves, iters, out)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        rows.append({"mode": mode, "waves_per_workgroup": waves, "workgroups": wgs,
                     "waves_per_simd": per_simd, "best_ms": round(best, 4),
                     "ms_per_unit": round(best / units, 4)})
        log(f"{mode:12s} {waves} waves/WG x {wgs} WGs ({per_simd}/SIMD): {best:.4f} ms, "
            f"{best / units:.4f} ms per unit")
    print(json.dumps({"metric": "MFMA / VALU co-execution probe, ms per launch (best of 5)",
                      "unit": "ms", "n_gpus": 1, "higher_is_better": False, "data": "synthetic",
                      "config": {"workload": "coexec probe", "compute_units": cus,
                                 "waves_w_and_w_plus_4_share_a_simd": paired,
                                 "iterations_per_wave": iters,
                                 "work_per_iteration": "8 MFMA 16x16x32 bf16 and/or 32 FMA"},
                      "rows": rows}), flush=True)
    return 0


def bench_writes(args) -> int:
    """What the append's writes cost the decode's reads: the decode of the continuous-batching
    mix (BS 16; pa_paged_attention, host order) timed alone, a scatter of the first N of its
    new tokens (pa_reshape_and_cache) timed alone, and the two alternating; the extra time
    of the pair over the sum is the cost of the scatter's dirty lines to the reads."""
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config

    dev = torch.device("cuda:0")
    w = make_config(2, seed=args.seed, block_size=16)
    tdt = torch.bfloat16
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)  # noqa: E731
    allr = np.arange(len(w.rec_slot))
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    kc0 = torch.zeros(pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                       tdt), dtype=tdt, device=dev)
    vc0 = torch.zeros(pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                                       tdt), dtype=tdt, device=dev)
    pk.reshape_and_cache(up(w.rec_key[allr]), up(w.rec_value[allr]),
                         torch.from_numpy(w.rec_slot[allr]).to(dev), kc0, vc0)
    R = max(4, args.replicas)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
    q, out = up(w.query), torch.empty_like(up(w.query))
    table = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    K, W = args.steps, args.warmup

    def timed(calls):
        for i in range(W):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    dec = [pk.prepare_paged_attention(q, table, lens, kc, vc, w.scale,
                                      max_context_len=w.max_context_len, out=out,
                                      host_context_lens=w.context_lens.copy())
           for kc, vc in pools]
    t_dec = timed(dec)
    rows = []
    for ntok in (8, 32, 64, 128, 256):
        sel = new[:ntok]
        key, val = up(w.rec_key[sel]), up(w.rec_value[sel])
        slot = torch.from_numpy(w.rec_slot[sel]).to(dev)
        sc = [pk.prepare_reshape_and_cache(key, val, slot, kc, vc) for kc, vc in pools]
        both = []
        for i in range(R):
            both += [sc[i], dec[i]]
        t_sc = timed(sc)
        t_both = 2 * timed(both)
        rows.append({"tokens_scattered": ntok,
                     "dirty_lines_at_most": ntok * w.num_kv_heads * (2 + w.head_dim // 8),
                     "scatter_us": round(t_sc, 2), "scatter_then_decode_us": round(t_both, 2),
                     "extra_us": round(t_both - t_sc - t_dec, 2)})
        log(f"{ntok} tokens: scatter {t_sc:.2f}, scatter+decode {t_both:.2f}, "
            f"extra {t_both - t_sc - t_dec:.2f} us (decode alone {t_dec:.2f})")
    print(json.dumps({"metric": "decode us after a scatter of N new tokens, continuous-batching mix",
                      "unit": "us", "n_gpus": 1, "steps": K, "warmup": W, "pool_replicas": R,
                      "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": w.name, "new_tokens": int(len(new))},
                      "decode_alone_us": round(t_dec, 2), "rows": rows}), flush=True)
    return 0


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path runs on one GPU and has no multi-GPU mode)", file=sys.stderr)
        return 2
    import torch

    import paged_kv_cache_425_amd as pk
    from workloads import make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (no HIP device visible)", file=sys.stderr)
        return 1
    pk.load_library()          # raises if the HIP library was not built
    if args.op == "copy_blocks":
        return bench_copy_blocks(args)
    if args.op == "prefill":
        return bench_prefill(args)
    if args.op == "fp8":
        return bench_fp8(args)
    if args.op == "swap":
        return bench_swap(args)
    if args.op == "ceiling":
        return bench_ceiling(args)
    if args.op == "math":
        return bench_math(args)
    if args.op == "suffixes":
        return bench_suffixes(args)
    if args.op == "balance":
        return bench_balance(args)
    if args.op == "coexec":
        return bench_coexec(args)
    if args.op == "writes":
        return bench_writes(args)
    dev = torch.device("cuda:0")

    t = time.perf_counter()
    w = make_config(args.config, seed=args.seed, block_size=args.block_size, variant=args.variant)
    log(f"workload {w.name}: S={w.num_seqs} Hq={w.num_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} BS={w.block_size} NB={w.num_blocks} max_len={w.max_context_len} "
        f"({time.perf_counter() - t:.1f} s to draw)")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # ---- device inputs ------------------------------------------------------
    # the step's new token of each sequence is its record at position L - 1
    new = np.array([w.seq_records[s][-1] for s in range(w.num_seqs)], dtype=np.int64)
    hist = np.setdiff1d(np.arange(len(w.rec_slot)), new)
    kshape = pk.k_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    vshape = pk.v_cache_shape(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, tdt)
    kc0 = torch.full(kshape, float("nan"), dtype=tdt, device=dev)
    vc0 = torch.full(vshape, float("nan"), dtype=tdt, device=dev)
    pk.reshape_and_cache(up(w.rec_key[hist]), up(w.rec_value[hist]),
                         torch.from_numpy(w.rec_slot[hist]).to(dev), kc0, vc0)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(max(1, args.replicas) - 1)]
    key_new, val_new = up(w.rec_key[new]), up(w.rec_value[new])
    slot_new = torch.from_numpy(w.rec_slot[new]).to(dev)
    query = up(w.query)
    table = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    out = torch.empty_like(query)
    part = args.partition_size if args.partition_size is not None else (w.partition_size or 0)
    need = pk.workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                             w.max_context_len, part, tdt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # the step as one launch (pa_decode_step) and as the two calls.  With --order host the
    # library sorts the scheduler's host copy of the lengths on every call (the copy a
    # serving loop keeps), so the host work of each step is inside the timed loop.
    host_lens = w.context_lens.copy()

    def prep_fused(order):
        hl = host_lens if order == "host" else None
        return [pk.prepare_decode_step(query, key_new, val_new, slot_new, table, lens, kc, vc,
                                       w.scale, max_context_len=w.max_context_len, out=out,
                                       partition_size=part, workspace=ws, host_context_lens=hl)
                for kc, vc in pools]
    other_order = "device" if args.order == "host" else "host"
    fused, fused_other = prep_fused(args.order), prep_fused(other_order)
    writes = [pk.prepare_reshape_and_cache(key_new, val_new, slot_new, kc, vc) for kc, vc in pools]
    decodes = [pk.prepare_paged_attention(query, table, lens, kc, vc, w.scale,
                                          max_context_len=w.max_context_len, out=out,
                                          partition_size=part, workspace=ws,
                                          host_context_lens=host_lens if args.order == "host"
                                          else None)
               for kc, vc in pools]
    nb = algorithmic_bytes(w)
    kv_unique = unique_kv_bytes(w)
    elt = 2 if w.dtype == "bf16" else 4
    new_bytes = 2 * w.num_seqs * w.num_kv_heads * w.head_dim * elt     # new K and V
    fused_bytes = nb["total"] + 2 * new_bytes + 8 * w.num_seqs          # read, written, slots
    K, W = args.steps, args.warmup
    part_used = part or pk.default_partition_size(w.num_seqs, w.num_kv_heads, w.max_context_len, tdt)
    needs_reduce = w.max_context_len > part_used

    def run_fused(n_rep: int, steps: int, calls=None) -> None:
        calls = fused if calls is None else calls
        for i in range(steps):
            calls[i % n_rep]()

    def run_two_calls(n_rep: int, steps: int) -> None:
        for i in range(steps):
            writes[i % n_rep]()
            decodes[i % n_rep]()

    def timed(fn, *a):
        """Wall time and HIP-event time of fn, with synchronisation on both sides.

        The events are recorded on the stream the launches go to (torch's current
        stream), once before the first and once after the last step, so they add
        no bubbles between launches."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        fn(*a)
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3

    R = len(pools)
    # ---- cold headline: the fused step, rotating over the pool copies ----------
    run_fused(R, W)
    wall, ev_s = timed(run_fused, R, K)
    log(f"cold fused step: {wall / K * 1e6:.1f} us/step wall, {ev_s / K * 1e6:.1f} us/launch "
        "(events)")
    # ---- the same step as two calls (reshape_and_cache, then paged_attention) --
    run_two_calls(R, W)
    wall2, ev2 = timed(run_two_calls, R, K)
    log(f"cold two-call step: {wall2 / K * 1e6:.1f} us/step wall")
    # ---- the fused step with the other order of the sequences -----------------
    run_fused(R, W, fused_other)
    wall3, ev3 = timed(run_fused, R, K, fused_other)
    log(f"cold fused step, {other_order} order: {wall3 / K * 1e6:.1f} us/step wall")

    # ---- warm (optional): one pool, repeated ----------------------------------
    warm = None
    if args.warm:
        run_fused(1, W)
        wall_w, ev_w = timed(run_fused, 1, K)
        log(f"warm fused step: {wall_w / K * 1e6:.1f} us/step wall")
        warm = {"us_per_step": round(wall_w / K * 1e6, 2),
                "value": round(kv_unique / (wall_w / K) / 1e9, 2),
                "launch_us_events": round(ev_w / K * 1e6, 2)}

    # ---- a prefix shared by every sequence: the step that computes it once per group ----
    pfx_len = int(w.info.get("shared_prefix_len", 0))
    plain = None
    step_name = "pa_decode_step: scatter of the new tokens + paged decode, one launch"
    if pfx_len and not args.plain_step:
        pfx_blocks = pfx_len // w.block_size
        hl = host_lens if args.order == "host" else None
        shared = [pk.prepare_decode_step_shared_prefix(
            query, key_new, val_new, slot_new, table, lens, kc, vc, w.scale,
            prefix_blocks=pfx_blocks, max_context_len=w.max_context_len, out=out,
            host_context_lens=hl) for kc, vc in pools]
        run_fused(R, W, shared)
        wall_p, ev_p = timed(run_fused, R, K, shared)
        log(f"cold shared-prefix step: {wall_p / K * 1e6:.1f} us/step wall, "
            f"{ev_p / K * 1e6:.1f} us/launch (events)")
        plain = {"step": "pa_decode_step", "us_per_step": round(wall / K * 1e6, 2),
                 "launch_us_events": round(ev_s / K * 1e6, 2),
                 "value": round(kv_unique / (wall / K) / 1e9, 2)}
        wall, ev_s = wall_p, ev_p
        step_name = (f"pa_decode_step_shared_prefix ({pfx_blocks} shared blocks), one launch: "
                     "per group of sequences the shared prefix read once, the scatter of the "
                     "new tokens + paged decode of the private suffixes, log-sum-exp merge")

    # host side of the headline call: the time the K calls take to enqueue, the GPU still busy
    # behind them (argument checks, the host sort of the lengths for the paired order, the
    # launch), next to the wall time per step less the kernel time from events
    head_calls = shared if (pfx_len and not args.plain_step) else fused
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_fused(R, K, head_calls)
    submit_s = time.perf_counter() - t0
    torch.cuda.synchronize()

    ms_step = wall / K * 1e3
    launch_avg_s = ev_s / K
    # HBM must deliver each distinct slot at least once: with shared blocks (a common prefix,
    # parallel samples) the unique bytes are the HBM figure and the logical bytes (every
    # sequence's own view) an effective rate served partly from the caches
    value = kv_unique / (ms_step * 1e-3) / 1e9
    value_logical = nb["kv"] / (ms_step * 1e-3) / 1e9
    fused_unique = fused_bytes - nb["kv"] + kv_unique
    achieved = fused_unique / launch_avg_s / 1e9
    traffic = load_traffic(w.name + ("" if part == (w.partition_size or 0) else
                                     "-default-partition" if part == 0 else f"-P{part}") +
                           ("-shared-prefix" if plain else ""))
    ceil = None
    if not args.no_ceiling:
        log("read ceiling (probe sweep) ...")
        ceil = measure_ceiling(nb["kv"], max(20, min(K, 100)), 5, replicas=R)
    kernels = "paged_decode_kernel" + (" + reduce_partitions_kernel" if needs_reduce else "")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "effective_logical_kv": {"value": round(value_logical, 2), "unit": "GB/s",
                                 "kv_bytes": nb["kv"]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, random block tables)",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "max_context_len": w.max_context_len,
                   "total_context_tokens": int(w.context_lens.astype(np.int64).sum()),
                   "partition_size": part_used,
                   "kv_bytes_per_step": nb["kv"], "kv_bytes_unique": kv_unique,
                   "seed": w.info["seed"],
                   "step": step_name,
                   "order": args.order + (" (host_context_lens sorted on the host every call)"
                                          if args.order == "host" else " (ranked in-kernel)"),
                   "pool_bytes_each": int(kc0.numel() * kc0.element_size()),
                   "pool_replicas": R, "parallelism": "none (1 GPU)"},
        "launch_us_events": round(launch_avg_s * 1e6, 2),
        "host": {"submit_us_per_call": round(submit_s / K * 1e6, 2),
                 "wall_minus_events_us_per_step": round((wall - ev_s) / K * 1e6, 2),
                 "note": "submit: enqueue time of one call (library checks, host sort of the "
                         "lengths, launch), hidden while it stays below the kernel time; "
                         "wall - events: the timed loop's start-up and drain, spread over K"},
        "two_call_step": {"us_per_step": round(wall2 / K * 1e6, 2),
                          "us_per_step_events": round(ev2 / K * 1e6, 2),
                          "value": round(kv_unique / (wall2 / K) / 1e9, 2)},
        f"{other_order}_order_step": {"us_per_step": round(wall3 / K * 1e6, 2),
                                      "launch_us_events": round(ev3 / K * 1e6, 2),
                                      "value": round(kv_unique / (wall3 / K) / 1e9, 2)},
        "warm": warm,
        "plain_step": plain,
        "roofline": {"kernel": ("pa_decode_step_shared_prefix: paged_decode_kernel "
                                "(shared-prefix mode)" if plain else f"pa_decode_step: {kernels}"),
                     "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": fused_unique},
        "ceiling": None if ceil is None else {
            "stream_GBs": ceil["stream"]["GB/s"], "gather_4k_GBs": ceil["gather"]["GB/s"],
            "probe": "pa_read_probe over the step's KV bytes, best of "
                     f"{len(CEILING_SHAPES)} launch shapes x default / nt loads, "
                     f"{R} rotating windows",
            "stream_shape": ceil["stream"], "gather_shape": ceil["gather"],
            "default_loads": ceil["default_loads"],
            "frac_of_stream": round(achieved / ceil["stream"]["GB/s"], 4),
            "frac_of_gather": round(achieved / ceil["gather"]["GB/s"], 4)},
        "pool_utilisation": pool_utilisation(w),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Benchmark: one decode step of paged MLA latent attention on one MI355X.

A step is one pass of the whole hot path over one batch: write the batch's newest
token rows into the paged cache (mla_cache_write), decode every request over its
context in page-aligned partitions (mla_decode_bf16, partials kept), then merge the
partitions by log-sum-exp (mla_merge_lse).  Inputs are synthetic and resident in
HBM before timing starts.

Default workload: the long-context batch, 4 requests x 262,144 tokens, 16 heads,
64-token pages drawn at random from a 32,768-page pool, 64 partitions per request.

Two timed passes of --steps steps each, eager launches on one stream: the first, between
two synchronisations, gives the reported value; the second records HIP events around every
kernel (per-kernel durations, the roofline figure), its timed steps enqueued behind untimed
ones so that the host stays ahead of the GPU.  --graph reports instead the step captured
as a HIP graph (10 steps per graph) and replayed (every warm-up replay checked bit for bit
against the eager result).  Prints one JSON line.  Each workload
is timed with the schedule that measured faster for it (per-request partitions or the
batch-balanced ranges).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload long_context] [--eager]

Other lines of the same path: --q-len (multi-token verify), --nope (NoPE-512 layer),
--geometry (GLA-g2, rank 256 / 768 / 1792), --balanced / --splits (schedule),
--flush-mib (decode times after a last-level-cache flush), --op gather | cache_write |
merge (the context gather, the cache write and the LSE merge on their own).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "latent-cache read GB/s (fraction of HBM peak) + decode tokens/s, H=16"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_context")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per request: > 1 times a speculative-decoding verify step "
                         "(mla_decode_mtp_*), which reads the cache once per request")
    ap.add_argument("--geometry", choices=("mla", "gla2", "rank256", "rank768", "rank1792"), default="mla",
                    help="gla2: GLA-g2 head groups on the same rows; rank256: a rank-256 layer (640-byte bf16 "
                         "rows made from the workload's rows; no cache write in the step)")
    ap.add_argument("--balanced", type=int, default=None, metavar="W",
                    help="batch-balanced decode with W workgroups (tokens cut evenly across requests); "
                         "default: the workload's measured schedule")
    ap.add_argument("--nope", action="store_true",
                    help="decode the workload as a NoPE-512 layer: 512-wide queries, rows written with a zero "
                         "rope part, which the NoPE kernels never read")
    ap.add_argument("--flush-mib", type=int, default=None, metavar="MIB",
                    help="also time each decode after a pass over MIB MiB of other memory (evicts the "
                         "last-level cache between repetitions); the roofline then uses these cold times. "
                         "Default: 1024 for workloads whose cache bytes fit in the 256 MB last-level "
                         "cache, 0 otherwise")
    ap.add_argument("--event-reps", type=int, default=50,
                    help="minimum number of steps in the per-kernel HIP-event pass (medians over at "
                         "least this many repetitions, whatever --steps is)")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="with --graph: steps captured per HIP graph (the largest divisor of --steps up "
                         "to this)")
    ap.add_argument("--row-loads", choices=("streaming", "cached"), default=None,
                    help="row loads of the decodes (MLA_FLAG_CACHED_ROWS per call for cached); default: the "
                         "workload's entry in workloads.BENCH_ROW_LOADS")
    ap.add_argument("--graph", action="store_true",
                    help="report the step replayed from a captured HIP graph instead of eager launches "
                         "(measured slower here for every workload: 1-7 %% per step)")
    ap.add_argument("--eager", action="store_true",
                    help="eager launches (the default; kept for older command lines)")
    ap.add_argument("--op", choices=("decode", "gather", "cache_write", "merge", "sparse"), default="decode",
                    help="gather: time mla_gather_context over the workload's whole context instead "
                         "(prefill-side context gather, fp8 rows upconverted to bf16)")
    ap.add_argument("--separate-write", action="store_true",
                    help="write the step's new rows with mla_cache_write before the decode (two launches) "
                         "instead of letting the decode write them (mla_decode_append_*, the default where "
                         "the configuration has that call: 576-value rows with rope, bf16 or fp8)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (counter calibration)")
    return ap.parse_args()


def _append_rows(w, T):
    """The step's new rows per request for mla_decode_append_*: positions L - T .. L - 1 of request b
    (the rows the cache already holds there, so every step writes the same bytes), [B, T, ...];
    a negative position gets slot -1 (not written)."""
    B, ps = w.batch, w.page_size
    lat = np.zeros((B, T, 512), np.uint16)
    pe = np.zeros((B, T, 64), np.uint16)
    slots = np.full((B, T), -1, np.int64)
    for b in range(B):
        for i in range(T):
            pos = int(w.seq_lens[b]) - T + i
            if pos < 0:
                continue
            s = int(w.block_table[b, pos // ps]) * ps + pos % ps
            r = int(np.searchsorted(w.slots, s))
            lat[b, i], pe[b, i], slots[b, i] = w.latent[r], w.k_pe[r], s
    return lat, pe, slots


def _copy_calibration(mib: int):
    """A plain copy of known size, for scaling the HBM byte counters of a profile."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def _read_ceiling(dev, stream, gib=2, reps=20, workgroups=2048):
    """Same-run streaming-read reference: median HIP-event time of `mla_bench_stream_read`
    (libmla_bench.so: every 16-byte word of a `gib` GiB buffer read once, each workgroup reading a
    contiguous range, four loads in flight per thread), with plain loads and with the non-temporal
    hint; `gbs` is the faster of the two.  This is what this machine streams from HBM with a kernel that does
    nothing but read."""
    import ctypes
    import torch
    from paged_mla_latent_amd.build import BENCH_LIB_PATH
    if not os.path.exists(BENCH_LIB_PATH):
        raise SystemExit(f"bench.py: {BENCH_LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(BENCH_LIB_PATH)
    lib.mla_bench_stream_read.restype = ctypes.c_int
    lib.mla_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(4 * workgroups, dtype=torch.int32, device=dev)

    def run(nt):
        rc = lib.mla_bench_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                       workgroups, nt, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"mla_bench_stream_read failed ({rc})")

    rates = {}
    for nt in (0, 1):
        for _ in range(3):
            run(nt)
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run(nt)
            b.record(stream)
            times.append((a, b))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in times]))
        rates["nontemporal" if nt else "plain"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, sink
    gbs = max(rates.values())
    return {"gbs": gbs, "frac": round(gbs / HBM_PEAK_GBS, 4), "gbs_plain": rates["plain"],
            "gbs_nontemporal": rates["nontemporal"],
            "how": f"mla_bench_stream_read over {gib} GiB, {workgroups} workgroups, median of {reps} HIP-event windows"}


RANKS = {"rank256": 256, "rank768": 768, "rank1792": 1792}


def _rank_cols(D):
    """Latent columns of a rank-D row made from a 512-wide one: column c is latent column c mod 512."""
    return np.arange(D) % 512


def _rank_rows(w, D, idx=None):
    """Rank-D rows (bf16 bits [n, D + 64]) made from the workload's rows: the latent columns
    of _rank_cols(D), then k_pe."""
    lat, pe = (w.latent, w.k_pe) if idx is None else (w.latent[idx], w.k_pe[idx])
    return np.concatenate([lat[:, _rank_cols(D)], pe], axis=1)


def _rank_q(w, D):
    """D + 64 query values per head, made from the workload's q like the rows."""
    return np.ascontiguousarray(np.concatenate([w.q[:, :, _rank_cols(D)], w.q[:, :, 512:]], axis=2))


def _geometry_q(w):
    """320 query values per head (the first 256 latent values, then the rope part)."""
    return _rank_q(w, 256)


def _cpu_baseline(w, requests, nope=False, q_mtp=None, geometry="mla", min_seconds=10.0):
    """Time the fp64 oracle on a bounded sample of the same workload, on the host cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    pool = w.poisoned_pool()
    idx = np.concatenate([np.searchsorted(w.slots, _request_slots(w, b)) for b in requests])
    oracle.cache_write(pool, w.latent[idx], None if nope else w.k_pe[idx], w.slots[idx], w.fmt)
    q = np.ascontiguousarray(w.q[:, :, :512]) if nope else (w.q if q_mtp is None else q_mtp)
    run = oracle.decode_nope if nope else (oracle.decode if q_mtp is None else oracle.decode_mtp)
    row_bytes = w.row_bytes - (128 if nope else 0)
    if geometry == "gla2":
        q, run = _geometry_q(w), oracle.decode_gla2
    elif geometry in RANKS:
        D = RANKS[geometry]
        flat = np.full((w.num_slots, D + 64), 0x7FC0, np.uint16)
        flat[w.slots[idx]] = _rank_rows(w, D, idx)
        q, pool, row_bytes = _rank_q(w, D), flat, 2 * (D + 64)

        def run(q, pool, bt, lens, ps, scale, fmt, requests):
            return oracle.decode_rank(q, pool, bt, lens, ps, scale, requests=requests)
    # Repeat the sample until about 10 s of host time has been spent.
    reps, t = 0, time.perf_counter()
    while True:
        run(q, pool, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=requests)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    tokens = int(sum(int(w.seq_lens[b]) for b in requests))
    per = dt / reps
    return {
        "value": round(tokens * row_bytes / per / 1e9, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 NumPy oracle ({run.__name__}) decoding requests {list(requests)} of the {w.name} batch "
                  f"({tokens} context tokens x {w.heads} heads), {reps} passes in {dt:.1f} s; "
                  f"{len(requests) / per:.1f} decode tokens/s; BLAS threads {threads}, "
                  f"host cpu_count {os.cpu_count()}",
    }


KERNEL_SOURCES = ("paged_mla_latent_amd/csrc/decode.hip", "paged_mla_latent_amd/csrc/mla_device.h",
                  "paged_mla_latent_amd/csrc/mla_internal.h", "paged_mla_latent_amd/csrc/cache_rows.h")


def _profiled_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from its committed counter profile
    (profiles/decode_<workload>_counters.txt), or None.

    None unless that profile exists, names the same kernel and the kernel sources still
    hash to what was profiled.
    """
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"decode_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != h.hexdigest()[:16] or vals.get("kernel") != kernel.split("<")[0]:
        return None
    return int(vals["decode_fetch_bytes"]) + int(vals["decode_write_bytes"])


def _request_slots(w, b):
    t = np.arange(int(w.seq_lens[b]), dtype=np.int64)
    return w.block_table[b].astype(np.int64)[t // w.page_size] * w.page_size + t % w.page_size


def _cpu_baseline_gather(w, requests, min_seconds=10.0):
    """Time the oracle's context gather on a bounded sample (whole requests) on the host cores."""
    import oracle
    pool = w.poisoned_pool()
    idx = np.concatenate([np.searchsorted(w.slots, _request_slots(w, b)) for b in requests])
    oracle.cache_write(pool, w.latent[idx], w.k_pe[idx], w.slots[idx], w.fmt)
    bt = w.block_table[requests]
    cu = np.concatenate([[0], np.cumsum(w.seq_lens[requests].astype(np.int64))])
    reps, t = 0, time.perf_counter()
    while True:
        oracle.gather_context(pool, bt, cu, None, w.page_size, w.fmt)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    rows = int(cu[-1])
    per = dt / reps
    return {
        "value": round(rows * (w.row_bytes + 1152) / per / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"NumPy oracle (gather_context) gathering requests {list(requests)} of the {w.name} batch "
                  f"({rows} rows), {reps} passes in {dt:.1f} s; single-threaded NumPy",
    }


def _bench_gather(args):
    """Context gather of every token of the workload into bf16 [tokens, 576] rows."""
    import torch
    import oracle
    import paged_mla_latent_amd as mla
    import workloads

    w = workloads.NAMED[args.workload]()
    dev = torch.device("cuda:0")
    fmt = mla.MLA_CACHE_BF16_576 if w.fmt == "bf16" else mla.MLA_CACHE_FP8_656

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    if w.fmt == "bf16":
        pool = torch.full((w.num_pages, w.page_size, 576), 0x7FC0, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        pool = torch.full((w.num_pages, w.page_size, 656), 0xFF, dtype=torch.uint8, device=dev)
    mla.mla_cache_write(bf16(w.latent), bf16(w.k_pe), torch.from_numpy(w.slots).to(dev), pool, fmt)
    bt = torch.from_numpy(w.block_table).to(dev)
    cu_np = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    cu = torch.from_numpy(cu_np).to(dev)
    rows = int(cu_np[-1])
    out = torch.empty((rows, 576), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        mla.mla_gather_context(pool, fmt, bt, cu, rows, out=out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        mla.mla_gather_context(pool, fmt, bt, cu, rows, out=out)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # spot check against the oracle: the first and last request's first rows
    check = [0, w.batch - 1]
    for b in check:
        n = min(64, int(w.seq_lens[b]))
        if n == 0:
            continue
        got = out[cu_np[b]: cu_np[b] + n].view(torch.int16).cpu().numpy().view(np.uint16)
        t = np.arange(n)
        slots = w.block_table[b].astype(np.int64)[t // w.page_size] * w.page_size + t % w.page_size
        raw = pool.view(torch.uint8).view(-1, w.row_bytes)[torch.from_numpy(slots).to(dev)].cpu().numpy()
        assert np.array_equal(got, oracle.upconvert_rows(raw, w.fmt)), f"gather of request {b} differs"
    moved = rows * (w.row_bytes + 1152)
    gbs = moved / (ms * 1e-3) / 1e9
    result = {
        "metric": "context gather GB/s (cache rows read + bf16 rows written)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.fmt, "data": "synthetic",
        "config": {"workload": w.name, "op": "gather", "rows": rows, "cache_row_bytes": w.row_bytes,
                   "bytes_per_step": moved},
        "kernel_ms": {"gather": round(ms, 4)},
        "roofline": {"kernel": f"gather_kernel<{'true' if w.fmt == 'fp8' else 'false'}>", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline_gather(w, [b for b in range(w.batch) if w.seq_lens[b] > 0][:2])
    print(json.dumps(result), flush=True)


def _time_events(fn, steps, warmup, stream):
    """Mean HIP-event milliseconds of fn() on `stream`, and the wall time of the timed loop."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])), time.perf_counter() - t0


def _bench_cache_write(args):
    """Cache write of every token of the workload (the pool fill): latent + k_pe + slot read,
    one row written per token."""
    import torch
    import oracle
    import paged_mla_latent_amd as mla
    import workloads

    w = workloads.NAMED[args.workload]()
    dev = torch.device("cuda:0")
    fmt = mla.MLA_CACHE_BF16_576 if w.fmt == "bf16" else mla.MLA_CACHE_FP8_656

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    shape = (w.num_pages, w.page_size, 576 if w.fmt == "bf16" else 656)
    pool = torch.zeros(shape, dtype=torch.bfloat16 if w.fmt == "bf16" else torch.uint8, device=dev)
    lat, pe, slots = bf16(w.latent), bf16(w.k_pe), torch.from_numpy(w.slots).to(dev)
    stream = torch.cuda.current_stream(dev)
    ms, wall = _time_events(lambda: mla.mla_cache_write(lat, pe, slots, pool, fmt), args.steps, args.warmup, stream)
    # the rows of a sample of tokens against the oracle's packing
    idx = np.random.default_rng(0).choice(w.slots.size, size=min(4096, w.slots.size), replace=False)
    got = pool.view(torch.uint8).view(-1, w.row_bytes)[torch.from_numpy(w.slots[idx]).to(dev)].cpu().numpy()
    assert np.array_equal(got, oracle.pack_rows(w.latent[idx], w.k_pe[idx], w.fmt)), "cache rows differ"
    T = int(w.slots.size)
    moved = T * (1024 + 128 + 8 + w.row_bytes)
    gbs = moved / (ms * 1e-3) / 1e9
    result = {
        "metric": "cache write GB/s (new rows read + cache rows written)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.fmt, "data": "synthetic",
        "config": {"workload": w.name, "op": "cache_write", "tokens": T, "cache_row_bytes": w.row_bytes,
                   "bytes_per_step": moved},
        "kernel_ms": {"cache_write": round(ms, 4)},
        "roofline": {"kernel": f"cache_write_{w.fmt}", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        n = 2048 if w.fmt == "fp8" else 65536
        host = w.poisoned_pool()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oracle.cache_write(host, w.latent[:n], w.k_pe[:n], w.slots[:n], w.fmt)
            reps += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(n * reps * (1024 + 128 + 8 + w.row_bytes) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"NumPy oracle (cache_write) writing the first {n} tokens of the {w.name} workload, {reps} "
                      f"passes in {dt:.1f} s; single-threaded NumPy"}
    print(json.dumps(result), flush=True)


def _bench_merge(args):
    """Log-sum-exp merge of the workload's split-decode partials (the bench's split count)."""
    import torch
    import oracle
    import paged_mla_latent_amd as mla
    import workloads

    w = workloads.NAMED[args.workload]()
    S = args.splits or workloads.BENCH_SPLITS[args.workload]
    if S < 2:
        raise SystemExit("--op merge needs a split count above 1")
    dev = torch.device("cuda:0")
    fmt = mla.MLA_CACHE_BF16_576 if w.fmt == "bf16" else mla.MLA_CACHE_FP8_656

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    shape = (w.num_pages, w.page_size, 576 if w.fmt == "bf16" else 656)
    pool = torch.zeros(shape, dtype=torch.bfloat16 if w.fmt == "bf16" else torch.uint8, device=dev)
    mla.mla_cache_write(bf16(w.latent), bf16(w.k_pe), torch.from_numpy(w.slots).to(dev), pool, fmt)
    decode = mla.mla_decode_bf16 if w.fmt == "bf16" else mla.mla_decode_fp8_656
    po, pl = decode(bf16(w.q), pool, torch.from_numpy(w.block_table).to(dev), torch.from_numpy(w.seq_lens).to(dev),
                    w.scale, num_splits=S, partials_only=True)
    po, pl = po.clone(), pl.clone()
    del pool
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms, wall = _time_events(lambda: mla.mla_merge_lse(po, pl, out=out, lse=lse), args.steps, args.warmup, stream)
    hpo, hpl = po.cpu().numpy(), pl.cpu().numpy()
    ref_o, ref_l = oracle.merge(hpo, hpl)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    live = np.isfinite(ref_l)
    assert np.allclose(o, ref_o, rtol=1e-5, atol=1e-6) and np.allclose(l[live], ref_l[live], atol=1e-5), "merge differs"
    moved = (S + 1) * w.batch * w.heads * 513 * 4
    gbs = moved / (ms * 1e-3) / 1e9
    result = {
        "metric": "LSE merge GB/s (partials read + merged rows written)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "op": "merge", "num_splits": S, "rows": w.batch * w.heads,
                   "bytes_per_step": moved},
        "kernel_ms": {"merge": round(ms, 4)},
        "roofline": {"kernel": "merge_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            oracle.merge(hpo, hpl)
            reps += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(moved * reps / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"NumPy oracle (merge) over the same {S} x {w.batch} x {w.heads} partials, {reps} passes in "
                      f"{dt:.1f} s"}
    print(json.dumps(result), flush=True)


def _bench_sparse(args):
    """Sparse decode step: every request's newest token attends to workloads.SPARSE_TOPK slots of
    its own context, listed per query (fewer for shorter contexts, -1 padded): the index-list
    decode, then the merge of its partitions."""
    import torch
    import oracle
    import paged_mla_latent_amd as mla
    import workloads

    w = workloads.NAMED[args.workload]()
    topk = workloads.SPARSE_TOPK
    idx_np = workloads.sparse_lists(w, topk)
    S = args.splits or workloads.SPARSE_SPLITS[args.workload]
    nope = args.nope
    row_loads = args.row_loads or workloads.BENCH_ROW_LOADS[args.workload]
    flags = mla.MLA_FLAG_CACHED_ROWS if row_loads == "cached" else 0
    dev = torch.device("cuda:0")
    fmt = mla.MLA_CACHE_BF16_576 if w.fmt == "bf16" else mla.MLA_CACHE_FP8_656

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # the pool at its full size, with the listed slots' rows written (the rest never read)
    used = np.unique(idx_np[idx_np >= 0]).astype(np.int64)
    rows_of = np.searchsorted(w.slots, used)
    if w.fmt == "bf16":
        pool = torch.full((w.num_pages, w.page_size, 576), 0x7FC0, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        pool = torch.full((w.num_pages, w.page_size, 656), 0xFF, dtype=torch.uint8, device=dev)
    mla.mla_cache_write(bf16(w.latent[rows_of]), bf16(w.k_pe[rows_of]), torch.from_numpy(used).to(dev), pool, fmt)
    q_np = np.ascontiguousarray(w.q[:, :, :512]) if nope else w.q
    q = bf16(q_np)
    idx = torch.from_numpy(idx_np).to(dev)
    name = f"mla_decode_sparse_{'nope_' if nope else ''}{'bf16' if w.fmt == 'bf16' else 'fp8_656'}"
    fn = getattr(mla, name)
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, mla.mla_decode_workspace_size(w.batch, w.heads, S)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(e=None):
        if e: e[0].record(stream)
        if S > 1:
            po, pl = fn(q, pool, idx, w.scale, num_splits=S, workspace=ws, partials_only=True, flags=flags)
            if e: e[1].record(stream)
            mla.mla_merge_lse(po, pl, out=out, lse=lse)
        else:
            fn(q, pool, idx, w.scale, num_splits=1, out=out, lse=lse, flags=flags)
            if e: e[1].record(stream)
        if e: e[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    reps = max(args.steps, args.event_reps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for _ in range(max(args.warmup, 8)):
        step()
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    warm = [e[0].elapsed_time(e[1]) for e in ev]
    merge = [e[1].elapsed_time(e[2]) for e in ev]
    # NoPE rows: the latent part only (bf16: 1,024 bytes; fp8: 512 codes + 16 scale bytes)
    row_bytes_read = w.row_bytes - (128 if nope else 0)
    valid = int((idx_np >= 0).sum())
    step_bytes = valid * row_bytes_read
    flush_mib = args.flush_mib if args.flush_mib is not None else (1024 if step_bytes < LLC_BYTES else 0)
    cold = warm
    if flush_mib:
        flush = torch.ones(flush_mib << 18, dtype=torch.float32, device=dev)
        ev_cold = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for e in ev_cold:
            flush.amax()
            step(e)
        torch.cuda.synchronize()
        cold = [e[0].elapsed_time(e[1]) for e in ev_cold]
        del flush
    t_decode = float(np.median(cold))
    # spot check: the first queries with 0, 1, some and all entries valid, against the oracle
    counts = (idx_np >= 0).sum(axis=1)
    picks = sorted({int(np.argmax(counts == c)) for c in (0, 1) if (counts == c).any()} |
                   {int(np.argmax(counts == topk)) if (counts == topk).any() else 0, int(np.argmin(counts))})
    compact = np.zeros((used.size, w.row_bytes), np.uint8)
    oracle.cache_write(compact, w.latent[rows_of], w.k_pe[rows_of], np.arange(used.size), w.fmt)
    local = np.where(idx_np >= 0, np.searchsorted(used, idx_np), -1)
    ref_o, ref_l = oracle.decode_sparse(q_np, compact, local, w.scale, w.fmt, tokens=picks)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for t in picks:
        if counts[t] == 0:
            assert (o[t] == 0).all() and np.isneginf(l[t]).all(), f"query {t}: an empty list is not (0, -inf)"
            continue
        err = np.abs(o[t] - ref_o[t]).max(axis=1) / np.abs(ref_o[t]).max(axis=1)
        assert err.max() <= 1e-2 and np.abs(l[t] - ref_l[t]).max() <= 1e-3, f"query {t} differs from the oracle"
    ms_step = wall * 1e3 / args.steps
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    decode_gbs = step_bytes / (t_decode * 1e-3) / 1e9
    rope = 0 if nope else 64
    kernel = f"decode_sparse_kernel<{f'Bf16Rows<512, {rope}>' if w.fmt == 'bf16' else f'Fp8Rows<{rope}, {str(nope).lower()}>'}>"
    result = {
        "metric": "sparse decode GB/s (listed cache rows read)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.fmt, "data": "synthetic",
        "decode_tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "config": {"workload": w.name, "op": "sparse", "queries": w.batch, "heads": w.heads, "topk": topk,
                   "valid_entries": valid, "num_splits": S, "layer": "nope-512" if nope else "rope-576",
                   "row_loads": row_loads, "row_bytes_read": row_bytes_read, "bytes_per_step": step_bytes,
                   "unique_cache_bytes": int(used.size) * row_bytes_read,
                   "step": "decode + merge" if S > 1 else "decode"},
        "flush_mib": flush_mib, "event_reps": reps,
        "kernel_ms_median": {"decode": round(float(np.median(warm)), 4), "merge": round(float(np.median(merge)), 4),
                             **({"decode_after_flush": round(t_decode, 4)} if flush_mib else {})},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(decode_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(decode_gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            threads = 1
        # the step's queries in turn (longest lists first) until about 10 s of host time
        order = [int(t) for t in np.argsort(-counts, kind="stable") if counts[t] > 0]
        n, done, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            t = order[n % len(order)]
            oracle.decode_sparse(q_np, compact, local, w.scale, w.fmt, tokens=[t])
            n, done = n + 1, done + int(counts[t]) * row_bytes_read
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 NumPy oracle (decode_sparse) on {n} queries of the same step (longest lists first), "
                      f"{dt:.1f} s; BLAS threads {threads}"}
    print(json.dumps(result), flush=True)


def main():
    args = _parse()
    if args.copy_calibration:
        _copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported by this build "
              f"(the multi-GPU split of this path is described in DESIGN.md but not built).", file=sys.stderr)
        sys.exit(2)

    if args.op == "gather":
        _bench_gather(args)
        return
    if args.op == "cache_write":
        _bench_cache_write(args)
        return
    if args.op == "merge":
        _bench_merge(args)
        return
    if args.op == "sparse":
        _bench_sparse(args)
        return

    import torch
    import paged_mla_latent_amd as mla
    import workloads

    w = workloads.NAMED[args.workload]()
    S = args.splits or workloads.BENCH_SPLITS[args.workload]
    balanced = args.balanced
    if balanced is None:
        default_bal = workloads.BENCH_SCHEDULE[args.workload] == "balanced"
        plain = args.geometry == "mla" and not args.splits
        balanced = workloads.BENCH_BALANCED_WORKGROUPS if (default_bal and plain) else 0
    row_loads = args.row_loads or workloads.BENCH_ROW_LOADS[args.workload]
    flags = mla.MLA_FLAG_CACHED_ROWS if row_loads == "cached" else 0  # per decode call
    dev = torch.device("cuda:0")
    fmt = mla.MLA_CACHE_BF16_576 if w.fmt == "bf16" else mla.MLA_CACHE_FP8_656

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- inputs resident in HBM ------------------------------------------------------
    if w.fmt == "bf16":
        pool = torch.full((w.num_pages, w.page_size, 576), 0x7FC0, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        pool = torch.full((w.num_pages, w.page_size, 656), 0xFF, dtype=torch.uint8, device=dev)
    nope, T = args.nope, args.q_len
    if nope and T != 1:
        raise SystemExit("--nope and --q-len > 1 are not combined by this benchmark")
    mla.mla_cache_write(bf16(w.latent), None if nope else bf16(w.k_pe), torch.from_numpy(w.slots).to(dev), pool, fmt)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    q_mtp = None
    if T > 1:
        q_mtp, ns, nl, npe = workloads.verify_step(w, T)
        q = bf16(q_mtp)
        new_lat, new_pe, new_slots = bf16(nl), bf16(npe), torch.from_numpy(ns).to(dev)
    else:
        q = bf16(w.q[:, :, :512]) if nope else bf16(w.q)
        new_lat, new_pe = bf16(w.new_latent), None if nope else bf16(w.new_k_pe)
        new_slots = torch.from_numpy(w.new_slots).to(dev)
    rows = T * w.heads  # query rows per request
    out = torch.empty((w.batch, rows, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, rows), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, mla.mla_decode_workspace_size(w.batch, rows, S)), dtype=torch.uint8, device=dev)
    if T > 1:
        mtp = mla.mla_decode_mtp_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_fp8_656
        out4, lse3 = out.view(w.batch, T, w.heads, 512), lse.view(w.batch, T, w.heads)

        def decode(q, pool, bt, lens, scale, num_splits, out=None, lse=None, workspace=None, partials_only=False,
                   flags=0):
            return mtp(q, pool, bt, lens, scale, num_splits=num_splits, workspace=workspace, flags=flags,
                       partials_only=partials_only, out=None if out is None else out4,
                       lse=None if lse is None else lse3)
    elif nope:
        decode = mla.mla_decode_nope_bf16 if w.fmt == "bf16" else mla.mla_decode_nope_fp8_656
    else:
        decode = mla.mla_decode_bf16 if w.fmt == "bf16" else mla.mla_decode_fp8_656
    groups = 1 if rows <= 16 else (2 if rows <= 32 else 4)
    rope = 0 if nope else 64
    kernel = f"decode_kernel<{f'Bf16Rows<512, {rope}>' if w.fmt == 'bf16' else f'Fp8Rows<{rope}, false>'}, {groups}, false>"
    geom, width, write_rows, row_bytes_read = args.geometry, 512, True, w.row_bytes - (128 if nope else 0)
    if geom != "mla":
        if nope or T > 1:
            raise SystemExit("--geometry is not combined with --nope or --q-len by this benchmark")
        width = 256
        q = bf16(_geometry_q(w))
        if geom == "gla2":
            decode = mla.mla_decode_gla2_bf16 if w.fmt == "bf16" else mla.mla_decode_gla2_fp8_656
            kernel = f"decode_kernel<{'Bf16Rows<512, 64>' if w.fmt == 'bf16' else 'Fp8Rows<64, false>'}, 1, true>"
        else:
            if w.fmt != "bf16":
                raise SystemExit(f"--geometry {geom} needs a bf16 workload")
            D = RANKS[geom]
            K, width = D + 64, D
            q = bf16(_rank_q(w, D))
            # rank-D rows assembled on the device from the workload's rows (see _rank_rows)
            del pool
            flat = torch.full((w.num_slots, K), 0x7FC0, dtype=torch.int16, device=dev).view(torch.bfloat16)
            cols = torch.from_numpy(_rank_cols(D)).to(dev)
            for c0 in range(0, w.slots.size, 1 << 18):
                sl = slice(c0, c0 + (1 << 18))
                flat[torch.from_numpy(w.slots[sl]).to(dev)] = torch.cat(
                    [bf16(w.latent[sl])[:, cols], bf16(w.k_pe[sl])], dim=1)
            pool = flat.view(w.num_pages, w.page_size, K)
            decode = {256: mla.mla_decode_rank256_bf16, 768: mla.mla_decode_rank768_bf16,
                      1792: mla.mla_decode_rank1792_bf16}[D]
            write_rows, row_bytes_read = False, 2 * K
            kernel = "decode_kernel<Bf16Rows<256, 64>, 1, false>" if D == 256 else f"decode_wide_kernel<{D}>"
            if D > 512:
                ws = torch.empty(max(1, mla.mla_decode_rank_workspace_size(w.batch, rows, S, D)), dtype=torch.uint8,
                                 device=dev)
        out = torch.empty((w.batch, rows, width), dtype=torch.float32, device=dev)
    gla_balanced = bool(balanced) and geom == "gla2"
    if balanced:
        if geom not in ("mla", "gla2"):
            raise SystemExit(f"--balanced is not combined with --geometry {geom} by this benchmark")
        if gla_balanced:
            decode_bal = mla.mla_decode_gla2_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_gla2_balanced_fp8_656
        elif nope:
            decode_bal = mla.mla_decode_balanced_nope_bf16 if w.fmt == "bf16" else mla.mla_decode_balanced_nope_fp8_656
        elif T > 1:
            decode_bal = mla.mla_decode_mtp_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_balanced_fp8_656
        else:
            decode_bal = mla.mla_decode_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_balanced_fp8_656
        ws = torch.empty(mla.mla_decode_balanced_workspace_size(w.batch, rows, balanced), dtype=torch.uint8,
                         device=dev)
        S = 1
        kernel = f"decode_flat_kernel<{f'Bf16Rows<512, {rope}>' if w.fmt == 'bf16' else f'Fp8Rows<{rope}, false>'}, {groups}, false>"
        if gla_balanced:
            kernel = f"decode_flat_kernel<{'Bf16Rows<512, 64>' if w.fmt == 'bf16' else 'Fp8Rows<64, false>'}, 1, true>"
    # The decode writes the step's new rows itself (one launch fewer) where it has that call.
    fused_write = write_rows and not args.separate_write and geom == "mla" and not nope
    if kernel.startswith(("decode_kernel<", "decode_flat_kernel<")):  # the row-writing template argument
        kernel = kernel[:-1] + (", true>" if fused_write else ", false>")
    if fused_write:
        a_lat, a_pe, a_slots = _append_rows(w, T)
        a_lat, a_pe, a_slots = bf16(a_lat), bf16(a_pe), torch.from_numpy(a_slots).to(dev)
        q_app = q.view(w.batch, T, w.heads, 576)
        if balanced:
            app_fn = mla.mla_decode_append_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_append_balanced_fp8_656
        else:
            app_fn = mla.mla_decode_append_bf16 if w.fmt == "bf16" else mla.mla_decode_append_fp8_656
        out4, lse3 = out.view(w.batch, T, w.heads, 512), lse.view(w.batch, T, w.heads)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    reps = max(args.steps, args.event_reps)  # per-kernel event windows: at least this many
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    if args.steps < args.event_reps:
        print(f"bench.py: {args.steps} timed steps give the value; the per-kernel medians use {reps} "
              f"event-timed steps", file=sys.stderr)
    flush_mib = args.flush_mib
    if flush_mib is None:  # rows that fit in the last-level cache are timed after a flush as well
        flush_mib = 1024 if w.tokens * w.row_bytes < LLC_BYTES else 0

    def step(e=None):
        if e: e[0].record(stream)
        if write_rows and not fused_write:
            mla.mla_cache_write(new_lat, new_pe, new_slots, pool, fmt)
        if e: e[1].record(stream)
        if fused_write:  # the decode window holds the row writes
            if balanced:
                app_fn(q_app, a_lat, a_pe, a_slots, pool, bt, lens, w.scale, num_workgroups=balanced, workspace=ws,
                       partials_only=True, flags=flags)
                if e: e[2].record(stream)
                mla.mla_merge_lse_balanced(ws, w.batch, rows, balanced, out=out, lse=lse)
            elif S > 1:
                po, pl = app_fn(q_app, a_lat, a_pe, a_slots, pool, bt, lens, w.scale, num_splits=S, workspace=ws,
                                partials_only=True, flags=flags)
                if e: e[2].record(stream)
                mla.mla_merge_lse(po, pl, out=out, lse=lse)
            else:
                app_fn(q_app, a_lat, a_pe, a_slots, pool, bt, lens, w.scale, num_splits=1, out=out4, lse=lse3,
                       flags=flags)
                if e: e[2].record(stream)
        elif gla_balanced:  # no partials-only form: the decode window holds the merge as well
            decode_bal(q, pool, bt, lens, w.scale, num_workgroups=balanced, workspace=ws, out=out, lse=lse,
                       flags=flags)
            if e: e[2].record(stream)
        elif balanced:
            decode_bal(q, pool, bt, lens, w.scale, num_workgroups=balanced, workspace=ws, partials_only=True,
                       flags=flags)
            if e: e[2].record(stream)
            mla.mla_merge_lse_balanced(ws, w.batch, rows, balanced, out=out, lse=lse)
        elif S > 1:
            po, pl = decode(q, pool, bt, lens, w.scale, num_splits=S, workspace=ws, partials_only=True, flags=flags)
            if e: e[2].record(stream)
            if width == 512:
                mla.mla_merge_lse(po, pl, out=out, lse=lse)
            else:
                mla.mla_merge_lse_width(po, pl, out=out, lse=lse)
        else:
            decode(q, pool, bt, lens, w.scale, num_splits=1, out=out, lse=lse, flags=flags)
            if e: e[2].record(stream)
        if e: e[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = eager_wall = time.perf_counter() - t0
    launch_mode = "eager"
    # Per-kernel HIP-event windows: the timed steps are enqueued behind untimed ones, with no
    # synchronisation between, so the host runs ahead of the GPU and no launch latency falls
    # inside a window (each window times its kernel as back-to-back execution runs it).
    for _ in range(max(args.warmup, 8)):
        step()
    for i in range(reps):
        step(ev[i])
    torch.cuda.synchronize()

    if args.graph and not args.eager:
        # n consecutive steps captured into one graph (as a serving loop captures a whole
        # forward pass, one decode per layer) and replayed K / n times: every step's kernels
        # still run, in order, with one host submission per n steps.  Every warm-up replay
        # must reproduce the eager result bit for bit.
        n_graph = max(d for d in range(1, min(args.graph_steps, args.steps) + 1) if args.steps % d == 0)
        eager_out, eager_lse = out.clone(), lse.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(n_graph):
                step()
        for _ in range(max(1, args.warmup // n_graph)):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse), "graph replay differs from eager"
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps // n_graph):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        launch_mode = f"hip_graph, {n_graph} steps per graph"

    ms_step = wall * 1e3 / args.steps
    ms_step_eager = eager_wall * 1e3 / args.steps
    win = {name: [e[a].elapsed_time(e[b]) for e in ev]
           for name, a, b in (("cache_write", 0, 1), ("decode", 1, 2), ("merge", 2, 3), ("step", 0, 3))}
    t_write, t_decode, t_merge = (float(np.mean(win[k])) for k in ("cache_write", "decode", "merge"))
    med = {k: round(float(np.median(v)), 4) for k, v in win.items()}
    if gla_balanced:  # the merge runs inside the decode call (its window holds both)
        del med["merge"]
        med["decode_with_merge"] = med.pop("decode")
    if fused_write:  # the row writes run inside the decode (its window holds both)
        del med["cache_write"]
        med["decode_with_row_writes"] = med.pop("decode")
    t_decode_warm = t_decode
    if flush_mib:
        # Each step again, eagerly, after reading flush_mib MiB of other memory, so that the
        # cache rows come from HBM rather than from the last-level cache.  The pass only reads
        # (a write pass would leave dirty lines whose write-back lands in the timed decode).
        flush = torch.ones(flush_mib << 18, dtype=torch.float32, device=dev)
        ev_cold = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        for i in range(reps):
            flush.amax()
            step(ev_cold[i])
        torch.cuda.synchronize()
        cold = [e[1].elapsed_time(e[2]) for e in ev_cold]
        t_decode = float(np.mean(cold))
        med["decode_after_flush"] = round(float(np.median(cold)), 4)
        del flush
    ceiling = _read_ceiling(dev, stream)
    # rows that see at least one token (query i of a verify step sees L - q_len + 1 + i)
    vis = (w.seq_lens[:, None] - T + 1 + np.arange(T)[None, :]) > 0
    live = np.repeat(vis, w.heads, axis=1)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o[live]).all() and np.isfinite(l[live]).all(), "non-finite decode output"
    assert np.isneginf(l[~live]).all() and (o[~live] == 0).all(), "a row that sees no token is not (0, -inf)"

    # bytes the decode must read: whole rows, rows without their rope part (NoPE), or
    # 640-byte rank-256 rows
    cache_bytes = w.tokens * row_bytes_read
    gbs = cache_bytes / (ms_step * 1e-3) / 1e9
    decode_gbs = cache_bytes / (t_decode * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.fmt,
        "data": "synthetic",
        "hbm_fraction": round(gbs / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(w.batch * T / (ms_step * 1e-3), 1),
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads, "context_tokens": w.tokens,
            "page_size": w.page_size, "pool_pages": w.num_pages, "num_splits": S,
            "schedule": f"batch-balanced, {balanced} workgroups" if balanced else "per-request partitions",
            # rank-768 rows are read in 64-byte row segments with plain loads
            "row_loads": "plain" if geom == "rank768" else row_loads,
            "layer": "nope-512" if nope else "rope-576", "query_tokens_per_request": T, "geometry": geom,
            "cache_row_bytes": 2 * (RANKS[geom] + 64) if geom in RANKS else w.row_bytes,
            "row_bytes_read": row_bytes_read,
            "step": ("decode + merge" if not write_rows
                     else "decode writing the new rows + merge" if fused_write else "cache write + decode + merge"),
            "cache_bytes_per_step": cache_bytes,
            # distinct rows read: below cache_bytes_per_step when requests share pages (high_slot),
            # whose figure is then an effective bandwidth, part of it served from the caches
            "unique_cache_bytes": int(w.slots.size) * row_bytes_read,
            "bandwidth": "effective (pages repeat across requests)" if w.slots.size < w.tokens else "hbm",
        },
        "launch": launch_mode,
        "flush_mib": flush_mib,
        "event_reps": reps,
        "kernel_ms_median": med,
        "read_ceiling": ceiling,
        "eager_ms_per_step": round(ms_step_eager, 4),
        "kernel_ms": {**({} if fused_write else {"cache_write": round(t_write, 4)}), "decode": round(t_decode_warm, 4),
                      "merge": round(t_merge, 4), **({"decode_after_flush": round(t_decode, 4)} if flush_mib else {})},
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": round(decode_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(decode_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if (nope or T > 1 or geom != "mla") else _profiled_traffic(w.name, kernel),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(w, list(range(min(w.batch, 4))), nope, q_mtp, geom)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

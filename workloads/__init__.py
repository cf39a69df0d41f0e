"""Seeded synthetic inputs for paged MLA latent decode.

This module only draws random numbers and lays them out: sequence lengths,
block tables (page placement), absorbed queries and the latent rows that a
request's tokens hold.  It contains none of the method's arithmetic (no
scores, no softmax, no quantisation, no LSE merge, no cache packing).  Both
sides of every parity check consume what it returns: the fp64 oracle under
``oracle/`` and the HIP library under ``paged_mla_latent_amd/``.  Neither of
those imports the other, and neither is imported here.

Row geometry (sabi-mla-vllm page, opening paragraph; vLLM PR #55543,
description): each cached token holds a 512-wide latent plus one shared
64-wide rotary key, 576 values.  Values are drawn N(0, 1) in float32 and
rounded to bf16 with round-to-nearest-even, the input precision the kernels
consume.

Draw order for every workload: lengths, then page assignment, then q, then
rows, all from ``numpy.random.default_rng(seed)``.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE
ROW_BYTES = {"bf16": 2 * ROW, "fp8": 656}

# Poison written into every pool byte that no request reads.  bf16 pools get
# the quiet NaN 0x7FC0 per element; fp8 pools get 0xFF per byte (NaN as an
# e4m3fn code, as an fp32 scale and as a bf16 rope value).
BF16_POISON = 0x7FC0
FP8_POISON_BYTE = 0xFF

DEFAULT_SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_as_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns (used only to build special inputs)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One batch of decode inputs.

    Attributes
    ----------
    name, fmt: workload label and cache format ("bf16" 1152-byte rows or "fp8" 656-byte rows).
    batch, heads, page_size, num_pages: geometry; the pool holds num_pages * page_size slots.
    seq_lens: int32 [B]; block_table: int32 [B, W], -1 past each request's last page.
    q: uint16 bf16 bits [B, H, 576], absorbed query = cat(q_latent[512], q_pe[64]).
    scale: softmax scale (a float32 value).
    slots: int64 [T], every slot some request reads, ascending and unique.
    latent: uint16 bf16 bits [T, 512]; k_pe: uint16 bf16 bits [T, 64]; row i belongs to slots[i].
    new_slots / new_latent / new_k_pe: the newest token of each non-empty request
        (deduplicated by slot); a decode step writes these rows before attending.
    """

    name: str
    fmt: str
    batch: int
    heads: int
    page_size: int
    num_pages: int
    seq_lens: np.ndarray
    block_table: np.ndarray
    q: np.ndarray
    scale: float
    slots: np.ndarray
    latent: np.ndarray
    k_pe: np.ndarray
    new_slots: np.ndarray
    new_latent: np.ndarray
    new_k_pe: np.ndarray

    @property
    def row_bytes(self) -> int:
        return ROW_BYTES[self.fmt]

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    @property
    def tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    def cache_bytes_read(self) -> int:
        """Latent-cache bytes one decode pass reads: one row per context token."""
        return self.tokens * self.row_bytes

    def poisoned_pool(self) -> np.ndarray:
        """Pool bytes [num_pages, page_size, row_bytes] before any row is written."""
        shape = (self.num_pages, self.page_size, self.row_bytes)
        if self.fmt == "bf16":
            pool = np.empty(shape[:2] + (ROW,), dtype=np.uint16)
            pool.fill(BF16_POISON)
            return pool.view(np.uint8).reshape(shape)
        pool = np.empty(shape, dtype=np.uint8)
        pool.fill(FP8_POISON_BYTE)
        return pool


def _block_table(page_lists, width: int) -> np.ndarray:
    bt = np.full((len(page_lists), max(width, 1)), -1, dtype=np.int32)
    for b, pages in enumerate(page_lists):
        bt[b, : len(pages)] = pages
    return bt


def make_workload(
    name: str,
    *,
    seq_lens,
    heads: int,
    page_size: int,
    num_pages: int,
    seed: int = 0,
    fmt: str = "bf16",
    scale: float = DEFAULT_SCALE,
    page_range: tuple[int, int] | None = None,
    pages_shared_across_requests: bool = False,
    row_scale_log10: tuple[float, float] | None = None,
    rng: np.random.Generator | None = None,
) -> Workload:
    """Build a workload from explicit lengths.

    seq_lens: int sequence, or a callable ``rng -> lengths`` so that the lengths
        are the first draw from the seeded generator.
    page_range: physical pages are drawn from [lo, hi) (default: the whole pool).
    pages_shared_across_requests: False draws all pages of all requests without
        replacement; True draws each request's pages without replacement but
        independently of the other requests (pages may repeat across requests,
        like shared prefixes).
    row_scale_log10: if given, every row is multiplied by 10**u, u uniform in the
        range, before rounding to bf16 (row-RMS spread for softmax range stress).
    """
    if fmt not in ROW_BYTES:
        raise ValueError(f"unknown cache format {fmt!r}")
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = seq_lens(rng) if callable(seq_lens) else seq_lens
    lens = np.asarray(lens, dtype=np.int64)
    if lens.ndim != 1 or (lens < 0).any():
        raise ValueError("seq_lens must be a 1-D array of non-negative lengths")
    batch = int(lens.shape[0])
    ps = int(page_size)
    npages_req = (lens + ps - 1) // ps
    lo, hi = (0, num_pages) if page_range is None else page_range
    if not (0 <= lo < hi <= num_pages):
        raise ValueError("bad page range")

    # Page assignment.
    if pages_shared_across_requests:
        page_lists = [lo + rng.choice(hi - lo, size=int(n), replace=False) for n in npages_req]
    else:
        total = int(npages_req.sum())
        if total > hi - lo:
            raise ValueError(f"{name}: needs {total} pages, pool range has {hi - lo}")
        perm = lo + rng.permutation(hi - lo)[:total]
        offs = np.concatenate([[0], np.cumsum(npages_req)])
        page_lists = [perm[offs[b] : offs[b + 1]] for b in range(batch)]
    width = int(npages_req.max()) if batch else 1
    block_table = _block_table(page_lists, width)

    # Queries.
    q = bf16_bits(rng.standard_normal((batch, heads, ROW), dtype=np.float32))

    # Slots some request reads: on page p, offsets [0, n_p) with n_p the longest
    # prefix of that page any request covers.
    fill = np.zeros(num_pages, dtype=np.int64)
    for b in range(batch):
        pages = page_lists[b]
        if len(pages) == 0:
            continue
        counts = np.full(len(pages), ps, dtype=np.int64)
        counts[-1] = lens[b] - (len(pages) - 1) * ps
        np.maximum.at(fill, pages, counts)
    used_pages = np.nonzero(fill)[0]
    slots = _slots_of_pages(used_pages, fill, ps)

    # Rows, drawn in ascending slot order, in chunks to bound host memory.
    T = int(slots.shape[0])
    latent = np.empty((T, LATENT), dtype=np.uint16)
    k_pe = np.empty((T, ROPE), dtype=np.uint16)
    chunk = 1 << 16
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        x = rng.standard_normal((e - s, ROW), dtype=np.float32)
        if row_scale_log10 is not None:
            u = rng.uniform(row_scale_log10[0], row_scale_log10[1], size=(e - s, 1))
            x = (x * np.power(10.0, u)).astype(np.float32)
        bits = bf16_bits(x)
        latent[s:e] = bits[:, :LATENT]
        k_pe[s:e] = bits[:, LATENT:]

    # Newest token of each non-empty request.
    new = []
    for b in range(batch):
        L = int(lens[b])
        if L:
            t = L - 1
            new.append(int(page_lists[b][t // ps]) * ps + t % ps)
    new_slots = np.unique(np.asarray(new, dtype=np.int64))
    idx = np.searchsorted(slots, new_slots)
    return Workload(
        name=name,
        fmt=fmt,
        batch=batch,
        heads=int(heads),
        page_size=ps,
        num_pages=int(num_pages),
        seq_lens=lens.astype(np.int32),
        block_table=block_table,
        q=q,
        scale=float(np.float32(scale)),
        slots=slots,
        latent=latent,
        k_pe=k_pe,
        new_slots=new_slots,
        new_latent=latent[idx].copy(),
        new_k_pe=k_pe[idx].copy(),
    )


def verify_step(w: Workload, q_len: int, seed: int = 1):
    """Inputs of a speculative-decoding verify step over workload w.

    Returns (q, new_slots, new_latent, new_k_pe): q uint16 bf16 bits [B, q_len, H, 576],
    N(0, 1) rounded to bf16; the slots of the last q_len positions of every request
    (ascending, unique) with the workload's own rows for them, which the step writes into
    the cache before attending.  Query i of request b sits at position L_b - q_len + i.
    """
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng.standard_normal((w.batch, q_len, w.heads, ROW), dtype=np.float32))
    new = []
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for t in range(max(0, L - q_len), L):
            new.append(int(w.block_table[b, t // w.page_size]) * w.page_size + t % w.page_size)
    new_slots = np.unique(np.asarray(new, dtype=np.int64))
    idx = np.searchsorted(w.slots, new_slots)
    return q, new_slots, w.latent[idx].copy(), w.k_pe[idx].copy()


def sparse_lists(w: Workload, topk: int, seed: int = 2) -> np.ndarray:
    """Per-query index lists for a sparse decode step over workload w: int32 [B, topk].

    Request b's list holds min(L_b, topk) distinct slots of its own context (token
    positions drawn uniformly without replacement, listed in random order, as an indexer's
    top-k would come), then -1 padding; an empty request's list is all -1.
    """
    rng = np.random.default_rng(seed)
    idx = np.full((w.batch, topk), -1, dtype=np.int32)
    ps = w.page_size
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        n = min(L, topk)
        if n == 0:
            continue
        t = rng.choice(L, size=n, replace=False)
        idx[b, :n] = w.block_table[b, t // ps].astype(np.int64) * ps + t % ps
    return idx


def _slots_of_pages(used_pages: np.ndarray, fill: np.ndarray, ps: int) -> np.ndarray:
    """Slots p*ps + [0, fill[p]) for every page p in used_pages, ascending."""
    if used_pages.size == 0:
        return np.zeros(0, dtype=np.int64)
    counts = fill[used_pages]
    starts = used_pages * ps
    total = int(counts.sum())
    rep_start = np.repeat(starts, counts)
    first = np.concatenate([[0], np.cumsum(counts)[:-1]])
    within = np.arange(total, dtype=np.int64) - np.repeat(first, counts)
    return rep_start + within


# --------------------------------------------------------------------------------------
# The named workloads.  Sizes follow the decode problem as the pages state it: H = 16
# heads of absorbed queries over 576-wide rows, pages of 64 slots, and the 64-bit
# addressing case above slot 2^31 / 576 (sabi-mla-vllm page, "B300 fix (0.2.0)").
# --------------------------------------------------------------------------------------

WRAP_SLOT = 2**31 // ROW  # 3,728,270: first slot whose int32 element offset overflows
FP8_WRAP_SLOT = 2**31 // 656  # 3,273,603: the same for the int32 byte offset of 656-byte rows


def tiny(seed: int = 0) -> Workload:
    """B=1, H=4, L=256, page 16, pool of 32 pages, pages = first 16 of a permutation."""
    return make_workload("tiny", seq_lens=[256], heads=4, page_size=16, num_pages=32, seed=seed)


def batched(seed: int = 0) -> Workload:
    """B=32, H=16, lengths uniform in [1024, 8192], page 64, pool of 2^21 slots."""
    return make_workload(
        "batched",
        seq_lens=lambda r: r.integers(1024, 8192, size=32, endpoint=True),
        heads=16, page_size=64, num_pages=(1 << 21) // 64, seed=seed)


def long_context(seed: int = 0) -> Workload:
    """B=4, H=16, every context 262,144 tokens, page 64, pool of 32,768 pages."""
    return make_workload(
        "long_context", seq_lens=[262144] * 4, heads=16, page_size=64,
        num_pages=32768, seed=seed)


HIGH_SLOT_POOL_PAGES = 70313  # 4,500,032 slots of 64, 5.18 GB of bf16 rows
HIGH_SLOT_FIRST_PAGE = -(-(WRAP_SLOT + 1) // 64)  # 58,255: first page wholly above the wrap slot


def high_slot(seed: int = 0) -> Workload:
    """4.5M-slot pool, B=64, lengths uniform in [19000, 76000], every page above the wrap slot.

    Only 12,058 pages of 64 lie above slot 3,728,270 while the batch needs about
    47.5k, so pages are distinct within a request and repeat across requests.
    """
    return make_workload(
        "high_slot",
        seq_lens=lambda r: r.integers(19000, 76000, size=64, endpoint=True),
        heads=16, page_size=64, num_pages=HIGH_SLOT_POOL_PAGES,
        page_range=(HIGH_SLOT_FIRST_PAGE, HIGH_SLOT_POOL_PAGES),
        pages_shared_across_requests=True, seed=seed)


def fp8_ragged_lengths(rng: np.random.Generator, batch: int = 48, max_len: int = 32768) -> np.ndarray:
    """Ragged lengths holding 0, 1, 17 and max_len; the rest uniform in [0, max_len]; shuffled."""
    fixed = np.array([0, 1, 17, max_len], dtype=np.int64)
    rest = rng.integers(0, max_len, size=batch - fixed.size, endpoint=True)
    lens = np.concatenate([fixed, rest])
    return lens[rng.permutation(lens.size)]


def fp8_ragged(seed: int = 0) -> Workload:
    """656-byte fp8 rows: B=48, H=16, ragged lengths incl. empty requests, page 64."""
    return make_workload(
        "fp8_ragged", seq_lens=fp8_ragged_lengths, heads=16, page_size=64,
        num_pages=32768, fmt="fp8", seed=seed)


NAMED = {
    "tiny": tiny,
    "batched": batched,
    "long_context": long_context,
    "high_slot": high_slot,
    "fp8_ragged": fp8_ragged,
}

# Partition counts the benchmark launches each named workload with.  The long-context
# workload uses 64 partitions per request (4 x 64 = 256 workgroups, one per compute
# unit); the others were picked by measurement (partitions are ceil(width / splits)
# pages, so a ragged batch has fewer non-empty partitions than batch x splits).
BENCH_SPLITS = {
    "tiny": 1,
    "batched": 8,
    "long_context": 64,
    "high_slot": 8,
    "fp8_ragged": 10,
}

# Workgroups of the batch-balanced decode in the bench's launch configuration (one per
# compute unit).
BENCH_BALANCED_WORKGROUPS = 256

# Schedule the benchmark times each named workload with, picked by measurement: per-request
# partitions for uniform or short contexts, batch-balanced ranges for long ragged batches.
BENCH_SCHEDULE = {
    "tiny": "per-request",
    "batched": "per-request",
    "long_context": "per-request",
    "high_slot": "balanced",
    "fp8_ragged": "balanced",
}

# Row-load policy of the decodes per named workload: streaming (non-temporal) loads
# where every row is read once per step; cached loads for the high-slot batch, whose requests
# share pages (12,058 pages above the wrap slot for about 47,500 page reads), so repeated rows
# can hit in the L2 and last-level cache.
# Sparse decode step of the benchmark (--op sparse): every request's newest token attends to
# SPARSE_TOPK slots of its own context (sparse_lists).  The pages do not give the list length;
# 2048 is the top-k of the published sparse-attention MLA models, used here as the reading.
SPARSE_TOPK = 2048
SPARSE_SPLITS = {"batched": 8, "long_context": 64, "high_slot": 4, "fp8_ragged": 5, "tiny": 1}

BENCH_ROW_LOADS = {
    "tiny": "streaming",
    "batched": "streaming",
    "long_context": "streaming",
    "high_slot": "cached",
    "fp8_ragged": "streaming",
}

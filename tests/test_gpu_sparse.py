"""Decode over per-query index lists (mla_decode_sparse_*) against the fp64 oracle on an MI355X.

vLLM pull request 55543 serves its NoPE-512 layers through a sparse backend that reads, for every
query token, the cache slots an indexer listed; its ragged mixed-batch test takes lists with 0, 1
and some valid entries followed by -1.  Here: lists with -1 tails and -1 entries anywhere, valid
counts 0, 1, partial and full, a repeated slot, list lengths with a ragged last tile, several
split counts, all four row forms (bf16 / fp8 656-byte rows, with and without the rotary part),
slots above 3,728,270 (where a 32-bit element offset of a 576-value row wraps) and every query of
the full-size sparse step the benchmark times.  Pools hold NaN (bf16) or 0xFF bytes (fp8) in
every slot no list names, so a stray read shows as a non-finite output.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_mla_latent_amd as mla
import workloads
from gpu_util import FMT_CODE, assert_parity, assert_rows_bitexact, bf16_dev, device_pool, device_rows, host_pool, say

pytestmark = pytest.mark.gpu

FNS = {("bf16", False): "mla_decode_sparse_bf16", ("fp8", False): "mla_decode_sparse_fp8_656",
       ("bf16", True): "mla_decode_sparse_nope_bf16", ("fp8", True): "mla_decode_sparse_nope_fp8_656"}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mla.library()
    yield
    torch.cuda.synchronize()


def _gpu(fmt, nope, q, pool, idx, scale, splits, check_status=None, flags=0):
    fn = getattr(mla, FNS[(fmt, nope)])
    out, lse = fn(bf16_dev(q), pool, torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda(), scale,
                  num_splits=splits, check_status=check_status, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _view(idx):
    """Stand-in for assert_parity: a query with no valid entry is an empty context."""
    counts = (np.asarray(idx) >= 0).sum(axis=1)
    return type("V", (), dict(batch=idx.shape[0], seq_lens=counts))


def _small_lists(w, topk, rng):
    """Lists over workload w's contexts: -1 tails, a list with -1 entries scattered through it, a
    repeated slot, and valid counts 0 / 1 / partial / full."""
    idx = workloads.sparse_lists(w, topk, seed=int(rng.integers(1 << 30)))
    full = np.nonzero((idx >= 0).sum(axis=1) == topk)[0]
    if full.size:
        b = int(full[0])
        holes = rng.choice(topk, size=topk // 3, replace=False)
        idx[b, holes] = -1  # -1 anywhere, not only at the tail
    if full.size > 1:
        b = int(full[1])
        idx[b, 5] = idx[b, 2]  # a slot listed twice counts twice
    return idx


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("nope", [False, True])
@pytest.mark.parametrize("heads", [16, 5])
def test_sparse_small(fmt, nope, heads):
    rng = np.random.default_rng(71 + heads)
    w = workloads.make_workload(f"sparse_{fmt}", seq_lens=[0, 1, 17, 300, 40, 700, 99, 1000], heads=heads,
                                page_size=16, num_pages=200, fmt=fmt, rng=rng)
    topk = 100  # six full tiles of 16 and a ragged tail of 4
    idx = _small_lists(w, topk, rng)
    counts = (idx >= 0).sum(axis=1)
    say(f"sparse small {fmt} nope={nope} H={heads} topk={topk} counts={counts.tolist()}")
    pd, ph = device_pool(w), host_pool(w)  # NoPE: the rope values are there but never read
    assert_rows_bitexact(w, pd, ph)
    q = np.ascontiguousarray(w.q[:, :, :512]) if nope else w.q
    ref_o, ref_l = oracle.decode_sparse(q, ph, idx, w.scale, fmt)
    for S in (1, 3, 7, 13):
        out, lse = _gpu(fmt, nope, q, pd, idx, w.scale, S)
        assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse {fmt} nope={nope} H={heads} S={S}")
    # partials left in the workspace, merged by mla_merge_lse: the same result bit for bit
    fn = getattr(mla, FNS[(fmt, nope)])
    args = (bf16_dev(q), pd, torch.from_numpy(idx).cuda(), w.scale)
    po, pl = fn(*args, num_splits=7, partials_only=True)
    o2, l2 = mla.mla_merge_lse(po, pl)
    o1, l1 = fn(*args, num_splits=7)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_sparse_list_length_edges(fmt):
    """topk 1, 15, 16, 17 and lists whose valid entries all sit in one partition of several."""
    rng = np.random.default_rng(81)
    w = workloads.make_workload(f"sparse_edges_{fmt}", seq_lens=[50, 3, 0, 64], heads=16, page_size=8,
                                num_pages=40, fmt=fmt, rng=rng)
    pd, ph = device_pool(w), host_pool(w)
    for topk in (1, 15, 16, 17, 64):
        idx = workloads.sparse_lists(w, topk, seed=topk)
        ref_o, ref_l = oracle.decode_sparse(w.q, ph, idx, w.scale, fmt)
        for S in (1, 2, 5):
            out, lse = _gpu(fmt, False, w.q, pd, idx, w.scale, S)
            assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse {fmt} topk={topk} S={S}")
    # valid entries only in the last partition: every other partition selects nothing
    idx = np.full((w.batch, 64), -1, np.int32)
    idx[:, 60:] = workloads.sparse_lists(w, 4, seed=9)
    ref_o, ref_l = oracle.decode_sparse(w.q, ph, idx, w.scale, fmt)
    out, lse = _gpu(fmt, False, w.q, pd, idx, w.scale, 4)
    assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse {fmt} last partition only")
    # the largest split count the boundary admits (one query, 2.2 GB of partials): one entry per
    # partition, the rest empty
    idx = workloads.sparse_lists(w, 17, seed=17)[:1]
    q1 = np.ascontiguousarray(w.q[:1])
    ref_o, ref_l = oracle.decode_sparse(q1, ph, idx, w.scale, fmt)
    out, lse = _gpu(fmt, False, q1, pd, idx, w.scale, 65535)
    assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse {fmt} S=65535")


# Slots around the places where narrower offsets would wrap, and the pool's last slots.
def _high_slots(num_slots):
    marks = [workloads.WRAP_SLOT, workloads.FP8_WRAP_SLOT, 2**32 // 1152, 2**32 // 656, num_slots - 40]
    near = np.concatenate([np.arange(m - 40, m + 40) for m in marks] + [np.arange(0, 40)])
    return np.unique(near[(near >= 0) & (near < num_slots)]).astype(np.int64)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_sparse_slots_above_the_wrap(fmt):
    """A 4.5M-slot pool (5.18 GB of bf16 rows, 2.95 GB of fp8 rows) with rows only around slot
    3,728,270 (and the other 32-bit wrap points) and at its end; the oracle decodes the same rows
    from a compact copy (the lists renumbered into it)."""
    rng = np.random.default_rng(91)
    num_slots = workloads.HIGH_SLOT_POOL_PAGES * 64
    slots = _high_slots(num_slots)
    n = slots.size
    lat = workloads.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    pe = workloads.bf16_bits(rng.standard_normal((n, 64)).astype(np.float32))
    if fmt == "bf16":
        pool = torch.full((num_slots // 64, 64, 576), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        pool = torch.full((num_slots // 64, 64, 656), 0xFF, dtype=torch.uint8, device="cuda")
    mla.mla_cache_write(bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots).cuda(), pool, FMT_CODE[fmt])
    compact = np.zeros((n, workloads.ROW_BYTES[fmt]), np.uint8)
    oracle.cache_write(compact, lat, pe, np.arange(n), fmt)
    got = device_rows(pool, slots, workloads.ROW_BYTES[fmt])
    assert np.array_equal(got, compact), "rows written above the wrap differ"
    T, H, topk = 12, 16, 256
    idx = np.full((T, topk), -1, np.int64)
    for t in range(T):
        k = [0, 1, 37, topk][t % 4]
        idx[t, :k] = rng.choice(slots, size=k, replace=False)
    idx[3, :8] = workloads.WRAP_SLOT + np.arange(8)  # the wrap slot and the first slots past it
    q = workloads.bf16_bits(rng.standard_normal((T, H, 576)).astype(np.float32))
    local = np.where(idx >= 0, np.searchsorted(slots, idx), -1)
    scale = workloads.DEFAULT_SCALE
    say(f"sparse high slots {fmt}: {n} rows, max slot {slots.max()}, T={T} topk={topk}")
    ref_o, ref_l = oracle.decode_sparse(q, compact, local, scale, fmt)
    for S in (1, 4):
        out, lse = _gpu(fmt, False, q, pool, idx.astype(np.int32), scale, S)
        assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse high slots {fmt} S={S}")
    del pool
    torch.cuda.empty_cache()


def _device_pool_for_lists(w, idx):
    """The workload's pool on the device with only the listed slots written (the rest poisoned)."""
    used = np.unique(idx[idx >= 0]).astype(np.int64)
    rows = np.searchsorted(w.slots, used)
    assert np.array_equal(w.slots[rows], used)
    if w.fmt == "bf16":
        pool = torch.full((w.num_pages, w.page_size, 576), 0x7FC0, dtype=torch.int16, device="cuda").view(
            torch.bfloat16)
    else:
        pool = torch.full((w.num_pages, w.page_size, 656), 0xFF, dtype=torch.uint8, device="cuda")
    mla.mla_cache_write(bf16_dev(w.latent[rows]), bf16_dev(w.k_pe[rows]), torch.from_numpy(used).cuda(), pool,
                        FMT_CODE[w.fmt])
    compact = np.zeros((used.size, w.row_bytes), np.uint8)
    oracle.cache_write(compact, w.latent[rows], w.k_pe[rows], np.arange(used.size), w.fmt)
    local = np.where(idx >= 0, np.searchsorted(used, idx), -1)
    return pool, compact, local


@pytest.mark.parametrize("name", ["high_slot", "fp8_ragged"])
def test_sparse_full_size_every_query(name):
    """The benchmark's sparse step at full size (every request's newest token over SPARSE_TOPK
    slots of its context, the bench's split count), every query against the oracle."""
    w = workloads.NAMED[name]()
    idx = workloads.sparse_lists(w, workloads.SPARSE_TOPK)
    S = workloads.SPARSE_SPLITS[name]
    say(f"sparse full size {name}: B={w.batch} topk={workloads.SPARSE_TOPK} S={S}")
    pool, compact, local = _device_pool_for_lists(w, idx)
    ref_o, ref_l = oracle.decode_sparse(w.q, compact, local, w.scale, w.fmt)
    flags = mla.MLA_FLAG_CACHED_ROWS if workloads.BENCH_ROW_LOADS[name] == "cached" else 0
    out, lse = _gpu(w.fmt, False, w.q, pool, idx, w.scale, S, flags=flags)
    assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse full {name} S={S}")
    nq = np.ascontiguousarray(w.q[:, :, :512])
    ref_o, ref_l = oracle.decode_sparse(nq, compact, local, w.scale, w.fmt)
    out, lse = _gpu(w.fmt, True, nq, pool, idx, w.scale, S, flags=flags)
    assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse full {name} NoPE S={S}")
    del pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_sparse_checked_build(fmt):
    """Checked build: an entry >= num_slots reads slot 0 instead and sets MLA_CHECK_BLOCK_ID;
    negative entries are not a broken precondition.  The pool the kernel sees is a prefix of a
    larger allocation holding valid rows, so a missed check gives a wrong result, never a fault."""
    rng = np.random.default_rng(101)
    view_slots, total = 300, 400
    lat = workloads.bf16_bits(rng.standard_normal((total, 512)).astype(np.float32))
    pe = workloads.bf16_bits(rng.standard_normal((total, 64)).astype(np.float32))
    R = workloads.ROW_BYTES[fmt]
    if fmt == "bf16":
        big = torch.empty((total, 1, 576), dtype=torch.bfloat16, device="cuda")
    else:
        big = torch.empty((total, 1, 656), dtype=torch.uint8, device="cuda")
    mla.mla_cache_write(bf16_dev(lat), bf16_dev(pe), torch.arange(total, dtype=torch.int64, device="cuda"), big,
                        FMT_CODE[fmt])
    host = np.zeros((total, R), np.uint8)
    oracle.cache_write(host, lat, pe, np.arange(total), fmt)
    pool = big[:view_slots]
    T, topk = 6, 40
    idx = np.stack([rng.choice(view_slots, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    idx[1, 20:] = -1
    idx[2, 3] = view_slots + 7     # outside the pool: read as slot 0
    idx[4, 39] = view_slots + 60
    q = workloads.bf16_bits(rng.standard_normal((T, 16, 576)).astype(np.float32))
    scale = workloads.DEFAULT_SCALE
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"sparse checked {fmt}")
    out, lse = _gpu(fmt, False, q, pool, idx, scale, 3, check_status=st)
    assert st.item() == mla.MLA_CHECK_BLOCK_ID
    eff = idx.copy()
    eff[eff >= view_slots] = 0
    ref_o, ref_l = oracle.decode_sparse(q, host[:view_slots], eff, scale, fmt)
    assert_parity(_view(idx), out, lse, ref_o, ref_l, what=f"sparse checked {fmt}")
    ok = idx.copy()
    ok[ok >= view_slots] = -1
    st.zero_()
    _gpu(fmt, False, q, pool, ok, scale, 3, check_status=st)
    assert st.item() == 0

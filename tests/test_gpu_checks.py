"""The checked build (libmla_checked.so) on an MI355X: precondition tests inside the kernels.

A wrong block-table offset reads the wrong memory and then faults (sabi-mla-vllm, "B300 fix
(0.2.0)": correct first token, then garbage, then an illegal memory access).  The checked build's
kernels test every block id a context uses against num_pages and every length against
block_table_stride * page_size before forming an address: a block id outside the pool reads page
0 instead, a length past the table is clamped to it, and the failed test's MLA_CHECK_* bit is
ORed into the caller's status word.

Every case here runs on memory laid out so that no read could leave an allocation even if a test
inside a kernel were missing: the pool the kernel sees is a view into a larger allocation with
guard pages on both sides (holding poison before it and valid rows after it), and the block
table is a view of a larger table whose extra row holds valid page ids.  A missed check then
shows up as a wrong or non-finite result, never as a fault.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_mla_latent_amd as mla
import workloads
from gpu_util import FMT_CODE, assert_parity, bf16_dev, say

pytestmark = pytest.mark.gpu

GUARD = 10  # guard pages before and after the pool view


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    mla.library(checked=True)
    yield
    torch.cuda.synchronize()


def _full_rows(w, seed=77):
    """Rows for every slot of the workload's pool (so that page 0 and every page hold finite rows)."""
    rng = np.random.default_rng(seed)
    slots = np.arange(w.num_slots, dtype=np.int64)
    bits = workloads.bf16_bits(rng.standard_normal((w.num_slots, 576)).astype(np.float32))
    have = np.searchsorted(slots, w.slots)
    bits[have, :512], bits[have, 512:] = w.latent, w.k_pe  # the workload's own rows where it has them
    return slots, bits[:, :512].copy(), bits[:, 512:].copy()


class Guarded:
    """A pool of w.num_pages pages with GUARD poisoned pages before it and GUARD pages of valid
    rows after it; the kernels see pool[:view_pages] (view_pages < w.num_pages puts the last
    pages of the workload beyond the view, inside the allocation)."""

    def __init__(self, w, view_pages):
        self.w = w
        slots, lat, pe = _full_rows(w)
        ps, R = w.page_size, w.row_bytes
        total = GUARD + w.num_pages + GUARD
        if w.fmt == "bf16":
            big = torch.full((total, ps, 576), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        else:
            big = torch.full((total, ps, 656), 0xFF, dtype=torch.uint8, device="cuda")
        mla.mla_cache_write(bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots + GUARD * ps).cuda(), big,
                            FMT_CODE[w.fmt])
        # pages after the workload's: valid rows too (copies of its first pages)
        big[GUARD + w.num_pages:] = big[GUARD:GUARD + GUARD]
        self.big = big
        self.pool = big[GUARD:GUARD + view_pages]
        self.host = w.poisoned_pool()
        oracle.cache_write(self.host, lat, pe, slots, w.fmt)
        self.view_pages = view_pages


def _tables(w, bt_np):
    """Device block table as a view of one with an extra row of valid page ids after it."""
    B, W = bt_np.shape
    big = np.zeros((B + 1, W), np.int32)
    big[:B] = bt_np
    dev = torch.from_numpy(big).cuda()
    return dev[:B]


def _effective(w, bt_np, lens_np, view_pages):
    """What the checked kernels compute with: block ids outside the view -> 0, lengths clamped."""
    W = bt_np.shape[1]
    lens = np.clip(lens_np.astype(np.int64), 0, W * w.page_size).astype(np.int32)
    bt = bt_np.copy()
    for b in range(w.batch):
        used = -(-int(lens[b]) // w.page_size)
        row = bt[b, :used]
        row[(row < 0) | (row >= view_pages)] = 0
    return bt, lens


def _case(fmt, seed=3):
    w = workloads.make_workload(f"checked_{fmt}", seq_lens=[300, 77, 500, 0, 33], heads=16, page_size=16,
                                num_pages=72, fmt=fmt, seed=seed)
    g = Guarded(w, view_pages=48)
    bt = w.block_table.copy()
    lens = w.seq_lens.copy()
    bt[1, 1] = -3                       # inside request 1's context: a negative id
    lens[2] = bt.shape[1] * w.page_size + 9  # past the table: clamped to the table
    return w, g, bt, lens


def _expected(w, g, bt, lens, q=None):
    bt_eff, lens_eff = _effective(w, bt, lens, g.view_pages)
    q = w.q if q is None else q
    return oracle.decode(q, g.host, bt_eff, lens_eff, w.page_size, w.scale, w.fmt), lens_eff


def _status():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 4])
def test_checked_decode_flags_and_contains_bad_ids(fmt, splits):
    w, g, bt, lens = _case(fmt)
    say(f"checked decode {fmt} splits={splits}")
    assert mla.mla_check_preconditions_host(bt, lens, w.page_size, g.view_pages) == 3
    fn = mla.mla_decode_bf16 if fmt == "bf16" else mla.mla_decode_fp8_656
    st = _status()
    out, lse = fn(bf16_dev(w.q), g.pool, _tables(w, bt), torch.from_numpy(lens).cuda(), w.scale, num_splits=splits,
                  check_status=st)
    torch.cuda.synchronize()
    assert st.item() == mla.MLA_CHECK_BLOCK_ID | mla.MLA_CHECK_SEQ_LEN
    (ro, rl), lens_eff = _expected(w, g, bt, lens)
    view = type("V", (), dict(batch=w.batch, seq_lens=lens_eff))
    assert_parity(view, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                  what=f"checked {fmt} S={splits}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_checked_balanced_and_verify_step(fmt):
    w, g, bt, lens = _case(fmt, seed=4)
    say(f"checked balanced / verify {fmt}")
    bt_d, lens_d = _tables(w, bt), torch.from_numpy(lens).cuda()
    fn = mla.mla_decode_balanced_bf16 if fmt == "bf16" else mla.mla_decode_balanced_fp8_656
    st = _status()
    out, lse = fn(bf16_dev(w.q), g.pool, bt_d, lens_d, w.scale, num_workgroups=64, check_status=st)
    torch.cuda.synchronize()
    assert st.item() == 3
    (ro, rl), lens_eff = _expected(w, g, bt, lens)
    view = type("V", (), dict(batch=w.batch, seq_lens=lens_eff))
    assert_parity(view, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                  what=f"checked balanced {fmt}")
    # verify step, 4 query tokens x 16 heads (four row groups)
    q4 = workloads.bf16_bits(np.random.default_rng(5).standard_normal((w.batch, 4, 16, 576)).astype(np.float32))
    fn = mla.mla_decode_mtp_bf16 if fmt == "bf16" else mla.mla_decode_mtp_fp8_656
    st = _status()
    out, lse = fn(bf16_dev(q4), g.pool, bt_d, lens_d, w.scale, num_splits=2, check_status=st)
    torch.cuda.synchronize()
    assert st.item() == 3
    bt_eff, lens_eff = _effective(w, bt, lens, g.view_pages)
    ro, rl = oracle.decode_mtp(q4, g.host, bt_eff, lens_eff, w.page_size, w.scale, w.fmt)
    o, l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    for i in range(4):
        li = np.maximum(0, lens_eff - 3 + i)
        view = type("V", (), dict(batch=w.batch, seq_lens=li))
        assert_parity(view, o[:, i], l[:, i], ro[:, i], rl[:, i], what=f"checked verify {fmt} query {i}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_checked_build_matches_release_on_valid_inputs(fmt):
    w = workloads.make_workload(f"valid_{fmt}", seq_lens=[900, 0, 17, 64], heads=16, page_size=16, num_pages=70,
                                fmt=fmt, seed=8)
    pool = torch.full((w.num_pages, 16, 576), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16) \
        if fmt == "bf16" else torch.full((w.num_pages, 16, 656), 0xFF, dtype=torch.uint8, device="cuda")
    mla.mla_cache_write(bf16_dev(w.latent), bf16_dev(w.k_pe), torch.from_numpy(w.slots).cuda(), pool, FMT_CODE[fmt])
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    fn = mla.mla_decode_bf16 if fmt == "bf16" else mla.mla_decode_fp8_656
    for splits in (1, 3):
        a = fn(bf16_dev(w.q), pool, bt, lens, w.scale, num_splits=splits)
        st = _status()
        b = fn(bf16_dev(w.q), pool, bt, lens, w.scale, num_splits=splits, check_status=st)
        torch.cuda.synchronize()
        assert st.item() == 0
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_checked_gather():
    fmt = "fp8"
    w, g, bt, lens = _case(fmt, seed=6)
    say("checked gather")
    starts = np.array([0, 0, bt.shape[1] * w.page_size - 5, 0, 10], np.int32)
    rows = np.array([300, 77, 12, 0, 20], np.int64)   # request 2: 5 rows inside the table, 7 past it
    cu = np.concatenate([[0], np.cumsum(rows)])
    st = _status()
    out = mla.mla_gather_context(g.pool, FMT_CODE[fmt], _tables(w, bt), torch.from_numpy(cu).cuda(), int(cu[-1]),
                                 seq_starts=torch.from_numpy(starts).cuda(), check_status=st)
    torch.cuda.synchronize()
    assert st.item() == 3
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bt_eff = bt.copy()
    bt_eff[(bt_eff < 0) | (bt_eff >= g.view_pages)] = 0
    keep = cu.copy()
    inside = np.minimum(rows, np.maximum(0, bt.shape[1] * w.page_size - starts))
    # rows inside the table: the oracle's gather with the substituted ids; rows past it: zeros
    for b in range(w.batch):
        cub = np.array([0, inside[b]])
        want = oracle.gather_context(g.host, bt_eff[b:b + 1], cub, starts[b:b + 1], w.page_size, fmt)
        assert np.array_equal(got[keep[b]:keep[b] + inside[b]], want), f"request {b}"
        assert (got[keep[b] + inside[b]:keep[b + 1]] == 0).all(), f"request {b}: rows past the table"

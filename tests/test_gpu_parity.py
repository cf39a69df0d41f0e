"""Parity of the HIP path (through the C ABI) with the fp64 oracle on an MI355X.

Each case: seeded workload -> rows written by mla_cache_write on the device and by
oracle.cache_write on the host -> row bytes compared bit for bit -> each side decodes
its own pool -> per (request, head) max |out - ref| <= 1e-2 * max |ref| and
|lse - ref_lse| <= 1e-3; empty contexts give exactly (+0, -inf).  Pools are filled
with NaN (bf16) or 0xFF bytes (fp8) wherever no request reads, so a stray read
shows up as a non-finite output.
"""
import types

import numpy as np
import pytest
import torch

import oracle
import paged_mla_latent_amd as mla
import workloads
from gpu_util import (FMT_CODE, assert_parity, assert_rows_bitexact, bf16_dev, device_pool, device_rows,
                      gpu_decode, host_pool, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    mla.library()
    yield
    torch.cuda.synchronize()


def _run_case(w, splits_list, requests=None, what="", balanced=()):
    say(f"case {what or w.name}: fmt={w.fmt} B={w.batch} H={w.heads} ps={w.page_size} "
        f"pages={w.num_pages} tokens={w.tokens} splits={splits_list} balanced={list(balanced)}")
    pd = device_pool(w)
    ph = host_pool(w)
    assert_rows_bitexact(w, pd, ph)
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt,
                                 requests=requests)
    for S in splits_list:
        out, lse = gpu_decode(w, pd, S)
        assert_parity(w, out, lse, ref_o, ref_l, requests, what=f"{what or w.name} S={S}")
    for W in balanced:
        out, lse = gpu_decode(w, pd, W, balanced=True)
        assert_parity(w, out, lse, ref_o, ref_l, requests, what=f"{what or w.name} balanced W={W}")
    return pd, ph


# ------------------------------------------------------------------------ small cases
@pytest.mark.parametrize("splits", [1, 2, 16])
def test_tiny_workload(splits):
    w = workloads.tiny()
    pd, ph = _run_case(w, [splits])
    got = pd.view(torch.uint8).cpu().numpy().reshape(-1)
    assert np.array_equal(got, ph.reshape(-1))  # whole pool, poison included


RAGGED = [0, 1, 15, 16, 17, 100, 333, 1000, 2500]


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("ps", [1, 3, 16, 24, 64, 784])
def test_ragged_lengths_and_page_sizes(fmt, ps):
    pages = sum(-(-L // ps) for L in RAGGED) + 7
    w = workloads.make_workload(f"ragged_ps{ps}", seq_lens=RAGGED, heads=16, page_size=ps, num_pages=pages,
                                fmt=fmt, seed=ps)
    # 9 x 40 workgroups exceed the compute units: the non-empty partitions are dispatched first
    _run_case(w, [1, 3, 40])


@pytest.mark.parametrize("heads", [1, 3, 8, 16])
def test_head_counts(heads):
    w = workloads.make_workload(f"heads{heads}", seq_lens=[700, 33, 1], heads=heads, page_size=64, num_pages=40,
                                seed=heads)
    _run_case(w, [1, 2])


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_row_magnitude_spread(fmt):
    """Row scales log-uniform over four decades, odd page size, shuffled pages."""
    w = workloads.make_workload("spread", seq_lens=[3000, 1500, 784, 785], heads=16, page_size=784, num_pages=16,
                                fmt=fmt, seed=21, row_scale_log10=(-2.0, 2.0))
    _run_case(w, [1, 4])


def test_split_count_invariance():
    w = workloads.make_workload("splits", seq_lens=[5000, 4097, 64, 0], heads=16, page_size=64, num_pages=200,
                                seed=5)
    _run_case(w, [1, 2, 7, 64, 200])


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_largest_split_count(fmt):
    """num_splits = 65,535, the largest the boundary admits, on a short batch: all but a few
    partitions are empty, the grid (2 x 65,535) is compacted, and the library's counted merge and
    the caller's merge of all 131,070 kept partials (every empty one written as (0, -inf)) both
    match the oracle."""
    S = 65535
    w = workloads.make_workload("max_splits", seq_lens=[1000, 0], heads=1, page_size=16, num_pages=80, fmt=fmt,
                                seed=8)
    pd, ph = device_pool(w), host_pool(w)
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt)
    out, lse = gpu_decode(w, pd, S)
    assert_parity(w, out, lse, ref_o, ref_l, what=f"{fmt} S={S}")
    fn = mla.mla_decode_bf16 if fmt == "bf16" else mla.mla_decode_fp8_656
    part_o, part_l = fn(bf16_dev(w.q), pd, torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(),
                        w.scale, num_splits=S, partials_only=True)
    po, pl = mla.mla_merge_lse(part_o, part_l)
    torch.cuda.synchronize()
    assert_parity(w, po.cpu().numpy().astype(np.float64), pl.cpu().numpy().astype(np.float64), ref_o, ref_l,
                  what=f"{fmt} S={S} partials merged by the caller")


def test_empty_and_single_token_requests():
    for fmt in ("bf16", "fp8"):
        w = workloads.make_workload("empties", seq_lens=[0, 0, 1, 2, 0], heads=16, page_size=16, num_pages=4,
                                    fmt=fmt, seed=2)
        _run_case(w, [1, 4])


def test_garbage_rope_control_on_gpu():
    """q_pe = 0: random rope bytes leave the output bit-identical; q_pe != 0 changes it."""
    w = workloads.make_workload("rope", seq_lens=[300, 77], heads=16, page_size=16, num_pages=30, seed=9)
    other = workloads.bf16_bits(np.random.default_rng(1).standard_normal(w.k_pe.shape).astype(np.float32) * 30)
    q0 = w.q.copy()
    q0[:, :, 512:] = 0
    pa = device_pool(w)
    pb = device_pool(w, k_pe=other)
    a = gpu_decode(w, pa, 1, q=q0)
    b = gpu_decode(w, pb, 1, q=q0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = gpu_decode(w, pa, 1)
    d = gpu_decode(w, pb, 1)
    assert np.abs(c[1] - d[1]).max() > 1e-3


# ------------------------------------------------------------------------ cache write
def _special_latent(rng, T):
    """bf16 latent rows with blocks that stress the fp8 quantiser."""
    x = rng.standard_normal((T, 512)).astype(np.float32)
    x[0] = 0.0
    x[1, :128] = -0.0
    x[1, 128:256] = np.float32(1e-38)  # bf16 subnormal-range values
    x[1, 256:384] = np.float32(3e38)   # near the top of the bf16 range
    ties = np.array([448.0, 1.0625, 1.1875, -1.0625, 0.0, -0.0, 2**-10, 3 * 2**-10, -448.0], np.float32)
    x[2, :ties.size] = ties
    x[2, ties.size:128] = 1.0
    x[3] *= np.float32(10.0) ** rng.uniform(-30, 30, size=512).astype(np.float32)
    x[4, ::2] = 0.0
    return workloads.bf16_bits(x)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_cache_write_bitexact(fmt):
    rng = np.random.default_rng(3)
    T = 300
    latent = _special_latent(rng, T)
    k_pe = rng.integers(0, 1 << 16, size=(T, 64), dtype=np.uint16)
    k_pe[(k_pe & 0x7F80) == 0x7F80] = 0x1234  # keep rope values finite
    R = oracle.ROW_BYTES[fmt]
    pool = (torch.full((8, 64, 576), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16) if fmt == "bf16"
            else torch.full((8, 64, 656), 0xFF, dtype=torch.uint8, device="cuda"))
    slots = rng.permutation(8 * 64)[:T].astype(np.int64)
    slots[5] = -1  # skipped
    mla.mla_cache_write(bf16_dev(latent), bf16_dev(k_pe), torch.from_numpy(slots).cuda(), pool, FMT_CODE[fmt])
    torch.cuda.synchronize()
    host = (np.full((8, 64, 576), 0x7FC0, np.uint16).view(np.uint8) if fmt == "bf16"
            else np.full((8, 64, 656), 0xFF, np.uint8)).reshape(-1, R)
    oracle.cache_write(host, latent, k_pe, slots, fmt)
    got = pool.view(torch.uint8).cpu().numpy().reshape(-1, R)
    bad = np.nonzero((got != host).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ; first slot {bad[0]}"


def _fp8_pool_write(latent, k_pe, rows):
    pool = torch.full((rows, 656), 0xAB, dtype=torch.uint8, device="cuda").view(rows, 1, 656)
    mla.mla_cache_write(bf16_dev(latent), bf16_dev(k_pe), torch.arange(rows, dtype=torch.int64, device="cuda"), pool,
                        mla.MLA_CACHE_FP8_656)
    torch.cuda.synchronize()
    return pool.view(rows, 656).cpu().numpy()


def _exhaustive_blocks(values, block_max):
    """Blocks of 128 bf16 patterns: 127 of `values` each plus one `block_max` (the block's absmax)."""
    per = 127
    n = -(-values.size // per)
    vals = np.concatenate([values, np.zeros(n * per - values.size, np.uint16)]).reshape(n, per)
    blocks = np.concatenate([np.full((n, 1), block_max, np.uint16), vals], axis=1)
    blocks = np.concatenate([blocks, np.zeros((-n % 4, 128), np.uint16)])  # whole rows of four blocks
    return blocks.reshape(-1, 512)


@pytest.mark.parametrize("block_max", [0x43E0, 0x447A, 0x4040])  # 448 (s = 1), 1000, 3 (s = 3/448)
def test_cache_write_fp8_exhaustive_bf16(block_max):
    """Every finite bf16 value x with |x| <= the block max, in blocks whose absmax is 448 (scale
    1), 1000 or 3 (scales 1000/448 and 3/448), quantised by mla_cache_write: bytes equal the
    oracle's packing bit for bit (the hardware e4m3 conversion's rounding, ties and subnormals)."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mag = workloads.bf16_as_f32(pats)
    lim = workloads.bf16_as_f32(np.array([block_max], np.uint16))[0]
    values = pats[np.isfinite(mag) & (np.abs(mag) <= lim)]
    latent = _exhaustive_blocks(values, block_max)
    say(f"exhaustive fp8 quantiser: {values.size} values, block max {lim}, {latent.shape[0]} rows")
    k_pe = np.zeros((latent.shape[0], 64), np.uint16)
    got = _fp8_pool_write(latent, k_pe, latent.shape[0])
    want = oracle.pack_rows(latent, k_pe, "fp8")
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first row {bad[0]}"


def test_cache_write_fp8_nonfinite_blocks_and_decode():
    """A latent block holding a NaN or an infinity is stored as the NaN block (scale 0x7FC00000, codes
    0x7F), bit-exact against the oracle; a request reading such a row decodes to NaN, the others
    are unaffected."""
    rng = np.random.default_rng(12)
    T = 64
    lat = workloads.bf16_bits(rng.standard_normal((T, 512)).astype(np.float32))
    specials = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFC1, 0x7F81], np.uint16)  # NaN, +inf, -inf, NaNs
    for i, pat in enumerate(specials):
        lat[i, 130 * i % 512] = pat
    k_pe = workloads.bf16_bits(rng.standard_normal((T, 64)).astype(np.float32))
    got = _fp8_pool_write(lat, k_pe, T)
    want = oracle.pack_rows(lat, k_pe, "fp8")
    assert np.array_equal(got, want)
    blk = (130 * np.arange(specials.size) % 512) // 128
    for i in range(specials.size):
        assert got[i, 512 + 4 * blk[i]:516 + 4 * blk[i]].view("<u4")[0] == 0x7FC00000
    # decode: request 0 reads row 2 (an infinity), request 1 only finite rows
    w = workloads.make_workload("nanrow", seq_lens=[40, 40], heads=16, page_size=16, num_pages=6, fmt="fp8", seed=3)
    lat_w = w.latent.copy()
    lat_w[np.searchsorted(w.slots, oracle.slot_of(w.block_table, 0, 5, 16)), 300] = 0x7F80
    pd = device_pool(w, latent=lat_w)
    out, lse = gpu_decode(w, pd, 1)
    assert np.isnan(out[0]).all() and np.isnan(lse[0]).all()
    ph = host_pool(w, latent=lat_w)
    ro, rl = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, "fp8")
    assert np.isnan(ro[0]).all()
    assert_parity(w, out, lse, ro, rl, requests=[1], what="finite request beside a NaN row")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_compact_dispatch_keeps_every_partial(fmt):
    """batch x splits above the compute units with the partials kept (no merge here): the
    compacted dispatch must still write every partition's partial, the empty ones as (0, -inf);
    the workspace is poisoned first, and the caller's own merge is checked against the oracle."""
    lens = [0, 1, 15, 1000, 0, 2500, 333, 17, 0]
    ps = 16
    pages = sum(-(-L // ps) for L in lens) + 3
    w = workloads.make_workload("compact_kept", seq_lens=lens, heads=16, page_size=ps, num_pages=pages, fmt=fmt,
                                seed=14)
    S = 40  # 9 x 40 = 360 workgroups > 256 compute units
    pd, ph = device_pool(w), host_pool(w)
    need = mla.mla_decode_workspace_size(w.batch, w.heads, S)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    fn = mla.mla_decode_bf16 if fmt == "bf16" else mla.mla_decode_fp8_656
    po, pl = fn(bf16_dev(w.q), pd, torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(),
                w.scale, num_splits=S, workspace=ws, partials_only=True)
    out, lse = mla.mla_merge_lse(po, pl)
    torch.cuda.synchronize()
    pl_h = pl.cpu().numpy()
    assert not np.isnan(pl_h).any(), "a partition left its partial unwritten"
    # the empty partitions' partials are exactly (+0, -inf)
    W = w.block_table.shape[1]
    c = -(-W // S)
    for b, L in enumerate(lens):
        n = -(-(-(-L // ps)) // c)
        assert np.isneginf(pl_h[n:, b]).all()
        assert (po[n:, b].cpu().numpy() == 0).all()
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, fmt)
    assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                  what=f"compact kept {fmt}")


def test_balanced_default_workgroups_is_one_per_compute_unit():
    w = workloads.make_workload("bal0", seq_lens=[3000, 17, 0, 900], heads=16, page_size=64, num_pages=70, seed=15)
    pd = device_pool(w)
    q, bt, lens = bf16_dev(w.q), torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mla.mla_decode_balanced_workspace_size(w.batch, w.heads, 0) == \
        mla.mla_decode_balanced_workspace_size(w.batch, w.heads, cus)
    a = mla.mla_decode_balanced_bf16(q, pd, bt, lens, w.scale, num_workgroups=0)
    b = mla.mla_decode_balanced_bf16(q, pd, bt, lens, w.scale, num_workgroups=cus)
    ws = mla.mla_decode_balanced_bf16(q, pd, bt, lens, w.scale, num_workgroups=0, partials_only=True)
    c = mla.mla_merge_lse_balanced(ws, w.batch, w.heads, 0)
    torch.cuda.synchronize()
    for x in (b, c):
        assert torch.equal(a[0], x[0]) and torch.equal(a[1], x[1])


# ------------------------------------------------------------------------------ merge
def test_merge_kernel_matches_oracle():
    rng = np.random.default_rng(4)
    S, B, H = 37, 3, 16
    po = rng.standard_normal((S, B, H, 512)).astype(np.float32)
    pl = (rng.standard_normal((S, B, H)) * 5).astype(np.float32)
    pl[rng.random((S, B, H)) < 0.3] = -np.inf  # empty partitions
    pl[:, 1, 3] = -np.inf                       # a fully empty (request, head)
    out, lse = mla.mla_merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(out[1, 3], np.zeros(512)) and np.isneginf(lse[1, 3])
    assert np.allclose(out, ro, rtol=1e-5, atol=1e-5)
    fin = np.isfinite(rl)
    assert np.allclose(lse[fin], rl[fin], rtol=0, atol=1e-5)


def test_merge_kernel_propagates_nan():
    """NaN partials beside empty ones give NaN, not the empty result; all-empty stays (0, -inf)."""
    S, B, H = 300, 1, 4
    po = np.ones((S, B, H, 512), np.float32)
    pl = np.full((S, B, H), -np.inf, np.float32)
    pl[123, 0, 0] = np.nan                  # NaN among empties
    pl[:, 0, 1] = 1.0
    pl[299, 0, 1] = np.nan                  # NaN among finite partials
    pl[7, 0, 2] = 3.0                       # one finite partial
    out, lse = mla.mla_merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    for h in (0, 1):
        assert np.isnan(lse[0, h]) and np.isnan(out[0, h]).all() and np.isnan(rl[0, h])
    assert abs(lse[0, 2] - 3.0) < 1e-6 and np.allclose(out[0, 2], 1.0)
    assert np.isneginf(lse[0, 3]) and (out[0, 3] == 0).all() and not np.signbit(out[0, 3]).any()


# ----------------------------------------------------------------- 64-bit addressing
@pytest.mark.parametrize("fmt, num_pages", [("bf16", 60000), ("fp8", 110000)])
def test_pages_beyond_32bit_offsets(fmt, num_pages):
    """Requests on the page that straddles slot 3,728,270 (int32 element offsets of 576-value
    rows wrap there), on the page that straddles slot 3,273,603 (int32 byte offsets of 656-byte
    rows wrap there) and on pages past 2^32 bytes."""
    ps = 64
    straddle = workloads.WRAP_SLOT // ps  # holds slots 3,728,256 .. 3,728,319
    straddle8 = workloads.FP8_WRAP_SLOT // ps  # holds slots 3,273,600 .. 3,273,663
    top = num_pages - 1
    assert top * ps * oracle.ROW_BYTES[fmt] > 2**32
    layout = [[straddle, straddle + 1, 17, top], [top - 1, top - 2, straddle + 2], [3, straddle, straddle8], [top]]
    lens = [4 * ps - 5, 3 * ps, 3 * ps - 7, 40]
    rng = np.random.default_rng(8)
    w = workloads.make_workload(f"wrap_{fmt}", seq_lens=lens, heads=16, page_size=ps, num_pages=num_pages,
                                fmt=fmt, seed=8)
    # Re-place the pages by hand (keeping the generated rows' slot order): rows follow slots, so
    # regenerate the workload's slot list from the new block table.
    bt = np.full_like(w.block_table, -1)
    for b, pages in enumerate(layout):
        bt[b, :len(pages)] = pages
    fill = {}
    for b, pages in enumerate(layout):
        for j, pg in enumerate(pages):
            n = min(ps, lens[b] - j * ps)
            fill[pg] = max(fill.get(pg, 0), n)
    slots = np.concatenate([pg * ps + np.arange(n) for pg, n in sorted(fill.items())]).astype(np.int64)
    T = slots.size
    lat = workloads.bf16_bits(rng.standard_normal((T, 512)).astype(np.float32))
    pe = workloads.bf16_bits(rng.standard_normal((T, 64)).astype(np.float32))
    w.block_table, w.slots, w.latent, w.k_pe = bt, slots, lat, pe
    assert any(s // ps == straddle for s in slots) and slots.max() * oracle.ROW_BYTES[fmt] > 2**32
    # both sides of the 656-byte rows' int32 byte-offset wrap are read
    assert any(s * 656 < 2**31 for s in slots if s // ps == straddle8)
    assert any(2**31 <= s * 656 < 2**32 for s in slots if s // ps == straddle8)
    say(f"case wrap_{fmt}: max slot {slots.max()} byte offset {slots.max() * oracle.ROW_BYTES[fmt]}")
    # teeth: an int32 element offset would land elsewhere for these slots
    assert any(oracle.element_offset_int32(int(s)) != oracle.element_offset(int(s)) for s in slots)
    _run_case(w, [1, 2], what=f"wrap_{fmt}")


# ------------------------------------------------------------------- full-size cases
def _sample(w, n=4):
    rng = np.random.default_rng(0)
    picks = {0, w.batch // 2, w.batch - 1}
    picks.update(rng.choice(w.batch, size=min(n, w.batch), replace=False).tolist())
    return sorted(picks)


# ------------------------------------------------------------------- batch-balanced mode
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("ps", [1, 3, 16, 24, 64])
def test_balanced_ragged(fmt, ps):
    """Workgroup ranges cut requests mid-page (at multiples of 16 tokens), cover several
    requests, or hold no token at all (W close to or above the token count).  Page size 24
    puts tiles across page boundaries (fp8 rows: fetched row by row)."""
    pages = sum(-(-L // ps) for L in RAGGED) + 7
    w = workloads.make_workload(f"bal_ps{ps}", seq_lens=RAGGED, heads=16, page_size=ps, num_pages=pages,
                                fmt=fmt, seed=40 + ps)
    # cost axis: 3,982 tokens + 8 non-empty requests x 512 = 8,078 positions
    _run_case(w, [], balanced=[1, 2, 7, 64, 256, 1000, 8077, 8078, 9000])


@pytest.mark.parametrize("heads", [1, 3, 16])
def test_balanced_heads_and_empties(heads):
    for fmt in ("bf16", "fp8"):
        w = workloads.make_workload("bal_empties", seq_lens=[0, 0, 1, 2, 0, 33, 0], heads=heads, page_size=16,
                                    num_pages=8, fmt=fmt, seed=3)
        # cost axis: 36 tokens + 3 x 512 = 1,572 positions; most ranges hold start-up only
        _run_case(w, [], balanced=[1, 3, 4, 36, 512, 1571, 1572, 2000])


def test_balanced_max_batch():
    """MLA_MAX_BALANCED_BATCH requests, short ragged lengths, many requests per workgroup."""
    lens = np.random.default_rng(11).integers(0, 40, size=mla.MLA_MAX_BALANCED_BATCH)
    pages = int(sum(-(-int(L) // 16) for L in lens)) + 3
    w = workloads.make_workload("bal_max", seq_lens=lens.tolist(), heads=4, page_size=16, num_pages=pages,
                                fmt="fp8", seed=12)
    _run_case(w, [], balanced=[1, 97, 256, 5000])


def test_balanced_all_empty():
    w = workloads.make_workload("bal_none", seq_lens=[0, 0, 0], heads=16, page_size=16, num_pages=2, seed=4)
    _run_case(w, [], balanced=[1, 256])


def test_balanced_matches_per_request_mode():
    """Same cache, two schedules: both within the bar of each other's reference."""
    w = workloads.make_workload("bal_vs", seq_lens=[5000, 4097, 64, 0, 1, 3000], heads=16, page_size=64,
                                num_pages=220, seed=6)
    _run_case(w, [1, 64], balanced=[256, 1024])


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_context_parallel_shares_merge(fmt):
    """Decode context parallelism rehearsed on one device: each request's pages are dealt out
    to 8 disjoint shares (as 8 devices would hold them), every share is decoded on its own with
    its partials kept (out = lse = NULL), and one mla_merge_lse over all shares' partials gives
    the whole requests' results (the partial-result merge contract of vLLM pull request 55543)."""
    ps, G, S = 64, 8, 4
    w = workloads.make_workload("cp_shares", seq_lens=[4096, 3000, 64, 0, 700], heads=16, page_size=ps,
                                num_pages=200, fmt=fmt, seed=31)
    pd, ph = device_pool(w), host_pool(w)
    q = bf16_dev(w.q)
    fn = mla.mla_decode_bf16 if fmt == "bf16" else mla.mla_decode_fp8_656
    parts_o, parts_l = [], []
    for share in range(G):
        # share g holds pages g, g + 8, ... of every request (a strided deal, so every share
        # sees every request's context spread out; a request shorter than the deal leaves
        # some shares empty)
        bt = np.zeros((w.batch, w.block_table.shape[1]), dtype=np.int32)
        lens = np.zeros(w.batch, dtype=np.int32)
        for b in range(w.batch):
            n_pages = -(-int(w.seq_lens[b]) // ps)
            mine = list(range(share, n_pages, G))
            bt[b, :len(mine)] = w.block_table[b, mine]
            last_full = n_pages - 1
            lens[b] = sum(ps if pg < last_full else int(w.seq_lens[b]) - ps * last_full for pg in mine)
        po, pl = fn(q, pd, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), w.scale, num_splits=S,
                    partials_only=True)
        parts_o.append(po.clone())
        parts_l.append(pl.clone())
    out, lse = mla.mla_merge_lse(torch.cat(parts_o), torch.cat(parts_l))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, ps, w.scale, fmt)
    assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                  what=f"context-parallel shares {fmt}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_balanced_partials_then_merge(fmt):
    """Decode with out == lse == NULL, then mla_merge_lse_balanced: bit-identical to one call."""
    w = workloads.make_workload("bal_two_step", seq_lens=[3000, 0, 17, 900, 64], heads=16, page_size=16,
                                num_pages=260, fmt=fmt, seed=8)
    pd = device_pool(w)
    q, bt, lens = bf16_dev(w.q), torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    fn = mla.mla_decode_balanced_bf16 if fmt == "bf16" else mla.mla_decode_balanced_fp8_656
    out1, lse1 = fn(q, pd, bt, lens, w.scale, num_workgroups=100)
    ws = fn(q, pd, bt, lens, w.scale, num_workgroups=100, partials_only=True)
    out2, lse2 = mla.mla_merge_lse_balanced(ws, w.batch, w.heads, 100)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("name", ["batched", "fp8_ragged", "high_slot"])
def test_balanced_full_size_sampled(name):
    """The named workloads at full size, batch-balanced with the bench's workgroup count."""
    w = workloads.NAMED[name]()
    W = workloads.BENCH_BALANCED_WORKGROUPS
    req = _sample(w)
    say(f"case {name} balanced: fmt={w.fmt} B={w.batch} tokens={w.tokens} W={W} oracle requests={req}")
    pd = device_pool(w)
    out, lse = gpu_decode(w, pd, W, balanced=True)
    live = w.seq_lens > 0
    assert np.isfinite(out[live]).all() and np.isfinite(lse[live]).all()
    assert np.isneginf(lse[~live]).all() and (out[~live] == 0).all() and not np.signbit(out[~live]).any()
    idx = np.searchsorted(w.slots, np.unique(np.concatenate([_request_slots(w, b) for b in req])))
    ph = w.poisoned_pool()
    ph.reshape(-1, w.row_bytes)[w.slots[idx]] = oracle.pack_rows(w.latent[idx], w.k_pe[idx], w.fmt)
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=req)
    assert_parity(w, out, lse, ref_o, ref_l, requests=req, what=f"{name} balanced W={W}")


def _request_slots(w, b):
    t = np.arange(int(w.seq_lens[b]), dtype=np.int64)
    return w.block_table[b].astype(np.int64)[t // w.page_size] * w.page_size + t % w.page_size


def _oracle_pool(w):
    """Host pool with every row of the workload packed by the oracle (in chunks)."""
    ph = w.poisoned_pool()
    for c in range(0, w.slots.size, 1 << 16):
        sl = slice(c, c + (1 << 16))
        oracle.cache_write(ph, w.latent[sl], w.k_pe[sl], w.slots[sl], w.fmt)
    return ph


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["batched", "fp8_ragged", "high_slot"])
def test_full_size_every_request(name):
    """Every request of the full-size ragged workloads, in the bench's schedule and split count,
    against the oracle decoding a pool of its own packing.  high_slot's requests share pages
    (a page read for the wrong request would still give finite values), so the sampled checks
    elsewhere are not enough there."""
    import time
    w = workloads.NAMED[name]()
    balanced = workloads.BENCH_SCHEDULE[name] == "balanced"
    S = workloads.BENCH_BALANCED_WORKGROUPS if balanced else workloads.BENCH_SPLITS[name]
    say(f"case {name} every request: fmt={w.fmt} B={w.batch} tokens={w.tokens} "
        f"{'balanced W' if balanced else 'splits'}={S}")
    flags = mla.MLA_FLAG_CACHED_ROWS if workloads.BENCH_ROW_LOADS[name] == "cached" else 0
    pd = device_pool(w)
    out, lse = gpu_decode(w, pd, S, balanced=balanced, flags=flags)
    del pd
    t = time.perf_counter()
    ph = _oracle_pool(w)
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt)
    say(f"  oracle: {time.perf_counter() - t:.1f} s")
    assert_parity(w, out, lse, ref_o, ref_l, what=f"{name} every request")


@pytest.mark.parametrize("name", ["batched", "long_context", "high_slot", "fp8_ragged"])
def test_full_size_workloads_sampled(name):
    """The named workloads at full size in the bench's launch configuration.

    Every row is written by mla_cache_write; the rows of the sampled requests plus 20,000
    random slots are compared bit for bit with the oracle's packing, and the oracle
    decodes the sampled requests from a host pool holding its own packing of their rows.
    """
    w = workloads.NAMED[name]()
    S = workloads.BENCH_SPLITS[name]
    req = _sample(w)
    say(f"case {name}: fmt={w.fmt} B={w.batch} tokens={w.tokens} splits={S} oracle requests={req}")
    pd = device_pool(w)
    out, lse = gpu_decode(w, pd, S)
    live = w.seq_lens > 0
    assert np.isfinite(out[live]).all() and np.isfinite(lse[live]).all()  # no stray read of a poisoned slot
    assert np.isneginf(lse[~live]).all() and (out[~live] == 0).all() and not np.signbit(out[~live]).any()
    rng = np.random.default_rng(1)
    req_slots = np.unique(np.concatenate([_request_slots(w, b) for b in req]))
    idx = np.unique(np.concatenate([np.searchsorted(w.slots, req_slots),
                                    rng.choice(w.slots.size, size=min(20000, w.slots.size), replace=False)]))
    assert np.array_equal(w.slots[np.searchsorted(w.slots, req_slots)], req_slots)
    want = oracle.pack_rows(w.latent[idx], w.k_pe[idx], w.fmt)
    got = device_rows(pd, w.slots[idx], w.row_bytes)
    assert np.array_equal(got, want), "cache rows differ"
    ph = w.poisoned_pool()
    ph.reshape(-1, w.row_bytes)[w.slots[idx]] = want
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=req)
    assert_parity(w, out, lse, ref_o, ref_l, requests=req, what=f"{name} S={S}")


# ---------------------------------------------------------------- multi-token verify
def _gpu_mtp(w, pool, q_bits, splits, balanced=False, flags=0):
    """Per-request split verify step (num_splits = splits), or the batch-balanced one with
    splits workgroups."""
    bt = torch.from_numpy(w.block_table).cuda()
    lens = torch.from_numpy(w.seq_lens).cuda()
    if balanced:
        fn = mla.mla_decode_mtp_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_balanced_fp8_656
        out, lse = fn(bf16_dev(q_bits), pool, bt, lens, w.scale, num_workgroups=splits, flags=flags)
    else:
        fn = mla.mla_decode_mtp_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_fp8_656
        out, lse = fn(bf16_dev(q_bits), pool, bt, lens, w.scale, num_splits=splits, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _assert_mtp_parity(w, out, lse, ref_o, ref_l, T, what, requests=None):
    """Per (request, query) the usual bar; queries that see no token give exactly (+0, -inf)."""
    requests = range(w.batch) if requests is None else requests
    for i in range(T):
        lens_i = np.maximum(0, w.seq_lens - T + 1 + i)
        view = types.SimpleNamespace(batch=w.batch, seq_lens=lens_i)
        assert_parity(view, out[:, i], lse[:, i], ref_o[:, i], ref_l[:, i], requests, what=f"{what} query {i}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("T, H", [(1, 16), (2, 16), (3, 16), (4, 16), (4, 4), (5, 3), (16, 4)])
def test_mtp_parity(fmt, T, H):
    lens = [0, 1, T - 1, T, T + 1, 17, 64, 65, 500, 2047, 3000]
    ps = 24 if T % 2 else 16  # 24: tiles that cross page boundaries
    pages = sum(-(-L // ps) for L in lens) + 4
    w = workloads.make_workload(f"mtp{T}x{H}", seq_lens=[max(0, L) for L in lens], heads=H, page_size=ps,
                                num_pages=pages, fmt=fmt, seed=70 + 4 * T + H)
    q = workloads.bf16_bits(np.random.default_rng(T * 100 + H).standard_normal((w.batch, T, H, 576))
                            .astype(np.float32))
    say(f"case mtp fmt={fmt} q_len={T} heads={H} rows={T * H}")
    pd, ph = device_pool(w), host_pool(w)
    ref_o, ref_l = oracle.decode_mtp(q, ph, w.block_table, w.seq_lens, ps, w.scale, fmt)
    for S in (1, 4, 16, 30):  # 11 x 30 workgroups: compacted dispatch
        out, lse = _gpu_mtp(w, pd, q, S)
        _assert_mtp_parity(w, out, lse, ref_o, ref_l, T, what=f"mtp {fmt} T={T} H={H} S={S}")
    # batch-balanced: a cost axis of 5,697-5,742 tokens + 9 or 10 non-empty requests x 512
    # (10,305-10,862 positions), cut into ranges that meet many requests, split one mid-page,
    # or hold start-up only
    for W in (1, 5, 64, 256, 10305, 12000):
        out, lse = _gpu_mtp(w, pd, q, W, balanced=True)
        _assert_mtp_parity(w, out, lse, ref_o, ref_l, T, what=f"mtp balanced {fmt} T={T} H={H} W={W}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_mtp_balanced_partials_then_merge(fmt):
    """Balanced verify step with out == lse == NULL, then mla_merge_lse_balanced over the
    q_len x heads query rows: bit-identical to one call."""
    T, H = 3, 16
    w = workloads.make_workload("mtp_bal_two_step", seq_lens=[3000, 0, 17, 900, 2], heads=H, page_size=16,
                                num_pages=260, fmt=fmt, seed=9)
    q = workloads.bf16_bits(np.random.default_rng(19).standard_normal((w.batch, T, H, 576)).astype(np.float32))
    pd = device_pool(w)
    qd, bt, lens = bf16_dev(q), torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    fn = mla.mla_decode_mtp_balanced_bf16 if fmt == "bf16" else mla.mla_decode_mtp_balanced_fp8_656
    out1, lse1 = fn(qd, pd, bt, lens, w.scale, num_workgroups=100)
    ws = fn(qd, pd, bt, lens, w.scale, num_workgroups=100, partials_only=True)
    out2, lse2 = mla.mla_merge_lse_balanced(ws, w.batch, T * H, 100)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(w.batch, T * H, -1), out2) and torch.equal(lse1.view(w.batch, T * H), lse2)


def test_mtp_balanced_matches_per_request_mode():
    """One cache, two schedules of the same verify step: each within the bar of the oracle."""
    T, H = 4, 16
    w = workloads.make_workload("mtp_bal_vs", seq_lens=[5000, 4097, 64, 0, 1, 3000], heads=H, page_size=64,
                                num_pages=220, fmt="fp8", seed=16)
    q = workloads.bf16_bits(np.random.default_rng(23).standard_normal((w.batch, T, H, 576)).astype(np.float32))
    pd, ph = device_pool(w), host_pool(w)
    ref_o, ref_l = oracle.decode_mtp(q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt)
    for S, bal in ((8, False), (256, True)):
        out, lse = _gpu_mtp(w, pd, q, S, balanced=bal)
        _assert_mtp_parity(w, out, lse, ref_o, ref_l, T, what=f"mtp fp8 {'W' if bal else 'S'}={S}")


def test_mtp_balanced_full_size_fp8_ragged_sampled():
    """Four verify tokens per request over the fp8 ragged batch, batch-balanced with the bench's
    workgroup count; the oracle checks the first, a middle and the last non-empty request."""
    w = workloads.NAMED["fp8_ragged"]()
    W, T = workloads.BENCH_BALANCED_WORKGROUPS, 4
    q = workloads.bf16_bits(np.random.default_rng(8).standard_normal((w.batch, T, w.heads, 576)).astype(np.float32))
    live = np.flatnonzero(w.seq_lens > 0)
    req = sorted({int(live[0]), int(live[len(live) // 2]), int(live[-1])})
    say(f"case mtp fp8_ragged balanced: q_len={T} W={W} oracle requests={req}")
    pd = device_pool(w)
    out, lse = _gpu_mtp(w, pd, q, W, balanced=True)
    seen = w.seq_lens[:, None] - T + 1 + np.arange(T)[None, :] > 0
    assert np.isfinite(out[seen]).all() and np.isfinite(lse[seen]).all()
    assert np.isneginf(lse[~seen]).all() and (out[~seen] == 0).all()
    ph = w.poisoned_pool()
    idx = np.unique(np.searchsorted(w.slots, np.concatenate([_request_slots(w, b) for b in req])))
    ph.reshape(-1, w.row_bytes)[w.slots[idx]] = oracle.pack_rows(w.latent[idx], w.k_pe[idx], w.fmt)
    ref_o, ref_l = oracle.decode_mtp(q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=req)
    _assert_mtp_parity(w, out, lse, ref_o, ref_l, T, what=f"mtp fp8_ragged balanced W={W}", requests=req)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_row_load_policies_agree(fmt):
    """Streaming (non-temporal) and cached row loads give bit-identical results, per-request,
    batch-balanced, verify-step and NoPE; the streaming result is checked against the oracle."""
    w = workloads.make_workload("row_loads", seq_lens=[3000, 0, 17, 900, 64, 1], heads=16, page_size=16,
                                num_pages=260, fmt=fmt, seed=21)
    q4 = workloads.bf16_bits(np.random.default_rng(29).standard_normal((w.batch, 4, 16, 576)).astype(np.float32))
    pd, ph = device_pool(w), host_pool(w)
    runs = {}
    for flags in (0, mla.MLA_FLAG_CACHED_ROWS):  # per call: streaming, then cached row loads
        runs[flags] = [gpu_decode(w, pd, 4, flags=flags), gpu_decode(w, pd, 64, balanced=True, flags=flags),
                       gpu_decode(w, pd, 4, nope=True, flags=flags), _gpu_mtp(w, pd, q4, 4, flags=flags),
                       _gpu_mtp(w, pd, q4, 64, True, flags=flags)]
    for a, b in zip(runs[0], runs[mla.MLA_FLAG_CACHED_ROWS]):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt)
    assert_parity(w, *runs[0][0], ref_o, ref_l, what="streaming loads S=4")


def test_calls_in_flight_on_two_streams_do_not_interfere():
    """The library keeps no state between calls: decodes in flight at once on two streams, with
    different formats, row-load flags, split counts, schedules and workspaces, give the bits that
    each gives alone."""
    wa = workloads.make_workload("streams_a", seq_lens=[3000, 17, 0, 1200], heads=16, page_size=64, num_pages=120,
                                 fmt="bf16", seed=31)
    wb = workloads.make_workload("streams_b", seq_lens=[900, 2500, 1], heads=8, page_size=16, num_pages=400,
                                 fmt="fp8", seed=32)
    pa, pb = device_pool(wa), device_pool(wb)
    qa, qb = bf16_dev(wa.q), bf16_dev(wb.q)
    bta, btb = torch.from_numpy(wa.block_table).cuda(), torch.from_numpy(wb.block_table).cuda()
    la, lb = torch.from_numpy(wa.seq_lens).cuda(), torch.from_numpy(wb.seq_lens).cuda()

    def call_a():
        return mla.mla_decode_bf16(qa, pa, bta, la, wa.scale, num_splits=8)

    def call_b():
        return mla.mla_decode_balanced_fp8_656(qb, pb, btb, lb, wb.scale, num_workgroups=64,
                                               flags=mla.MLA_FLAG_CACHED_ROWS)

    alone_a, alone_b = call_a(), call_b()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    runs = []
    for _ in range(4):
        with torch.cuda.stream(sa):
            ra = call_a()
        with torch.cuda.stream(sb):
            rb = call_b()
        runs.append((ra, rb))
    torch.cuda.synchronize()
    for ra, rb in runs:
        for x, y in zip(ra + rb, alone_a + alone_b):
            assert torch.equal(x, y)
    ref_o, ref_l = oracle.decode(wa.q, host_pool(wa), wa.block_table, wa.seq_lens, wa.page_size, wa.scale, "bf16")
    assert_parity(wa, alone_a[0].cpu().numpy().astype(np.float64), alone_a[1].cpu().numpy().astype(np.float64),
                  ref_o, ref_l, what="two streams, bf16")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_step_replays_from_a_hip_graph(fmt):
    """The calls enqueue kernels only (no allocation when the buffers are given, no
    synchronisation, no memset): a decode step (cache write, split decode with the library's own
    merge) captured in a HIP graph gives the eager bits on every replay, with eager work between
    the replays, and follows its inputs when they change in place."""
    w = workloads.make_workload("graph_step", seq_lens=[2000, 0, 513, 64], heads=16, page_size=64, num_pages=80,
                                fmt=fmt, seed=41)
    pd = device_pool(w)
    # the step rewrites each live request's newest row (same values) at its slot
    newest = [int(w.block_table[b, (L - 1) // w.page_size]) * w.page_size + (L - 1) % w.page_size
              for b, L in enumerate(w.seq_lens) if L > 0]
    last = np.array([np.nonzero(w.slots == sl)[0][0] for sl in newest])
    lat, pe, slots = bf16_dev(w.latent[last]), bf16_dev(w.k_pe[last]), torch.from_numpy(w.slots[last]).cuda()
    q = bf16_dev(w.q)
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    S = 8
    ws = torch.empty(mla.mla_decode_workspace_size(w.batch, w.heads, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")
    fn = mla.mla_decode_bf16 if fmt == "bf16" else mla.mla_decode_fp8_656

    def step():
        mla.mla_cache_write(lat, pe, slots, pd, FMT_CODE[fmt])
        fn(q, pd, bt, lens, w.scale, num_splits=S, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.fill_(7.0)  # eager work between the replays
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1])
    q.mul_(0.5)  # the inputs change in place: the replay reads them anew
    g.replay()
    torch.cuda.synchronize()
    got = (out.clone(), lse.clone())
    step()
    torch.cuda.synchronize()
    assert torch.equal(got[0], out) and torch.equal(got[1], lse)
    assert not torch.equal(got[1], eager[1])


def test_mtp_single_query_is_plain_decode():
    w = workloads.make_workload("mtp1", seq_lens=[3000, 5, 0, 777], heads=16, page_size=64, num_pages=70, seed=5)
    pd = device_pool(w)
    for S in (1, 7):
        a = _gpu_mtp(w, pd, w.q[:, None], S)
        b = gpu_decode(w, pd, S)
        assert np.array_equal(a[0][:, 0], b[0]) and np.array_equal(a[1][:, 0], b[1])


def test_mtp_full_size_long_context_sampled():
    """Four verify tokens per request over the long-context batch, at its bench split count."""
    w = workloads.NAMED["long_context"]()
    S = workloads.BENCH_SPLITS["long_context"]
    T = 4
    q = workloads.bf16_bits(np.random.default_rng(7).standard_normal((w.batch, T, w.heads, 576)).astype(np.float32))
    req = [0, w.batch - 1]
    say(f"case mtp long_context: q_len={T} splits={S} oracle requests={req}")
    pd = device_pool(w)
    out, lse = _gpu_mtp(w, pd, q, S)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    ph = w.poisoned_pool()
    idx = np.unique(np.searchsorted(w.slots, np.concatenate([_request_slots(w, b) for b in req])))
    ph.reshape(-1, w.row_bytes)[w.slots[idx]] = oracle.pack_rows(w.latent[idx], w.k_pe[idx], w.fmt)
    ref_o, ref_l = oracle.decode_mtp(q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=req)
    _assert_mtp_parity(w, out, lse, ref_o, ref_l, T, what=f"mtp long_context S={S}", requests=req)


# ------------------------------------------------------------------- context gather
def _gpu_gather(w, pool, cu, starts):
    out = mla.mla_gather_context(pool, FMT_CODE[w.fmt], torch.from_numpy(w.block_table).cuda(),
                                 torch.from_numpy(np.asarray(cu, np.int64)).cuda(), int(cu[-1]),
                                 None if starts is None else torch.from_numpy(np.asarray(starts, np.int32)).cuda())
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("ps", [1, 3, 16, 64])
def test_gather_parity(fmt, ps):
    """Random context windows of ragged requests, bit for bit against oracle.gather_context."""
    lens = [0, 1, 15, 17, 333, 2500, 64]
    pages = sum(-(-L // ps) for L in lens) + 3
    w = workloads.make_workload(f"gather_ps{ps}", seq_lens=lens, heads=1, page_size=ps, num_pages=pages, fmt=fmt,
                                seed=80 + ps)
    rng = np.random.default_rng(ps)
    starts = np.array([rng.integers(0, L + 1) for L in lens])
    counts = np.array([rng.integers(0, L - s + 1) for L, s in zip(lens, starts)])
    counts[-1] = lens[-1] - starts[-1]  # one window that runs to the end of its context
    cu = np.concatenate([[0], np.cumsum(counts)])
    say(f"case gather fmt={fmt} ps={ps} rows={cu[-1]}")
    pd, ph = device_pool(w), host_pool(w)
    got = _gpu_gather(w, pd, cu, starts)
    want = oracle.gather_context(ph, w.block_table, cu, starts, ps, fmt)
    assert got.shape == want.shape and np.array_equal(got, want)
    whole = np.concatenate([[0], np.cumsum(lens)])  # every token, seq_starts NULL
    assert np.array_equal(_gpu_gather(w, pd, whole, None), oracle.gather_context(ph, w.block_table, whole, None, ps, fmt))


@pytest.mark.parametrize("fmt, num_pages", [("bf16", 60000), ("fp8", 110000)])
def test_gather_beyond_32bit_offsets(fmt, num_pages):
    """Pages that straddle slot 3,728,270 and pages past 2^32 bytes, gathered whole."""
    ps = 64
    top, straddle = num_pages - 1, workloads.WRAP_SLOT // ps
    layout = [[straddle, top, 5], [top - 1, straddle + 1]]
    lens = [3 * ps - 9, 2 * ps]
    w = workloads.make_workload(f"gwrap_{fmt}", seq_lens=lens, heads=1, page_size=ps, num_pages=num_pages, fmt=fmt,
                                seed=9)
    bt = np.full_like(w.block_table, -1)
    for b, pg in enumerate(layout):
        bt[b, :len(pg)] = pg
    fill = {}
    for b, pg in enumerate(layout):
        for j, p in enumerate(pg):
            fill[p] = max(fill.get(p, 0), min(ps, lens[b] - j * ps))
    slots = np.concatenate([p * ps + np.arange(n) for p, n in sorted(fill.items())]).astype(np.int64)
    rng = np.random.default_rng(10)
    w.block_table, w.slots = bt, slots
    w.latent = workloads.bf16_bits(rng.standard_normal((slots.size, 512)).astype(np.float32))
    w.k_pe = workloads.bf16_bits(rng.standard_normal((slots.size, 64)).astype(np.float32))
    pd, ph = device_pool(w), host_pool(w)
    cu = np.concatenate([[0], np.cumsum(lens)])
    assert np.array_equal(_gpu_gather(w, pd, cu, None), oracle.gather_context(ph, bt, cu, None, ps, fmt))


def test_gather_full_size_fp8_ragged():
    """The whole fp8 ragged context (695,528 rows), upconverted; every row against the
    oracle's upconvert of the same cache bytes read back from the device."""
    w = workloads.NAMED["fp8_ragged"]()
    pd = device_pool(w)
    cu = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    say(f"case gather fp8_ragged: rows={cu[-1]}")
    got = _gpu_gather(w, pd, cu, None)
    slots = np.concatenate([_request_slots(w, b) for b in range(w.batch)])
    want = oracle.upconvert_rows(device_rows(pd, slots, w.row_bytes), "fp8")
    assert np.array_equal(got, want)


# ------------------------------------------------------------- other latent geometries
GEOM_LENS = [0, 1, 15, 17, 333, 2500]


@pytest.mark.parametrize("heads, ps", [(16, 64), (4, 3), (1, 16)])
def test_rank256_parity(heads, ps):
    """Rank-256 rows (320 bf16 values) placed on the device as generated; decode vs oracle.decode_rank."""
    pages = sum(-(-L // ps) for L in GEOM_LENS) + 3
    w = workloads.make_workload(f"r256_{heads}_{ps}", seq_lens=GEOM_LENS, heads=heads, page_size=ps, num_pages=pages,
                                seed=100 + heads + ps)
    rng = np.random.default_rng(heads * 7 + ps)
    pool = np.full((pages * ps, 320), 0x7FC0, np.uint16)
    pool[w.slots] = workloads.bf16_bits(rng.standard_normal((w.slots.size, 320)).astype(np.float32))
    q = workloads.bf16_bits(rng.standard_normal((w.batch, heads, 320)).astype(np.float32))
    ref_o, ref_l = oracle.decode_rank(q, pool, w.block_table, w.seq_lens, ps, w.scale)
    pd = bf16_dev(pool).view(pages, ps, 320)
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    for S in (1, 3):
        out, lse = mla.mla_decode_rank256_bf16(bf16_dev(q), pd, bt, lens, w.scale, num_splits=S)
        torch.cuda.synchronize()
        assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                      what=f"rank256 H={heads} ps={ps} S={S}")


@pytest.mark.parametrize("rank", [768, 1792])
@pytest.mark.parametrize("heads, ps", [(16, 64), (4, 3), (1, 16), (16, 1)])
def test_wide_rank_parity(rank, heads, ps):
    """Rank-768 / 1792 rows (D + 64 bf16 values); decode vs oracle.decode_rank, unsplit and split,
    and the partials left in the workspace merged by mla_merge_lse_width(D)."""
    K = rank + 64
    pages = sum(-(-L // ps) for L in GEOM_LENS) + 3
    w = workloads.make_workload(f"r{rank}_{heads}_{ps}", seq_lens=GEOM_LENS, heads=heads, page_size=ps,
                                num_pages=pages, seed=200 + heads + ps)
    rng = np.random.default_rng(rank + heads * 7 + ps)
    pool = np.full((pages * ps, K), 0x7FC0, np.uint16)
    pool[w.slots] = workloads.bf16_bits(rng.standard_normal((w.slots.size, K)).astype(np.float32))
    q = workloads.bf16_bits(rng.standard_normal((w.batch, heads, K)).astype(np.float32))
    ref_o, ref_l = oracle.decode_rank(q, pool, w.block_table, w.seq_lens, ps, w.scale)
    pd = bf16_dev(pool).view(pages, ps, K)
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    fn = mla.mla_decode_rank768_bf16 if rank == 768 else mla.mla_decode_rank1792_bf16
    for S in (1, 3, 40):
        out, lse = fn(bf16_dev(q), pd, bt, lens, w.scale, num_splits=S)
        torch.cuda.synchronize()
        assert out.shape == (w.batch, heads, rank)
        assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                      what=f"rank{rank} H={heads} ps={ps} S={S}")
    po, pl = fn(bf16_dev(q), pd, bt, lens, w.scale, num_splits=3, partials_only=True)
    out2, lse2 = mla.mla_merge_lse_width(po, pl)
    out3, lse3 = fn(bf16_dev(q), pd, bt, lens, w.scale, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(out2, out3) and torch.equal(lse2, lse3)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [2, 4, 16])
def test_gla2_parity(fmt, heads):
    """GLA-g2 on rows written by mla_cache_write; decode vs oracle.decode_gla2, and the
    256-wide partials merged by mla_merge_lse_width."""
    ps = 16
    pages = sum(-(-L // ps) for L in GEOM_LENS) + 3
    w = workloads.make_workload(f"gla2_{fmt}_{heads}", seq_lens=GEOM_LENS, heads=heads, page_size=ps,
                                num_pages=pages, fmt=fmt, seed=110 + heads)
    q = workloads.bf16_bits(np.random.default_rng(heads).standard_normal((w.batch, heads, 320)).astype(np.float32))
    pd, ph = device_pool(w), host_pool(w)
    ref_o, ref_l = oracle.decode_gla2(q, ph, w.block_table, w.seq_lens, ps, w.scale, fmt)
    fn = mla.mla_decode_gla2_bf16 if fmt == "bf16" else mla.mla_decode_gla2_fp8_656
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    for S in (1, 3):
        out, lse = fn(bf16_dev(q), pd, bt, lens, w.scale, num_splits=S)
        torch.cuda.synchronize()
        assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                      what=f"gla2 {fmt} H={heads} S={S}")
    po, pl = fn(bf16_dev(q), pd, bt, lens, w.scale, num_splits=5, partials_only=True)
    assert po.shape == (5, w.batch, heads, 256)
    out, lse = mla.mla_merge_lse_width(po, pl)
    torch.cuda.synchronize()
    assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                  what=f"gla2 {fmt} H={heads} partials + merge")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [2, 16])
def test_gla2_balanced_parity(fmt, heads):
    """GLA-g2 under the batch-balanced schedule on a ragged batch with empty requests, page sizes
    that cut tiles, and workgroup counts from one per request to many per request, against
    oracle.decode_gla2; bit-identical to itself across runs."""
    rng = np.random.default_rng(120 + heads)
    lens = [0, 1, 17, 700, 3000, 0, 64, 1500]
    for ps in (16, 24):
        pages = sum(-(-L // ps) for L in lens) + 3
        w = workloads.make_workload(f"gla2_bal_{fmt}_{heads}_{ps}", seq_lens=lens, heads=heads, page_size=ps,
                                    num_pages=pages, fmt=fmt, seed=130 + heads + ps)
        q = workloads.bf16_bits(rng.standard_normal((w.batch, heads, 320)).astype(np.float32))
        pd, ph = device_pool(w), host_pool(w)
        ref_o, ref_l = oracle.decode_gla2(q, ph, w.block_table, w.seq_lens, ps, w.scale, fmt)
        fn = mla.mla_decode_gla2_balanced_bf16 if fmt == "bf16" else mla.mla_decode_gla2_balanced_fp8_656
        bt, lens_d = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
        for W in (3, 16, 256):
            out, lse = fn(bf16_dev(q), pd, bt, lens_d, w.scale, num_workgroups=W)
            torch.cuda.synchronize()
            assert out.shape == (w.batch, heads, 256)
            assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o,
                          ref_l, what=f"gla2 balanced {fmt} H={heads} ps={ps} W={W}")
            again = fn(bf16_dev(q), pd, bt, lens_d, w.scale, num_workgroups=W)
            torch.cuda.synchronize()
            assert torch.equal(again[0], out) and torch.equal(again[1], lse)


# ------------------------------------------------------------------------- NoPE-512
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("ps", [3, 16, 24, 64])
def test_nope_parity(fmt, ps):
    """Zero-rope rows (k_pe NULL) bit for bit; NoPE decode against oracle.decode_nope."""
    lens = [0, 1, 15, 17, 333, 2500]
    pages = sum(-(-L // ps) for L in lens) + 5
    w = workloads.make_workload(f"nope_ps{ps}", seq_lens=lens, heads=16, page_size=ps, num_pages=pages, fmt=fmt,
                                seed=60 + ps)
    say(f"case nope fmt={fmt} ps={ps}")
    pd, ph = device_pool(w, zero_rope=True), host_pool(w, zero_rope=True)
    assert_rows_bitexact(w, pd, ph)
    q512 = np.ascontiguousarray(w.q[:, :, :512])
    ref_o, ref_l = oracle.decode_nope(q512, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt)
    for S in (1, 3):
        out, lse = gpu_decode(w, pd, S, nope=True)
        assert_parity(w, out, lse, ref_o, ref_l, what=f"nope {fmt} ps={ps} S={S}")
    for W in (1, 7, 256, 5000):  # batch-balanced NoPE
        out, lse = gpu_decode(w, pd, W, nope=True, balanced=True)
        assert_parity(w, out, lse, ref_o, ref_l, what=f"nope {fmt} ps={ps} balanced W={W}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_nope_never_reads_rope_bytes(fmt):
    """NaN in every rope value: NoPE decode gives the same bits as on zero rope, while the
    576-wide decode with q_pe = 0 turns NaN (zero-padding alone does not protect)."""
    w = workloads.make_workload("nope_nan", seq_lens=[700, 40], heads=16, page_size=16, num_pages=50, fmt=fmt,
                                seed=8)
    nan_pe = np.full(w.k_pe.shape, 0x7FC0, np.uint16)
    p0 = device_pool(w, zero_rope=True)
    pn = device_pool(w, k_pe=nan_pe)
    a = gpu_decode(w, p0, 2, nope=True)
    b = gpu_decode(w, pn, 2, nope=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q0 = w.q.copy()
    q0[:, :, 512:] = 0
    c = gpu_decode(w, p0, 2, q=q0)
    assert np.isfinite(c[1]).all()
    assert np.abs(c[1] - a[1]).max() < 1e-3  # same scores up to rounding when the rope is zero
    d = gpu_decode(w, pn, 2, q=q0)
    assert np.isnan(d[1]).all() and np.isnan(d[0]).all()  # as oracle.decode gives: every score NaN


@pytest.mark.parametrize("balanced", [False, True])
def test_nope_full_size_sampled(balanced):
    """The fp8 ragged workload as a NoPE layer, at its bench split count and batch-balanced."""
    w = workloads.NAMED["fp8_ragged"]()
    S = workloads.BENCH_BALANCED_WORKGROUPS if balanced else workloads.BENCH_SPLITS["fp8_ragged"]
    req = _sample(w)
    say(f"case nope fp8_ragged: B={w.batch} tokens={w.tokens} splits={S} balanced={balanced} oracle requests={req}")
    pd = device_pool(w, zero_rope=True)
    out, lse = gpu_decode(w, pd, S, nope=True, balanced=balanced)
    live = w.seq_lens > 0
    assert np.isfinite(out[live]).all() and np.isfinite(lse[live]).all()
    ph = w.poisoned_pool()
    idx = np.unique(np.searchsorted(w.slots, np.concatenate([_request_slots(w, b) for b in req])))
    ph.reshape(-1, w.row_bytes)[w.slots[idx]] = oracle.pack_rows(w.latent[idx], None, w.fmt)
    assert np.array_equal(device_rows(pd, w.slots[idx], w.row_bytes), ph.reshape(-1, w.row_bytes)[w.slots[idx]])
    q512 = np.ascontiguousarray(w.q[:, :, :512])
    ref_o, ref_l = oracle.decode_nope(q512, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt,
                                      requests=req)
    assert_parity(w, out, lse, ref_o, ref_l, requests=req, what=f"nope fp8_ragged S={S} balanced={balanced}")


def test_decode_is_bit_reproducible():
    """Fixed partitions and a fixed reduction order: two runs give identical bits."""
    w = workloads.make_workload("repro", seq_lens=[30000, 777], heads=16, page_size=64, num_pages=500, seed=6)
    pd = device_pool(w)
    a = gpu_decode(w, pd, 16)
    b = gpu_decode(w, pd, 16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_errors_reach_python_without_launch():
    w = workloads.tiny()
    pd = device_pool(w)
    q = bf16_dev(np.zeros((1, 17, 576), np.uint16))
    with pytest.raises(mla.MlaError, match="num_heads"):
        mla.mla_decode_bf16(q, pd, torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), 0.1)

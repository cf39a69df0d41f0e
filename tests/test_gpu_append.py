"""Decode steps that write their own new rows (mla_decode_append_*), against the two-call form.

Each case builds two device pools holding every context row except the step's new ones, whose
slots keep the NaN poison.  Pool B gets the new rows from mla_cache_write and is decoded by the
plain call (mla_decode_mtp_* / mla_decode_mtp_balanced_*); pool A is handed to the append call
with the same rows.  Pool A must end byte-identical to pool B (the rows are encoded as the cache
write encodes them; rows at negative positions are not written).  Per-request partitions: the
outputs must be bit-identical (the same partitions, the same bytes read).  Batch-balanced: the
append kernels charge every request a tokenless tail on the cost axis, so their ranges differ
from the plain call's; both outputs meet the oracle.  A read of a new row before its store would
return the poison and turn the output into NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_mla_latent_amd as mla
import workloads
from gpu_util import FMT_CODE, OUT_REL, LSE_ABS, bf16_dev, device_pool, say

pytestmark = pytest.mark.gpu


def _new_rows(w, T, free_slot):
    """Rows of positions L - T .. L - 1 of every request, [B, T, ...]; a negative position gets the
    (unused) slot free_slot, which the append call must leave alone, and zero rows."""
    B, ps = w.batch, w.page_size
    lat = np.zeros((B, T, 512), np.uint16)
    pe = np.zeros((B, T, 64), np.uint16)
    slots = np.full((B, T), free_slot, np.int64)
    for b in range(B):
        L = int(w.seq_lens[b])
        for i in range(T):
            P = L - T + i
            if P < 0:
                continue
            s = oracle.slot_of(w.block_table, b, P, ps)
            r = int(np.searchsorted(w.slots, s))
            assert w.slots[r] == s
            lat[b, i], pe[b, i], slots[b, i] = w.latent[r], w.k_pe[r], s
    return lat, pe, slots


def _req_slots(w, b):
    t = np.arange(int(w.seq_lens[b]), dtype=np.int64)
    return w.block_table[b].astype(np.int64)[t // w.page_size] * w.page_size + t % w.page_size


def _pools(w, slots_new):
    """Device pool without the new rows (their slots poisoned), twice."""
    keep = ~np.isin(w.slots, slots_new[slots_new >= 0])
    a = device_pool(w, latent=w.latent[keep], k_pe=w.k_pe[keep], slots=w.slots[keep])
    return a, a.clone()


def _run_case(w, T, q, balanced, count, free_slot):
    lat, pe, slots = _new_rows(w, T, free_slot)
    pa, pb = _pools(w, slots)
    qd, bt, lens = bf16_dev(q), torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    ld, ped, sd = bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots).cuda()
    # two-call form: the rows at non-negative positions only
    live = slots.reshape(-1) != free_slot
    mla.mla_cache_write(bf16_dev(lat.reshape(-1, 512)[live]), bf16_dev(pe.reshape(-1, 64)[live]),
                        torch.from_numpy(slots.reshape(-1)[live]).cuda(), pb, FMT_CODE[w.fmt])
    if balanced:
        plain = mla.mla_decode_mtp_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_balanced_fp8_656
        fused = mla.mla_decode_append_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_append_balanced_fp8_656
        ob, lb = plain(qd, pb, bt, lens, w.scale, num_workgroups=count)
        oa, la = fused(qd, ld, ped, sd, pa, bt, lens, w.scale, num_workgroups=count)
    else:
        plain = mla.mla_decode_mtp_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_fp8_656
        fused = mla.mla_decode_append_bf16 if w.fmt == "bf16" else mla.mla_decode_append_fp8_656
        ob, lb = plain(qd, pb, bt, lens, w.scale, num_splits=count)
        oa, la = fused(qd, ld, ped, sd, pa, bt, lens, w.scale, num_splits=count)
    torch.cuda.synchronize()
    if not balanced:
        assert torch.equal(oa, ob) and torch.equal(la, lb), "append call differs from cache write + decode"
    assert torch.equal(pa.view(torch.uint8), pb.view(torch.uint8)), "pools differ after the append call"
    return ((oa.cpu().numpy().astype(np.float64), la.cpu().numpy().astype(np.float64)),
            (ob.cpu().numpy().astype(np.float64), lb.cpu().numpy().astype(np.float64)))


def _oracle(w, q, requests=None):
    ph = w.poisoned_pool()
    oracle.cache_write(ph, w.latent, w.k_pe, w.slots, w.fmt)
    return oracle.decode_mtp(q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=requests)


def _oracle_check(w, T, ref, out, lse, what, requests=None):
    ref_o, ref_l = ref
    worst = 0.0
    for b in (range(w.batch) if requests is None else requests):
        for t in range(T):
            sees = int(w.seq_lens[b]) - T + 1 + t
            if sees <= 0:
                assert np.isneginf(lse[b, t]).all() and (out[b, t] == 0).all(), f"{what} b={b} t={t}"
                continue
            err = np.abs(out[b, t] - ref_o[b, t]).max(axis=1)
            scale = np.abs(ref_o[b, t]).max(axis=1)
            assert (err <= OUT_REL * scale).all(), f"{what} b={b} t={t}: out rel err {(err / scale).max():.3e}"
            assert (np.abs(lse[b, t] - ref_l[b, t]) <= LSE_ABS).all(), f"{what} b={b} t={t}: lse"
            worst = max(worst, float((err / scale).max()))
    say(f"  {what}: worst out rel err {worst:.2e}")


# Lengths: empty, shorter than q_len, 66 (with page size 16 and 3 partitions its last partition holds
# two tokens, so four new rows straddle a partition boundary), ragged others.
LENS = [3000, 0, 1, 66, 17, 700, 64, 1500]


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("T,H", [(1, 16), (2, 16), (4, 16), (8, 8)])
def test_append_matches_write_then_decode(fmt, T, H):
    w = workloads.make_workload(f"append_{fmt}_{T}", seq_lens=LENS, heads=H, page_size=16, num_pages=420, fmt=fmt,
                                seed=40 + T)
    free_slot = min(set(range(w.num_pages)) - set((w.slots // w.page_size).tolist())) * w.page_size + 3  # unused page
    q = workloads.bf16_bits(np.random.default_rng(50 + T).standard_normal((w.batch, T, H, 576)).astype(np.float32))
    ref = _oracle(w, q)
    for balanced, count in ((False, 1), (False, 3), (False, 16), (True, 3), (True, 64), (True, 256), (True, 12000)):
        what = f"append {fmt} T={T} H={H} {'W' if balanced else 'S'}={count}"
        say(f"case {what}")
        (out, lse), (out_b, lse_b) = _run_case(w, T, q, balanced, count, free_slot)
        if balanced or count == 3:
            _oracle_check(w, T, ref, out, lse, what)
        if balanced:
            _oracle_check(w, T, ref, out_b, lse_b, what + " (two calls)")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_append_balanced_partials_then_merge(fmt):
    """Balanced append call with out == lse == NULL, then mla_merge_lse_balanced: the one-call bits."""
    T, H, W = 2, 16, 40
    w = workloads.make_workload("append_two_step", seq_lens=[900, 0, 3, 2500], heads=H, page_size=64,
                                num_pages=80, fmt=fmt, seed=61)
    q = workloads.bf16_bits(np.random.default_rng(62).standard_normal((w.batch, T, H, 576)).astype(np.float32))
    lat, pe, slots = _new_rows(w, T, -1)
    fused = mla.mla_decode_append_balanced_bf16 if fmt == "bf16" else mla.mla_decode_append_balanced_fp8_656
    pa, _ = _pools(w, slots)
    pb = pa.clone()
    args = (bf16_dev(q), bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots).cuda())
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    o1, l1 = fused(*args, pa, bt, lens, w.scale, num_workgroups=W)
    ws = fused(*args, pb, bt, lens, w.scale, num_workgroups=W, partials_only=True)
    o2, l2 = mla.mla_merge_lse_balanced(ws, w.batch, T * H, W)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(w.batch, T * H, -1), o2) and torch.equal(l1.view(w.batch, T * H), l2)
    assert torch.equal(pa.view(torch.uint8), pb.view(torch.uint8))


@pytest.mark.parametrize("name,balanced,count", [("long_context", False, 64), ("fp8_ragged", True, 256)])
def test_append_full_size(name, balanced, count):
    """The bench's step configurations at full size: the pools agree on every new row; per request the
    append call gives the bits of cache write + decode, batch-balanced the oracle checks the first, a
    middle and the last non-empty request."""
    w = workloads.NAMED[name]()
    T = 1
    say(f"case append full size {name} {'W' if balanced else 'S'}={count}")
    q = w.q.reshape(w.batch, 1, w.heads, 576)
    lat, pe, slots = _new_rows(w, T, -1)
    pa, pb = _pools(w, slots)
    live = slots.reshape(-1) >= 0
    qd, bt, lens = bf16_dev(q), torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    mla.mla_cache_write(bf16_dev(lat.reshape(-1, 512)[live]), bf16_dev(pe.reshape(-1, 64)[live]),
                        torch.from_numpy(slots.reshape(-1)[live]).cuda(), pb, FMT_CODE[w.fmt])
    if balanced:
        plain = mla.mla_decode_mtp_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_balanced_fp8_656
        fused = mla.mla_decode_append_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_append_balanced_fp8_656
        ob, lb = plain(qd, pb, bt, lens, w.scale, num_workgroups=count)
        oa, la = fused(qd, bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots).cuda(), pa, bt, lens, w.scale,
                       num_workgroups=count)
    else:
        plain = mla.mla_decode_mtp_bf16 if w.fmt == "bf16" else mla.mla_decode_mtp_fp8_656
        fused = mla.mla_decode_append_bf16 if w.fmt == "bf16" else mla.mla_decode_append_fp8_656
        ob, lb = plain(qd, pb, bt, lens, w.scale, num_splits=count)
        oa, la = fused(qd, bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots).cuda(), pa, bt, lens, w.scale,
                       num_splits=count)
    torch.cuda.synchronize()
    if balanced:
        live_req = np.flatnonzero(w.seq_lens > 0)
        req = sorted({int(live_req[0]), int(live_req[len(live_req) // 2]), int(live_req[-1])})
        ph = w.poisoned_pool()
        idx = np.unique(np.concatenate([np.searchsorted(w.slots, _req_slots(w, b)) for b in req]))
        ph.reshape(-1, w.row_bytes)[w.slots[idx]] = oracle.pack_rows(w.latent[idx], w.k_pe[idx], w.fmt)
        ref = oracle.decode_mtp(q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, w.fmt, requests=req)
        _oracle_check(w, T, ref, oa.cpu().numpy().astype(np.float64), la.cpu().numpy().astype(np.float64),
                      f"append full size {name}", requests=req)
    else:
        assert torch.equal(oa, ob) and torch.equal(la, lb)
    R = w.row_bytes
    idx = torch.from_numpy(slots.reshape(-1)[live]).cuda()
    assert torch.equal(pa.view(torch.uint8).view(-1, R).index_select(0, idx),
                       pb.view(torch.uint8).view(-1, R).index_select(0, idx))
    seen = w.seq_lens > 0
    assert torch.isfinite(oa[torch.from_numpy(seen).cuda()]).all()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_append_step_replays_from_a_hip_graph(fmt):
    """A step of the append call (split decode writing its new rows, with the library's merge)
    captured in a HIP graph gives the eager bits on every replay, eager work between the replays;
    every replay rewrites the same rows."""
    T, H, S = 2, 16, 8
    w = workloads.make_workload("append_graph", seq_lens=[2000, 0, 513, 64], heads=H, page_size=64, num_pages=80,
                                fmt=fmt, seed=71)
    q = bf16_dev(workloads.bf16_bits(np.random.default_rng(72).standard_normal((w.batch, T, H, 576))
                                     .astype(np.float32)))
    lat, pe, slots = _new_rows(w, T, -1)
    pool, _ = _pools(w, slots)
    ld, ped, sd = bf16_dev(lat), bf16_dev(pe), torch.from_numpy(slots).cuda()
    bt, lens = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    ws = torch.empty(mla.mla_decode_workspace_size(w.batch, T * H, S), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, T, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, T, H), dtype=torch.float32, device="cuda")
    fn = mla.mla_decode_append_bf16 if fmt == "bf16" else mla.mla_decode_append_fp8_656

    def step():
        fn(q, ld, ped, sd, pool, bt, lens, w.scale, num_splits=S, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone(), pool.clone())
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
        assert torch.equal(pool.view(torch.uint8), eager[2].view(torch.uint8))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_checked_append_skips_slots_outside_the_pool(fmt):
    """Checked build: a new row whose slot lies outside [0, num_pages * page_size), or differs from
    the block table's slot for its position, is not written and sets MLA_CHECK_BLOCK_ID.  The pool
    the kernels see is a view into a larger allocation whose pages past the view stay poisoned, so a
    missing test would show up as a changed byte there, never as a fault; request 0 still meets the
    oracle."""
    T, H, guard = 1, 16, 4
    w = workloads.make_workload("append_checked", seq_lens=[300, 0, 17, 64], heads=H, page_size=16, num_pages=40,
                                fmt=fmt, seed=73)
    lat, pe, slots = _new_rows(w, T, -1)
    keep = ~np.isin(w.slots, slots[slots >= 0])
    width = 576 if fmt == "bf16" else 656
    if fmt == "bf16":
        big = torch.full((w.num_pages + guard, w.page_size, width), 0x7FC0, dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
    else:
        big = torch.full((w.num_pages + guard, w.page_size, width), 0xFF, dtype=torch.uint8, device="cuda")
    view = big[: w.num_pages]
    mla.mla_cache_write(bf16_dev(w.latent[keep]), bf16_dev(w.k_pe[keep]), torch.from_numpy(w.slots[keep]).cuda(),
                        view, FMT_CODE[fmt])
    torch.cuda.synchronize()
    guard_before = big[w.num_pages:].clone()
    bad = slots.copy()
    bad[2, 0] = w.num_pages * w.page_size + 5  # request 2's newest row: a slot in the first page past the view
    # request 3's newest row: a slot inside the pool but not the block table's for its position
    # (the row before it); it must stay as it is
    wrong = int(slots[3, 0]) - 1
    bad[3, 0] = wrong
    before_wrong = view.view(torch.uint8).reshape(-1, w.row_bytes)[wrong].clone()
    fn = mla.mla_decode_append_bf16 if fmt == "bf16" else mla.mla_decode_append_fp8_656
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = workloads.bf16_bits(np.random.default_rng(74).standard_normal((w.batch, T, H, 576)).astype(np.float32))
    out, lse = fn(bf16_dev(q), bf16_dev(lat), bf16_dev(pe), torch.from_numpy(bad).cuda(), view,
                  torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), w.scale,
                  num_splits=3, check_status=st)
    torch.cuda.synchronize()
    assert st.item() == mla.MLA_CHECK_BLOCK_ID
    assert torch.equal(big[w.num_pages:].view(torch.uint8), guard_before.view(torch.uint8)), "a row left the pool"
    assert torch.equal(view.view(torch.uint8).reshape(-1, w.row_bytes)[wrong], before_wrong), "a mismatched slot was written"
    ref = _oracle(w, q, requests=[0])
    _oracle_check(w, T, ref, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                  f"checked append {fmt}", requests=[0])

"""Pins of the fp64 oracle against things other than itself (CPU only).

Function                 pinned by
-----------------------  ------------------------------------------------------------
numerics.bf16_to_f64     torch's bfloat16 -> float64 cast over all 65,536 patterns
numerics.e4m3_decode     OCP E4M3 anchor values (golden); torch float8_e4m3fn, all codes
numerics.e4m3_encode     torch's float8_e4m3fn cast (round to nearest even) over every
                         bf16 value in [-464, 464] and 10^6 random fp32 values; round
                         trip on all finite codes; saturation above 448
numerics.quantize_block  hand-worked 656-byte row (golden); power-of-two round trip;
                         every NaN / infinity pattern gives the NaN block (stated rule)
mla.pack_rows/cache_write  hand-worked 656-byte row (golden); bf16 row = latent ++ k_pe
mla.slot_of/gather_rows  Python-int gather vs int64-array gather; page-move invariance
mla.element_offset*      wrap slot 3,728,270 printed on the sabi-mla-vllm page (golden)
mla.attend               closed forms (golden); pure-Python brute force (math.fsum);
                         1-token, uniform-score, duplication, hardmax, empty invariants;
                         a softmax-over-heads mistake planted in the oracle fails them
mla.decode               page-permutation invariance; garbage-rope control
mla.decode_sparse        pure-Python brute force over the listed rows (-1 anywhere, counts 0 / 1 /
                         partial, a repeated slot); equals the paged decode when a list enumerates
                         a request's slots; list order and -1 placement irrelevant; a -1 never
                         reads the pool's last row (a planted reading of it fails); NoPE-512
                         queries: brute force over the latent values, NaN rope ignored
mla.decode_mtp           pure-Python brute force with the causal limits written out;
                         each query equals decode over its truncated context; rows after a
                         query's position never change it (a planted off-by-one fails)
mla.attend_kv            pure-Python brute force with separate keys and values
mla.decode_rank          brute force on rank-256 rows written out by hand
mla.decode_gla2          equals decode_rank on each group's rows cut out of the 576-value
                         row; rewriting one group's latent half leaves the other group's
                         heads bit-identical (a swapped half fails)
mla.decode_nope          pure-Python brute force over the 512 latent values; equals decode
                         with q_pe = 0 on finite rope; unchanged by NaN rope bytes, which
                         turn decode with q_pe = 0 into NaN (the pages' control)
mla.pack_rows(k_pe=None) rope bytes zero, latent bytes as with any k_pe
mla.merge/split_ranges   split vs unsplit for S in {1, 2, 7, 64}; all-empty partials;
                         a NaN partial is not an empty one; partition coverage
numerics.f32_to_bf16_bits  torch's float32 -> bfloat16 cast: specials, exact ties, 10^6 random
mla.gather_context       hand-written gather loop (bf16 rows bit for bit); fp8 rows built
                         exactly representable upconvert to the bf16 gather; general fp8
                         rows land on a bf16 neighbour of the exact product within the
                         double-rounding bound; rope values copied
workloads.bf16_bits      torch's float32 -> bfloat16 cast (round to nearest even)
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla as omla
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(v):
    return np.float32(-0.0) if v == "-0.0" else np.float32(v)


# ----------------------------------------------------------------------------- formats
def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_anchor_values():
    g = _golden("e4m3_anchors.json")
    for code, val in g["codes"].items():
        got = oracle.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), code
    for code in g["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0])
    # max finite is 448, and there are exactly two NaN codes and no infinities
    t = oracle.E4M3_TABLE
    assert np.nanmax(np.abs(t)) == 448.0 and np.isnan(t).sum() == 2 and not np.isinf(t).any()


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_to_f32(bits)
    x = x[np.isfinite(x) & (np.abs(x) <= 464.0)]
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(1234)
    x = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-25, 6, 1_000_000))).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    big = np.array([448.0, 463.9, 464.0, 465.0, 1e6, 3e38, -500.0, -3e38], dtype=np.float32)
    assert oracle.e4m3_encode(big).tolist() == [0x7E] * 6 + [0xFE] * 2


def test_quantize_power_of_two_round_trip():
    """Latent = e4m3 values times 2^k with a block max of 448 * 2^k: quantise then dequantise is exact."""
    rng = np.random.default_rng(7)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for k in (-6, 0, 3):
        codes = rng.choice(finite, size=(5, 512))
        codes[:, ::128] = 0x7E  # each block's absmax is 448 * 2^k
        x = (oracle.e4m3_decode(codes) * 2.0**k).astype(np.float32)
        bits = workloads.bf16_bits(x)
        assert np.array_equal(oracle.bf16_to_f32(bits), x)  # e4m3 * 2^k is bf16-exact
        s, q = oracle.quantize_block128(bits)
        assert (s == np.float32(2.0**k)).all()
        back = oracle.e4m3_decode(q).reshape(5, 4, 128) * s[..., None]
        assert np.array_equal(back.reshape(5, 512), x.astype(np.float64))


def test_quantize_nonfinite_blocks_store_nan():
    """A 128-value block holding a NaN or an infinity stores the NaN scale 0x7FC00000 and 128
    codes 0x7F; the other blocks of the row quantise as if alone; the row decodes to NaN there."""
    rng = np.random.default_rng(11)
    x = workloads.bf16_bits(rng.standard_normal((1, 512)).astype(np.float32))
    specials = [p for p in range(1 << 16) if (p & 0x7F80) == 0x7F80]  # every NaN and infinity pattern
    assert len(specials) == 256
    for pat in specials:
        row = x.copy()
        row[0, 5] = pat          # block 0
        row[0, 256 + pat % 128] = pat  # block 2
        s, q = oracle.quantize_block128(row)
        sb = s.view(np.uint32)[0]
        assert sb[0] == 0x7FC00000 and sb[2] == 0x7FC00000
        assert (q[0, :128] == 0x7F).all() and (q[0, 256:384] == 0x7F).all()
        s1, q1 = oracle.quantize_block128(np.tile(x[:, 128:256], (1, 4)))
        assert s[0, 1] == s1[0, 0] and np.array_equal(q[0, 128:256], q1[0, :128])
    vals = omla.rows_from_bytes(oracle.pack_rows(row, np.zeros((1, 64), np.uint16), "fp8"), "fp8")
    assert np.isnan(vals[0, :128]).all() and np.isfinite(vals[0, 128:256]).all()
    # finite blocks beside it: unchanged whatever the other blocks hold
    s0, q0 = oracle.quantize_block128(x)
    assert s[0, 1] == s0[0, 1] and np.array_equal(q[0, 128:256], q0[0, 128:256])


# ----------------------------------------------------------------------- cache rows
def _golden_fp8_row():
    g = _golden("fp8_row_656.json")
    latent = np.zeros(512, dtype=np.float32)
    codes = np.zeros(512, dtype=np.uint8)
    scales = b""
    for k, blk in enumerate(g["blocks"]):
        latent[128 * k : 128 * k + 128] = _f32(blk["fill"])
        codes[128 * k : 128 * k + 128] = int(blk["fill_code"], 16)
        for i, v in blk["special"].items():
            latent[128 * k + int(i)] = _f32(v)
        for i, c in blk["special_codes"].items():
            codes[128 * k + int(i)] = int(c, 16)
        scales += bytes.fromhex(blk["scale_hex_le"])
    rope = np.array([int(g["rope"]["even" if j % 2 == 0 else "odd"], 16) for j in range(64)], dtype=np.uint16)
    expect = codes.tobytes() + scales + rope.astype("<u2").tobytes()
    return workloads.bf16_bits(latent), rope, expect


def test_fp8_row_matches_hand_worked_golden():
    latent_bits, rope, expect = _golden_fp8_row()
    assert len(expect) == 656
    got = oracle.pack_rows(latent_bits[None], rope[None], "fp8")
    assert got.shape == (1, 656)
    assert got[0].tobytes() == expect


def test_bf16_row_is_latent_then_rope_little_endian():
    rng = np.random.default_rng(3)
    lat = rng.integers(0, 1 << 16, size=(3, 512), dtype=np.uint16)
    pe = rng.integers(0, 1 << 16, size=(3, 64), dtype=np.uint16)
    rows = oracle.pack_rows(lat, pe, "bf16")
    assert rows.shape == (3, 1152)
    for t in range(3):
        b = rows[t].tobytes()
        assert b[:1024] == lat[t].astype("<u2").tobytes() and b[1024:] == pe[t].astype("<u2").tobytes()


def test_cache_write_places_rows_and_skips_negative_slots():
    w = workloads.make_workload("cw", seq_lens=[5, 9], heads=2, page_size=4, num_pages=8, seed=11)
    for fmt in ("bf16", "fp8"):
        pool = w.poisoned_pool() if fmt == "bf16" else np.full((8, 4, 656), 0xFF, np.uint8)
        before = pool.copy()
        slots = w.slots.copy()
        slots[1] = -1
        oracle.cache_write(pool, w.latent, w.k_pe, slots, fmt)
        R = oracle.ROW_BYTES[fmt]
        flat = pool.reshape(-1, R)
        packed = oracle.pack_rows(w.latent, w.k_pe, fmt)
        for i, s in enumerate(slots):
            if s >= 0:
                assert flat[s].tobytes() == packed[i].tobytes()
        untouched = np.setdiff1d(np.arange(flat.shape[0]), slots[slots >= 0])
        assert np.array_equal(flat[untouched], before.reshape(-1, R)[untouched])


def test_geometry_golden():
    g = _golden("geometry.json")
    assert oracle.ROW == g["values_per_row"]["value"] == g["latent_width"]["value"] + g["rope_width"]["value"]
    assert oracle.ROW_BYTES["bf16"] == g["row_bytes_bf16"]["value"]
    assert oracle.ROW_BYTES["fp8"] == g["row_bytes_fp8_ds_mla"]["value"]
    # 656 = 512 one-byte codes + 4 fp32 scales + 64 bf16 rope values
    assert oracle.ROW_BYTES["fp8"] == 512 + 4 * 4 + 64 * 2
    assert round(100 * (656 / g["row_bytes_true_nope_fp8"]["value"] - 1)) == g["fp8_over_nope_percent"]["value"]
    assert round(100 * (1 - 656 / 1152)) == g["fp8_saving_vs_bf16_percent"]["value"]


def test_int32_wrap_slot_golden():
    """The first slot holding an element whose int32 offset wraps is the one the page prints."""
    g = _golden("geometry.json")
    wrap = g["int32_wrap_slot"]["value"]

    def wraps(slot):
        return any(omla.element_offset_int32(slot, d) != omla.element_offset(slot, d) for d in (0, 575))

    assert not wraps(wrap - 1) and wraps(wrap)
    assert omla.element_offset_int32(wrap + 1, 0) < 0  # the next slot's start is already negative
    assert not wraps(g["h100_pool_slots"]["value"])
    assert wraps(g["h100_faulting_pool_slots"]["value"]) and wraps(g["b300_pool_slots"]["value"] - 1)


def test_high_slot_workload_would_catch_int32_offsets():
    """Every page of the high-slot workload sits where an int32 offset reads another row."""
    first = workloads.HIGH_SLOT_FIRST_PAGE
    assert first * 64 > workloads.WRAP_SLOT and (first - 1) * 64 <= workloads.WRAP_SLOT + 1
    for slot in (first * 64, first * 64 + 63, workloads.HIGH_SLOT_POOL_PAGES * 64 - 1):
        assert omla.element_offset_int32(slot) != omla.element_offset(slot)


# ------------------------------------------------------------------------- attention
def _vec(spec, n=576):
    v = np.zeros(n)
    for k, x in spec.items():
        v[int(k)] = x
    return v


def test_attend_closed_forms_golden():
    for case in _golden("attention_closed_form.json")["cases"]:
        q = _vec(case["q"])[None]
        rows = np.stack([_vec(r) for r in case["rows"]])
        out, lse = oracle.attend(q, rows, case["scale"])
        expect = np.zeros(512)
        for k, x in case["expect_out"].items():
            expect[int(k)] = x
        assert np.allclose(out[0], expect, rtol=0, atol=1e-12), case["name"]
        assert abs(lse[0] - case["expect_lse"]) < 1e-12, case["name"]


def _brute_attend(q, rows, scale):
    """Second formulation: explicit Python loops, math.fsum, math.exp."""
    H, L = len(q), len(rows)
    out, lse = [], []
    for h in range(H):
        s = [scale * math.fsum(q[h][d] * rows[t][d] for d in range(len(q[h]))) for t in range(L)]
        m = max(s)
        z = math.fsum(math.exp(x - m) for x in s)
        ls = m + math.log(z)
        w = [math.exp(x - ls) for x in s]
        out.append([math.fsum(w[t] * rows[t][d] for t in range(L)) for d in range(512)])
        lse.append(ls)
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("ps", [1, 2, 3])
def test_decode_matches_brute_force(ps):
    rng = np.random.default_rng(ps)
    w = workloads.make_workload("brute", seq_lens=[3, 4], heads=2, page_size=ps, num_pages=12, rng=rng)
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, "bf16")
    out, lse = oracle.decode(w.q, pool, w.block_table, w.seq_lens, ps, w.scale, "bf16")
    qf = oracle.bf16_to_f64(w.q)
    flat = pool.reshape(-1, 1152)
    for b in range(w.batch):
        rows = []
        for t in range(int(w.seq_lens[b])):
            slot = int(w.block_table[b][t // ps]) * ps + t % ps  # written out by hand
            rows.append(oracle.bf16_to_f64(flat[slot].view("<u2")).tolist())
        bo, bl = _brute_attend(qf[b].tolist(), rows, w.scale)
        assert np.max(np.abs(out[b] - bo)) < 1e-12 and np.max(np.abs(lse[b] - bl)) < 1e-12


def _rand_rows(rng, L, spread=False):
    rows = rng.standard_normal((L, 576))
    if spread:
        rows *= 10.0 ** rng.uniform(-2, 2, size=(L, 1))
    return rows


def test_one_token_returns_its_latent():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((16, 576))
    row = _rand_rows(rng, 1)
    out, lse = oracle.attend(q, row, 0.07)
    assert np.array_equal(out, np.broadcast_to(row[0, :512], (16, 512)))
    assert np.allclose(lse, 0.07 * (q @ row[0]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_uniform_scores_give_mean_and_log_length(how):
    rng = np.random.default_rng(6)
    L = 37
    q = np.zeros((4, 576)) if how == "zero_q" else rng.standard_normal((4, 576))
    rows = _rand_rows(rng, L, spread=True)
    out, lse = oracle.attend(q, rows, 0.0 if how == "zero_scale" else 0.3)
    assert np.allclose(out, rows[:, :512].mean(axis=0)[None], rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, math.log(L), rtol=0, atol=1e-12)


def test_duplicated_rows_shift_lse_by_ln2():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((8, 576))
    rows = _rand_rows(rng, 50, spread=True)
    o1, l1 = oracle.attend(q, rows, 0.072)
    o2, l2 = oracle.attend(q, np.concatenate([rows, rows[::-1]]), 0.072)
    assert np.allclose(o1, o2, rtol=1e-11, atol=1e-11 * np.abs(o1).max())
    assert np.allclose(l2, l1 + math.log(2), rtol=0, atol=1e-11)


def test_hardmax_limit():
    rng = np.random.default_rng(9)
    L = 40
    rows = _rand_rows(rng, L)
    q = np.zeros((1, 576))
    q[0, 3] = 1.0
    rows[:, 3] = 0.0
    rows[17, 3] = 60.0  # score gap 60 >> 50
    out, lse = oracle.attend(q, rows, 1.0)
    assert np.allclose(out[0], rows[17, :512], rtol=0, atol=L * math.exp(-50) * np.abs(rows).max())
    assert abs(lse[0] - 60.0) < L * math.exp(-50)


def test_empty_context_gives_zero_and_minus_inf():
    out, lse = oracle.attend(np.ones((3, 576)), np.zeros((0, 576)), 0.1)
    assert np.array_equal(out, np.zeros((3, 512))) and not np.signbit(out).any()
    assert np.isneginf(lse).all()
    w = workloads.make_workload("e", seq_lens=[0, 3, 0], heads=2, page_size=4, num_pages=4, seed=1)
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, "bf16")
    out, lse = oracle.decode(w.q, pool, w.block_table, w.seq_lens, 4, w.scale, "bf16")
    assert np.array_equal(out[[0, 2]], np.zeros((2, 2, 512))) and np.isneginf(lse[[0, 2]]).all()
    assert np.isfinite(out[1]).all() and np.isfinite(lse[1]).all()


def test_planted_softmax_over_heads_mistake_is_caught(monkeypatch):
    """The invariants have teeth: an oracle that normalises over heads fails them."""

    def wrong_attend(q, rows, scale):
        s = float(scale) * (q @ rows.T)
        p = np.exp(s - s.max(axis=0, keepdims=True))
        p = p / p.sum(axis=0, keepdims=True)  # over heads: the mistake
        return p @ rows[:, :512], np.log(np.exp(s).sum(axis=1))

    monkeypatch.setattr(omla, "attend", wrong_attend)
    rng = np.random.default_rng(10)
    q = rng.standard_normal((4, 576))
    row = _rand_rows(rng, 1)
    out, _ = omla.attend(q, row, 0.07)
    assert not np.allclose(out, np.broadcast_to(row[0, :512], (4, 512)))
    rows = _rand_rows(rng, 9)
    out, _ = omla.attend(np.zeros((4, 576)), rows, 0.07)
    assert not np.allclose(out, rows[:, :512].mean(axis=0)[None])


# ----------------------------------------------------------------- paging invariances
def _filled(w, fmt="bf16"):
    pool = w.poisoned_pool() if fmt == "bf16" else np.full((w.num_pages, w.page_size, 656), 0xFF, np.uint8)
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, fmt)
    return pool


def test_gather_formulations_agree():
    w = workloads.make_workload("g", seq_lens=[70, 1, 33], heads=2, page_size=16, num_pages=20, seed=2)
    pool = _filled(w)
    for b in range(3):
        L = int(w.seq_lens[b])
        a = oracle.gather_rows(pool, w.block_table, b, L, 16, "bf16")
        c = oracle.gather_rows_fast(pool, w.block_table, b, L, 16, "bf16")
        assert np.array_equal(a, c)


def test_physical_page_moves_are_invisible():
    w = workloads.make_workload("p", seq_lens=[100, 57], heads=4, page_size=8, num_pages=40, seed=3)
    pool = _filled(w)
    ref = oracle.decode(w.q, pool, w.block_table, w.seq_lens, 8, w.scale, "bf16")
    perm = np.random.default_rng(4).permutation(40)  # page p moves to perm[p]
    moved = np.empty_like(pool)
    moved[perm] = pool
    bt = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    got = oracle.decode(w.q, moved, bt, w.seq_lens, 8, w.scale, "bf16")
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_logical_page_order_is_irrelevant():
    w = workloads.make_workload("o", seq_lens=[96], heads=4, page_size=8, num_pages=12, seed=5)
    pool = _filled(w)
    o1, l1 = oracle.decode(w.q, pool, w.block_table, w.seq_lens, 8, w.scale, "bf16")
    bt = w.block_table.copy()
    bt[0] = bt[0][np.random.default_rng(6).permutation(12)]
    o2, l2 = oracle.decode(w.q, pool, bt, w.seq_lens, 8, w.scale, "bf16")
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_garbage_rope_control(fmt):
    """With q_pe = 0 any finite rope values leave the result bit-identical; with q_pe != 0 they change it."""
    w = workloads.make_workload("r", seq_lens=[40, 17], heads=4, page_size=16, num_pages=8, seed=7)
    other = np.random.default_rng(99).integers(0, 1 << 16, size=w.k_pe.shape, dtype=np.uint16)
    other = workloads.bf16_bits(np.nan_to_num(oracle.bf16_to_f32(other), nan=1.0, posinf=1.0, neginf=-1.0) % 50)
    q0 = w.q.copy()
    q0[:, :, 512:] = 0
    pools = []
    for pe in (w.k_pe, other):
        pool = w.poisoned_pool() if fmt == "bf16" else np.full((8, 16, 656), 0xFF, np.uint8)
        oracle.cache_write(pool, w.latent, pe, w.slots, fmt)
        pools.append(pool)
    a = oracle.decode(q0, pools[0], w.block_table, w.seq_lens, 16, w.scale, fmt)
    b = oracle.decode(q0, pools[1], w.block_table, w.seq_lens, 16, w.scale, fmt)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.decode(w.q, pools[0], w.block_table, w.seq_lens, 16, w.scale, fmt)
    d = oracle.decode(w.q, pools[1], w.block_table, w.seq_lens, 16, w.scale, fmt)
    assert np.max(np.abs(c[1] - d[1])) > 1e-3


# ----------------------------------------------------------------- multi-token verify
def test_mtp_matches_brute_force():
    rng = np.random.default_rng(41)
    T = 3
    w = workloads.make_workload("mtp_brute", seq_lens=[5, 2, 0], heads=2, page_size=2, num_pages=8, rng=rng)
    q = workloads.bf16_bits(rng.standard_normal((w.batch, T, w.heads, 576)).astype(np.float32))
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, "bf16")
    out, lse = oracle.decode_mtp(q, pool, w.block_table, w.seq_lens, 2, w.scale, "bf16")
    qf = oracle.bf16_to_f64(q)
    flat = pool.reshape(-1, 1152)
    # visible token counts written out by hand: L=5 -> 3, 4, 5; L=2 -> 0, 1, 2; L=0 -> 0, 0, 0
    visible = {0: [3, 4, 5], 1: [0, 1, 2], 2: [0, 0, 0]}
    for b in range(w.batch):
        for i in range(T):
            rows = []
            for t in range(visible[b][i]):
                slot = int(w.block_table[b][t // 2]) * 2 + t % 2
                rows.append(oracle.bf16_to_f64(flat[slot].view("<u2")).tolist())
            if not rows:
                assert (out[b, i] == 0).all() and np.isneginf(lse[b, i]).all()
                continue
            bo, bl = _brute_attend(qf[b, i].tolist(), rows, w.scale)
            assert np.max(np.abs(out[b, i] - bo)) < 1e-12 and np.max(np.abs(lse[b, i] - bl)) < 1e-12


def _full_pool(rng, slots, fmt="bf16"):
    """A pool of `slots` rows, every one finite and distinct (no poison), packed by the oracle."""
    lat = workloads.bf16_bits(rng.standard_normal((slots, 512)).astype(np.float32))
    pe = workloads.bf16_bits(rng.standard_normal((slots, 64)).astype(np.float32))
    R = oracle.ROW_BYTES[fmt]
    pool = np.zeros((slots, R), np.uint8)
    oracle.cache_write(pool, lat, pe, np.arange(slots), fmt)
    return pool


def test_sparse_matches_brute_force():
    """Index lists with -1 entries anywhere, valid counts 0, 1, partial and full, a repeated
    slot, against explicit Python loops over the listed rows."""
    rng = np.random.default_rng(51)
    pool = _full_pool(rng, 20)
    idx = np.array([[3, 7, -1, -1], [-1, -1, -1, -1], [19, -1, -1, -1], [5, -1, 0, 11], [2, 2, 9, 4]], np.int32)
    q = workloads.bf16_bits(rng.standard_normal((5, 2, 576)).astype(np.float32))
    out, lse = oracle.decode_sparse(q, pool, idx, 0.07, "bf16")
    qf = oracle.bf16_to_f64(q)
    for t in range(5):
        rows = [oracle.bf16_to_f64(pool[int(i)].view("<u2")).tolist() for i in idx[t] if i >= 0]
        if not rows:
            assert (out[t] == 0).all() and not np.signbit(out[t]).any() and np.isneginf(lse[t]).all()
            continue
        bo, bl = _brute_attend(qf[t].tolist(), rows, 0.07)
        assert np.max(np.abs(out[t] - bo)) < 1e-12 and np.max(np.abs(lse[t] - bl)) < 1e-12
    # one valid entry: that row's latent, exactly
    row = oracle.bf16_to_f64(pool[19].view("<u2"))
    assert np.array_equal(out[2], np.broadcast_to(row[:512], (2, 512)))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_sparse_equals_block_table_decode_over_the_same_slots(fmt):
    """A request's index list that enumerates its context's slots in token order (padded with a
    -1 tail) gives the paged decode's result; reordering the list or moving its -1 entries
    changes nothing beyond rounding."""
    rng = np.random.default_rng(52)
    w = workloads.make_workload("sparse_eq", seq_lens=[37, 1, 0, 64], heads=4, page_size=16, num_pages=12,
                                fmt=fmt, rng=rng)
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, fmt)
    ref_o, ref_l = oracle.decode(w.q, pool, w.block_table, w.seq_lens, w.page_size, w.scale, fmt)
    topk = 80
    idx = np.full((w.batch, topk), -1, np.int64)
    for b in range(w.batch):
        for t in range(int(w.seq_lens[b])):
            idx[b, t] = int(w.block_table[b][t // 16]) * 16 + t % 16
    out, lse = oracle.decode_sparse(w.q, pool, idx, w.scale, fmt)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l))
    assert np.allclose(out, ref_o, rtol=0, atol=1e-12) and np.allclose(lse[1:2], ref_l[1:2], atol=1e-12)
    shuffled = np.array([rng.permutation(r) for r in idx])  # -1 entries land anywhere
    out2, lse2 = oracle.decode_sparse(w.q, pool, shuffled, w.scale, fmt)
    fin = np.isfinite(lse)
    assert np.allclose(out2, out, rtol=0, atol=1e-12) and np.allclose(lse2[fin], lse[fin], rtol=0, atol=1e-12)


def test_sparse_never_reads_a_negative_entry():
    """A -1 entry must select nothing: array indexing would silently read the pool's last row,
    which here differs from every listed row."""
    rng = np.random.default_rng(53)
    pool = _full_pool(rng, 10)
    q = workloads.bf16_bits(rng.standard_normal((1, 2, 576)).astype(np.float32))
    with_tail, _ = oracle.decode_sparse(q, pool, np.array([[1, 2, -1]]), 0.07, "bf16")
    plain, _ = oracle.decode_sparse(q, pool, np.array([[1, 2]]), 0.07, "bf16")
    wrong, _ = oracle.decode_sparse(q, pool, np.array([[1, 2, 9]]), 0.07, "bf16")  # what -1 would read
    assert np.array_equal(with_tail, plain) and not np.allclose(with_tail, wrong)


def test_sparse_nope_brute_force_and_rope_ignored():
    """NoPE-512 queries (q [T, H, 512]): pure-Python brute force over the listed rows' 512 latent
    values; NaN rope values in every row change nothing (they never enter a score)."""
    rng = np.random.default_rng(54)
    pool = _full_pool(rng, 12)
    idx = np.array([[4, -1, 8, 1], [-1, -1, -1, -1], [11, -1, -1, -1]], np.int32)
    q = workloads.bf16_bits(rng.standard_normal((3, 2, 512)).astype(np.float32))
    out, lse = oracle.decode_sparse(q, pool, idx, 0.09, "bf16")
    qf = oracle.bf16_to_f64(q)
    for t in range(3):
        rows = [oracle.bf16_to_f64(pool[int(i)].view("<u2"))[:512].tolist() for i in idx[t] if i >= 0]
        if not rows:
            assert (out[t] == 0).all() and np.isneginf(lse[t]).all()
            continue
        bo, bl = _brute_attend(qf[t].tolist(), rows, 0.09)
        assert np.max(np.abs(out[t] - bo)) < 1e-12 and np.max(np.abs(lse[t] - bl)) < 1e-12
    nan_rope = pool.copy()
    nan_rope.view("<u2")[:, 512:] = 0x7FC0
    out2, lse2 = oracle.decode_sparse(q, nan_rope, idx, 0.09, "bf16")
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)
    with pytest.raises(ValueError):
        oracle.decode_sparse(q[:, :, :500], pool, idx, 0.09, "bf16")


def _mtp_case(seed, T=4):
    rng = np.random.default_rng(seed)
    w = workloads.make_workload("mtp", seq_lens=[50, 3, 17], heads=4, page_size=8, num_pages=12, rng=rng)
    q = workloads.bf16_bits(rng.standard_normal((w.batch, T, w.heads, 576)).astype(np.float32))
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, "bf16")
    return w, q, pool


def test_mtp_query_equals_decode_over_its_truncated_context():
    w, q, pool = _mtp_case(42)
    T = q.shape[1]
    out, lse = oracle.decode_mtp(q, pool, w.block_table, w.seq_lens, 8, w.scale, "bf16")
    for i in range(T):
        lens_i = np.maximum(0, w.seq_lens - T + 1 + i)
        o, l = oracle.decode(np.ascontiguousarray(q[:, i]), pool, w.block_table, lens_i, 8, w.scale, "bf16")
        assert np.array_equal(o, out[:, i]) and np.array_equal(l, lse[:, i])


def test_mtp_rows_after_a_query_do_not_change_it():
    """Rewriting the rows of positions > L - T + i leaves query i unchanged and changes the
    last query (which sees them).  The brute-force test above pins the exact limits."""
    w, q, pool = _mtp_case(43)
    T = q.shape[1]
    ref = oracle.decode_mtp(q, pool, w.block_table, w.seq_lens, 8, w.scale, "bf16")
    b, L = 0, int(w.seq_lens[0])
    for i in range(T - 1):
        p2 = pool.copy()
        t = np.arange(L - T + 1 + i, L)  # tokens query i must not see
        slots = w.block_table[b][t // 8].astype(np.int64) * 8 + t % 8
        p2.reshape(-1, 1152)[slots] = pool.reshape(-1, 1152)[slots][::-1] ^ np.uint8(0x01)
        o, l = oracle.decode_mtp(q, p2, w.block_table, w.seq_lens, 8, w.scale, "bf16")
        assert np.array_equal(o[b, i], ref[0][b, i]) and np.array_equal(l[b, i], ref[1][b, i])
        assert np.abs(l[b, T - 1] - ref[1][b, T - 1]).max() > 1e-9


# ------------------------------------------------------------- other latent geometries
def test_attend_kv_matches_brute_force():
    rng = np.random.default_rng(90)
    q, keys, vals = rng.standard_normal((2, 7)), rng.standard_normal((5, 7)), rng.standard_normal((5, 3))
    out, lse = oracle.attend_kv(q, keys, vals, 0.3)
    for h in range(2):
        s = [0.3 * math.fsum(q[h][d] * keys[t][d] for d in range(7)) for t in range(5)]
        m = max(s)
        ls = m + math.log(math.fsum(math.exp(x - m) for x in s))
        w = [math.exp(x - ls) for x in s]
        assert abs(lse[h] - ls) < 1e-12
        assert max(abs(out[h][c] - math.fsum(w[t] * vals[t][c] for t in range(5))) for c in range(3)) < 1e-12


def _rank_pool(rng, w, D):
    """bf16 bits [num_slots, D + 64] with random rows at the workload's slots (rest NaN)."""
    pool = np.full((w.num_pages * w.page_size, D + 64), 0x7FC0, np.uint16)
    pool[w.slots] = workloads.bf16_bits(rng.standard_normal((w.slots.size, D + 64)).astype(np.float32))
    return pool


def test_rank256_decode_matches_brute_force():
    rng = np.random.default_rng(91)
    w = workloads.make_workload("r256", seq_lens=[6, 3], heads=2, page_size=3, num_pages=6, rng=rng)
    pool = _rank_pool(rng, w, 256)
    q = workloads.bf16_bits(rng.standard_normal((2, 2, 320)).astype(np.float32))
    out, lse = oracle.decode_rank(q, pool, w.block_table, w.seq_lens, 3, w.scale)
    qf = oracle.bf16_to_f64(q)
    for b in range(2):
        rows = [oracle.bf16_to_f64(pool[int(w.block_table[b][t // 3]) * 3 + t % 3]).tolist()
                for t in range(int(w.seq_lens[b]))]
        for h in range(2):
            s = [w.scale * math.fsum(qf[b, h, d] * r[d] for d in range(320)) for r in rows]
            m = max(s)
            ls = m + math.log(math.fsum(math.exp(x - m) for x in s))
            assert abs(lse[b, h] - ls) < 1e-12
            for c in (0, 100, 255):
                ref = math.fsum(math.exp(x - ls) * r[c] for x, r in zip(s, rows))
                assert abs(out[b, h, c] - ref) < 1e-12


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_gla2_is_two_rank256_problems(fmt):
    rng = np.random.default_rng(92)
    w = workloads.make_workload("gla", seq_lens=[40, 0, 19], heads=4, page_size=8, num_pages=12, rng=rng, fmt=fmt)
    pool = w.poisoned_pool() if fmt == "bf16" else np.full((12, 8, 656), 0xFF, np.uint8)
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, fmt)
    q = workloads.bf16_bits(rng.standard_normal((3, 4, 320)).astype(np.float32))
    out, lse = oracle.decode_gla2(q, pool, w.block_table, w.seq_lens, 8, w.scale, fmt)
    vals = oracle.rows_from_bytes(pool.reshape(-1, oracle.ROW_BYTES[fmt])[w.slots], fmt)  # fp64, exact
    if fmt == "bf16":  # decode_rank takes bf16 rows; dequantised fp8 values need not be bf16 values
        for g in range(2):
            pg = np.full((12 * 8, 320), 0x7FC0, np.uint16)
            cut = np.concatenate([vals[:, 256 * g:256 * g + 256], vals[:, 512:]], axis=1)
            pg[w.slots] = workloads.bf16_bits(cut.astype(np.float32))  # exact: the values are bf16
            o, l = oracle.decode_rank(q[:, 2 * g:2 * g + 2], pg, w.block_table, w.seq_lens, 8, w.scale)
            assert np.array_equal(o, out[:, 2 * g:2 * g + 2]) and np.array_equal(l, lse[:, 2 * g:2 * g + 2])
    # rewriting group 1's latent half (fp8: its scale blocks 2 and 3) leaves group 0's heads
    # unchanged, and changes group 1's
    p2 = pool.copy()
    lat2 = w.latent.copy()
    lat2[:, 256:] = workloads.bf16_bits(rng.standard_normal((lat2.shape[0], 256)).astype(np.float32))
    oracle.cache_write(p2, lat2, w.k_pe, w.slots, fmt)
    o2, l2 = oracle.decode_gla2(q, p2, w.block_table, w.seq_lens, 8, w.scale, fmt)
    assert np.array_equal(o2[:, :2], out[:, :2]) and np.array_equal(l2[:, :2], lse[:, :2])
    live = w.seq_lens > 0
    assert np.abs(l2[live, 2:] - lse[live, 2:]).max() > 1e-6


# --------------------------------------------------------------------------- NoPE-512
@pytest.mark.parametrize("ps", [1, 3])
def test_nope_decode_matches_brute_force(ps):
    rng = np.random.default_rng(30 + ps)
    w = workloads.make_workload("nope_brute", seq_lens=[5, 2], heads=2, page_size=ps, num_pages=12, rng=rng)
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, "bf16")
    q512 = w.q[:, :, :512].copy()
    out, lse = oracle.decode_nope(q512, pool, w.block_table, w.seq_lens, ps, w.scale, "bf16")
    qf = oracle.bf16_to_f64(q512)
    flat = pool.reshape(-1, 1152)
    for b in range(w.batch):
        rows = []
        for t in range(int(w.seq_lens[b])):
            slot = int(w.block_table[b][t // ps]) * ps + t % ps
            rows.append(oracle.bf16_to_f64(flat[slot].view("<u2"))[:512].tolist())
        bo, bl = _brute_attend(qf[b].tolist(), rows, w.scale)
        assert np.max(np.abs(out[b] - bo)) < 1e-12 and np.max(np.abs(lse[b] - bl)) < 1e-12


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_nope_equals_decode_with_zero_q_pe_and_ignores_nan_rope(fmt):
    w = workloads.make_workload("nope", seq_lens=[40, 0, 17], heads=4, page_size=16, num_pages=8, seed=13, fmt=fmt)
    shape = (8, 16, 576) if fmt == "bf16" else (8, 16, 656)
    fresh = (lambda: w.poisoned_pool()) if fmt == "bf16" else (lambda: np.full(shape, 0xFF, np.uint8))
    zero_rope, nan_rope = fresh(), fresh()
    oracle.cache_write(zero_rope, w.latent, None, w.slots, fmt)
    nan_pe = np.full(w.k_pe.shape, 0x7FC0, np.uint16)  # bf16 NaN in every rope value
    oracle.cache_write(nan_rope, w.latent, nan_pe, w.slots, fmt)
    q0 = w.q.copy()
    q0[:, :, 512:] = 0
    q512 = w.q[:, :, :512].copy()
    args = (w.block_table, w.seq_lens, 16, w.scale, fmt)
    full0 = oracle.decode(q0, zero_rope, *args)
    n0 = oracle.decode_nope(q512, zero_rope, *args)
    n1 = oracle.decode_nope(q512, nan_rope, *args)
    live = w.seq_lens > 0
    assert np.max(np.abs(full0[0][live] - n0[0][live])) < 1e-12
    assert np.max(np.abs(full0[1][live] - n0[1][live])) < 1e-12
    assert np.array_equal(n0[0], n1[0]) and np.array_equal(n0[1], n1[1])  # rope bytes never read
    assert (n0[0][~live] == 0).all() and np.isneginf(n0[1][~live]).all()
    # the control: zero-padding q_pe does not protect against non-finite rope bytes
    bad = oracle.decode(q0, nan_rope, *args)
    assert np.isnan(bad[1][live]).all()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_pack_rows_without_k_pe_zeroes_the_rope_part(fmt):
    w = workloads.make_workload("zr", seq_lens=[9], heads=1, page_size=16, num_pages=2, seed=3)
    with_pe = oracle.pack_rows(w.latent, w.k_pe, fmt)
    no_pe = oracle.pack_rows(w.latent, None, fmt)
    rope = slice(1024, 1152) if fmt == "bf16" else slice(528, 656)
    keep = slice(0, 1024) if fmt == "bf16" else slice(0, 528)
    assert not no_pe[:, rope].any() and with_pe[:, rope].any()
    assert np.array_equal(no_pe[:, keep], with_pe[:, keep])


def test_fp8_decode_equals_bf16_decode_on_exactly_representable_rows():
    """Rows whose latent is e4m3 values times 2^k (block max 448 * 2^k) survive quantisation."""
    rng = np.random.default_rng(12)
    w = workloads.make_workload("x", seq_lens=[30, 65], heads=4, page_size=16, num_pages=10, seed=12)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=w.latent.shape)
    codes[:, ::128] = 0x7E
    k = rng.integers(-8, 2, size=(w.latent.shape[0], 4))
    vals = oracle.e4m3_decode(codes).reshape(-1, 4, 128) * (2.0 ** k)[..., None]
    lat = workloads.bf16_bits(vals.reshape(-1, 512).astype(np.float32))
    p16 = w.poisoned_pool()
    p8 = np.full((10, 16, 656), 0xFF, np.uint8)
    oracle.cache_write(p16, lat, w.k_pe, w.slots, "bf16")
    oracle.cache_write(p8, lat, w.k_pe, w.slots, "fp8")
    a = oracle.decode(w.q, p16, w.block_table, w.seq_lens, 16, w.scale, "bf16")
    b = oracle.decode(w.q, p8, w.block_table, w.seq_lens, 16, w.scale, "fp8")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------- split + merge
@pytest.mark.parametrize("S", [1, 2, 7, 64])
def test_split_then_merge_equals_unsplit(S):
    w = workloads.make_workload("s", seq_lens=[0, 1, 5, 300, 1000], heads=4, page_size=16,
                                num_pages=100, seed=S, row_scale_log10=(-1, 1))
    pool = _filled(w)
    q = oracle.bf16_to_f64(w.q)
    ref_o, ref_l = oracle.decode(w.q, pool, w.block_table, w.seq_lens, 16, w.scale, "bf16")
    po = np.zeros((S, w.batch, 4, 512))
    pl = np.zeros((S, w.batch, 4))
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        rows = oracle.gather_rows_fast(pool, w.block_table, b, L, 16, "bf16")
        rngs = oracle.split_ranges(L, 16, S, width=w.block_table.shape[1] if S % 2 else None)
        assert rngs[0][0] == 0 and rngs[-1][1] == L
        assert all(a[1] == c[0] for a, c in zip(rngs, rngs[1:]))
        assert all(t0 % 16 == 0 for t0, t1 in rngs if t1 > t0)
        for i, (t0, t1) in enumerate(rngs):
            po[i, b], pl[i, b] = oracle.attend(q[b], rows[t0:t1], w.scale)
    mo, ml = oracle.merge(po, pl)
    live = w.seq_lens > 0
    assert np.max(np.abs(mo[live] - ref_o[live])) < 1e-12
    assert np.max(np.abs(ml[live] - ref_l[live])) < 1e-12
    assert np.array_equal(mo[~live], ref_o[~live]) and np.isneginf(ml[~live]).all()


def test_merge_of_all_empty_partials():
    o, l = oracle.merge(np.full((5, 2, 3, 512), 7.0), np.full((5, 2, 3), -np.inf))
    assert np.array_equal(o, np.zeros((2, 3, 512))) and np.isneginf(l).all()


def test_merge_and_attend_propagate_nan():
    """A NaN partial (or score) is not an empty one: the merged result is NaN."""
    po = np.ones((3, 1, 2, 512))
    pl = np.array([[[np.nan, 1.0]], [[-np.inf, 2.0]], [[-np.inf, np.nan]]])
    o, l = oracle.merge(po, pl)
    assert np.isnan(l).all() and np.isnan(o).all()
    q = np.zeros((1, 576))
    q[0, 0] = 1.0
    rows = np.ones((3, 576))
    rows[1, 0] = np.nan
    o, l = oracle.attend(q, rows, 0.5)
    assert np.isnan(l).all() and np.isnan(o).all()


def test_merge_two_single_token_partials_is_a_two_token_softmax():
    """Closed form: partials over one token each are (row, score); merged = 2-token softmax."""
    o, l = oracle.merge(np.array([[np.eye(512)[0]], [np.eye(512)[1]]]), np.array([[1.0], [0.0]]))
    assert abs(o[0, 0] - 0.7310585786300049) < 1e-15 and abs(o[0, 1] - 0.2689414213699951) < 1e-15
    assert abs(l[0] - 1.3132616875182228) < 1e-15


# ------------------------------------------------------------------------ generators
def test_oracle_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(1_000_000).astype(np.float32) * np.float32(2.0) ** rng.integers(-140, 120, 1_000_000)
    ties = (rng.integers(0, 1 << 16, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)  # exact half-way
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 3.4028235e38, 1e-45, -1e-45,
                        1.1754942e-38, 2.0 ** -133], np.float32)
    for v in (x, ties, special):
        ours = oracle.f32_to_bf16_bits(v)
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(v)  # NaN stays NaN; the payload is not specified
        assert np.isnan(oracle.bf16_to_f32(ours[nan])).all()
        assert np.array_equal(ours[~nan], ref[~nan])
    nan = oracle.f32_to_bf16_bits(np.array([np.nan, -np.nan], np.float32))
    assert np.isnan(oracle.bf16_to_f32(nan)).all()


# ------------------------------------------------------------------- context gather
def test_gather_bf16_rows_by_hand():
    rng = np.random.default_rng(50)
    w = workloads.make_workload("g", seq_lens=[13, 0, 7], heads=1, page_size=4, num_pages=8, rng=rng)
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent, w.k_pe, w.slots, "bf16")
    starts = np.array([3, 0, 5])
    counts = np.array([9, 0, 2])
    cu = np.concatenate([[0], np.cumsum(counts)])
    got = oracle.gather_context(pool, w.block_table, cu, starts, 4, "bf16")
    flat = pool.reshape(-1, 1152)
    want = []
    for b in range(3):
        for j in range(counts[b]):
            t = starts[b] + j
            want.append(flat[int(w.block_table[b][t // 4]) * 4 + t % 4].view("<u2"))
    assert np.array_equal(got, np.array(want))


def test_fp8_upconvert_exact_on_representable_rows():
    rng = np.random.default_rng(51)
    w = workloads.make_workload("g8", seq_lens=[40, 25], heads=1, page_size=16, num_pages=6, seed=51)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=w.latent.shape)
    codes[:, ::128] = 0x7E
    k = rng.integers(-8, 2, size=(w.latent.shape[0], 4))
    vals = oracle.e4m3_decode(codes).reshape(-1, 4, 128) * (2.0 ** k)[..., None]
    lat = workloads.bf16_bits(vals.reshape(-1, 512).astype(np.float32))
    p16, p8 = w.poisoned_pool(), np.full((6, 16, 656), 0xFF, np.uint8)
    oracle.cache_write(p16, lat, w.k_pe, w.slots, "bf16")
    oracle.cache_write(p8, lat, w.k_pe, w.slots, "fp8")
    cu = np.concatenate([[0], np.cumsum(w.seq_lens)])
    a = oracle.gather_context(p16, w.block_table, cu, None, 16, "bf16")
    b = oracle.gather_context(p8, w.block_table, cu, None, 16, "fp8")
    assert np.array_equal(a, b)


def test_fp8_upconvert_rounds_the_exact_product():
    w = workloads.make_workload("g9", seq_lens=[300], heads=1, page_size=16, num_pages=20, seed=52,
                                row_scale_log10=(-3.0, 3.0))
    p8 = np.full((20, 16, 656), 0xFF, np.uint8)
    oracle.cache_write(p8, w.latent, w.k_pe, w.slots, "fp8")
    rows = p8.reshape(-1, 656)[w.slots]
    got = oracle.upconvert_rows(rows, "fp8")
    exact = oracle.rows_from_bytes(rows, "fp8")[:, :512]  # fp64, exact code * scale
    v = oracle.bf16_to_f64(got[:, :512])
    ulp16 = np.where(exact == 0, 0.0, 2.0 ** (np.floor(np.log2(np.abs(np.where(exact == 0, 1, exact)))) - 7))
    assert (np.abs(v - exact) <= 0.5 * ulp16 * (1 + 2.0 ** -16) + 1e-300).all()
    assert np.array_equal(got[:, 512:], w.k_pe)  # rope copied bit for bit


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.bf16_bits(x), ref)


def test_tiny_workload_structure():
    w = workloads.tiny()
    assert w.batch == 1 and w.heads == 4 and w.page_size == 16 and w.num_pages == 32
    assert w.seq_lens.tolist() == [256]
    expect = np.random.default_rng(0).permutation(32)[:16]  # lengths are fixed: pages are the first draw
    assert np.array_equal(w.block_table[0], expect)
    assert w.latent.shape == (256, 512) and w.q.shape == (1, 4, 576)
    assert np.float32(w.scale) == np.float32(1 / math.sqrt(192))


def test_ragged_lengths_and_tails():
    rng = np.random.default_rng(0)
    lens = workloads.fp8_ragged_lengths(rng)
    assert lens.size == 48 and {0, 1, 17, 32768} <= set(lens.tolist())
    assert lens.min() >= 0 and lens.max() <= 32768
    w = workloads.make_workload("t", seq_lens=[0, 1, 17, 64, 65], heads=2, page_size=16, num_pages=64, seed=0)
    for b, L in enumerate(w.seq_lens):
        n = -(-int(L) // 16)
        assert (w.block_table[b, :n] >= 0).all() and (w.block_table[b, n:] == -1).all()
    used = w.block_table[w.block_table >= 0]
    assert len(np.unique(used)) == used.size  # without replacement


def test_unread_slots_stay_poisoned():
    w = workloads.make_workload("u", seq_lens=[5, 20], heads=2, page_size=16, num_pages=6, seed=0)
    pool = _filled(w)
    flat = pool.reshape(-1, 1152)
    read = set()
    for b in range(2):
        for t in range(int(w.seq_lens[b])):
            read.add(oracle.slot_of(w.block_table, b, t, 16))
    assert read == set(w.slots.tolist())
    unread = [s for s in range(flat.shape[0]) if s not in read]
    assert (flat[unread].view("<u2") == workloads.BF16_POISON).all()

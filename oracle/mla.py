"""Paged MLA latent decode, written as its plain definition in fp64 (oracle side).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

What is computed (per request b and head h), following the pages:

* Each cached token holds one 576-wide row per layer: a 512-wide latent followed
  by one shared 64-wide rotary key (sabi-mla-vllm, opening paragraph: 576 cached
  values per token per layer; "What the plugin does": a paged 576-wide latent
  cache).  The absorbed query is cat(q_latent[512], q_pe[64]) (vLLM PR #55543,
  commit adding the zero-rope shim: q_pe is concatenated after the latent,
  mirroring the rope>0 path).
* Rows live in pages; a request's logical page j is physical page
  block_table[b, j], so token t sits in slot block_table[b, t // ps] * ps + t % ps,
  and the row starts at element slot * 576.  That product must not be formed in
  32-bit arithmetic: it wraps at slot 2^31 / 576 = 3,728,270 (sabi-mla-vllm,
  "B300 fix (0.2.0)").  Here every offset is a Python int.
* Scores s_t = scale * <q[b,h], row_t> over all 576 dims, softmax over the
  cache tokens (not over heads), output = softmax-weighted sum of the 512-wide
  latent part, plus the log-sum-exp of the scaled scores (vLLM PR #55543, review
  comment on the equivalence test: einsum of q_latent with the cached rows times
  the softmax scale, normalised over the last, cache-token, dimension).
* The LSE is the natural log (reading: the pages never name the base).
* A request with no tokens returns (0, -inf) (vLLM PR #55543, Tests: all-invalid
  rows neutralise to (0, -inf) per the decode-context-parallel merge contract).
* Partial results over disjoint token sets merge by log-sum-exp (vLLM PR #55543,
  description: FlashMLA sparse returns the decode LSE needed for DCP and MTP).
* A speculative-decoding verify step carries q_len = 1 + k query tokens per request, the
  last q_len positions of its sequence, and reads the cache once for all of them
  (qwen-mla-vllm, "16 GB GPUs": a verify step that reads the latent cache once per request
  instead of once per draft token).  Reading (the pages do not spell out the mask): the
  usual causal one, seq_lens counting the q_len new tokens, so query i of a request with
  L tokens attends to tokens 0 .. L - q_len + i.
* Prefill reads the cached context with 64-bit indices (sabi-mla-vllm, "B300 fix (0.2.0)":
  prefill gathers the cache with int64 indices) into a 576-wide workspace, upconverting
  fp8 rows to bf16 on the way (vLLM PR #55543, commit on the context-gather path: the
  gather reads 656-byte rows into a workspace 576 rows wide).  Reading (the pages give no
  formula): a bf16 row is copied; an fp8 latent value becomes bf16(fl32(code * scale)),
  the product rounded to float32 and then to bf16, both to nearest even; rope copied.
* Other latent geometries (qwen-mla-vllm, "How it works": per-layer latent ranks 256 /
  768 / 1792 plus a small rotary tail; opening section: GLA-g2 splits the latent into two
  head groups).  Readings (the pages give no row layout): a rank-D layer caches bf16 rows
  of D latent values followed by the 64 rope values; GLA-g2 keeps the 576-value / 656-byte
  row, heads [0, H/2) use latent values [0, 256) and heads [H/2, H) use [256, 512), both
  groups share the rope, and each head's output is its group's 256 values.
* Sparse (index-list) decode: each query token carries its own list of cache slots to attend
  to, already converted to global slot numbers (vLLM PR #55543, the tests commit: a ragged
  mixed batch whose valid counts include 0 and 1, with -1 tails, all-invalid rows giving
  (0, -inf); the review of the mocked index converter, which hands the kernel the converted
  per-query indices).  Reading: indices [T, topk] int32, shared by all heads of a query; an
  entry below zero selects nothing wherever it stands; attention runs over exactly the listed
  slots (a slot listed twice counts twice); row offsets are slot * row_bytes in 64-bit.
* NoPE-512 layers (no rotary part) keep the same row and write zeros into its rope part;
  their query has 512 values, padded with zeros to 576, so the rope part adds nothing to
  any score (vLLM PR #55543, description of the zero-rope approach).  decode_nope is the
  definition itself: scores over the 512 latent values only.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64, e4m3_decode, f32_to_bf16_bits, quantize_block128

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE
ROW_BYTES = {"bf16": 2 * ROW, "fp8": 656}
# fp8 656-byte row (reading of vLLM PR #55543, which lists the parts but not their
# order): [0, 512) e4m3 codes, [512, 528) four little-endian fp32 block scales,
# [528, 656) 64 little-endian bf16 rope values.
FP8_CODES = slice(0, 512)
FP8_SCALES = slice(512, 528)
FP8_ROPE = slice(528, 656)


# ------------------------------------------------------------------------ addressing
def slot_of(block_table: np.ndarray, b: int, t: int, page_size: int) -> int:
    """Slot of token t of request b (Python ints: no overflow)."""
    page = int(block_table[b, t // page_size])
    if page < 0:
        raise IndexError(f"request {b} token {t}: block table entry is {page}")
    return page * page_size + t % page_size


def element_offset(slot: int, d: int = 0) -> int:
    """Element offset of value d of the bf16 row in a slot, exact."""
    return slot * ROW + d


def element_offset_int32(slot: int, d: int = 0) -> int:
    """The same offset formed in wrapping two's-complement int32 arithmetic.

    This is the faulty addressing the sabi-mla-vllm "B300 fix" section describes;
    it exists only so that tests can show the high-slot cases would catch it.
    """
    v = (slot * ROW + d) & 0xFFFFFFFF
    return v - (1 << 32) if v >= (1 << 31) else v


# ----------------------------------------------------------------------- row values
def _pool_rows(pool: np.ndarray, fmt: str) -> np.ndarray:
    R = ROW_BYTES[fmt]
    flat = np.asarray(pool).view(np.uint8).reshape(-1)
    if flat.size % R:
        raise ValueError("pool size is not a whole number of rows")
    return flat.reshape(-1, R)


def rows_from_bytes(row_bytes: np.ndarray, fmt: str) -> np.ndarray:
    """fp64 values [n, 576] of raw rows [n, row_bytes] (exact)."""
    row_bytes = np.ascontiguousarray(row_bytes, dtype=np.uint8)
    n = row_bytes.shape[0]
    if fmt == "bf16":
        return bf16_to_f64(row_bytes.view("<u2").reshape(n, ROW))
    codes = row_bytes[:, FP8_CODES]
    scales = np.ascontiguousarray(row_bytes[:, FP8_SCALES]).view("<f4").reshape(n, 4)
    rope = np.ascontiguousarray(row_bytes[:, FP8_ROPE]).view("<u2").reshape(n, ROPE)
    out = np.empty((n, ROW), dtype=np.float64)
    lat = e4m3_decode(codes).reshape(n, 4, 128) * scales.astype(np.float64)[:, :, None]
    out[:, :LATENT] = lat.reshape(n, LATENT)
    out[:, LATENT:] = bf16_to_f64(rope)
    return out


def gather_rows(pool, block_table, b: int, length: int, page_size: int, fmt: str) -> np.ndarray:
    """Rows of tokens 0..length-1 of request b, fp64 [length, 576]."""
    rows = _pool_rows(pool, fmt)
    slots = np.fromiter((slot_of(block_table, b, t, page_size) for t in range(length)),
                        dtype=np.int64, count=length)
    return rows_from_bytes(rows[slots], fmt)


def gather_rows_fast(pool, block_table, b: int, length: int, page_size: int, fmt: str) -> np.ndarray:
    """Same rows as gather_rows, with the slot list built by array operations (int64)."""
    rows = _pool_rows(pool, fmt)
    t = np.arange(length, dtype=np.int64)
    pages = np.asarray(block_table[b], dtype=np.int64)[t // page_size]
    if (pages < 0).any():
        raise IndexError(f"request {b}: block table entry -1 inside the context")
    return rows_from_bytes(rows[pages * page_size + t % page_size], fmt)


# -------------------------------------------------------------------------- attention
def attend(q: np.ndarray, rows: np.ndarray, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Attention of queries q [H, 576] over rows [L, 576]; returns (out [H, 512], lse [H])."""
    H = q.shape[0]
    L = rows.shape[0]
    if L == 0:
        return np.zeros((H, LATENT)), np.full(H, -np.inf)
    s = float(scale) * (q @ rows.T)  # [H, L]
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m).sum(axis=1, keepdims=True)
    lse = m + np.log(z)
    p = np.exp(s - lse)  # softmax over the cache tokens
    return p @ rows[:, :LATENT], lse[:, 0]


def decode(q_bits, pool, block_table, seq_lens, page_size: int, scale: float, fmt: str,
           requests=None) -> tuple[np.ndarray, np.ndarray]:
    """Decode every request (or the listed ones) of a batch.

    q_bits: uint16 bf16 bits [B, H, 576]; pool: the cache bytes (any shape,
    row-major, num_slots * row_bytes bytes); block_table int32 [B, W];
    seq_lens [B]; scale: the softmax scale.  Returns out fp64 [B, H, 512] and
    lse fp64 [B, H]; requests not listed are left as NaN.
    """
    q = bf16_to_f64(q_bits)
    B, H, _ = q.shape
    out = np.full((B, H, LATENT), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        rows = gather_rows_fast(pool, block_table, b, int(seq_lens[b]), page_size, fmt)
        out[b], lse[b] = attend(q[b], rows, scale)
    return out, lse


def decode_mtp(q_bits, pool, block_table, seq_lens, page_size: int, scale: float, fmt: str,
               requests=None) -> tuple[np.ndarray, np.ndarray]:
    """Multi-token verify decode: q_bits [B, q_len, H, 576]; out [B, q_len, H, 512], lse [B, q_len, H].

    Query i of request b attends to its first max(0, L_b - q_len + 1 + i) tokens.
    """
    q = bf16_to_f64(q_bits)
    B, T, H, _ = q.shape
    out = np.full((B, T, H, LATENT), np.nan)
    lse = np.full((B, T, H), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(seq_lens[b])
        rows = gather_rows_fast(pool, block_table, b, L, page_size, fmt)
        for i in range(T):
            n = max(0, L - T + 1 + i)
            out[b, i], lse[b, i] = attend(q[b, i], rows[:n], scale)
    return out, lse


def decode_sparse(q_bits, pool, indices, scale: float, fmt: str, tokens=None) -> tuple[np.ndarray, np.ndarray]:
    """Sparse decode: q_bits [T, H, 576]; indices int [T, topk], the slots query t attends to
    (entries < 0 select nothing).  Returns out [T, H, 512], lse [T, H]; queries not listed in
    `tokens` are left as NaN.  q_bits [T, H, 512] is the NoPE-512 form (the layers the page
    serves through the sparse backend): scores over the latent values only, as decode_nope."""
    q = bf16_to_f64(q_bits)
    T, H, D = q.shape
    if D not in (ROW, LATENT):
        raise ValueError("sparse queries have 576 (or, NoPE-512, 512) values per head")
    rows_all = _pool_rows(pool, fmt)
    idx = np.asarray(indices, dtype=np.int64)
    out = np.full((T, H, LATENT), np.nan)
    lse = np.full((T, H), np.nan)
    for t in (range(T) if tokens is None else tokens):
        slots = idx[t][idx[t] >= 0]
        if (slots >= rows_all.shape[0]).any():
            raise IndexError(f"query {t}: slot outside the pool")
        out[t], lse[t] = attend(q[t], rows_from_bytes(rows_all[slots], fmt)[:, :D], scale)
    return out, lse


def attend_kv(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Attention of q [H, K] over keys [L, K] with values [L, V]: (out [H, V], lse [H])."""
    H = q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((H, values.shape[1])), np.full(H, -np.inf)
    s = float(scale) * (q @ keys.T)
    m = s.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
    return np.exp(s - lse) @ values, lse[:, 0]


def decode_gla2(q_bits, pool, block_table, seq_lens, page_size: int, scale: float, fmt: str,
                requests=None) -> tuple[np.ndarray, np.ndarray]:
    """GLA-g2 decode on the 576-value row: q_bits [B, H, 320] (group latent 256 ++ rope 64),
    H even; head h in group g = h // (H/2) scores latent[256g : 256g + 256] ++ rope.
    Returns out [B, H, 256], lse [B, H]."""
    q = bf16_to_f64(q_bits)
    B, H, D = q.shape
    if D != 256 + ROPE or H % 2:
        raise ValueError("GLA-g2 queries are [B, H, 320] with H even")
    out = np.full((B, H, 256), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        rows = gather_rows_fast(pool, block_table, b, int(seq_lens[b]), page_size, fmt)
        for g in range(2):
            hs = slice(g * H // 2, (g + 1) * H // 2)
            keys = np.concatenate([rows[:, 256 * g:256 * g + 256], rows[:, LATENT:]], axis=1)
            out[b, hs], lse[b, hs] = attend_kv(q[b, hs], keys, rows[:, 256 * g:256 * g + 256], scale)
    return out, lse


def decode_rank(q_bits, pool_bits, block_table, seq_lens, page_size: int, scale: float,
                requests=None) -> tuple[np.ndarray, np.ndarray]:
    """Decode of a rank-D layer: bf16 rows of D latent ++ 64 rope values, pool_bits uint16
    [num_slots, D + 64]; q_bits [B, H, D + 64].  out [B, H, D], lse [B, H]."""
    q = bf16_to_f64(q_bits)
    B, H, K = q.shape
    D = K - ROPE
    flat = np.asarray(pool_bits, dtype=np.uint16).reshape(-1, K)
    out = np.full((B, H, D), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(seq_lens[b])
        t = np.arange(L, dtype=np.int64)
        pages = np.asarray(block_table[b], dtype=np.int64)[t // page_size]
        rows = bf16_to_f64(flat[pages * page_size + t % page_size])
        out[b], lse[b] = attend_kv(q[b], rows, rows[:, :D], scale)
    return out, lse


def decode_nope(q_bits, pool, block_table, seq_lens, page_size: int, scale: float, fmt: str,
                requests=None) -> tuple[np.ndarray, np.ndarray]:
    """NoPE-512 decode: q_bits uint16 bf16 bits [B, H, 512]; scores s_t = scale * <q, latent_t>.

    Same pool, paging and results as decode; the rows' 64 rope values take no part,
    whatever bytes they hold.
    """
    q = bf16_to_f64(q_bits)
    B, H, D = q.shape
    if D != LATENT:
        raise ValueError("NoPE queries have 512 values per head")
    out = np.full((B, H, LATENT), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        rows = gather_rows_fast(pool, block_table, b, int(seq_lens[b]), page_size, fmt)[:, :LATENT]
        out[b], lse[b] = attend(q[b], rows, scale)
    return out, lse


def split_ranges(length: int, page_size: int, num_splits: int, width: int | None = None) -> list[tuple[int, int]]:
    """Token ranges of the partitions of one request (reading: whole pages per split).

    Partitions hold c = ceil(width / num_splits) whole pages, width being the block
    table's width (the most pages any request of the batch may use; default: this
    request's own page count P = ceil(L / ps)); split i covers pages
    [i*c, min((i+1)*c, P)), clipped to L tokens.  Trailing splits may be empty.  The
    merged result does not depend on this rule.
    """
    P = -(-length // page_size)
    c = max(1, -(-(P if width is None else width) // num_splits))
    out = []
    for i in range(num_splits):
        t0 = min(length, i * c * page_size)
        t1 = min(length, (i + 1) * c * page_size)
        out.append((t0, t1))
    return out


def merge(part_out: np.ndarray, part_lse: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Merge partials over disjoint token sets: part_out [S, ..., 512], part_lse [S, ...].

    M = max_p lse_p; if M = -inf the result is (0, -inf); otherwise
    w_p = exp(lse_p - M), lse = M + ln sum_p w_p, out = sum_p w_p out_p / sum_p w_p.
    """
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = part_lse.max(axis=0)
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp(part_lse - Ms)  # exp(-inf) = 0 for empty partitions
    W = w.sum(axis=0)
    Ws = np.where(empty, 1.0, W)
    out = (w[..., None] * part_out).sum(axis=0) / Ws[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, Ms + np.log(Ws))
    return out, lse


# --------------------------------------------------------------- context gather
def upconvert_rows(row_bytes: np.ndarray, fmt: str) -> np.ndarray:
    """bf16 bits [n, 576] of raw rows [n, row_bytes]: bf16 rows as stored; fp8 latent values
    bf16(fl32(code * scale)), rope values as stored."""
    row_bytes = np.ascontiguousarray(row_bytes, dtype=np.uint8)
    n = row_bytes.shape[0]
    if fmt == "bf16":
        return row_bytes.view("<u2").reshape(n, ROW).copy()
    codes = e4m3_decode(row_bytes[:, FP8_CODES]).astype(np.float32).reshape(n, 4, 128)  # exact
    scales = np.ascontiguousarray(row_bytes[:, FP8_SCALES]).view("<f4").reshape(n, 4, 1)
    prod = (codes * scales).astype(np.float32)  # IEEE float32 multiply
    out = np.empty((n, ROW), dtype=np.uint16)
    out[:, :LATENT] = f32_to_bf16_bits(prod.reshape(n, LATENT))
    out[:, LATENT:] = np.ascontiguousarray(row_bytes[:, FP8_ROPE]).view("<u2").reshape(n, ROPE)
    return out


def gather_context(pool, block_table, cu_rows, seq_starts, page_size: int, fmt: str) -> np.ndarray:
    """bf16 bits [cu_rows[-1], 576]: row cu_rows[b] + j is token seq_starts[b] + j of request b
    (seq_starts None: 0), upconverted as in upconvert_rows."""
    rows = _pool_rows(pool, fmt)
    cu_rows = np.asarray(cu_rows, dtype=np.int64)
    B = cu_rows.size - 1
    slots = []
    for b in range(B):
        start = 0 if seq_starts is None else int(seq_starts[b])
        for j in range(int(cu_rows[b + 1] - cu_rows[b])):
            slots.append(slot_of(block_table, b, start + j, page_size))
    slots = np.asarray(slots, dtype=np.int64)
    return upconvert_rows(rows[slots], fmt)


# ------------------------------------------------------------------------ cache write
def pack_rows(latent_bits: np.ndarray, k_pe_bits, fmt: str) -> np.ndarray:
    """Row bytes [T, row_bytes] for new tokens (latent [T, 512], k_pe [T, 64], bf16 bits).

    bf16: the 576 values latent ++ k_pe, little-endian (1152 bytes).
    fp8: per 128-value block a = max|x|, s = fl32(a/448), codes = e4m3(x/s);
    codes, then the 4 fp32 scales, then k_pe as bf16 (656 bytes).
    k_pe None (a NoPE layer): the rope part is written as zeros.
    """
    latent_bits = np.ascontiguousarray(latent_bits, dtype=np.uint16)
    T = latent_bits.shape[0]
    if k_pe_bits is None:
        k_pe_bits = np.zeros((T, ROPE), dtype=np.uint16)
    k_pe_bits = np.ascontiguousarray(k_pe_bits, dtype=np.uint16)
    if fmt == "bf16":
        row = np.concatenate([latent_bits, k_pe_bits], axis=1).astype("<u2")
        return row.view(np.uint8).reshape(T, ROW_BYTES["bf16"])
    s, codes = quantize_block128(latent_bits)
    out = np.empty((T, ROW_BYTES["fp8"]), dtype=np.uint8)
    out[:, FP8_CODES] = codes
    out[:, FP8_SCALES] = s.astype("<f4").view(np.uint8).reshape(T, 16)
    out[:, FP8_ROPE] = k_pe_bits.astype("<u2").view(np.uint8).reshape(T, 128)
    return out


def cache_write(pool: np.ndarray, latent_bits, k_pe_bits, slot_mapping, fmt: str) -> None:
    """Write new tokens' rows into the pool in place; negative slots are skipped."""
    rows = _pool_rows(pool, fmt)
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    keep = slot_mapping >= 0
    if (slot_mapping[keep] >= rows.shape[0]).any():
        raise IndexError("slot outside the pool")
    packed = pack_rows(np.asarray(latent_bits)[keep], None if k_pe_bits is None else np.asarray(k_pe_bits)[keep], fmt)
    rows[slot_mapping[keep]] = packed


"""Shared helpers for the GPU parity tests (not a test module).

The same seeded workload feeds both sides: the fp64 oracle builds its pool with
oracle.cache_write on the host, the HIP path builds its pool with mla_cache_write on
the device, the two pools are compared byte for byte, and then each side decodes its
own pool.
"""
import sys

import numpy as np
import torch

import oracle
import paged_mla_latent_amd as mla

FMT_CODE = {"bf16": mla.MLA_CACHE_BF16_576, "fp8": mla.MLA_CACHE_FP8_656}

# Parity bar: per (request, head) with a non-empty context,
# max_d |out - ref| <= OUT_REL * max_d |ref| and |lse - ref_lse| <= LSE_ABS.
OUT_REL = 1e-2
LSE_ABS = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def poisoned_device_pool(w) -> torch.Tensor:
    if w.fmt == "bf16":
        return torch.full((w.num_pages, w.page_size, 576), 0x7FC0, dtype=torch.int16, device="cuda").view(
            torch.bfloat16)
    return torch.full((w.num_pages, w.page_size, 656), 0xFF, dtype=torch.uint8, device="cuda")


def device_pool(w, latent=None, k_pe=None, slots=None, zero_rope=False) -> torch.Tensor:
    """Poisoned pool with the workload's rows written by mla_cache_write (zero_rope: k_pe NULL)."""
    pool = poisoned_device_pool(w)
    latent = w.latent if latent is None else latent
    k_pe = None if zero_rope else (w.k_pe if k_pe is None else k_pe)
    slots = w.slots if slots is None else slots
    mla.mla_cache_write(bf16_dev(latent), None if k_pe is None else bf16_dev(k_pe), torch.from_numpy(slots).cuda(),
                        pool, FMT_CODE[w.fmt])
    return pool


def host_pool(w, latent=None, k_pe=None, slots=None, zero_rope=False) -> np.ndarray:
    pool = w.poisoned_pool()
    oracle.cache_write(pool, w.latent if latent is None else latent,
                       None if zero_rope else (w.k_pe if k_pe is None else k_pe),
                       w.slots if slots is None else slots, w.fmt)
    return pool


def device_rows(pool: torch.Tensor, slots: np.ndarray, row_bytes: int) -> np.ndarray:
    """Raw bytes [len(slots), row_bytes] of the given slots, read back from the device pool."""
    flat = pool.view(torch.uint8).view(-1, row_bytes)
    idx = torch.from_numpy(np.ascontiguousarray(slots)).cuda()
    return flat.index_select(0, idx).cpu().numpy()


def assert_rows_bitexact(w, pool_dev: torch.Tensor, pool_host: np.ndarray, slots=None):
    slots = w.slots if slots is None else slots
    R = w.row_bytes
    got = device_rows(pool_dev, slots, R)
    want = pool_host.reshape(-1, R)[slots]
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first slot {slots[bad[0]]}"


def gpu_decode(w, pool: torch.Tensor, splits: int, q=None, nope=False, balanced=False, flags=0):
    """Decode on the device; nope=True uses the NoPE-512 kernels with the first 512 q values;
    balanced=True uses the batch-balanced kernels with `splits` workgroups; flags per call."""
    q = w.q if q is None else q
    if nope:
        q = np.ascontiguousarray(q[:, :, :512])
    q = bf16_dev(q)
    bt = torch.from_numpy(w.block_table).cuda()
    lens = torch.from_numpy(w.seq_lens).cuda()
    if balanced:
        if nope:
            fn = mla.mla_decode_balanced_nope_bf16 if w.fmt == "bf16" else mla.mla_decode_balanced_nope_fp8_656
        else:
            fn = mla.mla_decode_balanced_bf16 if w.fmt == "bf16" else mla.mla_decode_balanced_fp8_656
        out, lse = fn(q, pool, bt, lens, w.scale, num_workgroups=splits, flags=flags)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    if nope:
        fn = mla.mla_decode_nope_bf16 if w.fmt == "bf16" else mla.mla_decode_nope_fp8_656
    else:
        fn = mla.mla_decode_bf16 if w.fmt == "bf16" else mla.mla_decode_fp8_656
    out, lse = fn(q, pool, bt, lens, w.scale, num_splits=splits, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def assert_parity(w, out, lse, ref_out, ref_lse, requests=None, what=""):
    requests = range(w.batch) if requests is None else requests
    worst_rel, worst_lse = 0.0, 0.0
    for b in requests:
        if w.seq_lens[b] == 0:
            assert np.array_equal(out[b], np.zeros_like(out[b])) and not np.signbit(out[b]).any(), f"{what} b={b}"
            assert np.isneginf(lse[b]).all(), f"{what} b={b} lse {lse[b]}"
            continue
        assert np.isfinite(out[b]).all() and np.isfinite(lse[b]).all(), f"{what} b={b}: non-finite output"
        err = np.abs(out[b] - ref_out[b]).max(axis=1)
        scale = np.abs(ref_out[b]).max(axis=1)
        rel = err / scale
        dl = np.abs(lse[b] - ref_lse[b])
        worst_rel, worst_lse = max(worst_rel, rel.max()), max(worst_lse, dl.max())
        assert (err <= OUT_REL * scale).all(), f"{what} b={b}: out rel err {rel.max():.3e}"
        assert (dl <= LSE_ABS).all(), f"{what} b={b}: lse err {dl.max():.3e}"
    say(f"  {what}: worst out rel err {worst_rel:.2e}, worst lse err {worst_lse:.2e}")
    return worst_rel, worst_lse

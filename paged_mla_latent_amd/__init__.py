"""Python binding of libmla.so: paged MLA latent decode on AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream.  There is no
CPU path: if the library is missing, every call raises.

Entry points (same names as the C ABI in include/mla.h):

    mla_decode_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, ...)
    mla_decode_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, ...)
    mla_decode_nope_bf16 / mla_decode_nope_fp8_656(q [B, H, 512], ...)   NoPE-512 layers
    mla_decode_mtp_bf16 / mla_decode_mtp_fp8_656(q [B, q_len, H, 576], ...)   verify step
    mla_decode_rank256_bf16(q [B, H, 320], kv_cache [pages, ps, 320], ...)   rank-256 layer
    mla_decode_rank768_bf16 / mla_decode_rank1792_bf16(q [B, H, D + 64], ...)   rank-768 / 1792 layers
    mla_decode_gla2_bf16 / mla_decode_gla2_fp8_656(q [B, H, 320], ...)   GLA-g2 head groups
    mla_decode_balanced_bf16 / mla_decode_balanced_fp8_656(..., num_workgroups=0)   ragged batches
    mla_decode_balanced_nope_bf16 / mla_decode_balanced_nope_fp8_656(q [B, H, 512], ...)
    mla_merge_lse_width(part_out, part_lse, out=None, lse=None)   256- or 512-wide partials
    mla_merge_lse(part_out, part_lse, out=None, lse=None)
    mla_cache_write(latent, k_pe, slot_mapping, kv_cache, cache_format)   k_pe None: zero rope
    mla_gather_context(kv_cache, cache_format, block_table, cu_rows, total_rows, seq_starts=None)
    mla_decode_workspace_size(batch, num_heads, num_splits)
    mla_decode_balanced_workspace_size(batch, num_heads, num_workgroups)
    mla_merge_lse_balanced(workspace, batch, num_heads, num_workgroups, out=None, lse=None)

Every decode takes two per-call options: flags (MLA_FLAG_CACHED_ROWS: plain row loads for
batches that share pages within a step; 0: streaming loads) and check_status (a one-element
int32 device tensor the caller zeroes: the call then runs on the checked build,
libmla_checked.so, whose kernels OR MLA_CHECK_* bits into it when a block id lies outside the
pool or a length outside the block table).  The library keeps no other state.

Tensors: q bf16 [B, H, 576]; kv_cache bf16 [num_pages, page_size, 576] or uint8
[num_pages, page_size, 656]; block_table int32 [B, W]; seq_lens int32 [B];
out fp32 [B, H, 512]; lse fp32 [B, H]; latent bf16 [T, 512]; k_pe bf16 [T, 64];
slot_mapping int64 [T].  All on the same HIP device, contiguous.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
CHECKED_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_checked.so")

MLA_OK = 0
MLA_CACHE_BF16_576 = 0
MLA_CACHE_FP8_656 = 1
MLA_FLAG_CACHED_ROWS = 1
MLA_CHECK_BLOCK_ID = 1
MLA_CHECK_SEQ_LEN = 2
LATENT, ROPE, ROW = 512, 64, 576
ROW_BYTES = {MLA_CACHE_BF16_576: 1152, MLA_CACHE_FP8_656: 656}
MAX_HEADS = 16
MAX_Q_LEN = 16
MAX_QUERY_ROWS = 64
MLA_MAX_BALANCED_BATCH = 1024

EXPORTED = (
    "mla_decode_workspace_size", "mla_decode_bf16", "mla_decode_fp8_656", "mla_decode_nope_bf16",
    "mla_decode_nope_fp8_656", "mla_decode_mtp_bf16", "mla_decode_mtp_fp8_656", "mla_decode_rank256_bf16",
    "mla_decode_gla2_bf16", "mla_decode_gla2_fp8_656", "mla_merge_lse", "mla_merge_lse_width",
    "mla_cache_write", "mla_gather_context", "mla_status_string", "mla_last_error_message", "mla_abi_version",
    "mla_decode_balanced_workspace_size", "mla_decode_balanced_bf16", "mla_decode_balanced_fp8_656",
    "mla_merge_lse_balanced", "mla_decode_rank_workspace_size", "mla_decode_rank768_bf16",
    "mla_decode_rank1792_bf16", "mla_decode_balanced_nope_bf16", "mla_decode_balanced_nope_fp8_656",
    "mla_decode_mtp_balanced_bf16", "mla_decode_mtp_balanced_fp8_656", "mla_checked_build",
    "mla_check_preconditions_host", "mla_decode_bf16_noalloc", "mla_decode_sparse_bf16",
    "mla_decode_sparse_fp8_656", "mla_decode_sparse_nope_bf16", "mla_decode_sparse_nope_fp8_656",
    "mla_decode_gla2_balanced_bf16", "mla_decode_gla2_balanced_fp8_656", "mla_decode_append_bf16",
    "mla_decode_append_fp8_656", "mla_decode_append_balanced_bf16", "mla_decode_append_balanced_fp8_656",
)
MAX_SPARSE_TOKENS = 1 << 20
MAX_SPARSE_TOPK = 1 << 24
NOALLOC_SCRATCH_BYTES = 16 << 20


class MlaError(RuntimeError):
    """A libmla call returned a nonzero status."""

    def __init__(self, fn: str, status: int, name: str, message: str):
        super().__init__(f"{fn} failed: {name} ({status}): {message}")
        self.status = status


_libs: dict = {}


def library(checked: bool = False) -> ctypes.CDLL:
    """Load libmla.so, or with checked=True libmla_checked.so (once each).  Raises if it has not
    been built."""
    path = CHECKED_LIB_PATH if checked else LIB_PATH
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_mla_latent_amd.build`")
    lib = ctypes.CDLL(path)
    c_int, c_i32, c_i64, c_sz, c_f, vp = (ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                           ctypes.c_float, ctypes.c_void_p)
    lib.mla_decode_workspace_size.argtypes = [c_i32, c_i32, c_i32]
    lib.mla_decode_workspace_size.restype = c_sz
    lib.mla_decode_balanced_workspace_size.argtypes = [c_i32, c_i32, c_i32]
    lib.mla_decode_balanced_workspace_size.restype = c_sz
    c_u32 = ctypes.c_uint32
    dec = [vp, vp, c_i64, vp, c_i64, vp, c_i32, c_i32, c_i32, c_f, c_i32, vp, vp, vp, c_sz, c_u32, vp, vp]
    lib.mla_decode_rank_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32]
    lib.mla_decode_rank_workspace_size.restype = c_sz
    for name in ("mla_decode_bf16", "mla_decode_fp8_656", "mla_decode_nope_bf16", "mla_decode_nope_fp8_656",
                 "mla_decode_rank256_bf16", "mla_decode_gla2_bf16", "mla_decode_gla2_fp8_656",
                 "mla_decode_rank768_bf16", "mla_decode_rank1792_bf16",
                 "mla_decode_balanced_nope_bf16", "mla_decode_balanced_nope_fp8_656",
                 "mla_decode_balanced_bf16", "mla_decode_balanced_fp8_656", "mla_decode_gla2_balanced_bf16",
                 "mla_decode_gla2_balanced_fp8_656"):
        getattr(lib, name).argtypes = dec
        getattr(lib, name).restype = c_int
    mtp = [vp, vp, c_i64, vp, c_i64, vp, c_i32, c_i32, c_i32, c_i32, c_f, c_i32, vp, vp, vp, c_sz, c_u32, vp, vp]
    for name in ("mla_decode_mtp_bf16", "mla_decode_mtp_fp8_656", "mla_decode_mtp_balanced_bf16",
                 "mla_decode_mtp_balanced_fp8_656"):
        getattr(lib, name).argtypes = mtp
        getattr(lib, name).restype = c_int
    app = [vp, vp, vp, vp, vp, c_i64, vp, c_i64, vp, c_i32, c_i32, c_i32, c_i32, c_f, c_i32, vp, vp, vp, c_sz, c_u32,
           vp, vp]
    for name in ("mla_decode_append_bf16", "mla_decode_append_fp8_656", "mla_decode_append_balanced_bf16",
                 "mla_decode_append_balanced_fp8_656"):
        getattr(lib, name).argtypes = app
        getattr(lib, name).restype = c_int
    lib.mla_merge_lse_balanced.argtypes = [vp, c_sz, c_i32, c_i32, c_i32, vp, vp, vp]
    lib.mla_merge_lse_balanced.restype = c_int
    lib.mla_merge_lse.argtypes = [vp, vp, c_i32, c_i32, c_i32, vp, vp, vp]
    lib.mla_merge_lse.restype = c_int
    lib.mla_merge_lse_width.argtypes = [vp, vp, c_i32, c_i32, c_i32, c_i32, vp, vp, vp]
    lib.mla_merge_lse_width.restype = c_int
    lib.mla_cache_write.argtypes = [vp, vp, vp, c_i32, vp, c_i32, c_i64, vp]
    lib.mla_cache_write.restype = c_int
    lib.mla_gather_context.argtypes = [vp, c_i32, c_i64, c_i32, vp, c_i64, vp, vp, c_i32, c_i64, vp, vp, vp]
    lib.mla_gather_context.restype = c_int
    lib.mla_status_string.argtypes = [c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error_message.argtypes = []
    lib.mla_last_error_message.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = c_int
    lib.mla_decode_bf16_noalloc.argtypes = [vp, vp, c_i64, vp, c_i64, vp, c_i32, c_i32, c_i32, c_f, c_i32, vp, vp,
                                            c_u32, vp, vp]
    lib.mla_decode_bf16_noalloc.restype = c_int
    sparse = [vp, vp, c_i64, vp, c_i32, c_i32, c_i32, c_f, c_i32, vp, vp, vp, c_sz, c_u32, vp, vp]
    for name in ("mla_decode_sparse_bf16", "mla_decode_sparse_fp8_656", "mla_decode_sparse_nope_bf16",
                 "mla_decode_sparse_nope_fp8_656"):
        getattr(lib, name).argtypes = sparse
        getattr(lib, name).restype = c_int
    lib.mla_checked_build.argtypes = []
    lib.mla_checked_build.restype = c_int
    lib.mla_check_preconditions_host.argtypes = [vp, c_i64, vp, c_i32, c_i32, c_i64]
    lib.mla_check_preconditions_host.restype = c_int
    _libs[path] = lib
    return lib


def mla_check_preconditions_host(block_table, seq_lens, page_size: int, num_pages: int) -> int:
    """MLA_CHECK_* bits of host arrays (block_table int32 [B, W], seq_lens int32 [B]) against the
    decode preconditions; 0 when they hold."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if bt.ndim != 2 or lens.shape != (bt.shape[0],):
        raise ValueError("block_table must be [B, W] and seq_lens [B]")
    lib = library()
    rc = lib.mla_check_preconditions_host(bt.ctypes.data, bt.shape[1], lens.ctypes.data, bt.shape[0],
                                          int(page_size), int(num_pages))
    if rc < 0:
        _check("mla_check_preconditions_host", -rc)
    return rc


def _check(fn: str, status: int, lib=None) -> None:
    if status != MLA_OK:
        lib = lib or library()
        raise MlaError(fn, status, lib.mla_status_string(status).decode(), lib.mla_last_error_message().decode())


def _options(check_status, dev):
    """The library to call and the check_status pointer: a status tensor selects the checked build."""
    if check_status is None:
        return library(), None
    _need(check_status, "check_status", torch.int32, 1, dev)
    return library(checked=True), check_status.data_ptr()


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device: torch.device | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def mla_decode_workspace_size(batch: int, num_heads: int, num_splits: int) -> int:
    return int(library().mla_decode_workspace_size(batch, num_heads, num_splits))


def _decode(fn: str, cache_dtype: torch.dtype, row_bytes_last: int, q, kv_cache, block_table, seq_lens,
            softmax_scale, num_splits, out, lse, workspace, partials_only=False, q_dim=ROW, out_width=LATENT,
            flags=0, check_status=None):
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    _need(kv_cache, "kv_cache", cache_dtype, 3, dev)
    if kv_cache.shape[2] != row_bytes_last:
        raise ValueError(f"kv_cache rows must have {row_bytes_last} elements, got {kv_cache.shape[2]}")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, H, D = q.shape
    if D != q_dim:
        raise ValueError(f"q rows must have {q_dim} values, got {D}")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have one row per request")
    if partials_only:
        if num_splits < 2 or out is not None or lse is not None:
            raise ValueError("partials_only needs num_splits > 1 and no out/lse")
    else:
        if out is None:
            out = torch.empty((B, H, out_width), dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, 3, dev)
        _need(lse, "lse", torch.float32, 2, dev)
    ws_bytes = 0
    if num_splits > 1:
        need = (mla_decode_rank_workspace_size(B, H, num_splits, out_width) if out_width in (768, 1792)
                else mla_decode_workspace_size(B, H, num_splits))
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    status = getattr(lib, fn)(
        q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), B, H, kv_cache.shape[1], float(softmax_scale), int(num_splits),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, int(flags), status_ptr, _stream(dev))
    _check(fn, status, lib)
    if partials_only:
        n = num_splits * B * H
        flat = workspace.view(torch.uint8)[: n * (out_width + 1) * 4].view(torch.float32)
        return flat[: n * out_width].view(num_splits, B, H, out_width), flat[n * out_width:].view(num_splits, B, H)
    return out, lse


def mla_decode_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                    workspace=None, partials_only=False, flags=0, check_status=None):
    """Decode over a bf16 cache [num_pages, page_size, 576]; returns (out [B,H,512], lse [B,H]).

    partials_only=True (num_splits > 1) skips the merge and returns the partials
    (part_out [S,B,H,512], part_lse [S,B,H]) as views of the workspace.
    """
    return _decode("mla_decode_bf16", torch.bfloat16, ROW, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only,
                   flags=flags, check_status=check_status)


def mla_decode_bf16_noalloc(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                            flags=0, check_status=None):
    """mla_decode_bf16 without a workspace: the split partials go to the library's 16 MiB
    per-device scratch (for callers that cannot allocate; calls on one device must not overlap).
    out / lse are allocated here when not given (the library itself allocates nothing)."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    _need(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, H, D = q.shape
    if D != ROW or kv_cache.shape[2] != ROW:
        raise ValueError("q and kv_cache rows must have 576 values")
    if out is None:
        out = torch.empty((B, H, LATENT), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    status = lib.mla_decode_bf16_noalloc(
        q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), B, H, kv_cache.shape[1], float(softmax_scale), int(num_splits), out.data_ptr(),
        lse.data_ptr(), int(flags), status_ptr, _stream(dev))
    _check("mla_decode_bf16_noalloc", status, lib)
    return out, lse


def mla_decode_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                       workspace=None, partials_only=False, flags=0, check_status=None):
    """Decode over an fp8 cache uint8 [num_pages, page_size, 656]; returns (out, lse) or the partials."""
    return _decode("mla_decode_fp8_656", torch.uint8, 656, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only,
                   flags=flags, check_status=check_status)


def mla_decode_nope_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                         workspace=None, partials_only=False, flags=0, check_status=None):
    """NoPE-512 decode over a bf16 cache: q [B, H, 512]; the rows' rope part is never read."""
    return _decode("mla_decode_nope_bf16", torch.bfloat16, ROW, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=LATENT,
                   flags=flags, check_status=check_status)


def mla_decode_nope_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                            workspace=None, partials_only=False, flags=0, check_status=None):
    """NoPE-512 decode over an fp8 cache: q [B, H, 512]; the rows' rope bytes are never read."""
    return _decode("mla_decode_nope_fp8_656", torch.uint8, 656, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=LATENT,
                   flags=flags, check_status=check_status)


def _decode_sparse(fn: str, cache_dtype: torch.dtype, row_elems: int, q_dim: int, q, kv_cache, indices,
                   softmax_scale, num_splits, out, lse, workspace, flags, check_status, partials_only=False):
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    if not isinstance(kv_cache, torch.Tensor) or kv_cache.dim() not in (2, 3):
        raise ValueError("kv_cache must be [num_slots, row] or [num_pages, page_size, row]")
    _need(kv_cache, "kv_cache", cache_dtype, kv_cache.dim(), dev)
    if kv_cache.shape[-1] != row_elems:
        raise ValueError(f"kv_cache rows must have {row_elems} elements, got {kv_cache.shape[-1]}")
    _need(indices, "indices", torch.int32, 2, dev)
    T, H, D = q.shape
    if D != q_dim:
        raise ValueError(f"q rows must have {q_dim} values, got {D}")
    if indices.shape[0] != T:
        raise ValueError("indices must have one row per query token")
    if partials_only:
        if num_splits < 2 or out is not None or lse is not None:
            raise ValueError("partials_only needs num_splits > 1 and no out/lse")
    else:
        if out is None:
            out = torch.empty((T, H, LATENT), dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, 3, dev)
        _need(lse, "lse", torch.float32, 2, dev)
    ws_bytes = 0
    if num_splits > 1:
        if workspace is None:
            workspace = torch.empty(mla_decode_workspace_size(T, H, num_splits), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    num_slots = kv_cache.numel() // row_elems
    status = getattr(lib, fn)(
        q.data_ptr(), kv_cache.data_ptr(), num_slots, indices.data_ptr(), indices.shape[1], T, H,
        float(softmax_scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        int(flags), status_ptr, _stream(dev))
    _check(fn, status, lib)
    if partials_only:
        n = num_splits * T * H
        flat = workspace.view(torch.uint8)[: n * (LATENT + 1) * 4].view(torch.float32)
        return flat[: n * LATENT].view(num_splits, T, H, LATENT), flat[n * LATENT:].view(num_splits, T, H)
    return out, lse


def mla_decode_sparse_bf16(q, kv_cache, indices, softmax_scale, num_splits=1, out=None, lse=None, workspace=None,
                           flags=0, check_status=None, partials_only=False):
    """Decode over per-query index lists: q [T, H, 576], kv_cache bf16 [..., 576] (its slots),
    indices int32 [T, topk] (negative entries select nothing); returns (out [T,H,512], lse [T,H])."""
    return _decode_sparse("mla_decode_sparse_bf16", torch.bfloat16, ROW, ROW, q, kv_cache, indices, softmax_scale,
                          num_splits, out, lse, workspace, flags, check_status, partials_only)


def mla_decode_sparse_fp8_656(q, kv_cache, indices, softmax_scale, num_splits=1, out=None, lse=None,
                              workspace=None, flags=0, check_status=None, partials_only=False):
    """Index-list decode over an fp8 cache uint8 [..., 656]."""
    return _decode_sparse("mla_decode_sparse_fp8_656", torch.uint8, 656, ROW, q, kv_cache, indices, softmax_scale,
                          num_splits, out, lse, workspace, flags, check_status, partials_only)


def mla_decode_sparse_nope_bf16(q, kv_cache, indices, softmax_scale, num_splits=1, out=None, lse=None,
                                workspace=None, flags=0, check_status=None, partials_only=False):
    """NoPE-512 index-list decode over a bf16 cache: q [T, H, 512]."""
    return _decode_sparse("mla_decode_sparse_nope_bf16", torch.bfloat16, ROW, LATENT, q, kv_cache, indices,
                          softmax_scale, num_splits, out, lse, workspace, flags, check_status, partials_only)


def mla_decode_sparse_nope_fp8_656(q, kv_cache, indices, softmax_scale, num_splits=1, out=None, lse=None,
                                   workspace=None, flags=0, check_status=None, partials_only=False):
    """NoPE-512 index-list decode over an fp8 cache: q [T, H, 512]."""
    return _decode_sparse("mla_decode_sparse_nope_fp8_656", torch.uint8, 656, LATENT, q, kv_cache, indices,
                          softmax_scale, num_splits, out, lse, workspace, flags, check_status, partials_only)


def mla_decode_balanced_workspace_size(batch: int, num_heads: int, num_workgroups: int) -> int:
    return int(library().mla_decode_balanced_workspace_size(batch, num_heads, num_workgroups))


def _decode_balanced(fn: str, cache_dtype: torch.dtype, row_bytes_last: int, q, kv_cache, block_table, seq_lens,
                     softmax_scale, num_workgroups, out, lse, workspace, partials_only=False, q_dim=ROW, flags=0,
                     check_status=None, out_width=LATENT):
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    _need(kv_cache, "kv_cache", cache_dtype, 3, dev)
    if kv_cache.shape[2] != row_bytes_last:
        raise ValueError(f"kv_cache rows must have {row_bytes_last} elements, got {kv_cache.shape[2]}")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, H, D = q.shape
    if D != q_dim:
        raise ValueError(f"q rows must have {q_dim} values, got {D}")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have one row per request")
    if partials_only:
        if out is not None or lse is not None:
            raise ValueError("partials_only takes no out/lse")
    else:
        if out is None:
            out = torch.empty((B, H, out_width), dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, 3, dev)
        _need(lse, "lse", torch.float32, 2, dev)
    if workspace is None:
        need = mla_decode_balanced_workspace_size(B, H, num_workgroups)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    status = getattr(lib, fn)(
        q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), B, H, kv_cache.shape[1], float(softmax_scale), int(num_workgroups),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), int(flags), status_ptr,
        _stream(dev))
    _check(fn, status, lib)
    return workspace if partials_only else (out, lse)


def mla_decode_balanced_nope_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0, out=None,
                                  lse=None, workspace=None, partials_only=False, flags=0, check_status=None):
    """Batch-balanced NoPE-512 decode over a bf16 cache: q [B, H, 512]."""
    return _decode_balanced("mla_decode_balanced_nope_bf16", torch.bfloat16, ROW, q, kv_cache, block_table,
                            seq_lens, softmax_scale, num_workgroups, out, lse, workspace, partials_only, q_dim=LATENT,
                            flags=flags, check_status=check_status)


def mla_decode_balanced_nope_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0,
                                     out=None, lse=None, workspace=None, partials_only=False, flags=0, check_status=None):
    """Batch-balanced NoPE-512 decode over an fp8 cache: q [B, H, 512]."""
    return _decode_balanced("mla_decode_balanced_nope_fp8_656", torch.uint8, 656, q, kv_cache, block_table,
                            seq_lens, softmax_scale, num_workgroups, out, lse, workspace, partials_only, q_dim=LATENT,
                            flags=flags, check_status=check_status)


def mla_merge_lse_balanced(workspace, batch, num_heads, num_workgroups, out=None, lse=None):
    """Merge the partials a balanced decode left in `workspace` (partials_only=True).  After a
    balanced verify step num_heads is q_len * heads and out / lse are [B, q_len * heads, ...]."""
    lib = library()
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on a HIP device")
    dev = workspace.device
    if out is None:
        out = torch.empty((batch, num_heads, LATENT), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((batch, num_heads), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    status = lib.mla_merge_lse_balanced(workspace.data_ptr(), workspace.numel() * workspace.element_size(), batch,
                                        num_heads, num_workgroups, out.data_ptr(), lse.data_ptr(), _stream(dev))
    _check("mla_merge_lse_balanced", status)
    return out, lse


def mla_decode_balanced_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0, out=None,
                             lse=None, workspace=None, partials_only=False, flags=0, check_status=None):
    """Batch-balanced decode over a bf16 cache (B <= 1024): the batch's tokens cut into
    num_workgroups equal-cost ranges across request boundaries; returns (out [B,H,512], lse [B,H])."""
    return _decode_balanced("mla_decode_balanced_bf16", torch.bfloat16, ROW, q, kv_cache, block_table, seq_lens,
                            softmax_scale, num_workgroups, out, lse, workspace, partials_only,
                            flags=flags, check_status=check_status)


def mla_decode_balanced_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0, out=None,
                                lse=None, workspace=None, partials_only=False, flags=0, check_status=None):
    """Batch-balanced decode over an fp8 cache uint8 [num_pages, page_size, 656]."""
    return _decode_balanced("mla_decode_balanced_fp8_656", torch.uint8, 656, q, kv_cache, block_table, seq_lens,
                            softmax_scale, num_workgroups, out, lse, workspace, partials_only,
                            flags=flags, check_status=check_status)


def _decode_mtp(fn: str, cache_dtype: torch.dtype, row_bytes_last: int, q, kv_cache, block_table, seq_lens,
                softmax_scale, num_splits, out, lse, workspace, partials_only=False, flags=0, check_status=None):
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    _need(kv_cache, "kv_cache", cache_dtype, 3, dev)
    if kv_cache.shape[2] != row_bytes_last:
        raise ValueError(f"kv_cache rows must have {row_bytes_last} elements, got {kv_cache.shape[2]}")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, T, H, D = q.shape
    if D != ROW:
        raise ValueError(f"q rows must have {ROW} values, got {D}")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have one row per request")
    if partials_only:
        if num_splits < 2 or out is not None or lse is not None:
            raise ValueError("partials_only needs num_splits > 1 and no out/lse")
    else:
        if out is None:
            out = torch.empty((B, T, H, LATENT), dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, 4, dev)
        _need(lse, "lse", torch.float32, 3, dev)
    ws_bytes = 0
    if num_splits > 1:
        need = mla_decode_workspace_size(B, T * H, num_splits)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    status = getattr(lib, fn)(
        q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), B, T, H, kv_cache.shape[1], float(softmax_scale), int(num_splits),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, int(flags), status_ptr, _stream(dev))
    _check(fn, status, lib)
    if partials_only:  # [S, B, q_len * H, 512] / [S, B, q_len * H]: query rows act as heads
        n = num_splits * B * T * H
        flat = workspace.view(torch.uint8)[: n * (LATENT + 1) * 4].view(torch.float32)
        return flat[: n * LATENT].view(num_splits, B, T * H, LATENT), flat[n * LATENT:].view(num_splits, B, T * H)
    return out, lse


def _decode_mtp_balanced(fn: str, cache_dtype: torch.dtype, row_bytes_last: int, q, kv_cache, block_table, seq_lens,
                         softmax_scale, num_workgroups, out, lse, workspace, partials_only=False, flags=0,
                         check_status=None):
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    _need(kv_cache, "kv_cache", cache_dtype, 3, dev)
    if kv_cache.shape[2] != row_bytes_last:
        raise ValueError(f"kv_cache rows must have {row_bytes_last} elements, got {kv_cache.shape[2]}")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, T, H, D = q.shape
    if D != ROW:
        raise ValueError(f"q rows must have {ROW} values, got {D}")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have one row per request")
    if partials_only:
        if out is not None or lse is not None:
            raise ValueError("partials_only takes no out/lse")
    else:
        if out is None:
            out = torch.empty((B, T, H, LATENT), dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, 4, dev)
        _need(lse, "lse", torch.float32, 3, dev)
    if workspace is None:
        need = mla_decode_balanced_workspace_size(B, T * H, num_workgroups)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    status = getattr(lib, fn)(
        q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0], block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), B, T, H, kv_cache.shape[1], float(softmax_scale), int(num_workgroups),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), int(flags), status_ptr,
        _stream(dev))
    _check(fn, status, lib)
    return workspace if partials_only else (out, lse)


def mla_decode_mtp_balanced_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0, out=None,
                                 lse=None, workspace=None, partials_only=False, flags=0, check_status=None):
    """Batch-balanced verify step over a bf16 cache: q [B, q_len, H, 576] -> (out [B, q_len, H, 512],
    lse [B, q_len, H]); partials_only=True returns the workspace for mla_merge_lse_balanced(ws, B,
    q_len * H, num_workgroups)."""
    return _decode_mtp_balanced("mla_decode_mtp_balanced_bf16", torch.bfloat16, ROW, q, kv_cache, block_table,
                                seq_lens, softmax_scale, num_workgroups, out, lse, workspace, partials_only,
                                flags=flags, check_status=check_status)


def mla_decode_mtp_balanced_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0,
                                    out=None, lse=None, workspace=None, partials_only=False, flags=0, check_status=None):
    """Batch-balanced verify step over an fp8 cache uint8 [num_pages, page_size, 656]."""
    return _decode_mtp_balanced("mla_decode_mtp_balanced_fp8_656", torch.uint8, 656, q, kv_cache, block_table,
                                seq_lens, softmax_scale, num_workgroups, out, lse, workspace, partials_only,
                                flags=flags, check_status=check_status)


def mla_decode_mtp_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                        workspace=None, partials_only=False, flags=0, check_status=None):
    """Verify-step decode over a bf16 cache: q [B, q_len, H, 576] -> (out [B, q_len, H, 512], lse [B, q_len, H]).

    seq_lens count the q_len new tokens; query i sees tokens 0 .. L - q_len + i.
    partials_only=True (num_splits > 1) returns the partials [S, B, q_len * H, ...] instead."""
    return _decode_mtp("mla_decode_mtp_bf16", torch.bfloat16, ROW, q, kv_cache, block_table, seq_lens,
                       softmax_scale, num_splits, out, lse, workspace, partials_only,
                       flags=flags, check_status=check_status)


def mla_decode_mtp_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                           workspace=None, partials_only=False, flags=0, check_status=None):
    """Verify-step decode over an fp8 cache uint8 [num_pages, page_size, 656]."""
    return _decode_mtp("mla_decode_mtp_fp8_656", torch.uint8, 656, q, kv_cache, block_table, seq_lens,
                       softmax_scale, num_splits, out, lse, workspace, partials_only,
                       flags=flags, check_status=check_status)


def _decode_append(fn: str, cache_dtype: torch.dtype, row_bytes_last: int, balanced: bool, q, new_latent, new_k_pe,
                   new_slots, kv_cache, block_table, seq_lens, softmax_scale, count, out, lse, workspace,
                   partials_only=False, flags=0, check_status=None):
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    lib, status_ptr = _options(check_status, dev)
    _need(kv_cache, "kv_cache", cache_dtype, 3, dev)
    if kv_cache.shape[2] != row_bytes_last:
        raise ValueError(f"kv_cache rows must have {row_bytes_last} elements, got {kv_cache.shape[2]}")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, T, H, D = q.shape
    if D != ROW:
        raise ValueError(f"q rows must have {ROW} values, got {D}")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have one row per request")
    _need(new_latent, "new_latent", torch.bfloat16, 3, dev)
    _need(new_slots, "new_slots", torch.int64, 2, dev)
    if new_k_pe is not None:
        _need(new_k_pe, "new_k_pe", torch.bfloat16, 3, dev)
    if (tuple(new_latent.shape) != (B, T, LATENT) or tuple(new_slots.shape) != (B, T)
            or (new_k_pe is not None and tuple(new_k_pe.shape) != (B, T, ROPE))):
        raise ValueError("new_latent must be [B, q_len, 512], new_k_pe [B, q_len, 64] (or None), new_slots [B, q_len]")
    if partials_only:
        if out is not None or lse is not None or (not balanced and count < 2):
            raise ValueError("partials_only takes no out/lse (and, per request, num_splits > 1)")
    else:
        if out is None:
            out = torch.empty((B, T, H, LATENT), dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, 4, dev)
        _need(lse, "lse", torch.float32, 3, dev)
    if balanced:
        if workspace is None:
            workspace = torch.empty(max(mla_decode_balanced_workspace_size(B, T * H, count), 1), dtype=torch.uint8,
                                    device=dev)
    elif count > 1 and workspace is None:
        workspace = torch.empty(mla_decode_workspace_size(B, T * H, count), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = getattr(lib, fn)(
        q.data_ptr(), new_latent.data_ptr(), _ptr(new_k_pe), new_slots.data_ptr(), kv_cache.data_ptr(),
        kv_cache.shape[0], block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(), B, T, H,
        kv_cache.shape[1], float(softmax_scale), int(count), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        int(flags), status_ptr, _stream(dev))
    _check(fn, status, lib)
    if partials_only and balanced:
        return workspace
    if partials_only:  # [S, B, q_len * H, 512] / [S, B, q_len * H]: query rows act as heads
        n = count * B * T * H
        flat = workspace.view(torch.uint8)[: n * (LATENT + 1) * 4].view(torch.float32)
        return flat[: n * LATENT].view(count, B, T * H, LATENT), flat[n * LATENT:].view(count, B, T * H)
    return out, lse


def mla_decode_append_bf16(q, new_latent, new_k_pe, new_slots, kv_cache, block_table, seq_lens, softmax_scale,
                           num_splits=1, out=None, lse=None, workspace=None, partials_only=False, flags=0,
                           check_status=None):
    """Decode step that writes its new rows itself: new_latent [B, q_len, 512], new_k_pe [B, q_len, 64]
    (or None), new_slots int64 [B, q_len] go into the bf16 cache (row i of request b is position
    L_b - q_len + i), then q [B, q_len, H, 576] is decoded as by mla_decode_mtp_bf16."""
    return _decode_append("mla_decode_append_bf16", torch.bfloat16, ROW, False, q, new_latent, new_k_pe, new_slots,
                          kv_cache, block_table, seq_lens, softmax_scale, num_splits, out, lse, workspace,
                          partials_only, flags=flags, check_status=check_status)


def mla_decode_append_fp8_656(q, new_latent, new_k_pe, new_slots, kv_cache, block_table, seq_lens, softmax_scale,
                              num_splits=1, out=None, lse=None, workspace=None, partials_only=False, flags=0,
                              check_status=None):
    """mla_decode_append_bf16 over an fp8 cache uint8 [num_pages, page_size, 656] (rows quantised as
    mla_cache_write quantises them)."""
    return _decode_append("mla_decode_append_fp8_656", torch.uint8, 656, False, q, new_latent, new_k_pe, new_slots,
                          kv_cache, block_table, seq_lens, softmax_scale, num_splits, out, lse, workspace,
                          partials_only, flags=flags, check_status=check_status)


def mla_decode_append_balanced_bf16(q, new_latent, new_k_pe, new_slots, kv_cache, block_table, seq_lens,
                                    softmax_scale, num_workgroups=0, out=None, lse=None, workspace=None,
                                    partials_only=False, flags=0, check_status=None):
    """mla_decode_append_bf16 under the batch-balanced schedule (as mla_decode_mtp_balanced_bf16);
    partials_only=True returns the workspace for mla_merge_lse_balanced(ws, B, q_len * H, num_workgroups)."""
    return _decode_append("mla_decode_append_balanced_bf16", torch.bfloat16, ROW, True, q, new_latent, new_k_pe,
                          new_slots, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups, out, lse,
                          workspace, partials_only, flags=flags, check_status=check_status)


def mla_decode_append_balanced_fp8_656(q, new_latent, new_k_pe, new_slots, kv_cache, block_table, seq_lens,
                                       softmax_scale, num_workgroups=0, out=None, lse=None, workspace=None,
                                       partials_only=False, flags=0, check_status=None):
    """mla_decode_append_balanced_bf16 over an fp8 cache uint8 [num_pages, page_size, 656]."""
    return _decode_append("mla_decode_append_balanced_fp8_656", torch.uint8, 656, True, q, new_latent, new_k_pe,
                          new_slots, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups, out, lse,
                          workspace, partials_only, flags=flags, check_status=check_status)


def mla_decode_rank256_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                            workspace=None, partials_only=False, flags=0, check_status=None):
    """Rank-256 layer: kv_cache bf16 [pages, ps, 320], q [B, H, 320] -> out [B, H, 256], lse [B, H]."""
    return _decode("mla_decode_rank256_bf16", torch.bfloat16, 320, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=320, out_width=256,
                   flags=flags, check_status=check_status)


def mla_decode_rank_workspace_size(batch: int, num_heads: int, num_splits: int, latent_rank: int) -> int:
    return int(library().mla_decode_rank_workspace_size(batch, num_heads, num_splits, latent_rank))


def mla_decode_rank768_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                            workspace=None, partials_only=False, flags=0, check_status=None):
    """Rank-768 layer: kv_cache bf16 [pages, ps, 832], q [B, H, 832] -> out [B, H, 768], lse [B, H]."""
    return _decode("mla_decode_rank768_bf16", torch.bfloat16, 832, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=832, out_width=768,
                   flags=flags, check_status=check_status)


def mla_decode_rank1792_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                             workspace=None, partials_only=False, flags=0, check_status=None):
    """Rank-1792 layer: kv_cache bf16 [pages, ps, 1856], q [B, H, 1856] -> out [B, H, 1792], lse [B, H]."""
    return _decode("mla_decode_rank1792_bf16", torch.bfloat16, 1856, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=1856, out_width=1792,
                   flags=flags, check_status=check_status)


def mla_decode_gla2_balanced_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0, out=None,
                                  lse=None, workspace=None, flags=0, check_status=None):
    """GLA-g2 under the batch-balanced schedule, bf16 rows: q [B, H, 320] (H even) -> out [B, H, 256],
    lse [B, H]."""
    return _decode_balanced("mla_decode_gla2_balanced_bf16", torch.bfloat16, ROW, q, kv_cache, block_table,
                            seq_lens, softmax_scale, num_workgroups, out, lse, workspace, q_dim=320, flags=flags,
                            check_status=check_status, out_width=256)


def mla_decode_gla2_balanced_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_workgroups=0, out=None,
                                     lse=None, workspace=None, flags=0, check_status=None):
    """GLA-g2 under the batch-balanced schedule, fp8 656-byte rows: q [B, H, 320] (H even)."""
    return _decode_balanced("mla_decode_gla2_balanced_fp8_656", torch.uint8, 656, q, kv_cache, block_table,
                            seq_lens, softmax_scale, num_workgroups, out, lse, workspace, q_dim=320, flags=flags,
                            check_status=check_status, out_width=256)


def mla_decode_gla2_bf16(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                         workspace=None, partials_only=False, flags=0, check_status=None):
    """GLA-g2 on the 576-value row: q [B, H, 320] (H even) -> out [B, H, 256], lse [B, H]."""
    return _decode("mla_decode_gla2_bf16", torch.bfloat16, ROW, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=320, out_width=256,
                   flags=flags, check_status=check_status)


def mla_decode_gla2_fp8_656(q, kv_cache, block_table, seq_lens, softmax_scale, num_splits=1, out=None, lse=None,
                            workspace=None, partials_only=False, flags=0, check_status=None):
    """GLA-g2 on the 656-byte fp8 row: q [B, H, 320] (H even) -> out [B, H, 256], lse [B, H]."""
    return _decode("mla_decode_gla2_fp8_656", torch.uint8, 656, q, kv_cache, block_table, seq_lens,
                   softmax_scale, num_splits, out, lse, workspace, partials_only, q_dim=320, out_width=256,
                   flags=flags, check_status=check_status)


def mla_merge_lse_width(part_out, part_lse, out=None, lse=None):
    """Merge partials [S, B, R, W] / [S, B, R], W = 256, 512, 768 or 1792; returns (out [B, R, W], lse [B, R])."""
    lib = library()
    _need(part_out, "part_out", torch.float32, 4)
    dev = part_out.device
    _need(part_lse, "part_lse", torch.float32, 3, dev)
    S, B, R, W = part_out.shape
    if tuple(part_lse.shape) != (S, B, R):
        raise ValueError("part_lse must be [S, B, R]")
    if out is None:
        out = torch.empty((B, R, W), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, R), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    _check("mla_merge_lse_width", lib.mla_merge_lse_width(part_out.data_ptr(), part_lse.data_ptr(), S, B, R, W,
                                                          out.data_ptr(), lse.data_ptr(), _stream(dev)))
    return out, lse


def mla_merge_lse(part_out, part_lse, out=None, lse=None):
    """Merge partials [S, B, H, 512] / [S, B, H] by log-sum-exp; returns (out, lse)."""
    lib = library()
    _need(part_out, "part_out", torch.float32, 4)
    dev = part_out.device
    _need(part_lse, "part_lse", torch.float32, 3, dev)
    S, B, H, D = part_out.shape
    if D != LATENT or tuple(part_lse.shape) != (S, B, H):
        raise ValueError("part_out must be [S, B, H, 512] and part_lse [S, B, H]")
    if out is None:
        out = torch.empty((B, H, LATENT), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    _check("mla_merge_lse", lib.mla_merge_lse(part_out.data_ptr(), part_lse.data_ptr(), S, B, H,
                                              out.data_ptr(), lse.data_ptr(), _stream(dev)))
    return out, lse


def mla_cache_write(latent, k_pe, slot_mapping, kv_cache, cache_format):
    """Write rows for new tokens at slot_mapping (negative = skip) into kv_cache.

    k_pe None (a NoPE layer) writes zeros into the rows' rope part."""
    lib = library()
    _need(latent, "latent", torch.bfloat16, 2)
    dev = latent.device
    if k_pe is not None:
        _need(k_pe, "k_pe", torch.bfloat16, 2, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    if cache_format == MLA_CACHE_BF16_576:
        _need(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
        if kv_cache.shape[2] != ROW:
            raise ValueError("bf16 kv_cache rows must have 576 values")
    elif cache_format == MLA_CACHE_FP8_656:
        _need(kv_cache, "kv_cache", torch.uint8, 3, dev)
        if kv_cache.shape[2] != 656:
            raise ValueError("fp8 kv_cache rows must have 656 bytes")
    else:
        raise ValueError(f"unknown cache_format {cache_format}")
    T = latent.shape[0]
    if latent.shape[1] != LATENT or slot_mapping.shape[0] != T or (k_pe is not None and tuple(k_pe.shape) != (T, ROPE)):
        raise ValueError("latent must be [T, 512], k_pe [T, 64] (or None), slot_mapping [T]")
    num_slots = kv_cache.shape[0] * kv_cache.shape[1]
    _check("mla_cache_write", lib.mla_cache_write(latent.data_ptr(), _ptr(k_pe), slot_mapping.data_ptr(), T,
                                                  kv_cache.data_ptr(), int(cache_format), num_slots, _stream(dev)))


def mla_gather_context(kv_cache, cache_format, block_table, cu_rows, total_rows, seq_starts=None, out=None,
                       check_status=None):
    """Context rows of every request as bf16 [total_rows, 576] (fp8 rows upconverted).

    cu_rows int64 [B + 1] on the device (request b fills rows cu_rows[b] .. cu_rows[b+1]),
    total_rows = cu_rows[B] as a host int; seq_starts int32 [B] (None: gather from token 0);
    check_status: as for the decodes (runs the checked build)."""
    if cache_format == MLA_CACHE_BF16_576:
        _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    elif cache_format == MLA_CACHE_FP8_656:
        _need(kv_cache, "kv_cache", torch.uint8, 3)
    else:
        raise ValueError(f"unknown cache_format {cache_format}")
    dev = kv_cache.device
    lib, status_ptr = _options(check_status, dev)
    if kv_cache.shape[2] != (ROW if cache_format == MLA_CACHE_BF16_576 else 656):
        raise ValueError("kv_cache rows have the wrong width for cache_format")
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(cu_rows, "cu_rows", torch.int64, 1, dev)
    B = block_table.shape[0]
    if cu_rows.shape[0] != B + 1:
        raise ValueError("cu_rows must have batch + 1 entries")
    if seq_starts is not None:
        _need(seq_starts, "seq_starts", torch.int32, 1, dev)
        if seq_starts.shape[0] != B:
            raise ValueError("seq_starts must have one entry per request")
    if out is None:
        out = torch.empty((int(total_rows), ROW), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 2, dev)
    if out.shape[0] < total_rows or out.shape[1] != ROW:
        raise ValueError("out must be [total_rows, 576]")
    _check("mla_gather_context", lib.mla_gather_context(
        kv_cache.data_ptr(), int(cache_format), kv_cache.shape[0], kv_cache.shape[1], block_table.data_ptr(),
        block_table.shape[1], cu_rows.data_ptr(), _ptr(seq_starts), B, int(total_rows), out.data_ptr(),
        status_ptr, _stream(dev)), lib)
    return out

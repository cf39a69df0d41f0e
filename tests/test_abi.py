"""The C ABI boundary without a GPU: symbols, versions, argument validation.

Every call below carries at least one invalid argument, so the library must refuse
it on the host before touching any device; none of these tests launches a kernel.
"""
import ctypes
import os
import re

import pytest

import paged_mla_latent_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built (run __graft_entry__.build())")
    return mla.library()


def test_header_declares_the_four_operations():
    names = _declared_functions()
    for op in ("mla_decode_bf16", "mla_decode_fp8_656", "mla_merge_lse", "mla_cache_write"):
        assert op in names
    assert set(names) == set(mla.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(mla.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_only_the_c_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True, text=True).stdout
    text_syms = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert sorted(text_syms) == sorted(mla.EXPORTED)


def test_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 2
    names = [lib.mla_status_string(i).decode() for i in range(8)]
    assert names[:7] == ["MLA_OK", "MLA_ERR_NULL", "MLA_ERR_SHAPE", "MLA_ERR_ALIGN", "MLA_ERR_WORKSPACE",
                         "MLA_ERR_ARCH", "MLA_ERR_HIP"]
    assert names[7] == "MLA_ERR_UNKNOWN"


def test_workspace_size_formula(lib):
    assert mla.mla_decode_workspace_size(4, 16, 1) == 0
    n = 64 * 4 * 16
    want = (n * 513 * 4 + 64 + 255) // 256 * 256
    assert mla.mla_decode_workspace_size(4, 16, 64) == want
    assert mla.mla_decode_workspace_size(0, 16, 4) == 0 and mla.mla_decode_workspace_size(1, 0, 4) == 0


# A "pointer" value that is 16-byte aligned but never dereferenced: every call below
# fails validation before any device access.
P = 0x1000
MIS = 0x1008


def _decode(lib, fn="mla_decode_bf16", **kw):
    args = dict(q=P, kv=P, num_pages=10, bt=P, stride=4, lens=P, batch=2, heads=16, ps=64, scale=0.07,
                splits=1, out=P, lse=P, ws=None, ws_bytes=0, flags=0, cs=None)
    args.update(kw)
    rc = getattr(lib, fn)(args["q"], args["kv"], args["num_pages"], args["bt"], args["stride"], args["lens"],
                          args["batch"], args["heads"], args["ps"], args["scale"], args["splits"], args["out"],
                          args["lse"], args["ws"], args["ws_bytes"], args["flags"], args["cs"], None)
    return rc, lib.mla_last_error_message().decode()


DECODERS = ["mla_decode_bf16", "mla_decode_fp8_656", "mla_decode_nope_bf16", "mla_decode_nope_fp8_656",
            "mla_decode_rank256_bf16", "mla_decode_gla2_bf16", "mla_decode_gla2_fp8_656",
            "mla_decode_rank768_bf16", "mla_decode_rank1792_bf16"]


@pytest.mark.parametrize("fn", DECODERS)
@pytest.mark.parametrize("field", ["q", "kv", "bt", "lens", "out", "lse"])
def test_decode_rejects_null(lib, fn, field):
    rc, msg = _decode(lib, fn, **{field: None})
    assert rc == 1 and "NULL" in msg and fn in msg


@pytest.mark.parametrize("fn", DECODERS)
@pytest.mark.parametrize("kw, word", [
    (dict(heads=0), "num_heads"), (dict(heads=17), "num_heads"), (dict(batch=0), "batch"),
    (dict(batch=70000), "batch"), (dict(ps=0), "page_size"), (dict(num_pages=0), "num_pages"),
    (dict(stride=0), "block_table_stride"), (dict(splits=0), "num_splits"),
    (dict(splits=70000), "num_splits"), (dict(scale=float("nan")), "softmax_scale"),
    (dict(scale=float("inf")), "softmax_scale"), (dict(stride=1 << 40), "int32"),
])
def test_decode_rejects_bad_shapes(lib, fn, kw, word):
    rc, msg = _decode(lib, fn, **kw)
    assert rc == 2 and word in msg


BALANCED = ["mla_decode_balanced_bf16", "mla_decode_balanced_fp8_656", "mla_decode_balanced_nope_bf16",
            "mla_decode_balanced_nope_fp8_656", "mla_decode_gla2_balanced_bf16", "mla_decode_gla2_balanced_fp8_656"]


@pytest.mark.parametrize("fn", BALANCED)
@pytest.mark.parametrize("field", ["q", "kv", "bt", "lens", "out", "lse"])
def test_balanced_rejects_null(lib, fn, field):
    rc, msg = _decode(lib, fn, ws=P, ws_bytes=1 << 30, **{field: None})
    assert rc == 1 and "NULL" in msg and fn in msg


@pytest.mark.parametrize("fn", BALANCED)
@pytest.mark.parametrize("kw, word", [
    (dict(heads=0), "num_heads"), (dict(heads=17), "num_heads"), (dict(batch=0), "batch"),
    (dict(batch=1025), "batch"), (dict(ps=0), "page_size"), (dict(num_pages=0), "num_pages"),
    (dict(stride=0), "block_table_stride"), (dict(splits=-1), "num_workgroups"),
    (dict(splits=70000), "num_workgroups"), (dict(scale=float("nan")), "softmax_scale"),
    (dict(stride=1 << 40), "int32"),
])
def test_balanced_rejects_bad_shapes(lib, fn, kw, word):
    rc, msg = _decode(lib, fn, ws=P, ws_bytes=1 << 30, **kw)
    assert rc == 2 and word in msg


@pytest.mark.parametrize("fn", BALANCED)
def test_balanced_workspace(lib, fn):
    need = mla.mla_decode_balanced_workspace_size(2, 16, 512)
    # prefix sums [3] padded to 256 bytes, then 2 + 512 - 1 slots of 16 x 513 floats
    assert need == (256 + 513 * 16 * 513 * 4 + 255) // 256 * 256
    assert mla.mla_decode_balanced_workspace_size(0, 16, 4) == 0
    assert mla.mla_decode_balanced_workspace_size(2, 16, -1) == 0
    # 0 workgroups = one per compute unit of the current device: no device here, so 0 bytes
    assert mla.mla_decode_balanced_workspace_size(2, 16, 0) == 0
    rc, msg = _decode(lib, fn, splits=512)
    assert rc == 4 and "workspace" in msg
    rc, msg = _decode(lib, fn, splits=512, ws=P, ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg
    rc, msg = _decode(lib, fn, splits=512, ws=MIS, ws_bytes=need)
    assert rc == 3 and "aligned" in msg


def test_merge_balanced_validation(lib):
    need = mla.mla_decode_balanced_workspace_size(4, 16, 256)

    def call(ws=P, ws_bytes=need, batch=4, heads=16, wgs=256, out=P, lse=P):
        rc = lib.mla_merge_lse_balanced(ws, ws_bytes, batch, heads, wgs, out, lse, None)
        return rc, lib.mla_last_error_message().decode()

    for kw in (dict(ws=None), dict(out=None), dict(lse=None)):
        rc, msg = call(**kw)
        assert rc == 1 and "NULL" in msg
    for kw, word in ((dict(batch=0), "batch"), (dict(batch=1025), "batch"), (dict(heads=65), "num_heads"),
                     (dict(wgs=-1), "num_workgroups"), (dict(wgs=65536), "num_workgroups")):
        rc, msg = call(**kw)
        assert rc == 2 and word in msg
    rc, msg = call(out=MIS)
    assert rc == 3 and "aligned" in msg
    rc, msg = call(ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg


@pytest.mark.parametrize("field", ["q", "kv", "bt", "lens", "out", "lse"])
def test_decode_rejects_misaligned(lib, field):
    rc, msg = _decode(lib, **{field: MIS})
    assert rc == 3 and "aligned" in msg


def _mtp(lib, fn="mla_decode_mtp_bf16", **kw):
    args = dict(q=P, kv=P, num_pages=10, bt=P, stride=4, lens=P, batch=2, q_len=4, heads=16, ps=64, scale=0.07,
                splits=1, out=P, lse=P, ws=None, ws_bytes=0, flags=0, cs=None)
    args.update(kw)
    rc = getattr(lib, fn)(args["q"], args["kv"], args["num_pages"], args["bt"], args["stride"], args["lens"],
                          args["batch"], args["q_len"], args["heads"], args["ps"], args["scale"], args["splits"],
                          args["out"], args["lse"], args["ws"], args["ws_bytes"], args["flags"], args["cs"], None)
    return rc, lib.mla_last_error_message().decode()


@pytest.mark.parametrize("fn", ["mla_decode_mtp_bf16", "mla_decode_mtp_fp8_656"])
@pytest.mark.parametrize("kw, word", [
    (dict(q_len=0), "q_len"), (dict(q_len=17), "q_len"), (dict(q_len=5, heads=16), "q_len * num_heads"),
    (dict(q_len=16, heads=5), "q_len * num_heads"), (dict(heads=0), "num_heads"), (dict(splits=0), "num_splits"),
])
def test_mtp_rejects_bad_shapes(lib, fn, kw, word):
    rc, msg = _mtp(lib, fn, **kw)
    assert rc == 2 and word in msg and fn in msg


MTP_BALANCED = ["mla_decode_mtp_balanced_bf16", "mla_decode_mtp_balanced_fp8_656"]


@pytest.mark.parametrize("fn", MTP_BALANCED)
@pytest.mark.parametrize("kw, word", [
    (dict(q_len=0), "q_len"), (dict(q_len=17), "q_len"), (dict(q_len=5, heads=16), "q_len * num_heads"),
    (dict(heads=0), "num_heads"), (dict(heads=17, q_len=1), "num_heads"), (dict(batch=1025), "batch"),
    (dict(splits=-1), "num_workgroups"), (dict(splits=70000), "num_workgroups"),
    (dict(scale=float("nan")), "softmax_scale"),
])
def test_mtp_balanced_rejects_bad_shapes(lib, fn, kw, word):
    rc, msg = _mtp(lib, fn, ws=P, ws_bytes=1 << 30, **kw)
    assert rc == 2 and word in msg and fn in msg


@pytest.mark.parametrize("fn", MTP_BALANCED)
def test_mtp_balanced_workspace_counts_query_rows(lib, fn):
    need = mla.mla_decode_balanced_workspace_size(2, 4 * 16, 256)
    assert need > mla.mla_decode_balanced_workspace_size(2, 16, 256)
    rc, msg = _mtp(lib, fn, splits=256)
    assert rc == 4 and "workspace" in msg
    rc, msg = _mtp(lib, fn, splits=256, ws=P, ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg
    rc, msg = _mtp(lib, fn, splits=256, ws=P, ws_bytes=need, q=None)
    assert rc == 1 and "q is NULL" in msg and fn in msg
    rc, msg = _mtp(lib, fn, splits=256, ws=P, ws_bytes=need, out=MIS)
    assert rc == 3 and "aligned" in msg


APPEND = ["mla_decode_append_bf16", "mla_decode_append_fp8_656", "mla_decode_append_balanced_bf16",
          "mla_decode_append_balanced_fp8_656"]


def _append(lib, fn, **kw):
    args = dict(q=P, nl=P, npe=P, ns=P, kv=P, num_pages=10, bt=P, stride=4, lens=P, batch=2, q_len=1, heads=16,
                ps=64, scale=0.07, count=1, out=P, lse=P, ws=P, ws_bytes=1 << 30, flags=0, cs=None)
    args.update(kw)
    rc = getattr(lib, fn)(args["q"], args["nl"], args["npe"], args["ns"], args["kv"], args["num_pages"], args["bt"],
                          args["stride"], args["lens"], args["batch"], args["q_len"], args["heads"], args["ps"],
                          args["scale"], args["count"], args["out"], args["lse"], args["ws"], args["ws_bytes"],
                          args["flags"], args["cs"], None)
    return rc, lib.mla_last_error_message().decode()


@pytest.mark.parametrize("fn", APPEND)
@pytest.mark.parametrize("field", ["q", "nl", "ns", "kv", "bt", "lens", "out", "lse"])
def test_append_rejects_null(lib, fn, field):
    rc, msg = _append(lib, fn, **{field: None})
    assert rc == 1 and "NULL" in msg and fn in msg


@pytest.mark.parametrize("fn", APPEND)
@pytest.mark.parametrize("field", ["nl", "npe", "ns"])
def test_append_rejects_misaligned_rows(lib, fn, field):
    rc, msg = _append(lib, fn, **{field: MIS})
    assert rc == 3 and "aligned" in msg and fn in msg


@pytest.mark.parametrize("fn", APPEND)
@pytest.mark.parametrize("kw, word", [
    (dict(q_len=0), "q_len"), (dict(q_len=17), "q_len"), (dict(q_len=5, heads=16), "q_len * num_heads"),
    (dict(heads=0), "num_heads"), (dict(batch=0), "batch"), (dict(ps=0), "page_size"),
    (dict(scale=float("nan")), "softmax_scale"),
])
def test_append_rejects_bad_shapes(lib, fn, kw, word):
    rc, msg = _append(lib, fn, **kw)
    assert rc == 2 and word in msg and fn in msg


def test_append_takes_no_k_pe_and_the_schedules_counts(lib):
    # a NULL new_k_pe is valid (rope part written as zeros): only the missing device stops it
    for fn in APPEND:
        assert _append(lib, fn, npe=None)[0] == 5
    rc, msg = _append(lib, "mla_decode_append_bf16", count=0)
    assert rc == 2 and "num_splits" in msg
    rc, msg = _append(lib, "mla_decode_append_balanced_fp8_656", count=-1)
    assert rc == 2 and "num_workgroups" in msg
    rc, msg = _append(lib, "mla_decode_append_fp8_656", count=4, ws=None)
    assert rc == 4 and "workspace" in msg


def test_merge_balanced_takes_verify_rows(lib):
    need = mla.mla_decode_balanced_workspace_size(4, 64, 256)
    # 64 query rows per request (q_len 4 x 16 heads): valid, only the missing device stops it
    assert lib.mla_merge_lse_balanced(P, need, 4, 64, 256, P, P, None) == 5
    assert lib.mla_merge_lse_balanced(P, need, 4, 65, 256, P, P, None) == 2


@pytest.mark.parametrize("fn", ["mla_decode_gla2_bf16", "mla_decode_gla2_fp8_656", "mla_decode_gla2_balanced_bf16",
                                "mla_decode_gla2_balanced_fp8_656"])
def test_gla2_needs_an_even_head_count(lib, fn):
    rc, msg = _decode(lib, fn, heads=3, ws=P, ws_bytes=1 << 30)
    assert rc == 2 and "even" in msg


@pytest.mark.parametrize("fn", ["mla_decode_gla2_balanced_bf16", "mla_decode_gla2_balanced_fp8_656"])
def test_gla2_balanced_has_no_partials_only_form(lib, fn):
    rc, msg = _decode(lib, fn, out=None, lse=None, ws=P, ws_bytes=1 << 30)
    assert rc == 1 and "out is NULL" in msg


def test_merge_width_validation(lib):
    f = lib.mla_merge_lse_width
    assert f(P, P, 2, 1, 4, 384, P, P, None) == 2 and "width" in lib.mla_last_error_message().decode()
    assert f(None, P, 2, 1, 4, 256, P, P, None) == 1
    assert f(P, P, 2, 1, 0, 256, P, P, None) == 2
    assert f(MIS, P, 2, 1, 4, 256, P, P, None) == 3


def test_merge_width_accepts_wide_ranks(lib):
    f = lib.mla_merge_lse_width
    for width in (256, 512, 768, 1792):  # valid arguments: only the missing device stops the call
        rc = f(P, P, 2, 1, 4, width, P, P, None)
        assert rc == 5 and "width" not in lib.mla_last_error_message().decode()


@pytest.mark.parametrize("rank, fn", [(768, "mla_decode_rank768_bf16"), (1792, "mla_decode_rank1792_bf16")])
def test_wide_rank_workspace(lib, rank, fn):
    need = mla.mla_decode_rank_workspace_size(2, 16, 4, rank)
    assert need == (4 * 2 * 16 * (rank + 1) * 4 + 64 + 255) // 256 * 256
    assert mla.mla_decode_rank_workspace_size(2, 16, 1, rank) == 0
    assert mla.mla_decode_rank_workspace_size(2, 16, 4, 512) == 0
    assert mla.mla_decode_rank_workspace_size(0, 16, 4, rank) == 0
    rc, msg = _decode(lib, fn, splits=4, ws=P, ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg
    rc, msg = _decode(lib, fn, splits=4, ws=P, ws_bytes=mla.mla_decode_workspace_size(2, 16, 4))
    assert rc == 4  # the 512-wide size is too small for rank-wide partials


def test_mtp_workspace_counts_query_rows(lib):
    need = mla.mla_decode_workspace_size(2, 4 * 16, 8)
    rc, msg = _mtp(lib, splits=8, ws=P, ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg
    rc, msg = _mtp(lib, q=None)
    assert rc == 1 and "q is NULL" in msg


def test_decode_split_needs_workspace(lib):
    rc, msg = _decode(lib, splits=4)
    assert rc == 4 and "workspace" in msg
    need = mla.mla_decode_workspace_size(2, 16, 4)
    rc, msg = _decode(lib, splits=4, ws=P, ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg
    rc, msg = _decode(lib, splits=4, ws=MIS, ws_bytes=need)
    assert rc == 3


def test_merge_validation(lib):
    f = lib.mla_merge_lse
    assert f(None, P, 2, 1, 1, P, P, None) == 1
    assert f(P, P, 0, 1, 1, P, P, None) == 2
    assert f(P, P, 2, 0, 1, P, P, None) == 2
    assert f(P, P, 2, 1, 0, P, P, None) == 2
    assert f(MIS, P, 2, 1, 1, P, P, None) == 3
    assert "part_out" in lib.mla_last_error_message().decode()


def test_cache_write_validation(lib):
    f = lib.mla_cache_write
    assert f(P, P, P, -1, P, 0, 10, None) == 2
    assert f(P, P, P, 1, P, 7, 10, None) == 2
    assert f(P, P, P, 1, P, 0, 0, None) == 2
    assert f(None, P, P, 1, P, 0, 10, None) == 1
    assert f(P, P, None, 1, P, 0, 10, None) == 1
    assert f(P, P, P, 1, None, 1, 10, None) == 1
    assert f(MIS, None, P, 1, P, 1, 10, None) == 3  # k_pe NULL is allowed (zero rope)
    assert f(P, MIS, P, 1, P, 1, 10, None) == 3
    assert f(None, None, None, 0, None, 0, 10, None) == 0  # nothing to write: no device needed


def test_gather_validation(lib):
    f = lib.mla_gather_context
    #        kv fmt pages ps  bt stride cu  starts batch total out
    ok = dict(kv=P, fmt=0, pages=10, ps=16, bt=P, stride=4, cu=P, st=None, batch=2, total=100, out=P)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["kv"], a["fmt"], a["pages"], a["ps"], a["bt"], a["stride"], a["cu"], a["st"], a["batch"],
                 a["total"], a["out"], a.get("cs"), None), lib.mla_last_error_message().decode()
    for kw, rc, word in [(dict(fmt=5), 2, "cache_format"), (dict(total=-1), 2, "total_rows"),
                         (dict(total=1 << 40), 2, "total_rows"), (dict(total=(1 << 32) + 1), 2, "total_rows"), (dict(batch=0), 2, "batch"),
                         (dict(pages=0), 2, "num_pages"), (dict(ps=0), 2, "page_size"), (dict(stride=0), 2, "stride"),
                         (dict(kv=None), 1, "kv_cache"), (dict(cu=None), 1, "cu_rows"), (dict(out=None), 1, "out"),
                         (dict(bt=None), 1, "block_table"), (dict(st=MIS), 3, "aligned"), (dict(cu=MIS), 3, "aligned")]:
        got, msg = call(**kw)
        assert got == rc and word in msg and "mla_gather_context" in msg, (kw, got, msg)
    assert call(total=0, kv=None, out=None)[0] == 0  # nothing to gather: no device needed


ALL_DECODERS = DECODERS + ["mla_decode_balanced_bf16", "mla_decode_balanced_fp8_656", "mla_decode_balanced_nope_bf16",
                           "mla_decode_balanced_nope_fp8_656"]


@pytest.mark.parametrize("fn", ALL_DECODERS)
def test_decode_options_are_per_call(lib, fn):
    ws = dict(ws=P, ws_bytes=1 << 30)
    rc, msg = _decode(lib, fn, flags=2, **ws)
    assert rc == 2 and "flag" in msg and fn in msg
    rc, msg = _decode(lib, fn, flags=0x80000000, **ws)
    assert rc == 2 and "flag" in msg
    # the release build checks nothing, so it refuses a status word rather than ignore it
    rc, msg = _decode(lib, fn, cs=P, **ws)
    assert rc == 2 and "checked build" in msg
    # valid options: only the missing device stops the call
    assert _decode(lib, fn, flags=mla.MLA_FLAG_CACHED_ROWS, **ws)[0] == 5
    assert _decode(lib, fn, flags=0, **ws)[0] == 5


@pytest.mark.parametrize("fn", ["mla_decode_mtp_bf16", "mla_decode_mtp_balanced_fp8_656"])
def test_mtp_options_are_per_call(lib, fn):
    rc, msg = _mtp(lib, fn, flags=4, ws=P, ws_bytes=1 << 30)
    assert rc == 2 and "flag" in msg
    assert _mtp(lib, fn, flags=1, ws=P, ws_bytes=1 << 30)[0] == 5


@pytest.fixture(scope="module")
def checked_lib():
    if not os.path.exists(mla.CHECKED_LIB_PATH):
        pytest.fail("libmla_checked.so is not built (run __graft_entry__.build())")
    return mla.library(checked=True)


def test_checked_build_identifies_itself(lib, checked_lib):
    assert lib.mla_checked_build() == 0 and checked_lib.mla_checked_build() == 1
    assert checked_lib.mla_abi_version() == lib.mla_abi_version()


def test_checked_build_exports_the_same_abi(checked_lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mla.CHECKED_LIB_PATH], capture_output=True, text=True).stdout
    assert sorted(l.split()[-1] for l in out.splitlines() if " T " in l) == sorted(mla.EXPORTED)


@pytest.mark.parametrize("fn", ["mla_decode_bf16", "mla_decode_balanced_fp8_656", "mla_decode_rank768_bf16"])
def test_checked_build_takes_a_status_word(checked_lib, fn):
    ws = dict(ws=P, ws_bytes=1 << 30)
    assert _decode(checked_lib, fn, cs=P, **ws)[0] == 5  # accepted; no device here
    rc, msg = _decode(checked_lib, fn, cs=P + 2, **ws)
    assert rc == 3 and "check_status" in msg
    rc, msg = _decode(checked_lib, fn, flags=8, cs=P, **ws)
    assert rc == 2 and "flag" in msg


def test_gather_status_word(lib, checked_lib):
    a = (P, 0, 10, 16, P, 4, P, None, 2, 100, P)
    assert lib.mla_gather_context(*a, P, None) == 2 and "checked build" in lib.mla_last_error_message().decode()
    assert checked_lib.mla_gather_context(*a, P, None) == 5


def test_host_precondition_check():
    """The predicates the checked kernels apply, on host arrays: block ids a context uses in
    [0, num_pages), lengths in [0, stride * page_size]; entries past a context are not read."""
    import numpy as np
    f = mla.mla_check_preconditions_host
    bt = np.array([[3, 1, -1, -1], [0, 2, 4, 5]], np.int32)
    assert f(bt, [20, 64], page_size=16, num_pages=6) == 0          # -1 tails past the context
    assert f(bt, [33, 64], page_size=16, num_pages=6) == mla.MLA_CHECK_BLOCK_ID  # token 32 uses -1
    assert f(bt, [0, 64], page_size=16, num_pages=5) == mla.MLA_CHECK_BLOCK_ID   # page 5 of 5
    assert f(bt, [0, 48], page_size=16, num_pages=5) == 0            # ... not used at 48 tokens
    assert f(bt, [0, 65], page_size=16, num_pages=6) == mla.MLA_CHECK_SEQ_LEN    # past the table
    assert f(bt, [-1, 0], page_size=16, num_pages=6) == mla.MLA_CHECK_SEQ_LEN
    assert f(bt, [40, 65], page_size=16, num_pages=6) == mla.MLA_CHECK_SEQ_LEN | mla.MLA_CHECK_BLOCK_ID
    wrap = np.array([[58254, 70312]], np.int32)                      # high pages of a 70,313-page pool
    assert f(wrap, [128], page_size=64, num_pages=70313) == 0
    assert f(wrap, [128], page_size=64, num_pages=70312) == mla.MLA_CHECK_BLOCK_ID
    with pytest.raises(mla.MlaError):
        f(bt, [1, 1], page_size=0, num_pages=6)


def _noalloc(lib, **kw):
    a = dict(q=P, kv=P, num_pages=10, bt=P, stride=4, lens=P, batch=4, heads=16, ps=64, scale=0.07, splits=64,
             out=P, lse=P, flags=0, cs=None)
    a.update(kw)
    rc = lib.mla_decode_bf16_noalloc(a["q"], a["kv"], a["num_pages"], a["bt"], a["stride"], a["lens"], a["batch"],
                                     a["heads"], a["ps"], a["scale"], a["splits"], a["out"], a["lse"], a["flags"],
                                     a["cs"], None)
    return rc, lib.mla_last_error_message().decode()


def test_noalloc_validation(lib):
    assert mla.NOALLOC_SCRATCH_BYTES == 16 << 20
    # the long-context shape (4 requests x 16 heads x 64 splits) fits the scratch: only the device is missing
    assert mla.mla_decode_workspace_size(4, 16, 64) <= mla.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib)[0] == 5
    rc, msg = _noalloc(lib, splits=200)  # 200 x 4 x 16 partials: 26 MB
    assert rc == 4 and "scratch" in msg and "mla_decode_bf16_noalloc" in msg
    for kw in (dict(out=None), dict(lse=None)):
        rc, msg = _noalloc(lib, **kw)
        assert rc == 1 and "mla_decode_bf16_noalloc" in msg
    rc, msg = _noalloc(lib, heads=17)
    assert rc == 2 and "num_heads" in msg and "mla_decode_bf16_noalloc" in msg
    rc, msg = _noalloc(lib, flags=2)
    assert rc == 2 and "flag" in msg


SPARSE = ["mla_decode_sparse_bf16", "mla_decode_sparse_fp8_656", "mla_decode_sparse_nope_bf16",
          "mla_decode_sparse_nope_fp8_656"]


def _sparse(lib, fn, **kw):
    a = dict(q=P, kv=P, num_slots=100, idx=P, topk=64, tokens=3, heads=16, scale=0.07, splits=1, out=P, lse=P,
             ws=None, ws_bytes=0, flags=0, cs=None)
    a.update(kw)
    rc = getattr(lib, fn)(a["q"], a["kv"], a["num_slots"], a["idx"], a["topk"], a["tokens"], a["heads"], a["scale"],
                          a["splits"], a["out"], a["lse"], a["ws"], a["ws_bytes"], a["flags"], a["cs"], None)
    return rc, lib.mla_last_error_message().decode()


@pytest.mark.parametrize("fn", SPARSE)
def test_sparse_validation(lib, fn):
    for field in ("q", "kv", "idx", "out", "lse"):
        rc, msg = _sparse(lib, fn, **{field: None})
        assert rc == 1 and "NULL" in msg and fn in msg, field
    for kw, word in [(dict(tokens=0), "num_tokens"), (dict(tokens=(1 << 20) + 1), "num_tokens"),
                     (dict(heads=0), "num_heads"), (dict(heads=17), "num_heads"), (dict(topk=0), "topk"), (dict(topk=(1 << 24) + 1), "topk"),
                     (dict(num_slots=0), "num_slots"), (dict(splits=0), "num_splits"),
                     (dict(splits=70000), "num_splits"), (dict(scale=float("nan")), "softmax_scale"),
                     (dict(flags=4), "flag")]:
        rc, msg = _sparse(lib, fn, **kw)
        assert rc == 2 and word in msg and fn in msg, kw
    for field in ("q", "kv", "idx", "out", "lse"):
        rc, msg = _sparse(lib, fn, **{field: MIS})
        assert rc == 3 and "aligned" in msg, field
    need = mla.mla_decode_workspace_size(3, 16, 4)
    rc, msg = _sparse(lib, fn, splits=4)
    assert rc == 4 and "workspace" in msg
    rc, msg = _sparse(lib, fn, splits=4, ws=P, ws_bytes=need - 1)
    assert rc == 4 and str(need) in msg
    # valid arguments: only the device is missing here
    assert _sparse(lib, fn, splits=4, ws=P, ws_bytes=need)[0] == 5
    assert _sparse(lib, fn)[0] == 5
    rc, msg = _sparse(lib, fn, cs=P)
    assert rc == 2 and "checked build" in msg
    # out == lse == NULL: the partials stay in the workspace (num_splits > 1 only)
    assert _sparse(lib, fn, out=None, lse=None, splits=4, ws=P, ws_bytes=need)[0] == 5
    assert _sparse(lib, fn, out=None, lse=None)[0] == 1


@pytest.mark.parametrize("fn", SPARSE)
def test_sparse_checked_build_takes_a_status_word(checked_lib, fn):
    assert _sparse(checked_lib, fn, cs=P)[0] == 5  # accepted; only the device is missing
    rc, msg = _sparse(checked_lib, fn, cs=P + 2)
    assert rc == 3 and "check_status" in msg


def test_error_message_is_thread_local(lib):
    import threading
    _decode(lib, heads=99)
    main = lib.mla_last_error_message().decode()
    seen = []

    def other():
        seen.append(lib.mla_last_error_message().decode())
        _decode(lib, ps=0)

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [""]
    assert lib.mla_last_error_message().decode() == main and "num_heads" in main


def test_binding_marshalling_errors_without_device():
    import torch
    q = torch.zeros(1, 4, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        mla.mla_decode_bf16(q, q, torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, dtype=torch.int32), 0.1)
    with pytest.raises(TypeError, match="bfloat16"):
        mla.mla_decode_bf16(q.float(), q, None, None, 0.1)


def test_bench_helper_library_exports_its_header():
    """libmla_bench.so (bench.py's streaming-read reference) exports exactly what
    include/mla_bench.h declares, and validates its arguments before any launch."""
    import subprocess
    from paged_mla_latent_amd.build import BENCH_LIB_PATH
    if not os.path.exists(BENCH_LIB_PATH):
        pytest.fail("libmla_bench.so is not built (run __graft_entry__.build())")
    text = open(os.path.join(ROOT, "include", "mla_bench.h")).read()
    declared = re.findall(r"MLA_BENCH_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", text)
    out = subprocess.run(["nm", "-D", "--defined-only", BENCH_LIB_PATH], capture_output=True, text=True).stdout
    assert sorted(l.split()[-1] for l in out.splitlines() if " T " in l) == sorted(declared) == ["mla_bench_stream_read"]
    lib = ctypes.CDLL(BENCH_LIB_PATH)
    fn = lib.mla_bench_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert fn(None, 1024, P, 8, 0, None) == 1
    assert fn(P, 1024, None, 8, 0, None) == 1
    for nbytes, wgs in ((0, 8), (8, 8), (1000, 8), (1024, 0), (1024, 65536)):
        assert fn(P, nbytes, P, wgs, 0, None) == 2
    assert fn(P + 8, 1024, P, 8, 0, None) == 3 and fn(P, 1024, P + 2, 8, 1, None) == 3

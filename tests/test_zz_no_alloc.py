"""mla_decode_bf16_noalloc, the decode for callers that cannot allocate, on an MI355X.

Called through the C ABI (ctypes, raw pointers) and checked against mla_decode_bf16 on the same
inputs (same kernels: the results must agree bit for bit) and against the fp64 oracle, on two
calls in a row, the second with a smaller input (the scratch keeps the first call's contents).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_mla_latent_amd as mla
import workloads
from gpu_util import assert_parity, bf16_dev, device_pool, host_pool, say

pytestmark = pytest.mark.gpu


def _raw_noalloc(w, pool, splits):
    lib = mla.library()
    q = bf16_dev(w.q)
    bt = torch.from_numpy(w.block_table).cuda()
    lens = torch.from_numpy(w.seq_lens).cuda()
    out = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, w.heads), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.mla_decode_bf16_noalloc(q.data_ptr(), pool.data_ptr(), pool.shape[0], bt.data_ptr(), bt.shape[1],
                                     lens.data_ptr(), w.batch, w.heads, w.page_size, ctypes.c_float(w.scale), splits,
                                     out.data_ptr(), lse.data_ptr(), 0, None, ctypes.c_void_p(stream))
    assert rc == 0, lib.mla_last_error_message().decode()
    ref = mla.mla_decode_bf16(q, pool, bt, lens, w.scale, num_splits=splits)
    torch.cuda.synchronize()
    return (out, lse), ref


def test_noalloc_matches_the_workspace_decode_on_two_calls():
    assert torch.cuda.is_available()
    big = workloads.make_workload("noalloc_big", seq_lens=[20000, 0, 7777, 12345], heads=16, page_size=64,
                                  num_pages=700, seed=31)
    small = workloads.make_workload("noalloc_small", seq_lens=[300, 5], heads=4, page_size=16, num_pages=30, seed=32)
    for w, splits in ((big, 64), (small, 3)):
        say(f"noalloc: {w.name} B={w.batch} H={w.heads} splits={splits}")
        pd, ph = device_pool(w), host_pool(w)
        (out, lse), (ro_dev, rl_dev) = _raw_noalloc(w, pd, splits)
        assert torch.equal(out, ro_dev) and torch.equal(lse, rl_dev)
        ref_o, ref_l = oracle.decode(w.q, ph, w.block_table, w.seq_lens, w.page_size, w.scale, "bf16")
        assert_parity(w, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
                      what=f"noalloc {w.name}")
    # one split: no scratch at all; and a split count whose partials exceed the scratch is refused
    (out, lse), (ro_dev, rl_dev) = _raw_noalloc(small, device_pool(small), 1)
    assert torch.equal(out, ro_dev) and torch.equal(lse, rl_dev)
    with pytest.raises(mla.MlaError, match="scratch"):
        w = big
        mla.mla_decode_bf16_noalloc(bf16_dev(w.q), device_pool(w), torch.from_numpy(w.block_table).cuda(),
                                    torch.from_numpy(w.seq_lens).cuda(), w.scale, num_splits=2000)

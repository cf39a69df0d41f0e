"""bench.py's streaming-read reference (libmla_bench.so, include/mla_bench.h) on an MI355X: it
reads every 16-byte word of its buffer exactly once, so the XOR of its sink equals the XOR of
the buffer's words, for sizes that are and are not multiples of the grid's stride."""
import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_util import say
from paged_mla_latent_amd.build import BENCH_LIB_PATH

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("words,wgs", [(1, 1), (4096 * 8 + 3, 16), (1 << 20, 2048), (777_777, 300)])
def test_stream_read_reads_every_word_once(words, wgs, nt):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert os.path.exists(BENCH_LIB_PATH), "libmla_bench.so is not built"
    lib = ctypes.CDLL(BENCH_LIB_PATH)
    fn = lib.mla_bench_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    say(f"stream read: {words} words, {wgs} workgroups, nontemporal={nt}")
    rng = np.random.default_rng(words)
    host = rng.integers(0, 1 << 32, size=(words, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(4 * wgs, dtype=torch.int32, device="cuda")
    rc = fn(ctypes.c_void_p(buf.data_ptr()), words * 16, ctypes.c_void_p(sink.data_ptr()), wgs, nt,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.reshape(-1))
    assert got == want

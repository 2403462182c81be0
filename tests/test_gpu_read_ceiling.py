"""GPU: the benchmark's streaming-read kernels (libhbmread.so) read every word exactly once.

Each variant folds the words it reads into one XOR word per thread; the XOR of all those
words must equal the XOR of the buffer, for sizes that leave a ragged tail in both access
orders, so that a skipped or repeated tile would show.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hbm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    path = os.path.join(ROOT, "head_wise_sparse_rtp_amd", "libhbmread.so")
    assert os.path.exists(path), "libhbmread.so is not built"
    lib = ctypes.CDLL(path)
    lib.hbm_read.restype = ctypes.c_int
    lib.hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                             ctypes.c_int, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("n16,blocks", [(1, 3), (1000, 7), ((1 << 20) + 37, 64),
                                        ((1 << 20) + 37, 1000)])
def test_every_variant_reads_each_word_once(hbm, n16, blocks):
    print("[case] hbm_read n16", n16, "blocks", blocks, flush=True)
    rng = np.random.default_rng(n16 + blocks)
    words = rng.integers(0, 1 << 32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    want = int(np.bitwise_xor.reduce(words))
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    for var in range(8):
        sink.fill_(0x5A5A5A5A)
        rc = hbm.hbm_read(ctypes.c_void_p(buf.data_ptr()), 16 * n16,
                          ctypes.c_void_p(sink.data_ptr()), blocks, var,
                          ctypes.c_void_p(st.cuda_stream))
        assert rc == 0, (var, rc)
        got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
        assert got == want, (var, hex(got), hex(want))


def test_unknown_variant_is_refused(hbm):
    sink = torch.empty(256, dtype=torch.int32, device="cuda:0")
    buf = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    rc = hbm.hbm_read(ctypes.c_void_p(buf.data_ptr()), 16, ctypes.c_void_p(sink.data_ptr()), 1,
                      8, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 1

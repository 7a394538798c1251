"""The benchmark's streaming-ceiling probes read every byte exactly once: the XOR of the words they
fold equals the XOR of every 32-bit word of the buffer (contiguous sweep with a ragged tail, and
4 KB pages in a random order with an odd page count)."""

import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    path = os.path.join(ROOT, "long_context_online_amd", "libblasst_ceiling.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m long_context_online_amd.build`")
    L = ctypes.CDLL(path)
    L.blasst_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p]
    L.blasst_ceiling_stream_pages.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_void_p]
    return L


def _xor_all(words):
    return int(np.bitwise_xor.reduce(words.astype(np.uint32)))


@pytest.mark.parametrize("nbytes,grid", [(16 * 1024 * 1024 + 48, 64), (4096 * 7 + 16, 3), (1024 * 1024, 4096)])
def test_contiguous_reads_every_word_once(lib, nbytes, grid):
    import torch
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    x = torch.from_numpy(host.view(np.int32)).to("cuda")
    out = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.blasst_ceiling_stream_read(x.data_ptr(), nbytes, out.data_ptr(), grid, stream) == 0
    torch.cuda.synchronize()
    assert _xor_all(out.cpu().numpy().view(np.uint32)) == _xor_all(host)


@pytest.mark.parametrize("n_pages,grid", [(1023, 16), (4096, 1), (257, 4096)])
def test_pages_reads_every_page_once(lib, n_pages, grid):
    import torch
    rng = np.random.default_rng(n_pages)
    host = rng.integers(0, 2 ** 32, size=n_pages * 1024, dtype=np.uint64).astype(np.uint32)
    pool = torch.from_numpy(host.view(np.int32)).to("cuda")
    table = torch.from_numpy(rng.permutation(n_pages).astype(np.int32)).to("cuda")
    out = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.blasst_ceiling_stream_pages(pool.data_ptr(), table.data_ptr(), n_pages, out.data_ptr(), grid,
                                           stream) == 0
    torch.cuda.synchronize()
    assert _xor_all(out.cpu().numpy().view(np.uint32)) == _xor_all(host)

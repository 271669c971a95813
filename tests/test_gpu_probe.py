"""The measurement probes of libla_probe.so (include/la_probe.h) compute what
their header says, on the GPU: the read probe's per-thread fold of the
vectors it reads, and the matrix-core probe's sums growing with its rounds.
These probes only measure; the checks make sure the bytes and instructions
they are credited with were really read and issued."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

from tests.gpu_helpers import log, torch_cuda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "chunked_causal_linear_amd", "libla_probe.so"))
    lib.la_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.la_probe_read.restype = ctypes.c_int
    lib.la_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.la_probe_mfma.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("n16,grid", [(5000, 4), (256 * 4, 4), (3, 2)])
def test_read_probe_folds_every_vector(n16, grid):
    torch = torch_cuda()
    lib = _lib()
    log(f"la_probe_read n16={n16} grid={grid}")
    words = np.random.default_rng([7, n16, grid]).integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64)
    words = words.astype(np.uint32)
    x = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.full((grid * 256,), -1.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # one pass: thread t folds (XOR) the four words of vectors t, t + 256 grid, ...
    assert lib.la_probe_read(x.data_ptr(), n16, 1, grid, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    per_vec = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    want = np.zeros(grid * 256, dtype=np.uint32)
    for t in range(grid * 256):
        if t < n16:
            want[t] = np.bitwise_xor.reduce(per_vec[t::grid * 256])
    assert np.array_equal(out.cpu().numpy(), want.astype(np.float32))
    # two passes fold every vector twice: all zero
    assert lib.la_probe_read(x.data_ptr(), n16, 2, grid, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.zeros(grid * 256, dtype=np.float32))


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_probe_sums_grow_with_rounds(kind):
    """Every round adds the same products to each accumulator, so the sums
    after 2 and after 4 rounds differ by a factor of two (exactly for the int8
    kind; to fp32 rounding for bf16)."""
    torch = torch_cuda()
    lib = _lib()
    log(f"la_probe_mfma kind={kind}")
    grid = 4
    out2 = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    out4 = torch.empty_like(out2)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.la_probe_mfma(kind, 2, grid, out2.data_ptr(), stream) == 0
    assert lib.la_probe_mfma(kind, 4, grid, out4.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    a, b = out2.cpu().numpy().astype(np.float64), out4.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(a)) and np.all(a != 0)
    if kind == 1:
        assert np.array_equal(b, 2 * a)
    else:
        assert np.allclose(b, 2 * a, rtol=1e-5, atol=0)

"""libzscopy: the plain device copy bench.py times as the HBM ceiling.

Measurement only (no step of the method), but the benchmark's ceiling is
only meaningful if the copy is exact and refuses what it cannot copy.
"""
import ctypes as C

import numpy as np
import pytest


@pytest.fixture(scope="module")
def copylib(hip_built):
    # torch first, so that the library shares torch's HIP runtime instead of
    # bringing in a second one through its search path
    import torch  # noqa: F401
    lib = C.CDLL(hip_built.COPY)
    lib.zs_copy_ceiling.restype = C.c_int
    lib.zs_copy_ceiling.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p]
    lib.zs_copy_last_error.restype = C.c_char_p
    return lib


def test_refuses_before_any_launch(copylib):
    """Null, misaligned, ragged, overlapping or oversized requests return 1
    without touching a device (these calls make no HIP call); zero bytes is
    a no-op."""
    f = copylib.zs_copy_ceiling
    assert f(None, 0x1000, 16, None) == 1
    assert f(0x1000, None, 16, None) == 1
    assert f(0x1008, 0x2000, 16, None) == 1
    assert f(0x1000, 0x2008, 16, None) == 1
    assert f(0x1000, 0x2000, 24, None) == 1
    assert f(0x1000, 0x1010, 64, None) == 1
    huge = 16 * 256 * (1 << 31)  # one block past the largest grid
    assert f(0x1000, 0x1000 + huge, huge, None) == 1
    assert f(0x1000, 0x2000, 0, None) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 16 * 255, 16 * 257, 4096 * 1024 + 48])
def test_copy_is_exact(copylib, nbytes):
    """Every byte arrives, ragged grids included, and nothing past the end
    is written."""
    import torch
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    dst = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
    rc = copylib.zs_copy_ceiling(src.data_ptr(), dst.data_ptr(), nbytes,
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 0, copylib.zs_copy_last_error().decode()
    torch.cuda.synchronize()
    out = dst.cpu().numpy()
    assert np.array_equal(out[:nbytes], src.cpu().numpy())
    assert not out[nbytes:].any()

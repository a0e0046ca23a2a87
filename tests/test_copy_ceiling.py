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
    lib.zs_copy_shape.restype = C.c_int
    lib.zs_copy_shape.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_uint64, C.c_uint32,
                                  C.c_void_p]
    lib.zs_copy_shape_name.restype = C.c_char_p
    lib.zs_copy_shape_tile_bytes.restype = C.c_uint64
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


def _probe_fn(copylib):
    f = copylib.zs_stream_probe
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_uint32, C.c_void_p, C.c_uint32, C.c_void_p, C.c_uint32,
                  C.c_void_p, C.c_uint64, C.c_uint32, C.c_uint32, C.c_void_p, C.c_uint32,
                  C.c_void_p]
    return f


def _ptrs(addrs):
    return (C.c_void_p * max(1, len(addrs)))(*addrs)


def test_probe_refuses_before_any_launch(copylib):
    """Stream counts, vector widths, caps, alignment, ragged sizes and
    overlapping outputs are refused with 1 before any HIP call."""
    f = _probe_fn(copylib)
    A = 0x7F0000000000
    n = 4096
    g = _ptrs([A + k * 0x100000 for k in range(3)])
    i3 = _ptrs([A + 0x1000000 + k * 0x100000 for k in range(3)])
    o3 = _ptrs([A + 0x2000000 + k * 0x100000 for k in range(3)])
    sink = A + 0x3000000
    ok = dict(in16=g, n_in16=3, in32=i3, n_in32=3, out32=o3, n_out32=3, out16=A + 0x4000000,
              n=n, vecs=2, cap=0, sink=sink, magic=1)

    def call(**over):
        a = dict(ok, **over)
        return f(a["in16"], a["n_in16"], a["in32"], a["n_in32"], a["out32"], a["n_out32"],
                 a["out16"], a["n"], a["vecs"], a["cap"], a["sink"], a["magic"], None)

    assert call(n_in16=65) == 1
    assert call(n_in32=2) == 1
    assert call(n_out32=2) == 1
    assert call(vecs=3) == 1
    assert call(cap=9) == 1
    assert call(sink=None) == 1
    assert call(sink=sink + 2) == 1
    assert call(n=n + 2048) == 1                 # not a multiple of the 4096-element tile
    assert call(out16=A + 0x4000008) == 1        # misaligned output
    assert call(out16=A + 0x1000000 + 64) == 1   # output on an fp32 input
    assert call(out16=o3[1] + 16) == 1           # output on another output
    assert call(out16=sink - 16) == 1            # output on the sink
    assert call(in16=_ptrs([A, 0, A + 0x200000]), n_in16=3) == 1
    assert call(n=0) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("w,nin,nout,p16,vecs", [(3, 3, 3, True, 2), (1, 3, 3, True, 1),
                                                  (9, 0, 1, False, 2), (64, 0, 0, True, 2),
                                                  (0, 1, 1, False, 1), (0, 0, 3, True, 1),
                                                  (17, 3, 1, True, 2)])
def test_probe_moves_what_it_states(copylib, w, nin, nout, p16, vecs):
    """Each output word is the documented fold of the inputs, so every
    stream the probe states is really read and written."""
    import torch
    f = _probe_fn(copylib)
    tile = 2048 * vecs
    n = 3 * tile
    rng = np.random.default_rng(w * 100 + nin * 10 + nout)
    g = [torch.from_numpy(rng.integers(0, 2 ** 16, n, dtype=np.uint16).view(np.int16)).cuda()
         for _ in range(w)]
    i32 = [torch.from_numpy(rng.integers(0, 2 ** 32, n, dtype=np.uint32).view(np.int32)).cuda()
           for _ in range(nin)]
    o32 = [torch.zeros(n, dtype=torch.int32, device="cuda") for _ in range(nout)]
    o16 = torch.zeros(n, dtype=torch.int16, device="cuda") if p16 else None
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    rc = f(_ptrs([t.data_ptr() for t in g]), w, _ptrs([t.data_ptr() for t in i32]), nin,
           _ptrs([t.data_ptr() for t in o32]), nout, o16.data_ptr() if p16 else None, n, vecs,
           0, sink.data_ptr(), 0x12345678, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, copylib.zs_copy_last_error().decode()
    torch.cuda.synchronize()
    words = [t.cpu().numpy().view(np.uint32).reshape(-1, 4) for t in g]   # one row per vector
    fold = np.zeros((n // 8, 4), np.uint32)
    for x in words:
        fold += x
    ins = [t.cpu().numpy().view(np.uint32).reshape(-1, 2, 4) for t in i32]
    for k in range(nout):
        got = o32[k].cpu().numpy().view(np.uint32).reshape(-1, 2, 4)
        want = (ins[k] ^ fold[:, None, :]) if k < nin else np.repeat(fold[:, None, :], 2, 1)
        assert np.array_equal(got, want), f"fp32 output {k}"
    if p16:
        rest = fold.copy()
        for k in range(nout, nin):
            rest ^= ins[k][:, 0, :] ^ ins[k][:, 1, :]
        assert np.array_equal(o16.cpu().numpy().view(np.uint32).reshape(-1, 4), rest)


def test_copy_shapes_catalogue_and_refusals(copylib):
    """The copy-shape catalogue names every shape and its tile; requests it
    cannot run return 1 before any HIP call."""
    count = copylib.zs_copy_shape_count()
    assert count >= 10
    names = [copylib.zs_copy_shape_name(i) for i in range(count)]
    assert all(names) and len(set(names)) == count
    assert copylib.zs_copy_shape_name(count) is None and copylib.zs_copy_shape_name(-1) is None
    tiles = [copylib.zs_copy_shape_tile_bytes(i) for i in range(count)]
    assert tiles[0] == 4096 and all(t > 0 and (1 << 32) % t == 0 for t in tiles)
    f = copylib.zs_copy_shape
    assert f(count, 0x1000, 0x100000, 4096, 0, None) == 1
    assert f(-1, 0x1000, 0x100000, 4096, 0, None) == 1
    assert f(0, 0x1000, 0x100000, 4096, 9, None) == 1
    assert f(0, None, 0x100000, 4096, 0, None) == 1
    assert f(0, 0x1008, 0x100000, 4096, 0, None) == 1
    assert f(0, 0x1000, 0x100000, 4096 + 16, 0, None) == 1
    assert f(0, 0x1000, 0x1800, 4096, 0, None) == 1
    assert f(0, 0x1000, 0x100000, 0, 0, None) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("cap", [0, 2])
def test_every_copy_shape_is_exact(copylib, cap):
    """Every shape copies every byte of a buffer a few tiles long and writes
    nothing past it."""
    import torch
    count = copylib.zs_copy_shape_count()
    nbytes = 3 * max(copylib.zs_copy_shape_tile_bytes(i) for i in range(count)) * 8
    rng = np.random.default_rng(cap)
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    for i in range(count):
        dst = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
        rc = copylib.zs_copy_shape(i, src.data_ptr(), dst.data_ptr(), nbytes, cap,
                                   torch.cuda.current_stream().cuda_stream)
        assert rc == 0, (i, copylib.zs_copy_last_error().decode())
        torch.cuda.synchronize()
        out = dst.cpu().numpy()
        assert np.array_equal(out[:nbytes], src.cpu().numpy()), copylib.zs_copy_shape_name(i)
        assert not out[nbytes:].any(), copylib.zs_copy_shape_name(i)


def _wave_fn(copylib):
    f = copylib.zs_wave_probe
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_uint64,
                  C.c_uint32, C.c_uint32, C.c_double, C.c_double, C.c_void_p, C.c_uint32,
                  C.c_void_p]
    return f


def test_wave_probe_refuses_before_any_launch(copylib):
    """Stream counts, vector widths, caps, windows, alignment, sizes that are
    not whole 1024-element groups and overlapping outputs are refused with 1
    before any HIP call; a request with no stream at all too."""
    f = _wave_fn(copylib)
    A = 0x7F0000000000
    n = 4096
    g = _ptrs([A + k * 0x100000 for k in range(3)])
    ok = dict(in16=g, n_in16=3, sin=A + 0x1000000, sout=A + 0x2000000, out16=A + 0x3000000,
              n=n, vecs=2, cap=0, period=0.0, open=0.0, sink=A + 0x4000000, magic=1)

    def call(**over):
        a = dict(ok, **over)
        return f(a["in16"], a["n_in16"], a["sin"], a["sout"], a["out16"], a["n"], a["vecs"],
                 a["cap"], a["period"], a["open"], a["sink"], a["magic"], None)

    assert call(n_in16=65) == 1
    assert call(in16=None) == 1
    assert call(n_in16=0, sin=None, sout=None, out16=None) == 1
    assert call(vecs=3) == 1 and call(vecs=0) == 1
    assert call(cap=33) == 1
    assert call(sink=None) == 1 and call(sink=A + 0x4000002) == 1
    assert call(n=n + 512) == 1                  # not whole 1024-element groups
    assert call(period=-1.0, open=0.1) == 1
    assert call(period=30.0, open=0.0) == 1 and call(period=30.0, open=1.0) == 1
    assert call(period=2e6, open=0.5) == 1
    assert call(sin=A + 0x1000008) == 1          # misaligned state
    assert call(out16=A + 0x3000008) == 1        # misaligned output
    assert call(sout=A + 0x1000000 + 12 * n - 16) == 1   # state out on state in
    assert call(out16=A + 0x2000000 + 12 * n - 16) == 1  # 16-bit out on state out
    assert call(out16=g[2] + 2 * n - 16) == 1    # 16-bit out on a gradient stream
    assert call(out16=A + 0x4000000 - 16) == 1   # output on the sink
    assert call(in16=_ptrs([A, 0, A + 0x200000]), n_in16=3) == 1
    assert call(n=0) == 0
    assert call(n=0, period=30.72, open=0.125) == 0


def _wave_expected(gw, sin, sout, p16, magic, n):
    """The wave probe's documented outputs, word by word: one row per
    4-element vector (two 32-bit words of a 16-bit stream, four of a state
    array)."""
    q = np.arange(n // 4, dtype=np.uint64)
    s = np.zeros((n // 4, 2), np.uint32)
    for x in gw:   # fold = rotl(fold, 1) + the stream's words, in stream order
        s = ((s << np.uint32(1)) | (s >> np.uint32(31))) + x.view(np.uint32).reshape(-1, 2)
    base = s ^ np.stack([(4 * q).astype(np.uint32), np.full(n // 4, magic, np.uint32)], 1)
    b4 = np.concatenate([base, base], 1)
    state = None
    if sin is not None:
        # grouped: [group][array][1024] -> per vector, per array, four words
        state = sin.view(np.uint32).reshape(-1, 3, 256, 4).transpose(0, 2, 1, 3).reshape(-1, 3, 4)
    want_state = None
    if sout:
        want_state = (state ^ b4[:, None, :]) if state is not None else np.repeat(b4[:, None, :], 3, 1)
    rest = base.copy()
    if state is not None and not sout:
        for j in range(3):
            rest ^= np.stack([state[:, j, 0] ^ state[:, j, 2], state[:, j, 1] ^ state[:, j, 3]], 1)
    return want_state, (rest if p16 else None)


@pytest.mark.gpu
@pytest.mark.parametrize("w,sin,sout,p16,vecs,window", [
    (1, True, True, True, 1, None), (0, False, True, True, 1, None),
    (1, True, False, False, 1, None), (3, True, True, True, 2, None),
    (4, True, False, True, 2, None), (5, True, True, True, 2, None),
    (6, True, True, False, 2, None), (7, False, False, True, 2, None),
    (8, True, True, True, 2, None), (13, True, True, True, 1, None),
    (64, True, True, True, 2, None), (64, True, True, True, 2, (2.56, 0.25)),
    (9, True, True, True, 2, (5.12, 0.125))])
def test_wave_probe_moves_what_it_states(copylib, w, sin, sout, p16, vecs, window):
    """Every output word is the documented fold of the inputs, for every
    count of streams left after the rolling sum's last full round and with
    write windows, so every stream the probe states is really read and
    written where it says."""
    import torch
    f = _wave_fn(copylib)
    n = 3 * 4096
    magic = 0x9E3779B9
    rng = np.random.default_rng(1000 + w * 10 + vecs)
    gw = [rng.integers(0, 2 ** 16, n, dtype=np.uint16) for _ in range(w)]
    g = [torch.from_numpy(x.view(np.int16)).cuda() for x in gw]
    sin_h = rng.integers(0, 2 ** 32, 3 * n, dtype=np.uint32) if sin else None
    sin_d = torch.from_numpy(sin_h.view(np.int32)).cuda() if sin else None
    sout_d = torch.zeros(3 * n, dtype=torch.int32, device="cuda") if sout else None
    o16 = torch.zeros(n, dtype=torch.int16, device="cuda") if p16 else None
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    per, op = window or (0.0, 0.0)
    rc = f(_ptrs([t.data_ptr() for t in g]), w, sin_d.data_ptr() if sin else None,
           sout_d.data_ptr() if sout else None, o16.data_ptr() if p16 else None, n, vecs, 0,
           per, op, sink.data_ptr(), magic, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, copylib.zs_copy_last_error().decode()
    torch.cuda.synchronize()
    want_state, want16 = _wave_expected(gw, sin_h, sout, p16, magic, n)
    if sout:
        got = sout_d.cpu().numpy().view(np.uint32).reshape(-1, 3, 256, 4)
        got = got.transpose(0, 2, 1, 3).reshape(-1, 3, 4)
        assert np.array_equal(got, want_state)
    if p16:
        assert np.array_equal(o16.cpu().numpy().view(np.uint32).reshape(-1, 2), want16)

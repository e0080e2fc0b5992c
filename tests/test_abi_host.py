"""Host-side checks of the C ABI: the library loads, exports every function
include/qam.h declares, and rejects bad arguments before any launch (these
calls never reach the GPU, so they run without one)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from query_adaptive_mixed_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qam.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qam_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("qam_pack_slices", "qam_build_level_map", "qam_qmatvec"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    bound = {n for n, _, _ in L.SIGNATURES}
    assert set(declared_functions()) <= bound, set(declared_functions()) - bound


def test_version_and_empty_error(lib):
    assert lib.qam_version().decode().startswith("qam")
    assert lib.qam_packed_bytes(64, 64) == 64 * 64 + 4 * 64
    assert lib.qam_packed_bytes(0, 64) == 0


def _params(f=0.5, g=0.75, combine=0, n_stops=0):
    p = L.QamLensParams()
    p.f, p.g, p.combine, p.n_stops = f, g, combine, n_stops
    return p


def _ladder(bits=(0, 2, 4, 6, 8)):
    arr = (C.c_uint8 * len(bits))(*bits)
    return C.cast(arr, C.c_void_p), arr


FAKE = C.c_void_p(0x1000)   # never dereferenced: every case below fails a host check first


@pytest.mark.parametrize("kw,code", [
    (dict(f=1.5), -3), (dict(f=-0.1), -3), (dict(g=1.01), -3), (dict(combine=7), -3),
    (dict(n_stops=5), -3),
])
def test_level_map_rejects_bad_params(lib, kw, code):
    lad, keep = _ladder()
    lens = (L.QamLens * 1)()
    lens[0].cx, lens[0].cy, lens[0].r = 0.5, 0.5, 0.2
    p = _params(**kw)
    rc = lib.qam_build_level_map(FAKE, 8, lens, 1, C.byref(p), lad, 5, 1, FAKE, None)
    assert rc == code
    assert lib.qam_last_error().decode()


def test_level_map_rejects_bad_ladders_and_glass(lib):
    lens = (L.QamLens * 1)()
    lens[0].r = 0.2
    p = _params()
    for bits, n, glass, code in [((1, 2, 4), 3, 0, -4), ((0, 4, 2), 3, 0, -4), ((0,), 1, 0, -4),
                                 ((0, 2, 4, 6, 8), 5, 5, -3), ((0, 2, 4, 6, 8), 5, -1, -3)]:
        lad, keep = _ladder(bits)
        assert lib.qam_build_level_map(FAKE, 8, lens, 1, C.byref(p), lad, n, glass, FAKE, None) == code
    lad, keep = _ladder()
    assert lib.qam_build_level_map(None, 8, lens, 1, C.byref(p), lad, 5, 1, FAKE, None) == -1
    assert lib.qam_build_level_map(FAKE, 8, lens, 65, C.byref(p), lad, 5, 1, FAKE, None) == -3
    bad = (L.QamLens * 1)()
    bad[0].r = -1.0
    assert lib.qam_build_level_map(FAKE, 8, bad, 1, C.byref(p), lad, 5, 1, FAKE, None) == -3
    ps = _params(n_stops=2)
    ps.stops[0], ps.stops[1] = 0.5, 1.0           # not decreasing
    assert lib.qam_build_level_map(FAKE, 8, lens, 1, C.byref(ps), lad, 5, 1, FAKE, None) == -3
    # zero blocks: nothing to do, success without a launch
    assert lib.qam_build_level_map(None, 0, lens, 1, C.byref(p), lad, 5, 1, None, None) == 0


def test_pack_rejects_bad_shapes_and_alignment(lib):
    d = L.QamPacked()
    for N, K in [(63, 64), (64, 65), (0, 64), (64, 0), (64, 65536 + 64)]:
        assert lib.qam_pack_slices(FAKE, FAKE, N, K, C.c_void_p(0x10000), 1 << 40, C.byref(d), None) == -2
    assert lib.qam_pack_slices(None, FAKE, 64, 64, FAKE, 1 << 20, C.byref(d), None) == -1
    assert lib.qam_pack_slices(FAKE, FAKE, 64, 64, C.c_void_p(0x10010), 1 << 20, C.byref(d), None) == -5
    assert lib.qam_pack_slices(FAKE, FAKE, 64, 64, C.c_void_p(0x10000), 10, C.byref(d), None) == -3


def test_qmatvec_rejects_bad_arguments(lib):
    d = L.QamPacked()
    assert lib.qam_describe_packed(C.c_void_p(0x100000), 128, 256, C.byref(d)) == 0
    assert d.n_blocks == 2 and d.scales == 0x100000 + 128 * 256
    X, Y, M = C.c_void_p(0x200000), C.c_void_p(0x300000), C.c_void_p(0x400000)
    assert lib.qam_qmatvec(X, 0, 0, C.byref(d), M, 0, Y, None, 0, None) == -3        # B = 0
    assert lib.qam_qmatvec(X, 0, 9, C.byref(d), M, 0, Y, None, 0, None) == -3        # B > 8
    assert lib.qam_qmatvec(X, 5, 1, C.byref(d), M, 0, Y, None, 0, None) == -3        # dtype
    assert lib.qam_qmatvec(X, 0, 1, C.byref(d), M, 1, Y, None, 0, None) == -3        # per-request maps
    assert lib.qam_qmatvec(None, 0, 1, C.byref(d), M, 0, Y, None, 0, None) == -1
    assert lib.qam_qmatvec(C.c_void_p(0x200004), 0, 1, C.byref(d), M, 0, Y, None, 0, None) == -5
    assert lib.qam_qmatvec(X, 0, 1, C.byref(d), M, 0, C.c_void_p(0x200000 + 64), None, 0, None) == -3  # overlap
    big = L.QamPacked()
    assert lib.qam_describe_packed(C.c_void_p(0x10000000), 64, 8192, C.byref(big)) == 0
    need = lib.qam_qmatvec_workspace_bytes(64, 8192, 1)
    assert need > 0
    assert lib.qam_qmatvec(X, 0, 1, C.byref(big), M, 0, Y, None, 0, None) == -7
    assert lib.qam_qmatvec(X, 0, 1, C.byref(big), M, 0, Y, C.c_void_p(0x500000), need - 1, None) == -7
    bad = L.QamPacked()
    bad.N, bad.K, bad.n_blocks, bad.planes, bad.scales = 100, 64, 1, 0x100000, 0x100000 + 6400
    assert lib.qam_qmatvec(X, 0, 1, C.byref(bad), M, 0, Y, None, 0, None) == -2


def test_workspace_size_is_zero_for_bad_shapes_and_grows_with_batch(lib):
    assert lib.qam_qmatvec_workspace_bytes(100, 64, 1) == 0
    assert lib.qam_qmatvec_workspace_bytes(64, 64, 0) == 0
    assert lib.qam_qmatvec_workspace_bytes(8192, 28672, 8) >= lib.qam_qmatvec_workspace_bytes(8192, 28672, 1)


def test_map_weight_bytes_matches_the_oracle_memory_formula(lib):
    rng = np.random.default_rng(0)
    lad, keep = _ladder()
    for _ in range(20):
        lv = rng.integers(0, 5, size=int(rng.integers(1, 300))).astype(np.uint8)
        K = int(rng.integers(1, 100)) * 64
        mb, wb = C.c_double(), C.c_int64()
        assert lib.qam_map_weight_bytes(lv.ctypes.data_as(C.c_void_p), lv.size, K, lad, 5, C.byref(mb), C.byref(wb)) == 0
        w = np.full(lv.size, 64 * K)
        assert wb.value == O.weight_bytes(lv, w)
        assert abs(mb.value - O.mean_bits(lv, w)) < 1e-12
    bad = np.array([5], dtype=np.uint8)
    assert lib.qam_map_weight_bytes(bad.ctypes.data_as(C.c_void_p), 1, 64, lad, 5, None, None) == -3

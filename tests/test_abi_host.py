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
    # the product's maps take the ladder {0,2,4,6,8} only (a rung index is the
    # slices the product reads); other valid ladders go to qam_build_rung_map
    for bits in [(0, 4, 8), (0, 2, 4, 6, 10), (0, 1, 2, 3, 4, 5, 6, 7, 8)]:
        lad2, keep2 = _ladder(bits)
        assert lib.qam_build_level_map(FAKE, 8, lens, 1, C.byref(p), lad2, len(bits), 1, FAKE, None) == -4
        assert lib.qam_build_rung_map(None, 8, lens, 1, C.byref(p), lad2, len(bits), 1, FAKE, None) == -1
        assert lib.qam_build_rung_map(None, 0, lens, 1, C.byref(p), lad2, len(bits), 1, None, None) == 0
    lad3, keep3 = _ladder((1, 2, 4))
    assert lib.qam_build_rung_map(FAKE, 8, lens, 1, C.byref(p), lad3, 3, 0, FAKE, None) == -4


def test_zone_radius_params_are_checked(lib):
    lad, keep = _ladder()
    lens = (L.QamLens * 1)()
    lens[0].cx, lens[0].cy, lens[0].r = 0.5, 0.5, 0.2
    for mode, width in [(2, 1.0), (-1, 1.0), (L.QAM_RADIUS_ZONE, -1.0), (L.QAM_RADIUS_ZONE, float("nan")),
                        (L.QAM_RADIUS_ZONE, float("inf"))]:
        p = _params()
        p.radius_mode, p.width = mode, width
        assert lib.qam_build_level_map(FAKE, 8, lens, 1, C.byref(p), lad, 5, 1, FAKE, None) == -3
        assert lib.qam_build_rung_map(FAKE, 8, lens, 1, C.byref(p), lad, 5, 1, FAKE, None) == -3


def test_field_width_and_status_reject_before_any_launch(lib):
    FAKEW = C.c_void_p(0x20000000)
    d = C.c_double()
    assert lib.qam_field_width(None, 8, FAKEW, 256, C.byref(d), None) == -1
    assert lib.qam_field_width(FAKEW, 8, None, 256, C.byref(d), None) == -1
    assert lib.qam_field_width(FAKEW, 8, FAKEW, 256, None, None) == -1
    assert lib.qam_field_width(FAKEW, 0, FAKEW, 256, C.byref(d), None) == -2
    assert lib.qam_field_width(FAKEW, L.QAM_MAX_FIELD_BLOCKS + 1, FAKEW, 256, C.byref(d), None) == -2
    assert lib.qam_field_width(FAKEW, 8, FAKEW, 255, C.byref(d), None) == -7
    assert lib.qam_field_width(FAKEW, 8, C.c_void_p(0x20000008), 256, C.byref(d), None) == -5
    st = C.c_uint32()
    assert lib.qam_status(None, 1, C.byref(st), None) == -1
    assert lib.qam_status(FAKEW, 1, None, None) == -1
    assert lib.qam_status(FAKEW, 2, C.byref(st), None) == -3


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
    assert lib.qam_qmatvec(X, 0, 33, C.byref(d), M, 0, Y, None, 0, None) == -3       # B > 32
    assert lib.qam_qmatvec(X, 0, 9, C.byref(d), M, 0, Y, None, 0, None) == -7        # matrix cores: workspace
    assert lib.qam_qmatvec(X, 0, 2, C.byref(d), M, 1, Y, None, 0, None) == -7        # per-request maps too
    assert lib.qam_qmatvec(X, 5, 1, C.byref(d), M, 0, Y, None, 0, None) == -3        # dtype
    assert lib.qam_qmatvec(X, 5, 16, C.byref(d), M, 1, Y, None, 0, None) == -3       # dtype, matrix cores
    assert lib.qam_qmatvec(X, 0, 1, C.byref(d), M, 2, Y, None, 0, None) == -3        # per_request_maps flag
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


def test_qmatvec_noalloc_rejects_before_touching_the_device(lib):
    """Argument errors and shapes beyond the static scratch are returned by
    host checks alone (no device here)."""
    d = L.QamPacked()
    assert lib.qam_describe_packed(C.c_void_p(0x100000), 128, 256, C.byref(d)) == 0
    X, Y, M = C.c_void_p(0x200000), C.c_void_p(0x300000), C.c_void_p(0x400000)
    assert lib.qam_qmatvec_noalloc(X, 0, 0, C.byref(d), M, 0, Y, None) == -3        # B = 0
    assert lib.qam_qmatvec_noalloc(X, 0, 33, C.byref(d), M, 0, Y, None) == -3       # B > 32
    assert lib.qam_qmatvec_noalloc(X, 0, 1, C.byref(d), M, 2, Y, None) == -3        # per_request_maps flag
    assert lib.qam_qmatvec_noalloc(X, 7, 1, C.byref(d), M, 0, Y, None) == -3        # dtype
    assert lib.qam_qmatvec_noalloc(None, 0, 1, C.byref(d), M, 0, Y, None) == -1
    assert lib.qam_qmatvec_noalloc(X, 0, 1, None, M, 0, Y, None) == -1
    assert lib.qam_qmatvec_noalloc(C.c_void_p(0x200004), 0, 1, C.byref(d), M, 0, Y, None) == -5
    # 2048 blocks x 65536 columns at 32 requests needs ~92 MiB of workspace
    big = L.QamPacked()
    assert lib.qam_describe_packed(C.c_void_p(0x10000000), 131072, 65536, C.byref(big)) == 0
    assert lib.qam_qmatvec_workspace_bytes(131072, 65536, 32) > L.QAM_SCRATCH_BYTES
    X2 = C.c_void_p(0x8000000000)
    assert lib.qam_qmatvec_noalloc(X2, 0, 32, C.byref(big), M, 0, Y, None) == -7
    assert b"scratch" in lib.qam_last_error()


def test_workspace_size_is_zero_for_bad_shapes_and_grows_with_batch(lib):
    assert lib.qam_qmatvec_workspace_bytes(100, 64, 1) == 0
    assert lib.qam_qmatvec_workspace_bytes(64, 64, 0) == 0
    assert lib.qam_qmatvec_workspace_bytes(8192, 28672, 8) >= lib.qam_qmatvec_workspace_bytes(8192, 28672, 1)
    assert lib.qam_qmatvec_workspace_bytes(8192, 28672, 32) > 0
    assert lib.qam_qmatvec_workspace_bytes(8192, 28672, 33) == 0
    # every workspace holds the counters and the status word
    assert lib.qam_qmatvec_workspace_bytes(64, 64, 1) >= L.QAM_WS_COUNTER_BYTES
    # pre-pass route: the six limb columns of every tile of x for 16 (32) request slots
    assert lib.qam_qmatvec_workspace_bytes(64, 4096, 16) >= 64 * 6 * 1024
    assert lib.qam_qmatvec_workspace_bytes(64, 4096, 32) >= 64 * 12 * 1024


def test_group_tuning_is_checked(lib):
    items = (L.QamGemvItem * 1)()
    items[0].w = _fake_packed(128, 256)
    for field, bad in [("target_waves", 10), ("target_waves", -1), ("max_chunk_tiles", 2000), ("tail_pct", 101),
                       ("tail_div", 65), ("ksplit", 3), ("set_max", 4), ("set_max", 17), ("tiles_per_request", 65)]:
        t = L.QamTuning()
        setattr(t, field, bad)
        assert lib.qam_group_bytes_tuned(items, 1, 1, 0, C.byref(t)) == 0, field
        assert lib.qam_group_bytes_tuned(items, 1, 4, 1, C.byref(t)) == 0, field
        g = L.QamGroup()
        assert lib.qam_group_init_tuned(items, 1, 4, 0, 1, C.byref(t), FAKE, 1 << 30, C.byref(g), None) == -3
    assert lib.qam_group_bytes_tuned(items, 1, 1, 0, None) == lib.qam_group_bytes(items, 1, 1, 0) > 0
    t = L.QamTuning()
    t.set_max = 8
    # sets of 8 for 16 requests: two sets, the same column groups per set
    assert lib.qam_group_bytes_tuned(items, 1, 16, 1, C.byref(t)) > 0
    assert lib.qam_group_bytes_tuned(items, 1, 33, 1, C.byref(t)) == 0


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


# ------------------------------------------------------------------ escalation schedule (host)

def _schedule(lib, scores, rate):
    sc = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    out = np.zeros(sc.shape[0], dtype=np.uint8)
    n = C.c_int64(-1)
    rc = lib.qam_escalation_schedule(sc.ctypes.data_as(C.c_void_p), sc.shape[0], rate,
                                     out.ctypes.data_as(C.c_void_p), C.byref(n))
    return rc, out.astype(bool), n.value


@pytest.mark.parametrize("T", [0, 1, 7, 256, 1000])
@pytest.mark.parametrize("rate", [0.0, 0.16, 0.5, 1.0])
def test_escalation_schedule_matches_oracle(lib, T, rate):
    rng = np.random.default_rng(T * 10 + int(rate * 100))
    for scores in (rng.beta(2.0, 5.0, size=T), rng.integers(0, 4, size=T).astype(np.float64)):  # ties too
        rc, got, n = _schedule(lib, scores, rate)
        assert rc == 0
        want = O.escalation_schedule(scores, rate)
        assert np.array_equal(got, want)
        assert n == int(want.sum())


def test_escalation_schedule_decode_workload(lib):
    import workloads as WL
    scores = WL.escalation_scores(0, 256)
    rc, got, n = _schedule(lib, scores, 0.16)
    assert rc == 0 and n == 41
    assert np.array_equal(got, O.escalation_schedule(scores, 0.16))
    assert O.escalation_byte_ratio(got) == 0.66015625


def test_escalation_schedule_rejects(lib):
    assert _schedule(lib, [0.1, float("nan")], 0.5)[0] == -3
    assert _schedule(lib, [0.1, 0.2], 1.5)[0] == -3
    assert _schedule(lib, [0.1, 0.2], -0.1)[0] == -3


# ------------------------------------------------------------------ fused epilogue and decoder (host checks)

def _fake_packed(N, K, base=0x100000):
    d = L.QamPacked()
    d.N, d.K, d.n_blocks = N, K, N // 64
    d.planes = base
    d.scales = base + N * K
    return d


@pytest.mark.parametrize("ep,code", [
    ((2, 0, 1e-6), -3), ((0, 3, 1e-6), -3), ((1, 0, -1.0), -3), ((1, 0, float("nan")), -3),
])
def test_qmatvec_ep_rejects_bad_epilogue(lib, ep, code):
    e = L.QamEpilogue(*ep)
    w = _fake_packed(128, 256)
    rc = lib.qam_qmatvec_ep(FAKE, 0, 1, C.byref(w), FAKE, C.byref(e), FAKE, None, 0, None)
    assert rc == code
    assert lib.qam_last_error().decode()


def _decoder_desc(n_layers=2, H=256, Q=512, KV=128, F=384, V=1024, tweak=None):
    layers = (L.QamDecoderLayer * n_layers)()
    base = 0x10000000
    for i in range(n_layers):
        layers[i].qkv = _fake_packed(Q + 2 * KV, H, base)
        layers[i].o = _fake_packed(H, Q, base)
        layers[i].gate_up = _fake_packed(2 * F, H, base)
        layers[i].down = _fake_packed(H, F, base)
    d = L.QamDecoderDesc()
    d.n_layers, d.hidden, d.q_dim, d.kv_dim, d.ffn, d.vocab = n_layers, H, Q, KV, F, V
    d.layers = layers
    d.lm_head = _fake_packed(V, H, base)
    d.eps = 1e-6
    if tweak:
        tweak(d, layers)
    return d, layers


def test_decoder_bytes_layout(lib):
    d, keep = _decoder_desc()
    nb = lib.qam_decoder_bytes(C.byref(d))
    # workspace counters + h + qkv + m + logits + 5 maps, each 256-byte aligned
    floor = (64 * 1024 * 4 + 256 * 4 + (512 + 256) * 4 + 384 * 4 + 1024 * 4 + 5 * 256)
    assert nb >= floor and nb % 256 == 0


@pytest.mark.parametrize("tweak", [
    lambda d, l: setattr(d, "ffn", 100),
    lambda d, l: setattr(d, "hidden", 250),
    lambda d, l: setattr(l[1], "o", _fake_packed(256, 256, 0x10000000)),
    lambda d, l: setattr(d, "lm_head", _fake_packed(960, 256, 0x10000000)),
    lambda d, l: setattr(d, "n_layers", 0),
    lambda d, l: setattr(d, "eps", -1.0),
])
def test_decoder_rejects_bad_descriptions(lib, tweak):
    d, keep = _decoder_desc(tweak=tweak)
    assert lib.qam_decoder_bytes(C.byref(d)) == 0
    h = C.c_void_p()
    assert lib.qam_decoder_create(C.byref(d), FAKE, 1 << 30, C.byref(h), None) in (-2, -3)
    assert not h.value


def test_decoder_create_checks_memory_before_any_launch(lib):
    d, keep = _decoder_desc()
    nb = lib.qam_decoder_bytes(C.byref(d))
    h = C.c_void_p()
    assert lib.qam_decoder_create(C.byref(d), FAKE, nb - 1, C.byref(h), None) == -7
    assert lib.qam_decoder_create(C.byref(d), C.c_void_p(0x1010), nb, C.byref(h), None) == -5
    assert lib.qam_decoder_create(C.byref(d), None, nb, C.byref(h), None) == -1
    assert lib.qam_decoder_step(None, 2, None) == -1
    assert lib.qam_decoder_replay(None, 2, None) == -1


def test_build_level_maps_rejects(lib):
    lad, keep = _ladder()
    n_maps, n_lenses = 3, 2
    lenses = (L.QamLens * (n_maps * n_lenses))()
    for i in range(n_maps * n_lenses):
        lenses[i].cx, lenses[i].cy, lenses[i].r = 0.5, 0.5, 0.2
    params = (L.QamLensParams * n_maps)()
    for k in range(n_maps):
        params[k].f, params[k].g = 0.5, 1.0
    assert lib.qam_build_level_maps(FAKE, 8, lenses, n_lenses, params, lad, 5, 1, 0, FAKE, None) == -3
    assert lib.qam_build_level_maps(FAKE, 8, lenses, n_lenses, params, lad, 5, 1, 33, FAKE, None) == -3
    assert lib.qam_build_level_maps(FAKE, 8, lenses, n_lenses, params, lad, 5, 1, 3, None, None) == -1
    params[2].f = 1.5
    assert lib.qam_build_level_maps(FAKE, 8, lenses, n_lenses, params, lad, 5, 1, 3, FAKE, None) == -3
    params[2].f = 0.5
    lenses[5].r = -1.0
    assert lib.qam_build_level_maps(FAKE, 8, lenses, n_lenses, params, lad, 5, 1, 3, FAKE, None) == -3
    assert lib.qam_build_level_maps(FAKE, 8, lenses, 65, params, lad, 5, 1, 3, FAKE, None) == -3


def test_group_calls_reject_bad_descriptors_before_any_launch(lib):
    assert lib.qam_qmatvec_group(None, None) == -1
    g = L.QamGroup()          # zeroed: no table, no map
    assert lib.qam_qmatvec_group(C.byref(g), None) == -1
    out = (C.c_float * 4)()
    assert lib.qam_group_launch_times(None, 4, C.cast(out, C.c_void_p), None) == -1
    assert lib.qam_group_launch_times(C.byref(g), 4, C.cast(out, C.c_void_p), None) == -1
    g.table, g.wg_map, g.n_workgroups, g.B = 0x10000000, 0x10001000, 8, 1
    assert lib.qam_group_launch_times(C.byref(g), 4, C.cast(out, C.c_void_p), None) == -1   # no device memory
    g.dev_mem = 0x10002000
    g.route = 1               # the timing hook serves staged-limb groups only
    assert lib.qam_group_launch_times(C.byref(g), 4, C.cast(out, C.c_void_p), None) == -3
    g.route = 0
    assert lib.qam_group_launch_times(C.byref(g), 0, C.cast(out, C.c_void_p), None) == -3
    assert lib.qam_group_launch_times(C.byref(g), 4, None, None) == -1
    g.B = 2                   # the staged-limb route takes one request
    assert lib.qam_qmatvec_group(C.byref(g), None) == -3


def test_group_lens_rejects_before_any_launch(lib):
    """The launch that builds the maps checks the group, the ladder and the
    lens rules on the host; every rejection returns before any HIP call."""
    lens = (L.QamLens * 1)()
    lens[0].cx, lens[0].cy, lens[0].r = 0.5, 0.5, 0.2
    p = L.QamLensParams()
    p.f, p.g, p.combine = 0.5, 1.0, L.QAM_COMBINE_SUM
    lad = (C.c_uint8 * 5)(0, 2, 4, 6, 8)
    ladp = C.cast(lad, C.c_void_p)
    out = (C.c_float * 4)()

    def run(g, n_lenses=1, params=p, ladder=ladp, n_rungs=5, glass=1):
        return lib.qam_qmatvec_group_lens(C.byref(g) if g is not None else None, lens, n_lenses, C.byref(params),
                                          ladder, n_rungs, glass, None)

    assert run(None) == -1
    g = L.QamGroup()                      # zeroed: no table, no map
    assert run(g) == -1
    g.table, g.wg_map, g.n_workgroups, g.B = 0x10000000, 0x10001000, 8, 1
    assert run(g) == -1                   # no device memory
    g.dev_mem = 0x10002000
    assert run(g) == -3                   # no coordinates bound
    g.lens_ready = 1
    g.route = 1                           # pre-pass route: maps are not built in its launch
    assert run(g) == -3
    g.route = 0
    g.B = 2                               # the fused launch serves one request
    assert run(g) == -3
    g.B = 1
    assert run(g, ladder=None) == -1
    assert run(g, n_rungs=4) == -4        # the product ladder only
    lad2 = (C.c_uint8 * 5)(0, 2, 4, 6, 10)
    assert run(g, ladder=C.cast(lad2, C.c_void_p)) == -4
    assert run(g, glass=5) == -3
    assert run(g, n_lenses=65) == -3
    bad = L.QamLensParams()
    bad.f, bad.g, bad.combine = 1.5, 1.0, L.QAM_COMBINE_SUM
    assert run(g, params=bad) == -3
    assert lib.qam_group_lens_launch_times(C.byref(g), lens, 1, C.byref(p), ladp, 5, 1, 0,
                                           C.cast(out, C.c_void_p), None) == -3
    assert lib.qam_group_lens_launch_times(C.byref(g), lens, 1, C.byref(p), ladp, 5, 1, 4, None, None) == -1
    g.lens_ready = 0
    assert lib.qam_group_lens_launch_times(C.byref(g), lens, 1, C.byref(p), ladp, 5, 1, 4,
                                           C.cast(out, C.c_void_p), None) == -3


def test_gate_rejects_before_any_launch(lib):
    FAKEW = 0x20000000            # 256-byte aligned stand-ins, never dereferenced
    assert lib.qam_gate_workspace_bytes(1) == 0
    need = lib.qam_gate_workspace_bytes(151936)
    assert need >= 256 + 149 * 48
    assert lib.qam_gate(None, 100, 1.0, 0.1, FAKEW, FAKEW, need, None) == -1
    assert lib.qam_gate(FAKEW, 100, 1.0, 0.1, None, FAKEW, need, None) == -1
    assert lib.qam_gate(FAKEW, 1, 1.0, 0.1, FAKEW, FAKEW, need, None) == -2
    assert lib.qam_gate(FAKEW, 1 << 31, 1.0, 0.1, FAKEW, FAKEW, need, None) == -2
    assert lib.qam_gate_workspace_bytes(1 << 31) == 0
    assert lib.qam_gate(FAKEW, 100, float("nan"), 0.1, FAKEW, FAKEW, need, None) == -3
    assert lib.qam_gate(FAKEW, 151936, 1.0, 0.1, FAKEW, FAKEW, need - 1, None) == -7
    assert lib.qam_gate(FAKEW, 100, 1.0, 0.1, FAKEW, FAKEW + 8, need, None) == -5
    assert lib.qam_gate(FAKEW + 2, 100, 1.0, 0.1, FAKEW, FAKEW, need, None) == -5


def test_fit_focus_area_rejects_before_any_launch(lib):
    FAKEW = 0x20000000
    lens = (L.QamLens * 1)()
    lens[0].cx, lens[0].cy, lens[0].r = 0.5, 0.5, 0.2
    p = L.QamLensParams()
    p.f, p.g, p.combine = 0.0, 1.0, L.QAM_COMBINE_SUM
    lad = (C.c_uint8 * 5)(0, 2, 4, 6, 8)
    f, b = C.c_double(), C.c_int64()

    def call(n=8, coords=FAKEW, w=FAKEW, params=p, ladder=lad, n_rungs=5, glass=1, budget=100, iters=10,
             out=FAKEW, ws=FAKEW, ws_bytes=256, fo=True):
        return lib.qam_fit_focus_area(coords, n, w, lens, 1, C.byref(params) if params is not None else None,
                                      C.cast(ladder, C.c_void_p) if ladder is not None else None, n_rungs, glass,
                                      budget, iters, out, ws, ws_bytes, C.byref(f) if fo else None, C.byref(b), None)

    assert call(params=None) == -1
    assert call(fo=False) == -1
    assert call(coords=None) == -1
    assert call(n=0) == -2
    assert call(iters=61) == -3
    assert call(budget=-1) == -3
    assert call(ws_bytes=255) == -7
    assert call(ws=FAKEW + 8) == -5
    assert call(n_rungs=1) == -4
    assert call(glass=7) == -3


def test_layer_levels_rejects_before_any_launch(lib):
    FAKEW = 0x20000000            # 256-byte aligned stand-ins, never dereferenced
    w = L.QamPacked(N=640, K=128, n_blocks=10, planes=FAKEW, scales=FAKEW + 640 * 128)

    def rule(mode=L.QAM_LAYER_THRESHOLD, lam=1.0, share=0.5, g=1.0):
        return L.QamLayerRule(mode=mode, reserved=0, lam=lam, share=share, g=g)

    def call(y=FAKEW, B=2, ww=w, r=None, n_rungs=5, glass=1, shat=FAKEW, out=FAKEW):
        r = rule() if r is None else r
        return lib.qam_layer_levels(y, B, C.byref(ww) if ww is not None else None, C.byref(r), n_rungs, glass,
                                    shat, out, None)

    assert call(y=None) == -1
    assert call(shat=None) == -1
    assert call(out=None) == -1
    assert call(ww=None) == -1
    assert call(ww=L.QamPacked(N=640, K=128, n_blocks=9, planes=FAKEW, scales=FAKEW)) == -2
    assert call(ww=L.QamPacked(N=600, K=128, n_blocks=9, planes=FAKEW, scales=FAKEW)) == -2
    assert call(B=-1) == -3
    assert call(B=65536) == -3
    assert call(glass=5) == -4
    assert call(n_rungs=0, glass=0) == -4
    assert call(r=rule(mode=2)) == -3
    assert call(r=rule(g=1.5)) == -3
    assert call(r=rule(g=float("nan"))) == -3
    assert call(r=rule(lam=float("nan"))) == -3
    assert call(r=rule(mode=L.QAM_LAYER_SHARE, share=-0.1)) == -3
    assert call(r=rule(mode=L.QAM_LAYER_SHARE, share=float("nan"))) == -3
    assert call(y=FAKEW + 4) == -5
    assert call(shat=FAKEW + 4) == -5
    assert call(B=0, y=None, shat=None, out=None) == 0          # nothing to do, nothing launched


def test_layer_levels_group_rejects_before_any_launch(lib):
    FAKEW = 0x20000000

    def item(nb=10, y=FAKEW, shat=FAKEW, out=FAKEW):
        w = L.QamPacked(N=64 * nb, K=128, n_blocks=nb, planes=FAKEW, scales=FAKEW + 64 * nb * 128)
        return L.QamLayerItem(y_base=y, w=w, shat_out=shat, level_out=out)

    rule = L.QamLayerRule(mode=L.QAM_LAYER_SHARE, reserved=0, lam=1.0, share=0.5, g=1.0)

    def call(items, n=None, B=2, r=rule, glass=1):
        arr = (L.QamLayerItem * max(1, len(items)))(*items)
        return lib.qam_layer_levels_group(arr, len(items) if n is None else n, B, C.byref(r), 5, glass, None)

    assert lib.qam_layer_levels_group(None, 1, 2, C.byref(rule), 5, 1, None) == -1
    assert call([item()], n=0) == -3
    assert call([item()] * 17) == -3
    assert call([item(), item(y=None)]) == -1
    assert call([item(), item(nb=513)]) == -2
    assert call([item(), item(y=FAKEW + 4)]) == -5
    assert call([item()], glass=5) == -4
    assert call([item()], r=L.QamLayerRule(mode=L.QAM_LAYER_SHARE, reserved=0, lam=1.0, share=2.0, g=1.0)) == -3
    assert call([item(y=None, shat=None, out=None)], B=0) == 0      # nothing to do, nothing launched


def test_group_refine_rejects_before_any_launch(lib):
    FAKEW = 0x20000000
    assert lib.qam_qmatvec_group_refine(None, 1, None) == -1
    g = L.QamGroup()
    assert lib.qam_qmatvec_group_refine(C.byref(g), 1, None) == -1          # uninitialised
    g.table, g.wg_map, g.pre_map = FAKEW, FAKEW, FAKEW
    g.route, g.B, g.n_workgroups = 0, 4, 10
    assert lib.qam_qmatvec_group_refine(C.byref(g), 1, None) == -3          # staged route
    g.route = 1
    assert lib.qam_qmatvec_group_refine(C.byref(g), 0, None) == -3
    assert lib.qam_qmatvec_group_refine(C.byref(g), 4, None) == -3


def test_timeline_calls_refuse_in_the_product_library(lib):
    assert lib.qam_timeline_select(None, 0) == -3
    assert lib.qam_timeline_read(None, 0) == -3
    assert "without the timeline" in lib.qam_last_error().decode()


def test_timeline_library_exports_and_checks_arguments():
    path = os.path.join(ROOT, "query_adaptive_mixed_amd", "libqam_timeline.so")
    if not os.path.exists(path):
        pytest.skip("the timeline library is not built")
    tl = L.load(path)
    assert not [n for n in declared_functions() if not hasattr(tl, n)]
    assert tl.qam_timeline_select(None, -1) == -3
    assert tl.qam_timeline_select(None, L.QAM_TIMELINE_SLOTS + 1) == -3
    assert tl.qam_timeline_select(None, 2) == -1
    assert tl.qam_timeline_read(None, 1 << 30) == -1
    small = (C.c_uint64 * 4)()
    assert tl.qam_timeline_read(C.cast(small, C.c_void_p), 4) == -3

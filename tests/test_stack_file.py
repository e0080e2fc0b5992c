"""Stored-stack file: the oracle's writer and reader pinned by hand-computed
byte positions and header offsets, depth reads against truncation, and the
library's host-side header check (qam_stack_info) on oracle-written files.

No device is needed: qam_stack_info touches only the file.
"""

import ctypes as C
import json
import os

import numpy as np
import pytest

import oracle as O
import oracle.stack_file as S

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "stack_layout_examples.json")))


@pytest.fixture(scope="module")
def lib():
    from query_adaptive_mixed_amd import _lib as L
    return L.lib()


@pytest.mark.parametrize("ex", GOLD["positions"], ids=lambda e: f"r{e['row']}c{e['col']}s{e['s']}")
def test_digit_positions_match_hand_examples(ex):
    byte, bit = S.digit_position(ex["N"], ex["K"], ex["row"], ex["col"], ex["s"])
    assert (int(byte), int(bit)) == (ex["byte"], ex["bit"])


def test_one_code_lands_where_worked_by_hand():
    oc = GOLD["one_code"]
    W = np.zeros((64, 64), dtype=np.int8)
    W[oc["row"], oc["col"]] = oc["code"]
    pl = S.planes_of(W)
    for p in range(4):
        nz = [[int(i), int(pl[p][i])] for i in np.flatnonzero(pl[p])]
        assert nz == oc["nonzero_bytes"][str(p)], p


def test_every_digit_has_its_own_bit():
    """The position map is a bijection of (row, col, s) onto the plane bits."""
    N, K = 128, 192
    rows, cols = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    for s in range(4):
        byte, bit = S.digit_position(N, K, rows, cols, s)
        key = (byte * 8 + bit).ravel()
        assert key.min() >= 0 and key.max() < N * K * 2
        assert np.unique(key).size == N * K
        assert np.all(bit % 2 == 0)


def test_header_offsets_match_hand_example():
    hd, offs = S.layout([tuple(s) for s in GOLD["header"]["shapes"]])
    g = GOLD["header"]
    for k in ("data_offset", "plane_section_bytes", "scales_offset", "scales_bytes", "file_bytes"):
        assert hd[k] == g[k], k
    assert [o[0] for o in offs] == g["plane_offsets"]
    assert [o[1] for o in offs] == g["scales_offsets"]
    assert S.read_bytes(g["shapes"], 2) == g["read_bytes_4bit"]


@pytest.mark.parametrize("slices", [1, 2, 3, 4])
def test_depth_read_is_truncation(tmp_path, slices):
    """Reading the first d/2 sections gives the codes truncated to d bits
    (every int8 value, -128 included)."""
    rng = np.random.default_rng(slices)
    W1 = np.arange(256, dtype=np.int64).reshape(64, 4).repeat(16, axis=1).astype(np.uint8).view(np.int8)
    W2 = rng.integers(-128, 128, size=(192, 128)).astype(np.int8)
    sc1 = rng.uniform(0.001, 0.02, 64).astype(np.float32)
    sc2 = rng.uniform(0.001, 0.02, 192).astype(np.float32)
    path = str(tmp_path / "s.qamstack")
    S.write_stack(path, [("first", W1, sc1), ("second", W2, sc2)])
    got = S.read_stack(path, slices)
    assert [g[0] for g in got] == ["first", "second"]
    for (name, codes, sc), W, scw in zip(got, (W1, W2), (sc1, sc2)):
        assert np.array_equal(codes, O.truncate(W, 2 * slices)), name
        assert np.array_equal(sc, scw)


def test_file_length_and_zero_padding(tmp_path):
    rng = np.random.default_rng(3)
    mats = [(f"m{i}", rng.integers(-128, 128, size=(64 * (i + 1), 64)).astype(np.int8),
             np.ones(64 * (i + 1), np.float32)) for i in range(3)]
    data = S.stack_bytes(mats)
    hd, ents = S.read_header(data)
    assert len(data) == hd["file_bytes"]
    assert data[S.HEADER_BYTES + S.ENTRY_BYTES * 3:hd["data_offset"]] == bytes(hd["data_offset"] - 128 - 192)
    assert hd["magic"] == b"QAMSTACK" and hd["ladder"] == O.LADDER_BITS and hd["reserved"] == bytes(48)


# ------------------------------------------------------------------ library header check (host only)

def _write(tmp_path, data, name="f.qamstack"):
    p = str(tmp_path / name)
    with open(p, "wb") as f:
        f.write(data)
    return p


def _mats():
    rng = np.random.default_rng(11)
    return [("attn", rng.integers(-128, 128, size=(128, 64)).astype(np.int8), np.ones(128, np.float32)),
            ("", rng.integers(-128, 128, size=(64, 256)).astype(np.int8), np.ones(64, np.float32))]


def test_library_reads_oracle_header(lib, tmp_path):
    from query_adaptive_mixed_amd import _lib as L
    data = S.stack_bytes(_mats())
    p = _write(tmp_path, data)
    hd, ents = S.read_header(data)
    h = L.QamStackHeader()
    e = (L.QamStackEntry * 4)()
    assert lib.qam_stack_info(p.encode(), C.byref(h), e, 4) == 0
    assert bytes(h.magic) == b"QAMSTACK" and h.version == 1 and h.n_matrices == 2
    for k in ("data_offset", "plane_section_bytes", "scales_offset", "scales_bytes", "file_bytes"):
        assert getattr(h, k) == hd[k], k
    for i, ref in enumerate(ents):
        assert (e[i].N, e[i].K, e[i].plane_offset, e[i].scales_offset) == (ref["N"], ref["K"], ref["plane_offset"],
                                                                          ref["scales_offset"])
        assert e[i].name.decode() == ref["name"]


def _patched(data, off, raw):
    b = bytearray(data)
    b[off:off + len(raw)] = raw
    return bytes(b)


def test_library_rejects_malformed_files(lib, tmp_path):
    from query_adaptive_mixed_amd import _lib as L
    data = S.stack_bytes(_mats())
    h = L.QamStackHeader()
    bad = {
        "magic": _patched(data, 0, b"QAMSTACX"),
        "version": _patched(data, 8, (2).to_bytes(4, "little")),
        "count": _patched(data, 12, (0).to_bytes(4, "little")),
        "ladder": _patched(data, 20, bytes([0, 2, 4, 6, 7])),
        "reserved": _patched(data, 127, b"\x01"),
        "data_offset": _patched(data, 40, (8192).to_bytes(8, "little")),
        "entry_shape": _patched(data, 128, (100).to_bytes(8, "little")),
        "entry_offset": _patched(data, 128 + 64 + 16, (7).to_bytes(8, "little")),
        "truncated": data[:-1],
        "longer": data + b"\0",
        "short": data[:100],
    }
    for what, blob in bad.items():
        p = _write(tmp_path, blob, what)
        assert lib.qam_stack_info(p.encode(), C.byref(h), None, 0) == -8, what
    assert lib.qam_stack_info(str(tmp_path / "missing").encode(), C.byref(h), None, 0) == -8
    assert lib.qam_stack_info(None, C.byref(h), None, 0) == -1
    p = _write(tmp_path, data)
    assert lib.qam_stack_info(p.encode(), C.byref(h), None, 1) == -3      # entries_out NULL with room asked


def test_library_read_rejects_bad_arguments_before_device_work(lib, tmp_path):
    from query_adaptive_mixed_amd import _lib as L
    data = S.stack_bytes(_mats())
    p = _write(tmp_path, data).encode()
    d = (L.QamPacked * 2)()
    assert lib.qam_describe_packed(C.c_void_p(0x100000), 128, 64, C.byref(d[0])) == 0
    assert lib.qam_describe_packed(C.c_void_p(0x200000), 64, 256, C.byref(d[1])) == 0
    n = C.c_uint64(0)
    assert lib.qam_stack_read(p, 0, 0, 2, d, None, C.byref(n)) == -3       # slices
    assert lib.qam_stack_read(p, 5, 0, 2, d, None, C.byref(n)) == -3
    assert lib.qam_stack_read(p, 2, 1, 2, d, None, C.byref(n)) == -3       # range
    assert lib.qam_stack_read(p, 2, 0, 0, d, None, C.byref(n)) == -3
    assert lib.qam_stack_read(p, 2, 1, 1, d, None, C.byref(n)) == -2       # shape of destination 0
    assert lib.qam_stack_read(b"/nonexistent/x", 2, 0, 2, d, None, C.byref(n)) == -8
    assert lib.qam_stack_read(p, 2, 0, 2, None, None, C.byref(n)) == -1
    w = (L.QamPacked * 1)()
    assert lib.qam_stack_write(p, w, None, 0, None) == -3
    assert lib.qam_stack_write(p, w, None, 1, None) == -2                  # empty descriptor


def test_library_header_check_survives_random_corruption(lib, tmp_path):
    """Seeded byte flips and truncations of the header and table: every call
    returns OK (a flip the layout does not reject: a name byte) or
    QAM_ERR_IO, and never reads outside the file (run this under the
    host-sanitizer build to check the last part)."""
    from query_adaptive_mixed_amd import _lib as L
    rng = np.random.default_rng(2024)
    data = S.stack_bytes(_mats())
    hdr, ents = S.read_header(data)
    h = L.QamStackHeader()
    e = (L.QamStackEntry * 4)()
    table_end = S.HEADER_BYTES + S.ENTRY_BYTES * len(ents)
    name_bytes = set()
    for m in range(len(ents)):
        base = S.HEADER_BYTES + S.ENTRY_BYTES * m + 32
        name_bytes.update(range(base, base + S.NAME_BYTES))
    for case in range(300):
        b = bytearray(data)
        for _ in range(int(rng.integers(1, 4))):
            pos = int(rng.integers(0, table_end))
            b[pos] ^= int(rng.integers(1, 256))
        if case % 7 == 0:
            b = b[:int(rng.integers(0, len(b)))]
        p = _write(tmp_path, bytes(b), f"c{case}")
        rc = lib.qam_stack_info(p.encode(), C.byref(h), e, 4)
        changed = [i for i in range(min(len(b), len(data))) if b[i] != data[i]]
        if len(b) == len(data) and all(i in name_bytes for i in changed):
            assert rc == 0, case
        else:
            assert rc in (0, -8), (case, rc)

"""Plain writer and reader of the stored-stack file (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): it defines, from the
layout statement alone, the bytes a stack file must hold, so that the
library's writer can be compared with it byte for byte and its reader fed
files this module wrote.

[FoQLens] "Progress": one stored stack, a base with refinements over it,
read at 2, 4, 6 or 8 bits without repacking.  The pages give no file layout;
the one written here is this project's own and is stated in full:

* the digits: ``slice_digits`` of each int8 code (digit s = 3 is the top);
* plane p = 0..3 holds digit 3 - p of every code of a matrix;
* inside a plane: block b (rows 64b..64b+63) owns 16 K bytes, tile t
  (columns 64t..64t+63) of the block owns 1024 bytes, lane L = 0..63 of the
  tile owns 16 bytes = four little-endian 32-bit words j = 0..3; word j holds
  the digits of row 16 j + (L mod 16) and columns 16 (L div 16) + 4 u + i
  (u, i = 0..3), digit (u, i) at bit (8 i + 2 s - 2 u) mod 32 of the word;
* the file: a 128-byte header, one 64-byte entry per matrix, zeros up to
  ``data_offset`` (the table's end rounded up to 4096), then plane sections
  p = 0..3 (section p holds plane p of every matrix in order), then the fp32
  scales of every matrix in order.

A read at depth d takes the first d/2 sections and the scales.
"""

from __future__ import annotations

import struct

import numpy as np

from .qam_oracle import LADDER_BITS, ROWS_PER_BLOCK, residual_code, slice_digits

MAGIC = b"QAMSTACK"
VERSION = 1
HEADER_BYTES = 128
ENTRY_BYTES = 64
NAME_BYTES = 32
ALIGN = 4096

# header: magic, version, n_matrices, n_rungs, ladder[16], rows_per_block,
# data_offset, plane_section_bytes, scales_offset, scales_bytes, file_bytes,
# 48 reserved bytes
_HEADER = struct.Struct("<8sIII16sIQQQQQ48s")
_ENTRY = struct.Struct("<qqQQ32s")
assert _HEADER.size == HEADER_BYTES and _ENTRY.size == ENTRY_BYTES


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def digit_position(N: int, K: int, row, col, s):
    """(byte offset inside a plane, bit inside that byte) of digit ``s`` of
    code (row, col), straight from the layout statement."""
    row, col, s = np.asarray(row), np.asarray(col), np.asarray(s)
    b, r = row // 64, row % 64
    t, c = col // 64, col % 64
    j = r // 16
    lane = (r % 16) + 16 * (c // 16)
    u, i = (c % 16) // 4, c % 4
    word = b * 16 * K + t * 1024 + lane * 16 + j * 4
    bit = (8 * i + 2 * s - 2 * u) % 32
    return word + bit // 8, bit % 8        # little-endian word: bit k lives in byte k // 8


def planes_of(W) -> np.ndarray:
    """uint8 [4, N*K/4]: the four planes of int8 codes W [N, K]."""
    W = np.asarray(W)
    N, K = W.shape
    assert N % ROWS_PER_BLOCK == 0 and K % 64 == 0
    dig = slice_digits(W)                                  # [N, K, 4], digit s at [..., s]
    rows, cols = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    out = np.zeros((4, N * K // 4), dtype=np.uint8)
    for p in range(4):
        s = 3 - p
        byte, bit = digit_position(N, K, rows, cols, s)
        vals = (dig[..., s] << bit).astype(np.uint8)
        # every (byte, bit) pair is hit by exactly one digit, so the bytes are sums of disjoint bit fields
        np.add.at(out[p], byte.ravel(), vals.ravel())
    return out


def codes_from_planes(planes, N: int, K: int, slices: int) -> np.ndarray:
    """int64 codes at depth 2*slices read back from the first ``slices`` planes."""
    rows, cols = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    dig = np.zeros((N, K, 4), dtype=np.int64)
    for p in range(slices):
        s = 3 - p
        byte, bit = digit_position(N, K, rows, cols, s)
        dig[..., s] = (np.asarray(planes[p])[byte].astype(np.int64) >> bit) & 3
    return residual_code(dig, 2 * slices)


def layout(shapes):
    """Header fields and per-matrix (plane_offset, scales_offset) for shapes [(N, K)]."""
    plane, scales, offs = 0, 0, []
    for N, K in shapes:
        offs.append((plane, scales))
        plane += N * K // 4
        scales += 4 * N
    data = _round_up(HEADER_BYTES + ENTRY_BYTES * len(shapes), ALIGN)
    return dict(data_offset=data, plane_section_bytes=plane, scales_offset=data + 4 * plane,
                scales_bytes=scales, file_bytes=data + 4 * plane + scales), offs


def stack_bytes(mats) -> bytes:
    """The whole file for ``mats`` = [(name, W int8 [N, K], scales fp32 [N])]."""
    shapes = [np.asarray(W).shape for _, W, _ in mats]
    hd, offs = layout(shapes)
    ladder = bytes(LADDER_BITS) + bytes(16 - len(LADDER_BITS))
    head = _HEADER.pack(MAGIC, VERSION, len(mats), len(LADDER_BITS), ladder, ROWS_PER_BLOCK, hd["data_offset"],
                        hd["plane_section_bytes"], hd["scales_offset"], hd["scales_bytes"], hd["file_bytes"],
                        bytes(48))
    table = b"".join(_ENTRY.pack(N, K, po, so, (name or "").encode().ljust(NAME_BYTES, b"\0")[:NAME_BYTES])
                     for (name, _, _), (N, K), (po, so) in zip(mats, shapes, offs))
    buf = bytearray(hd["file_bytes"])
    buf[:HEADER_BYTES] = head
    buf[HEADER_BYTES:HEADER_BYTES + len(table)] = table
    planes = [planes_of(W) for _, W, _ in mats]
    for p in range(4):
        base = hd["data_offset"] + p * hd["plane_section_bytes"]
        for pl, (po, _) in zip(planes, offs):
            buf[base + po:base + po + pl.shape[1]] = pl[p].tobytes()
    for (_, _, sc), (so_pl, so) in zip(mats, offs):
        raw = np.asarray(sc, dtype="<f4").tobytes()
        buf[hd["scales_offset"] + so:hd["scales_offset"] + so + len(raw)] = raw
    return bytes(buf)


def write_stack(path: str, mats) -> None:
    with open(path, "wb") as f:
        f.write(stack_bytes(mats))


def read_header(data: bytes):
    """(header dict, entries list of dicts) of a stack file's bytes."""
    (magic, version, n, n_rungs, ladder, rpb, data_off, psec, soff, sbytes, fbytes,
     reserved) = _HEADER.unpack_from(data, 0)
    hd = dict(magic=magic, version=version, n_matrices=n, n_rungs=n_rungs, ladder=tuple(ladder[:n_rungs]),
              rows_per_block=rpb, data_offset=data_off, plane_section_bytes=psec, scales_offset=soff,
              scales_bytes=sbytes, file_bytes=fbytes, reserved=reserved)
    ents = []
    for m in range(n):
        N, K, po, so, name = _ENTRY.unpack_from(data, HEADER_BYTES + ENTRY_BYTES * m)
        ents.append(dict(N=N, K=K, plane_offset=po, scales_offset=so, name=name.rstrip(b"\0").decode()))
    return hd, ents


def read_stack(path: str, slices: int):
    """[(name, codes at depth 2*slices int64 [N, K], scales fp32 [N])] from a file."""
    with open(path, "rb") as f:
        data = f.read()
    hd, ents = read_header(data)
    out = []
    for e in ents:
        N, K = e["N"], e["K"]
        pb = N * K // 4
        planes = [np.frombuffer(data, np.uint8, pb, hd["data_offset"] + p * hd["plane_section_bytes"]
                                + e["plane_offset"]) for p in range(slices)]
        sc = np.frombuffer(data, "<f4", N, hd["scales_offset"] + e["scales_offset"]).astype(np.float32)
        out.append((e["name"], codes_from_planes(planes, N, K, slices), sc))
    return out


def read_bytes(shapes, slices: int) -> int:
    """Bytes a read at depth 2*slices moves: slices * sum(N K / 4) + sum(4 N)."""
    return sum(slices * N * K // 4 + 4 * N for N, K in shapes)

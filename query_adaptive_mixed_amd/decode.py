"""Packing a decoder-only model's matrices for libqam's decode driver.

The driver reads each layer with four products: q|k|v stacked as one
matrix, o, gate|up interleaved per 64-row block (32 gate rows, then the 32
matching up rows, so that one block's wavefront holds both halves of the
gated activation), and down; then the head.  This module only arranges rows
and packs them (offline, host-side layout); the step itself runs in libqam.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np
import torch

from .api import Decoder, PackedMatrix, pack_slices


def stack_rows(*mats: np.ndarray) -> np.ndarray:
    """Rows of the given matrices (or scale vectors) one after the other."""
    return np.ascontiguousarray(np.concatenate(mats, axis=0))


def interleave_gate_up(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """Rows (or scales) ordered per 64-row block as gate[32j:32j+32] then up[32j:32j+32]."""
    if gate.shape != up.shape or gate.shape[0] % 32:
        raise ValueError("gate and up need the same shape and a row count divisible by 32")
    F = gate.shape[0]
    g = gate.reshape((F // 32, 32) + gate.shape[1:])
    u = up.reshape((F // 32, 32) + up.shape[1:])
    return np.ascontiguousarray(np.concatenate([g, u], axis=1).reshape((2 * F,) + gate.shape[1:]))


def _pack(codes: np.ndarray, scales: np.ndarray, device) -> PackedMatrix:
    W = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.int8)).to(device)
    s = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).to(device)
    pm = pack_slices(W, s)
    torch.cuda.current_stream().synchronize()
    return pm


def build_decoder(field, n_layers: int, hidden: int, q_dim: int, kv_dim: int, ffn: int, eps: float = 1e-6,
                  target_waves: int = 0, waves_per_block: int = 0, max_chunk_tiles: int = 0, device="cuda",
                  progress=None) -> Decoder:
    """Pack a field made by ``workloads.decoder_field`` (per layer q, k, v, o,
    gate, up, down, then the head) and create the decoder over it."""
    layers = []
    for l in range(n_layers):
        i = 7 * l
        c = [field.codes(i + j) for j in range(7)]
        s = [field.scales(i + j) for j in range(7)]
        qkv = _pack(stack_rows(c[0], c[1], c[2]), stack_rows(s[0], s[1], s[2]), device)
        o = _pack(c[3], s[3], device)
        gu = _pack(interleave_gate_up(c[4], c[5]), interleave_gate_up(s[4], s[5]), device)
        down = _pack(c[6], s[6], device)
        layers.append((qkv, o, gu, down))
        if progress is not None:
            progress(l)
    lm = _pack(field.codes(7 * n_layers), field.scales(7 * n_layers), device)
    return Decoder(layers, lm, hidden, q_dim, kv_dim, ffn, eps=eps, target_waves=target_waves,
                   waves_per_block=waves_per_block, max_chunk_tiles=max_chunk_tiles, device=device)


def decoder_matrices(dec: Decoder) -> Sequence:
    """The packed matrices a decoder holds: [(qkv, o, gate_up, down), ...] and the head."""
    return dec._keep[1:], dec._keep[0]

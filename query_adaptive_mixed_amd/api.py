"""Thin Python binding over libqam (argument marshalling only).

PyTorch supplies device memory and the current HIP stream; every step of
the computation runs in libqam's kernels.  Names follow the C ABI:
``pack_slices``, ``build_level_map``, ``qmatvec`` plus the probes and
helpers ``unpack_codes``, ``map_weight_bytes`` and ``workspace_bytes``.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L

LADDER_BITS = (0, 2, 4, 6, 8)


def _stream_handle() -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor) -> C.c_void_p:
    return C.c_void_p(t.data_ptr())


def _require_cuda(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class PackedMatrix:
    """One packed matrix: the device buffer (slice planes + scales) and its descriptor."""
    buf: torch.Tensor            # uint8 [qam_packed_bytes(N, K)]
    desc: L.QamPacked

    @property
    def N(self) -> int:
        return int(self.desc.N)

    @property
    def K(self) -> int:
        return int(self.desc.K)

    @property
    def n_blocks(self) -> int:
        return int(self.desc.n_blocks)


def packed_bytes(N: int, K: int) -> int:
    return int(L.lib().qam_packed_bytes(N, K))


def pack_slices(W: torch.Tensor, scales: torch.Tensor, out: Optional[torch.Tensor] = None) -> PackedMatrix:
    """Split int8 codes W [N, K] and fp32 scales [N] into the slice-major packed layout."""
    _require_cuda(W, "W", torch.int8)
    _require_cuda(scales, "scales", torch.float32)
    N, K = W.shape
    nbytes = packed_bytes(N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    desc = L.QamPacked()
    L.check(L.lib().qam_pack_slices(_ptr(W), _ptr(scales), N, K, _ptr(out), out.numel(), C.byref(desc),
                                     _stream_handle()))
    return PackedMatrix(out, desc)


def unpack_codes(packed: PackedMatrix, level_map: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Debug probe: int8 [N, K] codes as the product kernels read them at the map's depths."""
    _require_cuda(level_map, "level_map", torch.uint8)
    if out is None:
        out = torch.empty((packed.N, packed.K), dtype=torch.int8, device=packed.buf.device)
    L.check(L.lib().qam_unpack_codes(C.byref(packed.desc), _ptr(level_map), _ptr(out), _stream_handle()))
    return out


def _fspath(path) -> bytes:
    return os.fsencode(os.fspath(path))


def stack_write(path, mats: Sequence[PackedMatrix], names: Optional[Sequence[Optional[str]]] = None) -> None:
    """Write packed matrices to a stack file (plane-major: a read at depth d
    is the first d/2 plane sections plus the scales)."""
    n = len(mats)
    descs = (L.QamPacked * n)(*[m.desc for m in mats])
    cnames = None
    if names is not None:
        if len(names) != n:
            raise ValueError("one name per matrix")
        cnames = (C.c_char_p * n)(*[None if v is None else v.encode() for v in names])
    L.check(L.lib().qam_stack_write(_fspath(path), descs, cnames, n, _stream_handle()))


def stack_info(path):
    """(header, entries) of a stack file, as ctypes structures."""
    hdr = L.QamStackHeader()
    L.check(L.lib().qam_stack_info(_fspath(path), C.byref(hdr), None, 0))
    n = int(hdr.n_matrices)
    ents = (L.QamStackEntry * n)()
    L.check(L.lib().qam_stack_info(_fspath(path), C.byref(hdr), ents, n))
    return hdr, list(ents)


def stack_read(path, bits: int, first: int = 0, count: Optional[int] = None, device=None,
               out: Optional[Sequence[PackedMatrix]] = None):
    """Load matrices [first, first + count) at ``bits`` (2, 4, 6 or 8) into
    device buffers (new ones, or ``out``); planes below that depth are zero.
    Returns (list of PackedMatrix, bytes read from the file)."""
    if bits not in (2, 4, 6, 8):
        raise ValueError("bits must be 2, 4, 6 or 8")
    hdr, ents = stack_info(path)
    if count is None:
        count = len(ents) - first
    if out is None:
        dev = torch.device("cuda") if device is None else torch.device(device)
        out = []
        for e in ents[first:first + count]:
            buf = torch.empty(packed_bytes(e.N, e.K), dtype=torch.uint8, device=dev)
            d = L.QamPacked()
            L.check(L.lib().qam_describe_packed(_ptr(buf), e.N, e.K, C.byref(d)))
            out.append(PackedMatrix(buf, d))
    if len(out) != count:
        raise ValueError(f"out holds {len(out)} matrices, {count} requested")
    descs = (L.QamPacked * count)(*[m.desc for m in out])
    nread = C.c_uint64(0)
    L.check(L.lib().qam_stack_read(_fspath(path), bits // 2, first, count, descs, _stream_handle(),
                                    C.byref(nread)))
    return list(out), int(nread.value)


class LensRules:
    """One map's lens-rule arguments, marshalled once for the C ABI:
    ``centres`` [n_lenses, 2] and ``radii`` [n_lenses] (host sequences), the
    focus area ``f`` and strength ``g``, ``combine`` ('sum' or 'max'), the
    ``glass`` rung, optional explicit ``stops`` and the ladder.  ``radius``
    is "lens" (R_i = r_i f / (1 - f)) or "zone" (R = f width for every lens,
    ``width`` the field's, e.g. from ``field_width``)."""

    def __init__(self, centres, radii, f: float, g: float, combine: str = "sum", glass: int = 1, stops=None,
                 ladder_bits: Sequence[int] = LADDER_BITS, radius: str = "lens", width: float = 0.0):
        centres = np.asarray(centres, dtype=np.float64).reshape(-1, 2)
        radii = np.asarray(radii, dtype=np.float64).reshape(-1)
        if centres.shape[0] != radii.shape[0]:
            raise ValueError("centres and radii disagree on the lens count")
        self.n_lenses = centres.shape[0]
        self.lenses = (L.QamLens * max(1, self.n_lenses))()
        for i in range(self.n_lenses):
            self.lenses[i].cx, self.lenses[i].cy = float(centres[i, 0]), float(centres[i, 1])
            self.lenses[i].r = float(radii[i])
        p = L.QamLensParams()
        p.f, p.g = float(f), float(g)
        p.combine = {"sum": L.QAM_COMBINE_SUM, "max": L.QAM_COMBINE_MAX}[combine]
        if stops is None:
            p.n_stops = 0
        else:
            st = np.asarray(stops, dtype=np.float64).reshape(-1)
            p.n_stops = int(st.shape[0])
            if p.n_stops > L.QAM_MAX_STOPS:
                raise ValueError("too many stops")
            for j, v in enumerate(st):
                p.stops[j] = float(v)
        p.radius_mode = {"lens": L.QAM_RADIUS_LENS, "zone": L.QAM_RADIUS_ZONE}[radius]
        p.width = float(width)
        self.params = p
        self.n_rungs = len(ladder_bits)
        self.ladder = (C.c_uint8 * self.n_rungs)(*ladder_bits)
        self.glass = int(glass)


def build_level_map(coords: torch.Tensor, centres, radii, f: float, g: float, combine: str = "sum",
                    glass: int = 1, ladder_bits: Sequence[int] = LADDER_BITS, stops=None,
                    out: Optional[torch.Tensor] = None, rules: Optional[LensRules] = None,
                    radius: str = "lens", width: float = 0.0) -> torch.Tensor:
    """Per-block rung indices (uint8 [n_blocks]) from the lens rules, on the
    product's ladder {0, 2, 4, 6, 8} (a rung index is the slices qmatvec reads).

    ``coords`` is a device fp64 [n_blocks, 2] tensor; ``centres`` [n_lenses, 2]
    and ``radii`` [n_lenses] are host sequences (or pass ``rules``, a
    LensRules, with centres = radii = None)."""
    return _build_map(coords, centres, radii, f, g, combine, glass, ladder_bits, stops, out, rules, radius, width,
                      "qam_build_level_map")


def build_rung_map(coords: torch.Tensor, centres, radii, f: float, g: float, combine: str = "sum",
                   glass: int = 1, ladder_bits: Sequence[int] = LADDER_BITS, stops=None,
                   out: Optional[torch.Tensor] = None, rules: Optional[LensRules] = None,
                   radius: str = "lens", width: float = 0.0) -> torch.Tensor:
    """The same rules on any ladder (rung indices of ``ladder_bits``, not read
    depths of qmatvec unless the ladder is {0, 2, 4, 6, 8})."""
    return _build_map(coords, centres, radii, f, g, combine, glass, ladder_bits, stops, out, rules, radius, width,
                      "qam_build_rung_map")


def _build_map(coords, centres, radii, f, g, combine, glass, ladder_bits, stops, out, rules, radius, width, fn):
    _require_cuda(coords, "coords", torch.float64)
    n_blocks = coords.shape[0]
    r = rules if rules is not None else LensRules(centres, radii, f, g, combine, glass, stops, ladder_bits, radius,
                                                  width)
    if out is None:
        out = torch.empty(n_blocks, dtype=torch.uint8, device=coords.device)
    L.check(getattr(L.lib(), fn)(_ptr(coords), n_blocks, r.lenses, r.n_lenses, C.byref(r.params),
                                 C.cast(r.ladder, C.c_void_p), r.n_rungs, r.glass, _ptr(out), _stream_handle()))
    return out


def field_width(coords: torch.Tensor) -> float:
    """The width D of a block field (its largest distance between two
    blocks), computed on the device; the zone radius is R = f D."""
    _require_cuda(coords, "coords", torch.float64)
    ws = torch.zeros(256, dtype=torch.uint8, device=coords.device)
    d = C.c_double()
    L.check(L.lib().qam_field_width(_ptr(coords), coords.shape[0], _ptr(ws), 256, C.byref(d), _stream_handle()))
    return d.value


def status(mem: torch.Tensor, clear: bool = True) -> int:
    """The status word (QAM_STATUS_* bits) of a workspace or of a group's or a
    decoder's device memory; 0 when every launch ran as documented."""
    out = C.c_uint32()
    L.check(L.lib().qam_status(_ptr(mem), int(bool(clear)), C.byref(out), _stream_handle()))
    return int(out.value)


def fit_focus_area(coords: torch.Tensor, block_weights: torch.Tensor, centres, radii, g: float, budget_bytes: int,
                   combine: str = "sum", glass: int = 1, iters: int = 40, stops=None,
                   ladder_bits: Sequence[int] = LADDER_BITS, out: Optional[torch.Tensor] = None,
                   radius: str = "lens", width: float = 0.0):
    """The byte-budget regulator: the largest focus area f whose lens map
    reads at most ``budget_bytes`` of weights (bisection, ``iters`` halvings).
    ``block_weights`` is a device int64 [n_blocks] tensor of w_b.  Returns
    (f, bytes, level map uint8 [n_blocks] at f)."""
    _require_cuda(coords, "coords", torch.float64)
    _require_cuda(block_weights, "block_weights", torch.int64)
    n_blocks = coords.shape[0]
    if block_weights.numel() != n_blocks:
        raise ValueError("one weight per block")
    r = LensRules(centres, radii, 0.0, g, combine, glass, stops, ladder_bits, radius, width)
    if out is None:
        out = torch.empty(n_blocks, dtype=torch.uint8, device=coords.device)
    ws = torch.zeros(256, dtype=torch.uint8, device=coords.device)
    f, b = C.c_double(), C.c_int64()
    L.check(L.lib().qam_fit_focus_area(_ptr(coords), n_blocks, _ptr(block_weights), r.lenses, r.n_lenses,
                                       C.byref(r.params), C.cast(r.ladder, C.c_void_p), r.n_rungs, r.glass,
                                       int(budget_bytes), int(iters), _ptr(out), _ptr(ws), 256, C.byref(f),
                                       C.byref(b), _stream_handle()))
    return f.value, b.value, out


class LensSets:
    """The lens-rule arguments of one map per request, marshalled once for the
    C ABI: ``lens_sets`` is a sequence of (centres [n_lenses, 2], radii
    [n_lenses]) pairs, all with the same lens count; ``f`` a scalar or one
    value per map."""

    def __init__(self, lens_sets, f, g: float = 1.0, combine: str = "sum", glass: int = 1,
                 ladder_bits: Sequence[int] = LADDER_BITS):
        self.n_maps = len(lens_sets)
        fs = np.broadcast_to(np.asarray(f, dtype=np.float64), (self.n_maps,))
        self.n_lenses = None
        self.lenses = None
        self.params = (L.QamLensParams * self.n_maps)()
        for k, (centres, radii) in enumerate(lens_sets):
            centres = np.asarray(centres, dtype=np.float64).reshape(-1, 2)
            radii = np.asarray(radii, dtype=np.float64).reshape(-1)
            if centres.shape[0] != radii.shape[0]:
                raise ValueError("centres and radii disagree on the lens count")
            if self.n_lenses is None:
                self.n_lenses = centres.shape[0]
                self.lenses = (L.QamLens * max(1, self.n_maps * self.n_lenses))()
            elif centres.shape[0] != self.n_lenses:
                raise ValueError("every map needs the same lens count")
            for i in range(self.n_lenses):
                lens = self.lenses[k * self.n_lenses + i]
                lens.cx, lens.cy, lens.r = float(centres[i, 0]), float(centres[i, 1]), float(radii[i])
            self.params[k].f, self.params[k].g = float(fs[k]), float(g)
            self.params[k].combine = {"sum": L.QAM_COMBINE_SUM, "max": L.QAM_COMBINE_MAX}[combine]
            self.params[k].n_stops = 0
        self.n_rungs = len(ladder_bits)
        self.ladder = (C.c_uint8 * self.n_rungs)(*ladder_bits)
        self.glass = int(glass)


def build_level_maps(coords: torch.Tensor, lens_sets=None, f=None, g: float = 1.0, combine: str = "sum",
                     glass: int = 1, ladder_bits: Sequence[int] = LADDER_BITS, out: Optional[torch.Tensor] = None,
                     sets: Optional[LensSets] = None) -> torch.Tensor:
    """One map per request (uint8 [n_maps, n_blocks]) from ``lens_sets`` and
    ``f`` as LensSets takes them, or from ``sets``, a LensSets."""
    _require_cuda(coords, "coords", torch.float64)
    n_blocks = coords.shape[0]
    st = sets if sets is not None else LensSets(lens_sets, f, g, combine, glass, ladder_bits)
    if out is None:
        out = torch.empty((st.n_maps, n_blocks), dtype=torch.uint8, device=coords.device)
    else:
        _require_cuda(out, "out", torch.uint8)
    L.check(L.lib().qam_build_level_maps(_ptr(coords), n_blocks, st.lenses, st.n_lenses, st.params,
                                         C.cast(st.ladder, C.c_void_p), st.n_rungs, st.glass, st.n_maps, _ptr(out),
                                         _stream_handle()))
    return out


def map_weight_bytes(level_map, K: int, ladder_bits: Sequence[int] = LADDER_BITS):
    """(mean bits, weight bytes) of a map over one matrix with K columns (host)."""
    lv = np.ascontiguousarray(np.asarray(level_map.cpu() if isinstance(level_map, torch.Tensor) else level_map,
                                         dtype=np.uint8))
    ladder = (C.c_uint8 * len(ladder_bits))(*ladder_bits)
    mb, wb = C.c_double(), C.c_int64()
    L.check(L.lib().qam_map_weight_bytes(lv.ctypes.data_as(C.c_void_p), lv.shape[0], K, C.cast(ladder, C.c_void_p),
                                         len(ladder_bits), C.byref(mb), C.byref(wb)))
    return mb.value, wb.value


def workspace_bytes(N: int, K: int, B: int = 1) -> int:
    return int(L.lib().qam_qmatvec_workspace_bytes(N, K, B))


class Workspace:
    """A device scratch buffer that grows on demand (new storage is zero-filled).
    libqam keeps its leading counter region zero after every call, so one
    buffer serves calls of any shape on a stream."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = torch.zeros(0, dtype=torch.uint8, device=self.device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 2 * self.buf.numel()), dtype=torch.uint8, device=self.device)
        return self.buf


_WS = {}


def default_workspace(device) -> Workspace:
    key = torch.device(device)
    if key not in _WS:
        _WS[key] = Workspace(key)
    return _WS[key]


_OUT_MODES = {"store": L.QAM_OUT_STORE, "add": L.QAM_OUT_ADD, "glu": L.QAM_OUT_GLU}


def qmatvec(x: torch.Tensor, packed: PackedMatrix, level_map: torch.Tensor, y: Optional[torch.Tensor] = None,
            workspace: Optional[Workspace] = None, rms_norm: bool = False, out_mode: str = "store",
            eps: float = 1e-6) -> torch.Tensor:
    """y fp32 = the mixed-depth product of x [B, K] (fp32 or bf16) with the packed matrix.

    ``level_map`` is uint8 [n_blocks] (shared by the B requests) or
    [B, n_blocks] (one map per request).  ``rms_norm`` multiplies in
    1 / sqrt(mean(x^2) + eps); ``out_mode`` is "store" (y [B, N]), "add"
    (y += product, y given) or "glu" (gate/up rows interleaved 32/32 per
    block, y [B, N/2] = silu(gate) * up); the last two and ``rms_norm`` take
    one request (B = 1)."""
    _require_cuda(level_map, "level_map", torch.uint8)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    _require_cuda(x, "x")
    if x.dtype == torch.float32:
        xdt = L.QAM_X_F32
    elif x.dtype == torch.bfloat16:
        xdt = L.QAM_X_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    B, K = x.shape
    if K != packed.K:
        raise ValueError(f"x has {K} columns, matrix has {packed.K}")
    per_request = level_map.dim() == 2
    if per_request:
        if tuple(level_map.shape) != (B, packed.n_blocks):
            raise ValueError("a per-request level_map must be [B, n_blocks]")
    elif level_map.numel() != packed.n_blocks:
        raise ValueError("level_map must have one entry per block")
    mode = _OUT_MODES[out_mode]
    n_out = packed.N // 2 if mode == L.QAM_OUT_GLU else packed.N
    if y is None:
        if mode == L.QAM_OUT_ADD:
            raise ValueError("out_mode 'add' needs y")
        y = torch.empty((B, n_out), dtype=torch.float32, device=x.device)
    else:
        _require_cuda(y, "y", torch.float32)
        if y.numel() != B * n_out:
            raise ValueError(f"y must hold {B} x {n_out} values")
    ws = workspace or default_workspace(x.device)
    need = workspace_bytes(packed.N, packed.K, B)
    if need == 0:
        raise L.QamError(-2, f"no workspace size for N={packed.N} K={packed.K} B={B}")
    wbuf = ws.get(need)
    if rms_norm or mode != L.QAM_OUT_STORE:
        if per_request:
            raise ValueError("fused epilogues take a shared level map")
        ep = L.QamEpilogue(int(bool(rms_norm)), mode, float(eps))
        L.check(L.lib().qam_qmatvec_ep(_ptr(x), xdt, B, C.byref(packed.desc), _ptr(level_map), C.byref(ep), _ptr(y),
                                       _ptr(wbuf), wbuf.numel(), _stream_handle()))
    else:
        L.check(L.lib().qam_qmatvec(_ptr(x), xdt, B, C.byref(packed.desc), _ptr(level_map), int(per_request),
                                    _ptr(y), _ptr(wbuf), wbuf.numel(), _stream_handle()))
    return y


def qmatvec_noalloc(x: torch.Tensor, packed: PackedMatrix, level_map: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """``qmatvec`` (plain store, no epilogue) through the library's static
    per-GPU scratch: the call allocates no device memory, so ``y`` must be
    given.  Shapes whose workspace exceeds QAM_SCRATCH_BYTES are rejected;
    calls that overlap on one GPU share the scratch and race."""
    _require_cuda(level_map, "level_map", torch.uint8)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    _require_cuda(x, "x")
    if x.dtype == torch.float32:
        xdt = L.QAM_X_F32
    elif x.dtype == torch.bfloat16:
        xdt = L.QAM_X_BF16
    else:
        raise TypeError("x must be float32 or bfloat16")
    B, K = x.shape
    if K != packed.K:
        raise ValueError(f"x has {K} columns, matrix has {packed.K}")
    per_request = level_map.dim() == 2
    if per_request:
        if tuple(level_map.shape) != (B, packed.n_blocks):
            raise ValueError("a per-request level_map must be [B, n_blocks]")
    elif level_map.numel() != packed.n_blocks:
        raise ValueError("level_map must have one entry per block")
    _require_cuda(y, "y", torch.float32)
    if y.numel() != B * packed.N:
        raise ValueError(f"y must hold {B} x {packed.N} values")
    L.check(L.lib().qam_qmatvec_noalloc(_ptr(x), xdt, B, C.byref(packed.desc), _ptr(level_map), int(per_request),
                                        _ptr(y), _stream_handle()))
    return y


class GroupedQmatvec:
    """Many matrices with their own x, y and level map, one launch per call
    (two on the pre-pass route).

    ``items`` is a sequence of (PackedMatrix, x [B, K], y [B, N], level_map)
    tuples, the maps all [n_blocks] (shared by the B requests) or all
    [B, n_blocks] (per request); the tensors are bound once (keep them alive
    and update them in place), and every ``run()`` recomputes all the y from
    the bound buffers.  A fifth element, the item's block coordinates (device
    fp64 [n_blocks, 2]), lets ``run_lens`` build the maps in the product
    launch (one request).  ``tuning`` (a dict of qam_tuning fields) sets the
    group's launch plan; the results do not depend on it."""

    def __init__(self, items, device="cuda", tuning: Optional[dict] = None):
        n = len(items)
        arr = (L.QamGemvItem * n)()
        B = None
        xdt = None
        per_request = None
        self._keep = []
        for i, item in enumerate(items):
            pm, x, y, lv = item[:4]
            cd = item[4] if len(item) > 4 else None
            _require_cuda(x, "x")
            _require_cuda(y, "y", torch.float32)
            if not isinstance(lv, torch.Tensor) or not lv.is_cuda or lv.dtype != torch.uint8:
                raise TypeError("level_map must be a uint8 device tensor")
            b = x.shape[0] if x.dim() == 2 else 1
            d = L.QAM_X_F32 if x.dtype == torch.float32 else (L.QAM_X_BF16 if x.dtype == torch.bfloat16 else None)
            if d is None:
                raise TypeError("x must be float32 or bfloat16")
            pr = lv.dim() == 2
            if B is None:
                B, xdt, per_request = b, d, pr
            elif (b, d, pr) != (B, xdt, per_request):
                raise ValueError("every item of a group needs the same batch, x dtype and map kind")
            stride = 0
            if pr:
                # [B, n_blocks], possibly a column slice of a [B, field blocks] array
                if tuple(lv.shape) != (B, pm.n_blocks) or lv.stride(1) != 1:
                    raise ValueError("a per-request level_map must be [B, n_blocks] with unit column stride")
                stride = lv.stride(0)
            else:
                _require_cuda(lv, "level_map")
            arr[i].w = pm.desc
            arr[i].x, arr[i].y, arr[i].level_map = x.data_ptr(), y.data_ptr(), lv.data_ptr()
            arr[i].level_stride = stride
            if cd is not None:
                _require_cuda(cd, "coords", torch.float64)
                if tuple(cd.shape) != (pm.n_blocks, 2) or cd.stride() != (2, 1):
                    raise ValueError("coords must be a contiguous fp64 [n_blocks, 2] tensor")
                arr[i].coords = cd.data_ptr()
            self._keep.append((pm, x, y, lv, cd))
        tun = L.QamTuning()
        for k, v in (tuning or {}).items():
            setattr(tun, k, int(v))
        nbytes = int(L.lib().qam_group_bytes_tuned(arr, n, B, int(per_request), C.byref(tun)))
        if nbytes == 0:
            raise L.QamError(-2, "invalid group items or tuning")
        self.mem = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.desc = L.QamGroup()
        L.check(L.lib().qam_group_init_tuned(arr, n, B, xdt, int(per_request), C.byref(tun), _ptr(self.mem), nbytes,
                                             C.byref(self.desc), _stream_handle()))

    def status(self, clear: bool = True) -> int:
        """The group's status word (QAM_STATUS_* bits, 0 if all is well)."""
        return status(self.mem, clear)

    @property
    def route(self) -> str:
        """"staged" (limbs staged inside the product kernel) or "prepass" (a limb pre-pass, then the product)."""
        return "prepass" if self.desc.route == 1 else "staged"

    def run(self) -> None:
        L.check(L.lib().qam_qmatvec_group(C.byref(self.desc), _stream_handle()))

    def run_lens(self, rules: LensRules) -> None:
        """One launch: every item's level map from ``rules`` (a LensRules) over
        its bound coordinates, written to its level_map, and its product."""
        L.check(L.lib().qam_qmatvec_group_lens(C.byref(self.desc), rules.lenses, rules.n_lenses,
                                               C.byref(rules.params), C.cast(rules.ladder, C.c_void_p),
                                               rules.n_rungs, rules.glass, _stream_handle()))


class LayerRule:
    """The rule by which a layer sets its blocks' rungs from its own base read
    (libqam's ``qam_layer_levels``): ``lam`` for the lambda 16^j thresholds
    or ``share`` for the top share, exactly one of them; ``g`` the focus
    strength (ceiling), ``glass`` the base rung, ``n_rungs`` the ladder
    length."""

    def __init__(self, lam: Optional[float] = None, share: Optional[float] = None, g: float = 1.0, glass: int = 1,
                 n_rungs: int = len(LADDER_BITS)):
        if (lam is None) == (share is None):
            raise ValueError("give exactly one of lam and share")
        r = L.QamLayerRule()
        r.mode = L.QAM_LAYER_THRESHOLD if share is None else L.QAM_LAYER_SHARE
        r.lam = float(lam) if lam is not None else 0.0
        r.share = float(share) if share is not None else 0.0
        r.g = float(g)
        self.rule = r
        self.glass = int(glass)
        self.n_rungs = int(n_rungs)


def layer_levels(y_base: torch.Tensor, packed: PackedMatrix, rule: LayerRule, shat: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None):
    """Per-request level maps uint8 [B, n_blocks] and the reduced scores fp64
    [B, n_blocks] from the product at the base depth ``y_base`` fp32 [B, N]."""
    _require_cuda(y_base, "y_base", torch.float32)
    if y_base.dim() == 1:
        y_base = y_base.unsqueeze(0)
    B, N = y_base.shape
    if N != packed.N:
        raise ValueError(f"y_base has {N} columns, the matrix {packed.N} rows")
    nb = packed.n_blocks
    if shat is None:
        shat = torch.empty((B, nb), dtype=torch.float64, device=y_base.device)
    if out is None:
        out = torch.empty((B, nb), dtype=torch.uint8, device=y_base.device)
    _require_cuda(shat, "shat", torch.float64)
    _require_cuda(out, "out", torch.uint8)
    if shat.numel() != B * nb or out.numel() != B * nb:
        raise ValueError("shat and out must hold B x n_blocks values")
    L.check(L.lib().qam_layer_levels(_ptr(y_base), B, C.byref(packed.desc), C.byref(rule.rule), rule.n_rungs,
                                     rule.glass, _ptr(shat), _ptr(out), _stream_handle()))
    return out, shat


class LayerDecides:
    """One layer that decides its own depths: the product at the base rung
    (a uniform map), the scores and levels on the device, then the product
    at those levels (a map per request; one shared map at B = 1).  Buffers
    are allocated once; ``run(x)`` returns y fp32 [B, N]."""

    def __init__(self, packed: PackedMatrix, B: int, rule: LayerRule, device="cuda"):
        self.packed, self.B, self.rule = packed, int(B), rule
        nb = packed.n_blocks
        self.base_map = torch.full((nb,), rule.glass, dtype=torch.uint8, device=device)
        self.y_base = torch.empty((self.B, packed.N), dtype=torch.float32, device=device)
        self.y = torch.empty((self.B, packed.N), dtype=torch.float32, device=device)
        self.shat = torch.empty((self.B, nb), dtype=torch.float64, device=device)
        self.levels = torch.empty((self.B, nb), dtype=torch.uint8, device=device)

    def run(self, x: torch.Tensor) -> torch.Tensor:
        qmatvec(x, self.packed, self.base_map, y=self.y_base)
        layer_levels(self.y_base, self.packed, self.rule, shat=self.shat, out=self.levels)
        qmatvec(x, self.packed, self.levels[0] if self.B == 1 else self.levels, y=self.y)
        return self.y


class LayerDecidesGroup:
    """Several matrices that decide their own depths, grouped: one grouped
    product at the glass (a uniform map), the scores and levels of each
    matrix on the device, one grouped product at those maps (per request;
    shared at B = 1).  ``items`` are (PackedMatrix, x [B, K], y [B, N])
    tuples, bound once like GroupedQmatvec's; ``run()`` recomputes every y,
    ``levels[i]`` holds matrix i's maps [B, n_blocks] afterwards.  Up to 16
    matrices of at most 512 blocks each share one level launch.  With
    ``refine`` (taken where the second product runs on the pre-pass route,
    from 2 requests, and the glass is D2-D6), the base product is written
    into y and the second product only adds the lifted blocks' slices above
    the glass (``qam_qmatvec_group_refine``): every block is read once to
    the glass and the lifted ones on from there; ``self.refine`` says which
    form runs."""

    def __init__(self, items, rule: LayerRule, device="cuda", refine: bool = True):
        self.rule = rule
        B0 = items[0][1].shape[0] if items[0][1].dim() == 2 else 1
        refine = bool(refine) and B0 >= 2 and 1 <= rule.glass <= 3 and rule.n_rungs == len(LADDER_BITS)
        base_items, second_items, self.parts = [], [], []
        for pm, x, y in items:
            B = x.shape[0] if x.dim() == 2 else 1
            nb = pm.n_blocks
            base_map = torch.full((nb,), rule.glass, dtype=torch.uint8, device=device)
            y_base = y if refine else torch.empty((B, pm.N), dtype=torch.float32, device=device)
            shat = torch.empty((B, nb), dtype=torch.float64, device=device)
            lv = torch.empty((B, nb), dtype=torch.uint8, device=device)
            base_items.append((pm, x, y_base, base_map))
            second_items.append((pm, x, y, lv[0] if B == 1 else lv))
            self.parts.append((pm, y_base, shat, lv))
        self.base = GroupedQmatvec(base_items, device=device)
        self.second = GroupedQmatvec(second_items, device=device)
        # at one request (the staged route) the second product is a full one
        # at the maps, which overwrites y
        self.refine = refine and self.second.route == "prepass"
        self.levels = [p[3] for p in self.parts]
        # one launch for every matrix when each has at most 512 blocks
        self._table = None
        n = len(self.parts)
        if n <= L.QAM_LAYER_GROUP_MAX and all(p[0].n_blocks <= 512 for p in self.parts):
            self._table = (L.QamLayerItem * n)()
            for i, (pm, y_base, shat, lv) in enumerate(self.parts):
                self._table[i].y_base, self._table[i].w = y_base.data_ptr(), pm.desc
                self._table[i].shat_out, self._table[i].level_out = shat.data_ptr(), lv.data_ptr()
            self._B = self.parts[0][1].shape[0]

    def decide(self) -> None:
        """The scores and levels from the base outputs of the last run."""
        if self._table is not None:
            L.check(L.lib().qam_layer_levels_group(self._table, len(self.parts), self._B, C.byref(self.rule.rule),
                                                   self.rule.n_rungs, self.rule.glass, _stream_handle()))
            return
        for pm, y_base, shat, lv in self.parts:
            layer_levels(y_base, pm, self.rule, shat=shat, out=lv)

    def refine_run(self) -> None:
        """The lifted blocks' slices above the glass, added to y."""
        L.check(L.lib().qam_qmatvec_group_refine(C.byref(self.second.desc), self.rule.glass, _stream_handle()))

    def run(self) -> None:
        self.base.run()
        self.decide()
        if self.refine:
            self.refine_run()
        else:
            self.second.run()


class Gate:
    """The escalation gate on the device: softmax entropy (nats) and top-two
    margin of a logits vector of length ``V``, and the decision
    entropy > tau_entropy or margin < tau_margin; one launch per ``run``.
    ``result()`` copies the outcome to the host (a synchronisation)."""

    def __init__(self, V: int, device="cuda"):
        n = int(L.lib().qam_gate_workspace_bytes(int(V)))
        if n == 0:
            raise ValueError("the gate needs at least two logits")
        self.V = int(V)
        self.ws = torch.zeros(n, dtype=torch.uint8, device=device)
        self.out = torch.zeros(C.sizeof(L.QamUncertainty), dtype=torch.uint8, device=device)
        self._host = torch.empty(C.sizeof(L.QamUncertainty), dtype=torch.uint8, pin_memory=True)

    def run(self, logits: torch.Tensor, tau_entropy: float = float("inf"),
            tau_margin: float = float("-inf")) -> None:
        _require_cuda(logits, "logits", torch.float32)
        if logits.numel() != self.V:
            raise ValueError(f"logits must hold {self.V} values")
        L.check(L.lib().qam_gate(_ptr(logits), self.V, float(tau_entropy), float(tau_margin), _ptr(self.out),
                                 _ptr(self.ws), self.ws.numel(), _stream_handle()))

    def result(self) -> dict:
        self._host.copy_(self.out, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        u = L.QamUncertainty.from_buffer_copy(self._host.numpy().tobytes())
        return dict(entropy=u.entropy, margin=u.margin, p1=u.p1, p2=u.p2, top1=int(u.top1), top2=int(u.top2),
                    escalate=bool(u.escalate))


class Decoder:
    """A decode step as a chain of fused mixed-depth products (libqam's decoder).

    ``layers`` is a sequence of (qkv, o, gate_up, down) PackedMatrix tuples
    (gate_up rows interleaved 32 gate / 32 up per 64-row block) and
    ``lm_head`` a PackedMatrix.  Write the step input into ``hidden`` and call
    ``step(rung)`` (eager) or ``capture(rung)`` once and ``replay(rung)``."""

    def __init__(self, layers, lm_head: PackedMatrix, hidden: int, q_dim: int, kv_dim: int, ffn: int,
                 eps: float = 1e-6, target_waves: int = 0, waves_per_block: int = 0, max_chunk_tiles: int = 0,
                 device="cuda"):
        n = len(layers)
        self._layers = (L.QamDecoderLayer * n)()
        self._keep = [lm_head]
        for i, (qkv, o, gu, down) in enumerate(layers):
            self._layers[i].qkv, self._layers[i].o = qkv.desc, o.desc
            self._layers[i].gate_up, self._layers[i].down = gu.desc, down.desc
            self._keep.append((qkv, o, gu, down))
        d = L.QamDecoderDesc()
        d.n_layers, d.hidden, d.q_dim, d.kv_dim, d.ffn, d.vocab = n, hidden, q_dim, kv_dim, ffn, lm_head.N
        d.layers = self._layers
        d.lm_head = lm_head.desc
        d.eps = float(eps)
        d.target_waves = int(target_waves)
        d.waves_per_block = int(waves_per_block)
        d.max_chunk_tiles = int(max_chunk_tiles)
        self._desc = d
        nbytes = int(L.lib().qam_decoder_bytes(C.byref(d)))
        if nbytes == 0:
            raise L.QamError(-2, "invalid decoder description")
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = C.c_void_p()
        L.check(L.lib().qam_decoder_create(C.byref(d), _ptr(self.mem), nbytes, C.byref(h), _stream_handle()))
        self._h = h
        self._destroy = L.lib().qam_decoder_destroy   # held here: module globals may be gone at interpreter exit
        self.n_layers = n
        self.n_ops = 4 * n + 1
        self.hidden = self._buffer(0, hidden)
        self.qkv = self._buffer(1, q_dim + 2 * kv_dim)
        self.m = self._buffer(2, ffn)
        self.logits = self._buffer(3, lm_head.N)
        self._capture_stream = None

    def _buffer(self, which: int, n: int) -> torch.Tensor:
        off = L.lib().qam_decoder_buffer(self._h, which) - self.mem.data_ptr()
        return self.mem[off:off + 4 * n].view(torch.float32)

    def run(self, rung: int, first: int, count: int = 1) -> None:
        """Enqueue products first .. first+count-1 of the step's chain."""
        L.check(L.lib().qam_decoder_run(self._h, int(rung), int(first), int(count), _stream_handle()))

    def step(self, rung: int) -> None:
        L.check(L.lib().qam_decoder_step(self._h, int(rung), _stream_handle()))

    def capture(self, rung: int) -> None:
        if self._capture_stream is None:
            self._capture_stream = torch.cuda.Stream(device=self.mem.device)
        s = self._capture_stream
        s.wait_stream(torch.cuda.current_stream())
        L.check(L.lib().qam_decoder_capture(self._h, int(rung), C.c_void_p(s.cuda_stream)))
        torch.cuda.current_stream().wait_stream(s)

    def replay(self, rung: int) -> None:
        L.check(L.lib().qam_decoder_replay(self._h, int(rung), _stream_handle()))

    def decode_gated(self, inputs: torch.Tensor, gate: "Gate", tau_entropy: float = float("inf"),
                     tau_margin: float = float("-inf"), rung_low: int = 2, rung_high: int = 4) -> np.ndarray:
        """T steps (inputs [T, hidden] fp32 on the device) with the escalation
        gate decided on the device each step, looped inside the library; both
        rungs must be captured.  Returns uint8 [T], 1 where a step was redone
        at ``rung_high``."""
        _require_cuda(inputs, "inputs", torch.float32)
        T = inputs.shape[0]
        if inputs.dim() != 2 or inputs.shape[1] != self.hidden.numel():
            raise ValueError("inputs must be [T, hidden]")
        if gate.V != self.logits.numel():
            raise ValueError("the gate must take the vocabulary's logits")
        esc = np.zeros(T, dtype=np.uint8)
        L.check(L.lib().qam_decoder_decode_gated(
            self._h, _ptr(inputs), T, int(rung_low), int(rung_high), float(tau_entropy), float(tau_margin),
            _ptr(gate.ws), gate.ws.numel(), _ptr(gate.out), C.c_void_p(gate._host.data_ptr()),
            esc.ctypes.data_as(C.c_void_p), _stream_handle()))
        return esc

    def decode_gated_async(self, inputs: torch.Tensor, gate: "Gate", tau_entropy: float = float("inf"),
                           tau_margin: float = float("-inf"), rung_low: int = 2, rung_high: int = 4,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The gated steps with the decision kept on the device (predicated
        high-rung graph, no per-step synchronisation); ``rung_low`` must be
        captured.  Returns uint8 [T] on the device (ready when the stream is)."""
        _require_cuda(inputs, "inputs", torch.float32)
        T = inputs.shape[0]
        if inputs.dim() != 2 or inputs.shape[1] != self.hidden.numel():
            raise ValueError("inputs must be [T, hidden]")
        if gate.V != self.logits.numel():
            raise ValueError("the gate must take the vocabulary's logits")
        if out is None:
            out = torch.zeros(max(1, T), dtype=torch.uint8, device=self.mem.device)
        s = torch.cuda.current_stream()
        if s.cuda_stream == 0:
            raise ValueError("decode_gated_async needs a stream other than the null stream")
        L.check(L.lib().qam_decoder_decode_gated_async(
            self._h, _ptr(inputs), T, int(rung_low), int(rung_high), float(tau_entropy), float(tau_margin),
            _ptr(gate.ws), gate.ws.numel(), _ptr(gate.out), _ptr(out), C.c_void_p(s.cuda_stream)))
        return out[:T]

    def status(self, clear: bool = True) -> int:
        """The decoder's status word (QAM_STATUS_* bits, 0 if all is well)."""
        return status(self.mem, clear)

    def __del__(self):
        h, destroy = getattr(self, "_h", None), getattr(self, "_destroy", None)
        self._h = None
        if h is not None and h.value and callable(destroy):
            destroy(h)


class Verifier:
    """Batched decode steps over a Decoder's weights (the verify pass of
    draft-and-verify).  Write B inputs into ``x[:B]`` and call
    ``step(rung, B)``; ``logits[:B]`` holds the result.  ``run`` enqueues
    single ops of the chain (op 0 loads the inputs, then qkv, o, gate_up,
    down per layer, then the head; each op forms its product's input from
    the previous op's output: residual add and norm, the q columns, the
    gated product)."""

    def __init__(self, dec: Decoder, max_batch: int):
        nbytes = int(L.lib().qam_verifier_bytes(C.byref(dec._desc), int(max_batch)))
        if nbytes == 0:
            raise L.QamError(-3, f"no verifier for max_batch={max_batch}")
        self.dec = dec
        self.max_batch = int(max_batch)
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=dec.mem.device)
        h = C.c_void_p()
        L.check(L.lib().qam_verifier_create(dec._h, self.max_batch, _ptr(self.mem), nbytes, C.byref(h),
                                            _stream_handle()))
        self._h = h
        self._destroy = L.lib().qam_verifier_destroy
        d = dec._desc
        H, Q, KV, F, V = int(d.hidden), int(d.q_dim), int(d.kv_dim), int(d.ffn), int(d.vocab)
        self.n_ops = 4 * dec.n_layers + 2
        self.x = self._buffer(L.QAM_VER_X, H)
        self.hidden = self._buffer(L.QAM_VER_H, H)
        self.qkv = self._buffer(L.QAM_VER_QKV, Q + 2 * KV)
        self.m = self._buffer(L.QAM_VER_M, F)
        self.xn_flat = self._buffer(L.QAM_VER_XN, H).reshape(-1)
        self.y_flat = self._buffer(L.QAM_VER_Y, max(H, 2 * F)).reshape(-1)
        self.logits = self._buffer(L.QAM_VER_LOGITS, V)

    def _buffer(self, which: int, n: int) -> torch.Tensor:
        off = L.lib().qam_verifier_buffer(self._h, which) - self.mem.data_ptr()
        return self.mem[off:off + 4 * n * self.max_batch].view(torch.float32).view(self.max_batch, n)

    def xn(self, B: int, n: int) -> torch.Tensor:
        """The last rms output as [B, n] (rows packed with stride n)."""
        return self.xn_flat[:B * n].view(B, n)

    def y(self, B: int, n: int) -> torch.Tensor:
        """The last o, gate|up or down product's output as [B, n]."""
        return self.y_flat[:B * n].view(B, n)

    def run(self, rung: int, B: int, first: int, count: int = 1) -> None:
        L.check(L.lib().qam_verifier_run(self._h, int(rung), int(B), int(first), int(count), _stream_handle()))

    def step(self, rung: int, B: int) -> None:
        L.check(L.lib().qam_verifier_step(self._h, int(rung), int(B), _stream_handle()))

    def capture(self, rung: int, B: int) -> None:
        if getattr(self, "_capture_stream", None) is None:
            self._capture_stream = torch.cuda.Stream(device=self.mem.device)
        s = self._capture_stream
        s.wait_stream(torch.cuda.current_stream())
        L.check(L.lib().qam_verifier_capture(self._h, int(rung), int(B), C.c_void_p(s.cuda_stream)))
        torch.cuda.current_stream().wait_stream(s)

    def replay(self, rung: int, B: int) -> None:
        L.check(L.lib().qam_verifier_replay(self._h, int(rung), int(B), _stream_handle()))

    def __del__(self):
        h, destroy = getattr(self, "_h", None), getattr(self, "_destroy", None)
        self._h = None
        if h is not None and h.value and callable(destroy):
            destroy(h)


def argmax_rows(v: torch.Tensor, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [rows]: first index of the row maximum of fp32 v [rows, n] (no NaN)."""
    _require_cuda(v, "v", torch.float32)
    if v.dim() == 1:
        v = v.unsqueeze(0)
    rows, n = v.shape
    if workspace is None:
        workspace = torch.zeros(rows, dtype=torch.int64, device=v.device)
    out = torch.empty(rows, dtype=torch.int32, device=v.device)
    L.check(L.lib().qam_argmax_rows(_ptr(v), rows, n, n, _ptr(out), _ptr(workspace), _stream_handle()))
    return out


def speculate(dec: Decoder, ver: Verifier, embed: torch.Tensor, first_token: int, n_tokens: int, k: int,
              draft_rung: int = 2, verify_rung: int = 4):
    """Greedy draft-and-verify decoding: (tokens int32 [n_tokens], stats dict)."""
    _require_cuda(embed, "embed", torch.float32)
    if embed.dim() != 2 or tuple(embed.shape) != (int(dec._desc.vocab), int(dec._desc.hidden)):
        raise ValueError("embed must be [vocab, hidden]")
    out = np.zeros(max(1, int(n_tokens)), dtype=np.int32)
    st = L.QamSpecStats()
    L.check(L.lib().qam_decoder_speculate(dec._h, ver._h, _ptr(embed), int(first_token), int(n_tokens), int(k),
                                          int(draft_rung), int(verify_rung), out.ctypes.data_as(C.c_void_p),
                                          C.byref(st), _stream_handle()))
    stats = {f: int(getattr(st, f)) for f, _ in L.QamSpecStats._fields_}
    return out[:int(n_tokens)], stats


def escalation_schedule(scores, rate: float) -> np.ndarray:
    """bool [T]: the steps re-run at 8 bits (the round(rate T) largest scores, ties to the earlier step)."""
    sc = np.ascontiguousarray(np.asarray(scores, dtype=np.float64).reshape(-1))
    out = np.zeros(sc.shape[0], dtype=np.uint8)
    n = C.c_int64()
    L.check(L.lib().qam_escalation_schedule(sc.ctypes.data_as(C.c_void_p), sc.shape[0], float(rate),
                                            out.ctypes.data_as(C.c_void_p), C.byref(n)))
    return out.astype(bool)


def last_variant() -> str:
    return L.lib().qam_last_variant().decode()

"""Per-phase timeline of a decode step's products, from the timeline build.

Build the library with its stamps first (``python -m
query_adaptive_mixed_amd.build --timeline``, giving libqam_timeline.so), then

    python -m query_adaptive_mixed_amd.timeline [--rung 2] [--layers 5 20]

builds the Qwen3-0.6B-shaped decoder on seeded synthetic weights, captures
its step graph at the rung, replays a few warm-up steps, chooses one layer's
four products and the next layer's q|k|v, replays one more step and prints,
per product, the spread of every wave's stamps (kernel entry, work start,
first x sub-chunk staged, last tile multiplied, row sums formed, the block's
waves combined, split-K arrival counted, wave exit) and the gap from the
previous product's last wave to this one's first.  Stamps are the 100 MHz
wall clock, so times are in steps of 10 ns.  The timeline build adds a few
instructions per wave; its times are close to, not equal to, the product
library's.
"""

from __future__ import annotations

import argparse
import ctypes as C
import os
import sys

import numpy as np

from . import _lib as L

POINTS = ["kernel entry", "work start", "x staged", "tiles done", "row sums", "waves combined",
          "arrival counted", "wave exit"]
TICKS_PER_US = 100.0


def _load_timeline_library() -> None:
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.environ.get("QAM_LIBRARY") or os.path.join(here, "libqam_timeline.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built: run `python -m query_adaptive_mixed_amd.build --timeline`")
    L._LIB = L.load(path)


def select(planes) -> None:
    """Choose the matrices (their planes pointers, at most QAM_TIMELINE_SLOTS)
    whose launches record stamps, and clear the stamps."""
    arr = (C.c_void_p * max(1, len(planes)))(*planes)
    L.check(L.lib().qam_timeline_select(C.cast(arr, C.c_void_p), len(planes)))


def read() -> np.ndarray:
    """The stamps, int64 [slot][workgroup][wave][point] (0: not reached)."""
    n = L.QAM_TIMELINE_SLOTS * L.QAM_TIMELINE_GROUPS * 8 * L.QAM_TIMELINE_POINTS
    buf = np.zeros(n, dtype=np.uint64)
    L.check(L.lib().qam_timeline_read(buf.ctypes.data_as(C.c_void_p), n))
    return buf.reshape(L.QAM_TIMELINE_SLOTS, L.QAM_TIMELINE_GROUPS, 8, L.QAM_TIMELINE_POINTS).astype(np.int64)


def summarise(stamps: np.ndarray, names) -> list:
    """One text block per chosen product: waves, span, the gap from the
    previous product's last wave, and each point's spread (us after the
    product's first wave entered)."""
    out, prev_end = [], None
    for s, name in enumerate(names):
        v = stamps[s]
        live = v[:, :, 0] > 0
        if not live.any():
            out.append(f"{name:10s} no stamps")
            continue
        t0 = v[:, :, 0][live].min()
        t_end = v[:, :, 7][live].max()
        gap = "" if prev_end is None else f", {(t0 - prev_end) / TICKS_PER_US:.2f} us after the previous product"
        out.append(f"{name:10s} {int(live.sum())} waves, span {(t_end - t0) / TICKS_PER_US:.2f} us{gap}")
        for p in range(1, L.QAM_TIMELINE_POINTS):
            w = v[:, :, p][live]
            w = w[w > 0]
            if len(w):
                q = (np.percentile(w, [0, 50, 100]) - t0) / TICKS_PER_US
                out.append(f"    {POINTS[p]:16s} n {len(w):4d}   min {q[0]:6.2f}   median {q[1]:6.2f}   max {q[2]:6.2f}")
        prev_end = t_end
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--rung", type=int, default=2, help="rung of the step (2 = D4)")
    ap.add_argument("--layers", type=int, nargs="+", default=[5, 20], help="layers whose products are stamped")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--n-layers", type=int, default=28, help="layers of the decoder (Qwen3-0.6B has 28)")
    args = ap.parse_args(argv)
    _load_timeline_library()
    import torch

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import workloads as WL
    from .decode import build_decoder

    shape = dict(n_layers=args.n_layers, hidden=1024, q_dim=2048, kv_dim=1024, ffn=3072)
    if not 1 <= args.n_layers <= 28 or any(not 0 <= l < args.n_layers for l in args.layers):
        raise SystemExit("layers must lie in [0, n_layers), n_layers in [1, 28]")
    dec = build_decoder(WL.qwen_decode_field(0), shape["n_layers"], shape["hidden"], shape["q_dim"],
                        shape["kv_dim"], shape["ffn"], eps=1e-6)
    xs = torch.from_numpy(WL.decode_inputs(0, args.warmup + 1, shape["hidden"])).cuda()
    dec.capture(args.rung)
    for i in range(args.warmup):
        dec.hidden.copy_(xs[i])
        dec.replay(args.rung)
    torch.cuda.synchronize()
    print(f"timeline of a decode step at rung {args.rung} (Qwen3-0.6B shapes, seeded synthetic weights); "
          f"library {os.path.basename(L.lib()._name)}")
    for layer in args.layers:
        qkv, o, gu, down = dec._keep[1 + layer]
        nxt = dec._keep[2 + layer][0] if layer + 1 < shape["n_layers"] else None
        mats = [qkv, o, gu, down] + ([nxt] if nxt is not None else [])
        names = ["q|k|v", "o", "gate|up", "down", "next q|k|v"][:len(mats)]
        select([m.desc.planes for m in mats])
        dec.hidden.copy_(xs[args.warmup])
        dec.replay(args.rung)
        torch.cuda.synchronize()
        print(f"== layer {layer}")
        for line in summarise(read(), names):
            print(line)
    select([])
    return 0


if __name__ == "__main__":
    sys.exit(main())

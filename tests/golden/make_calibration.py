"""Write calibration.json: the focus_area f that puts each lens workload at a
target mean bits/weight.  Calls only the CPU oracle (and the seeded input
generators), so every stored value comes from the oracle.

The pages set no byte budget ("memory is what your lenses cost", FoQLens
landing page); the workloads name target means instead, so f is found by
bisection: mean bits (rule 7) never decreases as f grows, and the stored f is
the smallest one (to 2^-40) whose map reaches the target.  The realised mean
is stored beside it.

Run:  python tests/golden/make_calibration.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import workloads as WL  # noqa: E402


def mean_at(f, coords, centres, radii, g, glass, w, combine="sum"):
    lv = O.level_map(coords, centres, radii, f, g, combine, 5, glass)
    return O.mean_bits(lv, w), lv


def calibrate(coords, centres, radii, g, glass, target, w, combine="sum"):
    lo, hi = 0.0, 1.0
    m_lo, _ = mean_at(lo, coords, centres, radii, g, glass, w, combine)
    if m_lo >= target:
        return lo, m_lo
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        m, _ = mean_at(mid, coords, centres, radii, g, glass, w, combine)
        if m >= target:
            hi = mid
        else:
            lo = mid
    m_hi, lv = mean_at(hi, coords, centres, radii, g, glass, w, combine)
    return hi, m_hi


def main():
    out = {"note": "focus_area f per workload from bisection on the oracle's rule-7 mean bits; "
                   "written by tests/golden/make_calibration.py"}
    # Gemma-E2B-scale field: 5 lenses, g = 0.75, glass D2, sum
    fld = WL.e2b_field(0)
    lp = WL.e2b_lenses(fld)
    w = fld.block_weights()
    m05, _ = mean_at(0.5, fld.coords, lp.centres, lp.radii, lp.g, lp.glass, w)
    f4, m4 = calibrate(fld.coords, lp.centres, lp.radii, lp.g, lp.glass, 4.0, w)
    out["e2b_field"] = {"g": lp.g, "glass": lp.glass, "combine": "sum", "mean_bits_at_f0.5": m05,
                        "target_4.0": {"f": f4, "mean_bits": m4}}
    # streaming stack: 4 lenses, g = 1, glass ZERO or D2, mean 2, 3, 4, 6, 8
    st = WL.streaming_stack(0)
    cen, rad = WL.stack_lenses(st)
    w = st.block_weights()
    ss = {"g": 1.0, "combine": "sum"}
    for glass in (0, 1):
        for target in (2.0, 3.0, 4.0, 6.0, 8.0):
            f, m = calibrate(st.coords, cen, rad, 1.0, glass, target, w)
            lv = O.level_map(st.coords, cen, rad, f, 1.0, "sum", 5, glass)
            ss[f"glass{glass}_target{target}"] = {"f": f, "mean_bits": m,
                                                   "lifted_fraction": float(np.mean(lv > glass))}
    out["streaming_stack"] = ss
    # batched layer: per request 3 lenses, g = 1, glass D2, mean 4 (per request)
    bl = WL.batched_layer(0)
    w = bl.block_weights()
    reqs = []
    for r, (c, rr) in enumerate(WL.request_lenses(bl, 32)):
        f, m = calibrate(bl.coords, c, rr, 1.0, 1, 4.0, w)
        reqs.append({"f": f, "mean_bits": m})
    out["batched_layer"] = {"g": 1.0, "glass": 1, "combine": "sum", "requests": reqs}
    with open(os.path.join(HERE, "calibration.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps({k: (v if k != "batched_layer" else "...") for k, v in out.items()}, indent=1)[:3000])


if __name__ == "__main__":
    main()

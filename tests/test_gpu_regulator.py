"""GPU parity of the byte-budget regulator (the largest focus area whose lens
map fits a weight-byte budget) against the CPU oracle: the same bisection on
exact integer byte counts, so f, its bytes and its map agree exactly."""

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def both(qam, coords, w, cen, rad, g, combine, glass, budget, iters, stops=None, radius="lens", width=0.0):
    want = O.fit_focus_area(coords, cen, rad, g, combine, 5, glass, w, budget, iters=iters, stops=stops,
                            radius=radius, width=width)
    f, b, lv = qam.fit_focus_area(torch.from_numpy(coords).cuda(), torch.from_numpy(np.asarray(w, np.int64)).cuda(),
                                  cen, rad, g, budget, combine=combine, glass=glass, iters=iters, stops=stops,
                                  radius=radius, width=width)
    torch.cuda.synchronize()
    assert f == want[0], (f, want[0])
    assert b == want[1]
    assert np.array_equal(lv.cpu().numpy(), want[2])
    return f, b


def test_regulator_on_the_e2b_field(qam):
    fld = WL.e2b_field(0)
    lp = WL.e2b_lenses(fld)
    w = fld.block_weights().astype(np.int64)
    full = O.weight_bytes(O.level_map(fld.coords, lp.centres, lp.radii, 1.0, lp.g, "sum", 5, lp.glass), w)
    low = O.weight_bytes(O.level_map(fld.coords, lp.centres, lp.radii, 0.0, lp.g, "sum", 5, lp.glass), w)
    four_bits = int(np.sum(w)) * 4 // 8           # a mean of 4 bits per weight
    for budget in (four_bits, low + (full - low) // 3, full - 1):
        f, b = both(qam, fld.coords, w, lp.centres, lp.radii, lp.g, "sum", lp.glass, budget, 40)
        assert b <= budget


def test_regulator_small_fields_and_ends(qam):
    rng = np.random.default_rng(77)
    for trial in range(8):
        n = int(rng.integers(1, 400))
        coords = rng.uniform(0, 1, size=(n, 2))
        k = int(rng.integers(1, 6))
        cen = coords[rng.choice(n, min(k, n), replace=False)]
        rad = rng.uniform(0.0, 0.4, size=cen.shape[0])
        w = 64 * rng.choice([64, 1536, 6144], size=n)
        g = float(rng.choice([1.0, 0.75, 0.5]))
        combine = "sum" if trial % 2 else "max"
        glass = int(rng.integers(0, 3))
        kappa = O.ceiling(g, 4, glass)
        stops = None
        if kappa > glass and trial % 3 == 0:
            stops = np.sort(rng.uniform(0.1, 2.0, size=kappa - glass))[::-1]
        lo = O.weight_bytes(O.level_map(coords, cen, rad, 0.0, g, combine, 5, glass, stops), w)
        hi = O.weight_bytes(O.level_map(coords, cen, rad, 1.0, g, combine, 5, glass, stops), w)
        for budget in (max(0, lo - 1), lo, (lo + hi) // 2, hi, hi + 64):
            both(qam, coords, w, cen, rad, g, combine, glass, budget, int(rng.integers(0, 45)), stops)


def test_regulator_zone_radius(qam):
    """The regulator on zones (R = f D, D the field width from the device):
    the same f, bytes and map as the oracle's bisection."""
    fld = WL.e2b_field(0)
    lp = WL.e2b_lenses(fld)
    w = fld.block_weights().astype(np.int64)
    D = qam.field_width(torch.from_numpy(fld.coords).cuda())
    assert D == O.field_width(fld.coords)
    four_bits = int(np.sum(w)) * 4 // 8
    for budget in (four_bits, four_bits // 2 + four_bits // 4):
        f, b = both(qam, fld.coords, w, lp.centres, lp.radii, lp.g, "sum", lp.glass, budget, 40,
                    radius="zone", width=D)
        assert b <= budget

"""Pins for the CPU oracle: each check comes from something other than the
oracle's own formula (hand-worked examples, a different arithmetic route,
closed forms, invariants, brute force on tiny inputs)."""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as WL

GOLD = os.path.join(os.path.dirname(__file__), "golden")
LADDER = (0, 2, 4, 6, 8)


def _load(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ------------------------------------------------------------------ truncation

def test_truncation_golden_examples():
    g = _load("truncation_examples.json")
    for case in g["cases"]:
        for d, want in zip(g["depths"], case["codes"]):
            assert int(O.truncate(np.int8(case["q"]), d)) == want, (case, d)


def test_truncation_exhaustive_floor_division_route():
    """All 256 codes x 5 depths against Python floor division (a different
    route from the oracle's shifts) and the truncation invariants."""
    q = np.arange(-128, 128, dtype=np.int64)
    for d in LADDER:
        c = O.truncate(q.astype(np.int8), d)
        if d == 0:
            assert np.all(c == 0)
            continue
        step = 2 ** (8 - d)
        want = np.array([(int(v) // step) * step for v in q])
        assert np.array_equal(c, want)
        assert np.all(c <= q) and np.all(q < c + step)     # floor within one step
        assert np.all(c % step == 0)                        # multiple of the step
        assert np.all((c >= -128) & (c <= 127))             # still an int8 code
    assert np.array_equal(O.truncate(q.astype(np.int8), 8), q)   # D8 is the stored code
    for d0, d1 in zip(LADDER[1:-1], LADDER[2:]):            # deeper never moves away from q
        assert np.all(np.abs(q - O.truncate(q.astype(np.int8), d1))
                      <= np.abs(q - O.truncate(q.astype(np.int8), d0)))


def test_truncation_equals_residual_slice_sum():
    """Base + refinements rebuilt from the 2-bit slices equals the top-d-bit read."""
    q = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    dig = O.slice_digits(q)
    assert dig.min() >= 0 and dig.max() <= 3
    # digits re-form the byte exactly
    u = (q.astype(np.int64) & 0xFF)
    assert np.array_equal(sum(dig[:, s] << (2 * s) for s in range(4)), u)
    for d in LADDER:
        assert np.array_equal(O.residual_code(dig, d), O.truncate(q, d))


def test_truncation_by_byte_mask_route():
    """Masking the low 8-d bits of the byte and re-reading it as int8."""
    q = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    for d in LADDER[1:]:
        mask = (0xFF << (8 - d)) & 0xFF
        want = (q.view(np.uint8) & np.uint8(mask)).view(np.int8).astype(np.int64)
        assert np.array_equal(O.truncate(q, d), want)


# ------------------------------------------------------------------ lens rules

def _case_map(case, lenses):
    cen = np.array([lenses[n][:2] for n in case["lenses"]], dtype=np.float64)
    rad = np.array([lenses[n][2] for n in case["lenses"]], dtype=np.float64)
    return O.level_map(np.array(case["blocks"], dtype=np.float64), cen, rad, case["f"],
                       case["g"], case["combine"], 5, case["glass"], case["stops"])


@pytest.mark.parametrize("idx", range(9))
def test_level_map_hand_examples(idx):
    g = _load("lens_hand_examples.json")
    case = g["cases"][idx]
    got = _case_map(case, g["lenses"])
    assert got.tolist() == case["levels"], case["name"]


def test_ceiling_closed_form():
    # g = 0 -> the glass; g = 1 -> the top rung, for every glass
    for m in range(1, 8):
        for gam in range(0, m + 1):
            assert O.ceiling(0.0, m, gam) == gam
            assert O.ceiling(1.0, m, gam) == m
    assert O.ceiling(0.75, 4, 1) == 3 and O.ceiling(0.5, 4, 0) == 2 and O.ceiling(0.34, 4, 1) == 2


def test_default_stops_closed_form():
    for n in range(1, 9):
        s = O.profile_stops(n)
        assert s[0] == 1.0
        assert all(Fraction(float(s[j - 1])) == Fraction(n - j + 1, n)
                   or abs(float(s[j - 1]) - (n - j + 1) / n) < 1e-16 for j in range(1, n + 1))
        assert np.all(np.diff(s) < 0)


def _ring_scan(rho_star, s, glass):
    """The ring rho* falls into, by walking the ring intervals outward:
    [0, s_kappa) -> kappa, [s_kappa, s_(kappa-1)) -> kappa-1, ...,
    [s_(gamma+1), inf) -> gamma."""
    n = len(s)
    edges = [0.0] + [float(v) for v in s[::-1]] + [math.inf]   # 0 < s_kappa < ... < s_(gamma+1) < inf
    for k in range(n + 1):
        if edges[k] <= rho_star < edges[k + 1]:
            return glass + n - k
    raise AssertionError("rho* outside every ring")


def test_single_lens_reduces_to_ring_of_rho():
    """With one lens, L = max(0, 1 - rho/s_last) and rho* = min(rho, s_last),
    so the level is the ring that rho itself falls into (brute-force ring scan).
    Checked on random tiny maps, away from exact ties."""
    rng = np.random.default_rng(123)
    for trial in range(300):
        n_rungs = int(rng.integers(2, 8))
        m = n_rungs - 1
        glass = int(rng.integers(0, m))
        g = float(rng.uniform(0, 1))
        f = float(rng.uniform(0.05, 0.95))
        kappa = O.ceiling(g, m, glass)
        n = kappa - glass
        stops = None
        if n > 0 and rng.uniform() < 0.5:
            stops = np.sort(rng.uniform(0.1, 2.5, size=n))[::-1]
            if np.any(np.diff(stops) >= 0):
                stops = None
        coords = rng.uniform(0, 1, size=(8, 2))
        cen = rng.uniform(0, 1, size=(1, 2))
        r = rng.uniform(0.05, 0.5, size=1)
        got = O.level_map(coords, cen, r, f, g, "sum", n_rungs, glass, stops)
        if n == 0:
            assert np.all(got == glass)
            continue
        s = O.profile_stops(n, stops)
        R = r[0] * f / (1 - f)
        for b in range(8):
            rho = math.hypot(coords[b, 0] - cen[0, 0], coords[b, 1] - cen[0, 1]) / R
            if min(abs(rho - v) for v in s) < 1e-9:
                continue
            assert got[b] == _ring_scan(min(rho, float(s[0])), s, glass)


def test_level_map_bruteforce_8_blocks_count_vs_scan():
    """The count form gamma + #{j : rho* < s_j} against the explicit ring scan,
    for many lenses, on random 8-block maps; rho* recomputed from a scalar
    walk of rules 4-6 with Python floats."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        glass = int(rng.integers(0, 4))
        g = float(rng.uniform(0, 1))
        f = float(rng.uniform(0.05, 0.9))
        combine = "sum" if trial % 2 == 0 else "max"
        nl = int(rng.integers(1, 5))
        coords = rng.uniform(0, 1, size=(8, 2))
        cen = rng.uniform(0, 1, size=(nl, 2))
        r = rng.uniform(0.05, 0.4, size=nl)
        got = O.level_map(coords, cen, r, f, g, combine, 5, glass)
        kappa = O.ceiling(g, 4, glass)
        n = kappa - glass
        if n == 0:
            assert np.all(got == glass)
            continue
        s = O.profile_stops(n)
        for b in range(8):
            lifts = []
            for i in range(nl):
                rho = math.sqrt((coords[b, 0] - cen[i, 0]) ** 2 + (coords[b, 1] - cen[i, 1]) ** 2) / (r[i] * f / (1 - f))
                lifts.append(max(0.0, 1.0 - rho / float(s[0])))
            L = min(1.0, sum(lifts)) if combine == "sum" else max(lifts)
            rs = float(s[0]) * (1.0 - L)
            if min(abs(rs - v) for v in s) < 1e-9:
                continue
            assert got[b] == _ring_scan(rs, s, glass)


def test_level_map_invariants():
    """Bounds and monotonicity: levels stay in [glass, kappa]; adding a lens,
    raising g or raising f never lowers a level; sum >= max; a block far
    outside every lens keeps the glass; the map is unchanged when every
    coordinate and size is scaled by 2 (exact in fp64)."""
    rng = np.random.default_rng(11)
    for trial in range(100):
        coords = rng.uniform(0, 1, size=(64, 2))
        cen = coords[rng.choice(64, 3, replace=False)]
        r = rng.uniform(0.05, 0.3, size=3)
        glass = int(rng.integers(0, 3))
        f, g = float(rng.uniform(0.1, 0.9)), float(rng.uniform(0, 1))
        base = O.level_map(coords, cen, r, f, g, "sum", 5, glass)
        kappa = O.ceiling(g, 4, glass)
        assert base.min() >= glass and base.max() <= kappa
        two = O.level_map(coords, cen[:2], r[:2], f, g, "sum", 5, glass)
        assert np.all(base >= two)
        assert np.all(O.level_map(coords, cen, r, f, min(1.0, g + 0.2), "sum", 5, glass) >= base)
        assert np.all(O.level_map(coords, cen, r, min(0.95, f + 0.05), g, "sum", 5, glass) >= base)
        mx = O.level_map(coords, cen, r, f, g, "max", 5, glass)
        assert np.all(base >= mx)
        far = O.level_map(np.array([[50.0, 50.0]]), cen, r, f, g, "sum", 5, glass)
        assert far[0] == glass
        scaled = O.level_map(coords * 2, cen * 2, r * 2, f, g, "sum", 5, glass)
        assert np.array_equal(scaled, base)


def test_level_map_centre_reaches_ceiling():
    rng = np.random.default_rng(3)
    coords = rng.uniform(0, 1, size=(32, 2))
    for glass in range(4):
        for g in (0.0, 0.3, 0.75, 1.0):
            got = O.level_map(coords, coords[[5]], [0.1], 0.5, g, "sum", 5, glass)
            assert got[5] == O.ceiling(g, 4, glass)


# ------------------------------------------------------------------ memory formula

def test_memory_uniform_maps_exact():
    w = np.full(8, 64 * 256, dtype=np.int64)
    for idx, d in enumerate(LADDER):
        assert O.mean_bits(np.full(8, idx), w) == d
        assert O.weight_bytes(np.full(8, idx), w) == 8 * 64 * 256 * d // 8


def test_memory_all_5pow8_maps_of_eight_equal_blocks():
    """Every one of the 390,625 maps over 8 equal blocks: the formula equals
    the plain average of the bits (exact rational arithmetic)."""
    w = np.full(8, 64 * 256, dtype=np.int64)
    maps = np.array(list(itertools.product(range(5), repeat=8)), dtype=np.int64)
    bits = np.array(LADDER, dtype=np.int64)[maps]
    want = bits.sum(axis=1)                       # 8 * mean, exact
    got = np.array([O.mean_bits(mp, w) for mp in maps[::97]])
    assert np.allclose(got * 8, want[::97], rtol=0, atol=1e-12)
    # the vectorised check over all maps: bytes are exact integers
    assert np.all(bits.sum(axis=1) * 64 * 256 // 8 == [int(v) * 2048 for v in want])
    for mp in maps[::3907]:
        assert O.weight_bytes(mp, w) == int(np.array(LADDER)[mp].sum()) * 2048


def test_memory_unequal_blocks_hand_example():
    # a K = 256 block at D2 and a K = 512 block at D8: (2*16384 + 8*32768) / 49152 = 6
    w = np.array([64 * 256, 64 * 512], dtype=np.int64)
    assert O.mean_bits(np.array([1, 4]), w) == 6.0
    assert O.weight_bytes(np.array([1, 4]), w) == (2 * 16384 + 8 * 32768) // 8


# ------------------------------------------------------------------ qmatvec

def _int_inputs(rng, N, K, B):
    W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    x = rng.integers(-3, 4, size=(B, K)).astype(np.float64)
    return W, x


def test_qmatvec_d8_equals_untruncated_int_product():
    rng = np.random.default_rng(5)
    W, x = _int_inputs(rng, 256, 384, 3)
    level = np.full(4, 4)
    y = O.qmatvec_ref(W, np.ones(256), x, level)
    want = x.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(y, want.astype(np.float64))


def test_qmatvec_uniform_depth_equals_masked_int_product():
    rng = np.random.default_rng(6)
    W, x = _int_inputs(rng, 192, 256, 2)
    for idx, d in enumerate(LADDER):
        y = O.qmatvec_ref(W, np.ones(192), x, np.full(3, idx))
        if d == 0:
            assert np.all(y == 0)
            continue
        mask = np.uint8((0xFF << (8 - d)) & 0xFF)
        c = (W.view(np.uint8) & mask).view(np.int8).astype(np.int64)
        assert np.array_equal(y, (x.astype(np.int64) @ c.T).astype(np.float64))


def test_qmatvec_mixed_map_blockwise_and_scaled():
    """A mixed map equals, block by block, the uniform-depth product of that
    block; scales multiply rows (float x, fp64)."""
    rng = np.random.default_rng(8)
    W = rng.integers(-127, 128, size=(320, 128), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=320)
    x = rng.standard_normal((2, 128))
    level = np.array([0, 1, 2, 3, 4])
    y = O.qmatvec_ref(W, sc, x, level)
    for b in range(5):
        rows = slice(64 * b, 64 * b + 64)
        d = LADDER[level[b]]
        if d == 0:
            assert np.all(y[:, rows] == 0)
            continue
        step = 2 ** (8 - d)
        c = np.floor_divide(W[rows].astype(np.int64), step) * step
        want = np.einsum("rk,nk->rn", x, c.astype(np.float64)) * sc[rows]
        assert np.allclose(y[:, rows], want, rtol=1e-13, atol=1e-15)


def test_qmatvec_per_request_maps_equal_separate_calls():
    rng = np.random.default_rng(9)
    W = rng.integers(-127, 128, size=(256, 64), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=256)
    x = rng.standard_normal((3, 64))
    maps = rng.integers(0, 5, size=(3, 4))
    y = O.qmatvec_ref(W, sc, x, maps, per_request=True)
    for r in range(3):
        assert np.allclose(y[r], O.qmatvec_ref(W, sc, x[r:r + 1], maps[r])[0], rtol=1e-12, atol=1e-12)


def test_qmatvec_brute_force_maps_table_cfg1():
    """Single 512x256 layer: the output for any map is assembled from a
    per-block, per-depth table; sampled maps against the oracle."""
    inp = WL.single_layer_512x256(0)
    W, sc, x = inp["W"], inp["scales"], inp["x"]
    table = np.zeros((8, 5, 64))
    for b in range(8):
        for idx, d in enumerate(LADDER):
            rows = slice(64 * b, 64 * b + 64)
            step = 2 ** (8 - d) if d else None
            c = np.zeros((64, 256)) if d == 0 else (np.floor_divide(W[rows].astype(np.int64), step) * step).astype(np.float64)
            table[b, idx] = (c @ x[0].astype(np.float64)) * sc[rows].astype(np.float64)
    rng = np.random.default_rng(1)
    for mp in rng.integers(0, 5, size=(300, 8)):
        y = O.qmatvec_ref(W, sc, x, mp)[0]
        want = np.concatenate([table[b, mp[b]] for b in range(8)])
        assert np.allclose(y, want, rtol=1e-13, atol=1e-16)


def test_tolerance_bounds_output_and_vanishes_on_zero():
    rng = np.random.default_rng(10)
    W = rng.integers(-127, 128, size=(128, 64), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=128)
    x = rng.standard_normal((1, 64))
    lvl = np.array([0, 3])
    tol = O.qmatvec_tolerance(W, sc, x, lvl)
    y = O.qmatvec_ref(W, sc, x, lvl)
    assert np.all(tol[:, :64] == 0)
    assert np.all(tol >= 1e-4 * np.abs(y) - 1e-18)


# ------------------------------------------------------------------ escalation

def test_escalation_schedule_closed_form():
    scores = WL.escalation_scores(0, 256)
    mask = O.escalation_schedule(scores, 0.16)
    assert mask.sum() == 41                                    # round(0.16 * 256) = round(40.96)
    assert scores[mask].min() > scores[~mask].max()            # exactly the 41 largest
    assert O.escalation_byte_ratio(mask) == float(Fraction(1, 2) + Fraction(41, 256))
    assert O.escalation_byte_ratio(mask) == 0.66015625
    assert O.escalation_byte_ratio(np.zeros(256, bool)) == 0.5
    assert O.escalation_byte_ratio(np.ones(256, bool)) == 1.5


# ------------------------------------------------------------------ glue

def test_rmsnorm_and_silu_closed_forms():
    x = np.array([[3.0, 4.0]])
    y = O.rmsnorm_ref(x, eps=0.0)                 # rms = sqrt(12.5)
    assert np.allclose(y, x / math.sqrt(12.5), rtol=1e-15)
    assert np.allclose(np.mean(O.rmsnorm_ref(np.random.default_rng(0).standard_normal((4, 100)), 0.0) ** 2, axis=1), 1.0)
    assert O.silu_mul_ref(0.0, 5.0) == 0.0
    assert abs(O.silu_mul_ref(1.0, 1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu_mul_ref(-50.0, 1.0)) < 1e-19


# ------------------------------------------------------------------ generators

def test_generators_are_seeded_and_shaped():
    a = WL.single_layer_512x256(0)
    b = WL.single_layer_512x256(0)
    assert np.array_equal(a["W"], b["W"]) and np.array_equal(a["x"], b["x"])
    assert a["W"].dtype == np.int8 and a["W"].min() >= -127 and a["W"].max() <= 127
    assert a["scales"].dtype == np.float32 and a["scales"].min() >= 0.001 and a["scales"].max() <= 0.02
    fld = WL.e2b_field(0)
    assert fld.n_blocks == 9360 and fld.n_weights == 1_132_462_080
    assert WL.qwen_decode_field(0).n_blocks == 7750
    assert WL.batched_layer(0).n_blocks == 352
    assert WL.streaming_stack(0).n_blocks == 4608 and WL.streaming_stack(0).n_weights == 3_758_096_384


# ---------------------------------------------------------------- the escalation gate's uncertainty

def test_uncertainty_closed_forms():
    """Uniform logits: H = ln V and margin 0; two logits a, b: the binary
    entropy of q = 1 / (1 + e^(b - a)); one logit L above V - 1 zeros: the
    two-level entropy; every case written from its closed form, not the
    oracle's formula."""
    for V in (2, 7, 151936):
        u = O.uncertainty(np.full(V, 3.25))
        assert abs(u["entropy"] - math.log(V)) <= 1e-12 * math.log(V)
        assert u["margin"] == 0.0 and (u["top1"], u["top2"]) == (0, 1)
    for a, b in ((0.0, 0.0), (2.0, -1.0), (-5.5, 7.25), (30.0, 0.0)):
        q = 1.0 / (1.0 + math.exp(b - a))
        want = -(q * math.log(q) + (1.0 - q) * math.log1p(-q)) if 0.0 < q < 1.0 else 0.0
        u = O.uncertainty([a, b])
        assert abs(u["entropy"] - want) <= 1e-12, (a, b)
        assert abs(u["margin"] - abs(2.0 * q - 1.0)) <= 1e-12
    V, L = 1000, 6.0
    d = math.exp(L) + (V - 1)
    p1, po = math.exp(L) / d, 1.0 / d
    want = -(p1 * math.log(p1) + (V - 1) * po * math.log(po))
    z = np.zeros(V)
    z[417] = L
    u = O.uncertainty(z)
    assert abs(u["entropy"] - want) <= 1e-12 and abs(u["margin"] - (p1 - po)) <= 1e-12
    assert (u["top1"], u["top2"]) == (417, 0)


def test_uncertainty_against_scipy_and_invariants():
    """Random logits: entropy equals scipy's entropy of scipy's softmax;
    shifting or permuting the logits changes nothing; -inf logits are tokens
    of probability 0 (the same as leaving them out)."""
    from scipy.special import softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(31)
    for V in (3, 100, 5000):
        z = rng.standard_normal(V) * rng.uniform(0.1, 8.0)
        u = O.uncertainty(z)
        assert abs(u["entropy"] - entropy(softmax(z))) <= 1e-10
        p = np.sort(softmax(z))[::-1]
        assert abs(u["margin"] - (p[0] - p[1])) <= 1e-12
        assert 0.0 <= u["entropy"] <= math.log(V) + 1e-12 and 0.0 <= u["margin"] <= 1.0
        us = O.uncertainty(z + 123.5)
        assert abs(us["entropy"] - u["entropy"]) <= 1e-10 and abs(us["margin"] - u["margin"]) <= 1e-12
        perm = rng.permutation(V)
        up = O.uncertainty(z[perm])
        assert abs(up["entropy"] - u["entropy"]) <= 1e-10
        assert perm[up["top1"]] == u["top1"]
        zi = np.concatenate([z, np.full(17, -np.inf)])
        ui = O.uncertainty(zi)
        assert abs(ui["entropy"] - u["entropy"]) <= 1e-12 and ui["top1"] == u["top1"]


def test_uncertainty_ties_and_no_distribution():
    z = np.array([1.0, 4.0, 2.0, 4.0, 4.0])
    u = O.uncertainty(z)
    assert (u["top1"], u["top2"]) == (1, 3) and u["margin"] == 0.0
    for bad in ([0.0, np.nan, 1.0], [0.0, np.inf], [-np.inf, -np.inf]):
        u = O.uncertainty(bad)
        assert math.isnan(u["entropy"]) and math.isnan(u["margin"])
        assert O.gate(bad, 10.0, -1.0)


def test_gate_rules():
    """Entropy above its threshold, or margin below its threshold, escalates;
    +inf / -inf thresholds switch a test off."""
    sharp = np.zeros(50)
    sharp[3] = 20.0                      # H ~ 0, margin ~ 1
    flat = np.zeros(50)                  # H = ln 50, margin 0
    assert not O.gate(sharp, 1.0, 0.1)
    assert O.gate(flat, 1.0, 0.1)
    assert O.gate(flat, math.inf, 0.1)           # the margin alone
    assert O.gate(flat, 1.0, -math.inf)          # the entropy alone
    assert not O.gate(flat, math.inf, -math.inf)
    assert not O.gate(flat, math.log(50) + 1e-9, -math.inf)


# ---------------------------------------------------------------- the byte-budget regulator

def _field(seed, n=60, n_lenses=3):
    rng = np.random.default_rng(seed)
    coords = rng.uniform(0, 1, size=(n, 2))
    cen = coords[rng.choice(n, n_lenses, replace=False)]
    rad = rng.uniform(0.05, 0.3, size=n_lenses)
    w = 64 * rng.choice([256, 1024, 4096], size=n)
    return coords, cen, rad, w


def test_fit_focus_area_against_a_fine_scan():
    """On small fields the regulator's f is the edge a brute-force scan finds:
    the map at f fits the budget, the map 2^-iters above it does not, and no
    f on a fine grid below the edge has more bytes than the budget."""
    for seed in range(6):
        coords, cen, rad, w = _field(seed)
        full = O.weight_bytes(O.level_map(coords, cen, rad, 1.0, 1.0, "sum", 5, 1), w)
        low = O.weight_bytes(O.level_map(coords, cen, rad, 0.0, 1.0, "sum", 5, 1), w)
        for frac in (0.2, 0.5, 0.8):
            budget = int(low + frac * (full - low))
            f, b, lv = O.fit_focus_area(coords, cen, rad, 1.0, "sum", 5, 1, w, budget, iters=30)
            assert b <= budget and b == O.weight_bytes(lv, w)
            above = O.weight_bytes(O.level_map(coords, cen, rad, min(1.0, f + 2.0 ** -30), 1.0, "sum", 5, 1), w)
            assert above > budget
            grid = np.linspace(0.0, f, 257)
            assert max(O.weight_bytes(O.level_map(coords, cen, rad, x, 1.0, "sum", 5, 1), w) for x in grid) <= budget


def test_fit_focus_area_ends_and_monotone():
    coords, cen, rad, w = _field(9)
    full = O.weight_bytes(O.level_map(coords, cen, rad, 1.0, 0.75, "max", 5, 1), w)
    low = O.weight_bytes(O.level_map(coords, cen, rad, 0.0, 0.75, "max", 5, 1), w)
    assert O.fit_focus_area(coords, cen, rad, 0.75, "max", 5, 1, w, full)[0] == 1.0
    f0, b0, _ = O.fit_focus_area(coords, cen, rad, 0.75, "max", 5, 1, w, low - 1)
    assert f0 == 0.0 and b0 == low > low - 1
    fs = [O.fit_focus_area(coords, cen, rad, 0.75, "max", 5, 1, w, low + k * (full - low) // 7, iters=24)[0]
          for k in range(8)]
    assert all(a <= b for a, b in zip(fs, fs[1:])) and fs[-1] == 1.0


# ---------------------------------------------------------------- layer decides

def test_layer_scores_hand_values():
    """[FoQLens] "FoQZones, the mechanism", layer-decides variant: reduced
    draft score |y_c|^2 Delta_c^2 Delta_c^2 / w_c, worked by hand."""
    K = 64
    y = np.zeros(192, np.float32)
    y[:64] = 1.0                      # block 0: |y|^2 = 64
    y[64 + 7] = 3.0                   # block 1: |y|^2 = 9
    sc = np.full(192, 0.5, np.float32)
    sc[64:128] = np.where(np.arange(64) % 2 == 0, 1.0, 3.0).astype(np.float32)   # mean scale^2 = 5
    sc[128:] = 2.0                    # block 2: y = 0
    got = O.layer_scores(y, sc, K)
    assert got.shape == (1, 3)
    # block 0: 64 * 0.25 * 0.25 / 4096 = 2^-10; block 1: 9 * 5 * 5 / 4096
    assert got[0, 0] == 2.0 ** -10
    assert got[0, 1] == 225.0 / 4096.0
    assert got[0, 2] == 0.0


def test_layer_scores_scaling_laws():
    """Exact powers of two move the score by exact factors: outputs x4 give
    x16 (the square of the output), scales x2 give x16 (the step enters
    squared, twice), K x2 halves it (weights of the block); each block is
    scored on its own rows only."""
    rng = np.random.default_rng(3)
    B, N, K = 3, 64 * 9, 128
    y = rng.standard_normal((B, N)).astype(np.float32)
    sc = rng.uniform(0.01, 0.2, N).astype(np.float32)
    base = O.layer_scores(y, sc, K)
    assert np.array_equal(O.layer_scores(y * 4, sc, K), base * 16)
    assert np.array_equal(O.layer_scores(y, sc * 2, K), base * 16)
    assert np.array_equal(O.layer_scores(y, sc, 2 * K), base / 2)
    y2 = y.copy()
    y2[1, 64 * 4:64 * 5] *= 4          # one block of one request
    got = O.layer_scores(y2, sc, K)
    want = base.copy()
    want[1, 4] *= 16
    assert np.array_equal(got, want)
    sc2 = sc.copy()
    sc2[64 * 6:64 * 7] *= 2            # one block's scales
    want = base.copy()
    want[:, 6] *= 16
    assert np.array_equal(O.layer_scores(y, sc2, K), want)
    # against a brute-force sum per block (in the same row order)
    for r in range(B):
        for c in range(N // 64):
            e = 0.0
            d = 0.0
            for i in range(64):
                e += float(y[r, 64 * c + i]) ** 2
                d += float(sc[64 * c + i]) ** 2
            d /= 64
            assert base[r, c] == (e * d * d) / (64 * K)


def test_layer_levels_threshold_rules():
    """level = glass + #{j >= 1 : s >= lambda 16^j}, capped at kappa."""
    lv = lambda s, g=1.0, lam=1.0, glass=1: O.layer_levels_threshold(np.array(s, np.float64), 5, glass, g, lam)
    assert lv([0.0, 15.999, 16.0, 255.0, 256.0, 4096.0, 65536.0, 1e300]).tolist() == [1, 1, 2, 2, 3, 4, 4, 4]
    assert lv([16.0, 256.0, 4096.0], g=0.7).tolist() == [2, 3, 3]        # kappa = 1 + floor(0.7 * 3) = 3
    assert lv([16.0, 256.0, 4096.0], g=0.5).tolist() == [2, 2, 2]        # kappa = 1 + floor(0.5 * 3) = 2
    assert lv([16.0, 4096.0], g=0.0).tolist() == [1, 1]                   # kappa = glass
    assert lv([0.5, 8.0, 128.0], lam=0.5).tolist() == [1, 2, 3]           # 0.5*16 = 8, 0.5*256 = 128
    assert lv([np.nan, np.inf], glass=0).tolist() == [0, 4]
    assert lv([1.0], lam=0.0).tolist() == [4]                              # every threshold is 0
    # scores x16 climb exactly one rung until the cap, once at or above
    # lambda (j starts at 1: below lambda 16 a block stays at the glass)
    rng = np.random.default_rng(4)
    s = np.exp(rng.uniform(-5, 12, 2000))
    a = lv(s, glass=0)
    b = lv(s * 16, glass=0)
    assert np.array_equal(b, np.minimum(a + (s >= 1.0), 4))
    assert np.array_equal(a[s < 16.0], np.zeros(int(np.sum(s < 16.0)), np.uint8))


def test_layer_levels_share_invariants():
    """Per request exactly floor(f n) blocks rise to kappa, every one of them
    scores at least every block left at the glass, and equal scores go in
    block order."""
    rng = np.random.default_rng(5)
    B, nb = 4, 77
    s = np.round(rng.uniform(0, 6, (B, nb)), 0)          # many ties
    s[2, 10] = np.nan
    for f in (0.0, 0.1, 0.5, 0.99, 1.0):
        lv = O.layer_levels_share(s, 5, 1, 1.0, f)
        for r in range(B):
            risen = np.nonzero(lv[r] == 4)[0]
            stay = np.nonzero(lv[r] == 1)[0]
            assert len(risen) + len(stay) == nb
            finite = int(np.sum(~np.isnan(s[r])))
            assert len(risen) == min(int(np.floor(f * nb)), finite)
            for a in risen:
                assert not np.isnan(s[r, a])
                for b in stay:
                    if np.isnan(s[r, b]):
                        continue
                    assert s[r, a] > s[r, b] or (s[r, a] == s[r, b] and a < b)
    lv = O.layer_levels_share(s, 5, 2, 0.5, 0.3)        # kappa = 2 + floor(0.5 * 2) = 3
    assert set(np.unique(lv).tolist()) == {2, 3}


def test_tolerance_hand_computed_read_depth():
    """The bound's |w| is taken at the block's read depth (hand-computed
    sums in tests/golden/tolerance_examples.json): codes 0..63 read as 0 at
    D2, so row 1 has a zero bound there; untruncated codes at D2 would give
    row 0 a sum of 47, not 136."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tolerance_examples.json")))
    K = g["K"]
    W = np.zeros((64, K), dtype=np.int8)
    sc = np.ones(64)
    for r in g["rows"]:
        W[r["row"]] = r["codes"]
        sc[r["row"]] = r["scale"]
    x = np.array(g["x"])
    listed = [r["row"] for r in g["rows"]]
    for lev, want in g["by_level_request0"].items():
        t = O.qmatvec_tolerance(W, sc, x[:1], np.array([int(lev)]), rel=1.0)
        assert t.shape == (1, 64)
        assert t[0, listed].tolist() == want, (lev, t[0, listed])
        assert np.all(np.delete(t[0], listed) == 0.0)
    # per-request maps: request 0 at D2, request 1 at D4
    t = O.qmatvec_tolerance(W, sc, x, np.array([[1], [2]]), per_request=True, rel=1.0)
    assert t[0, listed].tolist() == g["by_level_request0"]["1"]
    assert t[1, listed].tolist() == g["by_level_request1"]["2"]
    # the default rel is the 1e-4 of the bound
    assert np.allclose(O.qmatvec_tolerance(W, sc, x[:1], np.array([2]))[0, listed],
                       1e-4 * np.array(g["by_level_request0"]["2"]), rtol=1e-15, atol=0)


# ------------------------------------------------------------------ zone radius

def test_zone_radius_hand_examples():
    g = json.load(open(os.path.join(GOLD, "zone_hand_examples.json")))
    c = np.array(g["coords"])
    assert O.field_width(c) == g["width"]
    for f, want in g["maps"].items():
        got = O.level_map(c, [g["centre"]], [0.123], float(f), g["g"], "sum", 5, g["glass"],
                          radius="zone", width=g["width"])
        assert got.tolist() == want, (f, got)


def test_field_width_closed_forms():
    assert O.field_width(np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])) == math.sqrt(2.0)
    assert O.field_width(np.array([[0.3, 0.7]])) == 0.0
    xs = np.array([0.5, -1.25, 3.0, 0.0, 2.75])
    assert O.field_width(np.stack([xs, np.full(5, 0.1)], axis=1)) == 4.25     # collinear: max - min
    ang = np.arange(6) * (np.pi / 3)                                          # hexagon of radius 2
    hexa = np.stack([2 * np.cos(ang), 2 * np.sin(ang)], axis=1)
    assert abs(O.field_width(hexa) - 4.0) <= 4 * np.finfo(float).eps


def test_field_width_is_the_largest_pairwise_distance():
    rng = np.random.default_rng(21)
    for n in (2, 3, 9, 40):
        c = rng.uniform(-3, 3, size=(n, 2))
        D = O.field_width(c)
        pair = [math.dist(a, b) for a, b in itertools.combinations(c.tolist(), 2)]
        assert abs(D - max(pair)) <= 2 * np.finfo(float).eps * max(pair)
        # permutation and power-of-two translation change nothing
        assert O.field_width(c[rng.permutation(n)]) == D
        assert O.field_width(c + 4.0) == D or abs(O.field_width(c + 4.0) - D) <= 8 * np.finfo(float).eps * D


def test_zone_ends_centre_only_and_whole_network():
    """f = 0: only a block at the centre is lifted; f = 1 (R = D): a block is
    lifted exactly when it is nearer the centre than D."""
    rng = np.random.default_rng(22)
    for trial in range(6):
        c = rng.uniform(0, 1, size=(30, 2))
        D = O.field_width(c)
        k = int(rng.integers(0, 30))
        for glass in (0, 1):
            z0 = O.level_map(c, c[k:k + 1], [0.2], 0.0, 1.0, "sum", 5, glass, radius="zone", width=D)
            assert z0[k] == 4 and np.all(np.delete(z0, k) == glass)
            z1 = O.level_map(c, c[k:k + 1], [0.2], 1.0, 1.0, "sum", 5, glass, radius="zone", width=D)
            d = np.sqrt(((c - c[k]) ** 2).sum(axis=1))
            assert np.array_equal(z1 > glass, d < D)


def test_zone_monotone_in_f_and_ignores_lens_sizes():
    rng = np.random.default_rng(23)
    c = rng.uniform(0, 1, size=(60, 2))
    D = O.field_width(c)
    cen = c[rng.choice(60, 3, replace=False)]
    prev = None
    for f in np.linspace(0, 1, 21):
        a = O.level_map(c, cen, [0.05, 0.2, 0.3], f, 0.75, "sum", 5, 1, radius="zone", width=D)
        b = O.level_map(c, cen, [9.0, 0.0, 1.0], f, 0.75, "sum", 5, 1, radius="zone", width=D)
        assert np.array_equal(a, b)
        if prev is not None:
            assert np.all(a >= prev)
        prev = a


def test_regulator_zone_radius_edge():
    """The regulator on zones: its f fits and a fine scan finds nothing
    above it that fits (bytes never decrease as f grows)."""
    rng = np.random.default_rng(24)
    c = rng.uniform(0, 1, size=(80, 2))
    D = O.field_width(c)
    cen = c[rng.choice(80, 2, replace=False)]
    w = np.full(80, 64 * 256, dtype=np.int64)
    full = O.weight_bytes(np.full(80, 4), w)
    floor = O.weight_bytes(np.full(80, 1), w)            # every block at the glass (D2)
    assert O.fit_focus_area(c, cen, [0.1, 0.2], 1.0, "sum", 5, 1, w, floor - 1, radius="zone", width=D)[0] == 0.0
    for budget in (floor + full // 16, full // 2, (3 * full) // 4):
        f, b, lv = O.fit_focus_area(c, cen, [0.1, 0.2], 1.0, "sum", 5, 1, w, budget, iters=30,
                                    radius="zone", width=D)
        assert b <= budget and b == O.weight_bytes(lv, w)
        for f2 in np.linspace(f + 2.0 ** -29, 1.0, 60):
            lv2 = O.level_map(c, cen, [0.1, 0.2], f2, 1.0, "sum", 5, 1, radius="zone", width=D)
            assert O.weight_bytes(lv2, w) >= b
        above = O.level_map(c, cen, [0.1, 0.2], f + 2.0 ** -30, 1.0, "sum", 5, 1, radius="zone", width=D)
        assert O.weight_bytes(above, w) > budget or f == 1.0

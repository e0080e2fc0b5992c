"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: level maps and reconstructed int codes bit-exact; fp32 outputs within
1e-4 * sum_k |w_nk| |x_k| per row (w = scale * code at the block's depth),
so a ZERO block must give exactly 0; exact-integer special cases bit-exact.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
LADDER = (0, 2, 4, 6, 8)


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pack(qam, W, sc):
    return qam.pack_slices(dev(W), dev(sc.astype(np.float32)))


def check_y(y, W, sc, x, lv, what=""):
    ref = O.qmatvec_ref(W, sc, x, lv)
    tol = O.qmatvec_tolerance(W, sc, x, lv)
    err = np.abs(y.astype(np.float64) - ref)
    bad = err > tol
    assert not bad.any(), (what, int(bad.sum()), float((err / np.maximum(tol, 1e-300)).max()))
    zero_rows = np.repeat(np.asarray(lv) == 0, 64)
    assert np.all(y[:, zero_rows] == 0.0), what


# ------------------------------------------------------------------ codes

@pytest.mark.parametrize("N,K", [(64, 64), (512, 256), (192, 1088), (1024, 4096)])
def test_unpack_codes_bit_exact_every_depth(qam, N, K):
    rng = np.random.default_rng(N + K)
    W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N)
    pm = pack(qam, W, sc)
    nb = N // 64
    for lv in [np.full(nb, d, np.uint8) for d in range(5)] + [rng.integers(0, 5, nb).astype(np.uint8)]:
        got = host(qam.unpack_codes(pm, dev(lv)))
        want = np.concatenate([O.truncate(W[64 * b:64 * b + 64], LADDER[lv[b]]) for b in range(nb)])
        assert np.array_equal(got.astype(np.int64), want), lv
    # the scales travel with the planes
    got_sc = host(pm.buf[N * K:].view(torch.float32))
    assert np.array_equal(got_sc, sc.astype(np.float32))


def test_identity_batch_probe_reads_the_codes(qam):
    """x = e_k through the real product kernel gives y = scale * c[:, k] exactly."""
    rng = np.random.default_rng(3)
    N, K = 256, 512
    W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = np.ones(N, np.float32)
    pm = pack(qam, W, sc)
    lv = np.array([1, 2, 3, 4], np.uint8)
    cols = [0, 1, 63, 64, 200, 511]
    x = np.zeros((len(cols), K), np.float32)
    for i, k in enumerate(cols):
        x[i, k] = 1.0
    y = host(qam.qmatvec(dev(x), pm, dev(lv)))
    for i, k in enumerate(cols):
        want = np.concatenate([O.truncate(W[64 * b:64 * b + 64, k], LADDER[lv[b]]) for b in range(4)])
        assert np.array_equal(y[i].astype(np.int64), want)


# ------------------------------------------------------------------ level maps

def _gpu_map(qam, coords, centres, radii, f, g, combine, glass, stops=None, ladder=LADDER):
    """The product's map call on the product ladder; the rules on any other
    ladder through the rung-map call (the same kernel)."""
    fn = qam.build_level_map if tuple(ladder) == LADDER else qam.build_rung_map
    return host(fn(dev(coords.astype(np.float64)), centres, radii, f, g, combine, glass, ladder_bits=ladder,
                   stops=stops))


def test_level_map_hand_examples(qam):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lens_hand_examples.json")))
    for case in g["cases"]:
        cen = np.array([g["lenses"][n][:2] for n in case["lenses"]])
        rad = np.array([g["lenses"][n][2] for n in case["lenses"]])
        got = _gpu_map(qam, np.array(case["blocks"]), cen, rad, case["f"], case["g"], case["combine"],
                       case["glass"], case["stops"])
        assert got.tolist() == case["levels"], case["name"]


def test_level_map_single_layer_workload(qam):
    inp = WL.single_layer_512x256(0)
    lp = inp["lens"]
    want = O.level_map(inp["coords"], lp.centres, lp.radii, lp.f, lp.g, lp.combine, 5, lp.glass)
    got = _gpu_map(qam, inp["coords"], lp.centres, lp.radii, lp.f, lp.g, lp.combine, lp.glass)
    assert np.array_equal(got, want)


def test_level_map_bit_exact_random_fields(qam):
    rng = np.random.default_rng(17)
    for trial in range(40):
        n = int(rng.integers(1, 5000))
        coords = rng.uniform(-0.2, 1.2, size=(n, 2)) if trial % 2 else WL.clustered_coords(rng, n)
        nl = int(rng.integers(0, 12))
        centres = coords[rng.choice(n, min(nl, n), replace=False)] if nl else np.zeros((0, 2))
        radii = rng.uniform(0.0, 0.4, size=centres.shape[0])
        n_rungs = int(rng.integers(2, 9))
        ladder = tuple(range(0, 2 * n_rungs, 2))
        glass = int(rng.integers(0, n_rungs))
        f = float(rng.choice([0.0, 1.0, rng.uniform(0, 1), 0.5]))
        g = float(rng.choice([0.0, 1.0, rng.uniform(0, 1)]))
        combine = "sum" if rng.uniform() < 0.6 else "max"
        kappa = O.ceiling(g, n_rungs - 1, glass)
        stops = None
        if kappa > glass and rng.uniform() < 0.4:
            stops = np.sort(rng.uniform(0.05, 3.0, size=kappa - glass))[::-1]
            if np.any(np.diff(stops) >= 0):
                stops = None
        want = O.level_map(coords, centres, radii, f, g, combine, n_rungs, glass, stops)
        got = _gpu_map(qam, coords, centres, radii, f, g, combine, glass, stops, ladder)
        assert np.array_equal(got, want), (trial, np.nonzero(got != want)[0][:5])


@pytest.mark.parametrize("n_lenses", [16, 33, 64])
def test_level_map_many_lenses_and_rungs(qam, n_lenses):
    """Up to the lens-table limit (a whole wavefront of lenses per block) and
    the longest ladder: every map bit-identical to the oracle, also for a
    block count that leaves a ragged last workgroup."""
    rng = np.random.default_rng(300 + n_lenses)
    for trial in range(6):
        n = int(rng.integers(1, 3000))
        coords = rng.uniform(0, 1, size=(n, 2))
        centres = rng.uniform(-0.1, 1.1, size=(n_lenses, 2))
        radii = rng.uniform(0.0, 0.2, size=n_lenses)
        n_rungs = 16 if trial % 2 == 0 else int(rng.integers(2, 16))
        ladder = tuple(range(0, 2 * n_rungs, 2))
        glass = int(rng.integers(0, n_rungs))
        f = float(rng.choice([0.0, 1.0, rng.uniform(0, 1)]))
        g = float(rng.choice([1.0, rng.uniform(0, 1)]))
        combine = "sum" if trial % 3 else "max"
        kappa = O.ceiling(g, n_rungs - 1, glass)
        stops = None
        if kappa > glass and trial % 2:
            stops = np.sort(rng.uniform(0.05, 3.0, size=kappa - glass))[::-1]
            if np.any(np.diff(stops) >= 0):
                stops = None
        want = O.level_map(coords, centres, radii, f, g, combine, n_rungs, glass, stops)
        got = _gpu_map(qam, coords, centres, radii, f, g, combine, glass, stops, ladder)
        assert np.array_equal(got, want), (trial, np.nonzero(got != want)[0][:5])


def test_level_map_bit_exact_on_ties(qam):
    """A dyadic grid puts many blocks exactly on ring stops and lens edges."""
    xs = np.arange(0, 65) / 64.0
    coords = np.array([(a, b) for a in xs for b in xs])
    centres = np.array([[0.5, 0.5], [0.25, 0.75], [0.75, 0.25]])
    for f, g, glass, combine in [(0.5, 1.0, 0, "sum"), (0.5, 0.75, 1, "sum"), (0.5, 1.0, 1, "max"),
                                 (0.2, 1.0, 0, "max"), (0.8, 0.5, 0, "sum")]:
        for radii in ([0.25, 0.125, 0.375], [0.5, 0.5, 0.5]):
            want = O.level_map(coords, centres, radii, f, g, combine, 5, glass)
            got = _gpu_map(qam, coords, centres, radii, f, g, combine, glass)
            assert np.array_equal(got, want)


def test_level_map_workload_fields(qam):
    fld = WL.e2b_field(0)
    lp = WL.e2b_lenses(fld)
    want = O.level_map(fld.coords, lp.centres, lp.radii, lp.f, lp.g, lp.combine, 5, lp.glass)
    got = _gpu_map(qam, fld.coords, lp.centres, lp.radii, lp.f, lp.g, lp.combine, lp.glass)
    assert np.array_equal(got, want)
    st = WL.streaming_stack(0)
    cen, rad = WL.stack_lenses(st)
    for glass in (0, 1):
        for f in (0.1, 0.3, 0.6):
            want = O.level_map(st.coords, cen, rad, f, 1.0, "sum", 5, glass)
            got = _gpu_map(qam, st.coords, cen, rad, f, 1.0, "sum", glass)
            assert np.array_equal(got, want)


@pytest.mark.parametrize("n_lenses", [1, 3, 9, 21])
def test_level_maps_batched_bit_exact(qam, n_lenses):
    """One map per request in one call (launches of up to 8 maps, fewer when
    their lenses fill the table), every map bit-identical to the oracle."""
    rng = np.random.default_rng(70 + n_lenses)
    n_blocks, n_maps = 700, 32
    coords = rng.uniform(0, 1, size=(n_blocks, 2))
    sets = []
    for k in range(n_maps):
        idx = rng.choice(n_blocks, n_lenses, replace=False)
        sets.append((coords[idx], rng.uniform(0.05, 0.3, size=n_lenses)))
    fs = rng.uniform(0.0, 0.95, size=n_maps)
    for combine, glass, g in (("sum", 1, 1.0), ("max", 0, 0.75)):
        got = host(qam.build_level_maps(dev(coords), sets, fs, g=g, combine=combine, glass=glass))
        for k, (c, r) in enumerate(sets):
            want = O.level_map(coords, c, r, fs[k], g, combine, 5, glass)
            assert np.array_equal(got[k], want), (k, combine)


# ------------------------------------------------------------------ qmatvec

def test_qmatvec_single_layer_workload_all_maps_sampled(qam):
    inp = WL.single_layer_512x256(0)
    W, sc, x, lp = inp["W"], inp["scales"], inp["x"], inp["lens"]
    pm = pack(qam, W, sc)
    lv = O.level_map(inp["coords"], lp.centres, lp.radii, lp.f, lp.g, lp.combine, 5, lp.glass)
    y = host(qam.qmatvec(dev(x), pm, dev(lv)))
    check_y(y, W, sc, x, lv, "lens map")
    # a per-block, per-depth table checked once; then random maps through the kernel
    rng = np.random.default_rng(0)
    xd = dev(x)
    for mp in list(rng.integers(0, 5, size=(200, 8))) + [np.full(8, d) for d in range(5)]:
        mp = mp.astype(np.uint8)
        y = host(qam.qmatvec(xd, pm, dev(mp)))
        check_y(y, W, sc, x, mp, str(mp))


@pytest.mark.parametrize("B", [1, 2, 3, 5, 6, 8])
@pytest.mark.parametrize("K", [256, 512, 1536, 2048, 8960])
@pytest.mark.parametrize("N", [128, 512, 2048])
def test_qmatvec_shape_battery(qam, N, K, B):
    rng = np.random.default_rng(N * 7 + K * 3 + B)
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    x = rng.standard_normal((B, K)).astype(np.float32)
    lv = rng.integers(0, 5, size=N // 64).astype(np.uint8)
    pm = pack(qam, W, sc)
    y = host(qam.qmatvec(dev(x), pm, dev(lv)))
    assert ("qmatvec_staged" if B == 1 else "qmatvec_mfma") in qam.last_variant()
    check_y(y, W, sc, x, lv, (N, K, B))
    # the same map given once per request: at B = 1 the same route and bits;
    # above, the per-request form, whose column chunks can differ from the
    # shared form's (x is split into fixed point per chunk), so it meets the
    # same bound rather than the same bits
    lvr = np.ascontiguousarray(np.broadcast_to(lv, (B, lv.size)))
    yr = host(qam.qmatvec(dev(x), pm, dev(lvr)))
    if B == 1:
        assert np.array_equal(yr.view(np.uint32), y.view(np.uint32)), (N, K, B)
    check_y(yr, W, sc, x, lv, (N, K, B, "per-request"))


def test_qmatvec_exact_integer_cases(qam):
    """Integer x in [-3, 3] with scale 1: y is an exact integer; a D8 map is
    the untruncated int8 product (numpy int64, bit-exact)."""
    rng = np.random.default_rng(21)
    for N, K, B in [(512, 256, 1), (256, 8192, 2), (128, 28672, 1), (64, 65536, 1)]:
        W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        x = rng.integers(-3, 4, size=(B, K)).astype(np.float32)
        pm = pack(qam, W, np.ones(N, np.float32))
        for lv in (np.full(N // 64, 4, np.uint8), rng.integers(0, 5, N // 64).astype(np.uint8)):
            y = host(qam.qmatvec(dev(x), pm, dev(lv)))
            codes = np.concatenate([O.truncate(W[64 * b:64 * b + 64], LADDER[lv[b]]) for b in range(N // 64)])
            want = x.astype(np.int64) @ codes.T
            assert np.array_equal(y.astype(np.int64), want)
            assert np.all(np.abs(want) < 2 ** 24)


def test_qmatvec_large_integer_x_rounds_once(qam):
    """Integer x up to 2^21 in magnitude sits on the fixed-point grid exactly,
    so the only rounding is the final fp32 one: y == fl32(exact int64 sum)."""
    rng = np.random.default_rng(22)
    for N, K, B in [(256, 4096, 1), (128, 1600 - 1600 % 64, 3), (64, 12288, 8)]:
        W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        x = rng.integers(-(2 ** 21), 2 ** 21, size=(B, K)).astype(np.float32)
        x[:, 0] = -(2 ** 21)
        pm = pack(qam, W, np.ones(N, np.float32))
        lv = rng.integers(0, 5, N // 64).astype(np.uint8)
        lv[0] = 4
        y = host(qam.qmatvec(dev(x), pm, dev(lv)))
        codes = np.concatenate([O.truncate(W[64 * b:64 * b + 64], LADDER[lv[b]]) for b in range(N // 64)])
        want = (x.astype(np.int64) @ codes.T).astype(np.float32)
        assert np.array_equal(y, want), (N, K, B)


def test_qmatvec_edge_cases(qam):
    rng = np.random.default_rng(4)
    N, K = 256, 1024
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    W[0, :] = -128
    W[1, :] = 127
    W[2, :] = -127
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    sc[3] = 0.0
    x = rng.standard_normal((1, K)).astype(np.float32)
    pm = pack(qam, W, sc)
    for lv in (np.zeros(4, np.uint8), np.full(4, 4, np.uint8), np.array([1, 0, 4, 2], np.uint8)):
        y = host(qam.qmatvec(dev(x), pm, dev(lv)))
        check_y(y, W, sc, x, lv, lv)
    y = host(qam.qmatvec(dev(x), pm, dev(np.full(4, 3, np.uint8))))
    assert y[0, 3] == 0.0
    # x all zero gives exact zeros
    y = host(qam.qmatvec(dev(np.zeros((1, K), np.float32)), pm, dev(np.full(4, 4, np.uint8))))
    assert np.all(y == 0.0)
    # wide dynamic range of x (six decades) still meets the bound
    xr = (rng.choice([-1, 1], size=(2, K)) * 10.0 ** rng.uniform(-3, 3, size=(2, K))).astype(np.float32)
    lv = rng.integers(1, 5, 4).astype(np.uint8)
    y = host(qam.qmatvec(dev(xr), pm, dev(lv)))
    check_y(y, W, sc, xr, lv, "dynamic range")
    # a non-finite x poisons that request's non-ZERO outputs with NaN
    xn = x.copy()
    xn[0, 5] = np.inf
    y = host(qam.qmatvec(dev(xn), pm, dev(np.array([0, 4, 4, 4], np.uint8))))
    assert np.all(y[0, :64] == 0.0) and np.all(np.isnan(y[0, 64:]))


def test_qmatvec_bf16_activations(qam):
    rng = np.random.default_rng(5)
    N, K = 512, 2048
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    xb = torch.randn(2, K, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    x32 = xb.float().numpy()
    lv = rng.integers(0, 5, N // 64).astype(np.uint8)
    pm = pack(qam, W, sc)
    y = host(qam.qmatvec(xb.cuda(), pm, dev(lv)))
    check_y(y, W, sc, x32, lv, "bf16")


def test_qmatvec_deterministic_and_leaves_workspace_clean(qam):
    rng = np.random.default_rng(6)
    N, K = 2048, 28672
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    x = rng.standard_normal((1, K)).astype(np.float32)
    lv = rng.integers(0, 5, N // 64).astype(np.uint8)
    pm = pack(qam, W, sc)
    ws = qam.Workspace("cuda")
    xd, lvd = dev(x), dev(lv)
    y1 = host(qam.qmatvec(xd, pm, lvd, workspace=ws))
    y2 = host(qam.qmatvec(xd, pm, lvd, workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert int(np.abs(host(ws.buf[:4 * 65536].view(torch.int32))).sum()) == 0   # counters reset
    check_y(y1, W, sc, x, lv, "28672")


def test_qmatvec_one_workspace_across_shapes(qam):
    """Calls of different shapes share one workspace: the partials one call
    leaves behind never disturb the next call's arrival counters."""
    rng = np.random.default_rng(12)
    ws = qam.Workspace("cuda")
    for N, K, B in [(2048, 8960, 8), (8192, 4096, 1), (128, 8960, 3), (4096, 28672, 1), (64, 65536, 1),
                    (2048, 8960, 8)]:
        W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
        x = rng.standard_normal((B, K)).astype(np.float32)
        lv = rng.integers(0, 5, N // 64).astype(np.uint8)
        y = host(qam.qmatvec(dev(x), pack(qam, W, sc), dev(lv), workspace=ws))
        check_y(y, W, sc, x, lv, (N, K, B))
        assert int(np.abs(host(ws.buf[:4 * 65536].view(torch.int32))).sum()) == 0


def test_qmatvec_full_size_streaming_layer_sampled_rows(qam):
    """8192 x 28672 and 28672 x 8192 at a lens map near 4 bits, in the launch
    configuration the benchmark uses; 384 sampled rows against the oracle."""
    st = WL.streaming_stack(0)
    cen, rad = WL.stack_lenses(st)
    lv_all = O.level_map(st.coords, cen, rad, 0.3, 1.0, "sum", 5, 1)
    offs = st.block_offsets()
    rng = np.random.default_rng(8)
    for i in (0, 1):
        m = st.matrices[i]
        W = st.codes(i)
        sc = st.scales(i)
        x = st.x(i)
        lv = lv_all[offs[i]:offs[i] + m.n_blocks]
        pm = pack(qam, W, sc)
        y = host(qam.qmatvec(dev(x), pm, dev(lv)))
        rows = np.sort(rng.choice(m.N, 384, replace=False))
        Wr = W[rows]
        # oracle on the sampled rows only: each row keeps its own block's depth
        codes = np.stack([O.truncate(Wr[j], LADDER[lv[r // 64]]) for j, r in enumerate(rows)])
        ref = (codes.astype(np.float64) @ x[0].astype(np.float64)) * sc[rows].astype(np.float64)
        tol = 1e-4 * (np.abs(codes).astype(np.float64) @ np.abs(x[0]).astype(np.float64)) * sc[rows]
        err = np.abs(y[0, rows].astype(np.float64) - ref)
        assert np.all(err <= tol), (i, float((err / np.maximum(tol, 1e-300)).max()))
        del pm
        torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 2])
def test_grouped_qmatvec_matches_oracle(qam, B):
    """Several matrices with their own x, y and maps in one launch."""
    rng = np.random.default_rng(30 + B)
    shapes = [(1536, 1536), (6144, 1536), (1536, 6144), (64, 28672), (128, 256), (512, 8960)]
    items, host_in = [], []
    for i, (N, K) in enumerate(shapes):
        W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
        x = rng.standard_normal((B, K)).astype(np.float32)
        lv = (np.zeros(N // 64) if i == 4 else rng.integers(0, 5, N // 64)).astype(np.uint8)
        y = torch.full((B, N), float("nan"), device="cuda")
        items.append((pack(qam, W, sc), dev(x), y, dev(lv)))
        host_in.append((W, sc, x, lv))
    grp = qam.GroupedQmatvec(items)
    grp.run()
    first = [host(it[2]).copy() for it in items]
    for (W, sc, x, lv), y in zip(host_in, first):
        check_y(y, W, sc, x, lv, W.shape)
    grp.run()
    for it, y0 in zip(items, first):
        assert np.array_equal(host(it[2]).view(np.uint32), y0.view(np.uint32))


def _lens_field(rng, shapes, B, bf16=False):
    """A small field of matrices with block coordinates and random lenses."""
    n_blocks = sum(N // 64 for N, _ in shapes)
    coords = WL.clustered_coords(rng, n_blocks) if n_blocks > 8 else rng.uniform(0, 1, size=(n_blocks, 2))
    mats = []
    for N, K in shapes:
        W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
        x = rng.standard_normal((B, K)).astype(np.float32)
        if bf16:
            x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        mats.append((W, sc, x))
    return coords, mats


def _lens_group(qam, coords, mats, bf16=False):
    cd = dev(coords)
    lv = torch.full((coords.shape[0],), 0xEE, dtype=torch.uint8, device="cuda")   # stale: every rung is written
    items, o = [], 0
    for W, sc, x in mats:
        N = W.shape[0]
        xt = dev(x).to(torch.bfloat16) if bf16 else dev(x)
        y = torch.full((x.shape[0], N), float("nan"), device="cuda")
        items.append((pack(qam, W, sc), xt, y, lv[o:o + N // 64], cd[o:o + N // 64]))
        o += N // 64
    return qam.GroupedQmatvec(items), items, lv, cd


@pytest.mark.parametrize("B,bf16", [(1, False), (1, True)])
def test_group_lens_builds_the_maps_in_the_launch(qam, B, bf16):
    """The launch that builds the level maps writes every item's map
    bit-identical to the oracle's lens rules over the whole field, and its
    outputs are bit-identical to the map launch followed by the plain grouped
    product (hence within the tolerance of the oracle)."""
    rng = np.random.default_rng(500 + B + 10 * bf16)
    shapes = [(1536, 1536), (6144, 1536), (1536, 6144), (64, 28672), (128, 256), (512, 8960), (192, 64)]
    coords, mats = _lens_field(rng, shapes, B, bf16)
    grp, items, lv, cd = _lens_group(qam, coords, mats, bf16)
    assert grp.route == "staged"
    for trial, (n_lenses, f, g, combine, glass) in enumerate(
            [(5, 0.5, 0.75, "sum", 1), (9, 0.35, 1.0, "max", 0), (1, 1.0, 1.0, "sum", 2), (0, 0.5, 1.0, "sum", 3),
             (64, 0.1, 1.0, "sum", 0), (3, 0.0, 1.0, "sum", 1), (4, 0.6, 0.0, "sum", 2)]):
        cen = coords[rng.choice(coords.shape[0], n_lenses, replace=False)].copy()
        rad = rng.uniform(0.02, 0.4, size=n_lenses)
        if trial == 5:
            rad[0] = 0.0
            cen[0] = coords[7]          # radius 0: lifts only the block at its centre
        rules = qam.LensRules(cen, rad, f, g, combine, glass)
        want_map = O.level_map(coords, cen, rad, f, g, combine, 5, glass)
        lv.fill_(0xEE)
        grp.run_lens(rules)
        assert "group_lens" in qam.last_variant()
        assert np.array_equal(host(lv), want_map), trial
        fused = [host(it[2]).copy() for it in items]
        lv.fill_(0xEE)
        qam.build_level_map(cd, cen, rad, f, g, combine, glass, out=lv)
        grp.run()
        o = 0
        for (W, sc, x), it, yf in zip(mats, items, fused):
            N = W.shape[0]
            y = host(it[2])
            assert np.array_equal(y.view(np.uint32), yf.view(np.uint32)), (trial, W.shape)
            check_y(yf, W, sc, x, want_map[o:o + N // 64], (trial, W.shape))
            o += N // 64


def test_group_lens_needs_coordinates_and_the_staged_route(qam):
    rng = np.random.default_rng(520)
    coords, mats = _lens_field(rng, [(256, 512), (128, 256)], 1)
    cd = dev(coords)
    lv = torch.zeros(coords.shape[0], dtype=torch.uint8, device="cuda")
    W, sc, x = mats[0]
    no_coords = qam.GroupedQmatvec([(pack(qam, W, sc), dev(x), torch.empty((1, 256), device="cuda"), lv[:4])])
    rules = qam.LensRules(coords[:2], [0.2, 0.3], 0.5, 1.0)
    with pytest.raises(qam.QamError):
        no_coords.run_lens(rules)
    x3 = dev(np.repeat(x, 3, axis=0))
    pre = qam.GroupedQmatvec([(pack(qam, W, sc), x3, torch.empty((3, 256), device="cuda"), lv[:4], cd[:4])])
    assert pre.route == "prepass"
    with pytest.raises(qam.QamError):
        pre.run_lens(rules)
    ok = qam.GroupedQmatvec([(pack(qam, W, sc), dev(x), torch.empty((1, 256), device="cuda"), lv[:4], cd[:4])])
    with pytest.raises(qam.QamError):
        ok.run_lens(qam.LensRules(coords[:2], [0.2, 0.3], 0.5, 1.0, ladder_bits=(0, 2, 4, 8)))
    ok.run_lens(rules)
    assert np.array_equal(host(lv[:4]), O.level_map(coords[:4], coords[:2], [0.2, 0.3], 0.5, 1.0, "sum", 5, 1))


def test_graph_replays_match_eager(qam):
    """A captured step (level map + grouped product + a split-K single product)
    replayed several times, with eager work and synchronisations between the
    replays, gives exactly the eager result every time."""
    rng = np.random.default_rng(40)
    coords = rng.uniform(0, 1, size=(2 * 24 + 16, 2))
    cen, rad = coords[[3, 40]], np.array([0.2, 0.3])
    cd = dev(coords)
    lv = qam.build_level_map(cd, cen, rad, 0.6, 1.0, "sum", 1)
    mats = [(1536, 1536), (1536, 6144), (1024, 28672)]
    items, offs, o = [], [], 0
    for N, K in mats:
        W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
        x = dev(rng.standard_normal((1, K)).astype(np.float32))
        items.append((pack(qam, W, sc), x, torch.empty((1, N), device="cuda"), lv[o:o + N // 64]))
        o += N // 64
    grp = qam.GroupedQmatvec(items[:2])
    single = items[2]
    ws = qam.Workspace("cuda")
    y_single = torch.empty((1, 1024), device="cuda")

    def step():
        qam.build_level_map(cd, cen, rad, 0.6, 1.0, "sum", 1, out=lv)
        grp.run()
        qam.qmatvec(single[1], single[0], single[3], y=y_single, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = [host(it[2]).copy() for it in items[:2]] + [host(y_single).copy()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for it in items[:2]:
            it[2].fill_(float("nan"))
        y_single.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(it[2]) for it in items[:2]] + [host(y_single)]
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), rep
        step()                                 # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("scale", [1e-30, 1e-36, 1e-40, 1e30])
@pytest.mark.parametrize("B", [1, 4])
def test_qmatvec_extreme_magnitudes(qam, scale, B):
    """x far from 1 (down to the subnormal range, where 2^sh no longer fits a
    normal float, and near the top of the range) on both routes."""
    rng = np.random.default_rng(int(-np.log10(scale) * 10) + B if scale < 1 else B)
    N, K = 256, 2048
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    x = (rng.standard_normal((B, K)) * scale).astype(np.float32)
    lv = np.array([1, 2, 3, 4], np.uint8)
    pm = pack(qam, W, sc)
    y = host(qam.qmatvec(dev(x), pm, dev(lv)))
    check_y(y, W, sc, x, lv, (scale, B))


# ------------------------------------------------------------------ zone radius

def test_field_width_bit_exact(qam):
    """The field width on the device equals the oracle's, bit for bit."""
    rng = np.random.default_rng(800)
    for n in (1, 2, 7, 300, 4608):
        c = rng.uniform(-1, 2, size=(n, 2))
        assert qam.field_width(dev(c)) == O.field_width(c), n
    fld = WL.e2b_field(0)
    assert qam.field_width(dev(fld.coords)) == O.field_width(fld.coords)


def test_zone_radius_maps_bit_exact(qam):
    """Level maps with the zone radius R = f D: the hand examples, and random
    and workload fields at every kind of f, bit-identical to the oracle."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "zone_hand_examples.json")))
    c = np.array(g["coords"])
    for f, want in g["maps"].items():
        got = host(qam.build_level_map(dev(c), [g["centre"]], [0.123], float(f), g["g"], "sum", g["glass"],
                                       radius="zone", width=g["width"]))
        assert got.tolist() == want, f
    rng = np.random.default_rng(801)
    for trial in range(12):
        n = int(rng.integers(1, 4000))
        coords = rng.uniform(0, 1, size=(n, 2)) if trial % 2 else WL.clustered_coords(rng, n)
        D = qam.field_width(dev(coords))
        nl = int(rng.integers(0, 9))
        cen = coords[rng.choice(n, min(nl, n), replace=False)] if nl else np.zeros((0, 2))
        rad = rng.uniform(0.0, 0.4, size=cen.shape[0])
        f = float(rng.choice([0.0, 1.0, rng.uniform(0, 1)]))
        gg = float(rng.choice([1.0, 0.75, rng.uniform(0, 1)]))
        glass = int(rng.integers(0, 5))
        combine = "sum" if trial % 3 else "max"
        want = O.level_map(coords, cen, rad, f, gg, combine, 5, glass, radius="zone", width=D)
        got = host(qam.build_level_map(dev(coords), cen, rad, f, gg, combine, glass, radius="zone", width=D))
        assert np.array_equal(got, want), trial
    # the E2B-shaped field, one map rule set per f; the launch that builds the
    # map inside the product takes the zone rule too
    fld = WL.e2b_field(0)
    lp = WL.e2b_lenses(fld)
    D = qam.field_width(dev(fld.coords))
    for f in (0.0, 0.05, 0.2, 1.0):
        want = O.level_map(fld.coords, lp.centres, lp.radii, f, lp.g, "sum", 5, 1, radius="zone", width=D)
        got = host(qam.build_level_map(dev(fld.coords), lp.centres, lp.radii, f, lp.g, "sum", 1,
                                       radius="zone", width=D))
        assert np.array_equal(got, want), f
    rng2 = np.random.default_rng(802)
    shapes = [(256, 512), (192, 1024), (128, 256)]
    coords, mats = _lens_field(rng2, shapes, 1)
    grp, items, lv, cd = _lens_group(qam, coords, mats)
    D = qam.field_width(cd)
    cen = coords[[1, 5]]
    rules = qam.LensRules(cen, [0.3, 0.1], 0.4, 1.0, "sum", 1, radius="zone", width=D)
    grp.run_lens(rules)
    want = O.level_map(coords, cen, [0.3, 0.1], 0.4, 1.0, "sum", 5, 1, radius="zone", width=D)
    assert np.array_equal(host(lv), want)
    o = 0
    for (W, sc, x), it in zip(mats, items):
        N = W.shape[0]
        check_y(host(it[2]), W, sc, x, want[o:o + N // 64], ("zone", W.shape))
        o += N // 64

"""GPU parity of the pre-pass route (batches up to 32, shared or
per-request level maps) against the CPU oracle, through the C ABI."""

import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
LADDER = (0, 2, 4, 6, 8)
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(y, W, sc, x, lv, per_request, what):
    ref = O.qmatvec_ref(W, sc, x, lv, per_request=per_request)
    tol = O.qmatvec_tolerance(W, sc, x, lv, per_request=per_request)
    err = np.abs(y.astype(np.float64) - ref)
    bad = ~(err <= tol)
    assert not bad.any(), (what, int(bad.sum()), float(np.nanmax(err / np.maximum(tol, 1e-300))))
    B = x.shape[0]
    lvb = np.broadcast_to(np.asarray(lv).reshape(-1 if per_request else 1, W.shape[0] // 64), (B, W.shape[0] // 64))
    zero = np.repeat(lvb == 0, 64, axis=1)
    assert np.all(y[zero] == 0.0), what


def problem(seed, N, K, B):
    rng = np.random.default_rng(seed)
    W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    x = rng.standard_normal((B, K)).astype(np.float32)
    return rng, W, sc, x


@pytest.mark.parametrize("B", [2, 5, 16, 17, 32])
@pytest.mark.parametrize("N,K", [(128, 256), (512, 1536), (256, 8960), (1024, 4096)])
def test_per_request_maps(qam, N, K, B):
    rng, W, sc, x = problem(N + K + B, N, K, B)
    lv = rng.integers(0, 5, size=(B, N // 64)).astype(np.uint8)
    lv[:, 0] = 0            # a block nobody reads
    lv[0, -1] = 4           # requests at every depth in one block
    pm = qam.pack_slices(dev(W), dev(sc))
    y = host(qam.qmatvec(dev(x), pm, dev(lv)))
    assert "mfma" in qam.last_variant() and "per-request" in qam.last_variant()
    check(y, W, sc, x, lv, True, (N, K, B))


@pytest.mark.parametrize("B", [4, 8, 9, 16, 24, 32])
@pytest.mark.parametrize("N,K", [(192, 512), (512, 6144), (128, 28672)])
def test_shared_map_on_matrix_cores(qam, N, K, B):
    rng, W, sc, x = problem(N * 3 + K + B, N, K, B)
    lv = rng.integers(0, 5, size=N // 64).astype(np.uint8)
    pm = qam.pack_slices(dev(W), dev(sc))
    y = host(qam.qmatvec(dev(x), pm, dev(lv)))
    assert "mfma" in qam.last_variant() and "shared" in qam.last_variant()
    check(y, W, sc, x, lv, False, (N, K, B))


def test_per_request_exact_integers(qam):
    """Integer x, unit scales: every request's output is the exact int64
    product with its own truncated codes."""
    rng = np.random.default_rng(31)
    for N, K, B in [(256, 2048, 32), (128, 8192, 7), (64, 65536, 3)]:
        W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        x = rng.integers(-3, 4, size=(B, K)).astype(np.float32)
        lv = rng.integers(0, 5, size=(B, N // 64)).astype(np.uint8)
        pm = qam.pack_slices(dev(W), dev(np.ones(N, np.float32)))
        y = host(qam.qmatvec(dev(x), pm, dev(lv)))
        for r in range(B):
            codes = np.concatenate([O.truncate(W[64 * b:64 * b + 64], LADDER[lv[r, b]]) for b in range(N // 64)])
            assert np.array_equal(y[r].astype(np.int64), codes @ x[r].astype(np.int64)), (N, K, B, r)


def test_per_request_equals_single_requests(qam):
    """Request r of a per-request batch gives exactly what a batch of one with
    map r gives, up to the rounding the tolerance allows; with integer x both
    are exact, so they agree bit for bit."""
    rng = np.random.default_rng(32)
    N, K, B = 512, 4096, 16
    W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    x = rng.integers(-100, 101, size=(B, K)).astype(np.float32)
    sc = np.ones(N, np.float32)
    lv = rng.integers(0, 5, size=(B, N // 64)).astype(np.uint8)
    pm = qam.pack_slices(dev(W), dev(sc))
    yb = host(qam.qmatvec(dev(x), pm, dev(lv)))
    for r in range(B):
        y1 = host(qam.qmatvec(dev(x[r:r + 1]), pm, dev(lv[r])))
        assert np.array_equal(yb[r], y1[0]), r


def test_matrix_cores_bf16_and_nonfinite(qam):
    rng, W, sc, x = problem(33, 256, 3072, 20)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    lv = rng.integers(1, 5, size=(20, 4)).astype(np.uint8)
    lv[3, 2] = 0
    pm = qam.pack_slices(dev(W), dev(sc))
    y = host(qam.qmatvec(xb.cuda(), pm, dev(lv)))
    check(y, W, sc, xb.float().numpy(), lv, True, "bf16")
    xn = x.copy()
    xn[3, 100] = np.inf
    y = host(qam.qmatvec(dev(xn), pm, dev(lv)))
    assert np.all(np.isnan(y[3, :128])) and np.all(y[3, 128:192] == 0.0) and np.all(np.isnan(y[3, 192:]))
    ok = np.delete(np.arange(20), 3)
    check(y[ok], W, sc, x[ok], lv[ok], True, "other requests")


def test_matrix_core_route_is_deterministic_and_shares_a_workspace(qam):
    ws = qam.Workspace()
    outs = []
    for N, K, B in [(2048, 4096, 32), (256, 1024, 16), (2048, 4096, 32), (64, 14336, 8)]:
        rng, W, sc, x = problem(N + K, N, K, B)
        lv = rng.integers(0, 5, size=(B, N // 64)).astype(np.uint8)
        pm = qam.pack_slices(dev(W), dev(sc))
        y = host(qam.qmatvec(dev(x), pm, dev(lv), workspace=ws))
        check(y, W, sc, x, lv, True, (N, K, B))
        outs.append(y)
    assert np.array_equal(outs[0], outs[2])
    assert not host(ws.buf[:4 * 65536]).any()   # the counters are left zero


def test_batched_layer_workload(qam):
    """The batched multi-request layer (4096x4096, 14336x4096, 4096x14336),
    B = 32 requests, each with its own map from 3 lenses built on the GPU;
    outputs checked on sampled blocks against the oracle."""
    cal = json.load(open(os.path.join(HERE, "golden", "calibration.json")))["batched_layer"]
    fld = WL.batched_layer(0)
    B = 32
    reqs = WL.request_lenses(fld, B)
    coords = dev(fld.coords)
    maps = torch.empty((B, fld.n_blocks), dtype=torch.uint8, device="cuda")
    for r, (c, rr) in enumerate(reqs):
        qam.build_level_map(coords, c, rr, cal["requests"][r]["f"], 1.0, "sum", 1, out=maps[r])
    lv_all = host(maps)
    for r, (c, rr) in enumerate(reqs):
        assert np.array_equal(lv_all[r], O.level_map(fld.coords, c, rr, cal["requests"][r]["f"], 1.0, "sum", 5, 1))
    offs = fld.block_offsets()
    rng = np.random.default_rng(0)
    for i, m in enumerate(fld.matrices):
        W, sc, x = fld.codes(i), fld.scales(i), fld.x(i, B)
        pm = qam.pack_slices(dev(W), dev(sc))
        lv = np.ascontiguousarray(lv_all[:, offs[i]:offs[i] + m.n_blocks])
        y = host(qam.qmatvec(dev(x), pm, dev(lv)))
        blocks = np.sort(rng.choice(m.n_blocks, 12, replace=False))
        rows = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
        check(y[:, rows], W[rows], sc[rows], x, lv[:, blocks], True, m.name)


@pytest.mark.parametrize("B,per_request", [(16, True), (32, True), (8, False), (3, True)])
def test_grouped_matrix_cores(qam, B, per_request):
    """Several matrices in one grouped launch (pre-pass + product), each
    checked against the oracle; replays of a captured group agree bit for bit."""
    rng = np.random.default_rng(40 + B)
    shapes = [(256, 1024), (512, 4096), (128, 14336), (64, 64)]
    mats, items = [], []
    for N, K in shapes:
        W = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
        x = rng.standard_normal((B, K)).astype(np.float32)
        lv = rng.integers(0, 5, size=(B, N // 64) if per_request else N // 64).astype(np.uint8)
        pm = qam.pack_slices(dev(W), dev(sc))
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        mats.append((W, sc, x, lv))
        items.append((pm, dev(x), y, dev(lv)))
    g = qam.GroupedQmatvec(items)
    assert g.route == "prepass"
    g.run()
    first = [host(it[2]).copy() for it in items]
    for (W, sc, x, lv), y in zip(mats, first):
        check(y, W, sc, x, lv, per_request, (W.shape, B))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.run()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run()
    for rep in range(3):
        for it in items:
            it[2].fill_(float("nan"))
        graph.replay()
        for it, want in zip(items, first):
            assert np.array_equal(host(it[2]), want), rep
        qam.qmatvec(items[0][1], items[0][0], items[0][3])   # eager work between replays


@pytest.mark.parametrize("set_max", [8, 10, 13])
def test_request_set_sizes(qam, set_max):
    """Requests split into sets of at most `set_max` (fewer limb columns per
    set), a group's own launch plan: the same bits as sets of 16 with the
    same column chunks, and the oracle's values; groups built with other
    plans keep their own."""
    for B, per_request in ((16, True), (20, True), (32, True), (24, False)):
        rng, W, sc, x = problem(900 + B + set_max, 512, 4096, B)
        lv = rng.integers(0, 5, size=(B, 8) if per_request else 8).astype(np.uint8)
        pm = qam.pack_slices(dev(W), dev(sc))
        xd, lvd = dev(x), dev(lv)
        y16 = torch.full((B, 512), float("nan"), device="cuda")
        g16 = qam.GroupedQmatvec([(pm, xd, y16, lvd)], tuning={"tiles_per_request": 4})
        ys = torch.full((B, 512), float("nan"), device="cuda")
        gs = qam.GroupedQmatvec([(pm, xd, ys, lvd)], tuning={"tiles_per_request": 4, "set_max": set_max})
        assert g16.desc.sets == -(-B // 16) and gs.desc.sets == -(-B // set_max)
        gs.run()
        assert f"sets={-(-B // set_max)}" in qam.last_variant(), qam.last_variant()
        g16.run()
        assert f"sets={-(-B // 16)}" in qam.last_variant(), qam.last_variant()
        a, b = host(ys), host(y16)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (B, set_max)
        check(a, W, sc, x, lv, per_request, (B, set_max))
        gs.run()   # still its own plan, whatever ran in between
        assert np.array_equal(host(ys).view(np.uint32), b.view(np.uint32)), (B, set_max, "again")


@pytest.mark.parametrize("tuning", [{"ksplit": 1}, {"ksplit": 2}, {"target_waves": 2048},
                                    {"tiles_per_request": 64}])
def test_group_plans_give_oracle_values(qam, tuning):
    """Other launch plans (waves per set, launch width, chunk length) on a
    per-request batch still give the oracle's values."""
    rng, W, sc, x = problem(1300 + len(str(tuning)), 768, 6144, 16)
    lv = rng.integers(0, 5, size=(16, 12)).astype(np.uint8)
    lv[:, 1] = 0
    pm = qam.pack_slices(dev(W), dev(sc))
    y = torch.full((16, 768), float("nan"), device="cuda")
    g = qam.GroupedQmatvec([(pm, dev(x), y, dev(lv))], tuning=tuning)
    g.run()
    if "ksplit" in tuning:
        assert g.desc.ksplit == tuning["ksplit"]
    check(host(y), W, sc, x, lv, True, tuning)

"""GPU parity of the layer-decides level maps (FoQLens, "FoQZones, the
mechanism", the variant in which the layer decides) against the CPU oracle,
through the C ABI: the reduced draft scores and both rules bit for bit on the
same seeded base outputs, then the whole layer (base product, levels,
product at the levels) against the oracle's product, its maps checked
against the oracle's score bounds."""

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TAG = 9100


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def packed(qam, seed, N, K):
    W = WL.int8_codes(WL.stream(seed, TAG, 0), N, K)
    sc = WL.row_scales(WL.stream(seed, TAG, 1), N)
    return W, sc, qam.pack_slices(dev(W), dev(sc))


def base_outputs(seed, B, N, spread=4.0):
    """fp32 [B, N]: normal values with a per-block magnitude spread over a few
    powers of 16, so the scores fall on several rungs."""
    rng = WL.stream(seed, TAG, 2)
    y = WL.activations(rng, B, N)
    mag = np.exp2(rng.uniform(-spread, spread, (B, N // 64))).astype(np.float32)
    return (y.reshape(B, N // 64, 64) * mag[:, :, None]).reshape(B, N)


def device_levels(qam, y, pm, rule):
    lv, sh = qam.layer_levels(dev(y), pm, rule)
    torch.cuda.synchronize()
    return lv.cpu().numpy(), sh.cpu().numpy()


@pytest.mark.parametrize("B,N,K", [(1, 64, 64), (3, 64 * 37, 128), (32, 64 * 300, 4096), (5, 64 * 1000, 64),
                                   (2, 64 * 4099, 256)])
def test_scores_and_threshold_levels_bit_exact(qam, B, N, K):
    _, sc, pm = packed(qam, N + K, N, K)
    y = base_outputs(B + N, B, N)
    want_s = O.layer_scores(y, sc, K)
    med = float(np.median(want_s))
    for glass, g, lam in ((1, 1.0, med / 16), (0, 1.0, med / 256), (2, 0.5, med), (1, 0.75, want_s.flat[0] / 16),
                          (1, 1.0, 0.0), (1, 1.0, np.inf), (1, 1.0, -1.0)):
        lv, sh = device_levels(qam, y, pm, qam.LayerRule(lam=lam, g=g, glass=glass))
        assert np.array_equal(sh, want_s), (glass, g, lam)
        want = O.layer_levels_threshold(want_s, 5, glass, g, lam)
        assert np.array_equal(lv, want), (glass, g, lam, np.bincount(lv.ravel()), np.bincount(want.ravel()))
    assert len(np.unique(O.layer_levels_threshold(want_s, 5, 1, 1.0, med / 16))) >= min(3, want_s.size)


@pytest.mark.parametrize("B,nb", [(1, 1), (4, 77), (32, 300), (1, 512), (2, 513), (2, 2374), (3, 1000), (1, 16384)])
def test_share_levels_bit_exact_with_ties_and_nan(qam, B, nb):
    N, K = 64 * nb, 128
    _, sc, pm = packed(qam, nb, N, K)
    y = base_outputs(nb, B, N)
    y3 = y.reshape(B, nb, 64)
    if nb > 4:
        y3[:, 3] = y3[:, 1]                               # equal scores when the scales agree too
        y3[0, 2, 5] = np.nan                              # a NaN score never rises
    y = y3.reshape(B, N)
    sc3 = sc.reshape(nb, 64)
    if nb > 4:
        sc3[3] = sc3[1]
    sc = sc3.reshape(N)
    pm = qam.pack_slices(dev(WL.int8_codes(WL.stream(nb, TAG, 0), N, K)), dev(sc))
    want_s = O.layer_scores(y, sc, K)
    for f, g, glass in ((0.0, 1.0, 1), (0.1, 1.0, 1), (0.5, 0.5, 1), (0.999, 1.0, 0), (1.0, 1.0, 2)):
        lv, sh = device_levels(qam, y, pm, qam.LayerRule(share=f, g=g, glass=glass))
        assert np.array_equal(sh, want_s, equal_nan=True)
        want = O.layer_levels_share(want_s, 5, glass, g, f)
        assert np.array_equal(lv, want), (f, g, glass)


def test_all_equal_scores_rise_in_block_order(qam):
    nb, K = 513, 64
    N = 64 * nb
    pm = qam.pack_slices(dev(np.ones((N, K), np.int8)), dev(np.full(N, 0.01, np.float32)))
    y = np.ones((2, N), np.float32)
    lv, _ = device_levels(qam, y, pm, qam.LayerRule(share=0.25, glass=1))
    k = int(np.floor(0.25 * nb))
    assert np.array_equal(lv[0], np.r_[np.full(k, 4), np.full(nb - k, 1)].astype(np.uint8))
    assert np.array_equal(lv[1], lv[0])


def score_bounds(y_ref, tol, sc, K):
    """The oracle's scores at the ends of each output's tolerance interval:
    a device output within tol of y_ref gives a score between these."""
    lo = np.maximum(np.abs(y_ref) - tol, 0.0)
    hi = np.abs(y_ref) + tol
    return O.layer_scores(lo, sc, K), O.layer_scores(hi, sc, K)


@pytest.mark.parametrize("B", [1, 4, 32])
def test_layer_decides_end_to_end(qam, B):
    """Base product at the glass, levels on the device, product at the levels:
    each block's rung lies between the oracle's rungs at its score bounds (and
    equals them where they agree); the output matches the oracle's product
    with that map."""
    N, K = 64 * 96, 1024
    W, sc, pm = packed(qam, 77, N, K)
    x = WL.activations(WL.stream(77, TAG, 3), B, K)
    glass = 1
    ld = None
    y_ref = O.qmatvec_ref(W, sc, x, np.full(N // 64, glass, np.uint8))
    tol = O.qmatvec_tolerance(W, sc, x, np.full(N // 64, glass, np.uint8))
    s_lo, s_hi = score_bounds(y_ref, tol, sc, K)
    med = float(np.median(O.layer_scores(y_ref, sc, K)))
    for rule_kw in (dict(lam=med / 16), dict(lam=med / 300), dict(share=0.3)):
        rule = qam.LayerRule(glass=glass, **rule_kw)
        ld = qam.LayerDecides(pm, B, rule)
        y = ld.run(dev(x)).cpu().numpy()
        lv = ld.levels.cpu().numpy()
        if "lam" in rule_kw:
            a = O.layer_levels_threshold(s_lo, 5, glass, 1.0, rule_kw["lam"])
            b = O.layer_levels_threshold(s_hi, 5, glass, 1.0, rule_kw["lam"])
            assert np.all((a <= lv) & (lv <= b)), rule_kw
            assert np.mean(a == b) > 0.9
        else:
            k = int(np.floor(0.3 * (N // 64)))
            for r in range(B):
                risen, stay = lv[r] == 4, lv[r] == glass
                assert risen.sum() == k and (risen | stay).all()
                assert s_hi[r][risen].min() >= s_lo[r][stay].max()
        ref = O.qmatvec_ref(W, sc, x, lv, per_request=True)
        err = np.abs(y.astype(np.float64) - ref)
        assert np.all(err <= O.qmatvec_tolerance(W, sc, x, lv, per_request=True)), rule_kw


@pytest.mark.parametrize("B,refine", [(1, False), (2, True), (8, False), (8, True), (3, True), (32, True)])
def test_layer_decides_group(qam, B, refine):
    """The grouped form over three matrices of different shapes: every map
    between the oracle's maps at the score bounds, every output within the
    tolerance of the oracle's product at that map (with the refinement, the
    tolerance of the base read plus that of the product at the map: y is the
    base product plus the lifted blocks' slices above the glass); a second
    run repeats the first bit for bit."""
    shapes = [(64 * 40, 512), (64 * 17, 1024), (64 * 64, 256)]
    mats, items, xs = [], [], []
    for i, (N, K) in enumerate(shapes):
        W, sc, pm = packed(qam, 300 + i, N, K)
        x = WL.activations(WL.stream(300 + i, TAG, 3), B, K)
        mats.append((W, sc))
        xs.append(x)
        items.append((pm, dev(x), torch.empty((B, N), dtype=torch.float32, device="cuda")))
    glass = 1
    for rule_kw in (dict(lam=None), dict(share=0.25)):
        if rule_kw.get("lam", 0) is None:
            W, sc = mats[0]
            y_ref = O.qmatvec_ref(W, sc, xs[0], np.full(W.shape[0] // 64, glass, np.uint8))
            rule_kw = dict(lam=float(np.median(O.layer_scores(y_ref, sc, W.shape[1]))) / 16)
        grp = qam.LayerDecidesGroup(items, qam.LayerRule(glass=glass, **rule_kw), refine=refine)
        assert grp.refine == refine
        grp.run()
        first = [it[2].cpu().numpy().copy() for it in items]
        for i, ((W, sc), x) in enumerate(zip(mats, xs)):
            N, K = W.shape
            lv = grp.levels[i].cpu().numpy()
            uni = np.full(N // 64, glass, np.uint8)
            s_lo, s_hi = score_bounds(O.qmatvec_ref(W, sc, x, uni), O.qmatvec_tolerance(W, sc, x, uni), sc, K)
            if "lam" in rule_kw:
                a = O.layer_levels_threshold(s_lo, 5, glass, 1.0, rule_kw["lam"])
                b = O.layer_levels_threshold(s_hi, 5, glass, 1.0, rule_kw["lam"])
                assert np.all((a <= lv) & (lv <= b)), (i, rule_kw)
            else:
                k = int(np.floor(0.25 * (N // 64)))
                for r in range(B):
                    risen, stay = lv[r] == 4, lv[r] == glass
                    assert risen.sum() == k and (risen | stay).all()
                    assert s_hi[r][risen].min() >= s_lo[r][stay].max()
            ref = O.qmatvec_ref(W, sc, x, lv, per_request=True)
            tol = O.qmatvec_tolerance(W, sc, x, lv, per_request=True)
            if refine:
                tol = tol + O.qmatvec_tolerance(W, sc, x, uni)
            assert np.all(np.abs(first[i].astype(np.float64) - ref) <= tol), (i, rule_kw)
        grp.run()
        for i, it in enumerate(items):
            assert np.array_equal(it[2].cpu().numpy(), first[i]), i


@pytest.mark.parametrize("B", [1, 5])
def test_group_call_bit_exact(qam, B):
    """One launch for several matrices gives each matrix the scores and maps
    of the oracle, bit for bit, in both modes."""
    from query_adaptive_mixed_amd import _lib as L
    import ctypes as C
    nbs, K = (1, 77, 512, 200), 128
    tabs = []
    arr = (L.QamLayerItem * len(nbs))()
    for i, nb in enumerate(nbs):
        _, sc, pm = packed(qam, 500 + i, 64 * nb, K)
        y = base_outputs(500 + i, B, 64 * nb)
        if nb > 4:
            y.reshape(B, nb, 64)[:, 3] = y.reshape(B, nb, 64)[:, 1]
        yd = dev(y)
        sh = torch.empty((B, nb), dtype=torch.float64, device="cuda")
        lv = torch.empty((B, nb), dtype=torch.uint8, device="cuda")
        arr[i].y_base, arr[i].w, arr[i].shat_out, arr[i].level_out = yd.data_ptr(), pm.desc, sh.data_ptr(), lv.data_ptr()
        tabs.append((y, sc, pm, yd, sh, lv))
    for kw in (dict(share=0.3), dict(share=1.0, g=0.5), dict(lam=1e-9), dict(lam=0.0, glass=2)):
        rule = qam.LayerRule(**kw)
        L.check(L.lib().qam_layer_levels_group(arr, len(nbs), B, C.byref(rule.rule), rule.n_rungs, rule.glass, None))
        torch.cuda.synchronize()
        for y, sc, pm, yd, sh, lv in tabs:
            want_s = O.layer_scores(y, sc, K)
            assert np.array_equal(sh.cpu().numpy(), want_s), kw
            if "share" in kw:
                want = O.layer_levels_share(want_s, 5, rule.glass, kw.get("g", 1.0), kw["share"])
            else:
                want = O.layer_levels_threshold(want_s, 5, rule.glass, 1.0, kw["lam"])
            assert np.array_equal(lv.cpu().numpy(), want), (kw, pm.n_blocks)


def test_group_step_graph_replays_match_eager(qam):
    """The grouped layer step captured in a HIP graph: every replay, with
    eager work and synchronisations between them, leaves the same outputs
    and maps as the eager step."""
    B = 4
    items = []
    for i, (N, K) in enumerate([(64 * 40, 512), (64 * 224, 256)]):
        _, _, pm = packed(qam, 700 + i, N, K)
        x = dev(WL.activations(WL.stream(700 + i, TAG, 3), B, K))
        items.append((pm, x, torch.empty((B, N), dtype=torch.float32, device="cuda")))
    grp = qam.LayerDecidesGroup(items, qam.LayerRule(share=1.0 / 3.0, glass=1))
    grp.run()
    torch.cuda.synchronize()
    want_y = [it[2].cpu().numpy().copy() for it in items]
    want_lv = [lv.cpu().numpy().copy() for lv in grp.levels]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        grp.run()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp.run()
    for rep in range(3):
        for it in items:
            it[2].fill_(float("nan"))
        for lv in grp.levels:
            lv.fill_(0xEE)
        graph.replay()
        torch.cuda.synchronize()
        for i, it in enumerate(items):
            assert np.array_equal(it[2].cpu().numpy(), want_y[i]), (rep, i)
            assert np.array_equal(grp.levels[i].cpu().numpy(), want_lv[i]), (rep, i)
        grp.second.run()                       # eager work between replays
        torch.cuda.synchronize()


def test_refinement_and_full_second_product_agree_on_the_maps(qam):
    """Both forms of the grouped step take their maps from the same base
    product, so the maps are the same bits; a block no request lifts keeps
    its base outputs exactly under the refinement."""
    B = 6
    items_r, items_f, mats = [], [], []
    for i, (N, K) in enumerate([(64 * 50, 256), (64 * 30, 512)]):
        W, sc, pm = packed(qam, 900 + i, N, K)
        x = dev(WL.activations(WL.stream(900 + i, TAG, 3), B, K))
        items_r.append((pm, x, torch.empty((B, N), dtype=torch.float32, device="cuda")))
        items_f.append((pm, x, torch.empty((B, N), dtype=torch.float32, device="cuda")))
        mats.append((W, sc))
    rule = qam.LayerRule(share=0.2, glass=1)
    gr = qam.LayerDecidesGroup(items_r, rule, refine=True)
    gf = qam.LayerDecidesGroup(items_f, rule, refine=False)
    gr.base.run()
    torch.cuda.synchronize()
    base = [it[2].cpu().numpy().copy() for it in items_r]
    gr.decide()
    gr.refine_run()
    gf.run()
    torch.cuda.synchronize()
    for i, ((W, sc), it) in enumerate(zip(mats, items_r)):
        lv = gr.levels[i].cpu().numpy()
        assert np.array_equal(lv, gf.levels[i].cpu().numpy()), i
        y = it[2].cpu().numpy()
        kept = np.repeat(lv == 1, 64, axis=1)           # blocks left at the glass
        assert np.array_equal(y[kept], base[i][kept]), i
        assert not np.array_equal(y[~kept], base[i][~kept]), i


def test_layer_decides_batched_layer_full_size(qam):
    """The benchmark's configuration: the batched layer's three matrices
    (4096x4096, 14336x4096, 4096x14336), 32 requests, the top third of each
    request's blocks to D8 over a D2 glass, refinement above the glass.
    Every block's map is checked against the oracle's score bounds; outputs
    on sampled blocks against the oracle's product at the map."""
    fld = WL.batched_layer(0)
    B, glass = 32, 1
    items, mats = [], []
    for i, m in enumerate(fld.matrices):
        W, sc = fld.codes(i), fld.scales(i)
        pm = qam.pack_slices(dev(W), dev(sc))
        x = fld.x(i, B)
        items.append((pm, dev(x), torch.empty((B, m.N), dtype=torch.float32, device="cuda")))
        mats.append((W, sc, x))
    grp = qam.LayerDecidesGroup(items, qam.LayerRule(share=1.0 / 3.0, glass=glass))
    assert grp.refine
    grp.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for i, ((W, sc, x), it) in enumerate(zip(mats, items)):
        N, K = W.shape
        nb = N // 64
        lv = grp.levels[i].cpu().numpy()
        uni = np.full(nb, glass, np.uint8)
        y_ref = O.qmatvec_ref(W, sc, x, uni)
        tol_base = O.qmatvec_tolerance(W, sc, x, uni)
        s_lo, s_hi = score_bounds(y_ref, tol_base, sc, K)
        k = int(np.floor(nb / 3.0))
        for r in range(B):
            risen, stay = lv[r] == 4, lv[r] == glass
            assert risen.sum() == k and (risen | stay).all(), (i, r)
            assert s_hi[r][risen].min() >= s_lo[r][stay].max(), (i, r)
        blocks = np.sort(rng.choice(nb, 12, replace=False))
        rows = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
        ref = O.qmatvec_ref(W[rows], sc[rows], x, lv[:, blocks], per_request=True)
        tol = O.qmatvec_tolerance(W[rows], sc[rows], x, lv[:, blocks], per_request=True) + tol_base[:, rows]
        y = it[2].cpu().numpy()[:, rows].astype(np.float64)
        assert np.all(np.abs(y - ref) <= tol), i


@pytest.mark.parametrize("per_req", [False, True])
def test_group_refine_shared_and_per_request_maps(qam, per_req):
    """qam_qmatvec_group_refine on a group of either map kind: y holds the
    product at a uniform glass, the refinement takes each block to
    max(its rung, the glass); rungs at or below the glass leave y as it is."""
    from query_adaptive_mixed_amd import _lib as L
    import ctypes as C
    B, glass = 5, 2
    rng = WL.stream(1234, TAG, 4)
    mats, base_items, ref_items = [], [], []
    for i, (N, K) in enumerate([(64 * 9, 320), (64 * 21, 1024)]):
        W, sc, pm = packed(qam, 1100 + i, N, K)
        x = WL.activations(WL.stream(1100 + i, TAG, 3), B, K)
        nb = N // 64
        lv = rng.integers(0, 5, (B, nb) if per_req else nb).astype(np.uint8)
        y = torch.empty((B, N), dtype=torch.float32, device="cuda")
        xd = dev(x)
        base_items.append((pm, xd, y, dev(np.full(nb, glass, np.uint8))))
        ref_items.append((pm, xd, y, dev(lv)))
        mats.append((W, sc, x, lv))
    gb, gr = qam.GroupedQmatvec(base_items), qam.GroupedQmatvec(ref_items)
    assert gr.route == "prepass"
    gb.run()
    torch.cuda.synchronize()
    base = [it[2].cpu().numpy().copy() for it in ref_items]
    L.check(L.lib().qam_qmatvec_group_refine(C.byref(gr.desc), glass, None))
    torch.cuda.synchronize()
    for (W, sc, x, lv), it, y0 in zip(mats, ref_items, base):
        nb = W.shape[0] // 64
        eff = np.broadcast_to(np.maximum(lv, glass), (B, nb))
        uni = np.full(nb, glass, np.uint8)
        ref = O.qmatvec_ref(W, sc, x, eff, per_request=True)
        tol = O.qmatvec_tolerance(W, sc, x, eff, per_request=True) + O.qmatvec_tolerance(W, sc, x, uni)
        y = it[2].cpu().numpy()
        assert np.all(np.abs(y.astype(np.float64) - ref) <= tol)
        kept = np.repeat(np.broadcast_to(lv <= glass, (B, nb)), 64, axis=1)
        assert np.array_equal(y[kept], y0[kept])

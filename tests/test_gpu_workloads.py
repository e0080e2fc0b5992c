"""GPU parity at the benchmark's full sizes, in the launch configurations
bench.py times: the whole E2B-shaped field in one grouped launch (with and
without the level map built inside it), the
streaming stack (batch 1 and 8), the batched per-request layer (16 and 32
requests) and the full 28-layer Qwen3-0.6B-shaped decode step.  Outputs are
checked against the oracle on sampled blocks (every row of a sampled block,
each at its block's depth); level maps are checked whole and bit-exact.
"""

import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
HERE = os.path.dirname(os.path.abspath(__file__))
CAL = json.load(open(os.path.join(HERE, "golden", "calibration.json")))


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_blocks(y, W, sc, x, lv, blocks, per_request, what):
    """y [B, N] against the oracle on the rows of the sampled blocks."""
    rows = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
    lvs = lv[..., blocks]
    ref = O.qmatvec_ref(W[rows], sc[rows], x, lvs, per_request=per_request)
    tol = O.qmatvec_tolerance(W[rows], sc[rows], x, lvs, per_request=per_request)
    err = np.abs(y[:, rows].astype(np.float64) - ref)
    bad = ~(err <= tol)
    assert not bad.any(), (what, int(bad.sum()), float(np.nanmax(err / np.maximum(tol, 1e-300))))


def field_items(qam, fld, lv_dev, B):
    items = []
    offs = fld.block_offsets()
    for i, m in enumerate(fld.matrices):
        W = torch.from_numpy(fld.codes(i)).cuda()
        pm = qam.pack_slices(W, dev(fld.scales(i)))
        del W
        x = dev(fld.x(i, B))
        y = torch.full((B, m.N), float("nan"), device="cuda")
        items.append((pm, x, y, lv_dev[offs[i]:offs[i] + m.n_blocks]))
    return items


def test_e2b_field_grouped_launch(qam):
    """The default benchmark step: GPU level map (calibrated to 4.0 bits) and
    one grouped launch over all 210 matrices; three blocks of every matrix
    checked."""
    fld = WL.e2b_field(0)
    c = CAL["e2b_field"]
    lens = WL.e2b_lenses(fld, f=c["target_4.0"]["f"], g=c["g"])
    lv_dev = qam.build_level_map(dev(fld.coords), lens.centres, lens.radii, lens.f, lens.g, lens.combine, lens.glass)
    lv = host(lv_dev)
    assert np.array_equal(lv, O.level_map(fld.coords, lens.centres, lens.radii, lens.f, lens.g, lens.combine, 5,
                                          lens.glass))
    assert abs(O.mean_bits(lv, fld.block_weights()) - 4.0) < 1e-3
    items = field_items(qam, fld, lv_dev, 1)
    grp = qam.GroupedQmatvec(items)
    grp.run()
    assert "staged_group" in qam.last_variant()
    rng = np.random.default_rng(11)
    offs = fld.block_offsets()
    ys = []
    for i, m in enumerate(fld.matrices):
        blocks = np.sort(rng.choice(m.n_blocks, 3, replace=False))
        y = host(items[i][2])
        ys.append(y.copy())
        check_blocks(y, fld.codes(i), fld.scales(i), fld.x(i, 1), lv[offs[i]:offs[i] + m.n_blocks], blocks, False,
                     m.name)
    # another launch plan (longer chunks, no short tail) gives the oracle's
    # values too, and the group's status word stays clear
    grp2 = qam.GroupedQmatvec(items, tuning={"max_chunk_tiles": 96, "tail_pct": -1})
    grp2.run()
    assert grp.status() == 0 and grp2.status() == 0
    for i, m in enumerate(fld.matrices):
        if i % 10 == 0:
            blocks = np.sort(rng.choice(m.n_blocks, 3, replace=False))
            check_blocks(host(items[i][2]), fld.codes(i), fld.scales(i), fld.x(i, 1),
                         lv[offs[i]:offs[i] + m.n_blocks], blocks, False, m.name)


def test_e2b_field_map_built_in_the_launch(qam):
    """The launch bench.py times by default: one grouped launch over all 210
    matrices that builds the level map itself.  Its map is the oracle's, bit
    for bit, and its outputs are those of the map launch followed by the
    plain grouped product, bit for bit."""
    fld = WL.e2b_field(0)
    c = CAL["e2b_field"]
    lens = WL.e2b_lenses(fld, f=c["target_4.0"]["f"], g=c["g"])
    want = O.level_map(fld.coords, lens.centres, lens.radii, lens.f, lens.g, lens.combine, 5, lens.glass)
    cd = dev(fld.coords)
    lv_dev = torch.full((fld.n_blocks,), 0xEE, dtype=torch.uint8, device="cuda")
    items = field_items(qam, fld, lv_dev, 1)
    offs = fld.block_offsets()
    items = [it + (cd[offs[i]:offs[i] + m.n_blocks],) for i, (it, m) in enumerate(zip(items, fld.matrices))]
    grp = qam.GroupedQmatvec(items)
    grp.run_lens(qam.LensRules(lens.centres, lens.radii, lens.f, lens.g, lens.combine, lens.glass))
    assert "staged_group_lens" in qam.last_variant()
    assert np.array_equal(host(lv_dev), want)
    fused = [host(it[2]).copy() for it in items]
    lv_dev.fill_(0xEE)
    qam.build_level_map(cd, lens.centres, lens.radii, lens.f, lens.g, lens.combine, lens.glass, out=lv_dev)
    grp.run()
    rng = np.random.default_rng(12)
    for i, m in enumerate(fld.matrices):
        assert np.array_equal(host(items[i][2]).view(np.uint32), fused[i].view(np.uint32)), m.name
        if i % 7 == 0:
            blocks = np.sort(rng.choice(m.n_blocks, 3, replace=False))
            check_blocks(fused[i], fld.codes(i), fld.scales(i), fld.x(i, 1), want[offs[i]:offs[i] + m.n_blocks],
                         blocks, False, m.name)


@pytest.mark.parametrize("B", [1, 8])
def test_streaming_stack_grouped_launch(qam, B):
    """The streaming stack at 4.0 mean bits (glass D2), all 16 matrices in one
    grouped launch (the batch-1 kernel's matrix-core form at batch 1, the
    pre-pass route at batch 8)."""
    fld = WL.streaming_stack(0)
    c = CAL["streaming_stack"]["glass1_target4.0"]
    cen, rad = WL.stack_lenses(fld)
    lv_dev = qam.build_level_map(dev(fld.coords), cen, rad, c["f"], 1.0, "sum", 1)
    lv = host(lv_dev)
    assert np.array_equal(lv, O.level_map(fld.coords, cen, rad, c["f"], 1.0, "sum", 5, 1))
    offs = fld.block_offsets()
    rng = np.random.default_rng(12 + B)
    items = []
    for i, m in enumerate(fld.matrices):
        pm = qam.pack_slices(dev(fld.codes(i)), dev(fld.scales(i)))
        x = dev(fld.x(i, B))
        y = torch.full((B, m.N), float("nan"), device="cuda")
        items.append((pm, x, y, lv_dev[offs[i]:offs[i] + m.n_blocks]))
    grp = qam.GroupedQmatvec(items)
    grp.run()
    assert ("staged_group" if B == 1 else "qmatvec_mfma_group") in qam.last_variant()
    ys = []
    for i, m in enumerate(fld.matrices):
        blocks = np.sort(rng.choice(m.n_blocks, 3, replace=False))
        ys.append(host(items[i][2]).copy())
        check_blocks(ys[-1], fld.codes(i), fld.scales(i), fld.x(i, B),
                     lv[offs[i]:offs[i] + m.n_blocks], blocks, False, (m.name, B))
    if B == 1:   # bench.py's launch at batch 1: the map built inside it, the same map and bits
        cd = dev(fld.coords)
        items = [it + (cd[offs[i]:offs[i] + m.n_blocks],) for i, (it, m) in enumerate(zip(items, fld.matrices))]
        grp = qam.GroupedQmatvec(items)
        lv_dev.fill_(0xEE)
        grp.run_lens(qam.LensRules(cen, rad, c["f"], 1.0, "sum", 1))
        assert "staged_group_lens" in qam.last_variant()
        assert np.array_equal(host(lv_dev), lv)
        for i, m in enumerate(fld.matrices):
            assert np.array_equal(host(items[i][2]).view(np.uint32), ys[i].view(np.uint32)), m.name
    del items, grp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,xdt", [(16, "f32"), (32, "f32"), (32, "bf16")])
def test_batched_layer_grouped_launch(qam, B, xdt):
    """The batched layer as the benchmark runs it: per-request lens maps built
    on the GPU, one grouped matrix-core launch pair over the 3 matrices."""
    cal = CAL["batched_layer"]
    fld = WL.batched_layer(0)
    reqs = WL.request_lenses(fld, B)
    fs = [cal["requests"][r]["f"] for r in range(B)]
    maps = qam.build_level_maps(dev(fld.coords), reqs, fs, g=1.0, combine="sum", glass=1)
    lv = host(maps)
    for r, (cc, rr) in enumerate(reqs):
        assert np.array_equal(lv[r], O.level_map(fld.coords, cc, rr, fs[r], 1.0, "sum", 5, 1))
    offs = fld.block_offsets()
    items, xs = [], []
    for i, m in enumerate(fld.matrices):
        pm = qam.pack_slices(dev(fld.codes(i)), dev(fld.scales(i)))
        x = torch.from_numpy(fld.x(i, B)).cuda()
        if xdt == "bf16":
            x = x.to(torch.bfloat16)
        xs.append(x.float().cpu().numpy())
        y = torch.full((B, m.N), float("nan"), device="cuda")
        items.append((pm, x.contiguous(), y, dev(np.ascontiguousarray(lv[:, offs[i]:offs[i] + m.n_blocks]))))
    grp = qam.GroupedQmatvec(items)
    grp.run()
    assert "mfma_group" in qam.last_variant() and "per-request" in qam.last_variant()
    rng = np.random.default_rng(13)
    for i, m in enumerate(fld.matrices):
        blocks = np.sort(rng.choice(m.n_blocks, 8, replace=False))
        check_blocks(host(items[i][2]), fld.codes(i), fld.scales(i), xs[i],
                     lv[:, offs[i]:offs[i] + m.n_blocks], blocks, True, (m.name, B, xdt))


def test_qwen_decode_full_step(qam):
    """All 28 layers and the 151936-row head: every one of the 113 products
    checked on sampled blocks against the oracle on its actual input, at D4
    and at D8; a graph replay of the step then gives the same logits bit for
    bit."""
    from query_adaptive_mixed_amd.decode import build_decoder, interleave_gate_up, stack_rows
    cfg = dict(n_layers=28, hidden=1024, q_dim=2048, kv_dim=1024, ffn=3072)
    fld = WL.qwen_decode_field(0)
    dec = build_decoder(fld, cfg["n_layers"], cfg["hidden"], cfg["q_dim"], cfg["kv_dim"], cfg["ffn"], eps=1e-6)
    x0 = WL.decode_inputs(0, 1, 1024)[0]
    rng = np.random.default_rng(14)
    for rung in (2, 4):
        dec.hidden.copy_(dev(x0))
        op = 0
        for l in range(cfg["n_layers"]):
            c = [fld.codes(7 * l + j) for j in range(7)]
            s = [fld.scales(7 * l + j) for j in range(7)]
            mats = [(stack_rows(c[0], c[1], c[2]), stack_rows(s[0], s[1], s[2]), "qkv"), (c[3], s[3], "o"),
                    (interleave_gate_up(c[4], c[5]), interleave_gate_up(s[4], s[5]), "gate_up"), (c[6], s[6], "down")]
            for W, sc, name in mats:
                h = host(dec.hidden).astype(np.float64)[None]
                xin = {"qkv": O.rmsnorm_ref(h, 1e-6), "o": host(dec.qkv)[:2048].astype(np.float64)[None],
                       "gate_up": O.rmsnorm_ref(h, 1e-6), "down": host(dec.m).astype(np.float64)[None]}[name]
                dec.run(rung, op)
                op += 1
                lv = np.full(W.shape[0] // 64, rung, np.uint8)
                blocks = np.sort(rng.choice(W.shape[0] // 64, 2, replace=False))
                rows = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
                ref = O.qmatvec_ref(W[rows], sc[rows], xin, lv[blocks])
                tol = O.qmatvec_tolerance(W[rows], sc[rows], xin, lv[blocks])
                if name == "qkv":
                    got = host(dec.qkv)[None][:, rows]
                elif name in ("o", "down"):
                    got = host(dec.hidden)[None][:, rows]
                    ref = ref + h[:, rows]
                    tol = tol + 2.0 ** -24 * np.abs(ref)
                else:   # gate_up: the sampled blocks' 32 features each
                    g, u = ref[:, np.r_[0:32, 64:96]], ref[:, np.r_[32:64, 96:128]]
                    tg, tu = tol[:, np.r_[0:32, 64:96]], tol[:, np.r_[32:64, 96:128]]
                    ref = O.silu_mul_ref(g, u)
                    tol = 1.1 * tg * (np.abs(u) + tu) + np.abs(g / (1 + np.exp(-g))) * tu + 2.0 ** -23 * np.abs(ref)
                    feats = np.concatenate([np.arange(32 * b, 32 * b + 32) for b in blocks])
                    got = host(dec.m)[None][:, feats]
                err = np.abs(got.astype(np.float64) - ref)
                assert np.all(err <= tol), (rung, l, name, float(np.max(err / np.maximum(tol, 1e-300))))
        h = host(dec.hidden).astype(np.float64)[None]
        dec.run(rung, op)
        Wl, sl = fld.codes(7 * 28), fld.scales(7 * 28)
        blocks = np.sort(rng.choice(Wl.shape[0] // 64, 16, replace=False))
        lvh = np.full(Wl.shape[0] // 64, rung, np.uint8)
        check_blocks(host(dec.logits)[None], Wl, sl, O.rmsnorm_ref(h, 1e-6), lvh, blocks, False, ("head", rung))
        eager = host(dec.logits).copy()
        dec.capture(rung)
        for _ in range(2):
            dec.hidden.copy_(dev(x0))
            dec.replay(rung)
            assert np.array_equal(host(dec.logits), eager), rung

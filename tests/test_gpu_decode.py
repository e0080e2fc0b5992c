"""GPU parity of the fused epilogues and the decode driver against the oracle.

Every product is checked against the CPU oracle on the GPU's actual input
(the decoder's buffers are read between its products); the full step, the
one-product-at-a-time chain and HIP-graph replays must then agree bit for
bit, since they launch the same kernels with the same chunking.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
LADDER = (0, 2, 4, 6, 8)
EPS = 1e-6


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def within(got, ref, tol, what):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bad = ~(err <= tol)
    assert not bad.any(), (what, int(bad.sum()), float(np.nanmax(err / np.maximum(tol, 1e-300))))


def glu_ref(W, sc, x, lv):
    """Gate/up rows interleaved 32/32 per block: oracle values of both halves,
    silu(gate) * up, and a bound that carries each half's product bound
    through silu(g) * u (|silu'| <= 1.1) plus the final fp32 rounding."""
    N = W.shape[0]
    F = N // 2
    idx = np.arange(N).reshape(-1, 64)
    gate_rows, up_rows = idx[:, :32].reshape(-1), idx[:, 32:].reshape(-1)
    v = O.qmatvec_ref(W, sc, x, lv)
    t = O.qmatvec_tolerance(W, sc, x, lv)
    g, u = v[:, gate_rows], v[:, up_rows]
    tg, tu = t[:, gate_rows], t[:, up_rows]
    m = O.silu_mul_ref(g, u)
    silu = g / (1.0 + np.exp(-g))
    tol = 1.1 * tg * (np.abs(u) + tu) + np.abs(silu) * tu + 2.0 ** -23 * np.abs(m) + 1e-30
    assert m.shape[1] == F
    return m, tol


def test_epilogues_take_one_request(qam):
    """The fused epilogues serve the batch-1 decode step: two requests are
    rejected on the host, nothing launched."""
    rng = np.random.default_rng(3)
    W = rng.integers(-127, 128, size=(192, 1536), dtype=np.int64).astype(np.int8)
    pm = qam.pack_slices(dev(W), dev(np.ones(192, np.float32)))
    x = dev(rng.standard_normal((2, 1536)).astype(np.float32))
    with pytest.raises(qam.QamError):
        qam.qmatvec(x, pm, dev(np.full(3, 2, np.uint8)), rms_norm=True)


@pytest.mark.parametrize("N,K,B", [(256, 1024, 1), (512, 6144, 1), (192, 1536, 1), (128, 28672, 1)])
def test_epilogue_modes_match_oracle(qam, N, K, B):
    rng = np.random.default_rng(N + K + B)
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    x = (rng.standard_normal((B, K)) * 3.0).astype(np.float32)
    lv = rng.integers(0, 5, size=N // 64).astype(np.uint8)
    lv[0] = 0
    lv[-1] = 4
    pm = qam.pack_slices(dev(W), dev(sc))
    xd, ld = dev(x), dev(lv)
    xn = O.rmsnorm_ref(x, EPS)
    # RMS-normalised input, stored
    y = host(qam.qmatvec(xd, pm, ld, rms_norm=True, eps=EPS))
    within(y, O.qmatvec_ref(W, sc, xn, lv), O.qmatvec_tolerance(W, sc, xn, lv), "rms store")
    assert np.all(y[:, :64] == 0.0)
    # residual add (plain input)
    y0 = rng.standard_normal((B, N)).astype(np.float32)
    yd = dev(y0)
    qam.qmatvec(xd, pm, ld, y=yd, out_mode="add")
    y = host(yd)
    ref = y0.astype(np.float64) + O.qmatvec_ref(W, sc, x, lv)
    within(y, ref, O.qmatvec_tolerance(W, sc, x, lv) + 2.0 ** -24 * np.abs(ref), "add")
    assert np.array_equal(y[:, :64], y0[:, :64])   # a ZERO block leaves the residual as it is
    # residual add of an RMS-normalised product
    yd = dev(y0)
    qam.qmatvec(xd, pm, ld, y=yd, out_mode="add", rms_norm=True, eps=EPS)
    ref = y0.astype(np.float64) + O.qmatvec_ref(W, sc, xn, lv)
    within(host(yd), ref, O.qmatvec_tolerance(W, sc, xn, lv) + 2.0 ** -24 * np.abs(ref), "rms add")
    # gated pairs
    for rms in (False, True):
        xin = xn if rms else x
        y = host(qam.qmatvec(xd, pm, ld, out_mode="glu", rms_norm=rms, eps=EPS))
        m, tol = glu_ref(W, sc, xin, lv)
        assert y.shape == (B, N // 2)
        within(y, m, tol, ("glu", rms))
        assert np.all(y[:, :32] == 0.0)


def test_epilogue_rms_bf16(qam):
    rng = np.random.default_rng(5)
    N, K = 256, 3072
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    xb = torch.from_numpy(rng.standard_normal((1, K)).astype(np.float32)).to(torch.bfloat16)
    x = xb.float().numpy()
    lv = np.array([1, 2, 3, 4], np.uint8)
    pm = qam.pack_slices(dev(W), dev(sc))
    y = host(qam.qmatvec(xb.cuda(), pm, dev(lv), rms_norm=True, eps=EPS))
    xn = O.rmsnorm_ref(x, EPS)
    within(y, O.qmatvec_ref(W, sc, xn, lv), O.qmatvec_tolerance(W, sc, xn, lv), "rms bf16")


# ------------------------------------------------------------------ decoder

SMALL = dict(n_layers=2, hidden=256, q_dim=512, kv_dim=128, ffn=384, vocab=1024)


def _fused_weights(fld, n_layers):
    """Host copies of the fused matrices the decoder packs (for the oracle)."""
    from query_adaptive_mixed_amd.decode import interleave_gate_up, stack_rows
    out = []
    for l in range(n_layers):
        c = [fld.codes(7 * l + j) for j in range(7)]
        s = [fld.scales(7 * l + j) for j in range(7)]
        out.append([(stack_rows(c[0], c[1], c[2]), stack_rows(s[0], s[1], s[2])), (c[3], s[3]),
                    (interleave_gate_up(c[4], c[5]), interleave_gate_up(s[4], s[5])), (c[6], s[6])])
    head = (fld.codes(7 * n_layers), fld.scales(7 * n_layers))
    return out, head


def _make_decoder(qam, cfg, seed=0, target_waves=0, waves_per_block=0):
    from query_adaptive_mixed_amd.decode import build_decoder
    fld = WL.decoder_field(seed, cfg["n_layers"], cfg["hidden"], cfg["q_dim"], cfg["kv_dim"], cfg["ffn"],
                           cfg["vocab"])
    dec = build_decoder(fld, cfg["n_layers"], cfg["hidden"], cfg["q_dim"], cfg["kv_dim"], cfg["ffn"], eps=EPS,
                        target_waves=target_waves, waves_per_block=waves_per_block)
    return fld, dec


def _check_chain_against_oracle(qam, dec, fld, cfg, rung, x0, head_rows=None):
    """Run the step one product at a time; check each on its actual input."""
    mats, head = _fused_weights(fld, cfg["n_layers"])
    Q = cfg["q_dim"]
    dec.hidden.copy_(dev(x0))
    lv_of = lambda W: np.full(W.shape[0] // 64, rung, np.uint8)
    op = 0
    for l in range(cfg["n_layers"]):
        (Wqkv, sqkv), (Wo, so), (Wgu, sgu), (Wd, sd) = mats[l]
        h = host(dec.hidden).astype(np.float64)[None]
        dec.run(rung, op); op += 1
        xn = O.rmsnorm_ref(h, EPS)
        within(host(dec.qkv)[None], O.qmatvec_ref(Wqkv, sqkv, xn, lv_of(Wqkv)),
               O.qmatvec_tolerance(Wqkv, sqkv, xn, lv_of(Wqkv)), (l, "qkv"))
        q = host(dec.qkv)[:Q].astype(np.float64)[None]
        h = host(dec.hidden).astype(np.float64)[None]
        dec.run(rung, op); op += 1
        ref = h + O.qmatvec_ref(Wo, so, q, lv_of(Wo))
        within(host(dec.hidden)[None], ref, O.qmatvec_tolerance(Wo, so, q, lv_of(Wo)) + 2.0 ** -24 * np.abs(ref),
               (l, "o"))
        h = host(dec.hidden).astype(np.float64)[None]
        dec.run(rung, op); op += 1
        m, tol = glu_ref(Wgu, sgu, O.rmsnorm_ref(h, EPS), lv_of(Wgu))
        within(host(dec.m)[None], m, tol, (l, "gate_up"))
        mm = host(dec.m).astype(np.float64)[None]
        h = host(dec.hidden).astype(np.float64)[None]
        dec.run(rung, op); op += 1
        ref = h + O.qmatvec_ref(Wd, sd, mm, lv_of(Wd))
        within(host(dec.hidden)[None], ref, O.qmatvec_tolerance(Wd, sd, mm, lv_of(Wd)) + 2.0 ** -24 * np.abs(ref),
               (l, "down"))
    h = host(dec.hidden).astype(np.float64)[None]
    dec.run(rung, op)
    Wl, sl = head
    rows = np.arange(Wl.shape[0]) if head_rows is None else head_rows
    xn = O.rmsnorm_ref(h, EPS)
    lv = np.full(Wl.shape[0] // 64, rung, np.uint8)
    blocks = np.unique(rows // 64)
    sub = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
    ref = O.qmatvec_ref(Wl[sub], sl[sub], xn, lv[blocks])
    tol = O.qmatvec_tolerance(Wl[sub], sl[sub], xn, lv[blocks])
    within(host(dec.logits)[sub][None], ref, tol, "lm_head")
    return host(dec.logits).copy(), host(dec.hidden).copy()


@pytest.mark.parametrize("wpb,tw", [(0, 0), (1, 0), (2, 0), (8, 0), (4, 512)])
@pytest.mark.parametrize("rung", [2, 4, 1, 0])
def test_decoder_products_match_oracle(qam, rung, wpb, tw):
    """Every product of the chain against the oracle, for 1, 2, 4 and 8 waves
    per block (uneven tile shares: 4, 6 and 8 tiles over the waves) and with
    a wide launch that also splits K across workgroups."""
    fld, dec = _make_decoder(qam, SMALL, target_waves=tw, waves_per_block=wpb)
    x0 = WL.decode_inputs(0, 1, SMALL["hidden"])[0]
    logits, h = _check_chain_against_oracle(qam, dec, fld, SMALL, rung, x0)
    # the whole step launches the same products: bit-identical
    dec.hidden.copy_(dev(x0))
    dec.step(rung)
    assert np.array_equal(host(dec.logits), logits)
    assert np.array_equal(host(dec.hidden), h)
    if rung == 0:
        assert np.all(logits == 0.0)   # every block ZERO: nothing read, the residual untouched
        assert np.array_equal(h, x0)


def test_decoder_graph_replays_match_eager(qam):
    fld, dec = _make_decoder(qam, SMALL)
    xs = WL.decode_inputs(1, 4, SMALL["hidden"])
    eager = {}
    for rung in (2, 4):
        for t in range(2):
            dec.hidden.copy_(dev(xs[t]))
            dec.step(rung)
            eager[(rung, t)] = (host(dec.logits).copy(), host(dec.hidden).copy())
    dec.capture(2)
    dec.capture(4)
    for rep in range(3):
        for rung in (2, 4):
            for t in range(2):
                dec.hidden.copy_(dev(xs[t]))
                dec.replay(rung)
                lg, hh = host(dec.logits), host(dec.hidden)
                assert np.array_equal(lg, eager[(rung, t)][0]), (rep, rung, t)
                assert np.array_equal(hh, eager[(rung, t)][1]), (rep, rung, t)
        # eager work between replays
        dec.hidden.copy_(dev(xs[3]))
        dec.step(2)
        torch.cuda.synchronize()


def test_decoder_qwen_shapes_two_layers(qam):
    """Qwen3-0.6B shapes (hidden 1024, q 2048, kv 1024, ffn 3072, head
    151936x1024) at two layers, with the launch widths of the full model."""
    cfg = dict(n_layers=2, hidden=1024, q_dim=2048, kv_dim=1024, ffn=3072, vocab=151936)
    fld, dec = _make_decoder(qam, cfg)
    x0 = WL.decode_inputs(0, 1, 1024)[0]
    rows = np.random.default_rng(0).choice(151936, 4096, replace=False)
    for rung in (2, 4):
        _check_chain_against_oracle(qam, dec, fld, cfg, rung, x0, head_rows=rows)


def test_escalation_schedule_product_matches_oracle(qam):
    scores = WL.escalation_scores(0, 256)
    got = qam.escalation_schedule(scores, 0.16)
    assert np.array_equal(got, O.escalation_schedule(scores, 0.16))
    assert int(got.sum()) == 41


def test_decode_gated_matches_step_by_step_loop(qam):
    """The library's gated loop takes the same decisions, and leaves the same
    bits in the decoder's buffers, as the loop driven step by step from the
    host (replay the low rung, gate, replay the high rung on escalation)."""
    fld, dec = _make_decoder(qam, SMALL)
    T = 12
    xs = dev(WL.decode_inputs(5, T, SMALL["hidden"]))
    gate = qam.Gate(SMALL["vocab"])
    with pytest.raises(qam.QamError):                 # rungs not captured yet
        dec.decode_gated(xs, gate, 1.0)
    dec.capture(2)
    dec.capture(4)
    ent = []
    for t in range(T):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
        gate.run(dec.logits)
        ent.append(gate.result()["entropy"])
    srt = sorted(ent)
    tau = 0.5 * (srt[T // 2 - 1] + srt[T // 2])       # fires on half the steps
    want, last = [], None
    for t in range(T):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
        gate.run(dec.logits, tau)
        esc = gate.result()["escalate"]
        if esc:
            dec.hidden.copy_(xs[t])
            dec.replay(4)
        want.append(int(esc))
        last = (host(dec.logits).copy(), host(dec.hidden).copy())
    assert sum(want) == T // 2
    for rep in range(2):
        dec.hidden.zero_()
        got = dec.decode_gated(xs, gate, tau)
        assert got.tolist() == want, rep
        assert np.array_equal(host(dec.logits), last[0]) and np.array_equal(host(dec.hidden), last[1]), rep
    assert dec.decode_gated(xs[:0], gate, tau).size == 0
    assert dec.decode_gated(xs, gate, math.inf, -math.inf).sum() == 0      # never fires
    assert dec.decode_gated(xs, gate, -1.0).sum() == T                     # always fires (H >= 0 > -1)
    with pytest.raises(ValueError):
        dec.decode_gated(xs, qam.Gate(SMALL["vocab"] + 1), tau)
    with pytest.raises(qam.QamError):
        dec.decode_gated(xs, gate, tau, rung_low=1)


def test_decode_gated_async_matches_the_synchronising_loop(qam):
    """The gated steps with the decision left on the device (predicated
    high-rung graph, no per-step synchronisation) take the same decisions and
    leave the same bits as qam_decoder_decode_gated."""
    fld, dec = _make_decoder(qam, SMALL)
    T = 12
    xs = dev(WL.decode_inputs(6, T, SMALL["hidden"]))
    gate = qam.Gate(SMALL["vocab"])
    dec.capture(2)
    dec.capture(4)
    ent = []
    for t in range(T):
        dec.hidden.copy_(xs[t])
        dec.replay(2)
        gate.run(dec.logits)
        ent.append(gate.result()["entropy"])
    srt = sorted(ent)
    tau = 0.5 * (srt[T // 2 - 1] + srt[T // 2])
    want = dec.decode_gated(xs, gate, tau)
    last = (host(dec.logits).copy(), host(dec.hidden).copy())
    assert 0 < int(want.sum()) < T
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for rep in range(2):
            dec.hidden.zero_()
            got = dec.decode_gated_async(xs, gate, tau)
            side.synchronize()
            assert got.cpu().numpy().tolist() == want.tolist(), rep
            assert np.array_equal(dec.logits.cpu().numpy(), last[0]), rep
            assert np.array_equal(dec.hidden.cpu().numpy(), last[1]), rep
        # a second gate: the predicated graph is captured again for its flag
        gate2 = qam.Gate(SMALL["vocab"])
        got = dec.decode_gated_async(xs, gate2, -1.0)          # always fires
        side.synchronize()
        assert int(got.sum()) == T
        fired_last = dec.logits.cpu().numpy().copy()
        got = dec.decode_gated_async(xs, gate2, float("inf"))   # never fires
        side.synchronize()
        assert int(got.sum()) == 0
        never_last = dec.logits.cpu().numpy().copy()
        for rung, ref in ((4, fired_last), (2, never_last)):
            dec.hidden.copy_(xs[T - 1])
            dec.replay(rung)
            side.synchronize()
            assert np.array_equal(dec.logits.cpu().numpy(), ref), rung
    torch.cuda.current_stream().wait_stream(side)
    import query_adaptive_mixed_amd._lib as L
    from query_adaptive_mixed_amd.api import _ptr
    rc = L.lib().qam_decoder_decode_gated_async(dec._h, _ptr(xs), T, 2, 4, 1.0, -1.0, _ptr(gate.ws), gate.ws.numel(),
                                                 _ptr(gate.out), _ptr(xs), None)
    assert rc == -3                                               # the null stream is refused

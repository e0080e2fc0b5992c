"""Draft-and-verify on the device: the batched verify chain product by
product against the oracle, slot independence of its rows, the row argmax,
and the library's speculation loop against the oracle's loop driven by the
same draft and target steps."""

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
EPS = 1e-6
SMALL = dict(n_layers=2, hidden=256, q_dim=512, kv_dim=128, ffn=384, vocab=1024)


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


def fused_weights(fld, n_layers):
    from query_adaptive_mixed_amd.decode import interleave_gate_up, stack_rows
    out = []
    for l in range(n_layers):
        c = [fld.codes(7 * l + j) for j in range(7)]
        s = [fld.scales(7 * l + j) for j in range(7)]
        out.append([(stack_rows(c[0], c[1], c[2]), stack_rows(s[0], s[1], s[2])), (c[3], s[3]),
                    (interleave_gate_up(c[4], c[5]), interleave_gate_up(s[4], s[5])), (c[6], s[6])])
    return out, (fld.codes(7 * n_layers), fld.scales(7 * n_layers))


def make(qam, cfg, max_batch=8, seed=0):
    from query_adaptive_mixed_amd.decode import build_decoder
    fld = WL.decoder_field(seed, cfg["n_layers"], cfg["hidden"], cfg["q_dim"], cfg["kv_dim"], cfg["ffn"],
                           cfg["vocab"])
    dec = build_decoder(fld, cfg["n_layers"], cfg["hidden"], cfg["q_dim"], cfg["kv_dim"], cfg["ffn"], eps=EPS)
    return fld, dec, qam.Verifier(dec, max_batch)


def rms_tol(ref):
    return 2.0 ** -23 * np.abs(ref) + 1e-30


def add_norm_check(ver, B, H, h, y, what):
    """h += y and xn = rmsnorm(h), the step that opens a product's input."""
    hn = host(ver.hidden[:B])
    assert np.array_equal(hn, (h.astype(np.float32) + y.astype(np.float32))), (what, "residual")
    within(host(ver.xn(B, H)), O.rmsnorm_ref(hn.astype(np.float64), EPS), rms_tol(O.rmsnorm_ref(hn, EPS)),
           (what, "norm"))
    return host(ver.xn(B, H)).astype(np.float64)


def check_chain(qam, ver, fld, cfg, rung, B, X, head_rows=None):
    """Run the batched chain one op at a time; check every op on its actual
    inputs: each op forms its input (residual add and norm, the q columns,
    the gated product) from the previous op's output, then multiplies."""
    H, Q, F = cfg["hidden"], cfg["q_dim"], cfg["ffn"]
    mats, (Wl, sl) = fused_weights(fld, cfg["n_layers"])
    lv_of = lambda W: np.full(W.shape[0] // 64, rung, np.uint8)
    ver.x[:B].copy_(dev(X))
    ver.run(rung, B, 0)
    assert np.array_equal(host(ver.hidden[:B]), X)
    within(host(ver.xn(B, H)), O.rmsnorm_ref(X.astype(np.float64), EPS), rms_tol(O.rmsnorm_ref(X, EPS)), "init")
    xn = host(ver.xn(B, H)).astype(np.float64)
    op = 1
    for l in range(cfg["n_layers"]):
        (Wqkv, sqkv), (Wo, so), (Wgu, sgu), (Wd, sd) = mats[l]
        if l > 0:
            h, y = host(ver.hidden[:B]), host(ver.y(B, H))
        ver.run(rung, B, op); op += 1
        if l > 0:
            xn = add_norm_check(ver, B, H, h, y, (l, "down residual"))
        within(host(ver.qkv[:B]), O.qmatvec_ref(Wqkv, sqkv, xn, lv_of(Wqkv)),
               O.qmatvec_tolerance(Wqkv, sqkv, xn, lv_of(Wqkv)), (l, "qkv"))
        q = host(ver.qkv[:B])[:, :Q].astype(np.float64)
        ver.run(rung, B, op); op += 1
        within(host(ver.y(B, H)), O.qmatvec_ref(Wo, so, q, lv_of(Wo)), O.qmatvec_tolerance(Wo, so, q, lv_of(Wo)),
               (l, "o"))
        h, y = host(ver.hidden[:B]), host(ver.y(B, H))
        ver.run(rung, B, op); op += 1
        xn = add_norm_check(ver, B, H, h, y, (l, "o residual"))
        within(host(ver.y(B, 2 * F)), O.qmatvec_ref(Wgu, sgu, xn, lv_of(Wgu)),
               O.qmatvec_tolerance(Wgu, sgu, xn, lv_of(Wgu)), (l, "gate_up"))
        gu = host(ver.y(B, 2 * F)).astype(np.float64).reshape(B, -1, 2, 32)
        ver.run(rung, B, op); op += 1
        m_ref = O.silu_mul_ref(gu[:, :, 0, :], gu[:, :, 1, :]).reshape(B, F)
        within(host(ver.m[:B]), m_ref, 2.0 ** -23 * np.abs(m_ref) + 1e-30, (l, "gated"))
        mm = host(ver.m[:B]).astype(np.float64)
        within(host(ver.y(B, H)), O.qmatvec_ref(Wd, sd, mm, lv_of(Wd)), O.qmatvec_tolerance(Wd, sd, mm, lv_of(Wd)),
               (l, "down"))
    h, y = host(ver.hidden[:B]), host(ver.y(B, H))
    ver.run(rung, B, op)
    xn = add_norm_check(ver, B, H, h, y, "head residual")
    rows = np.arange(Wl.shape[0]) if head_rows is None else head_rows
    blocks = np.unique(rows // 64)
    sub = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
    lv = np.full(blocks.size, rung, np.uint8)
    within(host(ver.logits[:B])[:, sub], O.qmatvec_ref(Wl[sub], sl[sub], xn, lv),
           O.qmatvec_tolerance(Wl[sub], sl[sub], xn, lv), "lm_head")
    return host(ver.logits[:B]).copy()


@pytest.mark.parametrize("B", [1, 2, 3, 8])
@pytest.mark.parametrize("rung", [2, 4])
def test_verifier_chain_matches_oracle(qam, rung, B):
    fld, dec, ver = make(qam, SMALL)
    X = WL.decode_inputs(7, B, SMALL["hidden"])
    print(f"verifier chain rung={rung} B={B}", flush=True)
    logits = check_chain(qam, ver, fld, SMALL, rung, B, X)
    ver.x[:B].copy_(dev(X))
    ver.step(rung, B)
    assert np.array_equal(host(ver.logits[:B]), logits)


def test_verifier_rows_do_not_depend_on_slot_or_neighbours(qam):
    fld, dec, ver = make(qam, SMALL)
    B = 5
    X = WL.decode_inputs(9, B, SMALL["hidden"])
    ver.x[:B].copy_(dev(X))
    ver.step(4, B)
    full = host(ver.logits[:B]).copy()
    ver.x[:B].copy_(dev(X[::-1].copy()))
    ver.step(4, B)
    assert np.array_equal(host(ver.logits[:B]), full[::-1])
    for r in range(B):
        Z = np.zeros_like(X)
        Z[0] = X[r]
        ver.x[:B].copy_(dev(Z))
        ver.step(4, B)
        assert np.array_equal(host(ver.logits[0]), full[r]), r


def test_verifier_graph_replays_match_eager(qam):
    fld, dec, ver = make(qam, SMALL)
    B = 4
    X = WL.decode_inputs(12, B, SMALL["hidden"])
    ver.x[:B].copy_(dev(X))
    ver.step(4, B)
    eager = host(ver.logits[:B]).copy()
    ver.capture(4, B)
    for rep in range(3):
        ver.x[:B].copy_(dev(X))
        ver.replay(4, B)
        assert np.array_equal(host(ver.logits[:B]), eager), rep
        ver.x[:B].copy_(dev(X[::-1].copy()))          # eager work between replays
        ver.step(2, B)
        torch.cuda.synchronize()


@pytest.mark.parametrize("rows,n", [(1, 1), (1, 5), (3, 4096), (9, 4097), (2, 151936)])
def test_argmax_rows_first_index_of_the_maximum(qam, rows, n):
    rng = np.random.default_rng(rows * 7 + n)
    v = rng.standard_normal((rows, n)).astype(np.float32) - 3.0
    for r in range(rows):                       # ties: the maximum repeated, the first must win
        top = v[r].max() + 1.0
        pos = rng.choice(n, size=min(n, 3), replace=False)
        v[r, pos] = top
    if n > 10:
        v[0, :10] = -np.inf                     # infinities are ordinary values
    ws = torch.zeros(rows, dtype=torch.int64, device="cuda")
    got = host(qam.argmax_rows(dev(v), ws))
    assert np.array_equal(got, np.argmax(v, axis=1).astype(np.int32))
    assert int(host(ws).any()) == 0             # workspace left zero


def oracle_loop(qam, dec, ver, E_host, E_dev, first, n, k, draft_rung=2, verify_rung=4):
    """The oracle's loop, its draft and target steps run by the library:
    draft(t) = argmax of one step at the draft rung on E[t]; target(t) =
    argmax of row 0 of a verify pass of k + 1 rows with E[t] in row 0."""
    ws = torch.zeros(1, dtype=torch.int64, device="cuda")

    def draft_next(t):
        dec.hidden.copy_(E_dev[t])
        dec.step(draft_rung)
        return int(host(qam.argmax_rows(dec.logits.view(1, -1), ws))[0])

    def target_next(t):
        ver.x[:k + 1].zero_()
        ver.x[0].copy_(E_dev[t])
        ver.step(verify_rung, k + 1)
        return int(host(qam.argmax_rows(ver.logits[0:1].contiguous(), ws))[0])

    return O.speculative_decode(draft_next, target_next, first, n, k)


@pytest.mark.parametrize("k", [1, 3, 7])
def test_speculation_matches_oracle_loop(qam, k):
    fld, dec, ver = make(qam, SMALL)
    E = WL.embedding_table(3, SMALL["vocab"], SMALL["hidden"])
    Ed = dev(E)
    n = 24
    print(f"speculate small k={k}", flush=True)
    toks, st = qam.speculate(dec, ver, Ed, 5, n, k)
    ref_toks, ref_st = oracle_loop(qam, dec, ver, E, Ed, 5, n, k)
    assert toks.tolist() == ref_toks
    assert st == ref_st
    # captured draft graph, then captured verify graph: same tokens
    dec.capture(2)
    toks2, st2 = qam.speculate(dec, ver, Ed, 5, n, k)
    assert toks2.tolist() == ref_toks and st2 == ref_st
    ver.capture(4, k + 1)
    for rep in range(2):
        toks3, st3 = qam.speculate(dec, ver, Ed, 5, n, k)
        assert toks3.tolist() == ref_toks and st3 == ref_st, rep


def test_speculation_with_identical_rungs_keeps_every_draft(qam):
    """Draft and target both at D8: the one-request and batched products
    round differently, so near-ties may still disagree, but almost every
    draft is kept and the rounds emit the target chain."""
    fld, dec, ver = make(qam, SMALL)
    E = WL.embedding_table(4, SMALL["vocab"], SMALL["hidden"])
    Ed = dev(E)
    toks, st = qam.speculate(dec, ver, Ed, 11, 16, 3, draft_rung=4, verify_rung=4)
    ref_toks, ref_st = oracle_loop(qam, dec, ver, E, Ed, 11, 16, 3, draft_rung=4, verify_rung=4)
    assert toks.tolist() == ref_toks and st == ref_st
    assert st["accepted"] >= 0.8 * st["drafted"]


def test_speculation_rejects_bad_arguments(qam):
    fld, dec, ver = make(qam, SMALL, max_batch=4)
    Ed = dev(WL.embedding_table(0, SMALL["vocab"], SMALL["hidden"]))
    for kw in (dict(k=0), dict(k=4), dict(first_token=-1), dict(first_token=SMALL["vocab"]),
               dict(draft_rung=5), dict(n_tokens=-1)):
        args = dict(first_token=0, n_tokens=4, k=2)
        args.update(kw)
        with pytest.raises(qam.QamError):
            qam.speculate(dec, ver, Ed, args["first_token"], args["n_tokens"], args["k"],
                          draft_rung=args.get("draft_rung", 2))
    toks, st = qam.speculate(dec, ver, Ed, 0, 0, 2)
    assert toks.size == 0 and st["rounds"] == 0


def test_qwen_shapes_two_layers(qam):
    """Qwen3-0.6B shapes at two layers with the full 151936-token head."""
    cfg = dict(n_layers=2, hidden=1024, q_dim=2048, kv_dim=1024, ffn=3072, vocab=151936)
    fld, dec, ver = make(qam, cfg, max_batch=4)
    X = WL.decode_inputs(2, 4, 1024)
    rows = np.random.default_rng(1).choice(151936, 2048, replace=False)
    print("verifier chain qwen shapes B=4", flush=True)
    check_chain(qam, ver, fld, cfg, 4, 4, X, head_rows=rows)
    E_dev = torch.randn(151936, 1024, generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
    toks, st = qam.speculate(dec, ver, E_dev, 17, 12, 3)
    ref_toks, ref_st = oracle_loop(qam, dec, ver, None, E_dev, 17, 12, 3)
    assert toks.tolist() == ref_toks and st == ref_st

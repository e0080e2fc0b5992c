"""GPU parity of the escalation gate (softmax entropy and top-two margin of
the low pass's logits, and the decision) against the CPU oracle, through the
C ABI."""

import math

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

QWEN_VOCAB = 151936
TOL_H = 1e-9       # entropy: fp64 sums in another order than the oracle's
TOL_P = 1e-12      # probabilities and margin


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def run(qam, z, tau_h=math.inf, tau_m=-math.inf, gate=None):
    z = np.ascontiguousarray(z, dtype=np.float32)
    g = gate or qam.Gate(z.size)
    g.run(torch.from_numpy(z).cuda(), tau_h, tau_m)
    return g.result()


def agree(got, z, what):
    want = O.uncertainty(z.astype(np.float64))
    if math.isnan(want["entropy"]):
        assert math.isnan(got["entropy"]) and math.isnan(got["margin"]) and got["escalate"], what
        return want
    assert abs(got["entropy"] - want["entropy"]) <= TOL_H, (what, got["entropy"], want["entropy"])
    assert abs(got["margin"] - want["margin"]) <= TOL_P, what
    assert abs(got["p1"] - want["p1"]) <= TOL_P and abs(got["p2"] - want["p2"]) <= TOL_P, what
    assert (got["top1"], got["top2"]) == (want["top1"], want["top2"]), what
    return want


@pytest.mark.parametrize("V", [2, 3, 100, 4095, 4097, 65537, QWEN_VOCAB, 1_048_577 + 4096 * 300])
def test_gate_matches_oracle(qam, V):
    rng = np.random.default_rng(V)
    for scale in (0.05, 1.0, 6.0, 40.0):
        z = (rng.standard_normal(V) * scale).astype(np.float32)
        agree(run(qam, z), z, (V, scale))


def test_gate_ties_infinities_and_no_distribution(qam):
    V = 9000
    z = np.zeros(V, np.float32)
    agree(run(qam, z), z, "uniform")                  # H = ln V, margin 0, top two 0 and 1
    z[[5000, 17, 8999]] = 3.0
    agree(run(qam, z), z, "tied maxima")              # ties to the lower index: 17, then 5000
    z = np.random.default_rng(2).standard_normal(V).astype(np.float32)
    z[::3] = -np.inf                                  # tokens of probability 0
    agree(run(qam, z), z, "-inf logits")
    z = np.full(V, -np.inf, np.float32)
    z[4096 * 2 + 5] = 1.0                             # one finite logit, in a later slice
    agree(run(qam, z), z, "one finite logit")
    for bad in ("nan", "inf", "all -inf"):
        z = np.random.default_rng(3).standard_normal(V).astype(np.float32)
        if bad == "nan":
            z[7777] = np.nan
        elif bad == "inf":
            z[12] = np.inf
        else:
            z[:] = -np.inf
        got = run(qam, z, 100.0, -1.0)
        assert math.isnan(got["entropy"]) and got["escalate"], bad


def test_gate_decision_and_reuse(qam):
    """The decision follows the oracle's gate wherever the value is not within
    the tolerance of its threshold; one workspace serves calls of one length
    in a row (its counter returns to zero) and repeats give the same bits."""
    rng = np.random.default_rng(11)
    g = qam.Gate(QWEN_VOCAB)
    seen = []
    for t in range(12):
        z = (rng.standard_normal(QWEN_VOCAB) * rng.uniform(0.5, 30.0)).astype(np.float32)
        want = O.uncertainty(z.astype(np.float64))
        for tau_h, tau_m in ((want["entropy"] - 1e-6, -math.inf), (want["entropy"] + 1e-6, -math.inf),
                             (math.inf, want["margin"] + 1e-6), (math.inf, want["margin"] - 1e-6),
                             (5.0, 0.2)):
            got = run(qam, z, tau_h, tau_m, gate=g)
            assert got["escalate"] == O.gate(z.astype(np.float64), tau_h, tau_m), (t, tau_h, tau_m)
        a = run(qam, z, gate=g)
        b = run(qam, z, gate=g)
        assert a == b
        seen.append(a["entropy"])
    assert len(set(seen)) == len(seen)


def test_gate_rejects_bad_arguments(qam):
    from query_adaptive_mixed_amd import _lib as L
    lib = L.lib()
    assert lib.qam_gate_workspace_bytes(1) == 0
    g = qam.Gate(64)
    z = torch.zeros(64, device="cuda")
    with pytest.raises(ValueError):
        g.run(torch.zeros(65, device="cuda"))
    with pytest.raises(L.QamError):
        g.run(z, float("nan"), 0.0)
    rc = lib.qam_gate(z.data_ptr(), 64, 1.0, 0.0, g.out.data_ptr(), g.ws.data_ptr(), 8, None)
    assert rc == -7                                   # workspace too small

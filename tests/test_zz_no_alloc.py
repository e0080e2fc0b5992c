"""qam_qmatvec_noalloc (static per-GPU scratch) against qam_qmatvec.

Each case makes two calls in a row through the C ABI, the second with a
smaller input, and checks both outputs bit for bit against qam_qmatvec with
a workspace of its own on the same inputs, and against the oracle within
1e-4 * sum_k |w_nk| |x_k| per row.
"""

import ctypes as C

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make_case(qam, N, K, B, per_request, seed):
    rng = np.random.default_rng(seed)
    W = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
    x = rng.standard_normal((B, K)).astype(np.float32)
    nb = N // 64
    shape = (B, nb) if per_request else (nb,)
    lv = rng.integers(0, 5, size=shape).astype(np.uint8)
    pm = qam.pack_slices(dev(W), dev(sc))
    return W, sc, x, lv, pm


def check_oracle(y, W, sc, x, lv):
    B = x.shape[0]
    for r in range(B):
        lr = lv[r] if lv.ndim == 2 else lv
        ref = O.qmatvec_ref(W, sc, x[r:r + 1], lr)
        tol = O.qmatvec_tolerance(W, sc, x[r:r + 1], lr)
        err = np.abs(y[r:r + 1].astype(np.float64) - ref)
        assert (err <= tol).all(), (r, float((err / np.maximum(tol, 1e-300)).max()))


def run_noalloc_raw(qam, pm, xt, lvt, y):
    """Direct ctypes call of the C entry point (the binding adds only checks)."""
    from query_adaptive_mixed_amd import _lib as L
    B = xt.shape[0]
    rc = L.lib().qam_qmatvec_noalloc(C.c_void_p(xt.data_ptr()), L.QAM_X_F32, B, C.byref(pm.desc),
                                     C.c_void_p(lvt.data_ptr()), int(lvt.dim() == 2), C.c_void_p(y.data_ptr()),
                                     C.c_void_p(torch.cuda.current_stream().cuda_stream))
    L.check(rc)
    return y


# (first call), (second call, smaller); shapes span several tiles, chunks
# split along K, ragged block counts, and both routes (B = 1 staged limbs,
# B > 1 pre-pass, shared and per-request maps)
CASES = [
    ((2048, 8192, 1, False), (192, 1088, 1, False)),
    ((1024, 4096, 8, False), (256, 1024, 3, False)),
    ((1024, 4096, 32, True), (320, 640, 2, True)),
    ((4096, 14336, 16, True), (512, 256, 1, False)),
    ((512, 256, 1, False), (64, 64, 1, False)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_qmatvec(qam, first, second):
    for i, (N, K, B, per_req) in enumerate((first, second)):
        print(f"noalloc case N={N} K={K} B={B} per_request={per_req} call {i}", flush=True)
        W, sc, x, lv, pm = make_case(qam, N, K, B, per_req, seed=1000 * N + K + B)
        xt, lvt = dev(x), dev(lv)
        y_ref = qam.qmatvec(xt, pm, lvt)
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
        if i == 0:
            run_noalloc_raw(qam, pm, xt, lvt, y)
        else:
            qam.qmatvec_noalloc(xt, pm, lvt, y)
        torch.cuda.synchronize()
        yh, yr = y.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(yh.view(np.uint32), yr.view(np.uint32)), (N, K, B, per_req)
        if N * K <= 4096 * 4096:
            check_oracle(yh, W, sc, x, lv)


def test_noalloc_repeated_calls_stay_exact(qam):
    """The scratch keeps the last call's contents: a run of calls of mixed
    routes and sizes gives the same bits as qam_qmatvec every time."""
    seq = [(1024, 2048, 1, False), (256, 512, 4, True), (1024, 2048, 1, False), (128, 4096, 1, False),
           (256, 512, 4, True)]
    for j, (N, K, B, per_req) in enumerate(seq):
        print(f"noalloc sequence step {j}: N={N} K={K} B={B}", flush=True)
        W, sc, x, lv, pm = make_case(qam, N, K, B, per_req, seed=7 + j)
        xt, lvt = dev(x), dev(lv)
        y = torch.empty((B, N), dtype=torch.float32, device="cuda")
        qam.qmatvec_noalloc(xt, pm, lvt, y)
        y_ref = qam.qmatvec(xt, pm, lvt)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32)), j
        check_oracle(y.cpu().numpy(), W, sc, x, lv)


def test_noalloc_replays_from_a_captured_graph(qam):
    """The call as a caller under HIP graph capture uses it: captured once
    (after a first eager call has set the scratch up), replayed several
    times with eager work in between, every replay equal bit for bit to
    qam_qmatvec on the same inputs."""
    for (N, K, B, per_req) in [(1024, 4096, 1, False), (512, 2048, 8, True)]:
        print(f"noalloc graph N={N} K={K} B={B}", flush=True)
        W, sc, x, lv, pm = make_case(qam, N, K, B, per_req, seed=77 + B)
        xt, lvt = dev(x), dev(lv)
        y = torch.zeros((B, N), dtype=torch.float32, device="cuda")
        qam.qmatvec_noalloc(xt, pm, lvt, y)
        want = qam.qmatvec(xt, pm, lvt)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            qam.qmatvec_noalloc(xt, pm, lvt, y)
        torch.cuda.synchronize()
        for rep in range(3):
            y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().view(np.uint32), want.cpu().numpy().view(np.uint32)), rep
            other = torch.zeros_like(y)
            qam.qmatvec_noalloc(dev(np.ones_like(x)), pm, lvt, other)   # eager work on the same scratch
            torch.cuda.synchronize()

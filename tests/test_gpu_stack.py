"""Stored-stack file through the C ABI on the device: the library's writer
against the oracle's bytes, depth reads into caller device memory against
truncation, and products on loaded matrices against the oracle."""

import numpy as np
import pytest

import oracle as O
import oracle.stack_file as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qam():
    import query_adaptive_mixed_amd as Q
    return Q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


SHAPES = [(64, 64), (192, 1088), (512, 256), (128, 4096)]


def make_mats(seed=0):
    rng = np.random.default_rng(seed)
    mats = []
    for i, (N, K) in enumerate(SHAPES):
        W = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
        sc = rng.uniform(0.001, 0.02, size=N).astype(np.float32)
        mats.append((f"L0.m{i}", W, sc))
    return mats


def test_library_writes_the_oracle_bytes(qam, tmp_path):
    mats = make_mats(1)
    packed = [qam.pack_slices(dev(W), dev(sc)) for _, W, sc in mats]
    path = tmp_path / "lib.qamstack"
    print("stack write", path, flush=True)
    qam.stack_write(path, packed, [m[0] for m in mats])
    got = path.read_bytes()
    want = S.stack_bytes(mats)
    assert len(got) == len(want)
    assert got == want


@pytest.mark.parametrize("bits", [2, 4, 6, 8])
def test_depth_read_gives_truncated_codes(qam, tmp_path, bits):
    mats = make_mats(2)
    path = str(tmp_path / "o.qamstack")
    S.write_stack(path, mats)
    print(f"stack read bits={bits}", flush=True)
    loaded, nread = qam.stack_read(path, bits)
    assert nread == S.read_bytes(SHAPES, bits // 2)
    for (name, W, sc), pm in zip(mats, loaded):
        full = torch.full((pm.n_blocks,), 4, dtype=torch.uint8, device="cuda")   # read every plane
        codes = qam.unpack_codes(pm, full).cpu().numpy()
        assert np.array_equal(codes.astype(np.int64), O.truncate(W, bits)), name
        assert np.array_equal(pm.buf[W.size:].cpu().numpy().view(np.float32), sc)


def test_read_a_range_into_given_buffers(qam, tmp_path):
    mats = make_mats(3)
    path = str(tmp_path / "r.qamstack")
    S.write_stack(path, mats)
    # prefill the destinations with garbage: the read must overwrite or zero every byte
    out = []
    for _, W, sc in mats[1:3]:
        pm = qam.pack_slices(dev(np.full_like(W, 85)), dev(np.full_like(sc, 7.0)))
        out.append(pm)
    loaded, nread = qam.stack_read(path, 4, first=1, count=2, out=out)
    assert nread == S.read_bytes(SHAPES[1:3], 2)
    for (name, W, sc), pm in zip(mats[1:3], loaded):
        full = torch.full((pm.n_blocks,), 4, dtype=torch.uint8, device="cuda")
        assert np.array_equal(qam.unpack_codes(pm, full).cpu().numpy().astype(np.int64), O.truncate(W, 4)), name


@pytest.mark.parametrize("bits", [4, 8])
def test_products_on_loaded_matrices(qam, tmp_path, bits):
    """A matrix loaded at `bits` gives, at any map with depths <= bits, the
    same bits as the matrix packed in device memory, and the oracle's values."""
    mats = make_mats(4)
    path = str(tmp_path / "p.qamstack")
    S.write_stack(path, mats)
    loaded, _ = qam.stack_read(path, bits)
    rng = np.random.default_rng(bits)
    for (name, W, sc), pm in zip(mats, loaded):
        N, K = W.shape
        nb = N // 64
        lv = rng.integers(0, bits // 2 + 1, size=nb).astype(np.uint8)
        x = rng.standard_normal((1, K)).astype(np.float32)
        print(f"product on loaded {name} N={N} K={K} bits={bits}", flush=True)
        y = qam.qmatvec(dev(x), pm, dev(lv)).cpu().numpy()
        ref_pm = qam.pack_slices(dev(W), dev(sc))
        y_ref = qam.qmatvec(dev(x), ref_pm, dev(lv)).cpu().numpy()
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), name
        ref = O.qmatvec_ref(W, sc, x, lv)
        tol = O.qmatvec_tolerance(W, sc, x, lv)
        assert np.all(np.abs(y.astype(np.float64) - ref) <= tol), name


def test_write_then_read_round_trip_through_the_library(qam, tmp_path):
    mats = make_mats(5)
    packed = [qam.pack_slices(dev(W), dev(sc)) for _, W, sc in mats]
    path = tmp_path / "rt.qamstack"
    qam.stack_write(path, packed)
    hdr, ents = qam.stack_info(path)
    assert hdr.n_matrices == len(mats) and [e.name for e in ents] == [b""] * len(mats)
    loaded, _ = qam.stack_read(path, 8)
    for pm, src in zip(loaded, packed):
        assert torch.equal(pm.buf, src.buf)

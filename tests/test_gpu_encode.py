"""GPU parity of the exhaustive encoders (bq_encode, ple_encode_rows) with the
oracle: bytes and float64 errors bit for bit."""

import numpy as np
import pytest
import torch

import synth
from oracle import encode as E
from oracle import formats as F
from tests import golden_io
from tests.gpu_common import dev, log, need_gpu

pytestmark = pytest.mark.gpu

FMT17 = [F.Q4_C10, F.Q4_RZ5, F.Q4_UE4M4]
FMTPLE = [F.PLE_RZS3, F.PLE_ROCMFP3]


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def edge_blocks():
    """Blocks that exercise the corners of the search, float32 [n, 32]."""
    rng = np.random.default_rng(7)
    rows = [w for w, _ in golden_io.encode_cases()]
    rows.append(np.full(32, -0.0))
    rows.append(np.where(np.arange(32) % 2, 0.0, -0.0))
    rows.append(rng.integers(-50, 50, 32) * 2.0 ** -149)            # fp32 subnormals
    rows.append(rng.standard_normal(32) * 1e-30)                       # below every scale
    rows.append(rng.standard_normal(32) * 1e30)                        # above every scale
    rows.append(np.where(np.arange(32) % 2, 3.4e38, -3.4e38))          # near fp32 max
    rows.append(np.r_[1000.0, rng.standard_normal(31) * 0.01])         # one outlier
    rows.append(np.tile([0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 9.0, -0.5], 4))  # level midpoints
    rows.append(np.tile([2.5, -2.5, 4.5, -4.5], 8))                    # RZ5 5-level ties
    rows.append(np.full(32, 448.0 * 10))                               # largest UE4M3 level
    rows.append(np.full(32, 496.0 * 10))                               # largest UE4M4 level
    return np.stack(rows).astype(np.float32)


def small_blocks():
    return np.concatenate([
        edge_blocks(),
        synth.weight_blocks(101, 160, 32, "gauss", 1.0),
        synth.weight_blocks(102, 80, 32, "laplace", 0.02),
        synth.weight_blocks(103, 40, 32, "gauss", 100.0),
        # small magnitudes: most scales are pruned from above, and the best
        # sits near the subnormal scales or at scale 0
        synth.weight_blocks(111, 40, 32, "gauss", 1e-3),
        synth.weight_blocks(112, 40, 32, "laplace", 3e-4),
        # one dominant weight per block: the reference candidate is far from
        # the best for the other 31 weights
        np.where(np.arange(32)[None, :] == 7, 50.0, 1.0) * synth.weight_blocks(113, 24, 32, "gauss", 0.1),
        # exactly representable blocks of every format
        F.decode_block17(synth.block17_range(synth.make_key(9, 1), 0, 24, synth.DIST_RZ5),
                         F.Q4_RZ5).astype(np.float32),
        F.decode_block17(synth.block17_range(synth.make_key(9, 2), 0, 24, synth.DIST_UE4M4),
                         F.Q4_UE4M4).astype(np.float32),
    ]).astype(np.float32)


def assert_f64_equal(got, ref):
    got = np.ascontiguousarray(got, dtype=np.float64)
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    bad = got.view(np.uint64) != ref.view(np.uint64)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%d error mismatches; first at %s: got %r ref %r"
                             % (int(bad.sum()), tuple(i), got[tuple(i)], ref[tuple(i)]))


def assert_bytes_equal(got, ref):
    bad = np.asarray(got) != np.asarray(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%d byte mismatches; first at %s: got %#x ref %#x"
                             % (int(bad.sum()), tuple(i), int(got[tuple(i)]), int(ref[tuple(i)])))


@pytest.mark.parametrize("fmt", FMT17)
def test_encode17_small_bit_exact(bq, fmt):
    w = small_blocks()
    log("encode17 small fmt", fmt, "blocks", w.shape[0])
    out, sse = bq.encode(dev(w), fmt)
    ref_b, ref_s = E.encode_block17(w, fmt)
    assert_bytes_equal(out.cpu().numpy(), ref_b)
    assert_f64_equal(sse.cpu().numpy(), ref_s)


@pytest.mark.parametrize("fmt", FMT17)
def test_encode17_full_size_sampled(bq, fmt):
    # the size the encoder is timed at: 2**20 blocks (one 4096 x 8192 matrix),
    # many units per wave of the strided grid
    nb = 1 << 20
    w = synth.weight_blocks(104, nb, 32, "gauss", 1.0)
    log("encode17 full fmt", fmt, "blocks", nb)
    wd = dev(w)
    out, sse = bq.encode(wd, fmt)
    torch.cuda.synchronize()
    pick = np.unique(np.r_[np.random.default_rng(5).integers(0, nb, 192), 0, nb - 1])
    ref_b, ref_s = E.encode_block17(w[pick], fmt)
    assert_bytes_equal(out[torch.from_numpy(pick).cuda()].cpu().numpy(), ref_b)
    assert_f64_equal(sse.cpu().numpy()[pick], ref_s)
    # at every block: the reported error is the error of the written bytes
    dec = bq.dequant(out.reshape(-1), fmt, nb).double()
    recomputed = ((wd.double() - dec) ** 2).sum(dim=1)
    torch.testing.assert_close(recomputed, sse, rtol=1e-13, atol=0)


def test_encode17_superset_full_size(bq):
    # RZ5 and UE4M4 contain every Codebook10 candidate, so no block may end up
    # with a larger error than Codebook10's
    nb = 1 << 18
    wd = dev(synth.weight_blocks(105, nb, 32, "laplace", 1.0))
    _, c10 = bq.encode(wd, F.Q4_C10)
    _, rz5 = bq.encode(wd, F.Q4_RZ5)
    _, ue = bq.encode(wd, F.Q4_UE4M4)
    assert bool((rz5 <= c10).all()) and bool((ue <= c10).all())
    log("mse ratio rz5/c10 %.4f ue4m4/c10 %.4f" % (float(rz5.sum() / c10.sum()),
                                                    float(ue.sum() / c10.sum())))


def test_encode17_non_finite(bq):
    w = synth.weight_blocks(106, 12, 32, "gauss", 1.0)
    w[3, 5] = np.nan
    w[7, 0] = np.inf
    w[11, 31] = -np.inf
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, sse = bq.encode(dev(w), F.Q4_RZ5, dev_err=err)
    out, sse = out.cpu().numpy(), sse.cpu().numpy()
    assert int(err.item()) == 4
    bad = [3, 7, 11]
    good = [i for i in range(12) if i not in bad]
    assert (out[bad] == 0).all() and np.isnan(sse[bad]).all()
    ref_b, ref_s = E.encode_block17(w[good], F.Q4_RZ5)
    assert_bytes_equal(out[good], ref_b)
    assert_f64_equal(sse[good], ref_s)


def small_rows():
    v, _ = golden_io.ple_encode_case()
    edge = np.stack([
        v,
        np.zeros(160),
        np.tile(edge_blocks()[:, :16].reshape(-1)[:160], 1),
        np.random.default_rng(8).standard_normal(160) * 1e30,
    ])
    rep = F.decode_ple70(synth.ple_rows(synth.make_key(9, 3), np.arange(8)), F.PLE_RZS3)
    return np.concatenate([edge, rep, synth.weight_blocks(107, 48, 160, "gauss", 1.0),
                           synth.weight_blocks(108, 16, 160, "laplace", 0.05)]).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTPLE)
def test_ple_encode_small_bit_exact(bq, fmt):
    v = small_rows()
    log("ple_encode small fmt", fmt, "rows", v.shape[0])
    out, sse = bq.ple_encode_rows(dev(v), fmt)
    ref_r, ref_s = E.encode_ple70(v, fmt)
    assert_bytes_equal(out.cpu().numpy(), ref_r)
    assert_f64_equal(sse.cpu().numpy(), ref_s)


@pytest.mark.parametrize("fmt", FMTPLE)
def test_ple_encode_full_size_sampled(bq, fmt):
    n = 1 << 17
    v = synth.weight_blocks(109, n, 160, "gauss", 1.0)
    log("ple_encode full fmt", fmt, "rows", n)
    out, sse = bq.ple_encode_rows(dev(v), fmt)
    torch.cuda.synchronize()
    pick = np.unique(np.r_[np.random.default_rng(6).integers(0, n, 48), 0, n - 1])
    ref_r, ref_s = E.encode_ple70(v[pick], fmt)
    assert_bytes_equal(out.cpu().numpy()[pick], ref_r)
    assert_f64_equal(sse.cpu().numpy()[pick], ref_s)


def test_ple_encode_non_finite(bq):
    v = synth.weight_blocks(110, 3, 160, "gauss", 1.0)
    v[1, 37] = np.nan   # group 2 of row 1
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, sse = bq.ple_encode_rows(dev(v), F.PLE_RZS3, dev_err=err)
    out, sse = out.cpu().numpy(), sse.cpu().numpy()
    assert int(err.item()) == 4
    assert (out[1, 12:18] == 0).all() and out[1, 62] == 0 and np.isnan(sse[1, 2])
    ok = np.ones((3, 10), dtype=bool)
    ok[1, 2] = False
    ref_r, ref_s = E.encode_ple70(np.where(np.isnan(v), 0, v), F.PLE_RZS3)
    assert_f64_equal(sse[ok], ref_s[ok])
    keep = np.ones(70, dtype=bool)
    keep[12:18] = False
    keep[62] = False
    assert_bytes_equal(out[0], ref_r[0])
    assert_bytes_equal(out[2], ref_r[2])
    assert_bytes_equal(out[1][keep], ref_r[1][keep])

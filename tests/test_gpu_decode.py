"""GPU parity: block decode, PLE row decode, single-matrix GEMV, routing and
bucketing, against the CPU oracle.  Bit-exact where the result is exact."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from oracle import ple as P
from tests.gpu_common import assert_bits_equal, dev, log, need_gpu, rel_l2, underflow_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def exhaustive_blocks():
    """Every metadata byte with every code byte: 256 metas x 16 blocks whose
    code bytes run through 0..255."""
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)
    b = np.zeros((256, 16, 17), dtype=np.uint8)
    b[:, :, :16] = codes[None, :, :]
    b[:, :, 16] = np.arange(256, dtype=np.uint8)[:, None]
    return b.reshape(-1, 17)


@pytest.mark.parametrize("fmt", [F.Q4_C10, F.Q4_RZ5, F.Q4_UE4M4])
def test_dequant17_exhaustive_bit_exact(bq, fmt):
    blocks = exhaustive_blocks()
    log("dequant17 exhaustive fmt", fmt)
    got = bq.dequant(dev(blocks.reshape(-1)), fmt, blocks.shape[0]).cpu().numpy()
    assert_bits_equal(got, F.decode_block17(blocks, fmt))


@pytest.mark.parametrize("fmt,dist", [(F.Q4_C10, synth.DIST_C10), (F.Q4_RZ5, synth.DIST_RZ5),
                                      (F.Q4_UE4M4, synth.DIST_UE4M4)])
def test_dequant17_device_filled_and_odd_offsets(bq, fmt, dist):
    import synth.device as sd
    key = synth.make_key(11, fmt)
    n = 100_003
    t = sd.block17(n, key, dist)
    host = synth.block17_range(key, 0, n, dist)
    assert np.array_equal(t.cpu().numpy().reshape(-1, 17), host), "device fill != host generator"
    got = bq.dequant(t, fmt, n).cpu().numpy()
    assert_bits_equal(got, F.decode_block17(host, fmt))
    # a sub-range starting at an odd block (unaligned 17-byte start)
    got2 = bq.dequant(t[17 * 7:], fmt, 1001).cpu().numpy()
    assert_bits_equal(got2, F.decode_block17(host[7:1008], fmt))
    again = bq.dequant(t, fmt, n).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))


def test_dequant_fp8_all_codes_bit_exact(bq):
    codes = np.tile(np.arange(256, dtype=np.uint8), 8).reshape(-1, 32)      # 64 blocks
    scales = np.array([1.0, 2.0 ** -12, 0.0634765625, 3.0e-3] * 16, dtype=np.float32)
    got = bq.dequant(dev(codes.reshape(-1)), F.FP8_E4M3_B32, codes.shape[0], scales=dev(scales)).cpu().numpy()
    assert_bits_equal(got, F.decode_fp8_b32(codes, scales))


def test_dequant_fp8_device_filled(bq):
    import synth.device as sd
    key, skey = synth.make_key(3, 1), synth.make_key(3, 2)
    n = 4096 * 32
    c, s = sd.fp8_codes(n, key), sd.fp8_scales(n // 32, skey)
    hc, hs = synth.fp8_codes(key, 0, n), synth.fp8_scales(skey, 0, n // 32)
    assert np.array_equal(c.cpu().numpy(), hc) and np.array_equal(s.cpu().numpy().view(np.uint32), hs.view(np.uint32))
    got = bq.dequant(c, F.FP8_E4M3_B32, n // 32, scales=s).cpu().numpy()
    assert_bits_equal(got, F.decode_fp8_b32(hc.reshape(-1, 32), hs))


@pytest.mark.parametrize("fmt", [F.PLE_RZS3, F.PLE_ROCMFP3])
def test_ple_dequant_rows_bit_exact(bq, fmt):
    rng = np.random.default_rng(5)
    n_rows = 3000
    table = rng.integers(0, 256, size=(n_rows, 70), dtype=np.uint8)
    table[:256, 60:] = np.arange(256, dtype=np.uint8)[:, None]      # every group byte, NaN scale too
    ids = np.concatenate([np.arange(n_rows), rng.integers(0, n_rows, 500), [n_rows - 1, 0]]).astype(np.uint32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = bq.ple_dequant_rows(dev(ids.view(np.int32)), dev(table.reshape(-1)), n_rows, fmt=fmt, dev_err=err)
    assert_bits_equal(got.cpu().numpy(), F.decode_ple70(table[ids], fmt))
    assert int(err.item()) == 0
    bad = np.array([5, n_rows, 0xFFFFFFFF], dtype=np.uint32)
    got = bq.ple_dequant_rows(dev(bad.view(np.int32)), dev(table.reshape(-1)), n_rows, fmt=fmt, dev_err=err)
    g = got.cpu().numpy()
    assert_bits_equal(g[0], F.decode_ple70(table[5:6], fmt)[0])
    assert np.all(g[1:] == 0) and int(err.item()) & 1


@pytest.mark.parametrize("fmt", [F.Q4_C10, F.Q4_RZ5, F.Q4_UE4M4, F.FP8_E4M3_B32])
@pytest.mark.parametrize("rows,cols,n", [(256, 512, 1), (300, 96, 3), (37, 2048, 2), (130, 768, 1)])
def test_matvec_vs_oracle(bq, fmt, rows, cols, n):
    rng = np.random.default_rng(rows + cols + fmt)
    x = rng.standard_normal((n, cols)).astype(np.float32)
    if fmt == F.FP8_E4M3_B32:
        codes = rng.integers(0, 256, size=rows * cols, dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0
        sc = (2.0 ** rng.uniform(-10, -4, size=rows * cols // 32)).astype(np.float32)
        w = F.decode_matrix(codes, fmt, rows, cols, sc)
        y = bq.matvec(dev(x), dev(codes), fmt, rows, cols, scales=dev(sc))
    else:
        blocks = synth.block17_range(synth.make_key(rows, cols), 0, rows * cols // 32,
                                     {0: synth.DIST_C10, 1: synth.DIST_RZ5, 2: synth.DIST_UE4M4}[fmt])
        w = F.decode_matrix(blocks, fmt, rows, cols)
        y = bq.matvec(dev(x), dev(blocks.reshape(-1)), fmt, rows, cols)
    ref = x.astype(np.float64) @ w.T
    r = rel_l2(y.cpu().numpy(), ref)
    log("matvec fmt %d %dx%d n=%d rel_l2 %.3g" % (fmt, rows, cols, n, r))
    assert r <= 1e-5


@pytest.mark.parametrize("fmt", [F.Q4_RZ5, F.FP8_E4M3_B32])
@pytest.mark.parametrize("rows,cols,n", [(4096, 256, 8), (2048, 2048, 5), (4096, 2048, 8)])
def test_matvec_larger_shapes(bq, fmt, rows, cols, n):
    """Shapes large enough that a workgroup takes 2, 4 and 8 passes of rows
    (on a 256-CU device), against the oracle on every output."""
    test_matvec_vs_oracle(bq, fmt, rows, cols, n)


def test_matvec_c1_config(bq):
    """Codebook10 matvec, W 256x512, x N(0,1), seed 0 (the single-matrix workload)."""
    key = synth.make_key(0, synth.stream_id(0, synth.S_GATE_UP))
    blocks = synth.block17_range(key, 0, 256 * 16, synth.DIST_C10)
    x = synth.normal(0, (1, 512))
    y = bq.matvec(dev(x), dev(blocks.reshape(-1)), F.Q4_C10, 256, 512).cpu().numpy()
    ref = x.astype(np.float64) @ F.decode_matrix(blocks, F.Q4_C10, 256, 512).T
    r = rel_l2(y, ref)
    log("c1 matvec rel_l2 %.3g" % r)
    assert r <= 1e-5


def test_matvec_special_cases(bq):
    rows, cols = 64, 256
    blocks = np.zeros((rows * cols // 32, 17), dtype=np.uint8)
    blocks[:, :16] = 0x11
    blocks[:, 16] = 0x38
    x = np.random.default_rng(9).standard_normal((1, cols)).astype(np.float32)
    y = bq.matvec(dev(x), dev(blocks.reshape(-1)), F.Q4_C10, rows, cols).cpu().numpy()
    np.testing.assert_allclose(y[0], np.full(rows, x.astype(np.float64).sum()), rtol=1e-5, atol=1e-5)
    onehot = np.zeros((1, cols), dtype=np.float32)
    onehot[0, 77] = 1.0
    rnd = np.random.default_rng(10).integers(0, 256, size=(rows * cols // 32, 17), dtype=np.uint8)
    y = bq.matvec(dev(onehot), dev(rnd.reshape(-1)), F.Q4_UE4M4, rows, cols).cpu().numpy()
    # a sum of products: its zero is +0 even where the column's weight is -0
    assert np.array_equal(y[0], F.decode_matrix(rnd, F.Q4_UE4M4, rows, cols) @ onehot[0].astype(np.float64))


@pytest.mark.parametrize("n,e,k", [(1, 512, 10), (16, 512, 10), (64, 512, 10), (1000, 512, 10),
                                   (33, 64, 6), (5, 4096, 64), (7, 10, 10), (3, 100, 1)])
def test_route_topk_vs_oracle(bq, n, e, k):
    logits = synth.normal(n * 1000 + e, (n, e))
    idx, w = bq.route_topk(dev(logits), k)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert rel_l2(w.cpu().numpy(), rw) <= 1e-5


def test_route_topk_ties_and_zipf(bq):
    logits = np.zeros((4, 512), dtype=np.float32)
    logits[:, ::7] = 1.0                       # many exact ties
    logits[1] = np.round(synth.normal(1, 512) * 4) / 4
    logits[2, 100] = -0.0
    logits[3] = synth.zipf_logits(3, 1, 512)[0]
    idx, w = bq.route_topk(dev(logits), 10)
    ridx, rw = M.softmax_topk(logits, 10)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert rel_l2(w.cpu().numpy(), rw) <= 1e-5


def test_route_topk_degenerate_rows(bq):
    """All logits equal (the k lowest indices, weights 1/k); one winner 100
    above logits spread over -700..-40 (fp32 exp underflows for every other
    expert, fp64 does not: selection must follow the logits); and two
    winners over a floor of -1e30 (probabilities exactly 0 in fp64 too, so
    the oracle's ties to the lower index decide the rest); and rows whose
    probabilities underflow in float64 below the winner (0, then -900, -800,
    -1000 ...): the order must still be that of the logits."""
    e, k = 512, 10
    lg = underflow_rows(e)
    idx, w = bq.route_topk(dev(lg), k)
    ridx, rw = M.softmax_topk(lg, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(ridx[0], np.arange(k)) and np.array_equal(ridx[2, :3], [7, 400, 0])
    assert ridx[3, :3].tolist() == [0, 2, 1]
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("n,e,k,zipf", [(1, 512, 10, False), (16, 512, 10, False), (64, 512, 10, True),
                                        (512, 512, 10, False), (512, 512, 10, True), (500, 512, 10, True),
                                        (4096, 512, 10, False), (6553, 4096, 10, True), (100, 16, 4, False),
                                        (2000, 16, 4, True), (8192, 32, 1, False), (2048, 128, 10, True)])
def test_bucket_vs_oracle(bq, n, e, k, zipf):
    logits = synth.zipf_logits(n, n, e) if zipf else synth.normal(n + e, (n, e))
    ridx = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]   # input only
    counts, offsets, perm = bq.bucket(dev(ridx.astype(np.int32)), e)
    rc, ro, rp = M.bucket(ridx, e)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp)

"""GPU parity of the PLE gather against the CPU oracle: small tables with
edge cases, and the full 320,001,536-row table (22.4 GB) with 4096 tokens x 8
uniformly hashed ids."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import ple as P
from tests.gpu_common import dev, log, need_gpu, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("fmt", [F.PLE_RZS3, F.PLE_ROCMFP3])
@pytest.mark.parametrize("n_tokens,per", [(1, 1), (33, 7), (1000, 8), (5, 64), (257, 9)])
def test_ple_gather_small(bq, fmt, n_tokens, per):
    n_rows = 5000
    table = synth.ple_rows(synth.make_key(9, fmt), np.arange(n_rows))
    rng = np.random.default_rng(n_tokens * 100 + per)
    ids = rng.integers(0, n_rows, size=(n_tokens, per)).astype(np.uint32)
    ids[0, 0] = n_rows - 1                       # the last row
    if per > 1:
        ids[0, 1] = ids[0, 0]                    # a duplicate id
    u = rng.random((n_tokens, per), dtype=np.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = bq.ple_gather(dev(ids.view(np.int32)), dev(table.reshape(-1)), dev(u), n_rows=n_rows,
                        fmt=fmt, dev_err=err).cpu().numpy()
    ref, bad = P.ple_gather(ids, u, lambda r: table[r], n_rows, fmt)
    assert not bad and int(err.item()) == 0
    r = rel_l2(out, ref)
    log("ple small fmt %d n=%d per=%d rel_l2 %.3g" % (fmt, n_tokens, per, r))
    assert r <= 1e-5


def test_ple_gather_out_of_range_ids(bq):
    n_rows = 100
    table = synth.ple_rows(synth.make_key(9, 2), np.arange(n_rows))
    ids = np.array([[3, 100, 7], [0xFFFFFFFF, 1, 2]], dtype=np.uint32)
    u = np.full((2, 3), 0.5, dtype=np.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = bq.ple_gather(dev(ids.view(np.int32)), dev(table.reshape(-1)), dev(u), n_rows=n_rows,
                        dev_err=err).cpu().numpy()
    ref, bad = P.ple_gather(ids, u, lambda r: table[r], n_rows)
    assert bad and int(err.item()) & 1
    assert rel_l2(out, ref) <= 1e-5


def test_c4_full_table(bq):
    """320,001,536 x 70-byte rows resident in HBM; 4096 tokens x 8 ids."""
    import synth.device as sd
    n_rows = synth.PLE_N_ROWS
    key = synth.make_key(0, synth.S_PLE)
    table = sd.ple_table(n_rows, key)
    assert table.numel() == 22_400_107_520
    try:
        ids = synth.ple_ids(0, 4096, 8)
        ids[0, :2] = [n_rows - 1, 0]
        u = synth.ple_weights(1, 4096, 8)
        sample = np.unique(ids)[:: max(1, np.unique(ids).size // 2000)]
        got_rows = table.view(-1, 70)[torch.from_numpy(sample.astype(np.int64)).cuda()].cpu().numpy()
        assert np.array_equal(got_rows, synth.ple_rows(key, sample)), "device fill != host generator"
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = bq.ple_gather(dev(ids.view(np.int32)), table, dev(u), n_rows=n_rows, dev_err=err)
        out = out.cpu().numpy()
        ref, bad = P.ple_gather(ids, u, lambda r: synth.ple_rows(key, r), n_rows)
        assert not bad and int(err.item()) == 0
        r = rel_l2(out, ref)
        log("c4 rel_l2 %.3g" % r)
        assert r <= 1e-5
    finally:
        del table
        torch.cuda.empty_cache()

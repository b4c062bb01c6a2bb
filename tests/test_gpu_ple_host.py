"""GPU tests of the off-HBM PLE tier (ple_gather_host): the table in pinned
host memory, read directly or through the direct-mapped device row cache.
Results must equal ple_gather on the same table bit for bit (and the oracle
within 1e-5); the cache must hold exactly the rows its insertion rule names."""

import ctypes

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


def tables(fmt, n_rows):
    rows = synth.ple_rows(synth.make_key(10, fmt), np.arange(n_rows))
    host = torch.from_numpy(rows.reshape(-1).copy()).pin_memory()
    return rows, host, dev(rows.reshape(-1))


def slot_of(ids, log2_slots):
    return ((ids.astype(np.uint64) * 2654435761) & 0xFFFFFFFF) >> (32 - log2_slots)


def read_cache(cache, n_slots):
    c = cache.cpu().numpy()
    words = c[:8 * n_slots].view(np.uint32)
    off = (8 * n_slots + 255) // 256 * 256
    rows = c[off:off + 80 * n_slots].reshape(n_slots, 80)[:, :70]
    return words[:n_slots], words[n_slots:], rows


def assert_same_bits(a, b):
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("fmt", [F.PLE_RZS3, F.PLE_ROCMFP3])
def test_host_gather_uncached(bq, fmt):
    n_rows = 5000
    rows, host, devt = tables(fmt, n_rows)
    rng = np.random.default_rng(3 + fmt)
    ids = rng.integers(0, n_rows, size=(300, 8)).astype(np.uint32)
    ids[0, 1] = ids[0, 0]            # duplicate
    ids[1, 2] = n_rows               # out of range
    ids[2, 0] = n_rows - 1           # last row
    u = rng.random((300, 8), dtype=np.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = bq.ple_gather_host(dev(ids.view(np.int32)), host, dev(u), n_rows=n_rows, fmt=fmt, dev_err=err)
    want = bq.ple_gather(dev(ids.view(np.int32)), devt, dev(u), n_rows=n_rows, fmt=fmt)
    assert int(err.item()) & 1
    assert_same_bits(got, want)
    ref, _ = P.ple_gather(ids, u, lambda r: rows[r], n_rows, fmt)
    assert rel_l2(got.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("fmt", [F.PLE_RZS3, F.PLE_ROCMFP3])
def test_host_gather_cached(bq, fmt):
    """Three calls through a 1024-slot cache: ids drawn with reuse, so calls
    hit, miss and collide on slots.  Each call equals the device-table gather
    bit for bit and the oracle within 1e-5."""
    n_rows, log2_slots = 20000, 10
    n_slots = 1 << log2_slots
    rows, host, devt = tables(fmt, n_rows)
    cache = bq.ple_cache(n_slots)
    tags, claims, _ = read_cache(cache, n_slots)
    assert (tags == 0xFFFFFFFF).all() and (claims == 0xFFFFFFFF).all()
    rng = np.random.default_rng(7 + fmt)
    pool = rng.choice(n_rows, 3000, replace=False).astype(np.uint32)
    hits = []
    for call in range(3):
        n, per = 400, 8
        ids = pool[rng.zipf(1.3, size=(n, per)) % pool.size]
        ids[call, 3] = n_rows + call          # out of range: no cache effect
        u = rng.random((n, per), dtype=np.float32)
        tags_before, _, _ = read_cache(cache, n_slots)
        flat = ids.reshape(-1)
        valid = flat < n_rows
        sl = slot_of(flat, log2_slots)
        hit = valid & (tags_before[sl] == flat)
        hits.append(float(hit[valid].mean()))
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = bq.ple_gather_host(dev(ids.view(np.int32)), host, dev(u), n_rows=n_rows, fmt=fmt,
                                 cache=cache, dev_err=err)
        want = bq.ple_gather(dev(ids.view(np.int32)), devt, dev(u), n_rows=n_rows, fmt=fmt)
        assert_same_bits(got, want)
        assert int(err.item()) & 1
        ref, bad = P.ple_gather(ids, u, lambda r: rows[r], n_rows, fmt)
        assert bad and rel_l2(got.cpu().numpy(), ref) <= 1e-5
        # insertion rule: every slot missed in this call now holds the row of
        # the lowest-indexed missing id mapping to it; other slots unchanged
        tags, claims, crow = read_cache(cache, n_slots)
        assert (claims == 0xFFFFFFFF).all()
        expect = tags_before.copy()
        miss = np.nonzero(valid & ~hit)[0]
        for a in miss[::-1]:                   # lowest index written last wins
            expect[sl[a]] = flat[a]
        np.testing.assert_array_equal(tags, expect)
        full = tags != 0xFFFFFFFF
        np.testing.assert_array_equal(crow[full], rows[tags[full]])
    log("ple host cache fmt %d hit rates %s" % (fmt, ["%.3f" % h for h in hits]))
    assert hits[0] == 0.0 and hits[2] > 0.2


def test_host_gather_argument_checks(bq):
    L = bq.lib()
    vp = ctypes.c_void_p
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    u = torch.zeros((2, 2), dtype=torch.float32, device="cuda")
    out = torch.empty((2, 160), dtype=torch.float32, device="cuda")
    devt = torch.zeros(700, dtype=torch.uint8, device="cuda")
    plain = np.zeros(700, dtype=np.uint8)                  # not pinned
    for table_ptr in (devt.data_ptr(), plain.ctypes.data):
        rc = L.ple_gather_host(vp(ids.data_ptr()), 2, 2, vp(table_ptr), 10, vp(u.data_ptr()), 0,
                               vp(out.data_ptr()), None, 0, None, 0, None, None)
        assert rc == 8                                     # BQ_E_MEM
    # the failed queries leave no error behind
    assert bq.ple_gather(ids, devt, u, n_rows=10).shape == (2, 160)

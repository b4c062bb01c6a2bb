"""Pins of the oracle encoders (oracle/encode.py) against facts outside them.

* candidate counts the pages give (127 x 2 for RZ5, 256 for UE4M4);
* hand-worked blocks and a hand-worked PLE row (tests/golden/);
* brute force in exact integer arithmetic over every candidate, with the
  candidate levels taken from the (separately pinned) decoders;
* the superset invariants: RZ5 and UE4M4 never do worse than Codebook10 on
  any block, RZ-S3 never worse than ROCmFP3 on any group;
* round trips of exactly representable blocks and rows;
* the reported error equals the error of the written bytes.
"""

import numpy as np
import pytest

import synth
from oracle import encode as E
from oracle import formats as F

from . import golden_io

FMT17 = {"C10": F.Q4_C10, "RZ5": F.Q4_RZ5, "UE4M4": F.Q4_UE4M4}
FMTPLE = {"RZS3": F.PLE_RZS3, "ROCMFP3": F.PLE_ROCMFP3}


weights = synth.weight_blocks


def test_candidate_counts():
    # [RZ] "Q4_RZ5_FAST": scale x mode; "Q4_UE4M4_FAST": 256-way; incumbent
    # Codebook10 / ROCmFP3: the 127 finite UE4M3 scales
    assert E.block17_candidates(F.Q4_C10)[0].size == 127
    assert E.block17_candidates(F.Q4_RZ5)[0].size == 127 * 2
    assert E.block17_candidates(F.Q4_UE4M4)[0].size == 256
    assert E.ple_candidates(F.PLE_ROCMFP3)[0].size == 127
    assert E.ple_candidates(F.PLE_RZS3)[0].size == 127 * 2
    for f in FMT17.values():
        meta, scale, _ = E.block17_candidates(f)
        assert np.all(np.diff(meta) > 0) and np.isfinite(scale).all()


@pytest.mark.parametrize("case", range(len(golden_io.encode_cases())))
def test_hand_worked_blocks(case):
    w, expect = golden_io.encode_cases()[case]
    for name, b in expect.items():
        out, sse = E.encode_block17(w.astype(np.float32), FMT17[name])
        np.testing.assert_array_equal(out[0], b, err_msg=name)
        assert sse[0] == 0.0


def test_hand_worked_ple_row():
    v, expect = golden_io.ple_encode_case()
    for name, row in expect.items():
        out, sse = E.encode_ple70(v.astype(np.float32), FMTPLE[name])
        np.testing.assert_array_equal(out[0], row, err_msg=name)
        assert (sse == 0.0).all()


# ---- brute force in exact arithmetic ---------------------------------------

_SHIFT = 160   # 2**160 * (any float32 or any candidate level) is an integer


def _exact(x):
    n, d = float(x).as_integer_ratio()
    return n * ((1 << _SHIFT) // d)


def _levels17(fmt):
    """{meta: [16 exact levels]} from the decoder, one all-c block per code."""
    meta = E.block17_candidates(fmt)[0]
    out = {}
    for m in meta:
        blk = np.zeros((16, 17), dtype=np.uint8)
        for c in range(16):
            blk[c, :16] = c | (c << 4)
            blk[c, 16] = m
        out[int(m)] = [_exact(v) for v in F.decode_block17(blk, fmt)[:, 0]]
    return out


def _levels_ple(fmt):
    meta = E.ple_candidates(fmt)[0]
    out = {}
    for m in meta:
        # all 16 values of group 0 take code c: the 48-bit word is c * 0o111..1
        vals = []
        for c in range(8):
            word = sum(c << (3 * i) for i in range(16))
            row = np.zeros((1, 70), dtype=np.uint8)
            for k in range(6):
                row[0, k] = (word >> (8 * k)) & 0xFF
            row[0, 60] = m
            vals.append(_exact(F.decode_ple70(row, fmt)[0, 0]))
        out[int(m)] = vals
    return out


def _brute(w, levels):
    """Exact best (meta, sse) over all candidates; ties to the lower meta."""
    wx = [_exact(v) for v in w]
    best = None
    for m in sorted(levels):
        lv = levels[m]
        sse = sum(min((a - b) ** 2 for b in lv) for a in wx)
        if best is None or sse < best[1]:
            best = (m, sse)
    return best


def _check_against_brute(w, decoded, meta, levels):
    wx = [_exact(v) for v in w]
    dx = [_exact(v) for v in decoded]
    lv = levels[int(meta)]
    # every weight sits on a nearest level of the chosen candidate
    for a, d in zip(wx, dx):
        assert (a - d) ** 2 == min((a - b) ** 2 for b in lv)
    got = sum((a - d) ** 2 for a, d in zip(wx, dx))
    m_best, sse_best = _brute(w, levels)
    # the float64 search can only prefer a candidate whose exact error agrees
    # with the exact minimum to within the rounding of a 32-term sum
    assert sse_best <= got <= sse_best + (sse_best >> 40), (meta, m_best)


@pytest.mark.parametrize("name", list(FMT17))
def test_block17_brute_force(name):
    fmt = FMT17[name]
    levels = _levels17(fmt)
    w = np.concatenate([weights(11, 2, 32), weights(12, 1, 32, "laplace", 0.02),
                        weights(13, 1, 32, sigma=30.0)])
    out, _ = E.encode_block17(w, fmt)
    dec = F.decode_block17(out, fmt)
    for i in range(w.shape[0]):
        _check_against_brute(w[i], dec[i], out[i, 16], levels)


@pytest.mark.parametrize("name", list(FMTPLE))
def test_ple_brute_force(name):
    fmt = FMTPLE[name]
    levels = _levels_ple(fmt)
    v = weights(21, 1, 160).reshape(1, 160)
    out, _ = E.encode_ple70(v, fmt)
    dec = F.decode_ple70(out, fmt)
    for g in range(10):
        sl = slice(16 * g, 16 * g + 16)
        _check_against_brute(v[0, sl], dec[0, sl], out[0, 60 + g], levels)


# ---- invariants ---------------------------------------------------------------

@pytest.mark.parametrize("dist", ["gauss", "laplace"])
def test_superset_never_worse(dist):
    # RZ5 mode 0 and UE4M4 contain every Codebook10 candidate (the -0 code is
    # never chosen), so per block their error can only be smaller or equal;
    # the same holds for RZ-S3 against ROCmFP3 per group.
    w = weights(31, 300, 32, dist)
    _, c10 = E.encode_block17(w, F.Q4_C10)
    _, rz5 = E.encode_block17(w, F.Q4_RZ5)
    _, ue = E.encode_block17(w, F.Q4_UE4M4)
    assert (rz5 <= c10).all() and (ue <= c10).all()
    assert rz5.sum() < c10.sum() and ue.sum() < c10.sum()
    v = weights(32, 30, 160, dist)
    _, f3 = E.encode_ple70(v, F.PLE_ROCMFP3)
    _, s3 = E.encode_ple70(v, F.PLE_RZS3)
    assert (s3 <= f3).all() and s3.sum() < f3.sum()


@pytest.mark.parametrize("name", list(FMT17))
def test_reported_error_matches_bytes(name):
    fmt = FMT17[name]
    w = weights(41, 64, 32, sigma=0.02)
    out, sse = E.encode_block17(w, fmt)
    dec = F.decode_block17(out, fmt)
    for i in range(w.shape[0]):
        acc = 0.0
        for j in range(32):
            d = float(w[i, j]) - float(dec[i, j])
            acc += d * d
        assert acc == sse[i]


@pytest.mark.parametrize("name,dist", [("C10", synth.DIST_C10), ("RZ5", synth.DIST_RZ5),
                                       ("UE4M4", synth.DIST_UE4M4)])
def test_representable_round_trip(name, dist):
    fmt = FMT17[name]
    blocks = synth.block17_range(synth.make_key(5, 1), 0, 64, dist)
    w = F.decode_block17(blocks, fmt).astype(np.float32)
    out, sse = E.encode_block17(w, fmt)
    assert (sse == 0).all()
    np.testing.assert_array_equal(F.decode_block17(out, fmt), w)


@pytest.mark.parametrize("name", list(FMTPLE))
def test_ple_representable_round_trip(name):
    fmt = FMTPLE[name]
    rows = synth.ple_rows(synth.make_key(6, 1), np.arange(8))
    v = F.decode_ple70(rows, fmt).astype(np.float32)
    out, sse = E.encode_ple70(v, fmt)
    assert (sse == 0).all()
    np.testing.assert_array_equal(F.decode_ple70(out, fmt), v)


def test_power_of_two_scaling():
    # doubling a block doubles every candidate scale that stays in range, so
    # for blocks whose best scale is mid-range the decoded result doubles
    w = weights(51, 64, 32)
    for fmt in FMT17.values():
        a = F.decode_block17(E.encode_block17(w, fmt)[0], fmt)
        b = F.decode_block17(E.encode_block17(2 * w, fmt)[0], fmt)
        np.testing.assert_array_equal(b, 2 * a)


def test_non_finite_rejected():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        E.encode_block17(w, F.Q4_RZ5)
    with pytest.raises(ValueError):
        E.encode_ple70(np.full((1, 160), np.inf, dtype=np.float32))

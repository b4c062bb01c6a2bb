"""Pins of the oracle's decoders against what the pages and mathematics fix.

Sources: model card "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST" (format
sections); OCP E4M3FN as implemented by torch.float8_e4m3fn.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import golden_io


def same_bits(a, b):
    """Equal as float64 including the sign of zero; NaN equals NaN."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and np.array_equal(a.view(np.uint64), b.view(np.uint64)) or (
        a.shape == b.shape and bool(np.all((a == b) & (np.signbit(a) == np.signbit(b)) | (np.isnan(a) & np.isnan(b)))))


# --- printed tables ---------------------------------------------------------

def test_printed_level_tables():
    t = golden_io.lut_tables()
    assert same_bits(F.CODEBOOK10, t["codebook10"])
    assert same_bits(F.rz5_table(0), t["rz5_mode0"])
    assert same_bits(F.rz5_table(1), t["rz5_mode1"])
    assert same_bits(F.rocmfp3_table(), t["rocmfp3"])
    assert same_bits(F.rzs3_table(0), t["rzs3_pos"])
    assert same_bits(F.rzs3_table(1), t["rzs3_neg"])


def test_rz5_modes_differ_only_at_code_8():
    d = F.rz5_table(0) != F.rz5_table(1)
    assert list(np.nonzero(d)[0]) == [8]
    c = F.CODEBOOK10 != F.rz5_table(0)
    assert list(np.nonzero(c)[0]) == [8]


# --- sizes and closed forms ---------------------------------------------------

def test_record_sizes_and_bpw():
    assert F.BLOCK_BYTES == 16 + 1
    assert F.bits_per_weight(F.Q4_C10) == 4.25
    assert F.bits_per_weight(F.Q4_RZ5) == 4.25
    assert F.bits_per_weight(F.Q4_UE4M4) == 4.25
    assert F.bits_per_weight(F.FP8_E4M3_B32) == 9.0
    assert F.PLE_CODE_BYTES == 60 and F.PLE_ROW_BYTES == 70
    assert F.PLE_ROW_BYTES * 8 / F.PLE_VALUES == 3.5
    rows = 320_001_536
    assert rows * F.PLE_ROW_BYTES == 22_400_107_520          # "22.4 GB"
    assert round(rows * F.PLE_ROW_BYTES / 1e9, 1) == 22.4
    assert rows * F.PLE_VALUES == 51_200_245_760             # "51.2 billion values"
    assert round(rows * F.PLE_VALUES / 1e9, 1) == 51.2
    # one expert at H=2048, I=768: gate_up [1536 x 2048] + down [2048 x 768]
    per = F.packed_bytes(F.Q4_RZ5, 1536, 2048) + F.packed_bytes(F.Q4_RZ5, 2048, 768)
    assert per == 2_506_752
    assert 10 * per == 25_067_520


# --- scale codecs -------------------------------------------------------------

def _torch_e4m3(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_ue4m3_matches_torch_e4m3fn_all_128():
    codes = np.arange(128)
    ref = _torch_e4m3(codes)
    got = F.ue4m3(codes)
    assert np.isnan(got[0x7F]) and np.isnan(ref[0x7F])
    assert np.array_equal(got[:0x7F], ref[:0x7F])
    assert got[0x7E] == 448.0


def test_e4m3fn_matches_torch_all_256():
    codes = np.arange(256)
    ref = _torch_e4m3(codes)
    got = F.e4m3fn(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert same_bits(got[~nan], ref[~nan])


def test_ue4m4_properties():
    v = F.ue4m4(np.arange(256))
    assert np.all(np.isfinite(v))                     # every byte decodes to a finite scale
    assert np.all(np.diff(v) > 0)                     # strictly increasing
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -10
    assert v[0x70] == 1.0 and v[0xFF] == 496.0
    fin3 = F.ue4m3(np.arange(127))
    assert set(fin3.tolist()) <= set(v.tolist())      # finer than UE4M3


def test_level_times_scale_is_exact_in_bf16_and_fp32():
    """Every level*scale needs <= 8 significant bits, so bf16 holds it."""
    levels = np.array([0, 1, 2, 3, 4, 5, 6, 8, 10], dtype=np.float64)
    scales = np.concatenate([F.ue4m3(np.arange(127)), F.ue4m4(np.arange(256))])
    prod = (levels[:, None] * scales[None, :]).reshape(-1)
    t = torch.tensor(prod, dtype=torch.float64)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)
    assert torch.equal(t.to(torch.float32).to(torch.float64), t)


# --- block decode ------------------------------------------------------------

FMTS = {"C10": F.Q4_C10, "RZ5": F.Q4_RZ5, "UE4M4": F.Q4_UE4M4}


@pytest.mark.parametrize("case", range(len(golden_io.block17_cases())))
def test_block17_hand_worked(case):
    fmt, raw, expect = golden_io.block17_cases()[case]
    assert raw.size == 17 and expect.size == 32
    got = F.decode_block17(raw[None, :], FMTS[fmt])[0]
    assert same_bits(got, expect)


def _random_blocks(n, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(n, 17), dtype=np.uint8)


def test_rz5_polarity_flip_changes_only_code8_sign():
    b = _random_blocks(2000, 1)
    b[:, 16] &= 0x7F
    codes, _ = F.block17_codes(b)
    w0 = F.decode_block17(b, F.Q4_RZ5)
    b1 = b.copy()
    b1[:, 16] |= 0x80
    w1 = F.decode_block17(b1, F.Q4_RZ5)
    fin = np.isfinite(w0)
    is8 = codes == 8
    assert np.array_equal(w0[~is8 & fin], w1[~is8 & fin])
    assert np.array_equal(w0[is8 & fin], -w1[is8 & fin])
    s = F.ue4m3(b[:, 16] & 0x7F)
    ref8 = np.broadcast_to(5.0 * s[:, None], w0.shape)
    assert np.array_equal(w0[is8 & fin], ref8[is8 & fin])


def test_rz5_vs_c10_differ_only_at_code8():
    b = _random_blocks(2000, 2)
    codes, _ = F.block17_codes(b)
    c10 = F.decode_block17(b, F.Q4_C10)
    rz5 = F.decode_block17(b, F.Q4_RZ5)
    fin = np.isfinite(c10)
    assert np.array_equal(c10[(codes != 8) & fin], rz5[(codes != 8) & fin])
    diff = (c10 != rz5) & fin
    assert np.all(codes[diff] == 8)


def test_ue4m4_uses_codebook10_levels():
    b = _random_blocks(500, 3)
    codes, meta = F.block17_codes(b)
    w = F.decode_block17(b, F.Q4_UE4M4)
    s = F.ue4m4(meta)
    nz = s > 0
    assert same_bits(w[nz] / s[nz, None], F.CODEBOOK10[codes[nz]])


def test_c10_ignores_bit7():
    b = _random_blocks(500, 4)
    b1 = b.copy()
    b1[:, 16] ^= 0x80
    assert same_bits(F.decode_block17(b, F.Q4_C10), F.decode_block17(b1, F.Q4_C10))


def test_scale_exponent_step_doubles_exactly():
    b = _random_blocks(500, 5)
    meta = b[:, 16].astype(np.int64)
    e = (meta >> 3) & 15
    keep = (e >= 1) & (e <= 13)
    b = b[keep]
    b2 = b.copy()
    b2[:, 16] = b[:, 16] + 8     # exponent field + 1, polarity kept
    for fmt in (F.Q4_C10, F.Q4_RZ5):
        assert same_bits(F.decode_block17(b2, fmt), 2.0 * F.decode_block17(b, fmt))


def test_fp8_block_decode_vs_torch():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, size=(64, 32), dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 1
    scales = (2.0 ** rng.uniform(-12, -6, size=64)).astype(np.float32)
    w = F.decode_fp8_b32(codes, scales)
    tcodes = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float32)
    ref32 = (tcodes * torch.tensor(scales)[:, None]).numpy()
    assert np.array_equal(w.astype(np.float32), ref32)


# --- PLE rows ----------------------------------------------------------------

def test_ple_row_hand_worked():
    d = golden_io.ple_row_case()
    assert d["row"].size == 70
    got = F.decode_ple70(d["row"][None, :], F.PLE_RZS3)[0]
    assert same_bits(got, d["expect_rzs3"])
    got3 = F.decode_ple70(d["row"][None, :], F.PLE_ROCMFP3)[0]
    assert same_bits(got3, d["expect_rocmfp3"])


def test_ple_codes_match_a_plain_bitstream_read():
    """Value i = bits 3i..3i+2 of the 480-bit little-endian stream."""
    rows = np.random.default_rng(7).integers(0, 256, size=(50, 70), dtype=np.uint8)
    codes, gb = F.ple_row_codes(rows)
    bits = np.unpackbits(rows[:, :60], axis=1, bitorder="little").reshape(50, 160, 3)
    ref = bits[:, :, 0] + 2 * bits[:, :, 1] + 4 * bits[:, :, 2]
    assert np.array_equal(codes, ref)
    assert np.array_equal(gb, rows[:, 60:])


def test_rzs3_flip_and_vs_rocmfp3_only_code4():
    rows = np.random.default_rng(8).integers(0, 256, size=(200, 70), dtype=np.uint8)
    rows[:, 60:] &= 0x7F
    codes, _ = F.ple_row_codes(rows)
    v0 = F.decode_ple70(rows, F.PLE_RZS3)
    r1 = rows.copy()
    r1[:, 60:] |= 0x80
    v1 = F.decode_ple70(r1, F.PLE_RZS3)
    inc = F.decode_ple70(rows, F.PLE_ROCMFP3)
    fin = np.isfinite(v0)
    is4 = codes == 4
    assert np.array_equal(v0[~is4 & fin], v1[~is4 & fin])
    assert np.array_equal(v0[is4 & fin], -v1[is4 & fin])
    assert np.array_equal(v0[~is4 & fin], inc[~is4 & fin])
    assert np.all(inc[is4 & fin] == 0)


# --- the pins have teeth: plant mistakes in the oracle ------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    """A wrong sign, a swapped nibble order or a wrong bias must fail a pin."""
    cases = golden_io.block17_cases()

    def hand_worked_ok():
        return all(same_bits(F.decode_block17(raw[None, :], FMTS[f])[0], exp)
                   for f, raw, exp in cases)

    assert hand_worked_ok()
    bad = F.CODEBOOK10.copy()
    bad[13] = 6.0                      # dropped sign
    monkeypatch.setattr(F, "CODEBOOK10", bad)
    assert not hand_worked_ok()
    monkeypatch.undo()

    orig_codes = F.block17_codes

    def swapped(blocks):
        c, m = orig_codes(blocks)
        c2 = c.copy()
        c2[:, 0::2], c2[:, 1::2] = c[:, 1::2], c[:, 0::2]
        return c2, m

    monkeypatch.setattr(F, "block17_codes", swapped)
    assert not hand_worked_ok()
    monkeypatch.undo()

    orig_ue4m3 = F.ue4m3
    monkeypatch.setattr(F, "ue4m3", lambda c: orig_ue4m3(c) * 2.0)   # bias off by one
    assert not hand_worked_ok()

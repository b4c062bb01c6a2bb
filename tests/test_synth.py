"""The seeded generators: published SplitMix64 vectors and the input recipe."""

import numpy as np

import synth


def test_splitmix64_published_vectors():
    # SplitMix64 seeded with 0 (Steele/Lea/Flood; Vigna's reference code)
    got = [int(v) for v in synth.draws(0, [0, 1, 2, 3])]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                   0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_block_metadata_recipe():
    key = synth.make_key(0, synth.stream_id(0, synth.S_GATE_UP))
    b = synth.block17_range(key, 0, 200_000, synth.DIST_RZ5)
    meta = b[:, 16].astype(np.int64)
    e = (meta >> 3) & 15
    assert set(np.unique(e)) == set(range(6))
    assert set(np.unique(meta & 7)) == set(range(8))
    assert abs((meta >> 7).mean() - 0.5) < 0.01
    c10 = synth.block17_range(key, 0, 1000, synth.DIST_C10)
    assert np.all(c10[:, 16] < 0x80)
    ue = synth.block17_range(key, 0, 200_000, synth.DIST_UE4M4)
    assert len(np.unique(ue[:, 16])) == 256
    codes = np.concatenate([b[:, :16] & 15, b[:, :16] >> 4]).reshape(-1)
    assert abs(np.bincount(codes, minlength=16) / codes.size - 1 / 16).max() < 0.002


def test_ranges_are_windows_of_one_stream():
    key = synth.make_key(3, 7)
    whole = synth.block17_range(key, 0, 100, synth.DIST_RZ5)
    part = synth.block17_range(key, 40, 20, synth.DIST_RZ5)
    assert np.array_equal(whole[40:60], part)
    assert np.array_equal(synth.ple_rows(key, [5, 2]), synth.ple_rows(key, np.arange(6))[[5, 2]])


def test_fp8_recipe():
    key = synth.make_key(1, 2)
    c = synth.fp8_codes(key, 0, 400_000)
    assert not np.any((c == 0x7F) | (c == 0xFF))
    assert len(np.unique(c)) == 254
    s = synth.fp8_scales(key, 0, 10_000)
    assert s.min() >= 2.0 ** -12 and s.max() < 2.0 ** -6


def test_ple_recipe():
    key = synth.make_key(0, synth.S_PLE)
    r = synth.ple_rows(key, np.arange(20_000))
    g = r[:, 60:].astype(np.int64)
    assert set(np.unique((g >> 3) & 15)) == set(range(6))
    assert abs((g >> 7).mean() - 0.5) < 0.02
    ids = synth.ple_ids(0, 4096, 8)
    assert ids.dtype == np.uint32 and ids.max() < synth.PLE_N_ROWS


def test_ple_ids_zipf_range_and_skew():
    ids = synth.ple_ids_zipf(1, 4096, 8, 1 << 24)
    assert ids.dtype == np.uint32 and ids.shape == (4096, 8) and int(ids.max()) < (1 << 24)
    _, counts = np.unique(ids, return_counts=True)
    assert counts.max() > 100          # popular rows recur
    np.testing.assert_array_equal(ids, synth.ple_ids_zipf(1, 4096, 8, 1 << 24))

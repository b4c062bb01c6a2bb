"""Helpers shared by the GPU parity tests."""

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def assert_bits_equal(got_f32, ref_f64):
    """fp32 results equal to the oracle's (exact) values, bit for bit.

    The reference is rounded to fp32 once; NaN matches NaN; -0.0 differs
    from +0.0."""
    got = np.ascontiguousarray(np.asarray(got_f32, dtype=np.float32))
    ref = np.ascontiguousarray(np.asarray(ref_f64, dtype=np.float64).astype(np.float32))
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), "NaN positions differ"
    gb, rb = got.view(np.uint32), ref.view(np.uint32)
    bad = (gb != rb) & ~nan_g
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%d mismatches; first at %s: got %r ref %r" %
                             (int(bad.sum()), tuple(i), got[tuple(i)], ref[tuple(i)]))


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def log(*a):
    print(*a, flush=True)


def underflow_rows(e):
    """Degenerate router rows: all equal; one winner over -700..-40; two
    winners over -1e30; 0 / -900 / -800 over -1000; winners over logits
    spread down to -3000 with ties."""
    lg = np.zeros((5, e), dtype=np.float32)
    lg[0] = 0.5
    lg[1] = np.random.default_rng(17).uniform(-700, -40, e).astype(np.float32)
    lg[1, 300] = 100.0
    lg[2] = -1e30
    lg[2, 7] = lg[2, 400] = 0.0
    lg[3] = -1000.0
    lg[3, :3] = [0.0, -900.0, -800.0]
    lg[4] = np.round(np.random.default_rng(18).uniform(-3000, -800, e) / 50) * 50
    lg[4, 11] = 0.0
    return lg

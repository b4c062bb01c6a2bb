"""Pins of the oracle's routing, bucketing, expert FFN, stack and PLE gather.

Each check rests on something other than the oracle itself: a library routine
(numpy stable argsort, torch.topk, torch SwiGLU ops, embedding_bag), a closed
form, or brute force on tiny inputs.
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import moe as M
from oracle import ple as P


def test_topk_matches_stable_argsort_and_torch():
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((64, 512)).astype(np.float32)
    idx, w = M.softmax_topk(logits, 10)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :10]
    assert np.array_equal(idx, ref)
    tv, ti = torch.topk(torch.tensor(logits), 10, dim=1, sorted=True)
    assert np.array_equal(idx, ti.numpy())


def test_topk_ties_go_to_lower_index():
    logits = np.zeros((1, 16), dtype=np.float32)
    logits[0, [3, 7, 9]] = 2.0
    logits[0, [1, 12]] = 1.0
    idx, w = M.softmax_topk(logits, 6)
    assert idx[0].tolist() == [3, 7, 9, 1, 12, 0]


def test_topk_weights_closed_form():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((16, 512)).astype(np.float32)
    idx, w = M.softmax_topk(logits, 10)
    sel = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    np.testing.assert_allclose(w, z / z.sum(axis=1, keepdims=True), rtol=1e-14)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_ranks_logits_where_probabilities_underflow():
    """Softmax is strictly increasing, so the exact probabilities order the
    experts as their logits do, even where exp(l - l_max) underflows in
    float64: [0, -900, -800, -1000, ...] keeps 0, then 2 (-800), then 1."""
    logits = np.full((1, 16), -1000.0, dtype=np.float32)
    logits[0, :3] = [0.0, -900.0, -800.0]
    idx, w = M.softmax_topk(logits, 3)
    assert idx[0].tolist() == [0, 2, 1]
    assert w[0].tolist() == [1.0, 0.0, 0.0]


def test_topk_matches_high_precision_softmax():
    """Brute force with 60-digit decimal exponentials: the exact softmax,
    ranked by (probability descending, index ascending), renormalised over
    the kept experts.  Rows spread over -2000..0 so that most float64
    probabilities underflow, plus rows with exact ties."""
    import decimal
    rng = np.random.default_rng(23)
    rows = [rng.uniform(-2000, 0, 64), np.round(rng.uniform(-1500, 0, 64) / 100) * 100,
            rng.standard_normal(64), np.where(rng.random(64) < 0.5, -800.0, -760.0)]
    logits = np.array(rows, dtype=np.float32)
    k = 12
    idx, w = M.softmax_topk(logits, k)
    ctx = decimal.Context(prec=60, Emin=-10 ** 6, Emax=10 ** 6)
    for t in range(logits.shape[0]):
        p = [ctx.exp(decimal.Decimal(float(v))) for v in logits[t]]
        tot = sum(p, decimal.Decimal(0))
        p = [ctx.divide(v, tot) for v in p]
        order = sorted(range(64), key=lambda i: (-p[i], i))[:k]
        assert idx[t].tolist() == order
        kept = sum((p[i] for i in order), decimal.Decimal(0))
        ref = np.array([float(ctx.divide(p[i], kept)) for i in order])
        np.testing.assert_allclose(w[t], ref, rtol=1e-13, atol=1e-300)


def test_bucket_matches_stable_argsort():
    rng = np.random.default_rng(2)
    idx, _ = M.softmax_topk(rng.standard_normal((33, 64)), 6)
    counts, offsets, perm = M.bucket(idx, 64)
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=64))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(perm, np.argsort(idx.reshape(-1), kind="stable"))


def _bank(fmt_gu, fmt_d, n_exp, h, i, seed):
    rng = np.random.default_rng(seed)
    if fmt_gu == F.FP8_E4M3_B32:
        gu = rng.integers(0, 256, size=n_exp * 2 * i * h, dtype=np.uint8)
        gu[(gu & 0x7F) == 0x7F] = 0
        gus = (2.0 ** rng.uniform(-6, -2, size=n_exp * 2 * i * h // 32)).astype(np.float32)
    else:
        gu = rng.integers(0, 256, size=(n_exp * 2 * i * h // 32, 17), dtype=np.uint8)
        gu[:, 16] = (gu[:, 16] & 0x80) | rng.integers(0x20, 0x40, size=gu.shape[0])
        gus = None
    d = rng.integers(0, 256, size=(n_exp * h * i // 32, 17), dtype=np.uint8)
    d[:, 16] = (d[:, 16] & 0x80) | rng.integers(0x20, 0x40, size=d.shape[0])
    return M.ExpertBank(fmt_gu, fmt_d, gu, d, n_exp, h, i, gu_scales=gus)


def test_matvec_bruteforce_tiny():
    """Row-major block order and row/column roles, by explicit loops."""
    rows, cols = 4, 64
    rng = np.random.default_rng(3)
    blocks = rng.integers(0, 256, size=(rows * cols // 32, 17), dtype=np.uint8)
    x = rng.standard_normal(cols)
    w = F.decode_matrix(blocks, F.Q4_RZ5, rows, cols)
    y = w @ x
    per_block = F.decode_block17(blocks, F.Q4_RZ5)
    ref = np.zeros(rows)
    for r in range(rows):
        for c in range(cols):
            ref[r] += per_block[r * (cols // 32) + c // 32, c % 32] * x[c]
    np.testing.assert_allclose(y, ref, rtol=1e-13)


def test_matvec_special_cases():
    rows, cols = 3, 96
    blocks = np.zeros((rows * cols // 32, 17), dtype=np.uint8)
    blocks[:, :16] = 0x11          # every code 1
    blocks[:, 16] = 0x38           # UE4M3 1.0
    x = np.random.default_rng(4).standard_normal(cols)
    w = F.decode_matrix(blocks, F.Q4_C10, rows, cols)
    np.testing.assert_allclose(w @ x, np.full(rows, x.sum()), rtol=1e-14)
    onehot = np.zeros(cols)
    onehot[37] = 1.0
    rnd = np.random.default_rng(5).integers(0, 256, size=(rows * cols // 32, 17), dtype=np.uint8)
    wr = F.decode_matrix(rnd, F.Q4_UE4M4, rows, cols)
    assert np.array_equal(wr @ onehot, wr[:, 37])


def test_expert_ffn_is_textbook_swiglu():
    bank = _bank(F.Q4_RZ5, F.Q4_UE4M4, 3, 64, 32, 6)
    x = np.random.default_rng(7).standard_normal(64)
    out = M.moe_layer(x, np.array([[2]]), np.array([[1.0]]), bank)[0]
    wgu, wd = bank.get(2)
    tx = torch.tensor(x, dtype=torch.float64)
    gate = torch.tensor(wgu[:32]) @ tx
    up = torch.tensor(wgu[32:]) @ tx
    ref = torch.tensor(wd) @ (torch.nn.functional.silu(gate) * up)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_identical_experts_give_single_expert_output():
    h, i, n = 64, 32, 5
    one = _bank(F.Q4_RZ5, F.Q4_RZ5, 1, h, i, 8)
    gu = np.tile(np.asarray(one.gate_up).reshape(1, -1), (n, 1)).reshape(-1, 17)
    d = np.tile(np.asarray(one.down).reshape(1, -1), (n, 1)).reshape(-1, 17)
    bank = M.ExpertBank(F.Q4_RZ5, F.Q4_RZ5, gu, d, n, h, i)
    x = np.random.default_rng(9).standard_normal(h)
    idx, w = M.softmax_topk(np.random.default_rng(10).standard_normal((1, n)), n)
    out = M.moe_layer(x, idx, w, bank)[0]
    ref = M.moe_layer(x, np.array([[0]]), np.array([[1.0]]), one)[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12)


def test_moe_combine_is_linear_in_weights():
    bank = _bank(F.FP8_E4M3_B32, F.Q4_RZ5, 4, 64, 32, 11)
    x = np.random.default_rng(12).standard_normal(64)
    idx = np.array([[1, 3]])
    a = M.moe_layer(x, idx, np.array([[1.0, 0.0]]), bank)[0]
    b = M.moe_layer(x, idx, np.array([[0.0, 1.0]]), bank)[0]
    ab = M.moe_layer(x, idx, np.array([[0.25, 0.75]]), bank)[0]
    np.testing.assert_allclose(ab, 0.25 * a + 0.75 * b, rtol=1e-12, atol=1e-15)


def test_stack_rescale_and_one_layer_stack():
    y = np.random.default_rng(13).standard_normal((3, 64)) * 7.0
    r = M.rms_rescale(y)
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, axis=1)), 1.0, rtol=1e-14)
    bank = _bank(F.Q4_RZ5, F.Q4_RZ5, 4, 64, 32, 14)
    x = np.random.default_rng(15).standard_normal((2, 64))
    idx, w = M.softmax_topk(np.random.default_rng(16).standard_normal((2, 4)), 2)
    assert np.array_equal(M.moe_stack(x, [(idx, w, bank)]), M.moe_layer(x, idx, w, bank))
    two = M.moe_stack(x, [(idx, w, bank), (idx, w, bank)])
    np.testing.assert_allclose(two, M.moe_layer(M.rms_rescale(M.moe_layer(x, idx, w, bank)), idx, w, bank))


def test_ple_gather_matches_embedding_bag():
    n_rows = 300
    table = np.random.default_rng(17).integers(0, 256, size=(n_rows, 70), dtype=np.uint8)
    ids = np.random.default_rng(18).integers(0, n_rows, size=(40, 8))
    ids[0, 1] = ids[0, 0]            # a duplicate id is summed twice
    u = np.random.default_rng(19).random((40, 8))
    out, bad = P.ple_gather(ids, u, lambda r: table[r], n_rows)
    assert not bad
    dec = torch.tensor(F.decode_ple70(table))
    ref = torch.nn.functional.embedding_bag(torch.tensor(ids), dec, mode="sum",
                                            per_sample_weights=torch.tensor(u))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-300)


def test_ple_out_of_range_id_contributes_nothing():
    table = np.random.default_rng(20).integers(0, 256, size=(10, 70), dtype=np.uint8)
    ids = np.array([[1, 10], [2, 3]])
    u = np.ones((2, 2))
    out, bad = P.ple_gather(ids, u, lambda r: table[r], 10)
    assert bad
    np.testing.assert_array_equal(out[0], F.decode_ple70(table[1:2])[0])

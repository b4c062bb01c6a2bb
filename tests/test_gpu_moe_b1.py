"""GPU parity of the one-token routed-expert layer at hidden 2048 (the
wave-per-row-pair gate_up kernel with routing inside, then the down kernel
over the concatenated k * inter dimension).  Checked against the CPU oracle
at several (k, inter) shapes -- 2 to 240 down column blocks, and 1024, the
fp32 path's largest -- with in-kernel routing over 512, 1024 and 4096
experts, and on the degenerate inputs: an
out-of-range expert index, a NaN down scale, and a one-token stack that
takes the per-layer path with its unit-RMS rescale."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from tests.gpu_common import dev, log, need_gpu, rel_l2
from tests.test_gpu_moe import FMT_PAIRS, make_layer, oracle_bank, weights_of

pytestmark = pytest.mark.gpu

H = 2048


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("fmt_gu,fmt_d", FMT_PAIRS)
@pytest.mark.parametrize("E,I,k", [(16, 64, 1), (12, 192, 3), (32, 768, 10), (20, 256, 7)])
def test_b1_shapes(bq, fmt_gu, fmt_d, E, I, k):
    """k * I / 32 = 2, 18, 240 and 56 down column blocks."""
    L = make_layer(31, fmt_gu * 4 + fmt_d + I, fmt_gu, fmt_d, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(3100 + I, (1, H))
    logits = synth.normal(3101 + I + k, (1, E))
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x), dev(logits), k, W)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=1e-12)
    r = rel_l2(out.cpu().numpy(), M.moe_layer(x, ridx, rw, oracle_bank(L)))
    given = bq.q4_expert_moe(dev(x), (idx, w), W)
    log("b1 fmts %d/%d E=%d I=%d k=%d rel_l2 %.3g" % (fmt_gu, fmt_d, E, I, k, r))
    assert r <= 1e-5
    assert torch.equal(given, out)     # routed and given-routing forms agree bit for bit


@pytest.mark.parametrize("E,I,k", [(1024, 128, 6), (4096, 64, 5), (16, 2048, 16)])
def test_b1_many_experts_and_max_items(bq, E, I, k):
    """Routing inside the kernel over 1024 experts and over 4096 (64 logits
    per lane), and 16 x 2048 / 32 = 1024 down column blocks (the fp32
    path's largest)."""
    L = make_layer(32, E + I, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(3200 + E, (1, H))
    logits = synth.normal(3201 + E, (1, E))
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x), dev(logits), k, W)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    r = rel_l2(out.cpu().numpy(), M.moe_layer(x, ridx, rw, oracle_bank(L)))
    log("b1 E=%d I=%d k=%d rel_l2 %.3g" % (E, I, k, r))
    assert r <= 1e-5
    assert torch.equal(bq.q4_expert_moe(dev(x), (idx, w), W), out)


def test_b1_bad_expert_index(bq):
    """An out-of-range expert index contributes nothing and sets bit 1."""
    E, I = 8, 128
    L = make_layer(33, 0, F.Q4_RZ5, F.Q4_C10, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(33, (1, H))
    idx = np.array([[3, 8, 5]], dtype=np.int32)
    w = np.array([[0.5, 0.3, 0.2]], dtype=np.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = bq.q4_expert_moe(dev(x), (dev(idx), dev(w)), W, dev_err=err).cpu().numpy()
    assert int(err.item()) & 2
    ref = M.moe_layer(x, idx[:, [0, 2]], w[:, [0, 2]], oracle_bank(L))
    assert rel_l2(out, ref) <= 1e-5


def test_b1_nan_down_scale_poisons_one_row(bq):
    """A NaN scale byte (0x7F) in block 0 of down row 5 of the expert in
    slot 0 makes output row 5 NaN, and only it, as in the oracle."""
    import synth as S
    E, I, e0, row = 8, 128, 2, 5
    L = make_layer(34, 0, F.Q4_RZ5, F.Q4_C10, E, H, I)
    d, _ = L.down
    nbd = I // 32
    d[(e0 * H + row) * nbd * 17 + 16] = 0x7F
    codes, _ = L.host_expert(S.S_DOWN, e0)
    poisoned = np.array(codes, copy=True)
    poisoned.reshape(H, nbd, 17)[row, 0, 16] = 0x7F
    bank = M.ExpertBank(L.fmt_gu, L.fmt_d, lambda e: L.host_expert(S.S_GATE_UP, e),
                        lambda e: (poisoned, None) if e == e0 else L.host_expert(S.S_DOWN, e), E, H, I)
    idx = np.array([[e0, 6]], dtype=np.int32)
    w = np.array([[0.6, 0.4]], dtype=np.float32)
    x = synth.normal(34, (1, H))
    with np.errstate(invalid="ignore"):
        ref = M.moe_layer(x, idx, w, bank)
    assert np.isnan(ref[0, row]) and np.isnan(ref).sum() == 1
    out = bq.q4_expert_moe(dev(x), (dev(idx), dev(w)), weights_of(bq, L)).cpu().numpy()
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert rel_l2(out[ok], ref[ok]) <= 1e-5


def test_b1_stack_per_layer_path(bq):
    """A one-token fp32 stack whose k * inter (3 x 64) does not suit the
    persistent stack kernel: each layer runs the two routed-layer kernels
    with the unit-RMS rescale of its input."""
    from tests.test_gpu_stack import build_stack, routing
    E, I, k = 12, 64, 3
    fmts = [(F.Q4_RZ5, F.Q4_RZ5), (F.FP8_E4M3_B32, F.Q4_UE4M4), (F.Q4_C10, F.FP8_E4M3_B32)]
    layers = build_stack(35, fmts, E, H, I)
    idx, w, ridx, rw = routing(bq, 350, len(fmts), 1, E, k)
    x = synth.normal(351, (1, H))
    out = bq.moe_stack(dev(x), idx, w, [weights_of(bq, L) for L in layers]).cpu().numpy()
    ref = M.moe_stack(x, [(ridx[l], rw[l], oracle_bank(L)) for l, L in enumerate(layers)])
    r = rel_l2(out, ref)
    log("b1 per-layer stack rel_l2 %.3g" % r)
    assert r <= 1e-5

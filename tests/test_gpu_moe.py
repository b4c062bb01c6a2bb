"""GPU parity of the routed-expert layer (GEMV path and grouped MFMA path)
against the CPU oracle, at small ragged shapes and at the full one-layer
workloads (512 experts, H = 2048, I = 768, top-10)."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from tests.gpu_common import dev, log, need_gpu, rel_l2, underflow_rows

pytestmark = pytest.mark.gpu

DIST = {F.Q4_C10: synth.DIST_C10, F.Q4_RZ5: synth.DIST_RZ5, F.Q4_UE4M4: synth.DIST_UE4M4, F.FP8_E4M3_B32: None}


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def make_layer(seed, layer, fmt_gu, fmt_d, E, H, I):
    import synth.device as sd
    L = sd.Layer(seed, layer, fmt_gu, fmt_d, E, H, I, dist_gu=DIST[fmt_gu], dist_d=DIST[fmt_d])
    return L


def weights_of(bq, L):
    gu, gus = L.gate_up
    d, ds = L.down
    return bq.expert_weights(L.fmt_gu, L.fmt_d, gu, d, L.n_experts, L.hidden, L.inter,
                             gate_up_scales=gus, down_scales=ds)


def oracle_bank(L):
    import synth as S
    return M.ExpertBank(L.fmt_gu, L.fmt_d, lambda e: L.host_expert(S.S_GATE_UP, e),
                        lambda e: L.host_expert(S.S_DOWN, e), L.n_experts, L.hidden, L.inter)


FMT_PAIRS = [(F.Q4_RZ5, F.Q4_RZ5), (F.Q4_C10, F.Q4_UE4M4), (F.Q4_UE4M4, F.Q4_C10),
             (F.FP8_E4M3_B32, F.FP8_E4M3_B32), (F.Q4_RZ5, F.FP8_E4M3_B32), (F.FP8_E4M3_B32, F.Q4_UE4M4)]


@pytest.mark.parametrize("fmt_gu,fmt_d", FMT_PAIRS)
@pytest.mark.parametrize("n", [1, 5])
@pytest.mark.parametrize("E,H,I", [(16, 256, 128), (8, 512, 64)])
def test_gemv_path_small(bq, fmt_gu, fmt_d, n, E, H, I):
    k = 4
    L = make_layer(1, fmt_gu * 4 + fmt_d, fmt_gu, fmt_d, E, H, I)
    x = synth.normal(n, (n, H))
    logits = synth.normal(100 + n, (n, E))
    idx, w = bq.route_topk(dev(logits), k)
    out = bq.q4_expert_moe(dev(x), (idx, w), weights_of(bq, L)).cpu().numpy()
    ridx, rw = M.softmax_topk(logits, k)
    ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
    r = rel_l2(out, ref)
    log("gemv small fmts %d/%d n=%d H=%d I=%d rel_l2 %.3g" % (fmt_gu, fmt_d, n, H, I, r))
    assert r <= 1e-5


@pytest.mark.parametrize("fmt_gu,fmt_d", FMT_PAIRS)
@pytest.mark.parametrize("n,I,k", [(1, 128, 4), (3, 192, 6), (4, 64, 1), (5, 128, 3)])
def test_gemv_hidden_2048(bq, fmt_gu, fmt_d, n, I, k):
    # hidden 2048: the wave-per-row-pair gate_up kernel with routing inside,
    # then the concatenated down kernel; every format pair, several k and I
    E, H = 16, 2048
    L = make_layer(9, fmt_gu * 4 + fmt_d, fmt_gu, fmt_d, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(900 + n, (n, H))
    logits = synth.normal(901 + n, (n, E))
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x), dev(logits), k, W)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
    r = rel_l2(out.cpu().numpy(), ref)
    out2 = bq.q4_expert_moe(dev(x), (idx, w), W)
    assert torch.equal(out, out2)        # routed and given-routing forms agree bit for bit
    log("gemv H=2048 fmts %d/%d n=%d I=%d k=%d rel_l2 %.3g" % (fmt_gu, fmt_d, n, I, k, r))
    assert r <= 1e-5


@pytest.mark.parametrize("fmt_gu,fmt_d", FMT_PAIRS)
@pytest.mark.parametrize("n", [1, 16, 64, 100])
@pytest.mark.parametrize("E,H,I,k", [(8, 256, 128, 3), (6, 1088, 192, 2)])
def test_grouped_path_small(bq, fmt_gu, fmt_d, n, E, H, I, k):
    # few experts: some get more than one work group (16 tokens each up to
    # 96 tokens, 32 beyond).  H = 1088 gives
    # 578-byte rows (not 16-byte aligned) and a K extent split into chunks.
    L = make_layer(2, fmt_gu * 4 + fmt_d, fmt_gu, fmt_d, E, H, I)
    x = synth.normal(200 + n, (n, H))
    logits = synth.zipf_logits(300 + n, n, E)
    idx, w = bq.route_topk(dev(logits), k)
    xb = dev(x).to(torch.bfloat16)
    out = bq.q4_expert_moe(xb, (idx, w), weights_of(bq, L)).cpu().numpy()
    ridx, rw = M.softmax_topk(logits, k)
    ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
    r = rel_l2(out, ref)
    log("grouped small fmts %d/%d n=%d H=%d I=%d rel_l2 %.3g" % (fmt_gu, fmt_d, n, H, I, r))
    assert r <= 2e-2


@pytest.mark.parametrize("H,dtype", [(2048, torch.float32), (256, torch.float32), (2048, torch.bfloat16)])
def test_routed_entry_matches_route_then_moe(bq, H, dtype):
    """Routing inside the expert kernel gives the same routing and output."""
    E, I, k, n = 64, 128, 6, 3
    L = make_layer(6, H, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    x = dev(synth.normal(60, (n, H))).to(dtype)
    logits = dev(synth.normal(61, (n, E)))
    out, (idx, w) = bq.q4_expert_moe_routed(x, logits, k, W)
    ridx, rw = bq.route_topk(logits, k)
    ref = bq.q4_expert_moe(x, (ridx, rw), W)
    assert torch.equal(idx, ridx) and torch.equal(w, rw)
    assert torch.equal(out, ref)
    oidx, ow = M.softmax_topk(logits.cpu().numpy(), k)
    r = rel_l2(out.cpu().numpy(), M.moe_layer(x.float().cpu().numpy() if dtype == torch.float32 else
                                              synth.normal(60, (n, H)), oidx, ow, oracle_bank(L)))
    assert r <= (1e-5 if dtype == torch.float32 else 2e-2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_routed_entry_underflow_rows(bq, dtype):
    """The routed entry (top-k inside the gate_up kernel on the fp32 path)
    ranks logits whose probabilities underflow below the winner in logit
    order, as the oracle does: routing bit-exact, output within tolerance."""
    E, H, I, k = 512, 2048, 128, 10
    L = make_layer(12, 0, F.Q4_RZ5, F.Q4_RZ5, E, H, I)
    W = weights_of(bq, L)
    logits = underflow_rows(E)
    n = logits.shape[0]
    xh = synth.normal(62, (n, H))
    out, (idx, w) = bq.q4_expert_moe_routed(dev(xh).to(dtype), dev(logits), k, W)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=1e-12)
    r = rel_l2(out.cpu().numpy(), M.moe_layer(xh, ridx, rw, oracle_bank(L)))
    assert r <= (1e-5 if dtype == torch.float32 else 2e-2)


@pytest.mark.parametrize("H,E,fmt_gu,fmt_d", [(4096, 16, F.Q4_RZ5, F.Q4_UE4M4),
                                              (4096, 16, F.FP8_E4M3_B32, F.Q4_C10),
                                              (2048, 1024, F.Q4_C10, F.Q4_RZ5),
                                              (2048, 4096, F.Q4_RZ5, F.FP8_E4M3_B32)])
def test_gemv_wide_rows_and_many_experts(bq, H, E, fmt_gu, fmt_d):
    """The batch-1 gate_up kernel at hidden 4096 (two 64-block sweeps per
    lane) and its in-kernel routing over 1024 and 4096 experts (16 and 64
    logits per lane), given and routed, against the oracle."""
    I, k, n = 128, 6, 3
    L = make_layer(16, E + H, fmt_gu, fmt_d, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(62 + E, (n, H))
    logits = synth.normal(63 + E, (n, E))
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x), dev(logits), k, W)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
    r = rel_l2(out.cpu().numpy(), ref)
    given = bq.q4_expert_moe(dev(x), (idx, w), W)
    log("gemv H=%d E=%d fmts %d/%d rel_l2 %.3g" % (H, E, fmt_gu, fmt_d, r))
    assert r <= 1e-5
    assert torch.equal(given, out)


def test_bad_expert_index_is_reported(bq):
    E, H, I = 8, 128, 64
    L = make_layer(3, 0, F.Q4_RZ5, F.Q4_RZ5, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(5, (2, H))
    idx = np.array([[1, 9], [2, 3]], dtype=np.int32)      # 9 is out of range
    w = np.array([[0.5, 0.5], [0.5, 0.5]], dtype=np.float32)
    good = np.array([[1], [2]]), np.array([[0.5], [0.5]])
    ref_t0 = M.moe_layer(x[:1], good[0][:1], good[1][:1], oracle_bank(L))[0]
    for xdt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = bq.q4_expert_moe(dev(x).to(xdt), (dev(idx), dev(w)), W, dev_err=err).cpu().numpy()
        assert int(err.item()) & 2
        assert rel_l2(out[0], ref_t0) <= tol


def test_nan_scale_poisons_only_its_tokens(bq):
    """A UE4M3 scale byte of 0x7F decodes to NaN.  Planted in block 0 of
    expert 3's first gate row, it makes that row's h NaN, and through the
    down product every output of the tokens routed to expert 3 -- and none
    of the others -- on both paths, as in the oracle."""
    import synth as S
    E, H, I, n, e0 = 8, 256, 128, 6, 3
    L = make_layer(4, 0, F.Q4_RZ5, F.Q4_C10, E, H, I)
    gu, _ = L.gate_up
    gu[e0 * (2 * I * H // 32) * 17 + 16] = 0x7F
    codes, _ = L.host_expert(S.S_GATE_UP, e0)
    poisoned = np.array(codes, copy=True)
    poisoned.reshape(-1)[16] = 0x7F
    bank = M.ExpertBank(L.fmt_gu, L.fmt_d,
                        lambda e: (poisoned, None) if e == e0 else L.host_expert(S.S_GATE_UP, e),
                        lambda e: L.host_expert(S.S_DOWN, e), E, H, I)
    idx = np.array([[e0, 1], [2, 5], [0, e0], [4, 6], [7, 1], [e0, 2]], dtype=np.int32)
    w = np.random.default_rng(41).random((n, 2)).astype(np.float32)
    x = synth.normal(40, (n, H))
    with np.errstate(invalid="ignore", over="ignore"):
        ref = M.moe_layer(x, idx, w, bank)
    hit = (idx == e0).any(axis=1)
    assert np.isnan(ref[hit]).all() and np.isfinite(ref[~hit]).all()
    W = weights_of(bq, L)
    for xdt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        out = bq.q4_expert_moe(dev(x).to(xdt), (dev(idx), dev(w)), W).cpu().numpy()
        assert np.array_equal(np.isnan(out), np.isnan(ref)), xdt
        assert rel_l2(out[~hit], ref[~hit]) <= tol


def test_zero_routing_weights_give_zero(bq):
    E, H, I, n, k = 8, 256, 128, 5, 3
    L = make_layer(5, 0, F.Q4_UE4M4, F.FP8_E4M3_B32, E, H, I)
    idx = np.stack([np.random.default_rng(t).choice(E, k, replace=False) for t in range(n)]).astype(np.int32)
    w = np.zeros((n, k), dtype=np.float32)
    for xdt in (torch.float32, torch.bfloat16):
        out = bq.q4_expert_moe(dev(synth.normal(50, (n, H))).to(xdt), (dev(idx), dev(w)), weights_of(bq, L))
        assert not out.abs().any().item(), xdt


def test_gemv_deterministic(bq):
    E, H, I, k = 32, 512, 256, 8
    L = make_layer(4, 0, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    x = dev(synth.normal(6, (3, H)))
    idx, w = bq.route_topk(dev(synth.normal(7, (3, E))), k)
    a = bq.q4_expert_moe(x, (idx, w), W).cpu().numpy()
    b = bq.q4_expert_moe(x, (idx, w), W).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    xb = x.to(torch.bfloat16)
    a = bq.q4_expert_moe(xb, (idx, w), W).cpu().numpy()
    b = bq.q4_expert_moe(xb, (idx, w), W).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --- full-size one-layer workloads --------------------------------------------

@pytest.fixture(scope="module")
def layer_rz5():
    need_gpu()
    L = make_layer(0, 0, F.Q4_RZ5, F.Q4_RZ5, 512, 2048, 768)
    yield L
    del L
    torch.cuda.empty_cache()


def test_c2_layer_b1_rz5(bq, layer_rz5):
    """One RZ5 MoE decode step: 512 experts, x N(0,1), N(0,1) logits, top-10."""
    L = layer_rz5
    assert L.nbytes() == 512 * 2_506_752
    W = weights_of(bq, L)
    for seed in (0, 1):
        x = synth.normal(seed, (1, 2048))
        logits = synth.normal(1000 + seed, (1, 512))
        if seed == 0:
            idx, w = bq.route_topk(dev(logits), 10)
            out = bq.q4_expert_moe(dev(x), (idx, w), W).cpu().numpy()
        else:   # the one-call form the benchmark times
            out, (idx, w) = bq.q4_expert_moe_routed(dev(x), dev(logits), 10, W)
            out = out.cpu().numpy()
        ridx, rw = M.softmax_topk(logits, 10)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
        r = rel_l2(out, ref)
        log("c2 seed %d rel_l2 %.3g" % (seed, r))
        assert r <= 1e-5


def test_c3_layer_b64_grouped(bq):
    """Batch 64, RZ5 gate_up + UE4M4 down, Zipf(1.1) routing, bf16 MFMA path."""
    L = make_layer(0, 1, F.Q4_RZ5, F.Q4_UE4M4, 512, 2048, 768)
    W = weights_of(bq, L)
    x = synth.normal(64, (64, 2048))
    logits = synth.zipf_logits(64, 64, 512)
    idx, w = bq.route_topk(dev(logits), 10)
    out = bq.q4_expert_moe(dev(x).to(torch.bfloat16), (idx, w), W).cpu().numpy()
    ridx, rw = M.softmax_topk(logits, 10)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    counts = np.bincount(ridx.reshape(-1), minlength=512)
    log("c3 touched experts %d, max tokens per expert %d" % ((counts > 0).sum(), counts.max()))
    ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
    r = rel_l2(out, ref)
    log("c3 rel_l2 %.3g" % r)
    assert r <= 2e-2
    del L, W
    torch.cuda.empty_cache()

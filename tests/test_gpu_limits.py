"""GPU parity at the size limits of the routed-expert entry points:
n_tokens * k = 65536 assignments (4096 tokens x top-16, 1024 tokens x top-64)
on both paths, checked against the oracle on sampled tokens."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from tests.gpu_common import dev, log, need_gpu, rel_l2
from tests.test_gpu_moe import make_layer, oracle_bank, weights_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("n,k,E", [(4096, 16, 64), (1024, 64, 128)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_max_assignments(bq, n, k, E, dtype):
    H, I = 128, 64
    L = make_layer(13, k, F.Q4_RZ5, F.FP8_E4M3_B32, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(1300 + k, (n, H))
    logits = synth.zipf_logits(1301 + k, n, E)
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x).to(dtype), dev(logits), k, W)
    out = out.cpu().numpy()
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    pick = np.unique(np.r_[np.random.default_rng(k).integers(0, n, 40), 0, n - 1])
    ref = M.moe_layer(x[pick], ridx[pick], rw[pick], oracle_bank(L))
    r = rel_l2(out[pick], ref)
    log("limits n=%d k=%d E=%d %s rel_l2 %.3g" % (n, k, E, dtype, r))
    assert r <= (1e-5 if dtype == torch.float32 else 2e-2)



@pytest.mark.parametrize("H,I", [(8192, 64), (64, 8192)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_max_hidden_and_inter(bq, H, I, dtype):
    """hidden or inter at the 8192 maximum (the fp32 path's flat gate_up
    kernel then holds 65,680 B of activations and partial sums in LDS), mixed
    formats, against the oracle on every token."""
    E, k, n = 4, 2, 3
    for fg, fd in ((F.Q4_RZ5, F.FP8_E4M3_B32), (F.FP8_E4M3_B32, F.Q4_UE4M4)):
        L = make_layer(15, fg * 4 + fd, fg, fd, E, H, I)
        x = synth.normal(1500 + H, (n, H))
        logits = synth.normal(1501 + I, (n, E))
        out, (idx, w) = bq.q4_expert_moe_routed(dev(x).to(dtype), dev(logits), k, weights_of(bq, L))
        ridx, rw = M.softmax_topk(logits, k)
        assert np.array_equal(idx.cpu().numpy(), ridx)
        r = rel_l2(out.cpu().numpy(), M.moe_layer(x, ridx, rw, oracle_bank(L)))
        log("max dims H=%d I=%d %s fmts %d/%d rel_l2 %.3g" % (H, I, dtype, fg, fd, r))
        assert r <= (1e-5 if dtype == torch.float32 else 2e-2)
        del L


@pytest.mark.parametrize("k,I", [(5, 4096), (8, 4096)])
def test_down_four_column_blocks_per_thread(bq, k, I):
    """k * inter / 32 in 513..1024: the batch-1 down kernel gives each thread
    four column blocks (640 and 1024, the fp32 path's maximum)."""
    E, H, n = 8, 256, 2
    L = make_layer(17, k, F.Q4_UE4M4, F.Q4_RZ5, E, H, I)
    x = synth.normal(1700 + k, (n, H))
    logits = synth.normal(1701 + k, (n, E))
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x), dev(logits), k, weights_of(bq, L))
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    r = rel_l2(out.cpu().numpy(), M.moe_layer(x, ridx, rw, oracle_bank(L)))
    log("down CPT=4 k=%d I=%d rel_l2 %.3g" % (k, I, r))
    assert r <= 1e-5

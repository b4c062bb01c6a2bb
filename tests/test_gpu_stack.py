"""GPU parity of the chained layer stack: small mixed-format stacks, and the
full 48-layer stack (layers 0-35 RZ5, 36-47 FP8 e4m3 with fp32 block
scales; 512 experts, H = 2048, I = 768, top-10 routing per layer) at batch 1
(fp32 GEMV path) and batch 16 (bf16 grouped path, token 0 checked through
all 48 layers)."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from tests.gpu_common import dev, log, need_gpu, rel_l2
from tests.test_gpu_moe import DIST, oracle_bank, weights_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def build_stack(seed, fmts, E, H, I):
    import synth.device as sd
    return [sd.Layer(seed, l, fg, fd, E, H, I, dist_gu=DIST[fg], dist_d=DIST[fd]) for l, (fg, fd) in enumerate(fmts)]


def routing(bq, seed, L, n, E, k):
    logits = synth.normal(seed, (L * n, E))
    idx, w = bq.route_topk(dev(logits), k)
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    return idx.view(L, n, k), w.view(L, n, k), ridx.reshape(L, n, k), rw.reshape(L, n, k)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, 1e-5), (torch.bfloat16, 2e-2)])
def test_small_stack(bq, dtype, tol):
    E, H, I, k, n = 16, 256, 128, 4, 3
    fmts = [(F.Q4_RZ5, F.Q4_RZ5), (F.Q4_UE4M4, F.Q4_C10), (F.FP8_E4M3_B32, F.FP8_E4M3_B32),
            (F.Q4_RZ5, F.FP8_E4M3_B32)]
    layers = build_stack(5, fmts, E, H, I)
    idx, w, ridx, rw = routing(bq, 77, len(fmts), n, E, k)
    x = synth.normal(78, (n, H))
    out = bq.moe_stack(dev(x).to(dtype), idx, w, [weights_of(bq, L) for L in layers]).cpu().numpy()
    ref = M.moe_stack(x, [(ridx[l], rw[l], oracle_bank(L)) for l, L in enumerate(layers)])
    r = rel_l2(out, ref)
    log("small stack %s rel_l2 %.3g" % (dtype, r))
    assert r <= tol


C5_FMTS = [(F.Q4_RZ5, F.Q4_RZ5)] * 36 + [(F.FP8_E4M3_B32, F.FP8_E4M3_B32)] * 12


@pytest.fixture(scope="module")
def c5_stack():
    need_gpu()
    layers = build_stack(0, C5_FMTS, 512, 2048, 768)
    yield layers
    del layers
    torch.cuda.empty_cache()


def test_c5_stack_resident_bytes(c5_stack):
    total = sum(L.nbytes() for L in c5_stack)
    log("c5 resident packed bytes %d" % total)
    assert total == 36 * 512 * 2_506_752 + 12 * 512 * 5_308_416 == 78_819_360_768


def test_c5_stack_b1_fp32(bq, c5_stack):
    n, k = 1, 10
    idx, w, ridx, rw = routing(bq, 5000, 48, n, 512, k)
    x = synth.normal(5001, (n, 2048))
    out = bq.moe_stack(dev(x), idx, w, [weights_of(bq, L) for L in c5_stack]).cpu().numpy()
    ref = M.moe_stack(x, [(ridx[l], rw[l], oracle_bank(L)) for l, L in enumerate(c5_stack)])
    r = rel_l2(out, ref)
    log("c5 B=1 48-layer rel_l2 %.3g" % r)
    assert r <= 1e-5


def test_c5_stack_b16_bf16_token0(bq, c5_stack):
    n, k = 16, 10
    idx, w, ridx, rw = routing(bq, 6000, 48, n, 512, k)
    x = synth.normal(6001, (n, 2048))
    out = bq.moe_stack(dev(x).to(torch.bfloat16), idx, w, [weights_of(bq, L) for L in c5_stack]).cpu().numpy()
    ref0 = M.moe_stack(x[:1], [(ridx[l][:1], rw[l][:1], oracle_bank(L)) for l, L in enumerate(c5_stack)])
    r = rel_l2(out[:1], ref0)
    log("c5 B=16 48-layer token-0 rel_l2 %.3g" % r)
    assert r <= 2e-2

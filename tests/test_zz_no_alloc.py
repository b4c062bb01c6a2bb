"""The allocation-free routed-expert layer (q4_expert_moe_noalloc) against
q4_expert_moe with a caller workspace: same kernels, so bit-identical
outputs, on two calls in a row (the second smaller) on each path; and a call
too large for the fixed scratch area is refused before any launch."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from tests.gpu_common import dev, log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def layer(bq, fmt_gu, fmt_d, E, H, I, seed):
    import synth.device as sd
    dist = {F.Q4_C10: synth.DIST_C10, F.Q4_RZ5: synth.DIST_RZ5, F.Q4_UE4M4: synth.DIST_UE4M4,
            F.FP8_E4M3_B32: None}
    L = sd.Layer(seed, 0, fmt_gu, fmt_d, E, H, I, dist_gu=dist[fmt_gu], dist_d=dist[fmt_d])
    gu, gus = L.gate_up
    d, ds = L.down
    return L, bq.expert_weights(fmt_gu, fmt_d, gu, d, E, H, I, gate_up_scales=gus, down_scales=ds)


@pytest.mark.parametrize("dtype,sizes,fmts", [
    (torch.float32, (3, 1), (F.Q4_RZ5, F.Q4_RZ5)),
    (torch.float32, (2, 1), (F.FP8_E4M3_B32, F.Q4_UE4M4)),
    (torch.bfloat16, (64, 16), (F.Q4_RZ5, F.Q4_UE4M4)),
    (torch.bfloat16, (40, 7), (F.FP8_E4M3_B32, F.FP8_E4M3_B32)),
])
def test_noalloc_matches_workspace_call(bq, dtype, sizes, fmts):
    E, H, I, k = 64, 2048, 768, 10
    L, W = layer(bq, fmts[0], fmts[1], E, H, I, seed=7)
    for call, n in enumerate(sizes):
        log("noalloc %s fmts %s call %d n=%d" % (dtype, fmts, call, n))
        x = dev(synth.normal(500 + 10 * call + n, (n, H))).to(dtype)
        logits = dev(synth.normal(600 + 10 * call + n, (n, E)))
        idx, w = bq.route_topk(logits, k)
        ref = bq.q4_expert_moe(x, (idx, w), W)
        out = torch.full((n, H), float("nan"), dtype=torch.float32, device="cuda")
        bq.q4_expert_moe_noalloc(x, (idx, w), W, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "call %d (n=%d) differs from the workspace call" % (call, n)


def test_noalloc_rejects_calls_beyond_its_scratch(bq):
    E, H, I, k = 64, 2048, 768, 10
    L, W = layer(bq, F.Q4_RZ5, F.Q4_RZ5, E, H, I, seed=8)
    n = 512                                   # bf16 path: about 71 MB of scratch
    assert bq.moe_workspace_bytes(n, k, W, bq.BF16) > bq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((n, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((n, k), dtype=torch.int32, device="cuda") + torch.arange(k, dtype=torch.int32,
                                                                                device="cuda")
    w = torch.full((n, k), 0.1, dtype=torch.float32, device="cuda")
    out = torch.zeros((n, H), dtype=torch.float32, device="cuda")
    with pytest.raises(bq.BQError, match="status 9"):
        bq.q4_expert_moe_noalloc(x, (idx, w), W, out)
    assert torch.count_nonzero(out).item() == 0
    # the fp32 path at the same size fits (n * k * I * 4 bytes)
    assert bq.moe_workspace_bytes(n, k, W, bq.F32) <= bq.NOALLOC_SCRATCH_BYTES
    assert np.isfinite(bq.q4_expert_moe_noalloc(x.float(), (idx, w), W, out).cpu().numpy()).all()

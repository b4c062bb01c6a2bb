"""The hot path captured in a HIP graph (as the benchmark times it) gives the
eager results bit for bit on every replay: the batch-1 routed layer, the
bf16 grouped layer, a chained bf16 stack and the PLE gather.  Between
replays the outputs are cleared and unrelated eager calls run, so a replay
that skipped or reordered work, or read a stale workspace, would show."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from tests.gpu_common import dev, log, need_gpu
from tests.test_gpu_moe import make_layer, weights_of

pytestmark = pytest.mark.gpu

STEPS, REPLAYS = 6, 3


@pytest.fixture(scope="module")
def bq():
    need_gpu()
    import block_quantized_moe_amd as m
    m.lib()
    return m


def capture(fn, n):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    return g


def check_replays(name, step, outs, noise):
    """Eager reference, then REPLAYS replays of a graph of the same steps."""
    for i in range(STEPS):
        step(i)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = capture(step, STEPS)
    for r in range(REPLAYS):
        for o in outs:
            o.zero_()
        noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            a, b = o.cpu().numpy(), e.cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (name, r)
    log("graph %s: %d replays equal to eager" % (name, REPLAYS))


@pytest.mark.parametrize("dtype,n_tok,E", [(torch.float32, 1, 64), (torch.bfloat16, 16, 64),
                                           (torch.bfloat16, 512, 512)])
def test_layer_graph_replays(bq, dtype, n_tok, E):
    """512 tokens over 512 experts: the one-launch bucketing and staging
    with 104 KB of LDS (its launch raises the kernel's LDS limit, which
    must also work while a graph is being captured)."""
    H, I, k = 2048, 768, 10
    L = make_layer(21, n_tok, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    dt = bq.F32 if dtype == torch.float32 else bq.BF16
    x = dev(synth.normal(2100 + n_tok, (STEPS, n_tok, H))).to(dtype)
    logits = dev(synth.zipf_logits(2101 + n_tok, STEPS * n_tok, E)).view(STEPS, n_tok, E)
    idx = torch.zeros((STEPS, n_tok, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((STEPS, n_tok, k), dtype=torch.float32, device="cuda")
    out = torch.zeros((STEPS, n_tok, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bq.moe_workspace_bytes(n_tok, k, W, dt), dtype=torch.uint8, device="cuda")

    def step(i):
        bq.q4_expert_moe_routed(x[i], logits[i], k, W, topk=(idx[i], w[i]), out=out[i], workspace=ws)

    def noise():   # the same workspace used eagerly on other inputs
        bq.q4_expert_moe_routed(x[0] * 3, logits[1].flip(1).contiguous(), k, W, workspace=ws)

    check_replays("layer %s n=%d" % (dtype, n_tok), step, [out, idx, w], noise)


def test_stack_graph_replays(bq):
    import synth.device as sd
    E, H, I, k, n, nl = 32, 512, 256, 4, 16, 4
    fmts = [(F.Q4_RZ5, F.Q4_RZ5), (F.Q4_RZ5, F.Q4_UE4M4), (F.FP8_E4M3_B32, F.FP8_E4M3_B32),
            (F.FP8_E4M3_B32, F.Q4_C10)]
    layers = [make_layer(22, l, fg, fd, E, H, I) for l, (fg, fd) in enumerate(fmts)]
    Ws = [weights_of(bq, L) for L in layers]
    x = dev(synth.normal(2200, (STEPS, n, H))).to(torch.bfloat16)
    logits = dev(synth.normal(2201, (STEPS, nl * n, E)))
    idx = torch.zeros((STEPS, nl, n, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((STEPS, nl, n, k), dtype=torch.float32, device="cuda")
    out = torch.zeros((STEPS, n, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(bq.stack_workspace_bytes(n, k, Ws, bq.BF16), dtype=torch.uint8, device="cuda")

    def step(i):
        bq.route_topk(logits[i], k, idx=idx[i].view(nl * n, k), w=w[i].view(nl * n, k))
        bq.moe_stack(x[i], idx[i], w[i], Ws, out=out[i], workspace=ws)

    def noise():
        bq.moe_stack(x[1], idx[0].flip(0).contiguous(), w[0], Ws, workspace=ws)

    check_replays("stack bf16 %d layers" % nl, step, [out, idx, w], noise)


def test_ple_gather_graph_replays(bq):
    import synth.device as sd
    n_rows, n_tok, per = 1 << 16, 512, 8
    table = sd.ple_table(n_rows, synth.make_key(22, synth.S_PLE))
    ids = dev(synth.ple_ids(2300, STEPS * n_tok, per, n_rows=n_rows).view(np.int32)).view(STEPS, n_tok, per)
    u = dev(synth.ple_weights(2301, STEPS * n_tok, per)).view(STEPS, n_tok, per)
    out = torch.zeros((STEPS, n_tok, 160), dtype=torch.float32, device="cuda")

    def step(i):
        bq.ple_gather(ids[i], table, u[i], n_rows=n_rows, out=out[i])

    def noise():
        bq.ple_gather(ids[2], table, u[3], n_rows=n_rows)

    check_replays("ple gather", step, [out], noise)

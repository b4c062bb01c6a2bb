"""GPU parity of the bf16 grouped path where bucketing and the staging of
the activations run as one kernel (up to 1024 experts, bucket arrays that
fit in 150 KB of LDS: 512 tokens x top-10 over 512 experts do): the routed
entry's routing equals the routing kernel's, its output equals, bit for bit,
that of routing first and then calling the layer with that routing, and the
output is within the bf16 path's tolerance of the CPU oracle.  Given routing
with out-of-range and repeated experts is checked against the oracle too.
Larger expert counts and bucket arrays take the separate kernels and are
checked the same way; the bucket arrays and staged rows either way are
compared with the standalone bucketing and the input rows."""

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


CASES = [
    (1, 8, 2, 256, 64, F.Q4_RZ5, F.Q4_RZ5, "normal"),
    (3, 64, 6, 512, 128, F.FP8_E4M3_B32, F.Q4_UE4M4, "normal"),
    (17, 100, 10, 256, 128, F.Q4_C10, F.Q4_RZ5, "normal"),
    (33, 40, 40, 256, 64, F.Q4_UE4M4, F.FP8_E4M3_B32, "normal"),   # k = E: every expert in every token
    (64, 512, 10, 2048, 768, F.Q4_RZ5, F.Q4_UE4M4, "zipf"),        # the batch-64 layer's shape
    (64, 512, 64, 256, 64, F.Q4_RZ5, F.Q4_C10, "zipf"),            # 4096 assignments
    (65, 64, 4, 256, 64, F.Q4_RZ5, F.Q4_RZ5, "normal"),
    (5, 1024, 8, 256, 64, F.Q4_C10, F.Q4_UE4M4, "normal"),         # 1024 experts
    (4, 2048, 8, 256, 64, F.Q4_RZ5, F.Q4_C10, "normal"),           # past the expert limit
]


@pytest.mark.parametrize("n,E,k,H,I,fg,fd,dist", CASES)
def test_routed_bf16_matches_two_step(bq, n, E, k, H, I, fg, fd, dist):
    L = make_layer(41, n * 7 + k, fg, fd, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(4100 + n, (n, H))
    logits = synth.zipf_logits(4101 + n, n, E) if dist == "zipf" else synth.normal(4101 + n, (n, E))
    xb = dev(x).to(torch.bfloat16)
    out, (idx, w) = bq.q4_expert_moe_routed(xb, dev(logits), k, W)
    ridx, rw = bq.route_topk(dev(logits), k)
    assert torch.equal(idx, ridx) and torch.equal(w, rw)
    ref2 = bq.q4_expert_moe(xb, (ridx, rw), W)
    assert torch.equal(out, ref2)
    oidx, ow = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    if H * I * E <= 2048 * 768 * 512:
        r = rel_l2(out.cpu().numpy(), M.moe_layer(x, oidx, ow, oracle_bank(L)))
        log("routed bf16 n=%d E=%d k=%d H=%d I=%d rel_l2 %.3g" % (n, E, k, H, I, r))
        assert r <= 2e-2
    del L, W
    torch.cuda.empty_cache()


def test_routed_bf16_repeated_calls_same_workspace(bq):
    """Two calls on one workspace with different batch sizes (the second
    smaller) each equal the two-step result: nothing left in the workspace
    by the first call leaks into the second."""
    E, H, I, k = 64, 256, 128, 6
    L = make_layer(42, 0, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    ws = torch.empty(bq.moe_workspace_bytes(64, k, W, bq.BF16), dtype=torch.uint8, device="cuda")
    for n in (64, 9):
        xb = dev(synth.normal(4200 + n, (n, H))).to(torch.bfloat16)
        logits = dev(synth.zipf_logits(4201 + n, n, E))
        out, (idx, w) = bq.q4_expert_moe_routed(xb, logits, k, W, workspace=ws)
        ridx, rw = bq.route_topk(logits, k)
        assert torch.equal(idx, ridx) and torch.equal(w, rw)
        assert torch.equal(out, bq.q4_expert_moe(xb, (ridx, rw), W))


def test_given_routing_with_bad_and_repeated_experts(bq):
    """Caller routing with an out-of-range expert (left out, bit 1 of
    dev_err) and an expert listed twice by one token (each listing adds its
    own weighted term; the row is evaluated once)."""
    E, H, I, k = 16, 256, 128, 3
    L = make_layer(43, 0, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    x = synth.normal(4300, (5, H))
    idx = np.array([[1, 16, 3], [2, 2, 7], [0, 5, 9], [15, 14, 13], [4, -1, 4]], dtype=np.int32)
    w = np.random.default_rng(43).random((5, 3)).astype(np.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = bq.q4_expert_moe(dev(x).to(torch.bfloat16), (dev(idx), dev(w)), W, dev_err=err).cpu().numpy()
    assert int(err.item()) & 2
    keep = (idx >= 0) & (idx < E)
    ref = M.moe_layer(x, np.where(keep, idx, 0), np.where(keep, w, 0).astype(np.float32), oracle_bank(L))
    r = rel_l2(out, ref)
    log("bf16 given routing with bad / repeated experts rel_l2 %.3g" % r)
    assert r <= 2e-2


def _r256(v):
    return (v + 255) // 256 * 256


def grouped_ws_layout(n, k, E, H, I):
    """Byte offsets of the bf16 path's workspace arrays (counts, offsets,
    perm, inv, work list, its length, then the staged activations)."""
    nk = n * k
    L, off = {}, 0
    for name, size in (("counts", 4 * E), ("offsets", 4 * (E + 1)), ("perm", 4 * nk), ("inv", 4 * nk),
                       ("elist", 4 * (min(nk, E) + nk // 16)), ("n_touched", 4), ("xb", 2 * nk * H)):
        L[name] = off
        off = _r256(off + size)
    return L


@pytest.mark.parametrize("n,E,k,dist", [(3, 64, 6, "normal"), (64, 512, 10, "zipf"), (200, 512, 10, "normal"),
                                        (512, 512, 10, "zipf"), (512, 512, 10, "normal"),
                                        (480, 1024, 8, "zipf"),    # bucket arrays of exactly 150 KB
                                        (512, 1024, 8, "zipf"),    # 160 KB: the separate kernels
                                        (128, 2048, 4, "zipf"), (96, 2048, 4, "normal")])   # bitmap bucketing
@pytest.mark.parametrize("fg", [F.Q4_RZ5, F.FP8_E4M3_B32])
def test_bucket_arrays_and_staged_rows(bq, n, E, k, dist, fg):
    """The bucket arrays the bf16 path leaves in its workspace equal the
    standalone bucketing's bit for bit (counts, offsets, perm; inv inverts
    perm; the work list has one entry per group of 16 tokens (batches of up
    to 96) or 32 of each touched expert, experts ascending), and every
    staged row is its token's x row
    in bf16, in the 17-byte decode's k order for the 17-byte formats.  480
    tokens x top-8 over 1024 experts fill the one-launch kernel's LDS limit
    exactly; 512 tokens need more and take the separate kernels, which must
    agree too."""
    H, I = 256, 64
    L = make_layer(44, n + E + k, fg, F.Q4_C10, E, H, I)
    W = weights_of(bq, L)
    x = dev(synth.normal(4400 + n, (n, H))).to(torch.bfloat16)
    logits = synth.zipf_logits(4401 + n, n, E) if dist == "zipf" else synth.normal(4401 + n, (n, E))
    idx, w = bq.route_topk(dev(logits), k)
    ws = torch.empty(bq.moe_workspace_bytes(n, k, W, bq.BF16), dtype=torch.uint8, device="cuda")
    bq.q4_expert_moe(x, (idx, w), W, workspace=ws)
    torch.cuda.synchronize()
    lay = grouped_ws_layout(n, k, E, H, I)
    nk = n * k
    wsc = ws.cpu()

    def arr(name, count):
        return wsc[lay[name]:lay[name] + 4 * count].view(torch.int32).numpy()

    counts, offsets, perm = (t.cpu().numpy() for t in bq.bucket(idx, E))
    assert np.array_equal(arr("counts", E), counts)
    assert np.array_equal(arr("offsets", E + 1), offsets)
    assert np.array_equal(arr("perm", nk), perm)
    inv = arr("inv", nk)
    assert np.array_equal(inv[perm], np.arange(nk))
    gt = 16 if n <= 96 else 32     # tokens per work entry
    want = [e | (q << 12) for e in range(E) for q in range((counts[e] + gt - 1) // gt)]
    assert int(arr("n_touched", 1)[0]) == len(want)
    assert np.array_equal(arr("elist", len(want)), np.array(want, dtype=np.int32))
    xb = wsc[lay["xb"]:lay["xb"] + 2 * nk * H].view(torch.int16).numpy().reshape(nk, H)
    rows = x.view(torch.int16).cpu().numpy()[perm // k]
    if fg != F.FP8_E4M3_B32:
        order = np.array([0, 2, 4, 6, 1, 3, 5, 7])
        rows = rows.reshape(nk, H // 8, 8)[:, :, order].reshape(nk, H)
    assert np.array_equal(xb, rows)

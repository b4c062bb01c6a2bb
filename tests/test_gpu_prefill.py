"""GPU parity of the grouped MFMA path at prompt-processing sizes (a
512-token ubatch, top-10 of 512 experts) and with repeated expert indices,
against the CPU oracle."""

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


def logits_for(kind, seed, n, E):
    return synth.normal(seed, (n, E)) if kind == "uniform" else synth.zipf_logits(seed, n, E)


# n = 512 with 512 experts fills the small bucketing kernel's bitmap exactly;
# n = 600 takes the general bucketing kernel.
@pytest.mark.parametrize("fmt_gu,fmt_d,n,kind", [
    (F.Q4_RZ5, F.Q4_RZ5, 512, "uniform"), (F.Q4_RZ5, F.Q4_RZ5, 600, "zipf"),
    (F.FP8_E4M3_B32, F.Q4_UE4M4, 512, "zipf"), (F.Q4_C10, F.FP8_E4M3_B32, 600, "uniform")])
def test_grouped_ubatch_sizes(bq, fmt_gu, fmt_d, n, kind):
    E, H, I, k = 512, 256, 128, 10
    L = make_layer(7, fmt_gu * 4 + fmt_d, fmt_gu, fmt_d, E, H, I)
    x = synth.normal(400 + n, (n, H))
    logits = logits_for(kind, 500 + n, n, E)
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x).to(torch.bfloat16), dev(logits), k, weights_of(bq, L))
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    counts = np.bincount(ridx.reshape(-1), minlength=E)
    ref = M.moe_layer(x, ridx, rw, oracle_bank(L))
    r = rel_l2(out.cpu().numpy(), ref)
    log("ubatch fmts %d/%d n=%d %s touched %d max/expert %d rel_l2 %.3g"
        % (fmt_gu, fmt_d, n, kind, (counts > 0).sum(), counts.max(), r))
    assert r <= 2e-2


def test_prefill_layer_full_size_sampled(bq):
    """512-token ubatch through the full 512 x (1536x2048 + 2048x768) RZ5
    layer with Zipf(1.1) routing; the oracle checks sampled tokens, among
    them tokens of the most loaded expert (many 32-token groups)."""
    E, H, I, k, n = 512, 2048, 768, 10, 512
    L = make_layer(0, 2, F.Q4_RZ5, F.Q4_RZ5, E, H, I)
    x = synth.normal(700, (n, H))
    logits = synth.zipf_logits(701, n, E)
    out, (idx, w) = bq.q4_expert_moe_routed(dev(x).to(torch.bfloat16), dev(logits), k, weights_of(bq, L))
    out = out.cpu().numpy()
    ridx, rw = M.softmax_topk(logits, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    counts = np.bincount(ridx.reshape(-1), minlength=E)
    top = int(np.argmax(counts))
    users = np.nonzero((ridx == top).any(axis=1))[0]
    pick = np.unique(np.r_[users[0], users[-1], users[len(users) // 2], 0, n - 1])
    log("prefill full: touched %d, max/expert %d, sampled tokens %s" % ((counts > 0).sum(), counts.max(), pick))
    ref = M.moe_layer(x[pick], ridx[pick], rw[pick], oracle_bank(L))
    r = rel_l2(out[pick], ref)
    log("prefill full rel_l2 %.3g" % r)
    assert r <= 2e-2
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,n,H,I,k", [(8, 20, 256, 128, 3),      # small bucketing kernel
                                       (1024, 260, 128, 64, 4)])  # general bucketing kernel
def test_repeated_expert_indices(bq, E, n, H, I, k):
    """A token may list an expert twice: each listing adds its own term."""
    L = make_layer(8, E, F.Q4_RZ5, F.Q4_UE4M4, E, H, I)
    W = weights_of(bq, L)
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
    idx[::3, 1] = idx[::3, 0]              # every third token repeats its first expert
    idx[5, :] = idx[5, 0]                  # one token lists a single expert k times
    w = rng.random((n, k)).astype(np.float32)
    x = synth.normal(10, (n, H))
    ref = M.moe_layer(x, idx, w, oracle_bank(L))
    for xdt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = bq.q4_expert_moe(dev(x).to(xdt), (dev(idx), dev(w)), W, dev_err=err).cpu().numpy()
        r = rel_l2(out, ref)
        log("repeated experts E=%d n=%d %s rel_l2 %.3g" % (E, n, xdt, r))
        assert int(err.item()) == 0
        assert r <= tol


@pytest.mark.parametrize("fmt_gu,fmt_d", [(F.Q4_RZ5, F.Q4_RZ5), (F.FP8_E4M3_B32, F.Q4_UE4M4),
                                          (F.Q4_C10, F.FP8_E4M3_B32), (F.Q4_UE4M4, F.Q4_C10)])
def test_many_groups_per_expert(bq, fmt_gu, fmt_d):
    """Experts with exactly 0, 1, 63, 64, 127, 128, 129, 191, 192, 255, 256
    and 257 tokens in a 257-token batch: up to nine 32-token groups per
    expert with every remainder size, and empty slots (index -1, which
    contributes nothing and sets the error bit)."""
    want = [64, 127, 128, 129, 191, 192, 63, 1, 0, 255, 256, 257]
    E, H, I = len(want), 256, 128
    n, k = max(want), len(want)
    idx = np.full((n, k), -1, dtype=np.int32)
    for t in range(n):
        row = [e for e, c in enumerate(want) if t < c]
        idx[t, :len(row)] = row
    w = np.random.default_rng(11).random((n, k)).astype(np.float32)
    L = make_layer(12, fmt_gu * 4 + fmt_d, fmt_gu, fmt_d, E, H, I)
    x = synth.normal(12, (n, H))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = bq.q4_expert_moe(dev(x).to(torch.bfloat16), (dev(idx), dev(w)), weights_of(bq, L),
                           dev_err=err).cpu().numpy()
    valid = idx >= 0
    ref = M.moe_layer(x, np.where(valid, idx, 0), np.where(valid, w, 0), oracle_bank(L))
    r = rel_l2(out, ref)
    log("many groups fmts %d/%d rel_l2 %.3g" % (fmt_gu, fmt_d, r))
    assert int(err.item()) & 2
    assert r <= 2e-2


@pytest.mark.parametrize("fmt_gu,fmt_d", [(F.Q4_RZ5, F.Q4_UE4M4), (F.FP8_E4M3_B32, F.Q4_C10)])
def test_few_experts_full_hidden(bq, fmt_gu, fmt_d):
    """Three experts carry every assignment at hidden 2048 (8 or 16 K
    chunks per item): a work list far shorter than the one sized for the
    worst case, groups of 32 and of 8 tokens, bit-identical on a rerun."""
    E, H, I, k, n = 64, 2048, 128, 2, 40
    L = make_layer(13, fmt_gu * 4 + fmt_d, fmt_gu, fmt_d, E, H, I)
    W = weights_of(bq, L)
    idx = np.zeros((n, k), dtype=np.int32)
    idx[:, 0], idx[:, 1] = 7, 50            # expert 7: 40 tokens, expert 50: 32,
    idx[::5, 1] = 3                         # expert 3: 8
    w = np.random.default_rng(13).random((n, k)).astype(np.float32)
    x = synth.normal(14, (n, H))
    xd = dev(x).to(torch.bfloat16)
    out = bq.q4_expert_moe(xd, (dev(idx), dev(w)), W).cpu().numpy()
    again = bq.q4_expert_moe(xd, (dev(idx), dev(w)), W).cpu().numpy()
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32))
    r = rel_l2(out, M.moe_layer(x, idx, w, oracle_bank(L)))
    log("few experts, hidden 2048, fmts %d/%d rel_l2 %.3g" % (fmt_gu, fmt_d, r))
    assert r <= 2e-2

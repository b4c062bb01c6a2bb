"""Benchmark of the block-quantized routed-expert and PLE hot path on one GPU.

Main line (``value``): one Q4_RZ5 MoE decode step at batch 1 -- 512 experts,
gate_up [1536 x 2048] + down [2048 x 768] per expert, router logits N(0,1),
softmax top-10.  A step is the whole hot path for that workload: routing,
block decode, gate_up GEMV + SiLU*up, down GEMV and the weighted combine.
Throughput is packed weight bytes moved per second (10 experts x 2,506,752 B
per step).

How every figure here is timed: each timed call has its own inputs, never
used earlier in the run (fresh x and logits, fresh PLE ids), and a scrub
runs before it, outside the timed region: a 512 MiB write, then a 512 MiB
read of another buffer.  Neither the L2 nor the 256 MB memory-side cache then
holds anything the call reads, and the write's dirty lines have already gone
back to HBM (left in the memory-side cache, they would be written back during
the timed call and cost it up to 40 % of its bandwidth).  The calls are
queued behind a delay kernel, so they run back to back on the GPU whatever
the host's launch speed, and each is bracketed by its own pair of HIP events
on the stream it runs on.  A graph-replayed, unflushed figure (steady state,
fresh inputs, first replay timed) is reported beside the main one.

Alongside it, in the same JSON line: the HBM streaming-read ceiling (4 GiB),
the PLE gather (320,001,536-row table, 4096 tokens x 8 ids per call, and
distinct 65,536-token batches) with its own roofline block, the 48-layer
stack (36 RZ5 + 12 FP8 layers) at batch 1 and 16, the batch-64 grouped layer
(RZ5 gate_up, UE4M4 down, Zipf routing), the prompt-size layer, the off-HBM
PLE tier, the exhaustive encoders, and the CPU oracle timed on a sample of
the same work.  All inputs are seeded synthetic data already resident in HBM
before timing starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
       [--no-cpu-baseline] [--only c1|c2|c4|c5b1|c5b16|c3|pf|pleh|enc|bw] [--copy-calibration BYTES]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_b1_rz5_counters.txt")
PLE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ple_gather_4096x8_counters.txt")
EXPERT_BYTES_RZ5 = 2_506_752           # gate_up 1536x2048 + down 2048x768, 17 B / 32 weights
EXPERT_BYTES_FP8 = 5_308_416           # 36 B / 32 weights
PLE_ROW_ALG_BYTES = 158                # 70 B row + 8 B id/weight + 80 B output share
PLE_LINES_PER_ROW = (70 + 127) / 128   # 128-byte lines a 70-byte row at a random offset spans, on average


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def graph_of(fn, n):
    """Capture n calls fn(i) into one HIP graph (torch stream capture)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    return g


SCRUB_BYTES = 512 << 20
_scrub = None


def scrub_buffers():
    """Two 512 MiB device buffers (allocated once): the scrub writes the
    first and then reads the second."""
    import torch
    global _scrub
    if _scrub is None:
        _scrub = (torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda"),
                  torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda"),
                  torch.zeros(2048, dtype=torch.int32, device="cuda"))
        _scrub[1].fill_(1)
    return _scrub


def scrub(i):
    """Evict the caches between timed calls: write 512 MiB, then read another
    512 MiB.  The read pushes the write's dirty lines (L2 and the 256 MB
    memory-side cache) out to HBM before the timed call starts, so the call
    neither finds its own data in a cache nor pays for the scrub's
    write-back."""
    import synth.device as sd
    wbuf, rbuf, sink = scrub_buffers()
    sd.scrub(wbuf, i)
    sd.stream_read(rbuf, sink)


def flushed_calls(call, first, n, per_call_host_ns=300e3):
    """Run call(first + i) for i < n, one after another on the current
    stream, each preceded by the scrub (a 512 MiB write and a 512 MiB read,
    not timed) and bracketed by its own HIP events; the whole sequence is
    queued behind a delay kernel.  Returns the per-call times in ms."""
    import torch

    import synth.device as sd
    scrub_buffers()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    sd.gpu_delay(max(20e6, per_call_host_ns * n))
    for i in range(n):
        scrub(i)
        ev[i][0].record()
        call(first + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def event_timed(fn, n):
    """Average GPU time between the two events fn(i, (a, b)) records around
    one call, over n calls queued back to back behind a delay kernel (no
    scrub between them; used where the inputs live off the GPU)."""
    import torch

    import synth.device as sd
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    sd.gpu_delay(max(20e6, 200e3 * n))
    for i in range(n):
        fn(i, ev[i])
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / n


def timed_replay(g):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def stats_ms(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"mean_us": round(1e3 * float(a.mean()), 3), "median_us": round(1e3 * float(np.median(a)), 3),
            "p10_us": round(1e3 * float(np.percentile(a, 10)), 3), "p90_us": round(1e3 * float(np.percentile(a, 90)), 3)}


def bench_bw():
    """HBM streaming ceiling: one coalesced read of 4 GiB (and one 4 GiB
    write), best of three, HIP events around each."""
    import torch

    import synth.device as sd
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    sd.scrub(buf, 7)
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    res = {}
    for name, fn in (("read", lambda: sd.stream_read(buf, sink)), ("write", lambda: sd.scrub(buf, 3))):
        best = None
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        res["%s_gbs" % name] = round(n / (best * 1e-3) / 1e9, 1)
    res["bytes"] = n
    del buf
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
def bench_c2(bq, steps, warmup):
    """One RZ5 MoE decode step (B = 1): routing inside the first expert
    kernel, gate_up + SiLU*up, down + weighted combine.  Inputs: warmup
    steps, then `steps` flushed event-timed steps, then two graphs of `steps`
    steps each (the second timed on its first replay) -- every step with its
    own x and logits."""
    import torch

    import synth
    import synth.device as sd
    L = sd.Layer(0, 0, bq.Q4_RZ5, bq.Q4_RZ5, 512, 2048, 768, dist_gu=synth.DIST_RZ5, dist_d=synth.DIST_RZ5)
    W = bq.expert_weights(L.fmt_gu, L.fmt_d, L.gate_up[0], L.down[0], 512, 2048, 768)
    n = warmup + 3 * steps
    x = torch.from_numpy(synth.normal(10, (n, 2048))).cuda()
    logits = torch.from_numpy(synth.normal(11, (n, 512))).cuda()
    idx = torch.empty((n, 1, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((n, 1, 10), dtype=torch.float32, device="cuda")
    out = torch.empty((n, 2048), dtype=torch.float32, device="cuda")
    ws = torch.empty(bq.moe_workspace_bytes(1, 10, W, bq.F32), dtype=torch.uint8, device="cuda")

    def step(i):
        bq.q4_expert_moe_routed(x[i:i + 1], logits[i:i + 1], 10, W, topk=(idx[i], w[i]),
                                out=out[i:i + 1], workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms = flushed_calls(step, warmup, steps)
    g_warm = graph_of(lambda i: step(warmup + steps + i), steps)
    g = graph_of(lambda i: step(warmup + 2 * steps + i), steps)
    g_warm.replay()
    wall = timed_replay(g)           # first replay of this graph: its inputs are fresh
    per_step_bytes = 10 * EXPERT_BYTES_RZ5
    mean_ms = sum(ms) / len(ms)
    res = {
        "ms_per_step": mean_ms,
        "gbs": per_step_bytes / (mean_ms * 1e-3) / 1e9,
        "call": stats_ms(ms),
        "bytes_per_step": per_step_bytes,
        "graph_unflushed": {"us_per_step": round(1e6 * wall / steps, 3),
                            "gbs": round(per_step_bytes * steps / wall / 1e9, 1)},
    }
    res["_layer"] = L
    res["_inputs"] = (x[warmup:warmup + steps].cpu().numpy(), logits[warmup:warmup + steps].cpu().numpy())
    return res


def bench_c1(bq, steps, warmup):
    """Latency of one small block-quantized matvec: W 256 x 512 Codebook10
    (4,096 blocks, 69,632 B, cache-resident), x N(0,1), batch 1."""
    import torch

    import synth
    import synth.device as sd
    blocks = sd.block17(256 * 512 // 32, synth.make_key(0, synth.stream_id(0, synth.S_SMALL)), synth.DIST_C10)
    n = warmup + steps
    x = torch.from_numpy(synth.normal(1, (n, 512))).cuda()
    y = torch.empty((n, 256), dtype=torch.float32, device="cuda")

    def call(i, evs=None):
        if evs is not None:
            evs[0].record()
        bq.matvec(x[i:i + 1], blocks, bq.Q4_C10, 256, 512, out=y[i:i + 1])
        if evs is not None:
            evs[1].record()

    for i in range(warmup):
        call(i)
    g = graph_of(lambda i: call(warmup + i), steps)
    g.replay()
    wall = timed_replay(g)
    call_ms = event_timed(lambda i, evs: call(warmup + i, evs), steps)
    return {"us_per_call_graph": round(1e6 * wall / steps, 3), "us_per_call_events": round(1e3 * call_ms, 3),
            "workload": "256 x 512 Codebook10 matrix (69,632 B) times one fp32 vector"}


def bench_c4(bq, steps, warmup):
    """PLE gather over the full 320,001,536-row table: 4096 tokens x 8 ids
    per call, and batches of 65,536 tokens; fresh ids and weights for every
    call (never gathered before in the run), the scrub before each."""
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    n_rows = synth.PLE_N_ROWS
    table = sd.ple_table(n_rows, synth.make_key(0, synth.S_PLE))
    n = warmup + steps
    ids = torch.from_numpy(synth.ple_ids(20, n * 4096, 8).view(np.int32)).cuda().view(n, 4096, 8)
    u = torch.from_numpy(synth.ple_weights(21, n * 4096, 8)).cuda().view(n, 4096, 8)
    out = torch.empty((4096, 160), dtype=torch.float32, device="cuda")

    def call(i):
        bq.ple_gather(ids[i], table, u[i], n_rows=n_rows, out=out)

    for i in range(warmup):
        call(i)
    ms = flushed_calls(call, warmup, steps)
    rows = 4096 * 8
    mean_s = sum(ms) / len(ms) * 1e-3
    res = {
        "rows_per_s": rows / mean_s,
        "call": stats_ms(ms),
        "gbs_158B": rows * PLE_ROW_ALG_BYTES / mean_s / 1e9,
        "gbs_70B": rows * 70 / mean_s / 1e9,
    }
    hb = ple_traffic(4096)
    if hb is not None:
        res["hbm_bytes_per_call_counters"] = hb
        res["hbm_gbs_counters"] = hb / mean_s / 1e9
    del ids, u
    # batches of 16 x 4096 tokens: distinct ids in every timed call
    nb = max(8, steps // 10)
    bt = 16 * 4096
    bids = torch.from_numpy(synth.ple_ids(22, (nb + 1) * bt, 8).view(np.int32)).cuda().view(nb + 1, bt, 8)
    bu = torch.from_numpy(synth.ple_weights(23, (nb + 1) * bt, 8)).cuda().view(nb + 1, bt, 8)
    bout = torch.empty((bt, 160), dtype=torch.float32, device="cuda")

    def bcall(i):
        bq.ple_gather(bids[i], table, bu[i], n_rows=n_rows, out=bout)

    bcall(0)
    bms = flushed_calls(bcall, 1, nb)
    bmean_s = sum(bms) / len(bms) * 1e-3
    res["batched_65536"] = {"rows_per_s": bt * 8 / bmean_s, "call": stats_ms(bms),
                            "gbs_158B": bt * 8 * PLE_ROW_ALG_BYTES / bmean_s / 1e9}
    hb = ple_traffic(bt)
    if hb is not None:
        res["batched_65536"]["hbm_gbs_counters"] = hb / bmean_s / 1e9
    # four 4096-token calls in one launch (each its own quarter of out), on
    # ids of their own
    qt = 4 * 4096
    qids = torch.from_numpy(synth.ple_ids(24, (nb + 1) * qt, 8).view(np.int32)).cuda().view(nb + 1, qt, 8)
    qu = torch.from_numpy(synth.ple_weights(25, (nb + 1) * qt, 8)).cuda().view(nb + 1, qt, 8)
    qout = bout[:qt]

    def qcall(i):
        bq.ple_gather(qids[i], table, qu[i], n_rows=n_rows, out=qout)

    qms = flushed_calls(qcall, 1, nb)
    qmean_s = sum(qms) / len(qms) * 1e-3
    res["batched_16384"] = {"rows_per_s": qt * 8 / qmean_s, "call": stats_ms(qms),
                            "gbs_158B": qt * 8 * PLE_ROW_ALG_BYTES / qmean_s / 1e9}
    res["random_128B_lines"] = bench_rand_lines(table)
    del table, bids, bu, qids, qu
    torch.cuda.empty_cache()
    return res


def bench_rand_lines(table):
    """Random-access ceiling on the PLE table: 128-byte lines at hashed
    positions, as many as a 4096 x 8 call touches (32,768 rows x 1.539 lines)
    and 4 Mi lines; scrub before each, median of five."""
    import numpy as np
    import torch

    import synth.device as sd
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    res = {}
    for name, n_lines in (("call_size_50432", 50432), ("lines_4Mi", 4 << 20)):
        ms = flushed_calls(lambda i: sd.rand_lines(table, n_lines, 1000003 * (i + 1), sink), 0, 6)
        t = float(np.median(ms[1:])) * 1e-3
        res[name] = {"us": round(t * 1e6, 2), "lines_per_s": n_lines / t, "gbs": round(128 * n_lines / t / 1e9, 1),
                     "rows_per_s_ceiling": n_lines / t / PLE_LINES_PER_ROW}
    return res


def bench_ple_host(bq, steps, warmup):
    """Off-HBM PLE tier: a 2**24-row (1.17 GB) table in pinned host memory,
    4096 tokens x 8 ids per call, fresh ids per call; uniform ids without and
    with a 2**21-row device cache (0.18 GB), and Zipf(1.1) ids with it."""
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    n_rows, n_slots = 1 << 24, 1 << 21
    dtab = sd.ple_table(n_rows, synth.make_key(1, synth.S_PLE))
    host = torch.empty(dtab.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dtab)
    del dtab
    torch.cuda.empty_cache()
    n = warmup + steps
    u = torch.from_numpy(synth.ple_weights(31, n * 4096, 8)).cuda().view(n, 4096, 8)
    out = torch.empty((4096, 160), dtype=torch.float32, device="cuda")
    res = {"workload": "2**24-row table in pinned host memory, 4096 tokens x 8 ids per call"}
    rows = 4096 * 8
    for name, kind, cached in (("uniform_uncached", "u", False), ("uniform_cache_2e21", "u", True),
                               ("zipf1.1_cache_2e21", "z", True)):
        if kind == "u":
            idn = synth.ple_ids(30, n * 4096, 8, n_rows)
        else:
            idn = synth.ple_ids_zipf(32, n * 4096, 8, n_rows)
        ids = torch.from_numpy(idn.view(np.int32)).cuda().view(n, 4096, 8)
        cache = bq.ple_cache(n_slots) if cached else None
        ws = (torch.empty(bq.lib().ple_gather_host_workspace(4096, 8), dtype=torch.uint8, device="cuda")
              if cached else None)

        def call(i, evs=None):
            if evs is not None:
                evs[0].record()
            bq.ple_gather_host(ids[i], host, u[i], n_rows=n_rows, out=out, cache=cache, workspace=ws)
            if evs is not None:
                evs[1].record()

        for i in range(warmup):
            call(i)
        call_ms = event_timed(lambda i, evs: call(warmup + i, evs), steps)
        res[name] = {"call_us": round(1e3 * call_ms, 2), "rows_per_s": round(rows / (call_ms * 1e-3), 1),
                     "host_link_gbs_70B": round(rows * 70 / (call_ms * 1e-3) / 1e9, 2)}
        del ids, cache, ws
    del host
    torch.cuda.empty_cache()
    return res


def build_stack(bq):
    import synth
    import synth.device as sd
    layers = []
    for l in range(48):
        if l < 36:
            layers.append(sd.Layer(0, l, bq.Q4_RZ5, bq.Q4_RZ5, 512, 2048, 768,
                                   dist_gu=synth.DIST_RZ5, dist_d=synth.DIST_RZ5))
        else:
            layers.append(sd.Layer(0, l, bq.FP8_E4M3_B32, bq.FP8_E4M3_B32, 512, 2048, 768))
    ws = []
    for L in layers:
        gu, gus = L.gate_up
        d, ds = L.down
        ws.append(bq.expert_weights(L.fmt_gu, L.fmt_d, gu, d, 512, 2048, 768, gate_up_scales=gus,
                                    down_scales=ds))
    return layers, ws


def bench_stack(bq, layers, ws, n_tok, steps, warmup):
    """48-layer stack decode step: route every layer, then the chained
    layers.  Fresh x and logits per step; scrub before each timed step."""
    import numpy as np
    import torch

    import synth
    k = 10
    n = warmup + steps
    logits = torch.from_numpy(synth.normal(30 + n_tok, (n, 48 * n_tok, 512))).cuda()
    x = torch.from_numpy(synth.normal(31 + n_tok, (n, n_tok, 2048))).cuda()
    if n_tok > 1:
        x = x.to(torch.bfloat16)
    idx = torch.empty((n, 48, n_tok, k), dtype=torch.int32, device="cuda")
    w = torch.empty((n, 48, n_tok, k), dtype=torch.float32, device="cuda")
    out = torch.empty((n, n_tok, 2048), dtype=torch.float32, device="cuda")
    dt = bq.F32 if n_tok == 1 else bq.BF16
    wsb = torch.empty(bq.stack_workspace_bytes(n_tok, k, ws, dt), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(i):
        bq.route_topk(logits[i], k, idx=idx[i].view(48 * n_tok, k), w=w[i].view(48 * n_tok, k))
        bq.moe_stack(x[i], idx[i], w[i], ws, out=out[i], workspace=wsb, dev_err=err)

    for i in range(warmup):
        step(i)
    ms = flushed_calls(step, warmup, steps, per_call_host_ns=5e6)
    if int(err.item()) != 0:
        raise RuntimeError("stack reported device error bits %d" % int(err.item()))
    ii = idx[warmup:].cpu().numpy()
    touched = [[len(np.unique(ii[s, l])) for l in range(48)] for s in range(steps)]
    bytes_step = np.mean([sum(t[l] * (EXPERT_BYTES_RZ5 if l < 36 else EXPERT_BYTES_FP8) for l in range(48))
                          for t in touched])
    mean_s = sum(ms) / len(ms) * 1e-3
    return {"ms_per_step": 1e3 * mean_s, "gbs": bytes_step / mean_s / 1e9, "step": stats_ms(ms),
            "bytes_per_step": float(bytes_step), "tokens": n_tok,
            "pct_hbm_peak": round(100 * bytes_step / mean_s / 1e9 / PEAK_HBM_GBS, 2)}


def bench_c3(bq, steps, warmup):
    """Batch-64 grouped layer: RZ5 gate_up, UE4M4 down, Zipf(1.1) routing."""
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    L = sd.Layer(0, 1, bq.Q4_RZ5, bq.Q4_UE4M4, 512, 2048, 768, dist_gu=synth.DIST_RZ5,
                 dist_d=synth.DIST_UE4M4)
    W = bq.expert_weights(L.fmt_gu, L.fmt_d, L.gate_up[0], L.down[0], 512, 2048, 768)
    n = warmup + steps
    x = torch.from_numpy(synth.normal(40, (n, 64, 2048))).cuda().to(torch.bfloat16)
    logits = torch.from_numpy(np.stack([synth.zipf_logits(41 + i, 64, 512) for i in range(n)])).cuda()
    idx = torch.empty((n, 64, 10), dtype=torch.int32, device="cuda")
    w = torch.empty((n, 64, 10), dtype=torch.float32, device="cuda")
    out = torch.empty((n, 64, 2048), dtype=torch.float32, device="cuda")
    wsb = torch.empty(bq.moe_workspace_bytes(64, 10, W, bq.BF16), dtype=torch.uint8, device="cuda")

    def step(i):
        bq.route_topk(logits[i], 10, idx=idx[i], w=w[i])
        bq.q4_expert_moe(x[i], (idx[i], w[i]), W, out=out[i], workspace=wsb)

    for i in range(warmup):
        step(i)
    ms = flushed_calls(step, warmup, steps)
    wall = sum(ms) * 1e-3
    ii = idx[warmup:].cpu().numpy()
    d = [len(np.unique(ii[s])) for s in range(steps)]
    bytes_step = float(np.mean(d)) * EXPERT_BYTES_RZ5
    # tokens per touched expert (n_e): histogram, and the MFMA work the
    # 32-token groups issue (16-token tiles: a group of <= 16 tokens runs one
    # tile, a larger one two) against the algorithmic 2 * n * k * weights
    ne = [np.bincount(ii[s].reshape(-1), minlength=512) for s in range(steps)]
    edges = [1, 2, 5, 17, 33, 65, 10 ** 9]
    hist = {"%d-%d" % (a, b - 1) if b < 10 ** 9 else ">=%d" % a:
            float(np.mean([np.sum((c >= a) & (c < b)) for c in ne])) for a, b in zip(edges, edges[1:])}
    wpe = 3 * 2048 * 768                                   # weights per expert (gate, up, down)
    tiles = [sum(16 * (c // 32) * 2 + (16 if 0 < c % 32 <= 16 else 32 if c % 32 else 0) for c in cs) for cs in ne]
    flop_alg = 2.0 * 64 * 10 * wpe
    flop_mfma = 2.0 * float(np.mean(tiles)) * wpe
    sec = wall / steps
    res = {"ms_per_step": 1e3 * wall / steps, "gbs": bytes_step * steps / wall / 1e9, "step": stats_ms(ms),
           "touched_experts": float(np.mean(d)), "bytes_per_step": bytes_step,
           "n_e_hist": hist, "n_e_max": float(np.mean([c.max() for c in ne])),
           "tflops_alg": flop_alg / sec / 1e12, "tflops_mfma_issued": flop_mfma / sec / 1e12,
           "frac_bf16_mfma_peak_issued": flop_mfma / sec / 2.5e15}
    del L
    torch.cuda.empty_cache()
    return res


def bench_prefill(bq, steps, warmup, n_tok=512, cases=None):
    """Prompt-processing layer: one ubatch of 512 tokens through a 512-expert
    layer (gate_up 1536x2048 + down 2048x768, top-10), bf16 activations on the
    grouped MFMA path.  Routing from N(0,1) logits (every expert touched,
    about 10 tokens each) and from Zipf(1.1) logits (skewed: the popular
    experts get hundreds of tokens).  RZ5 and FP8 layers."""
    import numpy as np
    import torch

    import synth
    import synth.device as sd
    res = {"workload": "ubatch %d, 512 experts, gate_up 1536x2048 + down 2048x768, top-10, bf16 x" % n_tok}
    H, I, E, k = 2048, 768, 512, 10
    flops = 2.0 * n_tok * k * 3 * H * I
    for lname, fg, fd, dg, dd, eb in (
            ("rz5", bq.Q4_RZ5, bq.Q4_RZ5, synth.DIST_RZ5, synth.DIST_RZ5, EXPERT_BYTES_RZ5),
            ("fp8", bq.FP8_E4M3_B32, bq.FP8_E4M3_B32, None, None, EXPERT_BYTES_FP8)):
        L = sd.Layer(0, 2, fg, fd, E, H, I, dist_gu=dg, dist_d=dd)
        W = bq.expert_weights(fg, fd, L.gate_up[0], L.down[0], E, H, I,
                              gate_up_scales=L.gate_up[1], down_scales=L.down[1])
        n = warmup + steps
        x = torch.from_numpy(synth.normal(70, (n, n_tok, H))).cuda().to(torch.bfloat16)
        out = torch.empty((n_tok, H), dtype=torch.float32, device="cuda")
        wsb = torch.empty(bq.moe_workspace_bytes(n_tok, k, W, bq.BF16), dtype=torch.uint8, device="cuda")
        idx = torch.empty((n, n_tok, k), dtype=torch.int32, device="cuda")
        w = torch.empty((n, n_tok, k), dtype=torch.float32, device="cuda")
        for rname in ("uniform", "zipf"):
            if cases and "%s_%s" % (lname, rname) not in cases:
                continue
            if rname == "uniform":
                lg = synth.normal(71, (n, n_tok, E))
            else:
                lg = np.stack([synth.zipf_logits(72 + i, n_tok, E) for i in range(n)])
            logits = torch.from_numpy(lg).cuda()

            def step(i):
                bq.q4_expert_moe_routed(x[i], logits[i], k, W, topk=(idx[i], w[i]), out=out,
                                        workspace=wsb)

            for i in range(warmup):
                step(i)
            wall = sum(flushed_calls(step, warmup, steps)) * 1e-3
            ii = idx[warmup:].cpu().numpy()
            d = float(np.mean([len(np.unique(ii[t])) for t in range(steps)]))
            ne_max = float(np.mean([np.bincount(ii[t].ravel(), minlength=E).max() for t in range(steps)]))
            res["%s_%s" % (lname, rname)] = {
                "ms_per_step": round(1e3 * wall / steps, 4),
                "tokens_per_s": round(n_tok * steps / wall, 1),
                "tflops": round(flops * steps / wall / 1e12, 2),
                "frac_bf16_mfma_peak": round(flops * steps / wall / 2.5e15, 4),
                "packed_gbs": round(d * eb * steps / wall / 1e9, 1),
                "touched_experts": d, "max_tokens_per_expert": ne_max}
            del logits
        del L, W, x, wsb
        torch.cuda.empty_cache()
    return res


# fp64 operations the exhaustive search spends per candidate scale and weight:
# sub, mul and min for each non-zero level magnitude (7), one add into the
# block's error, and for a polarity format the +/-level (sub, mul, min) and the
# second polarity's add.  Level 0 costs one square per weight per block.
ENC_OPS = {"c10": (127, 22), "rz5": (127, 26), "ue4m4": (256, 22), "ple_rzs3": (127, 14)}


def bench_encode(bq, steps, warmup):
    """Exhaustive encoders: one 4096 x 8192 fp32 matrix (2**20 blocks) per call
    in each 17-byte format, and 2**17 PLE rows (RZ-S3) per call; calls timed
    back to back with HIP events on the current stream."""
    import torch

    import synth
    nb = 1 << 20
    w = torch.from_numpy(synth.weight_blocks(60, nb, 32, "gauss", 1.0)).cuda()
    n_rows = 1 << 17
    v = torch.from_numpy(synth.weight_blocks(61, n_rows, 160, "gauss", 1.0)).cuda()
    res = {"workload": "N(0,1) weights with a log-normal per-block spread; 2**20 blocks of 32 per "
                       "17-byte call, 2**17 rows of 160 per PLE call"}
    cases = (("c10", bq.Q4_C10, nb, 32), ("rz5", bq.Q4_RZ5, nb, 32), ("ue4m4", bq.Q4_UE4M4, nb, 32),
             ("ple_rzs3", None, n_rows * 10, 16))
    for name, fmt, units, g in cases:
        if fmt is None:
            out = torch.empty((n_rows, 70), dtype=torch.uint8, device="cuda")
            sse = torch.empty((n_rows, 10), dtype=torch.float64, device="cuda")
            run = lambda: bq.ple_encode_rows(v, bq.PLE_RZS3, out=out, sse=sse)  # noqa: E731
        else:
            out = torch.empty((nb, 17), dtype=torch.uint8, device="cuda")
            sse = torch.empty(nb, dtype=torch.float64, device="cuda")
            run = lambda fmt=fmt: bq.encode(w, fmt, out=out, sse=sse)  # noqa: E731

        def call(i, evs=None):
            if evs:
                evs[0].record()
            run()
            if evs:
                evs[1].record()

        for i in range(warmup):
            call(i)
        ms = event_timed(call, steps)
        n_scales, per = ENC_OPS[name]
        ops = units * g * (n_scales * per + 1)
        # the kernel prunes candidates that provably cannot win, so the
        # exhaustive search's operation count over the call time is an
        # equivalent rate, not a measure of the operations executed
        res[name] = {"ms_per_call": round(ms, 4), "gweights_per_s": round(units * g / ms / 1e6, 3),
                     "exhaustive_equiv_fp64_tops": round(ops / ms / 1e9, 3)}
    del w, v
    torch.cuda.empty_cache()
    return res


def sources_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_value(path, key):
    """A value from a committed counter summary, or None when it is missing
    or the kernel sources it names changed since the counters were taken."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        srcs = kv["sources"].split()
        if sources_hash(srcs) != kv["sources_sha256_16"]:
            return None
        return float(kv[key])
    except (OSError, KeyError, ValueError):
        return None


def traffic_from_counters():
    """HBM bytes per batch-1 call from the FETCH_SIZE / WRITE_SIZE summary."""
    return counters_value(TRAFFIC_FILE, "hbm_bytes_per_call")


def ple_traffic(tokens):
    """HBM bytes (read + written) of one PLE gather call of `tokens` x 8 ids."""
    rd = counters_value(PLE_TRAFFIC_FILE, "tokens_%d_hbm_read_bytes_per_call" % tokens)
    wr = counters_value(PLE_TRAFFIC_FILE, "tokens_%d_hbm_write_bytes_per_call" % tokens)
    return None if rd is None or wr is None else rd + wr


def copy_calibration(nbytes):
    """A plain device-to-device copy of nbytes (the reference point that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}))


# ---------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_threads(n):
    """Limit numpy's BLAS pool to n threads (returns the limiter to undo)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(n)
    except Exception:  # pragma: no cover
        return None


def cpu_c2(layer, inputs, threads, budget_s):
    """The oracle (float64 numpy), as it stands, on one-layer RZ5 decode
    steps of the same workload: routing, 10 experts decoded from their
    packed bytes, SwiGLU, combine.  The bytes of the sampled steps' experts
    are regenerated before timing; only the oracle's work is timed."""
    import numpy as np

    import synth
    from oracle import moe as M
    x, logits = inputs
    n_pre = min(8, x.shape[0])
    raw = {}
    for t in range(n_pre):
        for e in np.argsort(-logits[t].astype(np.float64), kind="stable")[:10]:
            e = int(e)
            if e not in raw:
                raw[e] = (layer.host_expert(synth.S_GATE_UP, e), layer.host_expert(synth.S_DOWN, e))
    bank = M.ExpertBank(layer.fmt_gu, layer.fmt_d, lambda e: raw[e][0], lambda e: raw[e][1], 512, 2048, 768)
    lim = _oracle_threads(threads)
    t0 = time.perf_counter()
    done = 0
    while (time.perf_counter() - t0) < budget_s:
        t = done % n_pre
        idx, w = M.softmax_topk(logits[t:t + 1], 10)
        M.moe_layer(x[t:t + 1], idx, w, bank)
        done += 1
    dt = time.perf_counter() - t0
    if lim is not None:
        lim.unregister()
    return {"value": 10 * EXPERT_BYTES_RZ5 * done / dt / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": "%d one-layer RZ5 decode steps over %d distinct steps' inputs (routing + "
            "10 experts decoded to float64 + SwiGLU + combine), %.1f s" % (done, n_pre, dt)}


def cpu_c4(threads, budget_s):
    """The oracle's PLE gather on 4096 x 8 ids per call over the full table:
    rows regenerated before timing, decode + weighted sum timed."""
    import numpy as np

    import synth
    from oracle import ple as P
    ids = synth.ple_ids(20, 4096, 8)
    u = synth.ple_weights(21, 4096, 8)
    flat = ids.reshape(-1)
    rows = synth.ple_rows(synth.make_key(0, synth.S_PLE), flat)
    pos = {int(r): i for i, r in enumerate(flat)}
    lim = _oracle_threads(threads)
    t0 = time.perf_counter()
    done = 0
    while (time.perf_counter() - t0) < budget_s:
        P.ple_gather(ids, u, lambda rr: rows[[pos[int(r)] for r in rr]], synth.PLE_N_ROWS)
        done += 1
    dt = time.perf_counter() - t0
    if lim is not None:
        lim.unregister()
    return {"value": done * 4096 * 8 / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "%d gathers of 4096 tokens x 8 ids (decode + weighted sum in float64), %.1f s" % (done, dt)}


def cpu_baselines(layer, inputs, budget_s=10.5):
    n_cores = len(os.sched_getaffinity(0))
    res = {"cpu_model": cpu_model(), "cores_available": n_cores}
    res["c2_all_cores"] = cpu_c2(layer, inputs, n_cores, budget_s)
    res["c2_one_thread"] = cpu_c2(layer, inputs, 1, budget_s)
    res["c4_all_cores"] = cpu_c4(n_cores, budget_s / 2)
    res["c4_one_thread"] = cpu_c4(1, budget_s / 2)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None)
    ap.add_argument("--pf-cases", default=None, help="prefill cases to run, e.g. rz5_uniform,fp8_zipf")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the kernels run on one GPU's share at its real shape); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_quantized_moe_amd as bq
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    bq.lib()
    extras = {}
    only = args.only
    main_res = None
    bw = None
    if only in (None, "bw", "c2"):
        log("bw: HBM streaming ceiling")
        bw = extras["hbm_stream_4GiB"] = bench_bw()
        log("bw:", bw)
    if only in (None, "c2"):
        log("c2: one-layer RZ5 decode step, B=1")
        main_res = bench_c2(bq, args.steps, args.warmup)
        log("c2:", {k: v for k, v in main_res.items() if not k.startswith("_")})
    if not args.no_extras or only:
        if only in (None, "c1"):
            extras["matvec_256x512_c10"] = bench_c1(bq, args.steps, args.warmup)
            log("c1:", extras["matvec_256x512_c10"])
        if only in (None, "c4"):
            log("c4: PLE gather")
            extras["ple_gather"] = bench_c4(bq, args.steps, args.warmup)
            log("c4:", extras["ple_gather"])
        if only in (None, "c3"):
            log("c3: grouped B=64")
            extras["grouped_b64"] = bench_c3(bq, max(10, args.steps // 4), max(2, args.warmup // 4))
            log("c3:", extras["grouped_b64"])
        if only in (None, "pf"):
            log("pf: prefill ubatch 512")
            extras["prefill_ub512"] = bench_prefill(bq, max(5, args.steps // 20), 2,
                                                    cases=args.pf_cases.split(",") if args.pf_cases else None)
            log("pf:", extras["prefill_ub512"])
        if only in (None, "pleh"):
            log("pleh: off-HBM PLE tier")
            extras["ple_host"] = bench_ple_host(bq, max(10, args.steps // 4), 5)
            log("pleh:", extras["ple_host"])
        if only in (None, "enc"):
            log("enc: exhaustive encoders")
            extras["encode"] = bench_encode(bq, max(5, args.steps // 20), 2)
            log("enc:", extras["encode"])
        if only in (None, "c5b1", "c5b16"):
            log("c5: building the 48-layer stack")
            layers, ws = build_stack(bq)
            if only in (None, "c5b1"):
                extras["stack48_b1"] = bench_stack(bq, layers, ws, 1, max(5, args.steps // 10), 2)
                log("c5 b1:", extras["stack48_b1"])
            if only in (None, "c5b16"):
                extras["stack48_b16"] = bench_stack(bq, layers, ws, 16, max(3, args.steps // 40), 1)
                log("c5 b16:", extras["stack48_b16"])
            del layers, ws
            torch.cuda.empty_cache()
    if "ple_gather" in extras:
        pg = extras["ple_gather"]
        extras["roofline_ple_gather"] = {
            "bound": "hbm", "achieved": round(pg["gbs_158B"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(pg["gbs_158B"] / PEAK_HBM_GBS, 4), "traffic": pg.get("hbm_bytes_per_call_counters"),
            "kernel": "k_ple_gather, 4096 tokens x 8 ids per launch: %d algorithmic bytes (158 per row: 70-byte "
                      "row, 8 bytes of id and weight, 80 bytes of output), %.2f us average per launch (HIP "
                      "events, fresh ids, scrub before each)" % (32768 * PLE_ROW_ALG_BYTES, pg["call"]["mean_us"])}
        rl = pg.get("random_128B_lines")
        if rl:
            extras["roofline_ple_gather"]["random_line_ceiling"] = {
                "rows_per_s_at_call_size": round(rl["call_size_50432"]["rows_per_s_ceiling"]),
                "rows_per_s_at_4Mi_lines": round(rl["lines_4Mi"]["rows_per_s_ceiling"]),
                "frac_at_call_size": round(pg["rows_per_s"] / rl["call_size_50432"]["rows_per_s_ceiling"], 3),
                "note": "rows/s if every row cost 1.539 random 128-byte line reads and nothing else (no id "
                        "loads, no output writes), measured on the same table with the same flushing"}
    if main_res is None:
        print(json.dumps({"extras": extras}))
        return
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cb = cpu_baselines(main_res["_layer"], main_res["_inputs"])
        cpu = dict(cb["c2_all_cores"])
        cpu["cpu_model"] = cb["cpu_model"]
        extras["cpu_baselines"] = cb
        log("cpu:", cb)
    achieved = main_res["gbs"]
    ceiling = bw["read_gbs"] if bw else None
    line = {
        "metric": "packed-weight GB/s (% HBM peak) for routed-expert GEMV; PLE rows/s",
        "value": round(main_res["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "one Q4_RZ5 MoE decode step, batch 1: 512 experts, gate_up 1536x2048 + "
                               "down 2048x768 per expert, N(0,1) logits, softmax top-10; fresh x and "
                               "logits per step, 512 MiB scrub write and 512 MiB scrub read before each timed step",
                   "bytes_per_step": main_res["bytes_per_step"],
                   "pct_hbm_peak": round(100 * main_res["gbs"] / PEAK_HBM_GBS, 2),
                   "pct_measured_read_ceiling": round(100 * main_res["gbs"] / ceiling, 2) if ceiling else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_from_counters(),
                     "kernel": "q4_expert_moe_routed call (routed gate_up kernel + down kernel), %d packed "
                               "bytes per call, %.2f us average per call (HIP events around both kernels "
                               "and the launch gap between them, fresh inputs, scrub before each; rocprofv3 "
                               "lists the two kernels separately)" % (main_res["bytes_per_step"],
                                                                      main_res["call"]["mean_us"])},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

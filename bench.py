"""Benchmark of the CSA decode hot path on one MI355X.

One step = one decode token for each of the B sequences through the whole
path, every kernel from libcsa, in three launches:
  1. csa_compress_score -- three compress jobs (fold the newest block of m
                      tokens of every sequence into its cache entry: split
                      FP8/BF16 row, RMSNorm, RoPE; the matching indexer key,
                      FP8; the new token's sliding-window row, m = 1) and the
                      ReLU multi-head indexer scores over every visible entry,
                      the new keys scored by the workgroups that write them
  2. topk_select   -- the k best entries, ascending
  3. hybrid_attn_decode -- sink MQA over the selected entries + window
`two_launches_topk_fused` times the same step with the top-k selected inside
the first launch (csa_compress_score_topk: the last workgroup to finish a
query's scores selects them), `four_launches` with csa_compress_batch and
indexer_score as two launches.
Inputs are seeded synthetic tensors already resident in HBM.  The per-layer
state a step reads (KV cache, index keys, window rows) exists in R copies
(default 13, about 2.4 GB) stepped in turn, so that it cannot stay in the
256 MB last-level cache between steps, as in a model whose every layer has its
own cache; `value_one_warm_cache` repeats one copy.  The R copies' steps are
captured in order in one HIP graph (a pass through R layers); W warm-up
steps, then exactly K timed steps between two synchronised events.  The workload is the CSA decode batch of 16
sequences of 65,536 tokens (16,384 compressed entries each, top-k 512, FP8
indexer 64 x 128, 64 query heads, head dim 512).

Prints one JSON line.  `roofline` is measured for the dominant launch
(csa_compress_score, whose indexer part moves most of the step's bytes): the
indexer's input bytes (every visible key, the index query and head weights)
over the launch's mean period when launched back to back between two events
on its stream (duration plus dispatch gap, so never shorter than the traced
duration); `kernels` gives every kernel's period the same way, its bytes and
FLOPs against the HBM and BF16 MFMA peaks; `hbm_frac_step` is the step's byte
model over the step time; `fp32_b1_ctx2048` times the all-float32 step of one
2,048-token sequence; `cpu_baseline` times the float64 oracle on a bounded
sample on the host, with every BLAS thread and with one.  `context_scan` repeats the
step at 256K and 1M tokens per sequence; `hca_decode` the HCA decode step
(32 x 262,144 tokens, every compressed entry attended); `ragged` a CSA layer
(MXFP4 indexer, top-1,024) and an HCA layer over 64 sequences of 1K to 1M
tokens; `prefill` the CSA prefill
chunk (2,048 tokens after 131,072 cached: compress, indexer, top-k 1,024,
prefill attention) and the contractions' MFMA rates; `cp_select_and_pad` the
context-parallel reassembly of a 1M-token sequence's compressed cache from 8
shards.  `--copy-probe MIB` only
runs a plain copy of known size, the reference for rocprofv3 byte counters.
"""
import argparse
import hashlib
import json
import os
import sys
import time
import types

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import compressed_sparse_long_csa_amd as csa  # noqa: E402
from compressed_sparse_long_csa_amd import synth  # noqa: E402

METRIC = "CSA/HCA decode query-tokens/s and achieved HBM GB/s at 64K-1M context"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
EPS, BASE = 1e-6, 10000.0


WORKLOAD = "csa_decode_b16_ctx65536"


def build_workload(name=WORKLOAD, B=None, L=None, seed=2):
    c = synth.WORKLOADS[name]
    inp = synth.workload_decode_inputs(name, seed=seed, B=B, L=L)
    m, D, R, d_I = c["m"], c["D"], c["R"], c["d_I"]
    rng = synth.rng_for(seed + 1000)
    Bn = inp.B
    # the newest complete block of every sequence, its index-key tokens, and the newest token
    kv_tok = rng.standard_normal((Bn * m, D), dtype=np.float32)
    kv_gate = rng.standard_normal((Bn * m, 1), dtype=np.float32)
    key_tok = rng.standard_normal((Bn * m, d_I), dtype=np.float32)
    key_gate = rng.standard_normal((Bn * m, 1), dtype=np.float32)
    win_tok = rng.standard_normal((Bn, D), dtype=np.float32)
    win_gate = np.zeros((Bn, 1), dtype=np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    W = dict(
        c=c, inp=inp, B=Bn, m=m, D=D, R=R, d_I=d_I,
        q=dev(inp.q), q_pos=dev(inp.q_pos), kv=dev(inp.kv), kv_off=dev(inp.kv_off),
        win=dev(inp.win), win_len=dev(inp.win_len), sinks=dev(inp.sinks),
        keys=dev(inp.keys), q_idx=dev(inp.q_idx), w=dev(inp.w),
        kv_tok=dev(kv_tok).to(torch.bfloat16), kv_gate=dev(kv_gate),
        key_tok=dev(key_tok).to(torch.bfloat16), key_gate=dev(key_gate),
        win_tok=dev(win_tok).to(torch.bfloat16), win_gate=dev(win_gate),
    )
    _step_state(W, inp, Bn, m)
    return W


def build_device_workload(L, B=16, seed=7):
    """The same CSA decode step at context L (B sequences), drawn on the
    device (seeded), for the context scan."""
    c = synth.WORKLOADS[WORKLOAD]
    m, D, R, d_I = c["m"], c["D"], c["R"], c["d_I"]
    d = synth.device_decode_inputs(seed, [L] * B, m=m, H=c["H"], D=D, R=R, n_win=128, csa=True,
                                   k=c["k"], H_I=c["H_I"], d_I=d_I)
    inp = types.SimpleNamespace(n_win=d["n_win"], scale=d["scale"], n_ent=d["n_ent"],
                                win_len=d["win_len"], kv_off=d["kv_off"], q_pos=d["q_pos"])
    gen = synth.device_generator(seed + 1000)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)  # noqa: E731
    W = dict(c=c, inp=inp, B=B, m=m, D=D, R=R, d_I=d_I, q=d["q"],
             q_pos=torch.as_tensor(d["q_pos"], device="cuda"), kv=d["kv"],
             kv_off=torch.as_tensor(d["kv_off"], device="cuda"), win=d["win"],
             win_len=torch.as_tensor(d["win_len"], device="cuda"), sinks=d["sinks"], keys=d["keys"],
             q_idx=d["q_idx"], w=d["w"],
             kv_tok=rnd(B * m, D).to(torch.bfloat16), kv_gate=rnd(B * m, 1),
             key_tok=rnd(B * m, d_I).to(torch.bfloat16), key_gate=rnd(B * m, 1),
             win_tok=rnd(B, D).to(torch.bfloat16), win_gate=torch.zeros((B, 1), device="cuda"))
    _step_state(W, inp, B, m)
    return W


def _step_state(W, inp, Bn, m):
    """Segments of the step's compress jobs, and the scratch / output tensors."""
    n_ent = torch.from_numpy(np.asarray(inp.n_ent))
    last = torch.from_numpy(np.asarray(inp.kv_off)) + n_ent - 1
    W["seg_off"] = (torch.arange(0, Bn + 1, dtype=torch.int64) * m).cuda()
    W["seg_pos0"] = ((n_ent - 1) * m).cuda()                # first token of the newest block
    W["seg_row"] = last.cuda()
    W["win_seg_off"] = torch.arange(0, Bn + 1, dtype=torch.int64).cuda()
    W["win_pos0"] = torch.from_numpy(np.asarray(inp.q_pos)).cuda()
    W["win_row"] = (torch.arange(Bn, dtype=torch.int64) * inp.n_win
                    + (torch.from_numpy(np.asarray(inp.win_len)).long() - 1)).cuda()
    W["n_valid"] = n_ent.cuda()
    W["ld"] = int(np.asarray(inp.n_ent).max())
    W["scores"] = torch.empty((Bn, W["ld"]), dtype=torch.float32, device="cuda")
    W["idx"] = torch.empty((Bn, W["c"]["k"]), dtype=torch.int32, device="cuda")
    W["out"] = torch.empty((Bn, W["c"]["H"], W["D"]), dtype=torch.bfloat16, device="cuda")


def make_replicas(W, R):
    """R copies of the per-layer state a decode step reads (KV cache, index
    keys, window rows); everything else is shared.  Stepping through the
    replicas in turn keeps the working set (R x ~40 MB) above twice the
    256 MB last-level cache, so the kernels read HBM, as a model whose every
    layer has its own cache does."""
    reps = [W]
    for _ in range(R - 1):
        Wr = dict(W)
        Wr["kv"], Wr["keys"], Wr["win"] = W["kv"].clone(), W["keys"].clone(), W["win"].clone()
        reps.append(Wr)
    return reps


def step_jobs(W):
    """The decode step's compress jobs: the newest block's KV entry, its
    indexer key, and the newest token's window row."""
    B, m, D, R, d_I = W["B"], W["m"], W["D"], W["R"], W["d_I"]

    def job(x, gate, n_tok, D, mm, off, pos0, rows, normalize, R_, out, fmt):
        return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=n_tok, D=D, m=mm, nseg=B,
                    seg_tok_off=off, seg_pos0=pos0, seg_out_row=rows, normalize=normalize,
                    norm_w=None, eps=EPS, rope_dim=R_, rope_base=BASE, out=out, out_fmt=fmt)
    return [job(W["kv_tok"], W["kv_gate"], B * m, D, m, W["seg_off"], W["seg_pos0"], W["seg_row"],
                1, R, W["kv"], csa.SPLIT),
            job(W["key_tok"], W["key_gate"], B * m, d_I, m, W["seg_off"], W["seg_pos0"],
                W["seg_row"], 0, 0, W["keys"], csa.FP8),
            job(W["win_tok"], W["win_gate"], B, D, 1, W["win_seg_off"], W["win_pos0"], W["win_row"],
                1, R, W["win"], csa.BF16)]


def make_step(W, check=False, fused=True, topk_fused=False):
    """The decode step's launches.  fused (the default): csa_compress_score,
    topk_select, hybrid_attn_decode; with topk_fused: csa_compress_score_topk,
    hybrid_attn_decode (two launches); not fused: csa_compress_batch,
    indexer_score, topk_select, hybrid_attn_decode."""
    c, inp = W["c"], W["inp"]
    B, m, D, R, d_I, H, k = W["B"], W["m"], W["D"], W["R"], W["d_I"], c["H"], c["k"]
    jobs = step_jobs(W)
    if topk_fused and "tk_ws" not in W:
        W["tk_ws"] = torch.zeros(csa.score_topk_workspace_bytes(B), dtype=torch.uint8, device="cuda")

    def k_compress_score_topk():
        csa.csa_compress_score_topk(jobs, W["q_idx"], W["w"], B, c["H_I"], d_I, W["keys"], csa.FP8, W["kv_off"],
                                    W["q_pos"], m, W["scores"], W["ld"], k, W["idx"], workspace=W["tk_ws"],
                                    check=check)

    def k_compress():
        csa.csa_compress_batch(jobs, check=check)

    def k_compress_score():
        csa.csa_compress_score(jobs, W["q_idx"], W["w"], B, c["H_I"], d_I, W["keys"], csa.FP8, W["kv_off"],
                               W["q_pos"], m, W["scores"], W["ld"], check=check)

    def k_indexer():
        csa.indexer_score(W["q_idx"], W["w"], B, c["H_I"], d_I, W["keys"], csa.FP8, W["kv_off"],
                          W["q_pos"], m, W["scores"], W["ld"], check=check)

    def k_topk():
        csa.topk_select(W["scores"], W["ld"], B, W["n_valid"], k, W["idx"], None, check=check)

    def k_attn():
        csa.hybrid_attn_decode(W["q"], csa.BF16, B, H, D, W["q_pos"], None, EPS, R, BASE, W["kv"],
                               csa.SPLIT, W["kv_off"], m, W["idx"], k, W["win"], csa.BF16,
                               inp.n_win, W["win_len"], W["sinks"], inp.scale, W["out"], csa.BF16,
                               csa.VARIANT_AUTO, check=check)

    if fused and topk_fused:
        kernels = [("csa_compress_score_topk", k_compress_score_topk), ("hybrid_attn_decode", k_attn)]
    elif fused:
        kernels = [("csa_compress_score", k_compress_score), ("topk_select", k_topk),
                   ("hybrid_attn_decode", k_attn)]
    else:
        kernels = [("csa_compress_batch", k_compress), ("indexer_score", k_indexer),
                   ("topk_select", k_topk), ("hybrid_attn_decode", k_attn)]

    def step():
        for _, f in kernels:
            f()
    return step, kernels


def algorithmic_bytes(W):
    """Bytes the method must move per step (each input read once, each output
    written once); scratch round trips (scores, idx) are counted per kernel."""
    inp, c = W["inp"], W["c"]
    B, D, R, m, d_I, H, k = W["B"], W["D"], W["R"], W["m"], W["d_I"], c["H"], c["k"]
    N = inp.n_ent.astype(np.int64)
    split = (D - R) + 2 * R
    sel = np.minimum(k, N)
    per_kernel = {
        "csa_compress_batch": (B * m * (2 * D + 4) + B * split            # KV entries
                               + B * m * (2 * d_I + 4) + B * d_I         # indexer keys
                               + B * (2 * D + 4) + B * 2 * D),           # window rows
        "indexer_score": int((N * (d_I + 4)).sum()) + B * c["H_I"] * (d_I + 4),
        "topk_select": int((N * 4).sum()) + B * k * 4,
        "hybrid_attn_decode": int((sel * split).sum()) + int(inp.win_len.sum()) * 2 * D
        + B * k * 4 + B * H * D * 2 * 2 + H * 4,
    }
    per_kernel["csa_compress_score"] = per_kernel["csa_compress_batch"] + per_kernel["indexer_score"]
    per_kernel["csa_compress_score_topk"] = per_kernel["csa_compress_score"] + B * k * 4
    # the indexer's inputs alone (every visible key, the index query and head
    # weights of each query): the step byte model's share of the launch, with
    # the score writes (scratch) and the compress jobs left out
    per_kernel["indexer_inputs"] = int((N * d_I).sum()) + B * c["H_I"] * (d_I + 4)
    step_bytes = (int((N * d_I).sum()) + B * c["H_I"] * (d_I + 4) + int((sel * split).sum())
                  + int(inp.win_len.sum()) * 2 * D + B * H * D * 2 * 2 + H * 4)
    return step_bytes, per_kernel


def algorithmic_flops(W):
    """Matrix FLOPs of the two contraction kernels (2 per multiply-add)."""
    inp, c = W["inp"], W["c"]
    N = inp.n_ent.astype(np.int64)
    sel = np.minimum(c["k"], N) + inp.win_len.astype(np.int64)
    idx = int(2 * N.sum() * c["H_I"] * W["d_I"])
    return {"indexer_score": idx, "csa_compress_score": idx, "csa_compress_score_topk": idx,
            "hybrid_attn_decode": int(2 * 2 * sel.sum() * c["H"] * W["D"])}


def time_graph(steps_r, steps, warmup, spread=0):
    """Replica r's step is captured once on its own and once more, in replica
    order, inside one graph of all R steps (a decode pass through R layers,
    as a model would capture it).  W warm-up steps, then exactly `steps` timed
    steps between two synchronised events: whole R-step graphs, then the
    single-step graphs of the remainder.  Returns ms per step; with spread > 0
    also the p10 / median / p90 of ms per step over `spread` replays of the
    R-step graph, each between its own pair of events."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for st in steps_r:
            st()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    singles = []
    for st in steps_r:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st()
        singles.append(g)
    R = len(singles)
    chain = singles[0]
    if R > 1:
        chain = torch.cuda.CUDAGraph()
        with torch.cuda.graph(chain):
            for st in steps_r:
                st()

    def run(n):
        for _ in range(n // R):
            chain.replay()
        for j in range(n % R):
            singles[j].replay()
    run(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if spread <= 0:
        return ms
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(spread + 1)]
    ev[0].record()
    for i in range(spread):
        chain.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) / R for i in range(spread)])
    return ms, {"p10": float(np.percentile(per, 10)), "median": float(np.median(per)),
                "p90": float(np.percentile(per, 90)), "graphs": spread, "steps_per_graph": R}


def time_eager(steps_r, steps, warmup):
    """The same steps launched one call at a time from Python (no graph):
    ms per step between two events; bound by the host's launch rate."""
    for i in range(warmup):
        steps_r[i % len(steps_r)]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        steps_r[i % len(steps_r)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _event_pairs(fs, steps):
    """Mean time between two events recorded around f() on the current stream,
    f taken in turn from fs.  A spin kernel is queued first, so every launch of
    the loop is enqueued before the GPU reaches it and host launch latency never
    sits between two events."""
    ev = []
    torch.cuda._sleep(int(2e7))
    for i in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fs[i % len(fs)]()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev]))


def _batch_period(fs, steps):
    """Mean time per launch of `steps` launches queued back to back (f taken in
    turn from fs) between two events, behind a spin kernel: each launch's
    duration plus the dispatch gap to the next."""
    torch.cuda._sleep(int(2e7))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fs[i % len(fs)]()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / steps


def kernel_periods(kernels_r, steps):
    """Every kernel's mean back-to-back launch period (us), launches rotating
    over the replicas."""
    names = [n for n, _ in kernels_r[0]]
    return {n: _batch_period([kr[j][1] for kr in kernels_r], steps) for j, n in enumerate(names)}


def time_kernels(kernels_r, steps, batch=None):
    """Average device duration (us) of every kernel, launches rotating over the
    replicas: events around each launch on the stream the kernel runs on
    (torch's current stream), less the time between two events with nothing in
    between.  `batch` (a dict) receives each kernel's back-to-back launch
    period as well."""
    empty = _event_pairs([lambda: None], steps)
    names = [n for n, _ in kernels_r[0]]
    out = {}
    for j, n in enumerate(names):
        out[n] = _event_pairs([kr[j][1] for kr in kernels_r], steps) - empty
        if batch is not None:
            batch[n] = _batch_period([kr[j][1] for kr in kernels_r], steps)
    return out, empty


def copy_probe(mb, reps):
    """A plain elementwise copy (y = x * 1) of mb MiB, reps times: the
    known-size reference (mb MiB read, mb MiB written per launch) for
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings."""
    n = mb * 1024 * 1024 // 4
    x = torch.ones(n, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_read_bytes_per_launch": n * 4, "launches": reps}), flush=True)


def copy_gbps(mb=512, reps=20):
    """Read + write bandwidth of torch's elementwise copy of mb MiB (two
    buffers used in turn, each larger than the last-level cache): the rate a
    plain streaming kernel reaches on this part, for comparison."""
    n = mb * 1024 * 1024 // 4
    xs = [torch.ones(n, device="cuda") for _ in range(2)]
    y = torch.empty_like(xs[0])
    fs = [lambda x=x: torch.mul(x, 1.0, out=y) for x in xs]
    fs[0]()
    torch.cuda.synchronize()
    us = _batch_period(fs, reps)
    return 2 * n * 4 / (us * 1e-6) / 1e9


def spot_check(W):
    """Compare the step's attention output for one sequence with the oracle."""
    from oracle import formats as OF
    from oracle import method as OM
    inp = W["inp"]
    b = 0
    N = int(inp.n_ent[b])
    idx = W["idx"][b].cpu().numpy()
    sel = idx[idx >= 0]
    kv = W["kv"].cpu().numpy()
    off = int(inp.kv_off[b])
    ents = np.zeros((N, W["D"]))
    ents[sel] = OF.decode_rows(kv[off + sel], csa.SPLIT, W["D"], W["R"])
    wl = int(inp.win_len[b])
    win = OF.decode_rows(W["win"][b, :wl].cpu().numpy(), csa.BF16, W["D"])
    q = OF.decode_rows(inp.q[b], csa.BF16, W["D"])
    ref = OM.decode_one(q, int(inp.q_pos[b]), ents, win, inp.sinks.astype(np.float64), inp.scale,
                        W["m"], idx=sel, R=W["R"])
    got = OF.decode_rows(W["out"][b].view(torch.uint8).cpu().numpy(), csa.BF16, W["D"]).reshape(ref.shape)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return float((np.abs(got - ref) / rms).max())


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _physical_cores():
    try:
        import psutil
        return psutil.cpu_count(logical=False)
    except Exception:  # pragma: no cover
        return None


def _oracle_sample(W, budget_s):
    """The float64 oracle (indexer -> top-k -> sink MQA) on the step's inputs,
    one decode query at a time, until the time budget is used: (queries, s)."""
    from oracle import formats as OF
    from oracle import method as OM
    inp = W["inp"]
    c = W["c"]
    kv = inp.kv
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = done % inp.B
        N = int(inp.n_ent[b])
        off = int(inp.kv_off[b])
        keys = OF.decode_rows(inp.keys[off: off + N], csa.FP8, c["d_I"])
        qi = OF.decode_rows(inp.q_idx[b], csa.FP8, c["d_I"])
        I = OM.indexer_scores(qi, inp.w[b].astype(np.float64), keys)
        sel = OM.top_k(I, c["k"])
        ents = np.zeros((N, W["D"]))
        ents[sel] = OF.decode_rows(kv[off + sel], csa.SPLIT, W["D"], W["R"])
        wl = int(inp.win_len[b])
        win = OF.decode_rows(inp.win[b, :wl], csa.BF16, W["D"])
        q = OF.decode_rows(inp.q[b], csa.BF16, W["D"])
        OM.decode_one(q, int(inp.q_pos[b]), ents, win, inp.sinks.astype(np.float64), inp.scale,
                      W["m"], idx=sel, R=W["R"])
        done += 1
    return done, time.perf_counter() - t0


def cpu_baseline(W, budget_s=12.0):
    """The oracle timed on the host: with every BLAS thread the process has
    (the reported value), and limited to one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = 1
    done, dt = _oracle_sample(W, budget_s)
    res = {"value": done / dt, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} decode queries (indexer over 16384 FP8 keys, top-512, sink MQA over "
                     f"512+128 entries) of the same batch in {dt:.1f} s",
           "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(), "host_physical_cores": _physical_cores()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, t1 = _oracle_sample(W, budget_s / 2)
        res["one_thread"] = {"value": d1 / t1, "unit": "query-tokens/s", "cores": 1,
                             "sample": f"{d1} decode queries in {t1:.1f} s"}
    return res


def traffic_record(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (null otherwise)."""
    from compressed_sparse_long_csa_amd.profiling import sources_sha256
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        srcs = rec["source"] if isinstance(rec["source"], list) else [rec["source"]]
        h = sources_sha256([os.path.join(ROOT, p) for p in srcs])
        return rec["bytes_per_launch"] if rec.get("source_sha256") == h else None
    except Exception:
        return None


def context_scan(contexts, steps, warmup):
    """The same decode step (B = 16) at longer contexts, the state replicated
    as for the headline line so that every step reads HBM.  Per context: ms
    per step, query-tokens/s, each kernel's device time and the indexer's HBM
    fraction."""
    rows = []
    for L in contexts:
        W = build_device_workload(L)
        step_bytes, kbytes = algorithmic_bytes(W)
        # copies of the state so that the bytes one pass over them reads exceed
        # twice the 256 MB last-level cache
        n_rep = max(1, -(-600_000_000 // step_bytes))
        reps = make_replicas(W, n_rep)
        made3 = [make_step(Wr, check=False) for Wr in reps]
        made = [make_step(Wr, check=False, topk_fused=True) for Wr in reps]
        for st, _ in made + made3:
            st()
        torch.cuda.synchronize()
        ms = time_graph([m[0] for m in made], steps, warmup)
        ms3 = time_graph([m[0] for m in made3], steps, warmup)
        per_us = kernel_periods([m[1] for m in made], max(20, min(60, steps)))
        per_us3 = kernel_periods([m[1] for m in made3], max(20, min(60, steps)))
        idx_gbps = kbytes["indexer_inputs"] / (per_us3["csa_compress_score"] * 1e-6) / 1e9
        best = min(ms, ms3)
        rows.append({"context": L, "ms_per_step": best, "query_tokens_per_s": W["B"] / (best * 1e-3),
                     "form": "two launches (top-k fused)" if ms <= ms3 else "three launches",
                     "step_hbm_gbps_algorithmic": step_bytes / (best * 1e-3) / 1e9,
                     "two_launches": {"ms_per_step": ms, "kernels_us": {n: round(v, 2) for n, v in per_us.items()}},
                     "three_launches": {"ms_per_step": ms3,
                                        "kernels_us": {n: round(v, 2) for n, v in per_us3.items()}},
                     "compress_score_gbps": idx_gbps, "compress_score_hbm_frac": idx_gbps / HBM_PEAK_GBPS,
                     "state_replicas": n_rep})
        del W, reps, made, made3
        torch.cuda.empty_cache()
    return rows


HCA = "hca_decode_b32_ctx262144"


PAGED_BLOCK_ROWS = 32          # one 128-token block of CSA entries


def paged_replica(Wr, seed):
    """The replica's KV cache and index keys moved into pools of shuffled
    32-entry blocks (a block table per sequence), and the step's new entry
    rows mapped to their pool rows."""
    inp, BR = Wr["inp"], PAGED_BLOCK_ROWS
    n_ent = np.asarray(inp.n_ent, np.int64)
    off = np.asarray(inp.kv_off, np.int64)
    nb = (n_ent + BR - 1) // BR
    bps = int(nb.max())
    total = int(nb.sum())
    perm = np.random.default_rng(seed).permutation(total).astype(np.int64)
    table = np.zeros((Wr["B"], bps), np.int32)
    src_rows, dst_rows = [], []
    j0 = 0
    for i in range(Wr["B"]):
        for j in range(int(nb[i])):
            phys = int(perm[j0 + j])
            table[i, j] = phys
            cnt = min(BR, int(n_ent[i]) - j * BR)
            src_rows.append(np.arange(cnt) + off[i] + j * BR)
            dst_rows.append(np.arange(cnt) + phys * BR)
        j0 += int(nb[i])
    src = torch.from_numpy(np.concatenate(src_rows)).cuda()
    dst = torch.from_numpy(np.concatenate(dst_rows)).cuda()
    Wp = dict(Wr)
    for name, rb in (("kv", Wr["kv"].shape[-1]), ("keys", Wr["keys"].shape[-1])):
        flat = Wr[name].reshape(-1, rb)
        pool = torch.zeros((total * BR, rb), dtype=flat.dtype, device="cuda")
        pool[dst] = flat[src]
        Wp[name] = pool
    last = n_ent - 1
    Wp["seg_row"] = torch.from_numpy(table[np.arange(Wr["B"]), last // BR].astype(np.int64) * BR
                                     + last % BR).cuda()
    # the window as each request's ring (random start); the newest row goes
    # to its ring slot
    n_win = inp.n_win
    wl = np.asarray(inp.win_len, np.int64)
    start = np.random.default_rng(seed + 1).integers(0, n_win, size=Wr["B"]).astype(np.int64)
    slots = (start[:, None] + np.arange(n_win)[None, :]) % n_win             # ring slot of window row t
    ring = torch.empty_like(Wr["win"])
    ring[torch.arange(Wr["B"]).cuda()[:, None], torch.from_numpy(slots).cuda()] = Wr["win"]
    Wp["win"] = ring
    Wp["win_start"] = torch.from_numpy(start.astype(np.int32)).cuda()
    Wp["win_row"] = torch.from_numpy(np.arange(Wr["B"]) * n_win + (start + wl - 1) % n_win).cuda()
    Wp["table"] = torch.from_numpy(table).cuda()
    Wp["bps"], Wp["pool_rows"] = bps, total * BR
    return Wp


def make_paged_step(Wp, fused=True, topk_fused=False):
    """The decode step over paged caches: csa_compress_score_paged (the new
    rows go to their pool rows and window ring slots; or, fused=False,
    csa_compress_batch then indexer_score_paged), topk_select,
    hybrid_attn_decode_paged."""
    c, inp = Wp["c"], Wp["inp"]
    B, m, D, R, d_I, H, k = Wp["B"], Wp["m"], Wp["D"], Wp["R"], Wp["d_I"], c["H"], c["k"]
    _, kern = make_step(Wp, check=False, fused=False)
    k_compress, k_topk = kern[0][1], kern[2][1]
    BR = PAGED_BLOCK_ROWS
    jobs = step_jobs(Wp)

    def k_indexer():
        csa.indexer_score_paged(Wp["q_idx"], Wp["w"], B, c["H_I"], d_I, Wp["keys"], csa.FP8, Wp["pool_rows"],
                                Wp["table"], Wp["bps"], BR, Wp["q_pos"], m, Wp["scores"], Wp["ld"], check=False)

    def k_compress_score():
        csa.csa_compress_score_paged(jobs, Wp["q_idx"], Wp["w"], B, c["H_I"], d_I, Wp["keys"], csa.FP8,
                                     Wp["pool_rows"], Wp["table"], B, Wp["bps"], BR, None, Wp["q_pos"], m,
                                     Wp["scores"], Wp["ld"], check=False)

    def k_attn():
        csa.hybrid_attn_decode_paged(Wp["q"], csa.BF16, B, H, D, Wp["q_pos"], None, EPS, R, BASE, Wp["kv"],
                                     csa.SPLIT, Wp["pool_rows"], Wp["table"], Wp["bps"], BR, m, Wp["idx"], k,
                                     Wp["win"], csa.BF16, inp.n_win, Wp["win_len"], Wp["sinks"], inp.scale,
                                     Wp["out"], csa.BF16, csa.VARIANT_AUTO, check=False, win_start=Wp["win_start"])
    if topk_fused and "tk_ws" not in Wp:
        Wp["tk_ws"] = torch.zeros(csa.score_topk_workspace_bytes(B), dtype=torch.uint8, device="cuda")

    def k_compress_score_topk():
        csa.csa_compress_score_topk_paged(jobs, Wp["q_idx"], Wp["w"], B, c["H_I"], d_I, Wp["keys"], csa.FP8,
                                          Wp["pool_rows"], Wp["table"], B, Wp["bps"], BR, None, Wp["q_pos"], m,
                                          Wp["scores"], Wp["ld"], k, Wp["idx"], workspace=Wp["tk_ws"], check=False)
    if fused and topk_fused:
        kernels = [("csa_compress_score_topk_paged", k_compress_score_topk), ("hybrid_attn_decode_paged", k_attn)]
    elif fused:
        kernels = [("csa_compress_score_paged", k_compress_score), ("topk_select", k_topk),
                   ("hybrid_attn_decode_paged", k_attn)]
    else:
        kernels = [("csa_compress_batch", k_compress), ("indexer_score_paged", k_indexer), ("topk_select", k_topk),
                   ("hybrid_attn_decode_paged", k_attn)]

    def step():
        for _, f in kernels:
            f()
    return step, kernels


def paged_leg(reps, steps, warmup):
    """The headline step with its KV cache and index keys paged in 32-entry
    blocks and its window kept as a ring: ms per step and each kernel's
    time, as three launches (compress + score in one) and as four."""
    pr = [paged_replica(Wr, 100 + j) for j, Wr in enumerate(reps)]
    made = [make_paged_step(Wp) for Wp in pr]
    made3 = [make_paged_step(Wp, topk_fused=True) for Wp in pr]
    made4 = [make_paged_step(Wp, fused=False) for Wp in pr]
    for st, _ in made + made3 + made4:
        st()
    torch.cuda.synchronize()
    ms = time_graph([m_[0] for m_ in made], steps, warmup)
    ms3 = time_graph([m_[0] for m_ in made3], steps, warmup)
    ms4 = time_graph([m_[0] for m_ in made4], steps, warmup)
    us = kernel_periods([m_[1] for m_ in made], max(20, min(100, steps)))
    us3 = kernel_periods([m_[1] for m_ in made3], max(20, min(100, steps)))
    us4 = kernel_periods([m_[1] for m_ in made4], max(20, min(100, steps)))
    out = {"block_rows": PAGED_BLOCK_ROWS, "window": "ring", "ms_per_step": ms, "query_tokens_per_s": pr[0]["B"] / (ms * 1e-3),
           "kernels_us": {n: round(v, 2) for n, v in us.items()},
           "two_launches_topk_fused": {"ms_per_step": ms3, "kernels_us": {n: round(v, 2) for n, v in us3.items()}},
           "four_launches": {"ms_per_step": ms4, "kernels_us": {n: round(v, 2) for n, v in us4.items()}}}
    del pr, made, made3, made4
    torch.cuda.empty_cache()
    return out


def hca_leg(steps, warmup):
    """The HCA decode workload: 32 sequences of 262,144 tokens, m' = 128, so
    2,048 compressed entries per sequence, every one attended (no indexer, no
    top-k), plus the 128-token window.  One step = csa_compress_batch (the
    newest 128-token block's entry and the new token's window row) +
    hybrid_attn_decode.  The state is replicated so that a pass over the
    copies reads more than 600 MB, and the copies' steps are captured in one
    graph, as for the CSA line.  Reports ms per step, query-tokens/s and the
    attention's algorithmic HBM rate and MFMA rate."""
    c = synth.WORKLOADS[HCA]
    B, L, m, H, D, R, n_win = c["B"], c["L"], c["m"], c["H"], c["D"], c["R"], c["n_win"]
    d = synth.device_decode_inputs(c["seed"] + 3000, [L] * B, m=m, H=H, D=D, R=R, n_win=n_win, csa=False)
    gen = synth.device_generator(c["seed"] + 3001)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)  # noqa: E731
    n_ent, kv_off_h, q_pos_h = d["n_ent"], d["kv_off"], d["q_pos"]
    win_len_h = d["win_len"]
    tc = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int64), device="cuda")  # noqa: E731
    kv_tok, kv_gate = rnd(B * m, D).to(torch.bfloat16), rnd(B * m, 1)
    win_tok, win_gate = rnd(B, D).to(torch.bfloat16), torch.zeros((B, 1), device="cuda")
    seg_off, seg_pos0, seg_row = tc(np.arange(B + 1) * m), tc((n_ent - 1) * m), tc(kv_off_h + n_ent - 1)
    wseg_off, wpos0 = tc(np.arange(B + 1)), tc(q_pos_h)
    wrow = tc(np.arange(B) * n_win + win_len_h.astype(np.int64) - 1)
    q_pos, kv_off = tc(q_pos_h), tc(kv_off_h)
    win_len = torch.as_tensor(win_len_h, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    state_bytes = d["kv"].numel() + d["win"].numel()
    n_rep = max(1, -(-600_000_000 // state_bytes))
    states = [(d["kv"], d["win"])] + [(d["kv"].clone(), d["win"].clone()) for _ in range(n_rep - 1)]

    def make(kv, win):
        def job(x, gate, mm, off, pos0, rows, dst, fmt):
            return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=B * mm, D=D, m=mm, nseg=B,
                        seg_tok_off=off, seg_pos0=pos0, seg_out_row=rows, normalize=1, norm_w=None, eps=EPS,
                        rope_dim=R, rope_base=BASE, out=dst, out_fmt=fmt)
        jobs = [job(kv_tok, kv_gate, m, seg_off, seg_pos0, seg_row, kv, csa.SPLIT),
                job(win_tok, win_gate, 1, wseg_off, wpos0, wrow, win, csa.BF16)]
        kernels = [("csa_compress_batch", lambda: csa.csa_compress_batch(jobs, check=False)),
                   ("hybrid_attn_decode", lambda: csa.hybrid_attn_decode(
                       d["q"], csa.BF16, B, H, D, q_pos, None, EPS, R, BASE, kv, csa.SPLIT, kv_off, m, None, 0,
                       win, csa.BF16, n_win, win_len, d["sinks"], d["scale"], out, csa.BF16, csa.VARIANT_AUTO,
                       check=False))]

        def step():
            for _, f in kernels:
                f()
        return step, kernels
    made = [make(kv, win) for kv, win in states]
    for st, _ in made:
        st()
    torch.cuda.synchronize()
    ms = time_graph([m_[0] for m_ in made], steps, warmup)
    per_us = kernel_periods([m_[1] for m_ in made], max(20, min(60, steps)))
    # the attention over a paged copy of the first state (one entry per
    # block: the pages' one HCA entry per 128-token block, blocks shuffled)
    # against the same contiguous state, both on that one copy
    kv0 = states[0][0].view(-1, states[0][0].shape[-1])
    n_rows = kv0.shape[0]
    perm = torch.randperm(n_rows, generator=torch.Generator().manual_seed(c["seed"] + 3002))
    pool = torch.empty_like(kv0)
    pool[perm.cuda()] = kv0
    table = torch.empty((B, int(n_ent.max())), dtype=torch.int32)
    for b in range(B):
        table[b, : int(n_ent[b])] = perm[int(kv_off_h[b]): int(kv_off_h[b]) + int(n_ent[b])].to(torch.int32)
    table = table.cuda()
    one = [[("contiguous", made[0][1][1][1]),
            ("paged", lambda: csa.hybrid_attn_decode_paged(
                d["q"], csa.BF16, B, H, D, q_pos, None, EPS, R, BASE, pool, csa.SPLIT, n_rows, table,
                table.shape[1], 1, m, None, 0, states[0][1], csa.BF16, n_win, win_len, d["sinks"], d["scale"], out,
                csa.BF16, csa.VARIANT_AUTO, check=False))]]
    one_us = kernel_periods(one, max(20, min(60, steps)))
    split = (D - R) + 2 * R
    attended = n_ent.astype(np.int64) + win_len_h.astype(np.int64)
    a_bytes = int(n_ent.sum()) * split + int(win_len_h.sum()) * 2 * D + B * H * D * 2 * 2 + H * 4
    a_flops = 4.0 * attended.sum() * H * D
    t = per_us["hybrid_attn_decode"] * 1e-6
    res = {"workload": HCA, "ms_per_step": ms, "query_tokens_per_s": B / (ms * 1e-3),
           "kernels_us": {n: round(v, 2) for n, v in per_us.items()},
           "attn_bytes": a_bytes, "attn_gbps": a_bytes / t / 1e9, "attn_hbm_frac": a_bytes / t / 1e9 / HBM_PEAK_GBPS,
           "attn_tflops": a_flops / t / 1e12, "attn_mfma_frac": a_flops / t / 1e12 / BF16_PEAK_TFLOPS,
           "state_replicas": n_rep,
           "attn_us_one_copy": {"contiguous": round(one_us["contiguous"], 2), "paged_block_rows_1": round(one_us["paged"], 2)}}
    del states, made, d, pool, table
    torch.cuda.empty_cache()
    return res


RAGGED = "ragged_csa_hca_b64_ctx1k_1m"


def ragged_leg(steps, warmup):
    """The ragged workload: 64 sequences with lengths log-uniform in [1K, 1M]
    tokens (seeded), one CSA layer (m = 4, MXFP4 indexer 64 x 128, top-1,024)
    and one HCA layer (m' = 128, every entry) per step.  CSA layer =
    csa_compress_batch (KV entry, MXFP4 key, window row) + indexer_score +
    topk_select + hybrid_attn_decode; HCA layer = csa_compress_batch (KV entry,
    window row) + hybrid_attn_decode; both captured in one graph.  The CSA
    state alone exceeds 600 MB, so it is not replicated.  Reports ms per step
    (both layers), query-tokens/s and each kernel's time, and the MXFP4
    indexer's algorithmic HBM rate."""
    c = synth.WORKLOADS[RAGGED]
    B, m, mh, H, D, R, n_win, k = c["B"], c["m"], c["m_hca"], c["H"], c["D"], c["R"], c["n_win"], c["k"]
    H_I, d_I = c["H_I"], c["d_I"]
    lengths = synth.log_uniform_lengths(synth.rng_for(c["seed"]), B, c["Lmin"], c["Lmax"])
    dc = synth.device_decode_inputs(c["seed"] + 4000, lengths, m=m, H=H, D=D, R=R, n_win=n_win, csa=True,
                                    k=k, idx_fmt=csa.MXFP4, H_I=H_I, d_I=d_I)
    dh = synth.device_decode_inputs(c["seed"] + 4001, lengths, m=mh, H=H, D=D, R=R, n_win=n_win, csa=False)
    gen = synth.device_generator(c["seed"] + 4002)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)  # noqa: E731
    tc = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int64), device="cuda")  # noqa: E731

    def layer(d, mm, with_index):
        n_ent, kv_off, q_pos, win_len = d["n_ent"], d["kv_off"], d["q_pos"], d["win_len"]
        st = dict(kv_tok=rnd(B * mm, D).to(torch.bfloat16), kv_gate=rnd(B * mm, 1),
                  key_tok=rnd(B * mm, d_I).to(torch.bfloat16), key_gate=rnd(B * mm, 1),
                  win_tok=rnd(B, D).to(torch.bfloat16), win_gate=torch.zeros((B, 1), device="cuda"),
                  seg_off=tc(np.arange(B + 1) * mm), seg_pos0=tc((n_ent - 1) * mm), seg_row=tc(kv_off + n_ent - 1),
                  wseg_off=tc(np.arange(B + 1)), wpos0=tc(q_pos), wrow=tc(np.arange(B) * n_win + win_len - 1),
                  q_pos=tc(q_pos), kv_off=tc(kv_off), n_valid=tc(n_ent), win_len=torch.as_tensor(win_len, device="cuda"))

        def job(x, gate, DD, m_, off, pos0, rows, normalize, R_, dst, fmt):
            return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=B * m_, D=DD, m=m_, nseg=B,
                        seg_tok_off=off, seg_pos0=pos0, seg_out_row=rows, normalize=normalize, norm_w=None,
                        eps=EPS, rope_dim=R_, rope_base=BASE, out=dst, out_fmt=fmt)
        jobs = [job(st["kv_tok"], st["kv_gate"], D, mm, st["seg_off"], st["seg_pos0"], st["seg_row"], 1, R,
                    d["kv"], csa.SPLIT),
                job(st["win_tok"], st["win_gate"], D, 1, st["wseg_off"], st["wpos0"], st["wrow"], 1, R,
                    d["win"], csa.BF16)]
        ld = int(n_ent.max())
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        kern = []
        if with_index:
            jobs.insert(1, job(st["key_tok"], st["key_gate"], d_I, mm, st["seg_off"], st["seg_pos0"], st["seg_row"],
                               0, 0, d["keys"], csa.MXFP4))
            scores = torch.empty((B, ld), dtype=torch.float32, device="cuda")
            idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
            kern = [("indexer_score", lambda: csa.indexer_score(d["q_idx"], d["w"], B, H_I, d_I, d["keys"], csa.MXFP4,
                                                                 st["kv_off"], st["q_pos"], mm, scores, ld, check=False)),
                    ("topk_select", lambda: csa.topk_select(scores, ld, B, st["n_valid"], k, idx, None, check=False))]
        else:
            idx = None
        pre = "csa" if with_index else "hca"
        kern = ([(pre + "_compress_batch", lambda: csa.csa_compress_batch(jobs, check=False))] + kern +
                [(pre + "_attn_decode", lambda: csa.hybrid_attn_decode(
                    d["q"], csa.BF16, B, H, D, st["q_pos"], None, EPS, R, BASE, d["kv"], csa.SPLIT, st["kv_off"], mm,
                    idx, k if with_index else 0, d["win"], csa.BF16, n_win, st["win_len"], d["sinks"], d["scale"],
                    out, csa.BF16, csa.VARIANT_AUTO, check=False))])
        return kern
    kern = layer(dc, m, True) + layer(dh, mh, False)

    def step():
        for _, f in kern:
            f()
    step()
    torch.cuda.synchronize()
    ms = time_graph([step], steps, warmup)
    per_us = kernel_periods([kern], max(20, min(60, steps)))
    n_ent = dc["n_ent"].astype(np.int64)
    idx_bytes = int(n_ent.sum()) * (68 + 4) + B * H_I * (68 + 4)
    res = {"workload": RAGGED, "lengths_min_median_max": [int(lengths.min()), int(np.median(lengths)),
                                                          int(lengths.max())],
           "ms_per_step": ms, "query_tokens_per_s": B / (ms * 1e-3),
           "kernels_us": {n: round(v, 2) for n, v in per_us.items()},
           "mxfp4_indexer_gbps": idx_bytes / (per_us["indexer_score"] * 1e-6) / 1e9,
           "mxfp4_indexer_hbm_frac": idx_bytes / (per_us["indexer_score"] * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    del dc, dh, kern
    torch.cuda.empty_cache()
    return res


PREFILL = "csa_prefill_ctx131072_chunk2048"


def fp32_leg(steps, warmup):
    """The all-float32 CSA decode step of one 2,048-token sequence (D = 128,
    8 heads, indexer 4 x 64, top-64, window 128): indexer, top-k and attention,
    captured in a HIP graph.  A latency workload: its time, no roofline."""
    name = "csa_decode_fp32_b1_ctx2048"
    c = synth.WORKLOADS[name]
    inp = synth.workload_decode_inputs(name, seed=c["seed"])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q, q_pos, kv, kv_off = dev(inp.q), dev(inp.q_pos), dev(inp.kv), dev(inp.kv_off)
    win, win_len, sinks = dev(inp.win), dev(inp.win_len), dev(inp.sinks)
    keys, q_idx, w = dev(inp.keys), dev(inp.q_idx), dev(inp.w)
    B, H, D, R, k = inp.B, inp.H, inp.D, inp.R, inp.k
    ld = int(inp.n_ent.max())
    n_valid = dev(np.asarray(inp.n_ent, np.int64))
    scores = torch.empty((B, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")

    def k_indexer():
        csa.indexer_score(q_idx, w, B, inp.H_I, inp.d_I, keys, csa.F32, kv_off, q_pos, inp.m, scores, ld,
                          check=False)

    def k_topk():
        csa.topk_select(scores, ld, B, n_valid, k, idx, None, check=False)

    def k_attn():
        csa.hybrid_attn_decode(q, csa.F32, B, H, D, q_pos, None, EPS, R, BASE, kv, csa.F32, kv_off, inp.m, idx, k,
                               win, csa.F32, inp.n_win, win_len, sinks, inp.scale, out, csa.F32,
                               csa.VARIANT_AUTO, check=False)
    kernels = [("indexer_score", k_indexer), ("topk_select", k_topk), ("hybrid_attn_decode", k_attn)]

    def step():
        for _, f in kernels:
            f()
    ms = time_graph([step], steps, warmup)
    us = kernel_periods([kernels], max(20, min(100, steps)))
    return {"workload": name, "ms_per_step": ms, "query_tokens_per_s": B / (ms * 1e-3),
            "kernels_us": {n: round(v, 2) for n, v in us.items()}, "graph": True}


def cp_leg(reps=20, S=8, L=1048576, m=4):
    """Context-parallel reassembly of one CSA layer's compressed cache: a
    1,048,576-token sequence cut into S shards, each shard's fixed-length run
    of compressed entries (576-byte rows, one padding row) joined by
    csa_select_and_pad into one run with the padding at the end.  Bytes: the
    valid rows read once, every output row written once.  Two copies of the
    runs alternate so the gather reads HBM."""
    rb = 576
    n_all = L // m
    cuts = np.linspace(0, L, S + 1).astype(np.int64)
    cuts[1:-1] += np.random.default_rng(8).integers(-1000, 1000, size=S - 1)   # cuts off block boundaries
    n_valid = [int(cuts[s + 1] // m - cuts[s] // m) if s + 1 < S else int(n_all - cuts[s] // m) for s in range(S)]
    cap = max(n_valid) + 1
    runs = [torch.randint(0, 256, (S * cap * rb,), dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty(S * cap * rb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    nv = torch.tensor(n_valid, dtype=torch.int64, device="cuda")
    fs = [lambda i=i: csa.csa_select_and_pad(runs[i], S, cap, rb, nv, outs[i], check=False) for i in range(2)]
    for f in fs:
        f()
    torch.cuda.synchronize()
    us = _batch_period(fs, reps)
    nbytes = sum(n_valid) * rb + S * cap * rb
    return {"workload": f"cp_reassembly_ctx{L}_{S}shards", "shards": S, "rows_per_shard": cap,
            "valid_rows": sum(n_valid), "us": us, "bytes": nbytes, "gbps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}


def prefill_leg(reps=10):
    """The CSA prefill workload: a chunk of 2,048 tokens after 131,072 cached,
    on inputs drawn on the device (seeded).  One pass = csa_compress_batch
    (the chunk's 512 KV entries, 512 index keys and 2,048 per-token window
    rows) + indexer_score (2,048 x 33,280 scores) + topk_select (k = 1,024)
    + hybrid_attn_prefill.  Reports each kernel's device time (events around
    single launches, less an empty pair), the pass time, and the two
    contractions' matrix FLOP rates against the BF16 MFMA peak.  Parity of
    this path is covered by the GPU tests, not re-checked here."""
    c = synth.WORKLOADS[PREFILL]
    cached, chunk, H, m, k = c["cached"], c["chunk"], c["H"], c["m"], c["k"]
    D, R, d_I, H_I, n_win = c["D"], c["R"], c["d_I"], c["H_I"], c["n_win"]
    gen = synth.device_generator(c["seed"] + 2000)
    cuda = "cuda"
    T = cached + chunk
    n_tot = T // m
    kv = synth.device_rows(gen, n_tot, D, csa.SPLIT, R)
    keys = synth.device_rows(gen, n_tot, d_I, csa.FP8)
    tok_pos0 = cached - n_win + 1
    tok = synth.device_rows(gen, T - tok_pos0, D, csa.BF16)
    q = synth.device_rows(gen, chunk * H, D, csa.BF16).reshape(chunk, H, -1)
    q_idx = synth.device_rows(gen, chunk * H_I, d_I, csa.FP8).reshape(chunk, H_I, -1)
    w = torch.rand((chunk, H_I), generator=gen, device=cuda, dtype=torch.float32)
    sinks = torch.randn(H, generator=gen, device=cuda, dtype=torch.float32)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=cuda, dtype=torch.float32)  # noqa: E731
    kv_tok, kv_gate = rnd(chunk, D).to(torch.bfloat16), rnd(chunk, 1)
    key_tok, key_gate = rnd(chunk, d_I).to(torch.bfloat16), rnd(chunk, 1)
    q_pos_h = (cached + np.arange(chunk)).astype(np.int64)
    n_ent_h = (q_pos_h + 1) // m
    q_pos = torch.as_tensor(q_pos_h, device=cuda)
    n_valid = torch.as_tensor(n_ent_h, device=cuda)
    zeros = torch.zeros(chunk, dtype=torch.int64, device=cuda)
    tp0 = torch.full((chunk,), tok_pos0, dtype=torch.int64, device=cuda)
    seg = torch.tensor([0, chunk], dtype=torch.int64, device=cuda)
    pos0 = torch.tensor([cached], dtype=torch.int64, device=cuda)
    scores = torch.empty((chunk, n_tot), dtype=torch.float32, device=cuda)
    idx = torch.empty((chunk, k), dtype=torch.int32, device=cuda)
    out = torch.empty((chunk, H, D), dtype=torch.bfloat16, device=cuda)

    def job(x, gate, DD, mm, row0, normalize, R_, dst, fmt):
        return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=chunk, D=DD, m=mm, nseg=1,
                    seg_tok_off=seg, seg_pos0=pos0, seg_out_row=torch.tensor([row0], dtype=torch.int64, device=cuda),
                    normalize=normalize, norm_w=None, eps=EPS, rope_dim=R_, rope_base=BASE, out=dst, out_fmt=fmt)
    jobs = [job(kv_tok, kv_gate, D, m, cached // m, 1, R, kv, csa.SPLIT),
            job(key_tok, key_gate, d_I, m, cached // m, 0, 0, keys, csa.FP8),
            job(kv_tok, torch.zeros((chunk, 1), device=cuda), D, 1, cached - tok_pos0, 1, R, tok, csa.BF16)]
    kernels = [
        ("csa_compress_batch", lambda: csa.csa_compress_batch(jobs, check=False)),
        ("indexer_score", lambda: csa.indexer_score(q_idx, w, chunk, H_I, d_I, keys, csa.FP8, zeros, q_pos, m,
                                                    scores, n_tot, check=False)),
        ("topk_select", lambda: csa.topk_select(scores, n_tot, chunk, n_valid, k, idx, None, check=False)),
        ("hybrid_attn_prefill", lambda: csa.hybrid_attn_prefill(
            q, csa.BF16, chunk, H, D, q_pos, None, EPS, R, BASE, kv, csa.SPLIT, zeros, m, idx, k, tok, csa.BF16,
            zeros, tp0, n_win, sinks, 1.0 / np.sqrt(D), out, csa.BF16, check=False)),
    ]
    for _, f in kernels:
        f()
    torch.cuda.synchronize()
    us = {n: _batch_period([f], reps) for n, f in kernels}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for _, f in kernels:
            f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    attended = np.minimum(k, n_ent_h) + np.minimum(n_win, q_pos_h - tok_pos0 + 1)
    f_idx = 2.0 * n_ent_h.sum() * H_I * d_I
    f_attn = 4.0 * attended.sum() * H * D
    tflops = lambda f, t: f / (t * 1e-6) / 1e12  # noqa: E731
    topk_bytes = int(n_ent_h.sum()) * 4 + chunk * k * 4
    res = {"workload": PREFILL, "ms_per_chunk": ms, "tokens_per_s": chunk / (ms * 1e-3),
           "kernels_us": {n: round(v, 1) for n, v in us.items()},
           "indexer_tflops": tflops(f_idx, us["indexer_score"]),
           # an FP8 contraction (run on BF16 MFMA over exactly widened codes)
           "indexer_frac_of_fp8_peak": tflops(f_idx, us["indexer_score"]) / FP8_PEAK_TFLOPS,
           "indexer_frac_of_bf16_peak": tflops(f_idx, us["indexer_score"]) / BF16_PEAK_TFLOPS,
           "attn_tflops": tflops(f_attn, us["hybrid_attn_prefill"]),
           "attn_mfma_frac": tflops(f_attn, us["hybrid_attn_prefill"]) / BF16_PEAK_TFLOPS,
           "topk_gbps": topk_bytes / (us["topk_select"] * 1e-6) / 1e9}
    # the same chunk over paged caches: entries and index keys in shuffled
    # 32-entry blocks (one 128-token block each) of two pools, one block-table
    # row that every query of the chunk names
    br = 32
    n_blk = (n_tot + br - 1) // br
    total = n_blk + 8
    perm = torch.randperm(total, generator=gen, device=cuda)[:n_blk]
    def paged(rows):
        rb = rows.shape[-1]
        pool = torch.zeros((total * br, rb), dtype=torch.uint8, device=cuda)
        padded = torch.zeros((n_blk * br, rb), dtype=torch.uint8, device=cuda)
        padded[:n_tot] = rows.view(n_tot, rb)
        pool.view(total, br, rb)[perm] = padded.view(n_blk, br, rb)
        return pool
    kv_pool, key_pool = paged(kv.view(n_tot, -1)), paged(keys.view(n_tot, -1))
    table = perm.to(torch.int32).reshape(1, n_blk).contiguous()
    q_row = torch.zeros(chunk, dtype=torch.int32, device=cuda)
    pk = [("indexer_score_paged_rows", lambda: csa.indexer_score_paged_rows(
              q_idx, w, chunk, H_I, d_I, key_pool, csa.FP8, total * br, table, 1, n_blk, br, q_row, q_pos, m,
              scores, n_tot, check=False)),
          ("hybrid_attn_prefill_paged", lambda: csa.hybrid_attn_prefill_paged(
              q, csa.BF16, chunk, H, D, q_pos, None, EPS, R, BASE, kv_pool, csa.SPLIT, total * br, table, 1, n_blk,
              br, q_row, m, idx, k, tok, csa.BF16, zeros, tp0, n_win, sinks, 1.0 / np.sqrt(D), out, csa.BF16,
              check=False))]
    kernels[1][1]()
    kernels[3][1]()
    ref_scores, ref_out = scores.clone(), out.clone()
    for _, f in pk:
        f()
    torch.cuda.synchronize()
    same = bool(torch.equal(ref_scores.view(torch.int32), scores.view(torch.int32)) and torch.equal(ref_out, out))
    del ref_scores, ref_out
    res["paged"] = {"block_rows": br, "kernels_us": {n: round(_batch_period([f], reps), 1) for n, f in pk},
                    "bits_equal_contiguous": same}
    del kv, keys, tok, scores, q, q_idx, kv_pool, key_pool
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--replicas", type=int, default=13,
                    help="per-layer state copies stepped in turn (1 = one warm cache)")
    ap.add_argument("--no-context-scan", action="store_true",
                    help="skip the same step at 256K and 1M contexts")
    ap.add_argument("--no-hca", action="store_true",
                    help="skip the HCA decode step (32 sequences of 262,144 tokens)")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged CSA (MXFP4) + HCA step (64 sequences, 1K to 1M tokens)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the headline step over paged caches (32-entry blocks)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the CSA prefill chunk (2,048 tokens after 131,072)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the CSA prefill chunk and print its object (for profiling)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (decode would "
              "shard by sequence, each GPU stepping its own sequences). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, max(1, args.steps))
        return
    if args.prefill_only:
        csa.load_library()
        print(json.dumps({"prefill": prefill_leg()}), flush=True)
        return
    csa.load_library()
    W = build_workload()
    step, _ = make_step(W, check=True)
    step()                                   # validated eager pass
    torch.cuda.synchronize()
    reps = make_replicas(W, max(1, args.replicas))
    made = [make_step(Wr, check=False) for Wr in reps]
    ms_warm = time_graph([made[0][0]], args.steps, args.warmup)
    ms, spread = time_graph([m[0] for m in made], args.steps, args.warmup, spread=200)
    ms_eager = time_eager([m[0] for m in made], min(args.steps, 300), min(args.warmup, 30))
    batch_us = {}
    event_us, event_floor_us = time_kernels([m[1] for m in made], max(20, min(100, args.steps)), batch_us)
    per_us = batch_us
    # the same step as two launches (the top-k selected inside the compress +
    # score launch) and as four (compress, then the indexer), for comparison
    made3 = [make_step(Wr, check=False, fused=True, topk_fused=True) for Wr in reps]
    ms3 = time_graph([m[0] for m in made3], args.steps, args.warmup)
    per_us3 = kernel_periods([m[1] for m in made3], max(20, min(100, args.steps)))
    made4 = [make_step(Wr, check=False, fused=False) for Wr in reps]
    ms4 = time_graph([m[0] for m in made4], args.steps, args.warmup)
    per_us4 = kernel_periods([m[1] for m in made4], max(20, min(100, args.steps)))
    made[0][0]()                             # replica 0 last, for the spot check
    torch.cuda.synchronize()
    step_bytes, kbytes = algorithmic_bytes(W)
    err = spot_check(W)
    B = W["B"]
    dom = "csa_compress_score"               # the launch that moves most of the step's bytes
    flops = algorithmic_flops(W)

    def table(us):
        kern = {}
        for n in us:
            t = us[n] * 1e-6
            kern[n] = {"us": us[n], "bytes": kbytes[n], "gbps": kbytes[n] / t / 1e9,
                       "hbm_frac": kbytes[n] / t / 1e9 / HBM_PEAK_GBPS}
            if n in flops:
                kern[n].update({"tflops": flops[n] / t / 1e12,
                                "mfma_frac": flops[n] / t / 1e12 / BF16_PEAK_TFLOPS})
        return kern
    kern = table(per_us)
    for n in kern:
        kern[n]["us_events_less_floor"] = event_us[n]
    ach = kbytes["indexer_inputs"] / (per_us[dom] * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": B / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8/bf16 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) before quantisation; no weights needed)",
        "config": {"workload": "csa_decode_b16_ctx65536", "batch": B, "context": 65536,
                   "entries_per_seq": int(W["inp"].n_ent[0]), "top_k": W["c"]["k"],
                   "heads": W["c"]["H"], "head_dim": W["D"], "indexer": "fp8 64x128",
                   "window": 128, "graph": True, "steps_per_graph": len(reps), "variant": "auto",
                   "state_replicas": len(reps)},
        "ms_per_step_spread": spread,
        "ms_per_step_no_graph": ms_eager,
        "value_one_warm_cache": B / (ms_warm * 1e-3),
        "hbm_gbps_algorithmic": step_bytes / (ms * 1e-3) / 1e9,
        "step_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBPS, "traffic": traffic_record(dom),
                     "kernel": dom, "bytes_per_launch": kbytes["indexer_inputs"],
                     "bytes_per_launch_with_jobs_and_scores": kbytes[dom], "us_per_launch": per_us[dom],
                     "us_per_launch_events_less_floor": event_us[dom],
                     "timing": "mean period of back-to-back launches between two events (duration "
                               "plus dispatch gap)"},
        "hbm_frac_step": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernels": kern,
        "two_launches_topk_fused": {"ms_per_step": ms3, "query_tokens_per_s": B / (ms3 * 1e-3),
                                    "kernels": table(per_us3)},
        "four_launches": {"ms_per_step": ms4, "query_tokens_per_s": B / (ms4 * 1e-3),
                          "kernels": table(per_us4)},
        "event_pair_floor_us": event_floor_us,
        "copy_probe_gbps": copy_gbps(),
        "check_max_err_over_rms": err,
    }
    line["fp32_b1_ctx2048"] = fp32_leg(args.steps, args.warmup)
    if not args.no_paged:
        line["paged"] = paged_leg(reps, args.steps, args.warmup)
    if not args.no_context_scan:
        line["context_scan"] = context_scan([262144, 1048576], args.steps, args.warmup)
    if not args.no_hca:
        line["hca_decode"] = hca_leg(args.steps, args.warmup)
    if not args.no_ragged:
        line["ragged"] = ragged_leg(args.steps, args.warmup)
    if not args.no_prefill:
        line["prefill"] = prefill_leg()
    line["cp_select_and_pad"] = cp_leg()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

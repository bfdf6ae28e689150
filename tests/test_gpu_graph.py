"""The whole decode step -- csa_compress_batch (KV entry, indexer key, window
row), indexer_score, topk_select, hybrid_attn_decode, or the same step with
csa_compress_score in place of the first two -- captured in one HIP graph and
replayed: every replay, with eager work and synchronisation between replays,
gives the bits of the eager step.  Also the CSA prefill indexer (shared-key
kernel) and top-k captured together, and the decode step over paged caches."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


def _decode_step(lengths, seed, fused=False):
    m, H, D, R, k, n_win, d_I, H_I = 4, 64, 512, 64, 512, 128, 128, 64
    d = synth.device_decode_inputs(seed, lengths, m=m, H=H, D=D, R=R, n_win=n_win, csa=True, k=k,
                                   H_I=H_I, d_I=d_I)
    B = d["B"]
    gen = synth.device_generator(seed + 1)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32)  # noqa: E731
    tc = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int64), device=DEV)  # noqa: E731
    n_ent, kv_off, q_pos, win_len = d["n_ent"], d["kv_off"], d["q_pos"], d["win_len"]
    st = dict(
        kv_tok=rnd(B * m, D).to(torch.bfloat16), kv_gate=rnd(B * m, 1),
        key_tok=rnd(B * m, d_I).to(torch.bfloat16), key_gate=rnd(B * m, 1),
        win_tok=rnd(B, D).to(torch.bfloat16), win_gate=torch.zeros((B, 1), device=DEV),
        seg_off=tc(np.arange(B + 1) * m), seg_pos0=tc((n_ent - 1) * m), seg_row=tc(kv_off + n_ent - 1),
        wseg_off=tc(np.arange(B + 1)), wpos0=tc(q_pos), wrow=tc(np.arange(B) * n_win + win_len - 1),
        q_pos=tc(q_pos), kv_off=tc(kv_off), n_valid=tc(n_ent),
        win_len=torch.as_tensor(win_len, device=DEV))
    ld = int(n_ent.max())

    def job(x, gate, mm, off, pos0, rows, DD, normalize, R_, dst, fmt):
        return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=B * mm, D=DD, m=mm, nseg=B,
                    seg_tok_off=off, seg_pos0=pos0, seg_out_row=rows, normalize=normalize, norm_w=None,
                    eps=EPS, rope_dim=R_, rope_base=ROPE_BASE, out=dst, out_fmt=fmt)
    jobs = [job(st["kv_tok"], st["kv_gate"], m, st["seg_off"], st["seg_pos0"], st["seg_row"], D, 1, R,
                d["kv"], csa.SPLIT),
            job(st["key_tok"], st["key_gate"], m, st["seg_off"], st["seg_pos0"], st["seg_row"], d_I, 0, 0,
                d["keys"], csa.FP8),
            job(st["win_tok"], st["win_gate"], 1, st["wseg_off"], st["wpos0"], st["wrow"], D, 1, R,
                d["win"], csa.BF16)]

    def run(scores, idx, out, check):
        if fused:
            csa.csa_compress_score(jobs, d["q_idx"], d["w"], B, H_I, d_I, d["keys"], csa.FP8, st["kv_off"],
                                   st["q_pos"], m, scores, ld, check=check)
        else:
            csa.csa_compress_batch(jobs, check=check)
            csa.indexer_score(d["q_idx"], d["w"], B, H_I, d_I, d["keys"], csa.FP8, st["kv_off"], st["q_pos"],
                              m, scores, ld, check=check)
        csa.topk_select(scores, ld, B, st["n_valid"], k, idx, None, check=check)
        csa.hybrid_attn_decode(d["q"], csa.BF16, B, H, D, st["q_pos"], None, EPS, R, ROPE_BASE, d["kv"],
                               csa.SPLIT, st["kv_off"], m, idx, k, d["win"], csa.BF16, n_win, st["win_len"],
                               d["sinks"], d["scale"], out, csa.BF16, csa.VARIANT_AUTO, check=check)

    def bufs():
        return (torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV),
                torch.empty((B, k), dtype=torch.int32, device=DEV),
                torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV))
    return run, bufs


def _replay_matches(run, bufs):
    eager = bufs()
    run(*eager, True)                                  # also writes the step's cache rows
    torch.cuda.synchronize()
    cap = bufs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(*cap, False)                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*cap, False)
    for rep in range(3):
        # poison the outputs (eager fill kernels); scores past a row's visible
        # entries are never written, so the score buffer gets its initial value
        cap[0].fill_(-7.0)
        for t in cap[1:]:
            t.view(torch.uint8).fill_(0x5a)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(cap, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
        other = bufs()
        run(*other, False)                             # eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(other, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("fused", [False, True])
def test_decode_step_in_a_graph(fused):
    run, bufs = _decode_step([65536, 20000, 4100, 129, 70000], seed=81, fused=fused)
    _replay_matches(run, bufs)


def test_prefill_indexer_and_topk_in_a_graph():
    """2,048 queries of one sequence: the shared-key indexer kernel and the
    top-k of 1,024, captured together."""
    gen = synth.device_generator(83)
    cached, chunk, m, k, d_I, H_I = 20000, 2048, 4, 1024, 128, 64
    n_tot = (cached + chunk) // m
    keys = synth.device_rows(gen, n_tot, d_I, csa.FP8)
    q_idx = synth.device_rows(gen, chunk * H_I, d_I, csa.FP8).reshape(chunk, H_I, -1)
    w = torch.rand((chunk, H_I), generator=gen, device=DEV, dtype=torch.float32)
    q_pos_h = (cached + np.arange(chunk)).astype(np.int64)
    q_pos = torch.as_tensor(q_pos_h, device=DEV)
    n_valid = torch.as_tensor((q_pos_h + 1) // m, device=DEV)
    zeros = torch.zeros(chunk, dtype=torch.int64, device=DEV)

    def run(scores, idx, check):
        csa.indexer_score(q_idx, w, chunk, H_I, d_I, keys, csa.FP8, zeros, q_pos, m, scores, n_tot, check=check)
        csa.topk_select(scores, n_tot, chunk, n_valid, k, idx, None, check=check)

    def bufs():
        return (torch.full((chunk, n_tot), -7.0, dtype=torch.float32, device=DEV),
                torch.empty((chunk, k), dtype=torch.int32, device=DEV))
    _replay_matches(run, bufs)


def test_paged_decode_step_in_a_graph():
    """indexer_score_paged -> topk_select -> hybrid_attn_decode_paged over
    shuffled 32-entry blocks and ring windows, captured and replayed."""
    from test_gpu_paged import _paginate, _ring
    inp = synth.decode_inputs(91, [65536, 9001, 2052, 130, 40000], m=4, H=64, D=512, R=64, k=512)
    B, ld, k, BR = inp.B, int(inp.n_ent.max()), inp.k, 32
    rng = np.random.default_rng(92)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    kpool, ktab, kbps, krows = _paginate(inp.keys.reshape(-1, 128), inp.n_ent, inp.kv_off, BR, rng)
    vpool, vtab, vbps, vrows = _paginate(inp.kv.reshape(-1, 576), inp.n_ent, inp.kv_off, BR, rng)
    ring, start = _ring(inp.win, inp.win_len, rng)
    d = dict(q_idx=dv(inp.q_idx), w=dv(inp.w), q_pos=dv(inp.q_pos), nv=dv(inp.n_ent), q=dv(inp.q),
             kpool=dv(kpool), ktab=dv(ktab), vpool=dv(vpool), vtab=dv(vtab), win=dv(ring), start=dv(start),
             win_len=dv(inp.win_len), sinks=dv(inp.sinks))

    def run(scores, idx, out, check):
        csa.indexer_score_paged(d["q_idx"], d["w"], B, 64, 128, d["kpool"], csa.FP8, krows, d["ktab"], kbps, BR,
                                d["q_pos"], 4, scores, ld, check=check)
        csa.topk_select(scores, ld, B, d["nv"], k, idx, None, check=check)
        csa.hybrid_attn_decode_paged(d["q"], csa.BF16, B, 64, 512, d["q_pos"], None, EPS, 64, ROPE_BASE, d["vpool"],
                                     csa.SPLIT, vrows, d["vtab"], vbps, BR, 4, idx, k, d["win"], csa.BF16,
                                     inp.n_win, d["win_len"], d["sinks"], inp.scale, out, csa.BF16,
                                     csa.VARIANT_AUTO, check=check, win_start=d["start"])

    def bufs():
        return (torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV),
                torch.empty((B, k), dtype=torch.int32, device=DEV),
                torch.empty((B, 64, 512), dtype=torch.bfloat16, device=DEV))
    _replay_matches(run, bufs)

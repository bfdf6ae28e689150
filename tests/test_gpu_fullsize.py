"""Full-size runs of the five workloads on the GPU, checked against the oracle
on sampled queries (the oracle computes them one by one) and, for the ragged
mixed batch, for bit-identical outputs across batch permutations, batch sizes
and variants.  Inputs are drawn on the device with a seeded generator; only
the sampled sequences' rows are copied back for the oracle.

Workloads: CSA decode 16 x 65,536 tokens; HCA decode 32 x 262,144 tokens;
CSA prefill of 2,048 queries after 131,072 cached tokens; a ragged batch of
64 sequences with log-uniform lengths in [1,024, 1,048,576] through a CSA
layer (MXFP4 indexer, top-1024) and an HCA layer (m' = 128)."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, assert_lowp_close, gpu_bytes
from oracle import formats as OF
from oracle import method as OM

pytestmark = pytest.mark.gpu
D, R, N_WIN = 512, 64, 128


def _host(t):
    return t.cpu().numpy()


def _indexer_topk(d, ld, k):
    B = d["B"]
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    kv_off = torch.as_tensor(d["kv_off"], device=DEV)
    q_pos = torch.as_tensor(d["q_pos"], device=DEV)
    csa.indexer_score(d["q_idx"], d["w"], B, d["H_I"], d["d_I"], d["keys"], d["idx_fmt"], kv_off,
                      q_pos, d["m"], scores, ld)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    csa.topk_select(scores, ld, B, torch.as_tensor(d["n_ent"], device=DEV), k, idx)
    return scores, idx


def _attend(d, idx, rows=None, variant=csa.VARIANT_AUTO):
    rows = list(range(d["B"])) if rows is None else list(rows)
    r = torch.as_tensor(np.asarray(rows, np.int64), device=DEV)
    H = d["H"]
    out = gpu_bytes(len(rows) * H * 2 * D)
    csa.hybrid_attn_decode(d["q"][r].contiguous(), csa.BF16, len(rows), H, D,
                           torch.as_tensor(d["q_pos"][rows], device=DEV), None, EPS, R, ROPE_BASE,
                           d["kv"], csa.SPLIT, torch.as_tensor(d["kv_off"][rows], device=DEV), d["m"],
                           idx[r].contiguous() if idx is not None else None,
                           d["k"] if idx is not None else 0, d["win"][r].contiguous(), csa.BF16,
                           N_WIN, torch.as_tensor(d["win_len"][rows], device=DEV), d["sinks"],
                           d["scale"], out, csa.BF16, variant)
    return _host(out).reshape(len(rows), H * 2 * D)


def _check_scores_and_set(d, b, scores, idx, k):
    """Oracle indexer scores and top-k of sequence b against the GPU's."""
    off, N = int(d["kv_off"][b]), int(d["n_ent"][b])
    keys = OF.decode_rows(_host(d["keys"][off: off + N]), d["idx_fmt"], d["d_I"])
    qi = OF.decode_rows(_host(d["q_idx"][b]), d["idx_fmt"], d["d_I"])
    ref = OM.indexer_scores(qi, _host(d["w"][b]).astype(np.float64), keys)
    got = _host(scores[b, :N]).astype(np.float64)
    err = np.abs(got - ref).max() / max(1.0, np.abs(ref).max())
    assert err <= 1e-5, f"sequence {b}: relative score error {err:.3g}"
    want = OM.top_k(ref, k)
    g = _host(idx[b])
    g = g[g >= 0]
    assert len(g) == len(want), f"sequence {b}: {len(g)} selected, oracle {len(want)}"
    kth = np.sort(ref)[-k] if N > k else -np.inf
    diff = np.setxor1d(g, want)
    assert np.all(np.abs(ref[diff] - kth) <= 1e-6 * max(1.0, abs(kth))), \
        f"sequence {b}: top-k differs from the oracle away from ties"
    return g


def _check_attention(d, b, got_row, sel):
    off, N = int(d["kv_off"][b]), int(d["n_ent"][b])
    ents = np.zeros((N, D))
    if sel is None:
        ents = OF.decode_rows(_host(d["kv"][off: off + N]), csa.SPLIT, D, R)
    elif len(sel):
        ents[sel] = OF.decode_rows(_host(d["kv"][off + torch.as_tensor(sel, device=DEV).long()]),
                                   csa.SPLIT, D, R)
    wl = int(d["win_len"][b])
    win = OF.decode_rows(_host(d["win"][b, :wl]), csa.BF16, D)
    q = OF.decode_rows(_host(d["q"][b]), csa.BF16, D)
    ref = OM.decode_one(q, int(d["q_pos"][b]), ents, win, _host(d["sinks"]).astype(np.float64),
                        d["scale"], d["m"], idx=sel, eps=EPS, R=R, base=ROPE_BASE)
    g = OF.decode_rows(got_row.reshape(d["H"], -1), csa.BF16, D)
    assert_lowp_close(g, ref, what=f"sequence {b}")


def test_csa_decode_b16_ctx65536():
    d = synth.device_decode_inputs(2, [65536] * 16, m=4, H=64, D=D, R=R, k=512)
    ld = int(d["n_ent"].max())
    scores, idx = _indexer_topk(d, ld, 512)
    out = _attend(d, idx)
    for b in (0, 9, 15):
        sel = _check_scores_and_set(d, b, scores, idx, 512)
        _check_attention(d, b, out[b], sel)


def test_hca_decode_b32_ctx262144():
    d = synth.device_decode_inputs(3, [262144] * 32, m=128, H=64, D=D, R=R, csa=False)
    out = _attend(d, None)
    for b in (0, 31):
        _check_attention(d, b, out[b], None)


def test_ragged_csa_hca_b64_ctx1k_1m():
    lengths = synth.log_uniform_lengths(synth.rng_for(5), 64, 1024, 1048576)
    picks = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 17, 40})
    for layer, m, k in (("csa", 4, 1024), ("hca", 128, 0)):
        d = synth.device_decode_inputs(50 + m, lengths, m=m, H=64, D=D, R=R, csa=k > 0, k=k or 512,
                                       idx_fmt=csa.MXFP4)
        idx = None
        if k:
            scores, idx = _indexer_topk(d, int(d["n_ent"].max()), k)
        base = _attend(d, idx)
        for b in picks:
            sel = _check_scores_and_set(d, b, scores, idx, k) if k else None
            _check_attention(d, b, base[b], sel)
        # the same bits under 3 batch permutations, alone (batch of 1) and in every variant
        rng = np.random.default_rng(51)
        for _ in range(3):
            perm = rng.permutation(d["B"])
            assert np.array_equal(_attend(d, idx, perm), base[perm]), f"{layer}: permutation changed bits"
        for v in (csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS):
            assert np.array_equal(_attend(d, idx, variant=v), base), f"{layer}: variant {v} changed bits"
        for b in picks:
            for v in (csa.VARIANT_AUTO, csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS):
                assert np.array_equal(_attend(d, idx, [b], v)[0], base[b]), \
                    f"{layer}: sequence {b} alone (variant {v}) changed bits"
        del d


def test_csa_prefill_ctx131072_chunk2048():
    cached, chunk, H, m, k = 131072, 2048, 64, 4, 1024
    gen = synth.device_generator(4)
    T = cached + chunk
    n_tot = T // m
    kv = synth.device_rows(gen, n_tot, D, csa.SPLIT, R)
    keys = synth.device_rows(gen, n_tot, 128, csa.FP8)
    tok_pos0 = cached - N_WIN + 1
    tok = synth.device_rows(gen, T - tok_pos0, D, csa.BF16)
    q = synth.device_rows(gen, chunk * H, D, csa.BF16).reshape(chunk, H, -1)
    q_idx = synth.device_rows(gen, chunk * 64, 128, csa.FP8).reshape(chunk, 64, -1)
    w = torch.rand((chunk, 64), generator=gen, device=DEV, dtype=torch.float32)
    sinks = torch.randn(H, generator=gen, device=DEV, dtype=torch.float32)
    q_pos = (cached + np.arange(chunk)).astype(np.int64)
    n_ent = (q_pos + 1) // m
    zeros = torch.zeros(chunk, dtype=torch.int64, device=DEV)
    qp = torch.as_tensor(q_pos, device=DEV)
    ld = n_tot
    scores = torch.full((chunk, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(q_idx, w, chunk, 64, 128, keys, csa.FP8, zeros, qp, m, scores, ld)
    idx = torch.empty((chunk, k), dtype=torch.int32, device=DEV)
    csa.topk_select(scores, ld, chunk, torch.as_tensor(n_ent, device=DEV), k, idx)
    out = gpu_bytes(chunk * H * 2 * D)
    scale = 1.0 / np.sqrt(D)
    csa.hybrid_attn_prefill(q, csa.BF16, chunk, H, D, qp, None, EPS, R, ROPE_BASE, kv, csa.SPLIT,
                            zeros, m, idx, k, tok, csa.BF16, zeros,
                            torch.full((chunk,), tok_pos0, dtype=torch.int64, device=DEV), N_WIN,
                            sinks, scale, out, csa.BF16)
    got = _host(out).reshape(chunk, H * 2 * D)
    d = dict(kv_off=np.zeros(chunk, np.int64), n_ent=n_ent, keys=keys, q_idx=q_idx, w=w,
             idx_fmt=csa.FP8, d_I=128)
    tok_rows = None
    for i in (0, 1023, chunk - 1):
        sel = _check_scores_and_set(d, i, scores, idx, k)
        N = int(n_ent[i])
        ents = np.zeros((N, D))
        ents[sel] = OF.decode_rows(_host(kv[torch.as_tensor(sel, device=DEV).long()]), csa.SPLIT, D, R)
        if tok_rows is None:
            tok_rows = OF.decode_rows(_host(tok), csa.BF16, D)
        qi = OF.decode_rows(_host(q[i]), csa.BF16, D)
        ref = OM.prefill_one(qi, int(q_pos[i]), ents, tok_rows, tok_pos0, _host(sinks).astype(np.float64),
                             scale, m, N_WIN, idx=sel, eps=EPS, R=R, base=ROPE_BASE)
        g = OF.decode_rows(got[i].reshape(H, -1), csa.BF16, D)
        assert_lowp_close(g, ref, what=f"prefill query {i}")

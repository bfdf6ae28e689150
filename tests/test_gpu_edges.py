"""Edge cases of the method on the GPU, each against the float64 oracle:

* sink logits at their limits (DeepSeek-V4 blog, 让注意力学会"忽略": the sink
  logit in the denominator lets a head attend to nothing; -inf gives plain
  softmax, a large value sends the total weight towards 0), at short contexts
  with -1-padded selected lists, on the fp32 and the MFMA path;
* MXFP4 index rows whose E8M0 scales spread far from 2^0, and index keys /
  queries written by csa_compress from N(0,1) tokens (DeepSeek-V4 blog,
  FP4精度加速: the indexer runs at FP4);
* one paged decode step -- paged indexer, top-k, paged attention with the
  window as a ring -- compared directly with the oracle (硅星人 article,
  classic-cache and state-cache paragraphs).

Bars: fp32 paths 1e-5 normwise per (query, head); BF16 outputs max
|gpu - oracle| <= 2e-2 * rms(oracle) per (query, head); scores 1e-5 relative
to the row's largest; top-k sets exact except at ties with the k-th score
within 1e-6."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from oracle import formats as OF
from oracle import method as OM

from gpu_common import (DEV, EPS, ROPE_BASE, assert_f32_close, assert_lowp_close, decode_out, dev,
                        gpu_bytes, oracle_decode_query, oracle_scores, run_decode, upload_decode)

pytestmark = pytest.mark.gpu

SINK_LIMITS = np.array([-np.inf, -1e30, -20.0, 20.0, 60.0], np.float32)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


def _sinks(H, seed):
    """Per head: the limit values in turn, then N(0,1) logits."""
    z = np.random.default_rng(seed).standard_normal(H).astype(np.float32)
    z[: min(H, 2 * len(SINK_LIMITS))] = np.resize(SINK_LIMITS, min(H, 2 * len(SINK_LIMITS)))
    return z


@pytest.mark.parametrize("path,csa_mode", [("f32", True), ("mfma", True), ("mfma", False), ("f32", False)])
def test_attention_sink_limits(path, csa_mode):
    """Sinks in {-inf, -1e30, -20, +20, +60} per head.  Contexts of 1 to 2,051
    tokens: no entry (window only), a selected list padded with -1 (k > N),
    and a full list.  A sink of +60 scales a head's output down by about e^-55;
    the comparison is relative to the oracle's own RMS per head, so it holds
    the kernel to the same relative error at that scale."""
    if path == "f32":
        m, H, D, R = (4, 8, 128, 64) if csa_mode else (4, 16, 256, 64)
        fmts = dict(kv_fmt=csa.F32, q_fmt=csa.F32, win_fmt=csa.F32)
    else:
        m, H, D, R = (4, 32, 512, 64) if csa_mode else (128, 16, 512, 64)
        fmts = dict(kv_fmt=csa.SPLIT, q_fmt=csa.BF16, win_fmt=csa.BF16)
    lengths = [1, 5, 64, 130, 2051] if csa_mode else [1, 127, 128, 900, 20000]
    k = 64
    inp = synth.decode_inputs(801 + H, lengths, m=m, H=H, D=D, R=R, n_win=128, csa=False, k=k, **fmts)
    inp.sinks = _sinks(H, 802)
    sel = synth.random_selection(np.random.default_rng(803), inp.n_ent, k) if csa_mode else None
    out, _ = run_decode(inp, dev(sel) if sel is not None else None)
    fmt = csa.F32 if path == "f32" else csa.BF16
    got = decode_out(out, fmt, inp.B, H, D)
    assert np.all(np.isfinite(got)), "non-finite output"
    for b in range(inp.B):
        s = sel[b][sel[b] >= 0] if sel is not None else None
        ref = oracle_decode_query(inp, b, s)
        if fmt == csa.F32:
            assert_f32_close(got[b], ref, what=f"sinks, length {lengths[b]}")
        else:
            assert_lowp_close(got[b], ref, what=f"sinks, length {lengths[b]}")


def test_attention_no_entries_and_minus_inf_sink_is_zero():
    """No compressed entry and no window: the attended set is empty.  The
    output is the empty weighted sum, zero, for every sink (including -inf,
    where the softmax denominator is empty as well)."""
    H, D, R = 16, 512, 64
    inp = synth.decode_inputs(811, [3, 2], m=4, H=H, D=D, R=R, n_win=128, csa=False)
    inp.sinks = _sinks(H, 812)
    bufs = upload_decode(inp)
    bufs["kv"] = gpu_bytes(576)                        # no visible entry: one spare row
    bufs["win_len"] = torch.zeros(inp.B, dtype=torch.int32, device=DEV)
    out = gpu_bytes(inp.B * H * D * 2).fill_(0x7f)
    csa.hybrid_attn_decode(bufs["q"], csa.BF16, inp.B, H, D, bufs["q_pos"], None, EPS, R, ROPE_BASE, bufs["kv"],
                           csa.SPLIT, bufs["kv_off"], 4, None, 0, bufs["win"], csa.BF16, inp.n_win,
                           bufs["win_len"], bufs["sinks"], inp.scale, out, csa.BF16)
    torch.cuda.synchronize()
    assert torch.all(out == 0), "an empty attended set must give a zero output"
    for b in range(inp.B):
        ref = OM.decode_one(OF.decode_rows(inp.q[b], csa.BF16, D), int(inp.q_pos[b]), np.zeros((0, D)),
                            np.zeros((0, D)), inp.sinks.astype(np.float64), inp.scale, 4, R=R)
        assert np.all(ref == 0.0)


@pytest.mark.parametrize("lo,hi,H_I", [(100, 155, 64), (100, 155, 16), (118, 137, 32)])
def test_indexer_mxfp4_wide_scales(lo, hi, H_I):
    """MXFP4 keys and index queries whose E8M0 scale bytes spread over
    [lo, hi) (2^-27 .. 2^27 around 1): the scaled FP4 MFMA must apply every
    block's scales exactly."""
    lengths = [40000, 4099, 130, 5]
    inp = synth.decode_inputs(820 + lo + H_I, lengths, m=4, H=16, D=512, R=64, idx_fmt=csa.MXFP4, H_I=H_I,
                              d_I=128, mx_scales=(lo, hi))
    B = inp.B
    ld = int(inp.n_ent.max())
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(dev(inp.q_idx), dev(inp.w), B, H_I, 128, dev(inp.keys), csa.MXFP4, dev(inp.kv_off),
                      dev(inp.q_pos), inp.m, scores, ld)
    got = scores.cpu().numpy().astype(np.float64)
    for b in range(B):
        N = int(inp.n_ent[b])
        ref = oracle_scores(inp, b)
        err = np.abs(got[b, :N] - ref).max() / max(1.0, np.abs(ref).max())
        assert err <= 1e-5, f"row {b}: relative score error {err:.3g}"
        assert np.all(got[b, N:] == -7.0)


@pytest.mark.parametrize("fmt", [csa.MXFP4, csa.FP8])
def test_indexer_on_compressed_keys(fmt):
    """Index keys written by csa_compress from N(0,1) tokens (m = 4, per-token
    gates) and index queries written by csa_compress with m = 1: real scale
    bytes (MXFP4) and real FP8 codes.  Scores, then top-512, against the
    oracle on the decoded bytes."""
    rng = synth.rng_for(830 + fmt)
    m, H_I, d_I, k = 4, 64, 128, 512
    lengths = np.array([20000, 9001, 2052], np.int64)
    n_ent = lengths // m
    B = len(lengths)
    T = int((n_ent * m).sum())
    tok = synth.token_inputs(0, T, d_I, rng=rng)
    qt = synth.token_inputs(0, B * H_I, d_I, rng=rng)
    rb = csa.row_bytes(fmt, d_I)
    keys = gpu_bytes(int(n_ent.sum()) * rb)
    seg_off = np.concatenate([[0], np.cumsum(n_ent * m)]).astype(np.int64)
    kv_off = np.concatenate([[0], np.cumsum(n_ent)[:-1]]).astype(np.int64)
    csa.csa_compress(dev(tok.x), csa.F32, dev(tok.gate), 1, T, d_I, m, B, dev(seg_off),
                     dev(np.zeros(B, np.int64)), dev(kv_off), 0, None, EPS, 0, ROPE_BASE, keys, fmt)
    q_idx = gpu_bytes(B * H_I * rb)
    csa.csa_compress(dev(qt.x), csa.F32, dev(qt.gate), 1, B * H_I, d_I, 1, 1,
                     dev(np.array([0, B * H_I], np.int64)), dev(np.zeros(1, np.int64)),
                     dev(np.zeros(1, np.int64)), 0, None, EPS, 0, ROPE_BASE, q_idx, fmt)
    w = rng.uniform(0.0, 1.0, size=(B, H_I)).astype(np.float32)
    ld = int(n_ent.max())
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    q_pos = lengths - 1
    csa.indexer_score(q_idx, dev(w), B, H_I, d_I, keys, fmt, dev(kv_off), dev(q_pos), m, scores, ld)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    csa.topk_select(scores, ld, B, dev(n_ent), k, idx)
    got = scores.cpu().numpy().astype(np.float64)
    got_i = idx.cpu().numpy()
    keys_h = keys.cpu().numpy().reshape(-1, rb)
    qh = q_idx.cpu().numpy().reshape(B, H_I, rb)
    if fmt == csa.MXFP4:
        sc = keys_h[:, d_I // 2:]
        assert len(np.unique(sc)) > 1, "compressed keys should carry varied scale bytes"
    for b in range(B):
        N = int(n_ent[b])
        K = OF.decode_rows(keys_h[kv_off[b]: kv_off[b] + N], fmt, d_I)
        ref = OM.indexer_scores(OF.decode_rows(qh[b], fmt, d_I), w[b].astype(np.float64), K)
        err = np.abs(got[b, :N] - ref).max() / max(1.0, np.abs(ref).max())
        assert err <= 1e-5, f"row {b}: relative score error {err:.3g}"
        want = OM.top_k(ref, k)
        g = got_i[b][got_i[b] >= 0]
        kth = np.sort(ref)[-k]
        diff = np.setxor1d(g, want)
        assert len(g) == len(want) and np.all(np.abs(ref[diff] - kth) <= 1e-6 * max(1.0, abs(kth))), \
            f"row {b}: top-k set differs from the oracle away from ties"


def _paginate(rows, n_ent, off, BR, rng, spare=3):
    n_ent = np.asarray(n_ent, np.int64)
    nb = (n_ent + BR - 1) // BR
    bps = int(max(1, nb.max()))
    total = int(nb.sum()) + spare
    perm = rng.permutation(total).astype(np.int32)
    pool = rng.integers(0, 256, size=(total * BR, rows.shape[1]), dtype=np.uint8)
    table = rng.integers(0, total, size=(len(n_ent), bps)).astype(np.int32)
    nxt = 0
    for i, n in enumerate(n_ent):
        for j in range(int(nb[i])):
            phys = int(perm[nxt])
            nxt += 1
            table[i, j] = phys
            lo = int(off[i]) + j * BR
            cnt = min(BR, int(n) - j * BR)
            pool[phys * BR: phys * BR + cnt] = rows[lo: lo + cnt]
    return pool, table, bps, total * BR


@pytest.mark.parametrize("idx_fmt", [csa.FP8, csa.MXFP4])
def test_paged_step_matches_oracle(idx_fmt):
    """Paged indexer (blocks of 32 keys), top-k 512, paged attention (blocks
    of 32 entries) with each window kept as a ring at a random start: scores,
    selected sets and outputs against the oracle, which reads the same rows
    in logical order."""
    lengths = [65536, 20000, 4100, 129, 3]
    inp = synth.decode_inputs(840 + idx_fmt, lengths, m=4, H=64, D=512, R=64, k=512, idx_fmt=idx_fmt)
    B, H, D, R, k = inp.B, inp.H, inp.D, inp.R, inp.k
    rng = np.random.default_rng(841)
    BR = 32
    krb = synth.row_bytes(idx_fmt, inp.d_I)
    kpool, ktab, kbps, kpool_rows = _paginate(inp.keys.reshape(-1, krb), inp.n_ent, inp.kv_off, BR, rng)
    rb = synth.row_bytes(csa.SPLIT, D, R)
    pool, tab, bps, pool_rows = _paginate(inp.kv.reshape(-1, rb), inp.n_ent, inp.kv_off, BR, rng)
    ring = rng.integers(0, 256, size=inp.win.shape, dtype=np.uint8)
    start = rng.integers(0, inp.n_win, size=B).astype(np.int32)
    for b in range(B):
        for t in range(int(inp.win_len[b])):
            ring[b, (start[b] + t) % inp.n_win] = inp.win[b, t]
    ld = int(inp.n_ent.max())
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score_paged(dev(inp.q_idx), dev(inp.w), B, inp.H_I, inp.d_I, dev(kpool), idx_fmt, kpool_rows,
                            dev(ktab), kbps, BR, dev(inp.q_pos), inp.m, scores, ld)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    csa.topk_select(scores, ld, B, dev(inp.n_ent), k, idx)
    out = gpu_bytes(B * H * D * 2)
    csa.hybrid_attn_decode_paged(dev(inp.q), csa.BF16, B, H, D, dev(inp.q_pos), None, EPS, R, ROPE_BASE,
                                 dev(pool), csa.SPLIT, pool_rows, dev(tab), bps, BR, inp.m, idx, k, dev(ring),
                                 csa.BF16, inp.n_win, dev(inp.win_len), dev(inp.sinks), inp.scale, out, csa.BF16,
                                 win_start=dev(start))
    torch.cuda.synchronize()
    got_s = scores.cpu().numpy().astype(np.float64)
    got_i = idx.cpu().numpy()
    got = decode_out(out, csa.BF16, B, H, D)
    for b in range(B):
        N = int(inp.n_ent[b])
        ref_s = oracle_scores(inp, b)
        if N:
            assert np.abs(got_s[b, :N] - ref_s).max() <= 1e-5 * max(1.0, np.abs(ref_s).max()), f"row {b} scores"
        want = OM.top_k(ref_s, k)
        g = got_i[b][got_i[b] >= 0]
        if N > k:
            kth = np.sort(ref_s)[-k]
            diff = np.setxor1d(g, want)
            assert np.all(np.abs(ref_s[diff] - kth) <= 1e-6 * max(1.0, abs(kth))), f"row {b} top-k"
        else:
            assert np.array_equal(g, want)
        assert_lowp_close(got[b], oracle_decode_query(inp, b, g), what=f"paged step b{b}")

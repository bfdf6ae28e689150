"""GPU parity: every libcsa entry point against the float64 oracle on the same
seeded bytes.  Tolerances: fp32 paths 1e-5 normwise per (query, head); BF16 /
FP8 / FP4 paths 2e-2 max-abs after dividing by the oracle's RMS per (query,
head); top-k index sets exact; quantised codes exact except where the
oracle's value sits on a rounding midpoint (both neighbours are correct)."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from oracle import formats as OF
from oracle import method as OM

from gpu_common import (DEV, EPS, ROPE_BASE, assert_f32_close, assert_lowp_close, decode_out,
                        dev, gpu_bytes, oracle_decode_query, oracle_scores, run_decode,
                        upload_decode)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa.load_library()


# ------------------------------------------------------------------ compressor
def _quant_ok(gpu_vals, y, fmt, tol):
    """Elementwise: the GPU value equals the oracle's rounding of y, or the two
    candidates are neighbours and y lies within `tol` (the fp32 error bound of
    the GPU's value) of their midpoint, where either rounding is correct."""
    rnd = {csa.BF16: OF.round_bf16, csa.FP8: OF.round_e4m3}[fmt]
    want = rnd(y)
    bad = gpu_vals != want
    if not bad.any():
        return 0
    mid = 0.5 * (gpu_vals[bad] + want[bad])
    near = np.abs(y[bad] - mid) <= tol[bad]
    assert near.all(), f"{int((~near).sum())} codes differ away from a rounding midpoint"
    return int(bad.sum())


def _compress_error_bound(x, g, m, y, R, normalize):
    """A loose bound of |fp32 result - exact| for the compressor: the gated sum
    of m terms (m * 2^-24 relative to sum_t w_t |x_t|), scaled by the norm
    factor, plus a few roundings of the result itself."""
    T, D = x.shape
    gb = g.reshape(T // m, m, g.shape[1])
    w = np.exp(gb - gb.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    S = (w * np.abs(x.reshape(T // m, m, D))).sum(axis=1)
    C = (w * x.reshape(T // m, m, D)).sum(axis=1)
    r = 1.0 / np.sqrt(np.mean(C * C, axis=1, keepdims=True) + EPS) if normalize else 1.0
    bound = (m + 4) * 2.0 ** -24 * S * r
    if R:
        pair = bound[:, D - R::2] + bound[:, D - R + 1::2]
        bound[:, D - R::2] = pair
        bound[:, D - R + 1::2] = pair
    return 2.0 * bound + 2.0 ** -20 * np.abs(y)


@pytest.mark.parametrize("m,gate_cols,out_fmt,D,R,x_fmt", [
    (4, 1, csa.F32, 128, 64, csa.F32), (128, 1, csa.F32, 128, 64, csa.F32), (4, "D", csa.F32, 64, 16, csa.F32),
    (4, 1, csa.SPLIT, 512, 64, csa.F32), (128, 1, csa.SPLIT, 512, 64, csa.F32), (1, 1, csa.BF16, 512, 64, csa.F32),
    (4, 1, csa.FP8, 128, 0, csa.F32), (4, 1, csa.MXFP4, 128, 0, csa.F32), (1, 1, csa.MXFP4, 128, 0, csa.F32),
    # BF16 tokens: m = 128 over 16-byte chunks (four token groups at D = 512), m = 32, per-channel gates
    (128, 1, csa.SPLIT, 512, 64, csa.BF16), (128, 1, csa.BF16, 128, 64, csa.BF16), (32, 1, csa.FP8, 128, 0, csa.BF16),
    (128, "D", csa.SPLIT, 256, 64, csa.BF16),
])
def test_compress_matches_oracle(m, gate_cols, out_fmt, D, R, x_fmt):
    gc = D if gate_cols == "D" else gate_cols
    seg_len = [m * 7, m * 3, 0, m * 11]               # ragged segments incl. an empty one
    seg_pos0 = [0, 4 * m, 96 * m, 1000 * m]
    T = sum(seg_len)
    tok = synth.token_inputs(11 + m, T, D, gc)
    if x_fmt == csa.BF16:                             # the kernel reads BF16; the oracle gets its values
        x_dev = torch.from_numpy(tok.x).to(DEV).to(torch.bfloat16)
        tok.x = x_dev.float().cpu().numpy()
    else:
        x_dev = dev(tok.x)
    off = np.concatenate([[0], np.cumsum(seg_len)]).astype(np.int64)
    nent = [s // m for s in seg_len]
    out_row = np.array([5, 5 + nent[0], 0, 5 + nent[0] + nent[1]], dtype=np.int64)
    n_rows = int(out_row[-1] + nent[-1])
    rb = csa.row_bytes(out_fmt, D, R)
    out = torch.zeros(n_rows * rb, dtype=torch.uint8, device=DEV)
    normalize = R > 0
    csa.csa_compress(x_dev, x_fmt, dev(tok.gate), gc, T, D, m, 4, dev(off),
                     dev(np.array(seg_pos0, np.int64)), dev(out_row), normalize, None, EPS, R,
                     ROPE_BASE, out, out_fmt)
    raw = out.cpu().numpy().reshape(n_rows, rb)
    flips = 0
    for s in range(4):
        if nent[s] == 0:
            continue
        x = tok.x[off[s]: off[s + 1]].astype(np.float64)
        g = tok.gate[off[s]: off[s + 1]].astype(np.float64)
        y = OM.compress_entries(x, g, m, seg_pos0[s], eps=EPS, R=R, normalize=normalize)
        tol = _compress_error_bound(x, g, m, y, R, normalize)
        rows = raw[out_row[s]: out_row[s] + nent[s]]
        if out_fmt == csa.F32:
            assert_f32_close(OF.decode_rows(rows, csa.F32, D), y, what="compress f32")
        elif out_fmt in (csa.BF16, csa.FP8):
            flips += _quant_ok(OF.decode_rows(rows, out_fmt, D), y, out_fmt, tol)
        elif out_fmt == csa.SPLIT:
            dec = OF.decode_rows(rows, csa.SPLIT, D, R)
            flips += _quant_ok(dec[:, : D - R], y[:, : D - R], csa.FP8, tol[:, : D - R])
            flips += _quant_ok(dec[:, D - R:], y[:, D - R:], csa.BF16, tol[:, D - R:])
        elif out_fmt == csa.MXFP4:
            want = OF.mxfp4_encode(y)
            for r in range(rows.shape[0]):
                for blk in range(D // 32):
                    if rows[r, D // 2 + blk] != want[r, D // 2 + blk]:
                        sl = slice(blk * 32, (blk + 1) * 32)
                        amax = np.abs(y[r, sl]).max()
                        p2 = 2.0 ** np.round(np.log2(amax))
                        assert abs(amax - p2) <= tol[r, sl].max()
                        flips += 1
                        continue
                    gv = OF.mxfp4_decode(rows[r:r + 1], D)[0, blk * 32:(blk + 1) * 32]
                    wv = OF.mxfp4_decode(want[r:r + 1], D)[0, blk * 32:(blk + 1) * 32]
                    sc = 2.0 ** (int(rows[r, D // 2 + blk]) - 127)
                    bad = gv != wv
                    if bad.any():
                        yy = y[r, blk * 32:(blk + 1) * 32][bad]
                        mid = 0.5 * (gv[bad] + wv[bad])
                        assert np.all(np.abs(yy - mid) <= tol[r, blk * 32:(blk + 1) * 32][bad])
                        flips += int(bad.sum())
    assert flips <= max(2, raw.size // 1000)


@pytest.mark.parametrize("n_jobs", [3, 4])
def test_compress_batch_matches_single_calls(n_jobs):
    """One csa_compress_batch launch writes the same bytes as the jobs' own
    csa_compress calls (KV entries, indexer keys, window rows, and an HCA
    MXFP4 job that takes the generic block path)."""
    specs = [(4, 512, 64, csa.SPLIT, True, [4 * 5, 0, 4 * 9]),
             (4, 128, 0, csa.FP8, False, [4 * 5, 0, 4 * 9]),
             (1, 512, 64, csa.BF16, True, [3, 1, 7]),
             (128, 128, 0, csa.MXFP4, False, [256, 128])][:n_jobs]
    jobs, singles = [], []
    for j, (m, D, R, fmt, norm, seg_len) in enumerate(specs):
        T = sum(seg_len)
        tok = synth.token_inputs(70 + j, T, D)
        nseg = len(seg_len)
        off = np.concatenate([[0], np.cumsum(seg_len)]).astype(np.int64)
        pos0 = (np.arange(nseg, dtype=np.int64) * 1000 + 17) * m
        rows = np.concatenate([[2], 2 + np.cumsum([s // m for s in seg_len])[:-1]]).astype(np.int64)
        n_rows = int(rows[-1] + seg_len[-1] // m)
        rb = csa.row_bytes(fmt, D, R)
        args = dict(x=dev(tok.x).to(torch.bfloat16), x_fmt=csa.BF16, gate=dev(tok.gate), gate_cols=1,
                    n_tok=T, D=D, m=m, nseg=nseg, seg_tok_off=dev(off), seg_pos0=dev(pos0),
                    seg_out_row=dev(rows), normalize=norm, norm_w=None, eps=EPS, rope_dim=R,
                    rope_base=ROPE_BASE, out_fmt=fmt)
        out_b = torch.full((n_rows * rb,), 0xA5, dtype=torch.uint8, device=DEV)
        out_s = out_b.clone()
        jobs.append(dict(args, out=out_b))
        singles.append(out_s)
        csa.csa_compress(*(args[f] for f in csa.binding.COMPRESS_JOB_FIELDS[:16]), out_s, fmt)
    csa.csa_compress_batch(jobs)
    for j, (job, ref) in enumerate(zip(jobs, singles)):
        assert torch.equal(job["out"], ref), f"job {j}: batch bytes differ from csa_compress"


# ------------------------------------------------------------------ indexer
@pytest.mark.parametrize("fmt,H_I,d_I,lengths", [
    (csa.F32, 4, 64, [2048, 777, 5]),
    (csa.FP8, 64, 128, [65536, 4099, 1000, 3]),
    (csa.FP8, 16, 128, [5000]),
    (csa.FP8, 128, 128, [20000, 70]),
    (csa.MXFP4, 64, 128, [40000, 1024, 9]),
    (csa.MXFP4, 32, 128, [9000, 300]),
    (csa.MXFP4, 16, 128, [3000]),
    (csa.F32, 64, 256, [1500, 64]),
])
def test_indexer_matches_oracle(fmt, H_I, d_I, lengths):
    inp = synth.decode_inputs(21, lengths, m=4, H=16, D=128 if fmt == csa.F32 else 512, R=64,
                              kv_fmt=csa.F32 if fmt == csa.F32 else csa.SPLIT,
                              q_fmt=csa.F32 if fmt == csa.F32 else csa.BF16,
                              win_fmt=csa.F32 if fmt == csa.F32 else csa.BF16,
                              k=64, idx_fmt=fmt, H_I=H_I, d_I=d_I)
    B = inp.B
    ld = int(inp.n_ent.max()) + 3
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(dev(inp.q_idx), dev(inp.w), B, H_I, d_I, dev(inp.keys), fmt,
                      dev(inp.kv_off), dev(inp.q_pos), inp.m, scores, ld)
    got = scores.cpu().numpy().astype(np.float64)
    for b in range(B):
        N = int(inp.n_ent[b])
        ref = oracle_scores(inp, b)
        if N:
            err = np.abs(got[b, :N] - ref).max() / max(1.0, np.abs(ref).max())
            assert err <= 1e-5, f"row {b}: relative score error {err:.3g}"
        assert np.all(got[b, N:] == -7.0), "scores past N must stay untouched"


@pytest.mark.parametrize("fmt", [csa.FP8, csa.MXFP4])
def test_indexer_long_contexts(fmt):
    """Long rows, where each wave streams a share of several 64-key groups and
    (FP8) the waves of a query take its groups in turn: every score of three
    ragged rows against the oracle."""
    lengths = [1048576, 600001, 4097]
    m, H_I, d_I = 4, 64, 128
    gen = synth.device_generator(23)
    n_ent = np.asarray(lengths) // m
    kv_off = np.concatenate([[0], np.cumsum(n_ent)[:-1]]).astype(np.int64)
    keys = synth.device_rows(gen, int(n_ent.sum()), d_I, fmt)
    B = len(lengths)
    q_idx = synth.device_rows(gen, B * H_I, d_I, fmt).reshape(B, H_I, -1)
    w = torch.rand((B, H_I), generator=gen, device=DEV, dtype=torch.float32)
    ld = int(n_ent.max())
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(q_idx, w, B, H_I, d_I, keys, fmt, torch.as_tensor(kv_off, device=DEV),
                      torch.as_tensor(np.asarray(lengths) - 1, device=DEV), m, scores, ld)
    got = scores.cpu().numpy().astype(np.float64)
    for b in range(B):
        N = int(n_ent[b])
        kb = OF.decode_rows(keys[kv_off[b]: kv_off[b] + N].cpu().numpy(), fmt, d_I)
        ref = OM.indexer_scores(OF.decode_rows(q_idx[b].cpu().numpy(), fmt, d_I),
                                w[b].cpu().numpy().astype(np.float64), kb)
        err = np.abs(got[b, :N] - ref).max() / max(1.0, np.abs(ref).max())
        assert err <= 1e-5, f"row {b}: relative score error {err:.3g}"
        assert np.all(got[b, N:] == -7.0), "scores past N must stay untouched"


@pytest.mark.parametrize("H_I", [64, 32, 16, 128])
def test_indexer_shared_keys_match_streaming_bits(H_I):
    """Large batches take the shared-key kernel (a workgroup multiplies one
    loaded key group against four queries of the same sequence).  Its scores
    must carry the same bits as the streaming kernel's for the same queries in
    a small batch, and match the oracle.  The batch mixes two sequences (one
    four-query block straddles them and streams per wave), ragged visible
    counts inside blocks, and a two-query tail block."""
    gen = synth.device_generator(61 + H_I)
    rng = np.random.default_rng(62 + H_I)
    m, d_I = 4, 128
    n_a, n_b = 40000, 5000                                   # keys of the two sequences
    keys = synth.device_rows(gen, n_a + n_b, d_I, csa.FP8)
    nq_a, nq_b = 701, 401                                    # 1102 queries: block 175 holds both
    q_pos = np.concatenate([rng.integers(0, n_a * m, nq_a), rng.integers(0, n_b * m, nq_b)]).astype(np.int64)
    q_pos[:8] = [n_a * m - 1, 3, 64 * m - 1, 64 * m, 2048 * m + 5, n_a * m - 2, 0, 17]
    key_off = np.concatenate([np.zeros(nq_a), np.full(nq_b, n_a)]).astype(np.int64)
    nq = nq_a + nq_b
    q_idx = synth.device_rows(gen, nq * H_I, d_I, csa.FP8).reshape(nq, H_I, -1)
    w = torch.rand((nq, H_I), generator=gen, device=DEV, dtype=torch.float32)
    ld = n_a
    big = torch.full((nq, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(q_idx, w, nq, H_I, d_I, keys, csa.FP8, dev(key_off), dev(q_pos), m, big, ld)
    picks = np.array([0, 1, 2, 3, 4, 5, 6, 7, 350, 699, 700, 701, 702, 703, 1100, 1101])
    small = torch.full((len(picks), ld), -7.0, dtype=torch.float32, device=DEV)
    pk = torch.as_tensor(picks, device=DEV)
    csa.indexer_score(q_idx[pk].contiguous(), w[pk].contiguous(), len(picks), H_I, d_I, keys, csa.FP8,
                      dev(key_off[picks]), dev(q_pos[picks]), m, small, ld)
    got_big = big.cpu().numpy()
    got_small = small.cpu().numpy()
    for r, i in enumerate(picks):
        assert np.array_equal(got_big[i].view(np.uint32), got_small[r].view(np.uint32)), f"query {i}: bits differ"
    keys_h = keys.cpu().numpy()
    for i in picks[[0, 1, 4, 8, 10, 11, 15]]:
        N = min(int((q_pos[i] + 1) // m), ld)
        kb = OF.decode_rows(keys_h[key_off[i]: key_off[i] + N], csa.FP8, d_I)
        ref = OM.indexer_scores(OF.decode_rows(q_idx[i].cpu().numpy(), csa.FP8, d_I),
                                w[i].cpu().numpy().astype(np.float64), kb)
        err = np.abs(got_big[i, :N] - ref).max() / max(1.0, np.abs(ref).max()) if N else 0.0
        assert err <= 1e-5, f"query {i}: relative score error {err:.3g}"
        assert np.all(got_big[i, N:] == -7.0), f"query {i}: scores past N must stay untouched"


# ------------------------------------------------------------------ top-k
@pytest.mark.parametrize("ld,k,tie_levels,n_valid", [
    (16384, 512, 0, None), (16384, 512, 5, None), (5000, 1024, 0, [5000, 4999, 1024, 1000, 1, 0]),
    (262144, 1024, 0, [262144, 100000]), (3000, 64, 3, [3000, 64, 65, 2]), (70000, 2048, 0, None),
    (33792, 1024, 0, [33792, 33000, 20000]), (34000, 1024, 2, [34000, 33792, 4097]),
    # rows past 33792 scores: slices + candidate merge
    (262144, 512, 7, [262144, 262100, 16385, 40000]), (1048576, 512, 0, [1048576, 500000]),
    (100000, 4096, 0, [100000, 4096, 4095]),
])
def test_topk_exact(ld, k, tie_levels, n_valid):
    nq = len(n_valid) if n_valid else 4
    s, nv = synth.random_scores(31 + k, nq, ld, n_valid, tie_levels)
    if tie_levels == 0:
        s[0, 100:300] = s[0, 50]                    # a run of exact ties
    idx = torch.empty((nq, k), dtype=torch.int32, device=DEV)
    tops = torch.empty((nq, k), dtype=torch.float32, device=DEV)
    csa.topk_select(dev(s), ld, nq, dev(nv), k, idx, tops)
    got = idx.cpu().numpy()
    gs = tops.cpu().numpy()
    # without the score output (rows placed from the compacted pass): the same indices
    idx2 = torch.empty((nq, k), dtype=torch.int32, device=DEV)
    csa.topk_select(dev(s), ld, nq, dev(nv), k, idx2)
    assert np.array_equal(idx2.cpu().numpy(), got)
    for i in range(nq):
        n = int(nv[i])
        want = OM.top_k(s[i, :n].astype(np.float64), k)
        c = len(want)
        assert np.array_equal(got[i, :c], want), f"row {i}"
        assert np.all(got[i, c:] == -1)
        assert np.array_equal(gs[i, :c], s[i, want])
        assert np.all(np.isneginf(gs[i, c:]))


def _sampled_positions(ld):
    """Row positions the selector samples for its threshold estimate: thread t
    of 1024 samples position 1024 (t % V) + t, V the registers per thread."""
    V = next(v for v in (4, 8, 16, 24, 33) if ld <= 1024 * v)
    t = np.arange(1024)
    p = 1024 * (t % V) + t
    return p[p < ld]


@pytest.mark.parametrize("case", ["top_at_samples", "top_off_samples", "ascending", "descending", "relu_zeros",
                                  "boundaries"])
def test_topk_value_layouts(case):
    """Layouts that defeat the sampled threshold estimate (too few or too many
    candidates) take the general selection; every layout gives the exact set."""
    rng = np.random.default_rng(11)
    rows = []
    if case == "boundaries":
        for ld in (513, 4096, 4097, 8192, 8193, 16384, 16385, 24576, 24577, 33792):
            rows.append((rng.standard_normal(ld).astype(np.float32), 512))
    else:
        for ld in (3000, 16384, 24000, 33792):
            x = rng.standard_normal(ld).astype(np.float32)
            ps = _sampled_positions(ld)
            if case == "top_at_samples":
                x[ps] += 20.0
            elif case == "top_off_samples":
                off = np.setdiff1d(np.arange(ld), ps)
                x[off[rng.choice(len(off), min(3000, len(off) // 2), replace=False)]] += 20.0
            elif case == "ascending":
                x = np.sort(x)
            elif case == "descending":
                x = np.sort(x)[::-1].copy()
            elif case == "relu_zeros":
                x = np.maximum(x, 0.0).astype(np.float32)
            rows.append((x, 512))
            rows.append((x, 1024))
    for x, k in rows:
        ld = len(x)
        s = x[None, :]
        idx = torch.empty((1, k), dtype=torch.int32, device=DEV)
        tops = torch.empty((1, k), dtype=torch.float32, device=DEV)
        csa.topk_select(dev(s), ld, 1, None, k, idx, tops)
        got = idx.cpu().numpy()[0]
        want = OM.top_k(x.astype(np.float64), k)
        assert np.array_equal(got[: len(want)], want), f"{case} ld={ld} k={k}"
        assert np.all(got[len(want):] == -1)
        assert np.array_equal(tops.cpu().numpy()[0, : len(want)], x[want])


def test_topk_long_rows_in_a_graph():
    """The long-row path (slices, then a candidate merge through the caller's
    workspace) captured in a HIP graph: every replay, with eager work in
    between, gives the eager result."""
    nq, ld, k = 3, 200000, 1024
    s, nv = synth.random_scores(77, nq, ld, [200000, 150000, 34000], 0)
    S, NV = dev(s), dev(nv)
    ws = torch.empty(csa.topk_workspace_bytes(nq, ld, k), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 0
    eager = torch.empty((nq, k), dtype=torch.int32, device=DEV)
    csa.topk_select(S, ld, nq, NV, k, eager)
    torch.cuda.synchronize()
    out = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        csa.topk_select(S, ld, nq, NV, k, out, check=False, workspace=ws)
    for _ in range(3):
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        other = torch.empty_like(eager)
        csa.topk_select(S, ld, nq, NV, k, other)       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    for i in range(nq):
        want = OM.top_k(s[i, : nv[i]].astype(np.float64), k)
        assert np.array_equal(eager.cpu().numpy()[i, : len(want)], want)


def test_topk_long_rows_on_two_streams():
    """Two long-row selections running concurrently on two streams, each with
    its own workspace, give the bits each gives alone (the caller owns the
    scratch, so concurrent calls do not share it)."""
    k = 512
    sa, nva = synth.random_scores(78, 8, 262144, [262144] * 6 + [100000, 40000], 0)
    sb, nvb = synth.random_scores(79, 5, 1048576, [1048576, 700000, 300000, 40000, 1048575], 3)
    A, NA, B_, NB = dev(sa), dev(nva), dev(sb), dev(nvb)
    ref_a = torch.empty((8, k), dtype=torch.int32, device=DEV)
    ref_b = torch.empty((5, k), dtype=torch.int32, device=DEV)
    csa.topk_select(A, 262144, 8, NA, k, ref_a)
    csa.topk_select(B_, 1048576, 5, NB, k, ref_b)
    torch.cuda.synchronize()
    wa = torch.empty(csa.topk_workspace_bytes(8, 262144, k), dtype=torch.uint8, device=DEV)
    wb = torch.empty(csa.topk_workspace_bytes(5, 1048576, k), dtype=torch.uint8, device=DEV)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(4):
        oa = torch.full((8, k), -7, dtype=torch.int32, device=DEV)
        ob = torch.full((5, k), -7, dtype=torch.int32, device=DEV)
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            csa.topk_select(A, 262144, 8, NA, k, oa, workspace=wa, stream=s1)
        with torch.cuda.stream(s2):
            csa.topk_select(B_, 1048576, 5, NB, k, ob, workspace=wb, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b), f"repetition {rep}"
        outs.append(oa)
    for i in range(5):
        want = OM.top_k(sb[i, : nvb[i]].astype(np.float64), k)
        assert np.array_equal(ref_b.cpu().numpy()[i, : len(want)], want)


def test_topk_workspace_errors_on_the_device_path():
    """A short workspace is refused before anything runs: the outputs keep
    their contents."""
    nq, ld, k = 2, 100000, 512
    s, nv = synth.random_scores(80, nq, ld, None, 0)
    out = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
    need = csa.topk_workspace_bytes(nq, ld, k)
    short = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(csa.CsaError, match="WORKSPACE"):
        csa.topk_select(dev(s), ld, nq, dev(nv), k, out, workspace=short)
    torch.cuda.synchronize()
    assert torch.all(out == -7)


@pytest.mark.parametrize("ld", [20000, 40000])
@pytest.mark.parametrize("case", ["all_equal", "two_levels", "with_inf", "huge_range", "negatives",
                                  "ties_at_kth"])
def test_topk_edge_rows(case, ld):
    rng = np.random.default_rng(5)
    nq, k = 3, 512
    nv = np.array([ld, 777, 513], np.int64)
    if case == "ties_at_kth":
        # a few copies of each row's k-th largest score: some of them are taken
        # (the lowest indices), the rest are not
        s = rng.standard_normal((nq, ld)).astype(np.float32)
        for i in range(nq):
            n = int(nv[i])
            kth = np.sort(s[i, :n])[n - k]
            s[i, rng.choice(n, size=7, replace=False)] = kth
    elif case == "all_equal":
        s = np.full((nq, ld), 1.5, np.float32)
    elif case == "two_levels":
        s = np.where(rng.random((nq, ld)) < 0.01, 2.0, 1.0).astype(np.float32)
    elif case == "with_inf":
        s = rng.standard_normal((nq, ld)).astype(np.float32)
        s[:, ::97] = -np.inf
        s[0, 5:300] = np.inf
    elif case == "huge_range":
        s = (rng.standard_normal((nq, ld)) * 10.0 ** rng.integers(-30, 30, (nq, ld))).astype(np.float32)
    else:
        s = -np.abs(rng.standard_normal((nq, ld))).astype(np.float32)
    idx = torch.empty((nq, k), dtype=torch.int32, device=DEV)
    csa.topk_select(dev(s), ld, nq, dev(nv), k, idx)
    got = idx.cpu().numpy()
    for i in range(nq):
        want = OM.top_k(s[i, : nv[i]].astype(np.float64), k)
        assert np.array_equal(got[i, : len(want)], want), f"{case} row {i}"
        assert np.all(got[i, len(want):] == -1)


# ------------------------------------------------------------------ attention
def _decode_case(cfg, lengths, seed, csa_mode):
    c = synth.WORKLOADS[cfg]
    return synth.decode_inputs(seed, lengths, m=c["m"], H=c["H"], D=c["D"], R=c["R"],
                               n_win=c["n_win"], kv_fmt=c["kv_fmt"], q_fmt=c["q_fmt"],
                               win_fmt=c["win_fmt"], csa=csa_mode, k=c.get("k", 512),
                               idx_fmt=c.get("idx_fmt", csa.FP8), H_I=c.get("H_I", 64),
                               d_I=c.get("d_I", 128))


@pytest.mark.parametrize("cfg,lengths,csa_mode", [
    ("csa_decode_fp32_b1_ctx2048", [2048, 300, 7], True), ("csa_decode_fp32_b1_ctx2048", [2048], False),
    ("csa_decode_b16_ctx65536", [65536, 9000, 2051, 130, 5], True),
    ("hca_decode_b32_ctx262144", [262144, 40000, 128, 127], False),
    ("csa_decode_b16_ctx65536", [4100, 777], False),
])
def test_attn_decode_matches_oracle(cfg, lengths, csa_mode):
    inp = _decode_case(cfg, lengths, 40 + synth.WORKLOADS[cfg]["seed"], csa_mode)
    rng = np.random.default_rng(99)
    sel = synth.random_selection(rng, inp.n_ent, inp.k) if csa_mode else None
    out, _ = run_decode(inp, dev(sel) if sel is not None else None)
    fmt = csa.F32 if inp.q_fmt == csa.F32 else csa.BF16
    got = decode_out(out, fmt, inp.B, inp.H, inp.D)
    for b in range(inp.B):
        s = sel[b][sel[b] >= 0] if sel is not None else None
        ref = oracle_decode_query(inp, b, s)
        if fmt == csa.F32:
            assert_f32_close(got[b], ref, what=f"{cfg} b{b}")
        else:
            assert_lowp_close(got[b], ref, what=f"{cfg} b{b}")


@pytest.mark.parametrize("H,csa_mode,k", [(16, True, 512), (128, True, 1024), (32, False, 0)])
def test_attn_decode_head_counts(H, csa_mode, k):
    """The MFMA path at other query-head counts (tiles of 16 heads), CSA with
    top-512 / top-1024 and HCA, in every variant (same bits)."""
    m = 4 if csa_mode else 128
    lengths = [40000, 3000, 130] if csa_mode else [262144, 5000]
    inp = synth.decode_inputs(46 + H, lengths, m=m, H=H, D=512, R=64, n_win=128, kv_fmt=csa.SPLIT,
                              q_fmt=csa.BF16, win_fmt=csa.BF16, csa=False, k=max(k, 1))
    sel = synth.random_selection(np.random.default_rng(47), inp.n_ent, k) if csa_mode else None
    idx_t = dev(sel) if sel is not None else None
    out, bufs = run_decode(inp, idx_t)
    got = decode_out(out, csa.BF16, inp.B, H, 512)
    for b in range(inp.B):
        s = sel[b][sel[b] >= 0] if sel is not None else None
        assert_lowp_close(got[b], oracle_decode_query(inp, b, s), what=f"H={H} b{b}")
    base = out.cpu().numpy()
    for v in (csa.VARIANT_HIGH_OCC, csa.VARIANT_LOW_OCC, csa.VARIANT_FULL_DIMS):
        o2, _ = run_decode(inp, idx_t, v, bufs)
        assert np.array_equal(o2.cpu().numpy(), base), f"H={H}: variant {v} changed the bits"


def test_degenerate_queries_and_empty_calls():
    """Queries with no visible entry (positions below m - 1: window only),
    one entry, and a partial first group, through indexer -> top-k ->
    attention against the oracle; then every entry point with an empty batch,
    which must enqueue nothing and write nothing."""
    m, H, D, R, k = 4, 16, 512, 64, 64
    lengths = [1, 3, 4, 5, 129]                       # N = 0, 0, 1, 1, 32
    inp = synth.decode_inputs(91, lengths, m=m, H=H, D=D, R=R, n_win=128, kv_fmt=csa.SPLIT,
                              q_fmt=csa.BF16, win_fmt=csa.BF16, csa=True, k=k, H_I=64, d_I=128)
    B = inp.B
    ld = max(1, int(inp.n_ent.max()))
    scores = torch.full((B, ld), -7.0, dtype=torch.float32, device=DEV)
    csa.indexer_score(dev(inp.q_idx), dev(inp.w), B, 64, 128, dev(inp.keys), csa.FP8, dev(inp.kv_off),
                      dev(inp.q_pos), m, scores, ld)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    csa.topk_select(scores, ld, B, dev(inp.n_ent), k, idx)
    got_s, got_i = scores.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        N = int(inp.n_ent[b])
        assert np.all(got_s[b, N:] == -7.0)
        if N:
            ref = oracle_scores(inp, b)
            assert np.abs(got_s[b, :N] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
        assert np.array_equal(np.sort(got_i[b][got_i[b] >= 0]), np.arange(N)), "N <= k keeps every entry"
        assert np.all(got_i[b, N:] == -1)
    out, _ = run_decode(inp, idx)
    got = decode_out(out, csa.BF16, B, H, D)
    for b in range(B):
        sel = got_i[b][got_i[b] >= 0]
        assert_lowp_close(got[b], oracle_decode_query(inp, b, sel), what=f"length {lengths[b]}")
    # empty calls: nothing written
    sentinel = torch.full((4,), -3.0, dtype=torch.float32, device=DEV)
    e64 = torch.zeros(0, dtype=torch.int64, device=DEV)
    csa.indexer_score(dev(inp.q_idx), dev(inp.w), 0, 64, 128, dev(inp.keys), csa.FP8, e64, e64, m, sentinel, 1)
    csa.topk_select(sentinel, 1, 0, None, 4, torch.zeros(0, dtype=torch.int32, device=DEV))
    obuf = torch.full((64,), 0x5a, dtype=torch.uint8, device=DEV)
    csa.hybrid_attn_decode(dev(inp.q), csa.BF16, 0, H, D, e64, None, EPS, R, ROPE_BASE, dev(inp.kv), csa.SPLIT,
                           e64, m, None, 0, dev(inp.win), csa.BF16, 128,
                           torch.zeros(0, dtype=torch.int32, device=DEV), dev(inp.sinks), inp.scale, obuf, csa.BF16)
    csa.csa_compress(torch.zeros(4, device=DEV), csa.F32, torch.zeros(1, device=DEV), 1, 0, 4, 1, 1,
                     torch.zeros(2, dtype=torch.int64, device=DEV), e64.new_zeros(1), e64.new_zeros(1),
                     0, None, EPS, 0, ROPE_BASE, obuf, csa.F32)
    torch.cuda.synchronize()
    assert torch.all(sentinel == -3.0) and torch.all(obuf == 0x5a)

"""csa_compress_score: a decode step's compress jobs and its indexer scores in
one launch.  Its results must be those of csa_compress_batch followed by
indexer_score -- every cache byte and every score bit, nothing written past a
query's visible keys -- and the score of each new key must agree with the
oracle's indexer on the key row that was written (硅星人 article on DeepSeek
V4, CSA paragraph and the indexer detail; DeepSeek-V4 blog, index visibility
rule)."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, dev
from test_gpu_paged import _paginate
from oracle import formats as OF
from oracle import method as OM

pytestmark = pytest.mark.gpu

M, D, R = 4, 512, 64
SENTINEL = -7.0


def _case(lengths, new, H_I, idx_fmt, seed, with_kv=True, key_job=True):
    """Device state of a decode step: the caches of synth.decode_inputs, the
    new tokens of the queries flagged in `new` (a complete block each, whose
    rows are their last visible rows), and the step's compress jobs."""
    lengths = np.asarray(lengths, np.int64)
    new = np.asarray(new, bool)
    assert np.all(lengths[new] % M == 0)
    inp = synth.decode_inputs(seed, lengths, m=M, H=16, D=D, R=R, idx_fmt=idx_fmt, H_I=H_I)
    B, d_I = inp.B, inp.d_I
    rng = np.random.default_rng(seed + 1)
    seg_len = np.where(new, M, 0).astype(np.int64)
    seg_off = np.concatenate([[0], np.cumsum(seg_len)]).astype(np.int64)
    n_tok = int(seg_off[-1])
    n_ent = inp.n_ent.astype(np.int64)
    rows = np.where(new, inp.kv_off + n_ent - 1, 0).astype(np.int64)
    pos0 = np.where(new, (n_ent - 1) * M, 0).astype(np.int64)
    st = dict(inp=inp, B=B, ld=int(max(1, n_ent.max())), n_tok=n_tok,
              key_tok=dev(rng.standard_normal((max(n_tok, 1), d_I)).astype(np.float32), torch.bfloat16),
              key_gate=dev(rng.standard_normal((max(n_tok, 1), 1)).astype(np.float32)),
              kv_tok=dev(rng.standard_normal((max(n_tok, 1), D)).astype(np.float32), torch.bfloat16),
              kv_gate=dev(rng.standard_normal((max(n_tok, 1), 1)).astype(np.float32)),
              seg_off=dev(seg_off), pos0=dev(pos0), rows=dev(rows),
              q_idx=dev(inp.q_idx), w=dev(inp.w), kv_off=dev(inp.kv_off), q_pos=dev(inp.q_pos),
              with_kv=with_kv, key_job=key_job)
    return st


def _run(st, fused, nq=None):
    inp, B = st["inp"], st["B"]
    nq = B if nq is None else nq
    keys, kv = dev(inp.keys), dev(inp.kv)
    scores = torch.full((B, st["ld"]), SENTINEL, dtype=torch.float32, device=DEV)

    def job(x, gate, Dj, normalize, Rj, out, fmt):
        return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=st["n_tok"], D=Dj, m=M, nseg=B,
                    seg_tok_off=st["seg_off"], seg_pos0=st["pos0"], seg_out_row=st["rows"],
                    normalize=normalize, norm_w=None, eps=EPS, rope_dim=Rj, rope_base=ROPE_BASE,
                    out=out, out_fmt=fmt)
    jobs = []
    if st["with_kv"]:
        jobs.append(job(st["kv_tok"], st["kv_gate"], D, 1, R, kv, csa.SPLIT))
    if st["key_job"]:
        jobs.append(job(st["key_tok"], st["key_gate"], inp.d_I, 0, 0, keys, inp.idx_fmt))
    args = (st["q_idx"], st["w"], nq, inp.H_I, inp.d_I, keys, inp.idx_fmt, st["kv_off"], st["q_pos"], M,
            scores, st["ld"])
    if fused:
        csa.csa_compress_score(jobs, *args)
    else:
        csa.csa_compress_batch(jobs)
        if nq > 0:
            csa.indexer_score(*args)
    torch.cuda.synchronize()
    return (keys.cpu().numpy(), kv.cpu().numpy(), scores.cpu().numpy())


def _same(st, nq=None):
    a = _run(st, False, nq)
    b = _run(st, True, nq)
    for name, x, y in zip(("keys", "kv", "scores"), a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name} differ from the two-call path"
    return b


def _check_new_scores(st, keys, scores, new):
    """Each new key's score against the oracle's indexer on the row written."""
    inp = st["inp"]
    rb = synth.row_bytes(inp.idx_fmt, inp.d_I)
    for b in np.flatnonzero(new):
        N = int(inp.n_ent[b])
        row = int(inp.kv_off[b]) + N - 1
        key = OF.decode_rows(keys.reshape(-1, rb)[row: row + 1], inp.idx_fmt, inp.d_I)
        qi = OF.decode_rows(inp.q_idx[b], inp.idx_fmt, inp.d_I)
        ref = OM.indexer_scores(qi, inp.w[b].astype(np.float64), key)[0]
        got = float(scores[b, N - 1])
        assert got != SENTINEL
        assert abs(got - ref) <= 1e-5 * max(1.0, abs(ref)), (b, got, ref)


@pytest.mark.parametrize("H_I", [64, 16, 128])
def test_fused_step_matches_two_calls(H_I):
    lengths = [65536, 9000, 2052, 132, 8, 40000, 4, 3, 65536, 1000]
    new = [True, False, True, True, True, False, True, False, True, True]
    st = _case(lengths, new, H_I, csa.FP8, 500 + H_I)
    keys, _, scores = _same(st)
    _check_new_scores(st, keys, scores, np.asarray(new))


def test_fused_every_query_new_key_bench_shape():
    """Sixteen sequences of 65,536 tokens, each completing a block."""
    st = _case([65536] * 16, [True] * 16, 64, csa.FP8, 77)
    keys, _, scores = _same(st)
    _check_new_scores(st, keys, scores, np.ones(16, bool))


def test_fused_long_rows_interleaved_shares():
    """Rows long enough that each wave takes several interleaved groups."""
    lengths = [262144, 100000, 262144, 50000, 4096, 262144, 8, 180000]
    new = [True, True, False, True, True, True, True, False]
    st = _case(lengths, new, 64, csa.FP8, 91)
    keys, _, scores = _same(st)
    _check_new_scores(st, keys, scores, np.asarray(new))


def test_fused_without_key_job_and_without_queries():
    st = _case([4096, 2052, 800], [True, True, True], 64, csa.FP8, 12, key_job=False)
    _same(st)
    st = _case([4096, 2052, 800], [True, True, True], 64, csa.FP8, 13)
    _same(st, nq=0)


def test_fused_mxfp4_keys_take_two_launches_with_the_same_results():
    lengths = [65536, 9000, 2052, 132]
    new = [True, False, True, True]
    st = _case(lengths, new, 64, csa.MXFP4, 33)
    keys, _, scores = _same(st)
    _check_new_scores(st, keys, scores, np.asarray(new))


def test_fused_rejects_a_key_job_of_the_wrong_shape():
    st = _case([4096, 2052], [True, True], 64, csa.FP8, 14)
    inp = st["inp"]
    keys = dev(inp.keys)
    scores = torch.empty((2, st["ld"]), dtype=torch.float32, device=DEV)
    bad = dict(x=st["key_tok"], x_fmt=csa.BF16, gate=st["key_gate"], gate_cols=1, n_tok=st["n_tok"],
               D=inp.d_I, m=M, nseg=1, seg_tok_off=st["seg_off"], seg_pos0=st["pos0"],
               seg_out_row=st["rows"], normalize=0, norm_w=None, eps=EPS, rope_dim=0,
               rope_base=ROPE_BASE, out=keys, out_fmt=csa.FP8)
    with pytest.raises(csa.CsaError):
        csa.csa_compress_score([bad], st["q_idx"], st["w"], 2, inp.H_I, inp.d_I, keys, csa.FP8, st["kv_off"],
                               st["q_pos"], M, scores, st["ld"], check=False)


def test_fused_scores_independent_of_batch_order():
    """The one-launch step gives every query the same score bits whatever the
    order of the batch (its segments permuted with it), and writes the same
    key rows (QbitAI piece on batch invariance)."""
    lengths = [65536, 9000, 2052, 132, 8, 40000, 4, 3]
    new = np.array([True, False, True, True, True, False, True, False])
    st = _case(lengths, new, 64, csa.FP8, 707)
    keys0, _, s0 = _run(st, True)
    perm = np.random.default_rng(708).permutation(st["B"])
    inp = st["inp"]
    seg_len = np.where(new, M, 0).astype(np.int64)
    # the same tokens, segments re-ordered with the queries
    tok_first = np.concatenate([[0], np.cumsum(seg_len)])[:-1]
    order = np.concatenate([np.arange(tok_first[b], tok_first[b] + seg_len[b]) for b in perm]).astype(np.int64)
    sp = dict(st)
    sp["seg_off"] = dev(np.concatenate([[0], np.cumsum(seg_len[perm])]).astype(np.int64))
    sp["pos0"] = dev(st["pos0"].cpu().numpy()[perm])
    sp["rows"] = dev(st["rows"].cpu().numpy()[perm])
    idx_t = torch.as_tensor(order, device=DEV) if order.size else None
    for name in ("key_tok", "key_gate", "kv_tok", "kv_gate"):
        sp[name] = st[name][idx_t].contiguous() if idx_t is not None else st[name]
    sp["q_idx"] = dev(inp.q_idx[perm])
    sp["w"] = dev(inp.w[perm])
    sp["kv_off"] = dev(inp.kv_off[perm])
    sp["q_pos"] = dev(inp.q_pos[perm])
    keys1, _, s1 = _run(sp, True)
    assert np.array_equal(keys1, keys0)
    assert np.array_equal(s1.view(np.uint32), s0[perm].view(np.uint32))


def _run_paged(st, BR, seed):
    """The step with the keys in shuffled blocks of a pool (硅星人 article,
    classic-cache paragraph): the key job writes each new key at the pool row that its query's
    table maps the last visible row to; the table rows are shuffled and named
    by q_block_row."""
    inp, B = st["inp"], st["B"]
    rng = np.random.default_rng(seed)
    rb = synth.row_bytes(inp.idx_fmt, inp.d_I)
    pool, tab, bps, pool_rows = _paginate(inp.keys.reshape(-1, rb), inp.n_ent, inp.kv_off, BR, rng)
    order = rng.permutation(B)                          # table row r holds query order[r]'s blocks
    table = tab[order]
    q_row = np.argsort(order).astype(np.int32)
    n_ent = inp.n_ent.astype(np.int64)
    last = [int(tab[b][(n - 1) // BR]) * BR + (n - 1) % BR if n > 0 else 0 for b, n in enumerate(n_ent)]
    rows_h = np.array([last[b] if st["seg_len"][b] else 0 for b in range(B)], np.int64)
    pool_d, kv = dev(pool), dev(inp.kv)
    scores = torch.full((B, st["ld"]), SENTINEL, dtype=torch.float32, device=DEV)

    def job(x, gate, Dj, normalize, Rj, out, fmt, rows):
        return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=st["n_tok"], D=Dj, m=M, nseg=B,
                    seg_tok_off=st["seg_off"], seg_pos0=st["pos0"], seg_out_row=rows,
                    normalize=normalize, norm_w=None, eps=EPS, rope_dim=Rj, rope_base=ROPE_BASE,
                    out=out, out_fmt=fmt)
    jobs = [job(st["kv_tok"], st["kv_gate"], D, 1, R, kv, csa.SPLIT, st["rows"]),
            job(st["key_tok"], st["key_gate"], inp.d_I, 0, 0, pool_d, inp.idx_fmt, dev(rows_h))]
    csa.csa_compress_score_paged(jobs, st["q_idx"], st["w"], B, inp.H_I, inp.d_I, pool_d, inp.idx_fmt, pool_rows,
                                 dev(table), B, bps, BR, dev(q_row), st["q_pos"], M, scores, st["ld"])
    torch.cuda.synchronize()
    return pool_d.cpu().numpy(), kv.cpu().numpy(), scores.cpu().numpy(), rows_h


@pytest.mark.parametrize("H_I,BR,fmt", [(64, 32, csa.FP8), (64, 16, csa.FP8), (128, 64, csa.FP8),
                                        (64, 32, csa.MXFP4)])
def test_fused_step_paged_matches_contiguous(H_I, BR, fmt):
    """csa_compress_score_paged gives the contiguous call's results: every new
    key's bytes at its pool row, the KV entries, and every score bit (FP8: one
    launch; MXFP4: the two launches)."""
    lengths = [65536, 9000, 2052, 132, 8, 40000, 4, 3, 65536, 1000]
    new = [True, False, True, True, True, False, True, False, True, True]
    st = _case(lengths, new, H_I, fmt, 700 + H_I + BR)
    st["seg_len"] = np.where(np.asarray(new), M, 0)
    keys_c, kv_c, scores_c = _run(st, True)
    pool, kv_p, scores_p, rows_h = _run_paged(st, BR, 800 + BR)
    assert np.array_equal(scores_c.view(np.uint32), scores_p.view(np.uint32)), "scores differ"
    assert np.array_equal(kv_c, kv_p), "KV entries differ"
    inp = st["inp"]
    rb = synth.row_bytes(inp.idx_fmt, inp.d_I)
    kc = keys_c.reshape(-1, rb)
    for b in np.flatnonzero(new):
        row_c = int(inp.kv_off[b]) + int(inp.n_ent[b]) - 1
        assert np.array_equal(kc[row_c], pool[rows_h[b]]), f"query {b}: new key bytes differ"

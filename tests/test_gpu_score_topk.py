"""csa_compress_score_topk: a decode step's compress jobs, indexer scores and
top-k selection in one launch.  Its results must be those of
csa_compress_score followed by topk_select -- every cache byte, every score
bit and the same index sets -- the sets must be the oracle's top-k of the
scores, and the workspace must be left at zero for the next call (硅星人
article on DeepSeek V4, CSA paragraph: the lightning indexer's scores feed a
top-k selector that keeps the k best entries; DeepSeek-V4 blog, index
visibility rule)."""
import numpy as np
import pytest
import torch

import compressed_sparse_long_csa_amd as csa
from compressed_sparse_long_csa_amd import synth
from gpu_common import DEV, EPS, ROPE_BASE, dev
from test_gpu_fused import SENTINEL, _case, _check_new_scores
from test_gpu_paged import _paginate
from oracle import method as OM

pytestmark = pytest.mark.gpu

M, D, R = 4, 512, 64
LENGTHS = [65536, 9000, 2052, 132, 8, 40000, 4, 3, 65536, 1000]
NEW = [True, False, True, True, True, False, True, False, True, True]


def _jobs(st, keys, kv, rows=None):
    inp, B = st["inp"], st["B"]

    def job(x, gate, Dj, normalize, Rj, out, fmt, r):
        return dict(x=x, x_fmt=csa.BF16, gate=gate, gate_cols=1, n_tok=st["n_tok"], D=Dj, m=M, nseg=B,
                    seg_tok_off=st["seg_off"], seg_pos0=st["pos0"], seg_out_row=r,
                    normalize=normalize, norm_w=None, eps=EPS, rope_dim=Rj, rope_base=ROPE_BASE,
                    out=out, out_fmt=fmt)
    jobs = []
    if st["with_kv"]:
        jobs.append(job(st["kv_tok"], st["kv_gate"], D, 1, R, kv, csa.SPLIT, st["rows"]))
    if st["key_job"]:
        jobs.append(job(st["key_tok"], st["key_gate"], inp.d_I, 0, 0, keys, inp.idx_fmt,
                        st["rows"] if rows is None else rows))
    return jobs


def _n_valid(st):
    inp = st["inp"]
    return np.minimum((inp.q_pos + 1) // M, st["ld"]).astype(np.int64)


def _two_calls(st, k, nq=None):
    inp, B = st["inp"], st["B"]
    nq = B if nq is None else nq
    keys, kv = dev(inp.keys), dev(inp.kv)
    scores = torch.full((B, st["ld"]), SENTINEL, dtype=torch.float32, device=DEV)
    idx = torch.full((B, k), -9, dtype=torch.int32, device=DEV)
    csa.csa_compress_score(_jobs(st, keys, kv), st["q_idx"], st["w"], nq, inp.H_I, inp.d_I, keys, inp.idx_fmt,
                           st["kv_off"], st["q_pos"], M, scores, st["ld"])
    if nq > 0:
        csa.topk_select(scores, st["ld"], nq, dev(_n_valid(st)), k, idx)
    torch.cuda.synchronize()
    return keys.cpu().numpy(), kv.cpu().numpy(), scores.cpu().numpy(), idx.cpu().numpy()


def _fused(st, k, ws, nq=None):
    inp, B = st["inp"], st["B"]
    nq = B if nq is None else nq
    keys, kv = dev(inp.keys), dev(inp.kv)
    scores = torch.full((B, st["ld"]), SENTINEL, dtype=torch.float32, device=DEV)
    idx = torch.full((B, k), -9, dtype=torch.int32, device=DEV)
    csa.csa_compress_score_topk(_jobs(st, keys, kv), st["q_idx"], st["w"], nq, inp.H_I, inp.d_I, keys,
                                inp.idx_fmt, st["kv_off"], st["q_pos"], M, scores, st["ld"], k, idx, workspace=ws)
    torch.cuda.synchronize()
    return keys.cpu().numpy(), kv.cpu().numpy(), scores.cpu().numpy(), idx.cpu().numpy()


def _workspace(nq):
    return torch.zeros(max(1, csa.score_topk_workspace_bytes(nq)), dtype=torch.uint8, device=DEV)


def _check(st, k, ws=None, nq=None, oracle=True):
    """Fused against the two calls (bytes, bits, sets) and against the oracle's
    top-k of the scores; the workspace is zero afterwards."""
    nq_ = st["B"] if nq is None else nq
    ws = _workspace(nq_) if ws is None else ws
    a = _two_calls(st, k, nq)
    b = _fused(st, k, ws, nq)
    for name, x, y in zip(("keys", "kv", "scores", "idx"), a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name} differ from the two-call path"
    assert not torch.any(ws != 0).item(), "workspace not left at zero"
    if oracle:
        scores, idx = b[2], b[3]
        n = _n_valid(st)
        for i in range(nq_):
            ref = OM.top_k(scores[i, : n[i]].astype(np.float64), k)
            want = np.full(k, -1, np.int64)
            want[: len(ref)] = ref
            assert np.array_equal(idx[i].astype(np.int64), want), f"query {i}: set differs from the oracle's top-k"
    return b


@pytest.mark.parametrize("H_I,k", [(64, 512), (16, 512), (128, 1024), (64, 64), (64, 4096)])
def test_score_topk_matches_two_calls_and_oracle(H_I, k):
    st = _case(LENGTHS, NEW, H_I, csa.FP8, 900 + H_I + k)
    keys, _, scores, _ = _check(st, k)
    _check_new_scores(st, keys, scores, np.asarray(NEW))


def test_score_topk_bench_shape_reused_workspace():
    """Sixteen 65,536-token sequences, top-512, three calls on one workspace
    with different data: each call leaves the workspace ready for the next."""
    ws = _workspace(16)
    for seed in (31, 32, 33):
        st = _case([65536] * 16, [True] * 16, 64, csa.FP8, seed)
        _check(st, 512, ws=ws)


def test_score_topk_long_rows_multi_tile():
    """Rows of 65,536 and 262,144 entries (several 16K-score tiles in the
    selection; long rows take interleaved shares in the indexer)."""
    st = _case([262144, 1048576, 300000, 5000], [True, True, False, True], 64, csa.FP8, 41)
    _check(st, 1024)


def test_score_topk_ties_and_signs():
    """Equal scores at the threshold (duplicated key rows), scores that are all
    zero or negative (negative head weights give -0 for every ReLU zero), and
    rows shorter than k."""
    st = _case([20000, 20000, 9000, 1200, 16, 6000], [True, True, False, True, False, True], 64, csa.FP8, 57)
    inp = st["inp"]
    rb = synth.row_bytes(inp.idx_fmt, inp.d_I)
    keys = inp.keys.reshape(-1, rb)
    o0, o1 = int(inp.kv_off[0]), int(inp.kv_off[1])
    n0, n1 = int(inp.n_ent[0]), int(inp.n_ent[1])
    keys[o0: o0 + n0] = keys[o0]                         # query 0: every key the same
    for j in range(o1, o1 + n1):                         # query 1: seven distinct keys, repeated
        keys[j] = keys[o1 + (j - o1) % 7]
    w = inp.w.copy()
    w[2] = -np.abs(w[2])                                  # query 2: every score <= 0
    w[3] = 0.0                                            # query 3: every score 0
    st["w"] = dev(w)
    inp.w[:] = w
    for k in (512, 1000):
        _check(st, k)


def test_score_topk_without_key_job_and_short_batches():
    st = _case(LENGTHS, NEW, 64, csa.FP8, 63, key_job=False)
    _check(st, 512)
    _check(st, 512, nq=3)                                # a batch shorter than the buffers
    st = _case(LENGTHS, NEW, 64, csa.FP8, 64)
    _check(st, 512, nq=0, oracle=False)                  # the jobs alone
    st = _case([4, 8, 3], [True, True, False], 64, csa.FP8, 65)
    _check(st, 512)


def test_score_topk_paged_matches_contiguous():
    """The paged form: the same scores and sets as the contiguous call (keys in
    shuffled 32-entry blocks of a pool, table rows named per query)."""
    BR = 32
    st = _case(LENGTHS, NEW, 64, csa.FP8, 71)
    st["seg_len"] = np.where(np.asarray(NEW), M, 0)
    _, _, scores_c, idx_c = _fused(st, 512, _workspace(st["B"]))
    inp, B = st["inp"], st["B"]
    rng = np.random.default_rng(72)
    rb = synth.row_bytes(inp.idx_fmt, inp.d_I)
    pool, tab, bps, pool_rows = _paginate(inp.keys.reshape(-1, rb), inp.n_ent, inp.kv_off, BR, rng)
    order = rng.permutation(B)
    table = tab[order]
    q_row = np.argsort(order).astype(np.int32)
    n_ent = inp.n_ent.astype(np.int64)
    last = [int(tab[b][(n - 1) // BR]) * BR + (n - 1) % BR if n > 0 else 0 for b, n in enumerate(n_ent)]
    rows_h = np.array([last[b] if st["seg_len"][b] else 0 for b in range(B)], np.int64)
    pool_d, kv = dev(pool), dev(inp.kv)
    scores = torch.full((B, st["ld"]), SENTINEL, dtype=torch.float32, device=DEV)
    idx = torch.full((B, 512), -9, dtype=torch.int32, device=DEV)
    ws = _workspace(B)
    csa.csa_compress_score_topk_paged(_jobs(st, pool_d, kv, rows=dev(rows_h)), st["q_idx"], st["w"], B, inp.H_I,
                                      inp.d_I, pool_d, inp.idx_fmt, pool_rows, dev(table), B, bps, BR, dev(q_row),
                                      st["q_pos"], M, scores, st["ld"], 512, idx, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), scores_c.view(np.uint32)), "scores differ"
    assert np.array_equal(idx.cpu().numpy(), idx_c), "index sets differ"
    assert not torch.any(ws != 0).item()


def test_score_topk_in_a_graph():
    """The one-launch step captured in a HIP graph and replayed with eager work
    between replays: every replay gives the eager results (the workspace is
    cleared by each replay for the next)."""
    st = _case([65536] * 8 + [3000] * 8, [True] * 16, 64, csa.FP8, 81)
    inp, B, k = st["inp"], st["B"], 512
    keys0 = dev(inp.keys)
    kv0 = dev(inp.kv)
    ws = _workspace(B)
    eager = _fused(st, k, ws)
    keys, kv = keys0.clone(), kv0.clone()
    scores = torch.full((B, st["ld"]), SENTINEL, dtype=torch.float32, device=DEV)
    idx = torch.full((B, k), -9, dtype=torch.int32, device=DEV)
    jobs = _jobs(st, keys, kv)

    def run():
        csa.csa_compress_score_topk(jobs, st["q_idx"], st["w"], B, inp.H_I, inp.d_I, keys, inp.idx_fmt,
                                    st["kv_off"], st["q_pos"], M, scores, st["ld"], k, idx, workspace=ws,
                                    check=False)          # (host-side checks copy to the host)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                            # warm-up on a side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        keys.copy_(keys0)
        kv.copy_(kv0)
        scores.fill_(SENTINEL)
        idx.fill_(-9)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(scores.cpu().numpy().view(np.uint32), eager[2].view(np.uint32)), rep
        assert np.array_equal(idx.cpu().numpy(), eager[3]), rep
        assert not torch.any(ws != 0).item(), rep
        other = _fused(st, k, ws)                        # eager work between replays
        assert np.array_equal(other[3], eager[3])


def test_score_topk_many_calls_on_one_workspace():
    """Thirty calls in a row over three batches (bench shape, ragged, long rows)
    sharing one workspace: every call gives the two-call path's sets and
    scores, and leaves the workspace at zero for the next."""
    cases = [_case([65536] * 16, [True] * 16, 64, csa.FP8, 91),
             _case(LENGTHS, NEW, 64, csa.FP8, 92),
             _case([262144, 100000, 40000], [True, False, True], 64, csa.FP8, 93)]
    refs = [_two_calls(st, 512) for st in cases]
    ws = _workspace(16)
    for rep in range(10):
        for st, ref in zip(cases, refs):
            got = _fused(st, 512, ws)
            assert np.array_equal(got[3], ref[3]), f"call {rep}: sets differ"
            assert np.array_equal(got[2].view(np.uint32), ref[2].view(np.uint32)), f"call {rep}: scores differ"
    assert not torch.any(ws != 0).item()
